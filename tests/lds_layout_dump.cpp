// Prints the kernels' LDS slot tables (from pa_layout.h) for the host-side bank-conflict
// check in test_lds_layout.py.  Built with hipcc; runs on the host only (no device calls).
//   vt <D> <row> <slot of chunk 0..D/8-1>...     decode V tile (fp8 and 4-bit caches)
//   dm <D> <row> <slot of chunk 0..D/8-1>...     decode K/V stage (bf16 cache)
//   pf <D> <row> <prefill_swz(row)>               prefill K/V tile
#include <cstdio>

#include "../paged_kv_cache_408_amd/csrc/pa_layout.h"

template <int D>
void dump() {
    for (int r = 0; r < 64; ++r) {
        std::printf("vt %d %d", D, r);
        for (int c = 0; c < D / 8; ++c) std::printf(" %d", vt_slot<D>(r, c));
        std::printf("\ndm %d %d", D, r);
        for (int c = 0; c < D / 8; ++c) std::printf(" %d", dma_slot<D>(r, c));
        std::printf("\npf %d %d %d\n", D, r, prefill_swz<D>(r));
    }
}

int main() {
    dump<64>();
    dump<128>();
    return 0;
}
