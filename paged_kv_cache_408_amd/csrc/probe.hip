// pa_probe_read: plain streaming reads of device memory, the references the decode's HBM rate is
// set against on the same device and at the same sizes.  Every byte of the range is loaded once
// (non-temporal 16-byte loads: the data is not kept in the caches), the loaded words are folded
// into one value per lane, and nothing is written unless that value equals a constant no input
// of this library produces, so the loads cannot be dropped and the kernel moves only the bytes
// it reads.  One work-group of four waves per compute unit, as the decode's uniform grid runs.
//  - PA_PROBE_GRID: a grid-stride sweep, every lane with eight loads in flight: at any moment
//    the whole device reads one compact window of memory.
//  - PA_PROBE_RANGES: work-group j reads its own contiguous range of 4 KiB tiles, wave w the
//    tiles w, w + 4, ... with four tiles in flight: the decode's partitions (a work-group
//    streams one request's share of the cache) without the block table.
//  - PA_PROBE_TILES: passes of two 4 KiB tiles taken through a caller-given order (e.g. the K and V
//    tiles each pass of the decode reads, from its block tables; entries are clamped into the
//    range), per work-group and wave as the decode's uniform grid splits them, each pass moved
//    straight to LDS: the decode's memory traffic without its arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pagedkv.h"
#include "pa_device.h"
#include "pa_error.h"

namespace {

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr uint32_t kNeverFolded = 0x9e3779b9u;
constexpr int kTileVecs = 256;                  // 16-byte vectors per 4 KiB tile

__device__ __forceinline__ uint32_t fold4(const v4u32& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kProbeThreads) void grid_probe_kernel(const v4u32* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
    constexpr int U = 8;
    const int64_t stride = int64_t(gridDim.x) * kProbeThreads;
    int64_t i = int64_t(blockIdx.x) * kProbeThreads + threadIdx.x;
    uint32_t fold = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        v4u32 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) fold ^= fold4(v[u]);
    }
    for (; i < n16; i += stride) fold ^= fold4(__builtin_nontemporal_load(src + i));
    if (fold == kNeverFolded) sink[blockIdx.x] = fold;
}

// Work-group j: tiles [j * ntiles / grid, (j + 1) * ntiles / grid) of src, wave w the tiles
// w, w + 4, ... with four tiles in flight (PA_PROBE_RANGES).
__global__ __launch_bounds__(kProbeThreads) void range_probe_kernel(const v4u32* __restrict__ src, int64_t ntiles,
                                                                    uint32_t* __restrict__ sink) {
    constexpr int TU = 4;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t0 = int64_t(blockIdx.x) * ntiles / gridDim.x, t1 = int64_t(blockIdx.x + 1) * ntiles / gridDim.x;
    uint32_t fold = 0;
    int64_t k = t0 + w;
    for (; k + 4 * (TU - 1) < t1; k += 4 * TU) {
        v4u32 v[TU][4];
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const v4u32* p = src + (k + 4 * u) * kTileVecs + lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[u][j] = __builtin_nontemporal_load(p + 64 * j);
        }
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) fold ^= fold4(v[u][j]);
    }
    for (; k < t1; k += 4) {
        const v4u32* p = src + k * kTileVecs + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) fold ^= fold4(__builtin_nontemporal_load(p + 64 * j));
    }
    if (fold == kNeverFolded) sink[blockIdx.x] = fold;
}

// PA_PROBE_TILES: passes of two tiles (entries 2 p and 2 p + 1 of `order`, clamped into src's
// nsrc tiles); work-group j takes passes [j * npass / grid, (j + 1) * npass / grid), wave w the
// passes w, w + 4, ...; each pass's 8 KiB go straight to LDS (a two-stage ring per wave, one
// pass in flight while the previous one has landed), as the decode's bf16 path moves K and V.
__global__ __launch_bounds__(kProbeThreads) void pass_probe_kernel(const unsigned char* __restrict__ src, int64_t nsrc,
                                                                   int64_t npass, const int32_t* __restrict__ order,
                                                                   uint32_t* __restrict__ sink) {
    __shared__ __align__(16) unsigned char ring[4][2][8192];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t p0 = int64_t(blockIdx.x) * npass / gridDim.x, p1 = int64_t(blockIdx.x + 1) * npass / gridDim.x;
    const int64_t nk = p1 - p0 > w ? (p1 - p0 - w + 3) / 4 : 0;
    // the tiles of this wave's passes, 64 passes at a time (lane i: pass w + 4 (k0 + i)), read ahead
    // of the loads that use them; an entry outside [0, nsrc) is clamped into it (a wrong order
    // reads the wrong tiles, never outside src)
    int ent_k = 0, ent_v = 0;
    auto read_tiles = [&](int64_t k0) {
        const int64_t p = min(p0 + w + 4 * (k0 + lane), p1 - 1);
        ent_k = min(max(order[2 * p], 0), int(nsrc - 1));
        ent_v = min(max(order[2 * p + 1], 0), int(nsrc - 1));
    };
    auto issue = [&](int64_t k, int st) {
        if ((k & 63) == 0) {
            read_tiles(k);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the ids, and the loads before them
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int id = __builtin_amdgcn_readlane(t == 0 ? ent_k : ent_v, int(k & 63));
            const unsigned char* a = src + int64_t(id) * 4096 + 16 * lane;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dma16_lane(a + 1024 * j, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[w][st][t * 4096 + 1024 * j])));
        }
    };
    uint32_t fold = 0;
    if (nk > 0) issue(0, 0);
    int st = 0;
    for (int64_t k = 0; k < nk; ++k) {
        if (k + 1 < nk) {
            issue(k + 1, st ^ 1);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // pass k has landed (pass k + 1 in flight)
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        fold ^= *reinterpret_cast<const uint32_t*>(&ring[w][st][16 * lane]);
        st ^= 1;
    }
    if (fold == kNeverFolded) sink[blockIdx.x] = fold;
}

}  // namespace

extern "C" int pa_probe_read(const void* src, int64_t bytes, int32_t pattern, const int32_t* tile_order,
                             int64_t order_len, void* sink, int64_t sink_bytes, void* stream) {
    pagedkv::clear_error();
    if (pattern != PA_PROBE_GRID && pattern != PA_PROBE_RANGES && pattern != PA_PROBE_TILES)
        return pagedkv::fail(PA_ERR_INVALID, "pa_probe_read: unknown pattern %d", pattern);
    const int64_t unit = pattern == PA_PROBE_GRID ? 16 : 4096;
    if (bytes < 0 || bytes % unit != 0 || (bytes > 0 && (!src || reinterpret_cast<uintptr_t>(src) % 16 != 0)))
        return pagedkv::fail(PA_ERR_INVALID, "pa_probe_read: %lld bytes at %p (16-byte aligned, a multiple of %lld)",
                             (long long)bytes, src, (long long)unit);
    if (pattern == PA_PROBE_TILES && bytes > 0 && (order_len < 0 || order_len % 2 != 0 || (order_len > 0 && !tile_order)))
        return pagedkv::fail(PA_ERR_INVALID, "pa_probe_read: PA_PROBE_TILES needs a tile order of pairs (%lld entries)",
                             (long long)order_len);
    if (pattern == PA_PROBE_TILES && order_len == 0) return PA_OK;
    if (bytes / 4096 > INT32_MAX || order_len > INT32_MAX)
        return pagedkv::fail(PA_ERR_INVALID, "pa_probe_read: more than 2^31 tiles");
    if (bytes == 0) return PA_OK;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        cus = 256;
    }
    if (!sink || sink_bytes < int64_t(cus) * 4)
        return pagedkv::fail(PA_ERR_INVALID, "pa_probe_read: sink of %lld bytes, %lld needed", (long long)sink_bytes,
                             (long long)cus * 4);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (pattern == PA_PROBE_GRID)
        hipLaunchKernelGGL(grid_probe_kernel, dim3(cus), dim3(kProbeThreads), 0, st, static_cast<const v4u32*>(src),
                           bytes / 16, static_cast<uint32_t*>(sink));
    else if (pattern == PA_PROBE_RANGES)
        hipLaunchKernelGGL(range_probe_kernel, dim3(cus), dim3(kProbeThreads), 0, st, static_cast<const v4u32*>(src),
                           bytes / 4096, static_cast<uint32_t*>(sink));
    else
        hipLaunchKernelGGL(pass_probe_kernel, dim3(cus), dim3(kProbeThreads), 0, st, static_cast<const unsigned char*>(src),
                           bytes / 4096, order_len / 2, tile_order, static_cast<uint32_t*>(sink));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pagedkv::fail(PA_ERR_DEVICE, "pa_probe_read: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}
