// Paged prefill attention (causal) for AMD Instinct MI355X (gfx950) and its C ABI entry.
//
// What is computed is stated in include/pagedkv.h (pa_prefill): several new tokens per request
// attend, through the request's block table, to every cached token up to their own position
// ("KV Cache Management", "Why Does This Exist?": a prompt's keys and values are computed and
// saved once; "KV Cache Optimization and PagedAttention", first paragraph: each token attends
// to every previous token).
//
// prefill_kernel: one work-group (8 wave64) per (query tile, KV head, request).  A query tile
// is 128 rows = 128 / G new tokens x the G query heads of the KV head, 16 rows per wave.  The
// work-group walks the request's K/V in tiles of 64 tokens, from position 0 up to the tile's
// last query position, through a double-buffered LDS tile that each wave fills for its 8
// token rows with global_load_lds_dwordx4 (HBM straight to LDS; 16-byte chunks of a row
// XOR-swizzled by row so that no LDS read conflicts on banks).  Two work-groups (16 waves, 128 VGPRs each) fit a compute unit.  Per
// 16 KV tokens each wave does what decode does for 16 heads:
//  - scores S^T[token][row] = K_step[16 x D] . Q^T[D x 16] with v_mfma_f32_16x16x32_bf16
//    (K read from LDS as the A operand, the wave's 16 query rows as the B operand, loaded once);
//  - the causal mask (token position > row position -> -inf), the online softmax per row with
//    the lazy rescale of the decode kernel, weights rounded to bf16; the denominator, the sum of
//    the rounded weights, comes from one more product of the weights with a column of ones;
//  - out[row][16 dims] += P . V with v_mfma_f32_16x16x32_bf16 over 32 tokens, V read
//    token-major per dim with ds_read_b64_tr_b16 from the same LDS tile (two reads of 4 tokens
//    form the B operand; the A operand holds the row's weights of the same 8 tokens).
// The softmax is updated once per 64-token tile (one row maximum, one ballot); 16-token steps
// past all of a wave's rows are skipped; tiles are loaded once per work-group for all of its
// rows.  Rows are normalised in registers and written as bf16.

#include "pa_device.h"
#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

struct PrefillArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* query_start;
    float score_scale;          // scale * log2(e)
    int num_seqs;
    int hkv;
    int max_blocks;
    int max_query_len;
    int max_seq_len;
    int qtiles;                 // query tiles per request in the grid
    int64_t num_blocks;
    int64_t num_query_tokens;
};

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8      // waves per work-group (4 or 8): 8 measured faster
#endif
constexpr int kPWaves = PA_PREFILL_WAVES;
static_assert(kPWaves == 4 || kPWaves == 8, "4 or 8 waves per work-group");
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPRows = 16 * kPWaves;   // query rows (token, head) per work-group
constexpr int kKvTile = 64;            // KV tokens per LDS tile
constexpr int kRW = kKvTile / kPWaves; // token rows of a tile each wave loads

// Slot XOR of a K/V tile row in LDS: chunk c of tile row R sits at slot c ^ swz(R).  Chosen so
// that both LDS read patterns are free of bank conflicts (64 banks of 4 bytes):
//  - the K operand reads one chunk of 16 consecutive rows: the slots must differ among rows that
//    share banks (D = 128: every row covers all banks once; D = 64: rows of equal parity);
//  - the transpose reads of V take chunks {2t, 2t + 1} of 4 consecutive rows (from a multiple
//    of 4) per 16 lanes, 8 rows per 32: those chunk pairs must be disjoint among rows that
//    share banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
    else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

template <int D, int BS, int G>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(const PrefillArgs a) {
    constexpr int ROWB = D * 2;                 // bytes of one bf16 token row
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    constexpr int NQK = D / 32;                 // 16x16x32 products per 16 tokens (scores)
    constexpr int NPV = D / 16;                 // 16-dim output tiles
    constexpr int TQ = kPRows / G;              // new tokens per work-group
    constexpr int NI = kRW * ROWB / 1024;       // DMA instructions per wave per K (or V) tile
    constexpr int RPI = 64 / CPR;               // token rows per DMA instruction
    constexpr int TB = kKvTile * ROWB;          // bytes of one K (or V) tile
    constexpr int WPB = BS < kRW ? 2 : 1;       // blocks behind one wave's kRW token rows
    static_assert(NI >= 1 && RPI <= BS && (WPB == 1 || 2 * BS == kRW), "tile shape");
    static_assert(G == 1 || G == 4 || G == 8, "query heads per KV head");

    __shared__ __align__(16) unsigned char s_kv[2][2][TB];   // [buffer][K, V][64 rows]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp4 = lane >> 4;
    const int hq = a.hkv * G;
    const int b = blockIdx.x % a.num_seqs;
    const int qt = a.qtiles - 1 - static_cast<int>(blockIdx.x / a.num_seqs);   // longest tiles first
    const int g = blockIdx.y;

    const int q0 = __builtin_amdgcn_readfirstlane(gld_i32(a.query_start + b));
    const int q1 = __builtin_amdgcn_readfirstlane(gld_i32(a.query_start + b + 1));
    if (q0 < 0 || q1 < q0 || q1 > a.num_query_tokens) return;   // no row of this request can be named
    const int n = q1 - q0;
    const int t0q = qt * TQ;
    if (t0q >= n) return;
    const int L_raw = __builtin_amdgcn_readfirstlane(gld_i32(a.seq_lens + b));
    const bool len_bad = L_raw < n || L_raw > a.max_seq_len || L_raw > a.max_blocks * BS || n > a.max_query_len;
    const int L = len_bad ? n : L_raw;
    const int ctx = L - n;                                    // tokens before the new ones
    const int tq_end = min(n, t0q + TQ);
    const int kv_end = ctx + tq_end;                          // positions this work-group reads
    const int ntiles = len_bad ? 0 : (kv_end + kKvTile - 1) / kKvTile;

    // this lane's query row (column of the score products): token t0q + r / G, head r % G
    const int r = 16 * w + col;
    const int my_tok = min(t0q + r / G, n - 1);
    const int my_pos = ctx + my_tok;
    const int wave_min = ctx + min(t0q + (16 * w) / G, n - 1);
    const int wave_max = ctx + min(t0q + (16 * w + 15) / G, n - 1);

    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
    U4 qb[NQK];
    {
        const uint16_t* qrow = qbase + (int64_t(q0 + my_tok) * hq + int64_t(g) * G + r % G) * D;
#pragma unroll
        for (int j = 0; j < NQK; ++j) qb[j] = gld16(qrow + 32 * j + 8 * grp4);
    }

    // block ids of this wave's rows for 64 tiles (lane j: tile k0 + j); ids outside the pool
    // within the positions read are flagged and every such id is replaced by 0
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    int ent_a = 0, ent_b = 0;
    bool bad = false;
    auto read_entries = [&](int k0) {
        const int tile = k0 + lane;
        const int e = (kKvTile * tile + kRW * w) / BS;
        ent_a = a.max_blocks > 0 ? gld_i32(table + min(e, a.max_blocks - 1)) : -1;
        if constexpr (WPB == 2) ent_b = a.max_blocks > 0 ? gld_i32(table + min(e + 1, a.max_blocks - 1)) : -1;
        const bool live = tile < ntiles;
        if (ent_a < 0 || ent_a >= a.num_blocks) {
            if (live && e * BS < kv_end) bad = true;
            ent_a = 0;
        }
        if constexpr (WPB == 2) {
            if (ent_b < 0 || ent_b >= a.num_blocks) {
                if (live && (e + 1) * BS < kv_end) bad = true;
                ent_b = 0;
            }
        }
    };
    read_entries(0);

    // DMA layout: tile row R holds its chunk c at slot c ^ swz(R); lane `lane` of the
    // wave's instruction i fills position 64 i + lane of the wave's kRW-row slice
    uint32_t src_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int pos = 64 * i + lane, row = pos / CPR, slot = pos % CPR;
        src_off[i] = uint32_t(row) * ROWB + 16u * uint32_t(slot ^ swz<D>(kRW * w + row));
    }
    const int64_t blk_bytes = int64_t(a.hkv) * BS * ROWB;
    const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(a.k_cache) + int64_t(g) * BS * ROWB;
    const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(a.v_cache) + int64_t(g) * BS * ROWB;

    auto issue = [&](int k, int bf) {
        if ((k & 63) == 0 && k > 0) read_entries(k);
        const int pos0 = kKvTile * k + kRW * w;
        const int b0 = __builtin_amdgcn_readlane(ent_a, k & 63);
        PA_LDS unsigned char* dk = (PA_LDS unsigned char*)&s_kv[bf][0][0] + kRW * w * ROWB;
        PA_LDS unsigned char* dv = (PA_LDS unsigned char*)&s_kv[bf][1][0] + kRW * w * ROWB;
        if constexpr (WPB == 1) {
            const int64_t off = int64_t(b0) * blk_bytes + int64_t(pos0 % BS) * ROWB;
#pragma unroll
            for (int i = 0; i < NI; ++i) dma16(kbytes + off, src_off[i], lds_addr(dk + 1024 * i));
#pragma unroll
            for (int i = 0; i < NI; ++i) dma16(vbytes + off, src_off[i], lds_addr(dv + 1024 * i));
        } else {   // rows 0..7 from the first block, 8..15 from the second
            const int b1 = __builtin_amdgcn_readlane(ent_b, k & 63);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bool second = i * RPI >= BS;
                const uint32_t off = src_off[i] - (second ? uint32_t(BS) * ROWB : 0u);
                const int64_t boff = int64_t(second ? b1 : b0) * blk_bytes;
                dma16(kbytes + boff, off, lds_addr(dk + 1024 * i));
                dma16(vbytes + boff, off, lds_addr(dv + 1024 * i));
            }
        }
    };

    float m_ref = -INFINITY;                          // row `col`, in scaled units
    f32x4v acc[NPV];                                  // out[row 4 * grp4 + i][16 t + col]
#pragma unroll
    for (int t = 0; t < NPV; ++t) acc[t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4v lsum = {0.0f, 0.0f, 0.0f, 0.0f};           // sum of row 4 * grp4 + i's weights (every column)
    const bf16x8v ones = __builtin_bit_cast(bf16x8v, u32x4v{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const float sc = a.score_scale;
    const bool pos_scale = sc > 0.0f;
    const float se = pos_scale ? sc : 1.0f;           // scale applied in the exponent

    if (ntiles > 0) issue(0, 0);
    for (int k = 0; k < ntiles; ++k) {
        const int bf = k & 1;
        wait_vmem<0>();                               // this wave's rows of tile k have landed
        if (kKvTile * (k + 1) > L) {                  // V rows past the request: zero (may hold anything)
            PA_LDS unsigned char* dv = (PA_LDS unsigned char*)&s_kv[bf][1][0] + kRW * w * ROWB;
            const int pos0 = kKvTile * k + kRW * w;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p = 64 * i + lane;
                if (pos0 + p / CPR >= L) lds_st16(dv + 16 * p, U4{0, 0, 0, 0});
            }
        }
        __syncthreads();                              // tile k complete; tile k - 1 no longer read
        if (k + 1 < ntiles) issue(k + 1, bf ^ 1);
        const PA_LDS unsigned char* kt = (const PA_LDS unsigned char*)&s_kv[bf][0][0];
        const PA_LDS unsigned char* vt = (const PA_LDS unsigned char*)&s_kv[bf][1][0];
        const int p_base = kKvTile * k;
        if (p_base > wave_max) continue;              // every row of this wave is before this tile
        const int nst = min(kKvTile / 16, (wave_max - p_base) / 16 + 1);   // steps of 16 with a visible token

        // scores of the tile's steps (independent chains of NQK products)
        f32x4v s4[kKvTile / 16];
#pragma unroll
        for (int st = 0; st < kKvTile / 16; ++st) {
            s4[st] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
            if (st < nst) {
                const int krow = 16 * st + col;
                const PA_LDS unsigned char* kp = kt + krow * ROWB;
#pragma unroll
                for (int j = 0; j < NQK; ++j) {
                    const U4 kv = lds_ld16(kp + 16 * ((4 * j + grp4) ^ swz<D>(krow)));
                    s4[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, kv),
                                                                     __builtin_bit_cast(bf16x8v, qb[j]), s4[st], 0, 0, 0);
                }
            }
        }
        // causal mask (tiles that reach past the wave's first row only), then one online-softmax
        // update per tile.  With a positive scale (the usual 1 / sqrt(d)) the maximum is taken on
        // the raw scores and the scale is folded into the exponent's fused multiply-add.
        if (!pos_scale) {
#pragma unroll
            for (int st = 0; st < kKvTile / 16; ++st) s4[st] *= sc;
        }
        if (p_base + kKvTile - 1 > wave_min) {
#pragma unroll
            for (int st = 0; st < kKvTile / 16; ++st) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (p_base + 16 * st + 4 * grp4 + i > my_pos) s4[st][i] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < kKvTile / 16; ++st)
            mx = fmaxf(fmaxf(mx, fmaxf(s4[st][0], s4[st][1])), fmaxf(s4[st][2], s4[st][3]));
        mx = pair16_max(pair32_max(mx)) * se;         // the row's maximum over the tile, scaled
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first tile
            m_ref = m_new;
#pragma unroll
            for (int i = 0; i < 4; ++i) {             // accumulator rows 4 * grp4 + i take that row's factor
                const float ai = __int_as_float(
                    __builtin_amdgcn_ds_bpermute(4 * (4 * grp4 + i), __float_as_int(alpha)));
                lsum[i] *= ai;
#pragma unroll
                for (int t = 0; t < NPV; ++t) acc[t][i] *= ai;
            }
        }
        uint32_t pw[kKvTile / 16][2];                 // weights rounded to bf16, in pairs
#pragma unroll
        for (int st = 0; st < kKvTile / 16; ++st) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x2v pr;
                pr[0] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s4[st][2 * h], se, -m_ref)));
                pr[1] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s4[st][2 * h + 1], se, -m_ref)));
                pw[st][h] = __builtin_bit_cast(uint32_t, pr);
            }
        }
        // out[row][16 dims] += P . V over 32 tokens per product: the A operand's 8 values of a
        // lane are its row's weights for tokens 4 grp4 .. +3 of step 2 s and of step 2 s + 1; the
        // B operand's are the same tokens' V values, two transpose reads
        const int vsub = 4 * grp4 + ((lane & 15) >> 2);
#pragma unroll
        for (int sp = 0; sp < kKvTile / 32; ++sp) {
            if (2 * sp >= nst) break;
            const bf16x8v pa = __builtin_bit_cast(bf16x8v, u32x4v{pw[2 * sp][0], pw[2 * sp][1], pw[2 * sp + 1][0],
                                                                 pw[2 * sp + 1][1]});
            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, lsum, 0, 0, 0);   // row sums of the rounded weights
            const int r0 = 32 * sp + vsub, r1 = r0 + 16;
#pragma unroll
            for (int t = 0; t < NPV; ++t) {
                const int c = 2 * t + ((lane & 3) >> 1);
                const i16x4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (PA_LDS i16x4v*)(vt + r0 * ROWB + 16 * (c ^ swz<D>(r0)) + 8 * (lane & 1)));
                const i16x4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (PA_LDS i16x4v*)(vt + r1 * ROWB + 16 * (c ^ swz<D>(r1)) + 8 * (lane & 1)));
                const i16x8v vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8v, vv), acc[t], 0, 0, 0);
            }
        }
    }

    // normalise each row and write it (rows past the request's new tokens are not written)
    const bool any_bad = __syncthreads_or(bad) || len_bad;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ri = 16 * w + 4 * grp4 + i;
        const float inv = any_bad ? __builtin_nanf("") : 1.0f / lsum[i];
        const int tok = t0q + ri / G;
        if (tok >= n) continue;
        uint16_t* orow = out + (int64_t(q0 + tok) * hq + int64_t(g) * G + ri % G) * D;
#pragma unroll
        for (int t = 0; t < NPV; ++t) gst(orow + 16 * t + col, f32_to_bf16(acc[t][i] * inv));
    }
}

template <int D, int BS>
int launch_g(int G, const PrefillArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: hipLaunchKernelGGL((prefill_kernel<D, BS, 1>), grid, dim3(kPThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<D, BS, 4>), grid, dim3(kPThreads), 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<D, BS, 8>), grid, dim3(kPThreads), 0, st, a); break;
        default: return fail(PA_ERR_UNSUPPORTED, "pa_prefill: %d query heads per KV head not in {1, 4, 8}", G);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "pa_prefill: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

template <int D>
int launch_bs(int BS, int G, const PrefillArgs& a, dim3 grid, hipStream_t st) {
    switch (BS) {
        case 8: return launch_g<D, 8>(G, a, grid, st);
        case 16: return launch_g<D, 16>(G, a, grid, st);
        case 32: return launch_g<D, 32>(G, a, grid, st);
        case 128: return launch_g<D, 128>(G, a, grid, st);
        default: return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d not in {8, 16, 32, 128}", BS);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                          float scale, int32_t block_size, int32_t num_seqs, int64_t num_query_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_seq_len,
                          int32_t q_dtype, int32_t cache_dtype, void* stream) {
    pagedkv::clear_error();
    if (q_dtype != PA_DTYPE_BF16 || cache_dtype != PA_DTYPE_BF16)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: (q dtype %d, cache dtype %d) not supported (bf16, bf16 only)",
                    q_dtype, cache_dtype);
    if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq < 0 || max_query_len < 0 || max_seq_len < 0)
        return fail(PA_ERR_INVALID, "pa_prefill: negative or zero size");
    if (num_q_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID, "pa_prefill: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                    num_kv_heads);
    if (!(scale == scale)) return fail(PA_ERR_INVALID, "pa_prefill: scale is NaN");
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !seq_lens || !query_start || (max_blocks_per_seq > 0 && !block_tables))
        return fail(PA_ERR_INVALID, "pa_prefill: NULL pointer");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_prefill: out, q and caches must be 16-byte aligned");
    if (int64_t(max_blocks_per_seq) * block_size < max_seq_len)
        return fail(PA_ERR_INVALID, "pa_prefill: max_blocks_per_seq * block_size < max_seq_len");
    if (max_query_len > max_seq_len) return fail(PA_ERR_INVALID, "pa_prefill: max_query_len > max_seq_len");
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d not in {64, 128}", head_dim);
    const int G = num_q_heads / num_kv_heads;
    if (G != 1 && G != 4 && G != 8)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: %d query heads per KV head not in {1, 4, 8}", G);
    const int TQ = kPRows / G;
    const int64_t qtiles = (int64_t(max_query_len) + TQ - 1) / TQ;
    if (qtiles * num_seqs > 0x7fffffff || num_kv_heads > 65535)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: grid of %lld x %d work-groups", (long long)(qtiles * num_seqs),
                    num_kv_heads);

    PrefillArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_start = query_start;
    a.score_scale = scale * kLog2e;
    a.num_seqs = num_seqs;
    a.hkv = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.max_query_len = max_query_len;
    a.max_seq_len = max_seq_len;
    a.qtiles = static_cast<int>(qtiles);
    a.num_blocks = num_blocks;
    a.num_query_tokens = num_query_tokens;
    const dim3 grid(static_cast<unsigned>(qtiles * num_seqs), static_cast<unsigned>(num_kv_heads));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (head_dim == 64) return launch_bs<64>(block_size, G, a, grid, st);
    return launch_bs<128>(block_size, G, a, grid, st);
}
