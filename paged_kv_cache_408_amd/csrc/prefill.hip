// Paged prefill attention (causal) for AMD Instinct MI355X (gfx950) and its C ABI entry.
//
// What is computed is stated in include/pagedkv.h (pa_prefill): several new tokens per request
// attend, through the request's block table, to every cached token up to their own position
// ("KV Cache Management", "Why Does This Exist?": a prompt's keys and values are computed and
// saved once; "KV Cache Optimization and PagedAttention", first paragraph: each token attends
// to every previous token).
//
// prefill_kernel: one work-group (8 wave64) per (query tile, KV head, request).  A query tile
// is 256 rows = 256 / G new tokens x the G query heads of the KV head, 32 rows per wave, so each
// K/V tile brought into LDS serves 256 rows.  The work-group walks the request's K/V in tiles of
// 64 tokens, from position 0 up to the tile's last query position, through a double-buffered
// LDS ring that each wave fills for its 8 token rows with global_load_lds_dwordx4 (HBM straight
// to LDS; 16-byte chunks of a row XOR-swizzled by row so that no LDS read conflicts on banks).
// One work-group (2 waves per SIMD) fits a compute unit at head dim 128.  Per 64-token tile
// each wave computes, with v_mfma_f32_32x32x16_bf16:
//  - scores S^T[token][row] = K[32 x D] . Q^T[D x 32] for both 32-token halves (K read from
//    LDS as the A operand, the wave's 32 query rows as the B operand, loaded once); a lane then
//    holds 16 of the 32 scores of its own row, the other 16 sit in the lane 32 apart;
//  - the causal mask on diagonal tiles only (token position > row position -> -inf), one
//    online-softmax update per tile (one row maximum across the lane pair, the lazy rescale),
//    weights rounded to bf16 by the hardware conversion; the denominator adds the rounded
//    weights two at a time (v_dot2c_f32_bf16 with a pair of ones);
//  - out^T[dim][row] += V^T[dim x 16] . P^T[16 x row] per 16 tokens and 32 dims: V^T comes from
//    two ds_read_b64_tr_b16 transpose reads of 4 tokens, P^T is the lane's own weights, so the
//    accumulators of a lane all belong to its row and take its rescale factor directly.
// Half tiles past all of a wave's rows are skipped; tiles are loaded once per work-group for all
// of its rows.  Rows are normalised in registers and written as bf16.
// fp8 and 4-bit caches: each wave loads its rows of the next tile into registers and writes
// them, widened to bf16 (exactly), into the same LDS tile; the compute part is the same.

#include "pa_device.h"
#include "pa_layout.h"
#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

struct PrefillArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* query_start;
    const float* k_scale;       // fp8 caches: per KV head
    const float* v_scale;
    float score_scale;          // scale * log2(e)
    int num_seqs;
    int hkv;
    int max_blocks;
    int max_query_len;
    int max_seq_len;
    int qtiles;                 // query tiles per request in the grid
    int ugrp;                   // units an XCD runs side by side (1 or 2)
    int64_t num_blocks;
    int64_t num_query_tokens;
};

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 2
#endif
constexpr int kStages = PA_PREFILL_STAGES; // K/V tiles in the LDS ring (2 or 3): alike
static_assert(PA_PREFILL_WAVES == 4 || PA_PREFILL_WAVES == 8, "4 or 8 waves per work-group");
static_assert(kStages == 2 || kStages == 3, "2 or 3 stages");
constexpr int kWRows = 32;             // query rows (token, head) per wave
constexpr int kKvTile = 64;            // KV tokens per LDS tile
// Waves per work-group: PA_PREFILL_WAVES over bf16 caches; 8 over fp8 and 4-bit ones, whose tile
// loads take 8 token rows per wave.
__host__ __device__ constexpr int pwaves(int cdt) { return cdt == PA_DTYPE_BF16 ? PA_PREFILL_WAVES : 8; }

// NaN-propagating maximum (v_maximum3_f32 on gfx950: no canonicalising moves before it)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <int CDT, int D, int BS, int G>
__global__ __launch_bounds__(64 * pwaves(CDT), 2) void prefill_kernel(const PrefillArgs a) {
    // bf16 caches: tiles straight from HBM into LDS by DMA.  fp8 and 4-bit caches: each wave
    // loads its rows of the next tile into registers one tile ahead and writes them to the
    // same LDS tile widened to bf16 (exactly: every E4M3 value, and every E2M1 value times its
    // block's power of two, is a bf16 number); fp8's per-head scales go into the score scale
    // and the output.
    constexpr bool kQ = CDT != PA_DTYPE_BF16;
    constexpr int kPWaves = pwaves(CDT);         // waves per work-group
    constexpr int kPRows = kWRows * kPWaves;    // query rows per work-group
    constexpr int kRW = kKvTile / kPWaves;      // token rows of a tile each wave loads
    constexpr bool kMx = CDT == PA_DTYPE_MXFP4;
    static_assert(CDT == PA_DTYPE_BF16 || CDT == PA_DTYPE_FP8_E4M3 || CDT == PA_DTYPE_MXFP4, "cache type");
    constexpr int ROWB = D * 2;                 // bytes of one bf16 token row
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    constexpr int NQK = D / 16;                 // 32x32x16 products per 32 tokens (scores)
    constexpr int NPV = D / 32;                 // 32-dim output tiles
    constexpr int TQ = kPRows / G;              // new tokens per work-group
    constexpr int NI = kRW * ROWB / 1024;       // DMA instructions per wave per K (or V) tile
    constexpr int RPI = 64 / CPR;               // token rows per DMA instruction
    constexpr int TB = kKvTile * ROWB;          // bytes of one K (or V) tile
    constexpr int WPB = BS < kRW ? 2 : 1;       // blocks behind one wave's kRW token rows
    static_assert(NI >= 1 && RPI <= BS && (WPB == 1 || 2 * BS == kRW), "tile shape");
    static_assert(!kQ || (kRW == 8 && WPB == 1 && kStages == 2), "quantized tiles: 8 rows per wave from one block, one tile ahead");
    static_assert(G == 1 || G == 4 || G == 8, "query heads per KV head");

    __shared__ __align__(16) unsigned char s_kv[kStages][2][TB];   // [stage][K, V][64 rows]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c32 = lane & 31, hi = lane >> 5;
    const int hq = a.hkv * G;
    // Work-groups are dealt to the 8 XCDs in turn (work-group i to XCD i % 8).  Work unit
    // u = (request, KV head) belongs to XCD u % 8, which runs its units in groups of ugrp side by
    // side, one group after another, the longest query tiles of the group first (the group's
    // units alternating): the work-groups resident on an XCD share one or two units' K/V in that
    // XCD's L2, a long request's heads go to different XCDs, and the last work-groups an XCD
    // starts are the group's shortest.
    const int xcd = static_cast<int>(blockIdx.x % 8);
    const int jx = static_cast<int>(blockIdx.x / 8);
    const int gw = a.qtiles * a.ugrp;                       // work-groups of one group of units
    const int jr = jx % gw;
    const int u = ((jx / gw) * a.ugrp + jr % a.ugrp) * 8 + xcd;
    if (u >= a.num_seqs * a.hkv) return;                 // the grid is rounded up to whole groups
    const int qt = a.qtiles - 1 - jr / a.ugrp;
    const int g = u % a.hkv;
    const int b = u / a.hkv;

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
    const int r = kWRows * w + c32;
    const int my_tok = min(t0q + r / G, n - 1);
    const int my_pos = ctx + my_tok;
    const int wave_min = ctx + min(t0q + (kWRows * w) / G, n - 1);
    const int wave_max = ctx + min(t0q + (kWRows * w + kWRows - 1) / G, n - 1);

    // q row as the B operand of product j: dims 16 j + 8 hi .. +7 (the A operand, K, reads the
    // same dims of its token row).  The scale's sign goes into q (negating bf16 values and
    // every score is exact), so the softmax always works with a positive factor in the
    // exponent; a zero scale becomes q = 0 (every visible token weighted equally).
    float sc = a.score_scale;
    float vsc = 1.0f;
    if constexpr (CDT == PA_DTYPE_FP8_E4M3) {
        sc *= __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gld_f32(a.k_scale + g))));
        vsc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gld_f32(a.v_scale + g))));
    }
    const float se = sc > 0.0f ? sc : sc < 0.0f ? -sc : 1.0f;
    const uint32_t qflip = sc < 0.0f ? 0x80008000u : 0u;
    const uint32_t qkeep = sc == 0.0f ? 0u : 0xffffffffu;
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
    U4 qb[NQK];
    {
        const uint16_t* qrow = qbase + (int64_t(q0 + my_tok) * hq + int64_t(g) * G + r % G) * D;
#pragma unroll
        for (int j = 0; j < NQK; ++j) {
            const U4 v = gld16(qrow + 16 * j + 8 * hi);
            qb[j] = U4{(v.x ^ qflip) & qkeep, (v.y ^ qflip) & qkeep, (v.z ^ qflip) & qkeep, (v.w ^ qflip) & qkeep};
        }
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

    // DMA layout: tile row R holds its chunk c at slot c ^ prefill_swz(R); lane `lane` of the
    // wave's instruction i fills position 64 i + lane of the wave's kRW-row slice
    uint32_t src_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int pos = 64 * i + lane, row = pos / CPR, slot = pos % CPR;
        src_off[i] = uint32_t(row) * ROWB + 16u * uint32_t(slot ^ prefill_swz<D>(kRW * w + row));
    }
    const int64_t blk_bytes = int64_t(a.hkv) * BS * ROWB;
    const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(a.k_cache) + int64_t(g) * BS * ROWB;
    const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(a.v_cache) + int64_t(g) * BS * ROWB;

    // quantized tiles: lane l loads row l / 8 of the wave's 8 rows, dims (D / 8) (l % 8) ..
    // + D / 8: fp8 D / 8 bytes; 4-bit D / 16 code bytes and the scale byte of their block
    constexpr int QCB = kMx ? D / 16 : D / 8;             // cache bytes per lane (codes)
    constexpr int64_t kQTile = kMx ? int64_t(BS) * (D / 2 + D / 32) : int64_t(BS) * D;   // (block, head) tile bytes
    const int qrow = lane >> 3, qcf = lane & 7;
    uint32_t qk[QCB / 4 > 0 ? QCB / 4 : 1], qv[QCB / 4 > 0 ? QCB / 4 : 1];   // pending codes (one tile ahead)
    uint32_t qks = 0, qvs = 0;                             // pending 4-bit scale bytes
    auto issue_q = [&](int k) {
        if ((k & 63) == 0 && k > 0) read_entries(k);
        const int b0 = __builtin_amdgcn_readlane(ent_a, k & 63);
        const int rib = (kKvTile * k + kRW * w) % BS + qrow;   // row inside the block
        const int64_t tbase = (int64_t(b0) * a.hkv + g) * kQTile;
        const unsigned char* kt = reinterpret_cast<const unsigned char*>(a.k_cache) + tbase;
        const unsigned char* vt = reinterpret_cast<const unsigned char*>(a.v_cache) + tbase;
        const uint32_t co = uint32_t(rib * (kMx ? D / 2 : D) + QCB * qcf);
        if constexpr (QCB == 16) {
            const U4 x = gld16(kt + co), y = gld16(vt + co);
            qk[0] = x.x; qk[1] = x.y; qk[2] = x.z; qk[3] = x.w;
            qv[0] = y.x; qv[1] = y.y; qv[2] = y.z; qv[3] = y.w;
        } else if constexpr (QCB == 8) {
            const uint2 x = gld8(kt + co), y = gld8(vt + co);
            qk[0] = x.x; qk[1] = x.y;
            qv[0] = y.x; qv[1] = y.y;
        } else {
            qk[0] = *(const PA_GLOBAL uint32_t*)(kt + co);
            qv[0] = *(const PA_GLOBAL uint32_t*)(vt + co);
        }
        if constexpr (kMx) {
            const uint32_t so = uint32_t(BS * (D / 2) + rib * (D / 32) + (qcf * (D / 8)) / 32);
            qks = gld_u8(kt + so);
            qvs = gld_u8(vt + so);
        }
    };
    // the pending rows of tile k, widened to bf16, into `stage`; rows past what this
    // work-group reads are zero.  The 8 lanes of a row are one phase of a 16-byte LDS write,
    // which collides on chunks equal modulo 128 bytes: lanes 4..7 of a row write their two
    // chunks in the other order from lanes 0..3 (on odd rows the other way round), so the 8 chunks
    // written together are 8 different positions modulo 128 bytes.
    auto store_q = [&](int k, int stage) {
        constexpr int NC = D / 64;                          // bf16 chunks per lane
        const int R = kRW * w + qrow;                       // tile row
        const bool live = kKvTile * k + R < kv_end;
        U4 ck[NC], cv[NC];
        if constexpr (kMx) {
            const float ksf = e8m0_to_f32(qks), vsf = e8m0_to_f32(qvs);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                ck[c] = e2m1x8_to_bf16(qk[c], ksf);
                cv[c] = e2m1x8_to_bf16(qv[c], vsf);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                uint32_t o[4];
                e4m3x8_to_bf16(qk[2 * c], qk[2 * c + 1], o);
                ck[c] = U4{o[0], o[1], o[2], o[3]};
                e4m3x8_to_bf16(qv[2 * c], qv[2 * c + 1], o);
                cv[c] = U4{o[0], o[1], o[2], o[3]};
            }
        }
        PA_LDS unsigned char* dk = (PA_LDS unsigned char*)&s_kv[stage][0][0] + R * ROWB;
        PA_LDS unsigned char* dv = (PA_LDS unsigned char*)&s_kv[stage][1][0] + R * ROWB;
        const int sw = prefill_swz<D>(R);
        const bool swap = NC == 2 && ((R ^ (qcf >> 2)) & 1);   // this lane writes its second chunk first
        auto sel = [&](const U4& x, const U4& y) {       // x, or y on a swapping lane (no indexing by lane)
            return U4{swap ? y.x : x.x, swap ? y.y : x.y, swap ? y.z : x.z, swap ? y.w : x.w};
        };
        auto keep = [&](const U4& x) { return live ? x : U4{0, 0, 0, 0}; };
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = NC == 2 ? (swap ? 1 - i : i) : i;
            const int slot = (NC * qcf + c) ^ sw;
            if constexpr (NC == 2) {
                lds_st16(dk + 16 * slot, keep(i == 0 ? sel(ck[0], ck[1]) : sel(ck[1], ck[0])));
                lds_st16(dv + 16 * slot, keep(i == 0 ? sel(cv[0], cv[1]) : sel(cv[1], cv[0])));
            } else {
                lds_st16(dk + 16 * slot, keep(ck[0]));
                lds_st16(dv + 16 * slot, keep(cv[0]));
            }
        }
    };

    auto issue = [&](int k, int bf) {
        if constexpr (kQ) {
            issue_q(k);
            (void)bf;
            return;
        }
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
        } else {   // the first BS rows from the first block, the rest from the second
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

    float m_ref = -INFINITY;                          // this lane's row, in scaled units
    f32x16v acc[NPV];                                 // out^T[32 t + 8 (i / 4) + 4 hi + i % 4][row]
#pragma unroll
    for (int t = 0; t < NPV; ++t) acc[t] = f32x16v{};
    float lsum = 0.0f;                                // this lane's part of the row's denominator
    const bf16x2v ones2 = __builtin_bit_cast(bf16x2v, 0x3f803f80u);

    // transpose-read addressing of the V^T operand: lane group l / 16 reads 4 token rows
    // (4 hi + (l % 16) / 4 of a 16-token step, then 8 more) at 4 dims of a 32-dim tile
    const int vrow = 4 * hi + ((lane & 15) >> 2);
    const int vchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vbyte = 8 * (lane & 1);
    // The swizzle depends on a row's low 4 bits only, so every lane's LDS offsets within a tile
    // are a per-lane part (below) plus a constant: K row 32 sb + c32 at dims 16 j + 8 hi; V rows
    // 32 sb + 16 h + vrow (+ 8) at dims 32 t + 4 (l % 4) + 16 ((l / 16) % 2)
    uint32_t ko[NQK], vo0[NPV], vo1[NPV];
#pragma unroll
    for (int j = 0; j < NQK; ++j) ko[j] = c32 * ROWB + 16 * ((2 * j + hi) ^ prefill_swz<D>(c32));
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
        vo0[t] = vrow * ROWB + 16 * ((4 * t + vchunk) ^ prefill_swz<D>(vrow)) + vbyte;
        vo1[t] = (vrow + 8) * ROWB + 16 * ((4 * t + vchunk) ^ prefill_swz<D>(vrow + 8)) + vbyte;
    }

    // V rows of tile k past what this work-group reads: zero (they may hold anything, and a
    // weight of 0 times a NaN would spoil a row)
    auto zero_tail = [&](int k, int stage) {
        if (kKvTile * (k + 1) <= kv_end) return;
        PA_LDS unsigned char* dv = (PA_LDS unsigned char*)&s_kv[stage][1][0] + kRW * w * ROWB;
        const int pos0 = kKvTile * k + kRW * w;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int p = 64 * i + lane;
            if (pos0 + p / CPR >= kv_end) lds_st16(dv + 16 * p, U4{0, 0, 0, 0});
        }
    };

#pragma unroll
    for (int k = 0; k < kStages - 1; ++k)
        if (k < ntiles) issue(k, k);
    int bf = 0;                                       // stage of tile k
    for (int k = 0; k < ntiles; ++k) {
        if constexpr (kQ) {
            store_q(k, bf);                           // this wave's rows of tile k, widened
        } else {
            if (kStages == 3 && k + 1 < ntiles) wait_vmem<2 * NI>();   // tile k + 1 may still be in flight
            else wait_vmem<0>();                      // this wave's rows of tile k have landed
            zero_tail(k, bf);
        }
        __syncthreads();                              // tile k complete; tile k - 1 no longer read
        if (k + kStages - 1 < ntiles) issue(k + kStages - 1, bf == 0 ? kStages - 1 : bf - 1);   // the stage of tile k - 1
        const int bf_cur = bf;
        bf = bf == kStages - 1 ? 0 : bf + 1;
        const PA_LDS unsigned char* kt = (const PA_LDS unsigned char*)&s_kv[bf_cur][0][0];
        const PA_LDS unsigned char* vt = (const PA_LDS unsigned char*)&s_kv[bf_cur][1][0];
        const int p_base = kKvTile * k;
        if (p_base > wave_max) continue;              // every row of this wave is before this tile
        const int nsb = min(2, (wave_max - p_base) / 32 + 1);   // 32-token halves with a visible token

        // scores of the tile's halves (independent chains of NQK products)
        auto scores = [&](int sb) {
            const PA_LDS unsigned char* kp = kt + 32 * sb * ROWB;
            f32x16v acc_s = f32x16v{};
            U4 kf[NQK];                                // every read in flight before the first product
#pragma unroll
            for (int j = 0; j < NQK; ++j) kf[j] = lds_ld16(kp + ko[j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NQK; ++j)
                acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, kf[j]),
                                                                __builtin_bit_cast(bf16x8v, qb[j]), acc_s, 0, 0, 0);
            return acc_s;
        };
        f32x16v s[2];
        if (nsb == 2) {
            // both halves' K operands read ahead of their products, the two chains interleaved
            U4 k0[NQK], k1[NQK];
#pragma unroll
            for (int j = 0; j < NQK; ++j) {
                k0[j] = lds_ld16(kt + ko[j]);
                k1[j] = lds_ld16(kt + 32 * ROWB + ko[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            s[0] = f32x16v{};
            s[1] = f32x16v{};
#pragma unroll
            for (int j = 0; j < NQK; ++j) {
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, k0[j]),
                                                               __builtin_bit_cast(bf16x8v, qb[j]), s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, k1[j]),
                                                               __builtin_bit_cast(bf16x8v, qb[j]), s[1], 0, 0, 0);
            }
        } else {
            s[0] = scores(0);
            s[1] = f32x16v{} - INFINITY;              // past every row of the wave
        }
        // causal mask (tiles that reach past the wave's first row only), then one online-softmax
        // update per tile: the maximum is taken on the raw scores and the scale is folded into
        // the exponent's fused multiply-add
        if (p_base + kKvTile - 1 > wave_min) {
            const int lim = my_pos - p_base - 4 * hi;     // register i of half sb is token 32 sb + 8 (i / 4) + i % 4 + 4 hi
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * sb + 8 * (i >> 2) + (i & 3) > lim) s[sb][i] = -INFINITY;
            }
        }
        float m8[8];                                  // a tree of maxima (independent chains)
#pragma unroll
        for (int i = 0; i < 8; ++i) m8[i] = vmax(vmax(s[0][2 * i], s[0][2 * i + 1]), vmax(s[1][2 * i], s[1][2 * i + 1]));
        float mx = vmax(vmax(vmax(m8[0], m8[1]), vmax(m8[2], m8[3])), vmax(vmax(m8[4], m8[5]), vmax(m8[6], m8[7])));
        mx = pair32_max(mx) * se;                     // the row's maximum over the tile, scaled
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first tile
            m_ref = m_new;
            lsum *= alpha;
#pragma unroll
            for (int t = 0; t < NPV; ++t) acc[t] *= alpha;
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            if (sb >= nsb) break;
            uint32_t pw[8];                           // weights rounded to bf16, in pairs (regs 2 e, 2 e + 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x2v pr;
                pr[0] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][2 * e], se, -m_ref)));
                pr[1] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][2 * e + 1], se, -m_ref)));
                lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lsum, false);
                pw[e] = __builtin_bit_cast(uint32_t, pr);
            }
            // out^T += V^T . P^T over the half's two 16-token steps: the B operand's 8 values of a
            // lane are its weights for tokens 4 hi + {0..3, 8..11} of the step (its registers
            // 8 h .. 8 h + 7), the A operand's are the same tokens' V values at dim 32 t + lane % 32
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8v pb = __builtin_bit_cast(bf16x8v, u32x4v{pw[4 * h], pw[4 * h + 1], pw[4 * h + 2], pw[4 * h + 3]});
                const PA_LDS unsigned char* vs = vt + (32 * sb + 16 * h) * ROWB;
#pragma unroll
                for (int t = 0; t < NPV; ++t) {
                    const i16x4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4v*)(vs + vo0[t]));
                    const i16x4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4v*)(vs + vo1[t]));
                    const i16x8v vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, vv), pb, acc[t], 0, 0, 0);
                }
            }
        }
    }


    // normalise the row and write it (rows past the request's new tokens are not written)
    const bool any_bad = __syncthreads_or(bad) || len_bad;
    const float denom = pair32_sum(lsum);
    const int tok = t0q + r / G;
    if (tok >= n) return;
    const float inv = any_bad ? __builtin_nanf("") : vsc / denom;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (int64_t(q0 + tok) * hq + int64_t(g) * G + r % G) * D;
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            bf16x2v lo, hi2;                              // round to nearest even (hardware conversion)
            lo[0] = static_cast<__bf16>(acc[t][4 * qd] * inv);
            lo[1] = static_cast<__bf16>(acc[t][4 * qd + 1] * inv);
            hi2[0] = static_cast<__bf16>(acc[t][4 * qd + 2] * inv);
            hi2[1] = static_cast<__bf16>(acc[t][4 * qd + 3] * inv);
            gst(reinterpret_cast<u32x2v*>(orow + 32 * t + 8 * qd + 4 * hi),
                u32x2v{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi2)});
        }
    }
}

template <int CDT, int D, int BS>
int launch_g(int G, const PrefillArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: hipLaunchKernelGGL((prefill_kernel<CDT, D, BS, 1>), grid, dim3(64 * pwaves(CDT)), 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<CDT, D, BS, 4>), grid, dim3(64 * pwaves(CDT)), 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<CDT, D, BS, 8>), grid, dim3(64 * pwaves(CDT)), 0, st, a); break;
        default: return fail(PA_ERR_UNSUPPORTED, "pa_prefill: %d query heads per KV head not in {1, 4, 8}", G);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "pa_prefill: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

template <int CDT, int D>
int launch_bs(int BS, int G, const PrefillArgs& a, dim3 grid, hipStream_t st) {
    switch (BS) {
        case 8: return launch_g<CDT, D, 8>(G, a, grid, st);
        case 16: return launch_g<CDT, D, 16>(G, a, grid, st);
        case 32: return launch_g<CDT, D, 32>(G, a, grid, st);
        case 128: return launch_g<CDT, D, 128>(G, a, grid, st);
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
                          int32_t q_dtype, int32_t cache_dtype, const float* k_scale, const float* v_scale,
                          void* stream) {
    pagedkv::clear_error();
    if (q_dtype != PA_DTYPE_BF16 ||
        (cache_dtype != PA_DTYPE_BF16 && cache_dtype != PA_DTYPE_FP8_E4M3 && cache_dtype != PA_DTYPE_MXFP4))
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: (q dtype %d, cache dtype %d) not supported (bf16 q; bf16, fp8 or 4-bit cache)",
                    q_dtype, cache_dtype);
    if (cache_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID, "pa_prefill: fp8 cache needs k_scale and v_scale");
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
    if (cache_dtype != PA_DTYPE_BF16 && block_size < 8)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d below 8", block_size);
    if (int64_t(max_blocks_per_seq) * block_size < max_seq_len)
        return fail(PA_ERR_INVALID, "pa_prefill: max_blocks_per_seq * block_size < max_seq_len");
    if (max_query_len > max_seq_len) return fail(PA_ERR_INVALID, "pa_prefill: max_query_len > max_seq_len");
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d not in {64, 128}", head_dim);
    const int G = num_q_heads / num_kv_heads;
    if (G != 1 && G != 4 && G != 8)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: %d query heads per KV head not in {1, 4, 8}", G);
    const int TQ = kWRows * pwaves(cache_dtype) / G;   // new tokens per work-group
    const int64_t qtiles = (int64_t(max_query_len) + TQ - 1) / TQ;
    const int64_t upx = (int64_t(num_seqs) * num_kv_heads + 7) / 8;          // (request, KV head) units per XCD
    const int ugrp = upx >= 2 ? 2 : 1;
    const int64_t units8 = (upx + ugrp - 1) / ugrp * ugrp * 8;    // units, whole groups on every XCD
    if (qtiles * units8 > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: grid of %lld work-groups", (long long)(qtiles * units8));

    PrefillArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_start = query_start;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.score_scale = scale * kLog2e;
    a.num_seqs = num_seqs;
    a.hkv = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.max_query_len = max_query_len;
    a.max_seq_len = max_seq_len;
    a.qtiles = static_cast<int>(qtiles);
    a.ugrp = ugrp;
    a.num_blocks = num_blocks;
    a.num_query_tokens = num_query_tokens;
    const dim3 grid(static_cast<unsigned>(qtiles * units8));
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (cache_dtype) {
        case PA_DTYPE_FP8_E4M3:
            return head_dim == 64 ? launch_bs<PA_DTYPE_FP8_E4M3, 64>(block_size, G, a, grid, st)
                                  : launch_bs<PA_DTYPE_FP8_E4M3, 128>(block_size, G, a, grid, st);
        case PA_DTYPE_MXFP4:
            return head_dim == 64 ? launch_bs<PA_DTYPE_MXFP4, 64>(block_size, G, a, grid, st)
                                  : launch_bs<PA_DTYPE_MXFP4, 128>(block_size, G, a, grid, st);
        default:
            return head_dim == 64 ? launch_bs<PA_DTYPE_BF16, 64>(block_size, G, a, grid, st)
                                  : launch_bs<PA_DTYPE_BF16, 128>(block_size, G, a, grid, st);
    }
}
