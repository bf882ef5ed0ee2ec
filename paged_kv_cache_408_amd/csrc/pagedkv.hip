// Paged KV cache kernels for AMD Instinct MI355X (gfx950, CDNA4) and their C ABI.
//
// What is computed is stated in include/pagedkv.h.  The pages behind it:
//  - "PagedAttention: Optimizing KV Cache Utilization in Large Language Models",
//    "The Mechanics of PagedAttention" (K/V written into scattered physical blocks through
//    a per-request page table) and "The Math: Block Attention Calculation"
//    (softmax(q.K^T / sqrt(d_k)) with K located through the page table);
//  - "KV Cache Optimization and PagedAttention" (fixed-size blocks, copy-on-write of
//    shared prefix blocks);
//  - "KV Cache Management", "What to Read Next" (8-bit KV cache).
//
// Kernels
//  kv_write_kernel       one lane per 8 elements of a (token, head) row; bit copy or fp8
//                        quantisation; slots < 0 or beyond the pool are skipped.
//  decode_mfma_kernel    bf16 and fp8 caches: one work-group (4 wave64) per (partition, KV
//                        head, request) work item; scores and P.V on the matrix cores with the
//                        query heads of a KV head padded to 16 (see its own comment).  Uniform
//                        batches use a (partition, KV head, request) grid; ragged ones a compact
//                        work-item list walked by about one work-group per resident slot.
//  decode_valu_kernel    f32 caches: the same passes with the contractions on the vector ALU
//                        (lanes per token row for q.k with DPP sums; one 16-byte vector per
//                        lane for P.V; weights handed over through LDS).
//  Both: the G = Hq/Hkv query heads of a KV head share every K/V load (each cached byte is
//  read once, non-temporally); a wave takes every 4th pass of 16 tokens with the next pass's
//  loads in flight (bf16: in an LDS ring filled by DMA loads); the online softmax rescales only when a score passes its reference by
//  2^8; the waves' states are merged in LDS; a single-partition request writes `out`,
//  otherwise the partition's (m, l, acc) goes to the workspace and the last work-group of the
//  (request, KV head) merges the partitions by log-sum-exp in the same launch (ticket
//  counters, agent-scope stores and loads).
//  zero_kernel           clears a workspace (a plain store kernel, no memset node).
//  copy_blocks_kernel    whole-block copies: copy-on-write inside a pool, and swapping blocks
//                        between the device pool and a pinned host pool (read and written
//                        over the host link by the kernel itself).
//  upload_kernel         a step's block-table rows, lengths and slots from pinned host memory
//                        to the device, read at system scope on the stream of the kernels that
//                        use them.
//
// Reduction order depends only on logical token positions (never on physical block ids),
// so results are bit-identical under any placement of the blocks.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <type_traits>

#include "pa_device.h"
#include "pa_layout.h"
#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

// Decode launch shape, fixed at build time: waves per work-group, K/V passes in flight per
// wave, and whether K/V are read with non-temporal loads (they are streamed exactly once).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 2
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
#ifndef PA_DECODE_STAGES
#define PA_DECODE_STAGES 2     // bf16 decode: 0 = K/V through registers; n >= 2 = n-stage LDS ring
                               // (2 keeps two work-groups per compute unit at D = 128)
#endif
#ifndef PA_DECODE_STAGES_FP8
#define PA_DECODE_STAGES_FP8 0 // the same for fp8 caches
#endif
constexpr int kWaves = PA_DECODE_WAVES;
constexpr int kThreads = 64 * kWaves;
// Waves per work-group of the matrix-core decode when it walks the compact item list (ragged
// batches).  Items there are short (a request's last partition, often a few hundred tokens),
// so each item's start -- the table read, then the first K/V loads -- is latency, not
// bandwidth.  Two-wave work-groups keep twice as many items in flight per compute unit as
// four-wave ones (4 work-groups instead of 2 at 256 VGPRs); the uniform grid, whose items are
// long, keeps kWaves.
constexpr int kListWaves = 2;
constexpr int kDepth = PA_DECODE_DEPTH;
constexpr bool kNonTemporal = PA_DECODE_NT != 0;
constexpr int kStagesBf16 = PA_DECODE_STAGES;
constexpr int kStagesFp8 = PA_DECODE_STAGES_FP8;
static_assert(kStagesBf16 == 0 || (kStagesBf16 >= 2 && kStagesBf16 <= 6), "LDS ring of 2 to 6 stages");
static_assert(kStagesFp8 == 0 || (kStagesFp8 >= 2 && kStagesFp8 <= 6), "LDS ring of 2 to 6 stages");
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves per work-group");
static_assert(kListWaves == 2 || kListWaves == 4, "2 or 4 waves per work-group on the item list");
static_assert(kDepth >= 2 && kDepth <= 4, "2 to 4 passes in flight");
constexpr int kMergeGroup = 16;   // partitions merged together at the first merge level


// ------------------------------------------------------------------ element formats

// float32 -> OCP E4M3FN code: round to nearest even, saturate to +-448, NaN -> 0x7F|sign.
// Normal range (|x| >= 2^-6): keep 3 mantissa bits of the binary32 pattern with a
// round-half-even carry that may ripple into the exponent, then rebias 127 -> 7.
// Subnormal range (|x| < 2^-6): the code is |x| / 2^-9 rounded half-even (v_rndne_f32).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;         // >= 448 (and inf): saturate
    if (a < 0x3c800000u) {                             // < 2^-6: multiples of 2^-9
        const float qv = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | static_cast<uint32_t>(qv);
    }
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // (exp127 << 3) | m3, rounded
    return sign | (r - (120u << 3));
}

// Two E4M3FN codes (bytes 0/1 or 2/3 of w) -> float32, exact.
template <bool HI>
__device__ __forceinline__ float2v e4m3x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
}


// 16-byte load of cached K/V: non-temporal when configured (read once, never reused).
__device__ __forceinline__ U4 ld16_stream(const void* p) {
    if constexpr (kNonTemporal) {
        const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
        return U4{v[0], v[1], v[2], v[3]};
    } else {
        return ld16(p);
    }
}

__device__ __forceinline__ U4 gld16_stream(const void* p) {
    const PA_GLOBAL u32x4v* gp = (const PA_GLOBAL u32x4v*)p;
    const u32x4v v = kNonTemporal ? __builtin_nontemporal_load(gp) : *gp;
    return U4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint32_t u4_get(const U4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ------------------------------------------------------------------ KV write

template <int IDT, int CDT>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const typename Elem<IDT>::T* __restrict__ k, const typename Elem<IDT>::T* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t num_tokens, typename Elem<CDT>::T* __restrict__ kc,
    typename Elem<CDT>::T* __restrict__ vc, int64_t num_slots, int hkv, int d, int bs,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
    using IT = typename Elem<IDT>::T;
    const int per_row = d / 8;  // lanes per (token, head) row, 8 elements each
    const int64_t total = num_tokens * hkv * per_row;
    for (int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; gid < total;
         gid += int64_t(gridDim.x) * blockDim.x) {
        const int64_t row = gid / per_row;
        const int col = static_cast<int>(gid - row * per_row) * 8;
        const int64_t t = row / hkv;
        const int h = static_cast<int>(row - t * hkv);
        const int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        const int64_t blk = s / bs, r = s - blk * bs;
        const int64_t src = row * d + col;
        const int64_t dst = ((blk * hkv + h) * bs + r) * d + col;
        if constexpr (CDT == IDT) {
            // bit copy of 8 elements (16 or 32 bytes)
            constexpr int nvec = 8 * sizeof(IT) / 16;
#pragma unroll
            for (int i = 0; i < nvec; ++i) {
                reinterpret_cast<U4*>(kc + dst)[i] = reinterpret_cast<const U4*>(k + src)[i];
                reinterpret_cast<U4*>(vc + dst)[i] = reinterpret_cast<const U4*>(v + src)[i];
            }
        } else {
            static_assert(CDT == PA_DTYPE_FP8_E4M3 && (IDT == PA_DTYPE_BF16 || IDT == PA_DTYPE_F32), "unsupported pair");
            const float ks = k_scale[h], vs = v_scale[h];
            float kf[8], vf[8];
            if constexpr (IDT == PA_DTYPE_BF16) {
                const U4 kx = ld16(k + src), vx = ld16(v + src);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t kw = u4_get(kx, i / 2), vw = u4_get(vx, i / 2);
                    kf[i] = bf16_to_f32((i & 1) ? (kw >> 16) : (kw & 0xffffu));
                    vf[i] = bf16_to_f32((i & 1) ? (vw >> 16) : (vw & 0xffffu));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const U4 kx = ld16(k + src + 4 * j), vx = ld16(v + src + 4 * j);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        kf[4 * j + i] = __uint_as_float(u4_get(kx, i));
                        vf[4 * j + i] = __uint_as_float(u4_get(vx, i));
                    }
                }
            }
            uint32_t ko[2] = {0, 0}, vo[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // correctly rounded float32 quotient (IEEE division, no fast-math)
                const uint32_t kq = f32_to_e4m3(kf[i] / ks);
                const uint32_t vq = f32_to_e4m3(vf[i] / vs);
                ko[i / 4] |= kq << (8 * (i % 4));
                vo[i / 4] |= vq << (8 * (i % 4));
            }
            uint2* kd = reinterpret_cast<uint2*>(kc + dst);
            uint2* vd = reinterpret_cast<uint2*>(vc + dst);
            *kd = make_uint2(ko[0], ko[1]);
            *vd = make_uint2(vo[0], vo[1]);
        }
    }
}

// One MXFP4 block: 32 bf16 values (16 dwords) -> 16 code bytes (element 0 in the low nibble)
// and the E8M0 scale byte.  E = floor(log2(max |x|)) - 2 from the exponent field of the largest
// magnitude (bf16 magnitudes order like their bit patterns), clamped to -127; x / 2^E is exact
// (a power-of-two scaling that stays below 8) wherever it reaches the rounding thresholds.
// Round to nearest even on the E2M1 grid with saturation: the code counts the thresholds
// passed, a tie going to the neighbour whose mantissa bit is 0.
__device__ __forceinline__ void mx4_quantize(const uint32_t (&x)[16], uint32_t (&codes)[4], uint32_t& scale) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, max(x[i] & 0x7fffu, (x[i] >> 16) & 0x7fffu));
    if (amax >= 0x7f80u) {                                // NaN or infinity in the block
        scale = 0xffu;
        codes[0] = codes[1] = codes[2] = codes[3] = 0u;
        return;
    }
    const int eb = int(amax >> 7);                        // exponent field of the largest magnitude
    const int E = eb == 0 ? -127 : max(eb - 127 - 2, -127);
    const float inv = __uint_as_float(uint32_t(127 - E) << 23);   // 2^-E (E <= 125)
    scale = uint32_t(E + 127);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t word = x[4 * w + e / 2];
            const uint32_t b = (e & 1) ? (word >> 16) : (word & 0xffffu);
            const float a = bf16_to_f32(b & 0x7fffu) * inv;
            uint32_t q = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                         uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
            q |= (b >> 12) & 0x8u;                        // sign
            c |= q << (4 * e);
        }
        codes[w] = c;
    }
}

// MXFP4 write: one lane per (token, KV head, block of 32 dims) for K and for V.
__global__ __launch_bounds__(256) void kv_write_mx4_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const int64_t* __restrict__ slots, int64_t num_tokens,
                                                           uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                           int64_t num_slots, int hkv, int d, int bs) {
    const int groups = d / 32;
    const int64_t tile = int64_t(bs) * (d / 2 + d / 32);    // bytes of one (block, head) tile
    const int64_t total = num_tokens * hkv * groups;
    for (int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; gid < total;
         gid += int64_t(gridDim.x) * blockDim.x) {
        const int64_t row = gid / groups;                   // (token, head)
        const int gi = static_cast<int>(gid - row * groups);
        const int64_t t = row / hkv;
        const int h = static_cast<int>(row - t * hkv);
        const int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        const int64_t blk = s / bs, r = s - blk * bs;
        const int64_t base = (blk * hkv + h) * tile;
        const int64_t code_off = base + r * (d / 2) + gi * 16;
        const int64_t scale_off = base + int64_t(bs) * (d / 2) + r * groups + gi;
        const int64_t src = row * d + gi * 32;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const uint16_t* x = kv ? v : k;
            uint8_t* cache = kv ? vc : kc;
            uint32_t words[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const U4 u = ld16(x + src + 8 * i);
                words[4 * i] = u.x;
                words[4 * i + 1] = u.y;
                words[4 * i + 2] = u.z;
                words[4 * i + 3] = u.w;
            }
            uint32_t codes[4], scale;
            mx4_quantize(words, codes, scale);
            *reinterpret_cast<U4*>(cache + code_off) = U4{codes[0], codes[1], codes[2], codes[3]};
            cache[scale_off] = static_cast<uint8_t>(scale);
        }
    }
}

// ------------------------------------------------------------------ block copy

// Whole-block copies from one pool to another (or within one pool: copy-on-write).  Either
// pool may be pinned host memory, which the loads and stores reach over the host link.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* dk, uint8_t* dv, const uint8_t* sk,
                                                          const uint8_t* sv, const int64_t* __restrict__ pairs,
                                                          int num_pairs, int64_t src_blocks, int64_t dst_blocks,
                                                          int64_t block_bytes) {
    const int64_t vec_per_block = block_bytes / 16;
    const int64_t total = int64_t(num_pairs) * vec_per_block;
    for (int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; gid < total;
         gid += int64_t(gridDim.x) * blockDim.x) {
        const int64_t pi = gid / vec_per_block;
        const int64_t off = (gid - pi * vec_per_block) * 16;
        const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
        const U4 k = ld16(sk + src * block_bytes + off);
        const U4 v = ld16(sv + src * block_bytes + off);
        *reinterpret_cast<U4*>(dk + dst * block_bytes + off) = k;
        *reinterpret_cast<U4*>(dv + dst * block_bytes + off) = v;
    }
}

// Host -> device copy of a step's block-table rows, lengths and slots (pa_upload): 16-byte
// loads at system scope (sc0 sc1), which bypass the device caches and so see what the host
// wrote to pinned memory before the launch; plain stores.  One kernel on the caller's stream
// keeps the copy on the queue of the kernels that read the result.
__global__ __launch_bounds__(256) void upload_kernel(uint8_t* __restrict__ dst, const uint8_t* src, int n16) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, n16 * 16, 0x00020000);
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n16; i += gridDim.x * 256) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, 17);   // sc0 | sc1
        *(PA_GLOBAL u32x4v*)(dst + int64_t(i) * 16) = u32x4v{v[0], v[1], v[2], v[3]};
    }
}

// ------------------------------------------------------------------ decode: layout

template <int CDT, int D, int BS, int G>
struct Cfg {
    static constexpr int E = Elem<CDT>::bytes;
    static constexpr int EPV = 16 / E;                  // elements per 16-byte vector
    static constexpr int ROW_VECS = D / EPV;            // vectors per token row
    static constexpr int K_TARGET = CDT == PA_DTYPE_BF16 ? 32 : 16;
    static constexpr int KVPL = (K_TARGET / EPV) < (ROW_VECS / 4) ? (K_TARGET / EPV) : (ROW_VECS / 4);
    static constexpr int KL = ROW_VECS / KVPL;          // lanes per row, K phase
    static constexpr int TPP = 64 / KL;                 // tokens per pass
    static constexpr int EPL = KVPL * EPV;              // K elements per lane
    static constexpr int VL = ROW_VECS;                 // lanes per row, V phase
    static constexpr int VRG = 64 / VL;                 // row groups, V phase
    static constexpr int VR = TPP / VRG;                // V rows per lane per pass
    static constexpr int BPP = TPP > BS ? TPP / BS : 1; // blocks touched by one pass
    static_assert(KVPL >= 1 && KL >= 4 && KL <= 8 && VR >= 1, "layout");
    static_assert(BPP <= 2, "a pass spans at most two blocks");
};

// Partition granule: a multiple of every layout's 4 * TPP (32 or 64 tokens) and of the
// block size, so partitions start on pass and block boundaries.
inline int partition_unit(int block_size) { return block_size > 64 ? block_size : 64; }

// Compute units of the current device (cached per device; 256 if it cannot be queried).
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();   // leave no sticky error for the next launch check
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Partition size in tokens.  An explicit request is rounded up to the granule.  Automatic
// (requested == 0): one work-group per compute unit -- with fewer (request, KV head) pairs
// than compute units, each request is cut into ceil(CUs / pairs) equal partitions of
// ceil(max_seq_len / parts) tokens; with at least as many pairs as compute units, long
// requests are cut into partitions of kAutoRaggedPartition tokens so that no single
// work-group holds a long tail.
constexpr int kAutoRaggedPartition = 512;

int64_t resolve_partition(int64_t num_seqs, int64_t hkv, int64_t max_seq_len, int requested, int block_size,
                          int cache_dtype) {
    const int64_t unit = partition_unit(block_size);
    int64_t pt;
    if (requested > 0) {
        pt = requested;
    } else {
        // compressed caches (fp8, 4-bit) are bound by the per-pass work, not by the bytes, and
        // gain from two resident work-groups per compute unit; bf16 streams best with one
        const int64_t per_cu = (cache_dtype == PA_DTYPE_FP8_E4M3 || cache_dtype == PA_DTYPE_MXFP4) ? 2 : 1;
        const int64_t pairs = num_seqs * hkv;
        const int64_t slots = per_cu * device_cu_count();
        if (pairs >= slots) {
            pt = kAutoRaggedPartition;
        } else {
            const int64_t parts = (slots + pairs - 1) / pairs;
            pt = (max_seq_len + parts - 1) / parts;
        }
    }
    pt = (pt + unit - 1) / unit * unit;
    return pt < unit ? unit : pt;
}

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const float* k_scale;
    const float* v_scale;
    const void* k_new;     // pa_decode_append: each request's new token's K and V rows (q's dtype), else null
    const void* v_new;
    int* ws_ctr;           // merge tickets, ctr_stride per (request, KV head): one per group of partitions
                           // (level 1), the last one for the groups (level 2); zero between calls
    float* ws_m;           // level-1 partials: one row per (request, q head, partition)
    float* ws_l;
    float* ws_acc;
    float* ws_m2;          // level-2 partials: one row per (request, q head, group of partitions)
    float* ws_l2;
    float* ws_acc2;
    float score_scale;     // scale * log2(e)
    int list;              // 1: grid walks the compact item list (dynamic LDS: num_seqs + 1 ints)
    int num_seqs;
    int hkv;
    int64_t num_blocks;
    int max_blocks;
    int max_seq_len;
    int part_tokens;
    int max_parts;
    int ctr_stride;        // tickets (and level-2 rows) per (request, KV head): a bound on the merge groups
                           // of any partition size, plus one
};

// ------------------------------------------------------------------ decode: partitions and merge

__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer view of a float array for agent-scope (sc1) vector loads; out-of-range reads
// return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_view(const float* base, int64_t n_floats) {
    const int64_t bytes = n_floats * 4;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0,
                                             static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes), 0x00020000);
}

// Column layout shared by finish_partition and merge_rows: the G x D outputs of a (request, KV
// head) as NC float4 columns (head h = col / (D / 4), dims 4 (col % (D / 4)) .. + 3).  Thread t
// of an NT-thread work-group takes column t % NC (row slice t / NC) or, when the columns
// outnumber the threads, columns cb NT + t for its NCB column batches cb.
template <int D, int G, int NT>
struct MergeCols {
    static constexpr int NC = G * D / 4;                 // float4 columns
    static constexpr int NS = NT / NC > 0 ? NT / NC : 1; // row slices (1 when columns outnumber threads)
    static constexpr int NCB = NC > NT ? NC / NT : 1;    // column batches per thread
    static_assert(NC <= NT || NC % NT == 0, "whole column batches");
    __device__ static int col(int t, int cb) { return NC > NT ? cb * NT + t : t % NC; }
    __device__ static int slice(int t) { return NC > NT ? 0 : t / NC; }
};

// A work-group's own partial row, per column batch of the thread: the same floats it would have
// written to the workspace (max, sum, accumulator slice).
template <int NCB>
struct OwnRow {
    float m[NCB], l[NCB];
    float4 acc[NCB];
};

// Log-sum-exp merge of `count` consecutive partial rows (m, l, acc[D]) of each of the G heads
// of one (request, KV head): head h's rows are row0 + h * head_stride + [0, count).  The block's
// threads take float4 columns of the G x D outputs (MergeCols) and split the rows among
// themselves; each keeps an online (max, sum, accumulator) state, and the slices are combined
// in LDS.  Row own_r (if >= 0) is not read from memory: its values are the calling
// work-group's own, passed in registers, and are merged at the same place in the same order,
// so the result is the same bits either way.  A NaN max in any row (a bad block id) makes the
// result NaN.  Writes `out` (rounded) or, when out == nullptr, one partial row per head to
// (m_dst, l_dst, acc_dst) with the given head stride, by agent-scope stores.
template <int QDT, int D, int G, int NT>
__device__ __forceinline__ void merge_rows(const float* m_src, const float* l_src, const float* acc_src, int64_t row0,
                           int64_t head_stride, int count, typename Elem<QDT>::T* out, float* m_dst, float* l_dst,
                           float* acc_dst, int64_t dst_head_stride, int own_r,
                           const OwnRow<MergeCols<D, G, NT>::NCB>& own) {
    using MC = MergeCols<D, G, NT>;
    constexpr int NC = MC::NC, NS = MC::NS, NCB = MC::NCB;
    __shared__ float s_mm[NS][NC], s_ll[NS][NC];
    __shared__ float4 s_num[NS][NC];
    const int t = threadIdx.x;
    for (int cb = 0; cb < NCB; ++cb) {
    const int col = MC::col(t, cb), slice = MC::slice(t);
    const int h = col / (D / 4), c4 = col % (D / 4);
    const bool active = slice < NS;
    float M = -INFINITY, den = 0.0f;
    float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool nan_seen = false;
    if (active) {
        const int64_t rh = row0 + int64_t(h) * head_stride;     // rows rh .. rh + count - 1
        const auto racc = coherent_view(acc_src + rh * D, int64_t(count) * D);
        for (int r = slice; r < count; r += NS) {
            float mr, lr;
            float4 v;
            if (r == own_r) {
                mr = own.m[cb];
                lr = own.l[cb];
                v = own.acc[cb];
            } else {
                mr = load_agent(m_src + rh + r);
                lr = load_agent(l_src + rh + r);
                const auto vi = __builtin_amdgcn_raw_buffer_load_b128(racc, (r * D + c4 * 4) * 4, 0, 16);
                v = make_float4(__int_as_float(vi[0]), __int_as_float(vi[1]), __int_as_float(vi[2]), __int_as_float(vi[3]));
            }
            nan_seen |= __builtin_isnan(mr);
            if (mr > M) {   // new maximum: rescale the state (exp2(-inf) = 0 on the first row)
                const float f = __builtin_amdgcn_exp2f(M - mr);
                den *= f;
                num.x *= f; num.y *= f; num.z *= f; num.w *= f;
                M = mr;
            }
            const float wgt = __builtin_amdgcn_exp2f(mr - M);
            den = fmaf(wgt, lr, den);
            num.x = fmaf(wgt, v.x, num.x);
            num.y = fmaf(wgt, v.y, num.y);
            num.z = fmaf(wgt, v.z, num.z);
            num.w = fmaf(wgt, v.w, num.w);
        }
        if (nan_seen) M = __builtin_nanf("");
        s_mm[slice][col] = M;
        s_ll[slice][col] = den;
        s_num[slice][col] = num;
    }
    __syncthreads();
    if (slice != 0) return;
    float Mt = s_mm[0][col];
    bool nan_any = __builtin_isnan(Mt);
#pragma unroll
    for (int sl = 1; sl < NS; ++sl) {
        nan_any |= __builtin_isnan(s_mm[sl][col]);
        Mt = fmaxf(Mt, s_mm[sl][col]);
    }
    float dt = 0.0f;
    float4 nt = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        const float f = __builtin_amdgcn_exp2f(s_mm[sl][col] - Mt);   // 0 for an empty slice
        dt = fmaf(f, s_ll[sl][col], dt);
        const float4 v = s_num[sl][col];
        nt.x = fmaf(f, v.x, nt.x); nt.y = fmaf(f, v.y, nt.y); nt.z = fmaf(f, v.z, nt.z); nt.w = fmaf(f, v.w, nt.w);
    }
    if (nan_any) { Mt = dt = __builtin_nanf(""); }
    if (out != nullptr) {
        const float o[4] = {nt.x / dt, nt.y / dt, nt.z / dt, nt.w / dt};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (QDT == PA_DTYPE_BF16) out[h * D + c4 * 4 + e] = f32_to_bf16(o[e]);
            else out[h * D + c4 * 4 + e] = o[e];
        }
    } else {
        float* ad = acc_dst + int64_t(h) * dst_head_stride * D + c4 * 4;
        store_agent(ad + 0, nt.x);
        store_agent(ad + 1, nt.y);
        store_agent(ad + 2, nt.z);
        store_agent(ad + 3, nt.w);
        if (c4 == 0) {
            store_agent(m_dst + int64_t(h) * dst_head_stride, Mt);
            store_agent(l_dst + int64_t(h) * dst_head_stride, dt);
        }
    }
    }   // column batches
}

// End of one partition of one (request, KV head): merges the waves' states held in LDS
// (m[w][h], l[w][h] and acc[w][h][d] at acc + w * acc_wave_stride; scores in log2 units, acc
// unnormalised; the acc area is then reused to stage the partial row) into this work-group's own partial (max, sum, accumulator), in registers in
// the merge's column layout, then writes `out` when the request has a single partition, or
// else takes part in the log-sum-exp merge of the request's partitions, in up to two levels:
// the last of each group of kMergeGroup partitions merges that group; with more than one
// group, the last group-merger then merges the groups.
// A work-group learns that it is its group's last in one of two ways:
//  - the group's ticket, read (agent scope) while the waves' states are merged, already counts
//    every other member: it merges at once, with its own row from registers, and writes no
//    partial and takes no ticket (every other member has taken its ticket and will not touch
//    the counter again, so it resets it);
//  - otherwise it writes its partial row with agent-scope stores (coherent across the XCDs'
//    L2s), drains the store counter so that they are visible at agent scope, and takes a
//    ticket; the member that draws the last one merges, reading the others' rows with
//    agent-scope loads.
// Both paths merge the same rows in the same order with the same values, so the output does not
// depend on which one ran.  The first is taken only where EARLY is set (bf16 caches: measured
// 1% faster on the Llama-shaped layer and 2% on the ragged batch; with it, fp8 caches were 5%
// slower on the ragged batch, whose many short items mostly end up on the second path and then
// pay the ticket read too, and 4-bit caches 3-7% slower on both workloads).  No work-group waits for another, and no agent-scope fence (whose L2
// write-back/invalidate would serialise the work-groups of an XCD) is used.  Counters are left
// at zero.  Work-group uniform; ends with a barrier, so the caller may reuse the LDS arrays
// afterwards.
template <int QDT, int D, int G, int NW, bool EARLY>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, int b, int g, int part, int nparts, float vsc, bool any_bad,
                                 const float* s_m, const float* s_l, float* s_acc, int acc_wave_stride) {
    using QT = typename Elem<QDT>::T;
    constexpr int NT = 64 * NW;
    using MC = MergeCols<D, G, NT>;
    constexpr int NC = MC::NC, NCB = MC::NCB;
    __shared__ int s_last;
    const int hq = a.hkv * G;
    QT* out = reinterpret_cast<QT*>(a.out) + (int64_t(b) * hq + int64_t(g) * G) * D;
    const bool single = nparts == 1;
    const int ngroups = (nparts + kMergeGroup - 1) / kMergeGroup;
    const int grp = part / kMergeGroup;
    const int first = grp * kMergeGroup, count = min(kMergeGroup, nparts - first);
    const int64_t bg = int64_t(b) * a.hkv + g;
    int* ctr = a.ws_ctr + bg * a.ctr_stride + grp;
    int seen = 0;
    if (EARLY && !single && threadIdx.x == 0) seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const int t = threadIdx.x;
    OwnRow<NCB> own;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = MC::col(t, cb);
        const int h = col / (D / 4), c4 = col % (D / 4);
        float M = s_m[h];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_m[ww * G + h]);
        float den = 0.0f;
        float num[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float f = __builtin_amdgcn_exp2f(s_m[ww * G + h] - M);   // 0 for an idle wave
            const float* src = s_acc + ww * acc_wave_stride + h * D + 4 * c4;
#pragma unroll
            for (int e = 0; e < 4; ++e) num[e] = fmaf(f, src[e], num[e]);
            den = fmaf(f, s_l[ww * G + h], den);
        }
        if (any_bad) {
#pragma unroll
            for (int e = 0; e < 4; ++e) num[e] = __builtin_nanf("");
            den = __builtin_nanf("");
            M = __builtin_nanf("");
        }
        if (single) {
            if (NC > NT || t < NC) {   // one thread per column
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float o = num[e] / den * vsc;
                    if constexpr (QDT == PA_DTYPE_BF16) gst(out + h * D + 4 * c4 + e, f32_to_bf16(o));
                    else gst(out + h * D + 4 * c4 + e, o);
                }
            }
        } else {
            own.m[cb] = M;
            own.l[cb] = den;
            own.acc[cb] = make_float4(num[0] * vsc, num[1] * vsc, num[2] * vsc, num[3] * vsc);
        }
    }
    if (single) {
        __syncthreads();
        return;
    }
    bool early = false;
    if constexpr (EARLY) {
        if (threadIdx.x == 0) s_last = seen == count - 1;
        __syncthreads();
        early = s_last;
        __syncthreads();             // s_last is rewritten below
    }
    if (early) {
        if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // the partial row, written by consecutive lanes to consecutive floats (whole 64-byte
        // segments per store): staged through the waves' state area, which no thread reads
        // once every thread has passed this barrier
        __syncthreads();
        float* stage = s_acc;
        __shared__ float s_om[G], s_ol[G];
        if (NC > NT || t < NC) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int col = MC::col(t, cb);
                const int h = col / (D / 4), c4 = col % (D / 4);
                float* p = stage + h * D + 4 * c4;
                p[0] = own.acc[cb].x;
                p[1] = own.acc[cb].y;
                p[2] = own.acc[cb].z;
                p[3] = own.acc[cb].w;
                if (c4 == 0) {
                    s_om[h] = own.m[cb];
                    s_ol[h] = own.l[cb];
                }
            }
        }
        __syncthreads();
        for (int idx = t; idx < G * D; idx += NT) {
            const int h = idx / D, dim = idx - h * D;
            const int64_t row = (int64_t(b) * hq + int64_t(g) * G + h) * a.max_parts + part;
            store_agent(a.ws_acc + row * D + dim, stage[idx]);
            if (dim == 0) {
                store_agent(a.ws_m + row, s_om[h]);
                store_agent(a.ws_l + row, s_ol[h]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            const int ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = ticket == count - 1;
            if (s_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const bool merge1 = s_last;
        __syncthreads();             // s_last is rewritten below
        if (!merge1) return;
    }
    const int64_t rows1 = (int64_t(b) * hq + int64_t(g) * G) * a.max_parts;    // head h: + h * max_parts
    if (ngroups == 1) {
        merge_rows<QDT, D, G, NT>(a.ws_m, a.ws_l, a.ws_acc, rows1 + first, a.max_parts, count, out, nullptr, nullptr,
                                  nullptr, 0, part - first, own);
        __syncthreads();
        return;
    }
    const int64_t rows2 = (int64_t(b) * hq + int64_t(g) * G) * a.ctr_stride;
    merge_rows<QDT, D, G, NT>(a.ws_m, a.ws_l, a.ws_acc, rows1 + first, a.max_parts, count, nullptr, a.ws_m2 + rows2 + grp,
                              a.ws_l2 + rows2 + grp, a.ws_acc2 + (rows2 + grp) * D, a.ctr_stride, part - first, own);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        int* ctr2 = a.ws_ctr + bg * a.ctr_stride + (a.ctr_stride - 1);
        const int ticket = __hip_atomic_fetch_add(ctr2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = ticket == ngroups - 1;
        if (s_last) __hip_atomic_store(ctr2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const bool merge2 = s_last;
    __syncthreads();
    if (!merge2) return;
    merge_rows<QDT, D, G, NT>(a.ws_m2, a.ws_l2, a.ws_acc2, rows2, a.ctr_stride, ngroups, out, nullptr, nullptr, nullptr, 0,
                              -1, own);
    __syncthreads();
}

template <int CDT, int QDT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(const DecodeArgs a) {
    using C = Cfg<CDT, D, BS, G>;
    using CT = typename Elem<CDT>::T;
    using QT = typename Elem<QDT>::T;
    constexpr bool kDot2 = CDT == PA_DTYPE_BF16;   // bf16 cache: v_dot2 on packed pairs
    constexpr int KL = C::KL, TPP = C::TPP, EPV = C::EPV, KVPL = C::KVPL, VL = C::VL, VRG = C::VRG,
                  VR = C::VR, BPP = C::BPP;

    __shared__ float s_p[kWaves][TPP][G];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ float s_acc[kWaves][G][D];

    const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform per wave
    const int hq = a.hkv * G;
    const int t0 = part * a.part_tokens;
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;

    // ---- block ids of this wave's passes, 64 at a time: lane j holds the first (and for
    // BPP == 2 the second) block of pass w + kWaves * (k0 + j).  The table is read before the
    // request's length is known (indexes clamped to the row), so its latency overlaps the
    // length's; `check_entries` then flags ids outside the pool inside the live range and
    // replaces every such id by 0, so every address stays inside the cache.
    int ent_a = 0, ent_b = 0;
    auto read_entries = [&](int k0) {
        const int e = (t0 + (w + kWaves * (k0 + lane)) * TPP) / BS;
        ent_a = a.max_blocks > 0 ? table[min(e, a.max_blocks - 1)] : -1;
        if constexpr (BPP == 2) ent_b = a.max_blocks > 0 ? table[min(e + 1, a.max_blocks - 1)] : -1;
    };
    read_entries(0);

    // ---- q slice of this lane (K-phase layout): vectors j*KL + kc of the row
    const int krow = lane / KL, kc = lane % KL;
    const QT* qrow = reinterpret_cast<const QT*>(a.q) + (int64_t(b) * hq + int64_t(g) * G) * D;
    uint32_t qpk[kDot2 ? G : 1][kDot2 ? C::EPL / 2 : 1];
    float qf[kDot2 ? 1 : G][kDot2 ? 1 : C::EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int j = 0; j < KVPL; ++j) {
            const int d0 = (j * KL + kc) * EPV;
            if constexpr (kDot2) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(qrow + h * D + d0);
#pragma unroll
                for (int e = 0; e < EPV / 2; ++e) qpk[h][j * (EPV / 2) + e] = src[e];
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const QT x = qrow[h * D + d0 + e];
                    if constexpr (QDT == PA_DTYPE_BF16) qf[h][j * EPV + e] = bf16_to_f32(x);
                    else qf[h][j * EPV + e] = x;
                }
            }
        }
    }

    const int L_raw = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    const bool len_bad = L_raw < 0 || L_raw > a.max_seq_len || L_raw > a.max_blocks * BS;
    const int L = len_bad ? 0 : L_raw;
    const int nparts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
    if (part >= nparts) return;

    QT* out = reinterpret_cast<QT*>(a.out) + (int64_t(b) * hq + int64_t(g) * G) * D;
    if (L == 0) {   // empty request (zeros) or invalid length (NaN); single partition
        const float fill = len_bad ? __builtin_nanf("") : 0.0f;
        for (int i = threadIdx.x; i < G * D; i += kThreads) {
            if constexpr (QDT == PA_DTYPE_BF16) out[i] = f32_to_bf16(fill); else out[i] = fill;
        }
        return;
    }

    const int t1 = min(L, t0 + a.part_tokens);
    const int npass = (t1 - t0 + TPP - 1) / TPP;
    const int nk = npass > w ? (npass - w + kWaves - 1) / kWaves : 0;   // passes w, w+kWaves, ...
    const CT* kbase = reinterpret_cast<const CT*>(a.k_cache);
    const CT* vbase = reinterpret_cast<const CT*>(a.v_cache);
    const int64_t head_tile = int64_t(g) * (BS * D);
    const int64_t block_stride = int64_t(a.hkv) * (BS * D);

    float sc = a.score_scale;
    float vsc = 1.0f;
    if constexpr (CDT == PA_DTYPE_FP8_E4M3) {
        sc *= a.k_scale[g];
        vsc = a.v_scale[g];
    }

    float m_ref[G], l_run[G], acc[G][EPV];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_ref[h] = -INFINITY;
        l_run[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[h][e] = 0.0f;
    }
    bool bad = false;
    const int vrg = lane / VL, vcol = lane % VL;

    auto check_entries = [&](int k0) {
        const int kk = k0 + lane;
        const bool live = kk < nk;
        if (ent_a < 0 || ent_a >= a.num_blocks) {
            if (live) bad = true;
            ent_a = 0;
        }
        if constexpr (BPP == 2) {
            const int e = (t0 + (w + kWaves * kk) * TPP) / BS;
            if (ent_b < 0 || ent_b >= a.num_blocks) {
                if (live && (e + 1) * BS < t1) bad = true;
                ent_b = 0;
            }
        }
    };
    check_entries(0);

    // ---- issue the K and V loads of pass k (no masking: rows past the end still lie in a
    // valid block; their contributions are masked in compute)
    auto issue = [&](int k, U4 (&kb)[KVPL], U4 (&vb)[VR]) {
        if ((k & 63) == 0 && k > 0) {
            read_entries(k);
            check_entries(k);
        }
        const int tb = t0 + (w + kWaves * k) * TPP;
        const int b0 = __builtin_amdgcn_readlane(ent_a, k & 63);
        const int b1 = BPP == 2 ? __builtin_amdgcn_readlane(ent_b, k & 63) : b0;
        const int row0 = BPP == 2 ? 0 : tb % BS;
        {
            const int blk = (BPP == 2 && krow >= BS) ? b1 : b0;
            const int row = BPP == 2 ? krow % BS : row0 + krow;
            const CT* p = kbase + (int64_t(blk) * block_stride + head_tile) + (row * D + kc * EPV);
#pragma unroll
            for (int j = 0; j < KVPL; ++j) kb[j] = ld16_stream(p + j * KL * EPV);
        }
#pragma unroll
        for (int r = 0; r < VR; ++r) {
            const int rt = vrg + r * VRG;
            const int blk = (BPP == 2 && rt >= BS) ? b1 : b0;
            const int row = BPP == 2 ? rt % BS : row0 + rt;
            vb[r] = ld16_stream(vbase + (int64_t(blk) * block_stride + head_tile) + (row * D + vcol * EPV));
        }
    };

    auto compute = [&](int k, U4 (&kb)[KVPL], U4 (&vb)[VR]) {
        const int tb = t0 + (w + kWaves * k) * TPP;
        const bool partial = tb + TPP > t1;     // uniform: the pass runs past the partition end
        // scores of this lane's token row for the G heads
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float accs = 0.0f;
#pragma unroll
            for (int j = 0; j < KVPL; ++j) {
                if constexpr (kDot2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        accs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qpk[h][j * 4 + e]),
                                                               __builtin_bit_cast(bf16x2v, u4_get(kb[j], e)),
                                                               accs, false);
                } else if constexpr (CDT == PA_DTYPE_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) accs = fmaf(qf[h][j * 4 + e], __uint_as_float(u4_get(kb[j], e)), accs);
                } else {  // fp8
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wv = u4_get(kb[j], e);
                        const float2v lo = e4m3x2_to_f32<false>(wv);
                        const float2v hi = e4m3x2_to_f32<true>(wv);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 0], lo.x, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 1], lo.y, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 2], hi.x, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 3], hi.y, accs);
                    }
                }
            }
            s[h] = group_sum<KL>(accs) * sc;
        }
        if (partial) {
            const bool kvalid = tb + krow < t1;
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = kvalid ? s[h] : -INFINITY;
        }
        // online softmax: rescale only when a score passes the reference by the threshold
        bool over = false;
#pragma unroll
        for (int h = 0; h < G; ++h) over |= s[h] > m_ref[h] + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float m_new = fmaxf(m_ref[h], wave_max_of_groups<KL>(s[h]));
                const float alpha = __builtin_amdgcn_exp2f(m_ref[h] - m_new);   // 0 on the first pass
                m_ref[h] = m_new;
                l_run[h] *= alpha;
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[h][e] *= alpha;
            }
        }
        if (kc == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) s_p[w][krow][h] = __builtin_amdgcn_exp2f(s[h] - m_ref[h]);
        }
        wave_sync_lds();
        if (partial) {   // rows past the end may hold anything: never multiply them in
#pragma unroll
            for (int r = 0; r < VR; ++r)
                if (tb + vrg + r * VRG >= t1) vb[r] = U4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < VR; ++r) {
            const int rt = vrg + r * VRG;
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = s_p[w][rt][h];
            float vf[EPV];
            if constexpr (CDT == PA_DTYPE_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[e] = __uint_as_float(u4_get(vb[r], e));
            } else if constexpr (CDT == PA_DTYPE_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = u4_get(vb[r], e);
                    vf[2 * e] = __uint_as_float(x << 16);
                    vf[2 * e + 1] = __uint_as_float(x & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = u4_get(vb[r], e);
                    const float2v lo = e4m3x2_to_f32<false>(x);
                    const float2v hi = e4m3x2_to_f32<true>(x);
                    vf[4 * e + 0] = lo.x;
                    vf[4 * e + 1] = lo.y;
                    vf[4 * e + 2] = hi.x;
                    vf[4 * e + 3] = hi.y;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                l_run[h] += pv[h];
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
            }
        }
        wave_sync_lds();   // s_p is rewritten by the next pass
    };

    // ---- software-pipelined pass loop: kDepth register sets in a ring; the loads of passes
    // k+1 .. k+kDepth-1 are in flight while pass k is computed.  The steady-state loop issues
    // unconditionally; the tail drains the ring.
    {
        U4 kb[kDepth][KVPL], vb[kDepth][VR];
#pragma unroll
        for (int i = 0; i < kDepth - 1; ++i)
            if (i < nk) issue(i, kb[i], vb[i]);
        int k = 0;
        for (; k + 2 * kDepth - 2 < nk; k += kDepth) {   // every pass issued below exists
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                issue(k + i + kDepth - 1, kb[(i + kDepth - 1) % kDepth], vb[(i + kDepth - 1) % kDepth]);
                compute(k + i, kb[i], vb[i]);
            }
        }
        for (; k < nk; k += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                if (k + i < nk) {
                    if (k + i + kDepth - 1 < nk)
                        issue(k + i + kDepth - 1, kb[(i + kDepth - 1) % kDepth], vb[(i + kDepth - 1) % kDepth]);
                    compute(k + i, kb[i], vb[i]);
                }
            }
        }
    }

    // ---- reduce the V-phase row groups of this wave
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l_run[h] = sum_over_row_groups<VL>(l_run[h]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[h][e] = sum_over_row_groups<VL>(acc[h][e]);
    }
    if (lane < VL) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) s_acc[w][h][lane * EPV + e] = acc[h][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[w][h] = m_ref[h];
            s_l[w][h] = l_run[h];
        }
    }
    const bool any_bad = __syncthreads_or(bad);
    finish_partition<QDT, D, G, kWaves, false>(a, b, g, part, nparts, vsc, any_bad, &s_m[0][0], &s_l[0][0], &s_acc[0][0][0],
                                G * D);
}

// ------------------------------------------------------------------ decode: matrix-core kernel
//
// bf16 and fp8 caches.  Passes of 16 tokens per wave, as in decode_valu_kernel, but both
// contractions run on the matrix cores with the query heads of a KV head padded to 16:
//  - scores S[token][head] = K_tile[16 x D] . q^T[D x 16] with v_mfma_f32_16x16x32_bf16.  K is
//    the A operand loaded straight from the cache: lane l holds 8 consecutive dims of token
//    row l % 16 (fp8 rows are widened to bf16 exactly); q is the B operand, loaded once per
//    partition with the same dims-to-lanes map.  The result gives lane l the scores of tokens
//    4 * (l / 16) + i for head l % 16;
//  - that is exactly the A-operand layout of v_mfma_f32_16x16x16bf16_1k, so the softmax
//    weights P[head][token] (rounded to bf16) feed out[head][16 dims] += P . V_tile[16 x 16]
//    directly.  The B operand needs V token-major per dim: each wave writes its V tile to
//    LDS (16-byte chunks XOR-swizzled by row) and reads it back with ds_read_b64_tr_b16,
//    which hands lane i of each 16-lane group element i % 4 of the 8 bytes read by lane
//    4 * e + i / 4 as its element e.
// Where K/V travel (chosen per cache type at build time):
//  - bf16: an LDS ring of kStagesBf16 stages per wave filled by global_load_lds_dwordx4 (HBM
//    straight to LDS, no registers held for loads in flight).  The DMA places each row's
//    16-byte chunks XOR-swizzled by row, so K is read back as the A operand and V through
//    the transpose reads from the stage itself, with no copy;
//  - fp8: two passes in registers (K converted there; V converted while written to the
//    bf16 LDS tile).  An fp8 ring would need that copy out of the stage as an extra LDS
//    round trip per pass, which measured slower.
// Work distribution: with the request lengths' prefix sums in LDS, a grid of about one
// resident work-group per slot walks a compact list of (request, partition, KV head) items
// -- first every full partition, then each request's last one -- so no work-group is
// launched for a partition that does not exist.  Batches too large for the LDS list use a
// grid over (partition, KV head, request) with early exit instead.


template <int CDT, int D>
struct MCfg {
    static constexpr int E = Elem<CDT>::bytes;          // 2 (bf16) or 1 (fp8)
    static constexpr int ROWB = D * E;                   // bytes of one cached token row
    static constexpr int NQK = D / 32;                   // 16x16x32 products per pass (scores)
    static constexpr int NPV = D / 16;                   // 16x16x16 products per pass (one per 16 dims)
    static constexpr int KLD = NQK * E / 2;              // 16-byte K loads per lane per pass
    static constexpr int CPR = ROWB / 16;                // 16-byte chunks per cached row
    static constexpr int VLD = 16 * CPR / 64;            // 16-byte V loads per lane per pass
    static constexpr int TROWB = D * 2;                  // bytes per row of the bf16 V tile in LDS
    static constexpr int SGB = 0;                        // no per-row scales
    static_assert(VLD >= 1 && KLD >= 1, "layout");
};

// MXFP4 caches: a pass loads per lane 16 bytes of K codes (D 128; 8 for D 64) of row `col`
// (dims NQK * 8 * grp4 .. + NQK * 8, one 32-dim block for D 128) and the same of V (row
// lane / 4, quarter lane % 4), plus each one's block scale: two "loads" of K and of V.
template <int D>
struct MCfg<PA_DTYPE_MXFP4, D> {
    static constexpr int E = 0;                          // marks the 4-bit layout
    static constexpr int ROWB = D / 2;                   // code bytes of one token row
    static constexpr int SGB = D / 32;                   // scale bytes of one token row
    static constexpr int NQK = D / 32;
    static constexpr int NPV = D / 16;
    static constexpr int KLD = 2;                        // codes, scale
    static constexpr int CPR = ROWB / 16;
    static constexpr int VLD = 2;                        // codes, scale
    static constexpr int TROWB = D * 2;
};

constexpr int kMaxListSeqs = 8192;   // batches up to this size use the compact item list


// pa_decode_append: the row of request b's new token (logical position pos) for KV head g,
// written through the block table exactly as pa_kv_write writes a slot: a bit copy (bf16), the
// fp8 quantisation with the head's scale, or the MXFP4 block quantisation.  Called by the one
// wave that reads position pos; the new row is loaded together with its block id, so the wave
// waits for one load and one store.  A block id outside the pool is not written (the decode
// turns the request's output into NaN).
template <int CDT, int D, int BS>
__device__ __forceinline__ void append_row(const DecodeArgs& a, int b, int g, int pos, int lane) {
    const int64_t src = (int64_t(b) * a.hkv + g) * D;            // the request's row of head g
    const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + src;
    const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + src;
    unsigned char* kc = static_cast<unsigned char*>(const_cast<void*>(a.k_cache));
    unsigned char* vc = static_cast<unsigned char*>(const_cast<void*>(a.v_cache));
    const int r = pos % BS;
    if constexpr (CDT == PA_DTYPE_MXFP4) {
        constexpr int NB = D / 32;                                  // 32-dim blocks per row
        if (lane >= 2 * NB) return;
        const bool isv = lane >= NB;
        const int c = lane % NB;
        const uint16_t* x16 = (isv ? vn : kn) + 32 * c;
        uint32_t x[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const U4 u = gld16(x16 + 8 * i);
            x[4 * i] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
        }
        const int blk = gld_i32(a.block_tables + int64_t(b) * a.max_blocks + pos / BS);
        if (blk < 0 || blk >= a.num_blocks) return;
        uint32_t codes[4], scale;
        mx4_quantize(x, codes, scale);
        const int64_t tile = (int64_t(blk) * a.hkv + g) * (int64_t(BS) * (D / 2 + D / 32));
        unsigned char* base = (isv ? vc : kc) + tile;
        *reinterpret_cast<U4*>(base + r * (D / 2) + 16 * c) = U4{codes[0], codes[1], codes[2], codes[3]};
        base[int64_t(BS) * (D / 2) + r * (D / 32) + c] = static_cast<unsigned char>(scale);
    } else {
        constexpr int LPR = D / 8;                                  // lanes per row, 8 elements each
        if (lane >= 2 * LPR) return;
        const bool isv = lane >= LPR;
        const int c = lane % LPR;
        const U4 x = gld16((isv ? vn : kn) + 8 * c);
        const float sc = CDT == PA_DTYPE_BF16 ? 1.0f : gld_f32((isv ? a.v_scale : a.k_scale) + g);
        const int blk = gld_i32(a.block_tables + int64_t(b) * a.max_blocks + pos / BS);
        if (blk < 0 || blk >= a.num_blocks) return;
        const int64_t row = (int64_t(blk) * a.hkv + g) * BS + r;
        if constexpr (CDT == PA_DTYPE_BF16) {
            *reinterpret_cast<U4*>((isv ? vc : kc) + row * D * 2 + 16 * c) = x;
        } else {
            uint32_t o[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wd = u4_get(x, i / 2);
                const uint32_t bits = (i & 1) ? (wd >> 16) : (wd & 0xffffu);
                // correctly rounded float32 quotient (IEEE division, no fast-math), as pa_kv_write
                o[i / 4] |= f32_to_e4m3(bf16_to_f32(bits) / sc) << (8 * (i % 4));
            }
            *reinterpret_cast<uint2*>((isv ? vc : kc) + row * D + 8 * c) = make_uint2(o[0], o[1]);
        }
    }
}

template <int CDT, int QDT, int D, int BS, int G, int NW, bool DYN>
__global__ __launch_bounds__(64 * NW, 2) void decode_mfma_kernel(const DecodeArgs a) {
    using M = MCfg<CDT, D>;
    constexpr int NT = 64 * NW;                           // threads per work-group
    using CT = typename Elem<CDT>::T;
    using QT = typename Elem<QDT>::T;
    constexpr int TPP = 16;                               // tokens per pass
    constexpr int BPP = BS < TPP ? TPP / BS : 1;          // blocks touched by one pass (1 or 2)
    static_assert(QDT == PA_DTYPE_BF16 &&
                      (CDT == PA_DTYPE_BF16 || CDT == PA_DTYPE_FP8_E4M3 || CDT == PA_DTYPE_MXFP4), "bf16 q");
    constexpr bool kMx = CDT == PA_DTYPE_MXFP4;
    static_assert(G <= 16 && BPP <= 2, "shape");
    constexpr int KT = TPP * M::ROWB;                     // bytes of one cached K (or V) tile
    constexpr int VTB = TPP * M::TROWB;                   // bytes of one bf16 V tile
    // LDS per wave: the V tile (registers path) or the ring of K/V stages plus, for fp8, the
    // bf16 V tile the transpose reads use
    constexpr int kStages = kMx ? 0 : M::E == 2 ? kStagesBf16 : kStagesFp8;
    constexpr int WAVE_LDS = kStages > 0 ? kStages * 2 * KT + (M::E == 1 ? VTB : 0) : VTB;
    static_assert(G * D * 4 <= WAVE_LDS, "a wave's merge slice fits in its LDS");

    // per-wave V tile (bf16, swizzled); after a partition's passes the same bytes hold the
    // wave's accumulator slice acc[G][D] (float) for the merge across waves
    __shared__ __align__(16) unsigned char s_tile[NW][WAVE_LDS];
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    extern __shared__ int s_pref[];                       // compact item list: B + 1 prefix sums

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform per wave
    const int col = lane & 15, grp4 = lane >> 4;          // MFMA column (head / dim) and row group
    const int hq = a.hkv * G;
    const CT* kbase = reinterpret_cast<const CT*>(a.k_cache);
    const CT* vbase = reinterpret_cast<const CT*>(a.v_cache);
    PA_LDS unsigned char* tile = (PA_LDS unsigned char*)&s_tile[w][0];

    auto nparts_of = [&](int L_raw) {
        const bool bad_len = L_raw < 0 || L_raw > a.max_seq_len || L_raw > a.max_blocks * BS;
        return (!bad_len && L_raw > 0) ? (L_raw + a.part_tokens - 1) / a.part_tokens : 1;
    };

    // ---- one partition of one (request, KV head)
    auto process = [&](int b, int g, int part) {
        const int t0 = part * a.part_tokens;
        const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;

        // block ids of this wave's passes, 64 at a time (lane j: pass w + NW * (k0 + j)),
        // read before the length is known; `check_entries` flags ids outside the pool inside
        // the live range and replaces every such id by 0
        int ent_a = 0, ent_b = 0;
        auto read_entries = [&](int k0) {
            const int e = (t0 + (w + NW * (k0 + lane)) * TPP) / BS;
            ent_a = a.max_blocks > 0 ? gld_i32(table + min(e, a.max_blocks - 1)) : -1;
            if constexpr (BPP == 2) ent_b = a.max_blocks > 0 ? gld_i32(table + min(e + 1, a.max_blocks - 1)) : -1;
        };
        read_entries(0);

        // q as the B operand of the score products: head `col` (zero beyond the group), the
        // dims this lane's K operand holds
        U4 qb[M::NQK];
        {
            const QT* qrow = reinterpret_cast<const QT*>(a.q) + (int64_t(b) * hq + int64_t(g) * G + col) * D;
#pragma unroll
            for (int j = 0; j < M::NQK; ++j) {
                const int d0 = kMx ? M::NQK * 8 * grp4 + 8 * j
                               : M::E == 2 ? 32 * j + 8 * grp4 : 64 * (j >> 1) + 16 * grp4 + 8 * (j & 1);
                qb[j] = col < G ? gld16(qrow + d0) : U4{0, 0, 0, 0};
            }
        }

        const int L_raw = __builtin_amdgcn_readfirstlane(gld_i32(a.seq_lens + b));
        const bool len_bad = L_raw < 0 || L_raw > a.max_seq_len || L_raw > a.max_blocks * BS;
        const int L = len_bad ? 0 : L_raw;
        const int nparts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
        if (part >= nparts) return;                       // grid mapping only
        if (L == 0) {   // empty request (zeros) or invalid length (NaN); single partition
            QT* out = reinterpret_cast<QT*>(a.out) + (int64_t(b) * hq + int64_t(g) * G) * D;
            const float fill = len_bad ? __builtin_nanf("") : 0.0f;
            for (int i = threadIdx.x; i < G * D; i += NT) gst(out + i, f32_to_bf16(fill));
            __syncthreads();
            return;
        }

        const int t1 = min(L, t0 + a.part_tokens);
        const int npass = (t1 - t0 + TPP - 1) / TPP;
        const int nk = npass > w ? (npass - w + NW - 1) / NW : 0;
        float sc = a.score_scale;
        float vsc = 1.0f;
        if constexpr (CDT == PA_DTYPE_FP8_E4M3) {
            sc *= __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gld_f32(a.k_scale + g))));
            vsc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gld_f32(a.v_scale + g))));
        }

        bool bad = false;
        auto check_entries = [&](int k0) {
            const int kk = k0 + lane;
            const bool live = kk < nk;
            if (ent_a < 0 || ent_a >= a.num_blocks) {
                if (live) bad = true;
                ent_a = 0;
            }
            if constexpr (BPP == 2) {
                const int e = (t0 + (w + NW * kk) * TPP) / BS;
                if (ent_b < 0 || ent_b >= a.num_blocks) {
                    if (live && (e + 1) * BS < t1) bad = true;
                    ent_b = 0;
                }
            }
        };
        check_entries(0);

        // pa_decode_append: the new token (position L - 1) of KV head g is read by one pass of
        // the request's last partition, and each wave loads only its own passes, so only the
        // wave that runs that pass (`app_wave`) touches the row.  Over the bf16 ring that wave
        // loads the new row beside its first passes, and when that pass's tile has landed in
        // LDS it overwrites the row there and stores it to the cache (the tile's load was
        // complete, so the store cannot race it).  The other cache types write the row first
        // and drain the memory counter (the stores have completed) before the wave's first load.
        constexpr bool kPatch = kStages > 0 && M::E == 2;
        const bool app_wave = a.k_new != nullptr && part == nparts - 1 && w == ((L - 1 - t0) / TPP) % NW;
        if (!kPatch && app_wave) {
            append_row<CDT, D, BS>(a, b, g, L - 1, lane);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }

        float m_ref = -INFINITY, l_run = 0.0f;            // head `col`
        f32x4v acc[M::NPV];                               // out[head 4*grp4 + i][16 t + col]
#pragma unroll
        for (int t = 0; t < M::NPV; ++t) acc[t] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

        // lane byte offsets inside a 16-token tile (loop invariant): K row `col` at 16 * grp4;
        // V chunk `lane` of each 1 KiB group of chunks
        const uint32_t k_lane = uint32_t(col) * M::ROWB + 16u * grp4;
        const uint32_t v_lane = uint32_t(lane / M::CPR) * M::ROWB + 16u * (lane % M::CPR);
        // (block, head) tiles: D * E bytes per token row, or for MXFP4 the codes then the scales
        constexpr int64_t kTile = kMx ? int64_t(BS) * (M::ROWB + M::SGB) : int64_t(BS) * D * M::E;
        const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kbase) + int64_t(g) * kTile;
        const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(vbase) + int64_t(g) * kTile;
        const int64_t blk_bytes = int64_t(a.hkv) * kTile;

        if constexpr (kStages == 0) {
            auto issue = [&](int k, U4 (&kb)[M::KLD], U4 (&vb)[M::VLD]) {
                if ((k & 63) == 0 && k > 0) {
                    read_entries(k);
                    check_entries(k);
                }
                const int tb = t0 + (w + NW * k) * TPP;
                const int b0 = __builtin_amdgcn_readlane(ent_a, k & 63);
                if constexpr (kMx) {
                    // K row `col`, V row lane / 4 (quarter lane % 4); rows 8..15 in the second
                    // block when blocks hold 8 tokens
                    const int b1 = BPP == 2 ? __builtin_amdgcn_readlane(ent_b, k & 63) : b0;
                    const int vr = lane >> 2, part = lane & 3;
                    // one block: uniform base (the pass's first row) + 32-bit lane offsets;
                    // two blocks of 8 rows: rows 8..15 from the second
                    const int kr = BPP == 2 ? col % BS : col;
                    const int vrr = BPP == 2 ? vr % BS : vr;
                    const uint32_t r0c = BPP == 2 ? 0u : uint32_t(tb % BS) * M::ROWB;   // codes of the first row
                    const uint32_t r0s = BPP == 2 ? 0u : uint32_t(tb % BS) * M::SGB;    // its scales
                    const unsigned char* kt = kbytes + int64_t((BPP == 2 && col >= BS) ? b1 : b0) * blk_bytes;
                    const unsigned char* vt = vbytes + int64_t((BPP == 2 && vr >= BS) ? b1 : b0) * blk_bytes;
                    const unsigned char* ktc = kt + r0c;
                    const unsigned char* vtc = vt + r0c;
                    const unsigned char* kts = kt + (BS * M::ROWB + r0s);
                    const unsigned char* vts = vt + (BS * M::ROWB + r0s);
                    if constexpr (D == 128) {
                        kb[0] = gld16_stream(ktc + uint32_t(kr * M::ROWB + 16 * grp4));
                        vb[0] = gld16_stream(vtc + uint32_t(vrr * M::ROWB + 16 * part));
                    } else {
                        const uint2 k8 = gld8(ktc + uint32_t(kr * M::ROWB + 8 * grp4));
                        const uint2 v8 = gld8(vtc + uint32_t(vrr * M::ROWB + 8 * part));
                        kb[0] = U4{k8.x, k8.y, 0u, 0u};
                        vb[0] = U4{v8.x, v8.y, 0u, 0u};
                    }
                    kb[1].x = gld_u8(kts + uint32_t(kr * M::SGB + (D == 128 ? grp4 : grp4 / 2)));
                    vb[1].x = gld_u8(vts + uint32_t(vrr * M::SGB + (D == 128 ? part : part / 2)));
                } else if constexpr (BPP == 1) {
                    // one block: uniform base + 32-bit lane offset (+ immediate offsets)
                    const uint32_t row0b = uint32_t(tb % BS) * M::ROWB;
                    const unsigned char* kp = kbytes + int64_t(b0) * blk_bytes + row0b;
                    const unsigned char* vp = vbytes + int64_t(b0) * blk_bytes + row0b;
    #pragma unroll
                    for (int j = 0; j < M::KLD; ++j) kb[j] = gld16_stream(kp + (k_lane + 64u * j));
    #pragma unroll
                    for (int r = 0; r < M::VLD; ++r) vb[r] = gld16_stream(vp + (v_lane + 1024u * r));
                } else {
                    // two blocks of 8 rows: rows 0..7 from the first, 8..15 from the second
                    const int b1 = __builtin_amdgcn_readlane(ent_b, k & 63);
                    const unsigned char* kp = kbytes + int64_t(col >= BS ? b1 : b0) * blk_bytes;
                    const uint32_t krow = k_lane - (col >= BS ? uint32_t(BS) * M::ROWB : 0u);
    #pragma unroll
                    for (int j = 0; j < M::KLD; ++j) kb[j] = gld16_stream(kp + (krow + 64u * j));
    #pragma unroll
                    for (int r = 0; r < M::VLD; ++r) {
                        const uint32_t off = v_lane + 1024u * r;          // byte offset inside the 16 rows
                        const bool second = off >= uint32_t(BS) * M::ROWB;
                        const unsigned char* vp = vbytes + int64_t(second ? b1 : b0) * blk_bytes;
                        vb[r] = gld16_stream(vp + (off - (second ? uint32_t(BS) * M::ROWB : 0u)));
                    }
                }
            };

            auto compute = [&](int k, U4 (&kb)[M::KLD], U4 (&vb)[M::VLD]) {
                const int tb = t0 + (w + NW * k) * TPP;
                // a pass past the end of the partition masks its rows beyond t1; the others
                // (all but the last) skip every mask
                auto body = [&](auto partial_c) {
                constexpr bool partial = decltype(partial_c)::value;
                // V tile -> LDS as bf16 (rows past the end zeroed: they may hold anything)
                if constexpr (kMx) {
                    constexpr int NCD = D / 32;           // code dwords per lane (8 dims each)
                    const int vr = lane >> 2, part = lane & 3;
                    const uint32_t keep = (partial && tb + vr >= t1) ? 0u : ~0u;
                    const float vsf = e8m0_to_f32(vb[1].x);
                    PA_LDS unsigned char* rowp = tile + vr * M::TROWB;
    #pragma unroll
                    for (int wi = 0; wi < NCD; ++wi) {
                        U4 c = e2m1x8_to_bf16(u4_get(vb[0], wi), vsf);
                        if constexpr (partial) c = U4{c.x & keep, c.y & keep, c.z & keep, c.w & keep};
                        lds_st16(rowp + 16 * vt_slot<D>(vr, NCD * part + wi), c);
                    }
                }
    #pragma unroll
                for (int r = 0; r < (kMx ? 0 : M::VLD); ++r) {
                    const int ci = 64 * r + lane, vr = ci / M::CPR, c = ci % M::CPR;
                    U4 v = vb[r];
                    if constexpr (partial) {
                        const uint32_t keep = tb + vr >= t1 ? 0u : ~0u;
                        v = U4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
                    }
                    PA_LDS unsigned char* rowp = tile + vr * M::TROWB;
                    if constexpr (M::E == 2) {
                        lds_st16(rowp + 16 * vt_slot<D>(vr, c), v);
                    } else {
                        uint32_t lo[4], hi[4];
                        e4m3x8_to_bf16(v.x, v.y, lo);
                        e4m3x8_to_bf16(v.z, v.w, hi);
                        lds_st16(rowp + 16 * vt_slot<D>(vr, 2 * c), U4{lo[0], lo[1], lo[2], lo[3]});
                        lds_st16(rowp + 16 * vt_slot<D>(vr, 2 * c + 1), U4{hi[0], hi[1], hi[2], hi[3]});
                    }
                }
                // scores: S[token][head] over the D dims
                f32x4v s4 = {0.0f, 0.0f, 0.0f, 0.0f};
                const float ksf = kMx ? e8m0_to_f32(kb[kMx ? 1 : 0].x) : 0.0f;
    #pragma unroll
                for (int j = 0; j < M::NQK; ++j) {
                    U4 kv;
                    if constexpr (kMx) {
                        kv = e2m1x8_to_bf16(u4_get(kb[0], j), ksf);
                    } else if constexpr (M::E == 2) {
                        kv = kb[j];
                    } else {
                        const U4& src = kb[j >> 1];
                        uint32_t o[4];
                        if (j & 1) e4m3x8_to_bf16(src.z, src.w, o); else e4m3x8_to_bf16(src.x, src.y, o);
                        kv = U4{o[0], o[1], o[2], o[3]};
                    }
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, kv),
                                                                 __builtin_bit_cast(bf16x8v, qb[j]), s4, 0, 0, 0);
                }
                float sv[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i)
                    sv[i] = (partial && tb + 4 * grp4 + i >= t1) ? -INFINITY : s4[i] * sc;
                // online softmax per head (lanes col, col + 16, col + 32, col + 48 share head col);
                // the state is rescaled only when a score passes the reference by the threshold
                float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                mx = pair16_max(pair32_max(mx));
                if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold) != 0) {
                    const float m_new = fmaxf(m_ref, mx);
                    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first pass
                    m_ref = m_new;
                    l_run *= alpha;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {   // acc rows hold head 4 * grp4 + i: its factor is lane's
                        const float ai = __int_as_float(
                            __builtin_amdgcn_ds_bpermute(4 * (4 * grp4 + i), __float_as_int(alpha)));
    #pragma unroll
                        for (int t = 0; t < M::NPV; ++t) acc[t][i] *= ai;
                    }
                }
                // weights rounded to bf16 by the hardware conversion (nearest even); the
                // denominator sums the rounded weights, two at a time
                uint32_t pw[2];
    #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x2v pr;
                    pr[0] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[2 * h] - m_ref));
                    pr[1] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[2 * h + 1] - m_ref));
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, __builtin_bit_cast(bf16x2v, 0x3f803f80u), l_run, false);
                    pw[h] = __builtin_bit_cast(uint32_t, pr);
                }
                const i16x4v pa = __builtin_bit_cast(i16x4v, make_uint2(pw[0], pw[1]));
                // out[head][dims] += P . V, V read back token-major per dim.  The transposed reads
                // are issued NB at a time ahead of their products (scheduling barriers keep the
                // compiler from pairing each read with its product behind a wait of its own, as it
                // does at this register pressure); fp8 takes batches of four (two under 16-token
                // blocks), which fit its registers, the 4-bit path all of them
                const int vrow = 4 * grp4 + ((lane & 15) >> 2);
                constexpr int NB = (M::NPV > 4 && !kMx) ? (BS < 16 ? 2 : 4) : M::NPV;
                i16x4v vts[M::NPV];
                auto read_vt = [&](int t) {
                    const int c = 2 * t + ((lane & 3) >> 1);
                    PA_LDS unsigned char* src = tile + vrow * M::TROWB + 16 * vt_slot<D>(vrow, c) + 8 * (lane & 1);
                    vts[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4v*)src);
                };
    #pragma unroll
                for (int t = 0; t < NB; ++t) read_vt(t);
    #pragma unroll
                for (int t0 = 0; t0 < M::NPV; t0 += NB) {
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int t = t0 + NB; t < min(t0 + 2 * NB, M::NPV); ++t) read_vt(t);
    #pragma unroll
                    for (int t = t0; t < t0 + NB; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vts[t], acc[t], 0, 0, 0);
                }
                };
                if (tb + TPP > t1) body(std::true_type{});
                else body(std::false_type{});
            };

            {
                U4 kb[kDepth][M::KLD], vb[kDepth][M::VLD];
    #pragma unroll
                for (int i = 0; i < kDepth - 1; ++i)
                    if (i < nk) issue(i, kb[i], vb[i]);
                int k = 0;
                for (; k + 2 * kDepth - 2 < nk; k += kDepth) {   // every pass issued below exists
    #pragma unroll
                    for (int i = 0; i < kDepth; ++i) {
                        issue(k + i + kDepth - 1, kb[(i + kDepth - 1) % kDepth], vb[(i + kDepth - 1) % kDepth]);
                        compute(k + i, kb[i], vb[i]);
                    }
                }
                for (; k < nk; k += kDepth) {
    #pragma unroll
                    for (int i = 0; i < kDepth; ++i) {
                        if (k + i < nk) {
                            if (k + i + kDepth - 1 < nk)
                                issue(k + i + kDepth - 1, kb[(i + kDepth - 1) % kDepth], vb[(i + kDepth - 1) % kDepth]);
                            compute(k + i, kb[i], vb[i]);
                        }
                    }
                }
            }
        } else {
        // ---- K/V through an LDS ring of kStages stages per wave, filled by DMA loads.
        // A tile's 16-byte chunk position p (row p / CPR) holds data chunk stage_slot(row, p % CPR)
        // of its row, so that the K reads (16 rows at one chunk) and the V transpose reads spread
        // over the banks.  Lane `lane` of DMA instruction i fills position 64 i + lane.
        constexpr int CPR = M::CPR;
        constexpr int NI = KT / 1024;                     // DMA instructions per tile
        constexpr int NIP = 2 * NI;                       // per pass (K and V)
        constexpr int RPI = 64 / CPR;                     // rows per DMA instruction
        static_assert(KT % 1024 == 0 && NI >= 1, "tile of whole KiB");
        // bf16 stages use dma_slot (a conflict-free layout for both operand reads); the fp8
        // stage keeps chunk p % CPR XOR row % CPR of its 128-byte rows
        auto stage_slot = [](int row, int c) { return M::E == 2 ? dma_slot<D>(row, c) : c ^ (row % CPR); };
        uint32_t src_off[NI];                             // source byte offset inside the 16 rows
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int pos = 64 * i + lane, row = pos / CPR, slot = pos % CPR;
            src_off[i] = uint32_t(row) * M::ROWB + 16u * uint32_t(stage_slot(row, slot));
        }
        PA_LDS unsigned char* ring = tile;                // stage s: K at ring + 2 s KT, V at + KT
        PA_LDS unsigned char* vtile = tile + kStages * 2 * KT;   // fp8: bf16 V tile
        auto stage_k = [&](int st) { return ring + st * (2 * KT); };
        U4 new_row = U4{0, 0, 0, 0};                     // pa_decode_append over the ring (kPatch)
        int new_blk = -1;
        const int new_pass = ((L - 1 - t0) / TPP) / NW;   // app_wave's pass holding position L - 1

        auto issue_dma = [&](int k, int st) {
            if ((k & 63) == 0 && k > 0) {   // next 64 passes' block ids (the compiler's wait drains the ring)
                read_entries(k);
                check_entries(k);
            }
            const int tb = t0 + (w + NW * k) * TPP;
            const int b0 = __builtin_amdgcn_readlane(ent_a, k & 63);
            PA_LDS unsigned char* dk = stage_k(st);
            PA_LDS unsigned char* dv = dk + KT;
            if constexpr (BPP == 1) {
                const uint32_t row0b = uint32_t(tb % BS) * M::ROWB;
                const unsigned char* kp = kbytes + int64_t(b0) * blk_bytes + row0b;
                const unsigned char* vp = vbytes + int64_t(b0) * blk_bytes + row0b;
#pragma unroll
                for (int i = 0; i < NI; ++i) dma16(kp, src_off[i], lds_addr(dk + 1024 * i));
#pragma unroll
                for (int i = 0; i < NI; ++i) dma16(vp, src_off[i], lds_addr(dv + 1024 * i));
            } else {   // rows 0..7 from the first block, 8..15 from the second
                const int b1 = __builtin_amdgcn_readlane(ent_b, k & 63);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    if constexpr (RPI <= BS) {   // every row of instruction i in one block
                        const bool second = i * RPI >= BS;
                        const uint32_t off = src_off[i] - (second ? uint32_t(BS) * M::ROWB : 0u);
                        dma16(kbytes + int64_t(second ? b1 : b0) * blk_bytes, off, lds_addr(dk + 1024 * i));
                        dma16(vbytes + int64_t(second ? b1 : b0) * blk_bytes, off, lds_addr(dv + 1024 * i));
                    } else {
                        const int row = (64 * i + lane) / CPR;
                        const bool second = row >= BS;
                        const uint32_t off = src_off[i] - (second ? uint32_t(BS) * M::ROWB : 0u);
                        dma16_lane(kbytes + int64_t(second ? b1 : b0) * blk_bytes + off, lds_addr(dk + 1024 * i));
                        dma16_lane(vbytes + int64_t(second ? b1 : b0) * blk_bytes + off, lds_addr(dv + 1024 * i));
                    }
                }
            }
        };

        auto compute_dma = [&](int k, int st) {
            const int tb = t0 + (w + NW * k) * TPP;
            const bool partial = tb + TPP > t1;
            PA_LDS unsigned char* dk = stage_k(st);
            PA_LDS unsigned char* dv = dk + KT;
            if constexpr (kPatch) {
                if (app_wave && k == new_pass && lane < 2 * CPR) {
                    // the new token's row: chunk c of tile row L - 1 - tb, then the cache
                    const int r = L - 1 - tb, c = lane % CPR;
                    lds_st16((lane < CPR ? dk : dv) + 16 * (r * CPR + stage_slot(r, c)), new_row);
                    // the id's test stays here: hoisted out of the loop it would wait for the
                    // load right after it was issued
                    int nb = new_blk;
                    asm volatile("" : "+v"(nb));
                    if (nb >= 0 && nb < a.num_blocks) {
                        unsigned char* cache = static_cast<unsigned char*>(const_cast<void*>(lane < CPR ? a.k_cache : a.v_cache));
                        const int64_t row = (int64_t(nb) * a.hkv + g) * BS + (L - 1) % BS;
                        *reinterpret_cast<U4*>(cache + row * M::ROWB + 16 * c) = new_row;
                    }
                }
            }
            // V as a bf16 tile the transpose reads understand (rows past the end zeroed)
            PA_LDS unsigned char* vt;
            if constexpr (M::E == 2) {
                vt = dv;
                if (partial) {
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int pos = 64 * i + lane;
                        if (tb + pos / CPR >= t1) lds_st16(dv + 16 * pos, U4{0, 0, 0, 0});
                    }
                }
            } else {
                vt = vtile;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int pos = 64 * i + lane, row = pos / CPR, c = (pos % CPR) ^ (row % CPR);
                    const uint32_t keep = (partial && tb + row >= t1) ? 0u : ~0u;
                    U4 v = lds_ld16(dv + 16 * pos);
                    v = U4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
                    uint32_t lo[4], hi[4];
                    e4m3x8_to_bf16(v.x, v.y, lo);
                    e4m3x8_to_bf16(v.z, v.w, hi);
                    PA_LDS unsigned char* rowp = vtile + row * M::TROWB;
                    lds_st16(rowp + 16 * dma_slot<D>(row, 2 * c), U4{lo[0], lo[1], lo[2], lo[3]});
                    lds_st16(rowp + 16 * dma_slot<D>(row, 2 * c + 1), U4{hi[0], hi[1], hi[2], hi[3]});
                }
            }
            // scores: K rows as the A operand read from the stage
            f32x4v s4 = {0.0f, 0.0f, 0.0f, 0.0f};
            const PA_LDS unsigned char* krow = dk + col * M::ROWB;
#pragma unroll
            for (int j = 0; j < M::NQK; ++j) {
                U4 kv;
                if constexpr (M::E == 2) {
                    kv = lds_ld16(krow + 16 * stage_slot(col, 4 * j + grp4));
                } else {
                    const U4 src = lds_ld16(krow + 16 * stage_slot(col, 4 * (j >> 1) + grp4));
                    uint32_t o[4];
                    if (j & 1) e4m3x8_to_bf16(src.z, src.w, o); else e4m3x8_to_bf16(src.x, src.y, o);
                    kv = U4{o[0], o[1], o[2], o[3]};
                }
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, kv),
                                                             __builtin_bit_cast(bf16x8v, qb[j]), s4, 0, 0, 0);
            }
            float sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sv[i] = (partial && tb + 4 * grp4 + i >= t1) ? -INFINITY : s4[i] * sc;
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mx = pair16_max(pair32_max(mx));
            if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold) != 0) {
                const float m_new = fmaxf(m_ref, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first pass
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __int_as_float(
                        __builtin_amdgcn_ds_bpermute(4 * (4 * grp4 + i), __float_as_int(alpha)));
#pragma unroll
                    for (int t = 0; t < M::NPV; ++t) acc[t][i] *= ai;
                }
            }
            uint32_t pw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[i] = weight_to_bf16(__builtin_amdgcn_exp2f(sv[i] - m_ref));
                l_run += bf16_to_f32(pw[i]);
            }
            const i16x4v pa = __builtin_bit_cast(i16x4v, make_uint2(pw[0] | (pw[1] << 16), pw[2] | (pw[3] << 16)));
            // the transposed reads all issued before their products (see the register path)
            const int vrow = 4 * grp4 + ((lane & 15) >> 2);
            i16x4v vts[M::NPV];
#pragma unroll
            for (int t = 0; t < M::NPV; ++t) {
                const int c = 2 * t + ((lane & 3) >> 1);
                PA_LDS unsigned char* src = vt + vrow * M::TROWB + 16 * dma_slot<D>(vrow, c) + 8 * (lane & 1);
                vts[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4v*)src);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < M::NPV; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vts[t], acc[t], 0, 0, 0);
        };

        // the compiler's own loads (q, table, length) complete before the ring starts
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < kStages - 1; ++i)
            if (i < nk) issue_dma(i, i);
        if constexpr (kPatch) {
            // the new row (lanes [0, CPR): K chunks, [CPR, 2 CPR): V chunks) and its block id,
            // issued after the first passes: the ring's waits, which leave only newer loads
            // outstanding, complete them before the pass that needs them
            if (app_wave) {
                if (lane < 2 * CPR)
                    new_row = gld16(static_cast<const uint16_t*>(lane < CPR ? a.k_new : a.v_new) +
                                    (int64_t(b) * a.hkv + g) * D + 8 * (lane % CPR));
                // a per-lane index: a uniform one lets the compiler move the id into a scalar
                // register at once, which waits for this load and the passes just issued
                int e = (L - 1) / BS;
                asm volatile("" : "+v"(e));
                new_blk = gld_i32(table + e);
            }
        }
        int k = 0;
        int st = 0;                                       // stage of pass k
        for (; k + kStages - 1 < nk; ++k) {               // pass k + kStages - 1 exists
            const int st_new = st == 0 ? kStages - 1 : st - 1;   // (k + kStages - 1) % kStages
            issue_dma(k + kStages - 1, st_new);
            wait_vmem<(kStages - 1) * NIP>();             // all but the newest kStages - 1 passes landed
            compute_dma(k, st);
            st = st + 1 == kStages ? 0 : st + 1;
        }
        for (; k < nk; ++k) {                             // the last passes: drain
            wait_vmem<0>();
            compute_dma(k, st);
            st = st + 1 == kStages ? 0 : st + 1;
        }
        }   // kStages

        // this wave's state -> LDS (the accumulator slice overwrites the wave's own V tile)
        l_run = pair16_sum(pair32_sum(l_run));
        PA_LDS float* s_acc_w = (PA_LDS float*)tile;
        if (grp4 == 0 && col < G) {
            s_m[w][col] = m_ref;
            s_l[w][col] = l_run;
        }
#pragma unroll
        for (int t = 0; t < M::NPV; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * grp4 + i;
                if (h < G) s_acc_w[h * D + 16 * t + col] = acc[t][i];
            }
        }
        const bool any_bad = __syncthreads_or(bad);
        finish_partition<QDT, D, G, NW, CDT == PA_DTYPE_BF16>(a, b, g, part, nparts, vsc, any_bad, &s_m[0][0], &s_l[0][0],
                                    reinterpret_cast<float*>(&s_tile[0][0]), int(sizeof(s_tile[0]) / 4));
    };

    // ---- work items: the compact list (in LDS, the prefix sums of each request's full
    // partitions, all but its last, whose differences also give each request's last partition),
    // or one item per work-group of the (partition, KV head, request) grid
    int F = 0;
    int64_t total = 1;
    if (a.list) {
        const int B = a.num_seqs;
        const int per = (B + NT - 1) / NT;
        const int i0 = min(B, int(threadIdx.x) * per), i1 = min(B, i0 + per);
        int local = 0;
        for (int i = i0; i < i1; ++i) {                   // each request's full partitions, in place
            const int full = nparts_of(gld_i32(a.seq_lens + i)) - 1;
            s_pref[i] = full;
            local += full;
        }
        __shared__ int s_wsum[NW];
        int incl = local;                                 // work-group exclusive scan of `local`
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_wsum[w] = incl;
        __syncthreads();
        int run = incl - local;
        for (int ww = 0; ww < w; ++ww) run += s_wsum[ww];
        for (int i = i0; i < i1; ++i) {                   // -> exclusive prefix sums
            const int full = s_pref[i];
            s_pref[i] = run;
            run += full;
        }
        if (threadIdx.x == NT - 1) s_pref[B] = run;
        __syncthreads();
        F = __builtin_amdgcn_readfirstlane(s_pref[B]);
        total = int64_t(F + B) * a.hkv;
    }
    // Items are dealt round robin.  In the DYN instances (launched for item lists of a few long
    // requests over bf16 caches), when nearly every item is a full partition (all of one size),
    // the last one and a half rounds are instead handed out by a counter after the tickets, so
    // that work-groups on faster compute units take more of them; each claim is issued when a
    // work-group starts its current item and read when that item ends (a work-group's last claim
    // has returned before it counts itself out), and the last work-group to exit resets the
    // counter and its own.  Items of mixed sizes (ragged batches) stay dealt round robin: there,
    // long and short items interleaved keep more bytes in flight than a counter's claims, which
    // also stall the waits of the claiming wave.  The other instances carry none of this code.
    int* const queue = (DYN && a.list && a.ws_ctr != nullptr)
                           ? a.ws_ctr + int64_t(a.num_seqs) * hq * a.ctr_stride : nullptr;
    const int nslots = a.list ? int(gridDim.x) : 1;
    const bool dyn = queue != nullptr && int64_t(F) >= 9 * int64_t(a.num_seqs) &&   // >= 90% full partitions
                     total >= 2 * int64_t(nslots);
    __shared__ int64_t s_base, s_item;                    // the first counted item; a claimed item
    int n_left = 1;                                       // round-robin items left to this work-group
    if (a.list) {
        const int64_t n_static = dyn ? total - (3 * nslots) / 2 : total;
        n_left = int64_t(blockIdx.x) < n_static ? int((n_static - 1 - blockIdx.x) / nslots) + 1 : 0;
        if (threadIdx.x == 0) s_base = n_static;
    }
    auto take_claim = [&](int claim) {                    // the item `claim` of the counted ones
        if (threadIdx.x == 0) s_item = s_base + claim;
        __syncthreads();
        const int64_t v = s_item;
        __syncthreads();
        return int64_t(__builtin_amdgcn_readfirstlane(int(v >> 32))) << 32 |
               uint32_t(__builtin_amdgcn_readfirstlane(int(v & 0xffffffff)));
    };
    int64_t it = a.list ? blockIdx.x : 0;
    if (dyn && n_left == 0)                               // no round-robin item: claim the first at once
        it = take_claim(threadIdx.x == 0 ? __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0);
    while (it < total) {
        --n_left;
        const bool dyn_next = dyn && n_left <= 0;
        int claim = 0;
        if (dyn_next && threadIdx.x == 0) claim = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int b, g, part;
        if (a.list) {
            const int u = static_cast<int>(it / a.hkv);
            g = static_cast<int>(it % a.hkv);
            if (u < F) {   // the request whose full partitions cover u
                int lo = 0, hi = a.num_seqs;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_pref[mid] <= u) lo = mid; else hi = mid;
                }
                b = lo;
                part = u - s_pref[lo];
            } else {
                b = u - F;
                part = s_pref[b + 1] - s_pref[b];         // its full partitions precede it
            }
        } else {
            b = blockIdx.z;
            g = blockIdx.y;
            part = blockIdx.x;
        }
        process(__builtin_amdgcn_readfirstlane(b), __builtin_amdgcn_readfirstlane(g),
                __builtin_amdgcn_readfirstlane(part));
        it = dyn_next ? take_claim(claim) : it + nslots;
    }
    if (DYN && dyn && threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == int(gridDim.x) - 1) {                 // every work-group has stopped claiming
            __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ workspace clear

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t n_words) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n_words; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// ------------------------------------------------------------------ fixed scratch (pa_decode_noalloc)
//
// Split-K partials and merge tickets of pa_decode_noalloc: a file-scope device array, which
// every device the library runs on holds until the process ends.  In host code this name
// denotes a host-side stand-in, not device memory: host code uses only the device address that
// hipGetSymbolAddress returns for the current device (kept per device below).
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

// ------------------------------------------------------------------ host helpers

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dt) { return dt == PA_DTYPE_F32 ? 4 : dt == PA_DTYPE_BF16 ? 2 : dt == PA_DTYPE_FP8_E4M3 ? 1 : 0; }

// Bytes of one (block, KV head) tile of the cache, or 0 for an unknown type.
int64_t tile_bytes(int dt, int bs, int d) {
    if (dt == PA_DTYPE_MXFP4) return int64_t(bs) * (d / 2 + d / 32);
    return int64_t(bs) * d * elem_bytes(dt);
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PA_OK;
}

// The address a kernel uses for the byte range [p, p + bytes) when that range lies inside
// one HIP allocation in device memory or pinned host memory; anything else (pageable host
// memory, a range running past its allocation) is refused before a launch could fault.
int device_view(const void* p, int64_t bytes, const char* fn, const char* what, const void** out) {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();   // leave no sticky error for the next call to report
        return fail(PA_ERR_INVALID, "%s: %s is not memory known to HIP", fn, what);
    }
    if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeHost)
        return fail(PA_ERR_INVALID, "%s: %s is neither device nor pinned host memory (type %d)", fn, what,
                    static_cast<int>(at.type));
    unsigned int host_flags = 0;
    if (at.type == hipMemoryTypeHost && hipHostGetFlags(&host_flags, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();   // host memory that HIP did not allocate or register
        return fail(PA_ERR_INVALID, "%s: %s is host memory not allocated by HIP", fn, what);
    }
    void* start = nullptr;
    size_t size = 0;
    if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, const_cast<void*>(p)) != hipSuccess ||
        hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PA_ERR_INVALID, "%s: the allocation holding %s cannot be queried", fn, what);
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(start), hi = lo + size, q = reinterpret_cast<uintptr_t>(p);
    if (q < lo || q + static_cast<uintptr_t>(bytes) > hi)
        return fail(PA_ERR_INVALID, "%s: %s [%p, +%lld) runs past its allocation [%p, +%zu)", fn, what, p,
                    (long long)bytes, start, size);
    *out = at.type == hipMemoryTypeHost && at.devicePointer ? at.devicePointer : p;
    return PA_OK;
}

int grid_for(int64_t work, int per_block) {
    int64_t blocks = (work + per_block - 1) / per_block;
    if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
    return static_cast<int>(blocks < 1 ? 1 : blocks);
}

// Workspace (each region 256-byte aligned):
//   [tickets: requests x q heads x stride int32]   stride = ticket_groups + 1 per (request, KV
//                                                   head): level-1 tickets, then the level-2 one;
//    then 2 int32: the item list's claim counter and its exit counter
//   [m1, l1: rows1][acc1: rows1 x d]   rows1 = requests x q heads x partitions
//   [m2, l2: rows2][acc2: rows2 x d]   rows2 = requests x q heads x stride (only with > 1 group)
// (q heads bound the KV heads the tickets are indexed by.)  ticket_groups bounds the merge
// groups of every partition size (partitions hold at least 64 tokens), so the tickets' place
// and size depend only on (requests, q heads, max_seq_len).  Every launch leaves its tickets
// and counters at zero, so a workspace reused with another partition size, block size, cache type, head dim or
// device finds zeros where its tickets are, never a stale partial row.
struct WsLayout {
    int64_t ctr_off, m_off, l_off, acc_off, m2_off, l2_off, acc2_off, bytes;
    int groups, stride;
};

WsLayout ws_layout(int64_t seqs_x_heads, int64_t max_seq_len, int64_t parts, int d) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    WsLayout w;
    w.groups = static_cast<int>((parts + kMergeGroup - 1) / kMergeGroup);
    const int64_t max_parts_any = (std::max<int64_t>(max_seq_len, 1) + 63) / 64;
    w.stride = static_cast<int>((max_parts_any + kMergeGroup - 1) / kMergeGroup) + 1;
    const int64_t rows1 = seqs_x_heads * parts, rows2 = w.groups > 1 ? seqs_x_heads * w.stride : 0;
    w.ctr_off = 0;
    w.m_off = up((seqs_x_heads * w.stride + 2) * 4);   // + the item list's claim and exit counters
    w.l_off = w.m_off + up(rows1 * 4);
    w.acc_off = w.l_off + up(rows1 * 4);
    w.m2_off = w.acc_off + up(rows1 * int64_t(d) * 4);
    w.l2_off = w.m2_off + up(rows2 * 4);
    w.acc2_off = w.l2_off + up(rows2 * 4);
    w.bytes = w.acc2_off + up(rows2 * int64_t(d) * 4);
    return w;
}

// Resident work-groups per compute unit of the matrix-core decode kernel instance
// <CDT, QDT, D, BS, G, NW> at a given dynamic LDS size (cached per instance for the last size
// asked: every instance has the same function type, so the cache is keyed by the template
// arguments, not by the type).
template <int CDT, int QDT, int D, int BS, int G, int NW, bool DYN>
int resident_per_cu(int dyn_lds) {
    static std::atomic<int64_t> cache{-1};
    const int64_t c = cache.load(std::memory_order_relaxed);
    if (c >= 0 && int(c >> 32) == dyn_lds) return int(c & 0xffffffff);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<CDT, QDT, D, BS, G, NW, DYN>, 64 * NW,
                                                     dyn_lds) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 1;
    }
    cache.store((int64_t(dyn_lds) << 32) | n, std::memory_order_relaxed);
    return n;
}

template <int CDT, int QDT, int D, int BS, int G>
int launch_decode(DecodeArgs a, int B, hipStream_t st) {
    if constexpr (CDT == PA_DTYPE_F32) {
        dim3 grid(a.max_parts, a.hkv, B);
        hipLaunchKernelGGL((decode_valu_kernel<CDT, QDT, D, BS, G>), grid, dim3(kThreads), 0, st, a);
    } else {
        // The (partition, KV head, request) grid of kWaves-wave work-groups is used when all
        // of it is resident at once (uniform batches: no work-group waits for a slot, none of
        // them is empty); otherwise, up to kMaxListSeqs requests, the compact item list on
        // about one kListWaves-wave work-group per slot.
        const int64_t grid_items = int64_t(B) * a.max_parts * a.hkv;
        const int lds = (B + 1) * 4;
        const int64_t cus = device_cu_count();
        const int64_t grid_slots = B <= kMaxListSeqs ? cus * resident_per_cu<CDT, QDT, D, BS, G, kWaves, false>(0) : 0;
        if (B <= kMaxListSeqs && grid_items > grid_slots) {
            a.list = 1;
            const int64_t slots = cus * resident_per_cu<CDT, QDT, D, BS, G, kListWaves, false>(lds);
            // a few long requests (at most a quarter as many (request, KV head) pairs as slots)
            // over a bf16 cache: the instance that may hand out the last items by a counter
            bool counted = false;
            if constexpr (CDT == PA_DTYPE_BF16) {
                if (int64_t(B) * a.hkv * 4 <= slots) {
                    const int64_t dslots = cus * resident_per_cu<CDT, QDT, D, BS, G, kListWaves, true>(lds);
                    hipLaunchKernelGGL((decode_mfma_kernel<CDT, QDT, D, BS, G, kListWaves, true>),
                                       dim3(static_cast<int>(dslots)), dim3(64 * kListWaves), lds, st, a);
                    counted = true;
                }
            }
            if (!counted) {
                hipLaunchKernelGGL((decode_mfma_kernel<CDT, QDT, D, BS, G, kListWaves, false>),
                                   dim3(static_cast<int>(slots)), dim3(64 * kListWaves), lds, st, a);
            }
        } else {
            a.list = 0;
            hipLaunchKernelGGL((decode_mfma_kernel<CDT, QDT, D, BS, G, kWaves, false>), dim3(a.max_parts, a.hkv, B),
                               dim3(kThreads), 0, st, a);
        }
    }
    return check_launch("pa_decode");
}

template <int CDT, int QDT, int D, int BS>
int dispatch_g(int G, const DecodeArgs& a, int B, hipStream_t st) {
    switch (G) {
        case 1: return launch_decode<CDT, QDT, D, BS, 1>(a, B, st);
        case 4: return launch_decode<CDT, QDT, D, BS, 4>(a, B, st);
        case 8: return launch_decode<CDT, QDT, D, BS, 8>(a, B, st);
    }
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: num_q_heads/num_kv_heads = %d not in {1, 4, 8}", G);
}

template <int CDT, int QDT, int D>
int dispatch_bs(int BS, int G, const DecodeArgs& a, int B, hipStream_t st) {
    switch (BS) {
        case 8: return dispatch_g<CDT, QDT, D, 8>(G, a, B, st);
        case 16: return dispatch_g<CDT, QDT, D, 16>(G, a, B, st);
        case 32: return dispatch_g<CDT, QDT, D, 32>(G, a, B, st);
        case 128: return dispatch_g<CDT, QDT, D, 128>(G, a, B, st);
    }
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d not in {8, 16, 32, 128}", BS);
}

template <int CDT, int QDT>
int dispatch_d(int D, int BS, int G, const DecodeArgs& a, int B, hipStream_t st) {
    switch (D) {
        case 64: return dispatch_bs<CDT, QDT, 64>(BS, G, a, B, st);
        case 128: return dispatch_bs<CDT, QDT, 128>(BS, G, a, B, st);
    }
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not in {64, 128}", D);
}

bool supported_pair(int qdt, int cdt) {
    return (qdt == PA_DTYPE_F32 && cdt == PA_DTYPE_F32) || (qdt == PA_DTYPE_BF16 && cdt == PA_DTYPE_BF16) ||
           (qdt == PA_DTYPE_BF16 && cdt == PA_DTYPE_FP8_E4M3) || (qdt == PA_DTYPE_BF16 && cdt == PA_DTYPE_MXFP4);
}

// Per device: the fixed scratch's device address and how many of its leading bytes are zero once
// the device has passed the calls enqueued so far (the next call's tickets must start at zero).
struct ScratchDevice {
    void* ptr = nullptr;
    int64_t zero_bytes = 0;
};
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
ScratchDevice g_scratch[kMaxScratchDevices];

int decode_call(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* seq_lens, float scale,
                int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
                const float* k_scale, const float* v_scale,
                void* workspace, int64_t workspace_bytes, int32_t partition_tokens, void* stream,
                const void* k_new, const void* v_new) {
    if (!supported_pair(q_dtype, cache_dtype))
        return fail(PA_ERR_UNSUPPORTED, "%s: (q dtype %d, cache dtype %d) not supported", fn, q_dtype, cache_dtype);
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq < 0 ||
        max_seq_len < 0 || partition_tokens < 0)
        return fail(PA_ERR_INVALID, "%s: negative or zero size", fn);
    if (num_q_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID, "%s: num_q_heads %d not a multiple of num_kv_heads %d", fn, num_q_heads, num_kv_heads);
    if (!(scale == scale)) return fail(PA_ERR_INVALID, "%s: scale is NaN", fn);
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !seq_lens || (max_blocks_per_seq > 0 && !block_tables))
        return fail(PA_ERR_INVALID, "%s: NULL pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "%s: out, q and caches must be 16-byte aligned", fn);
    if (cache_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID, "%s: fp8 cache needs k_scale and v_scale", fn);
    if (int64_t(max_blocks_per_seq) * block_size < max_seq_len)
        return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq * block_size < max_seq_len", fn);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d not in {8, 16, 32, 128}", fn, block_size);

    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.k_new = k_new;
    a.v_new = v_new;
    a.score_scale = scale * kLog2e;
    a.num_seqs = num_seqs;
    a.hkv = num_kv_heads;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.max_seq_len = max_seq_len;

    const int unit = partition_unit(block_size);
    int64_t pt = resolve_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens, block_size, cache_dtype);
    int64_t parts = max_seq_len > 0 ? (int64_t(max_seq_len) + pt - 1) / pt : 1;
    if (parts > 1) {
        const WsLayout lay = ws_layout(int64_t(num_seqs) * num_q_heads, max_seq_len, parts, head_dim);
        if (!workspace) {
            // no workspace: one partition per request
            pt = (max_seq_len + unit - 1) / unit * unit;
            parts = 1;
        } else if (workspace_bytes < lay.bytes || !aligned16(workspace)) {
            return fail(PA_ERR_INVALID, "%s: workspace of %lld bytes, %lld needed (16-byte aligned)", fn,
                        (long long)workspace_bytes, (long long)lay.bytes);
        } else {
            char* base = static_cast<char*>(workspace);
            a.ws_ctr = reinterpret_cast<int*>(base + lay.ctr_off);
            a.ctr_stride = lay.stride;
            a.ws_m2 = reinterpret_cast<float*>(base + lay.m2_off);
            a.ws_l2 = reinterpret_cast<float*>(base + lay.l2_off);
            a.ws_acc2 = reinterpret_cast<float*>(base + lay.acc2_off);
            a.ws_m = reinterpret_cast<float*>(base + lay.m_off);
            a.ws_l = reinterpret_cast<float*>(base + lay.l_off);
            a.ws_acc = reinterpret_cast<float*>(base + lay.acc_off);
        }
    }
    if (pt > int64_t(max_seq_len) + unit) pt = (int64_t(max_seq_len) + unit - 1) / unit * unit;   // one partition
    if (pt < unit) pt = unit;
    if (parts > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: %lld partitions per request", fn, (long long)parts);
    a.part_tokens = static_cast<int>(pt);
    a.max_parts = static_cast<int>(parts);

    const int G = num_q_heads / num_kv_heads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (cache_dtype == PA_DTYPE_F32)
        return dispatch_d<PA_DTYPE_F32, PA_DTYPE_F32>(head_dim, block_size, G, a, num_seqs, st);
    if (cache_dtype == PA_DTYPE_BF16)
        return dispatch_d<PA_DTYPE_BF16, PA_DTYPE_BF16>(head_dim, block_size, G, a, num_seqs, st);
    if (cache_dtype == PA_DTYPE_MXFP4)
        return dispatch_d<PA_DTYPE_MXFP4, PA_DTYPE_BF16>(head_dim, block_size, G, a, num_seqs, st);
    return dispatch_d<PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16>(head_dim, block_size, G, a, num_seqs, st);
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

int pa_kv_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int32_t in_dtype, int32_t cache_dtype,
                const float* k_scale, const float* v_scale, void* stream) {
    pagedkv::clear_error();
    if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0)
        return fail(PA_ERR_INVALID, "pa_kv_write: num_tokens=%lld num_blocks=%lld num_kv_heads=%d",
                    (long long)num_tokens, (long long)num_blocks, num_kv_heads);
    if (!supported_pair(in_dtype, cache_dtype) && !(in_dtype == PA_DTYPE_F32 && cache_dtype == PA_DTYPE_FP8_E4M3))
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: (input dtype %d, cache dtype %d) not supported", in_dtype, cache_dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: head_dim %d not in {64, 128}", head_dim);
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: block_size %d not in {8, 16, 32, 128}", block_size);
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_kv_write: caches must be non-NULL and 16-byte aligned");
    if (cache_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID, "pa_kv_write: fp8 cache needs k_scale and v_scale");
    if (cache_dtype == PA_DTYPE_MXFP4 && (k_scale || v_scale))
        return fail(PA_ERR_INVALID, "pa_kv_write: an MXFP4 cache carries its own scales (k_scale, v_scale must be NULL)");
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v))
        return fail(PA_ERR_INVALID, "pa_kv_write: k, v, slot_mapping must be non-NULL; k, v 16-byte aligned");
    const int64_t work = num_tokens * num_kv_heads * (head_dim / 8);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t num_slots = num_blocks * block_size;
    const int grid = grid_for(work, 256);
    if (cache_dtype == PA_DTYPE_F32) {
        hipLaunchKernelGGL((kv_write_kernel<PA_DTYPE_F32, PA_DTYPE_F32>), dim3(grid), dim3(256), 0, st,
                           (const float*)k, (const float*)v, slot_mapping, num_tokens, (float*)k_cache,
                           (float*)v_cache, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale);
    } else if (cache_dtype == PA_DTYPE_BF16) {
        hipLaunchKernelGGL((kv_write_kernel<PA_DTYPE_BF16, PA_DTYPE_BF16>), dim3(grid), dim3(256), 0, st,
                           (const uint16_t*)k, (const uint16_t*)v, slot_mapping, num_tokens, (uint16_t*)k_cache,
                           (uint16_t*)v_cache, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale);
    } else if (cache_dtype == PA_DTYPE_FP8_E4M3 && in_dtype == PA_DTYPE_F32) {
        hipLaunchKernelGGL((kv_write_kernel<PA_DTYPE_F32, PA_DTYPE_FP8_E4M3>), dim3(grid), dim3(256), 0, st,
                           (const float*)k, (const float*)v, slot_mapping, num_tokens, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale);
    } else if (cache_dtype == PA_DTYPE_FP8_E4M3) {
        hipLaunchKernelGGL((kv_write_kernel<PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3>), dim3(grid), dim3(256), 0, st,
                           (const uint16_t*)k, (const uint16_t*)v, slot_mapping, num_tokens, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale);
    } else {
        const int mx_grid = grid_for(num_tokens * num_kv_heads * (head_dim / 32), 256);
        hipLaunchKernelGGL(kv_write_mx4_kernel, dim3(mx_grid), dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v,
                           slot_mapping, num_tokens, (uint8_t*)k_cache, (uint8_t*)v_cache, num_slots, num_kv_heads,
                           head_dim, block_size);
    }
    return check_launch("pa_kv_write");
}

int64_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t partition_tokens,
                                  int32_t block_size, int32_t cache_dtype) {
    pagedkv::clear_error();
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
        max_seq_len < 0 || partition_tokens < 0 || block_size <= 0) {
        return fail(PA_ERR_INVALID, "pa_decode_workspace_bytes: bad sizes");
    }
    const int64_t pt = resolve_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens, block_size, cache_dtype);
    const int64_t parts = max_seq_len > 0 ? (int64_t(max_seq_len) + pt - 1) / pt : 1;
    if (parts <= 1) return 0;
    return ws_layout(int64_t(num_seqs) * num_q_heads, max_seq_len, parts, head_dim).bytes;
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, int32_t block_size, int32_t cache_dtype) {
    pagedkv::clear_error();
    if (num_seqs < 0 || num_kv_heads <= 0 || max_seq_len < 0 || partition_tokens < 0 || block_size <= 0)
        return fail(PA_ERR_INVALID, "pa_decode_partition_tokens: bad sizes");
    const int64_t pt = resolve_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens, block_size, cache_dtype);
    return pt > 0x3fffffff ? 0x3fffffff : static_cast<int32_t>(pt);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, float scale,
              int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
              const float* k_scale, const float* v_scale,
              void* workspace, int64_t workspace_bytes, int32_t partition_tokens, void* stream) {
    pagedkv::clear_error();
    return decode_call("pa_decode", out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_seq_len, q_dtype,
                       cache_dtype, k_scale, v_scale, workspace, workspace_bytes, partition_tokens, stream, nullptr,
                       nullptr);
}

int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens, float scale, int32_t block_size,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t q_dtype,
                     int32_t cache_dtype, const float* k_scale, const float* v_scale, void* workspace,
                     int64_t workspace_bytes, int32_t partition_tokens, void* stream) {
    pagedkv::clear_error();
    if (cache_dtype == PA_DTYPE_F32 || q_dtype == PA_DTYPE_F32)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_append: float32 caches (use pa_kv_write, then pa_decode)");
    if (num_seqs > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)))
        return fail(PA_ERR_INVALID, "pa_decode_append: k_new and v_new must be non-NULL and 16-byte aligned");
    return decode_call("pa_decode_append", out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_seq_len,
                       q_dtype, cache_dtype, k_scale, v_scale, workspace, workspace_bytes, partition_tokens, stream,
                       k_new, v_new);
}

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
                      const float* k_scale, const float* v_scale, int32_t partition_tokens, void* stream) {
    pagedkv::clear_error();
    const int64_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                   partition_tokens, block_size, cache_dtype);
    if (need <= 0 || num_seqs == 0)   // a single partition per request (no scratch), or sizes pa_decode rejects
        return pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype,
                         k_scale, v_scale, nullptr, 0, partition_tokens, stream);
    if (need > int64_t(PA_NOALLOC_SCRATCH_BYTES))
        return fail(PA_ERR_INVALID,
                    "pa_decode_noalloc: these sizes need %lld bytes of split-K scratch, more than the fixed %lld "
                    "(call pa_decode with a workspace)", (long long)need, (long long)PA_NOALLOC_SCRATCH_BYTES);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        (void)hipGetLastError();
        return fail(PA_ERR_DEVICE, "pa_decode_noalloc: no current device below %d", kMaxScratchDevices);
    }
    const int64_t pt = resolve_partition(num_seqs, num_kv_heads, max_seq_len, partition_tokens, block_size, cache_dtype);
    const int64_t parts = (int64_t(max_seq_len) + pt - 1) / pt;
    const int64_t tickets = ws_layout(int64_t(num_seqs) * num_q_heads, max_seq_len, parts, head_dim).m_off;

    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchDevice& sd = g_scratch[dev];
    if (!sd.ptr) {   // first call on this device, with it current: look the array's address up once
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(PA_ERR_DEVICE, "pa_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        }
        sd.ptr = p;
        sd.zero_bytes = 0;   // the contents at load are not relied on
    }
    char* base = static_cast<char*>(sd.ptr);
    if (sd.zero_bytes < tickets) {   // the tickets must start at zero: clear what earlier calls left there
        const int64_t words = (tickets - sd.zero_bytes) / 4;
        hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                           reinterpret_cast<uint32_t*>(base + sd.zero_bytes), words);
        if (int rc = check_launch("pa_decode_noalloc")) return rc;
        sd.zero_bytes = tickets;
    }
    const int rc = pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_seq_len, q_dtype,
                             cache_dtype, k_scale, v_scale, base, int64_t(PA_NOALLOC_SCRATCH_BYTES), partition_tokens,
                             stream);
    if (rc == PA_OK) sd.zero_bytes = tickets;   // partial rows follow the tickets, which the launch leaves at zero
    return rc;
}

int pa_decode_workspace_init(void* workspace, int64_t workspace_bytes, void* stream) {
    pagedkv::clear_error();
    if (workspace_bytes < 0 || workspace_bytes % 4 != 0)
        return fail(PA_ERR_INVALID, "pa_decode_workspace_init: %lld bytes is not a multiple of 4", (long long)workspace_bytes);
    if (workspace_bytes == 0) return PA_OK;
    if (!workspace || !aligned16(workspace))
        return fail(PA_ERR_INVALID, "pa_decode_workspace_init: NULL or misaligned workspace");
    const int64_t words = workspace_bytes / 4;
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(workspace), words);
    return check_launch("pa_decode_workspace_init");
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst, int32_t num_pairs,
                   int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t cache_dtype, void* stream) {
    pagedkv::clear_error();
    if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID, "pa_copy_blocks: bad sizes");
    const int64_t tb = tile_bytes(cache_dtype, block_size, head_dim);
    if (tb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: cache dtype %d", cache_dtype);
    const int64_t block_bytes = int64_t(num_kv_heads) * tb;
    if (block_bytes % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block of %lld bytes", (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !src_dst || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_copy_blocks: NULL or misaligned pointer");
    const int grid = grid_for(int64_t(num_pairs) * (block_bytes / 16), 256);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), src_dst,
                       num_pairs, num_blocks, num_blocks, block_bytes);
    return check_launch("pa_copy_blocks");
}

int pa_upload(void* dst, const void* src, int64_t bytes, void* stream) {
    pagedkv::clear_error();
    if (bytes < 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 31))
        return fail(PA_ERR_INVALID, "pa_upload: %lld bytes (a multiple of 16 below 2^31)", (long long)bytes);
    if (bytes == 0) return PA_OK;
    if (!dst || !src || !aligned16(dst) || !aligned16(src))
        return fail(PA_ERR_INVALID, "pa_upload: NULL or misaligned pointer");
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), s0 = reinterpret_cast<uintptr_t>(src);
    if (d0 < s0 + static_cast<uintptr_t>(bytes) && s0 < d0 + static_cast<uintptr_t>(bytes))
        return fail(PA_ERR_INVALID, "pa_upload: source and destination overlap");
    const void *dv, *sv;
    if (int rc = device_view(dst, bytes, "pa_upload", "dst", &dv)) return rc;
    if (int rc = device_view(src, bytes, "pa_upload", "src", &sv)) return rc;
    const int n16 = static_cast<int>(bytes / 16);
    hipLaunchKernelGGL(upload_kernel, dim3(grid_for(n16, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(const_cast<void*>(dv)), static_cast<const uint8_t*>(sv), n16);
    return check_launch("pa_upload");
}

int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int64_t* src_dst, int32_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t cache_dtype, void* stream) {
    pagedkv::clear_error();
    if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0)
        return fail(PA_ERR_INVALID, "pa_swap_blocks: bad sizes");
    const int64_t tb = tile_bytes(cache_dtype, block_size, head_dim);
    if (tb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: cache dtype %d", cache_dtype);
    const int64_t block_bytes = int64_t(num_kv_heads) * tb;
    if (block_bytes % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: block of %lld bytes", (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!dst_k || !dst_v || !src_k || !src_v || !src_dst || !aligned16(dst_k) || !aligned16(dst_v) ||
        !aligned16(src_k) || !aligned16(src_v) || reinterpret_cast<uintptr_t>(src_dst) % 8 != 0)
        return fail(PA_ERR_INVALID, "pa_swap_blocks: NULL or misaligned pointer");
    const void *dk, *dv, *sk, *sv, *pr;
    if (int rc = device_view(dst_k, dst_num_blocks * block_bytes, "pa_swap_blocks", "dst_k", &dk)) return rc;
    if (int rc = device_view(dst_v, dst_num_blocks * block_bytes, "pa_swap_blocks", "dst_v", &dv)) return rc;
    if (int rc = device_view(src_k, src_num_blocks * block_bytes, "pa_swap_blocks", "src_k", &sk)) return rc;
    if (int rc = device_view(src_v, src_num_blocks * block_bytes, "pa_swap_blocks", "src_v", &sv)) return rc;
    if (int rc = device_view(src_dst, int64_t(num_pairs) * 16, "pa_swap_blocks", "src_dst", &pr)) return rc;
    const int grid = grid_for(int64_t(num_pairs) * (block_bytes / 16), 256);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(const_cast<void*>(dk)), static_cast<uint8_t*>(const_cast<void*>(dv)),
                       static_cast<const uint8_t*>(sk), static_cast<const uint8_t*>(sv),
                       static_cast<const int64_t*>(pr), num_pairs, src_num_blocks, dst_num_blocks, block_bytes);
    return check_launch("pa_swap_blocks");
}

}  // extern "C"
