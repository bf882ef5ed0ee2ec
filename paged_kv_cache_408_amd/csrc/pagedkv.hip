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
//  decode_partial_kernel one work-group (4 wave64) per (partition, KV head, request).  The
//                        G = Hq/Hkv query heads of a KV head share every K/V load, so each
//                        cached byte is read once.  Per pass of TPP tokens a wave:
//                          K phase: KL lanes per token row, each lane a few 16-byte loads of
//                            that row (every group of 4 lanes reads 64 contiguous bytes);
//                            partial dot products with the lane's slice of q (v_dot2 on
//                            bf16 pairs), reduced across the KL lanes;
//                          online softmax: wave max of the pass, rescale of the running
//                            state, p = exp2(s - m) (scores carry scale * log2(e));
//                          V phase: one 16-byte vector of a row per lane, consecutive lanes
//                            covering consecutive bytes (1 KiB per wave load); p is handed
//                            from the K-phase lanes through LDS; acc[h][dims] += p * v.
//                        The 4 waves' states are merged in LDS; a single-partition request
//                        writes `out`, otherwise (m, l, acc) goes to the workspace.
//  decode_merge_kernel   log-sum-exp merge of the partitions of each (request, q head).
//  copy_blocks_kernel    whole-block copies for copy-on-write.
//
// Reduction order depends only on logical token positions (never on physical block ids),
// so results are bit-identical under any placement of the blocks.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element formats

template <int DT> struct Elem;
template <> struct Elem<PA_DTYPE_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elem<PA_DTYPE_BF16> { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Elem<PA_DTYPE_FP8_E4M3> { using T = uint8_t; static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

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

// ------------------------------------------------------------------ cross-lane helpers

__device__ __forceinline__ float xor_shfl(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct alignas(16) U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 ld16(const void* p) { return *reinterpret_cast<const U4*>(p); }

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
            static_assert(CDT == PA_DTYPE_FP8_E4M3 && IDT == PA_DTYPE_BF16, "unsupported pair");
            const float ks = k_scale[h], vs = v_scale[h];
            const U4 kx = ld16(k + src), vx = ld16(v + src);
            uint32_t ko[2] = {0, 0}, vo[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t kw = u4_get(kx, i / 2), vw = u4_get(vx, i / 2);
                const uint32_t kb = (i & 1) ? (kw >> 16) : (kw & 0xffffu);
                const uint32_t vb = (i & 1) ? (vw >> 16) : (vw & 0xffffu);
                // correctly rounded float32 quotient (IEEE division, no fast-math)
                const uint32_t kq = f32_to_e4m3(bf16_to_f32(kb) / ks);
                const uint32_t vq = f32_to_e4m3(bf16_to_f32(vb) / vs);
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

// ------------------------------------------------------------------ block copy

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                          const int64_t* __restrict__ pairs, int num_pairs,
                                                          int64_t num_blocks, int64_t block_bytes) {
    const int64_t vec_per_block = block_bytes / 16;
    const int64_t total = int64_t(num_pairs) * vec_per_block;
    for (int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; gid < total;
         gid += int64_t(gridDim.x) * blockDim.x) {
        const int64_t pi = gid / vec_per_block;
        const int64_t off = (gid - pi * vec_per_block) * 16;
        const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        *reinterpret_cast<U4*>(kc + dst * block_bytes + off) = ld16(kc + src * block_bytes + off);
        *reinterpret_cast<U4*>(vc + dst * block_bytes + off) = ld16(vc + src * block_bytes + off);
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

inline int effective_partition(int requested, int unit) {
    int pt = requested > 0 ? requested : 512;
    return (pt + unit - 1) / unit * unit;
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
    float* ws_m;
    float* ws_l;
    float* ws_acc;
    float score_scale;     // scale * log2(e)
    int hkv;
    int64_t num_blocks;
    int max_blocks;
    int max_seq_len;
    int part_tokens;
    int max_parts;
};

// ------------------------------------------------------------------ decode: pass 1

template <int CDT, int QDT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeArgs a) {
    using C = Cfg<CDT, D, BS, G>;
    using CT = typename Elem<CDT>::T;
    using QT = typename Elem<QDT>::T;
    constexpr bool kDot2 = CDT == PA_DTYPE_BF16;   // bf16 cache: v_dot2 on packed pairs

    __shared__ float s_p[kWaves][C::TPP][G];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ float s_acc[kWaves][G][D];

    const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int hq = a.hkv * G;

    const int L_raw = a.seq_lens[b];
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

    const int t0 = part * a.part_tokens;
    const int t1 = min(L, t0 + a.part_tokens);
    const int npass = (t1 - t0 + C::TPP - 1) / C::TPP;
    const int nblk = (L + BS - 1) / BS;
    const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks;
    const CT* kbase = reinterpret_cast<const CT*>(a.k_cache);
    const CT* vbase = reinterpret_cast<const CT*>(a.v_cache);

    float sc = a.score_scale;
    float vsc = 1.0f;
    if constexpr (CDT == PA_DTYPE_FP8_E4M3) {
        sc *= a.k_scale[g];
        vsc = a.v_scale[g];
    }

    // ---- q slice of this lane (K-phase layout): vectors j*KL + c of the row
    const int krow = lane / C::KL, kc = lane % C::KL;
    const QT* qrow = reinterpret_cast<const QT*>(a.q) + (int64_t(b) * hq + int64_t(g) * G) * D;
    uint32_t qpk[kDot2 ? G : 1][kDot2 ? C::EPL / 2 : 1];
    float qf[kDot2 ? 1 : G][kDot2 ? 1 : C::EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int j = 0; j < C::KVPL; ++j) {
            const int d0 = (j * C::KL + kc) * C::EPV;
            if constexpr (kDot2) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(qrow + h * D + d0);
#pragma unroll
                for (int e = 0; e < C::EPV / 2; ++e) qpk[h][j * (C::EPV / 2) + e] = src[e];
            } else {
#pragma unroll
                for (int e = 0; e < C::EPV; ++e) {
                    const QT x = qrow[h * D + d0 + e];
                    if constexpr (QDT == PA_DTYPE_BF16) qf[h][j * C::EPV + e] = bf16_to_f32(x);
                    else qf[h][j * C::EPV + e] = x;
                }
            }
        }
    }

    float m_run[G], l_run[G], acc[G][C::EPV];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < C::EPV; ++e) acc[h][e] = 0.0f;
    }
    bool bad = false;
    const int vrg = lane / C::VL, vcol = lane % C::VL;

    for (int i = w; i < npass; i += kWaves) {
        const int tbase = t0 + i * C::TPP;
        // ---- block ids of this pass (uniform scalar loads; clamped to the live entries)
        const int e0 = tbase / BS;
        int blk[C::BPP];
#pragma unroll
        for (int q2 = 0; q2 < C::BPP; ++q2) {
            const int e = min(e0 + q2, nblk - 1);
            int id = table[e];
            if (id < 0 || id >= a.num_blocks) {
                // only an error if a live token of this pass lies in that block
                if ((e0 + q2) * BS < t1) bad = true;
                id = 0;
            }
            blk[q2] = id;
        }
        // ---- issue K and V loads
        const int tk = tbase + krow;
        const bool kvalid = tk < t1;
        U4 kv[C::KVPL];
        {
            const int bi = C::BPP == 1 ? 0 : (krow / BS);
            const CT* rowp = kbase + ((int64_t(blk[bi]) * a.hkv + g) * BS + (tk % BS)) * D;
#pragma unroll
            for (int j = 0; j < C::KVPL; ++j) {
                kv[j] = kvalid ? ld16(rowp + (j * C::KL + kc) * C::EPV) : U4{0, 0, 0, 0};
            }
        }
        U4 vv[C::VR];
#pragma unroll
        for (int r = 0; r < C::VR; ++r) {
            const int row = vrg + r * C::VRG;
            const int tv = tbase + row;
            const int bi = C::BPP == 1 ? 0 : (row / BS);
            const CT* rowp = vbase + ((int64_t(blk[bi]) * a.hkv + g) * BS + (tv % BS)) * D;
            vv[r] = tv < t1 ? ld16(rowp + vcol * C::EPV) : U4{0, 0, 0, 0};
        }

        // ---- scores of this lane's token for the G heads
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float accs = 0.0f;
#pragma unroll
            for (int j = 0; j < C::KVPL; ++j) {
                if constexpr (kDot2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        accs = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2v, qpk[h][j * 4 + e]),
                            __builtin_bit_cast(bf16x2v, u4_get(kv[j], e)), accs, false);
                    }
                } else if constexpr (CDT == PA_DTYPE_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        accs = fmaf(qf[h][j * 4 + e], __uint_as_float(u4_get(kv[j], e)), accs);
                } else {  // fp8
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wv = u4_get(kv[j], e);
                        const float2v lo = e4m3x2_to_f32<false>(wv);
                        const float2v hi = e4m3x2_to_f32<true>(wv);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 0], lo.x, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 1], lo.y, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 2], hi.x, accs);
                        accs = fmaf(qf[h][j * 16 + 4 * e + 3], hi.y, accs);
                    }
                }
            }
#pragma unroll
            for (int m = 1; m < C::KL; m <<= 1) accs += xor_shfl(accs, m);
            s[h] = kvalid ? accs * sc : -INFINITY;
        }

        // ---- online softmax over the pass
        float p[G], alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[h];
#pragma unroll
            for (int m = C::KL; m < 64; m <<= 1) mx = fmaxf(mx, xor_shfl(mx, m));
            const float m_new = fmaxf(m_run[h], mx);
            alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);
            p[h] = __builtin_amdgcn_exp2f(s[h] - m_new);
            m_run[h] = m_new;
        }
        if (kc == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) s_p[w][krow][h] = p[h];
        }
        wave_sync_lds();

        // ---- V phase
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l_run[h] *= alpha[h];
#pragma unroll
            for (int e = 0; e < C::EPV; ++e) acc[h][e] *= alpha[h];
        }
#pragma unroll
        for (int r = 0; r < C::VR; ++r) {
            const int row = vrg + r * C::VRG;
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = s_p[w][row][h];
            float vf[C::EPV];
            if constexpr (CDT == PA_DTYPE_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[e] = __uint_as_float(u4_get(vv[r], e));
            } else if constexpr (CDT == PA_DTYPE_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = u4_get(vv[r], e);
                    vf[2 * e] = __uint_as_float(x << 16);
                    vf[2 * e + 1] = __uint_as_float(x & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = u4_get(vv[r], e);
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
                for (int e = 0; e < C::EPV; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
            }
        }
        wave_sync_lds();   // s_p is rewritten by the next pass
    }

    // ---- reduce the V-phase row groups of this wave
#pragma unroll
    for (int m = C::VL; m < 64; m <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            l_run[h] += xor_shfl(l_run[h], m);
#pragma unroll
            for (int e = 0; e < C::EPV; ++e) acc[h][e] += xor_shfl(acc[h][e], m);
        }
    }
    if (lane < C::VL) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < C::EPV; ++e) s_acc[w][h][lane * C::EPV + e] = acc[h][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[w][h] = m_run[h];
            s_l[w][h] = l_run[h];
        }
    }
    const bool any_bad = __syncthreads_or(bad);

    // ---- merge the waves (fixed order) and write
    const bool single = nparts == 1;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D, dim = idx - h * D;
        float M = s_m[0][h];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = __builtin_amdgcn_exp2f(s_m[ww][h] - M);   // 0 for an idle wave
            num = fmaf(f, s_acc[ww][h][dim], num);
            den = fmaf(f, s_l[ww][h], den);
        }
        if (any_bad) {
            num = __builtin_nanf("");
            den = __builtin_nanf("");
            M = __builtin_nanf("");
        }
        if (single) {
            const float o = num / den * vsc;
            if constexpr (QDT == PA_DTYPE_BF16) out[idx] = f32_to_bf16(o); else out[idx] = o;
        } else {
            const int64_t row = (int64_t(b) * hq + int64_t(g) * G + h) * a.max_parts + part;
            a.ws_acc[row * D + dim] = num * vsc;
            if (dim == 0) {
                a.ws_m[row] = M;
                a.ws_l[row] = den;
            }
        }
    }
}

// ------------------------------------------------------------------ decode: merge

template <int QDT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const DecodeArgs a, int block_size) {
    using QT = typename Elem<QDT>::T;
    const int h = blockIdx.x, b = blockIdx.y;
    const int hq = gridDim.x;
    const int L_raw = a.seq_lens[b];
    const bool len_bad = L_raw < 0 || L_raw > a.max_seq_len || L_raw > a.max_blocks * block_size;
    const int L = len_bad ? 0 : L_raw;
    const int nparts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
    if (nparts <= 1) return;   // written by the partition kernel
    const int64_t row0 = (int64_t(b) * hq + h) * a.max_parts;
    const int dim = threadIdx.x;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_m[row0 + p]);
    float num = 0.0f, den = 0.0f;
    for (int p = 0; p < nparts; ++p) {
        const float f = __builtin_amdgcn_exp2f(a.ws_m[row0 + p] - M);
        num = fmaf(f, a.ws_acc[(row0 + p) * D + dim], num);
        den = fmaf(f, a.ws_l[row0 + p], den);
    }
    // a NaN partial (bad block id) must win over fmaxf's NaN-dropping
    for (int p = 0; p < nparts; ++p) {
        if (__builtin_isnan(a.ws_m[row0 + p])) den = __builtin_nanf("");
    }
    const float o = num / den;
    QT* out = reinterpret_cast<QT*>(a.out) + (int64_t(b) * hq + h) * D;
    if constexpr (QDT == PA_DTYPE_BF16) out[dim] = f32_to_bf16(o); else out[dim] = o;
}

// ------------------------------------------------------------------ host helpers

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dt) { return dt == PA_DTYPE_F32 ? 4 : dt == PA_DTYPE_BF16 ? 2 : dt == PA_DTYPE_FP8_E4M3 ? 1 : 0; }

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PA_OK;
}

int grid_for(int64_t work, int per_block) {
    int64_t blocks = (work + per_block - 1) / per_block;
    if (blocks > 65536) blocks = 65536;  // grid-stride loops cover the rest
    return static_cast<int>(blocks < 1 ? 1 : blocks);
}

struct WsLayout {
    int64_t m_off, l_off, acc_off, bytes;
};

WsLayout ws_layout(int64_t rows, int d) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    WsLayout w;
    w.m_off = 0;
    w.l_off = up(rows * 4);
    w.acc_off = w.l_off + up(rows * 4);
    w.bytes = w.acc_off + up(rows * int64_t(d) * 4);
    return w;
}

template <int CDT, int QDT, int D, int BS, int G>
int launch_decode(const DecodeArgs& a, int B, hipStream_t st) {
    dim3 grid(a.max_parts, a.hkv, B);
    hipLaunchKernelGGL((decode_partial_kernel<CDT, QDT, D, BS, G>), grid, dim3(kThreads), 0, st, a);
    int rc = check_launch("pa_decode (partition pass)");
    if (rc != PA_OK) return rc;
    if (a.max_parts > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<QDT, D>), dim3(a.hkv * G, B), dim3(D), 0, st, a, BS);
        rc = check_launch("pa_decode (merge)");
    }
    return rc;
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
           (qdt == PA_DTYPE_BF16 && cdt == PA_DTYPE_FP8_E4M3);
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
    if (!supported_pair(in_dtype, cache_dtype))
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: (input dtype %d, cache dtype %d) not supported", in_dtype, cache_dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: head_dim %d not in {64, 128}", head_dim);
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_kv_write: block_size %d not in {8, 16, 32, 128}", block_size);
    if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_kv_write: caches must be non-NULL and 16-byte aligned");
    if (cache_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID, "pa_kv_write: fp8 cache needs k_scale and v_scale");
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
    } else {
        hipLaunchKernelGGL((kv_write_kernel<PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3>), dim3(grid), dim3(256), 0, st,
                           (const uint16_t*)k, (const uint16_t*)v, slot_mapping, num_tokens, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale);
    }
    return check_launch("pa_kv_write");
}

int64_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition_tokens, int32_t block_size) {
    pagedkv::clear_error();
    if (num_seqs < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) || max_seq_len < 0 ||
        block_size <= 0) {
        return fail(PA_ERR_INVALID, "pa_decode_workspace_bytes: bad sizes");
    }
    const int unit = partition_unit(block_size);
    const int pt = effective_partition(partition_tokens, unit);
    const int64_t parts = max_seq_len > 0 ? (int64_t(max_seq_len) + pt - 1) / pt : 1;
    if (parts <= 1) return 0;
    return ws_layout(int64_t(num_seqs) * num_q_heads * parts, head_dim).bytes;
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, float scale,
              int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
              const float* k_scale, const float* v_scale,
              void* workspace, int64_t workspace_bytes, int32_t partition_tokens, void* stream) {
    pagedkv::clear_error();
    if (!supported_pair(q_dtype, cache_dtype))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: (q dtype %d, cache dtype %d) not supported", q_dtype, cache_dtype);
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq < 0 ||
        max_seq_len < 0 || partition_tokens < 0)
        return fail(PA_ERR_INVALID, "pa_decode: negative or zero size");
    if (num_q_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID, "pa_decode: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
    if (!(scale == scale)) return fail(PA_ERR_INVALID, "pa_decode: scale is NaN");
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !seq_lens || (max_blocks_per_seq > 0 && !block_tables))
        return fail(PA_ERR_INVALID, "pa_decode: NULL pointer");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_decode: out, q and caches must be 16-byte aligned");
    if (cache_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID, "pa_decode: fp8 cache needs k_scale and v_scale");
    if (int64_t(max_blocks_per_seq) * block_size < max_seq_len)
        return fail(PA_ERR_INVALID, "pa_decode: max_blocks_per_seq * block_size < max_seq_len");
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not in {64, 128}", head_dim);
    if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d not in {8, 16, 32, 128}", block_size);

    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.score_scale = scale * kLog2e;
    a.hkv = num_kv_heads;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.max_seq_len = max_seq_len;

    const int unit = partition_unit(block_size);
    int pt = effective_partition(partition_tokens, unit);
    int64_t parts = max_seq_len > 0 ? (int64_t(max_seq_len) + pt - 1) / pt : 1;
    if (parts > 1) {
        const WsLayout lay = ws_layout(int64_t(num_seqs) * num_q_heads * parts, head_dim);
        if (!workspace) {
            // no workspace: one partition per request
            pt = (max_seq_len + unit - 1) / unit * unit;
            parts = 1;
        } else if (workspace_bytes < lay.bytes || !aligned16(workspace)) {
            return fail(PA_ERR_INVALID, "pa_decode: workspace of %lld bytes, %lld needed (16-byte aligned)",
                        (long long)workspace_bytes, (long long)lay.bytes);
        } else {
            char* base = static_cast<char*>(workspace);
            a.ws_m = reinterpret_cast<float*>(base + lay.m_off);
            a.ws_l = reinterpret_cast<float*>(base + lay.l_off);
            a.ws_acc = reinterpret_cast<float*>(base + lay.acc_off);
        }
    }
    if (pt <= 0) pt = unit;
    if (parts > 65535) return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld partitions per request", (long long)parts);
    a.part_tokens = pt;
    a.max_parts = static_cast<int>(parts);

    const int G = num_q_heads / num_kv_heads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (cache_dtype == PA_DTYPE_F32)
        return dispatch_d<PA_DTYPE_F32, PA_DTYPE_F32>(head_dim, block_size, G, a, num_seqs, st);
    if (cache_dtype == PA_DTYPE_BF16)
        return dispatch_d<PA_DTYPE_BF16, PA_DTYPE_BF16>(head_dim, block_size, G, a, num_seqs, st);
    return dispatch_d<PA_DTYPE_FP8_E4M3, PA_DTYPE_BF16>(head_dim, block_size, G, a, num_seqs, st);
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst, int32_t num_pairs,
                   int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t cache_dtype, void* stream) {
    pagedkv::clear_error();
    const int eb = elem_bytes(cache_dtype);
    if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: cache dtype %d", cache_dtype);
    if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID, "pa_copy_blocks: bad sizes");
    const int64_t block_bytes = int64_t(num_kv_heads) * block_size * head_dim * eb;
    if (block_bytes % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block of %lld bytes", (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !src_dst || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID, "pa_copy_blocks: NULL or misaligned pointer");
    const int grid = grid_for(int64_t(num_pairs) * (block_bytes / 16), 256);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), src_dst, num_pairs,
                       num_blocks, block_bytes);
    return check_launch("pa_copy_blocks");
}

}  // extern "C"
