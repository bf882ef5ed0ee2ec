// Device helpers shared by the kernels of libpagedkv (gfx950): element formats, cross-lane
// reductions, explicit global / LDS accesses and the global -> LDS copies.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pagedkv.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

template <int DT> struct Elem;
template <> struct Elem<PA_DTYPE_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elem<PA_DTYPE_BF16> { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Elem<PA_DTYPE_FP8_E4M3> { using T = uint8_t; static constexpr int bytes = 1; };
template <> struct Elem<PA_DTYPE_MXFP4> { using T = uint8_t; static constexpr int bytes = 0; };   // half a byte + scales

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ cross-lane helpers
//
// Reductions use DPP lane permutations (quad_perm, row_ror, row_half_mirror) inside a
// 16-lane row and the gfx950 permlane swaps across rows: v_permlane16_swap exchanges the
// odd rows of one register with the even rows of the other, v_permlane32_swap the upper
// half of one with the lower half of the other.  Given the same value in both operands,
// the two results of a swap hold the value of the lane and of its partner 16 (or 32) lanes
// away, in some order, so any symmetric combination of them is the pair reduction.

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;    // row_ror:4
constexpr int kDppRowRor8 = 0x128;    // row_ror:8
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float pair16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over the KL (4 or 8) consecutive lanes that share a token row.
template <int KL>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    if constexpr (KL == 8) x += dpp<kDppRowHalfMirror>(x);
    return x;
}

// Max over the wave of a value that is already uniform within groups of KL lanes.
template <int KL>
__device__ __forceinline__ float wave_max_of_groups(float x) {
    if constexpr (KL == 4) x = fmaxf(x, dpp<kDppRowRor4>(x));
    x = fmaxf(x, dpp<kDppRowRor8>(x));
    x = pair16_max(x);
    return pair32_max(x);
}

// Sum over the 64 / VL lanes that share lane % VL (VL in {4, 8, 16, 32}).
template <int VL>
__device__ __forceinline__ float sum_over_row_groups(float x) {
    if constexpr (VL == 4) x += dpp<kDppRowRor4>(x);
    if constexpr (VL <= 8) x += dpp<kDppRowRor8>(x);
    if constexpr (VL <= 16) x = pair16_sum(x);
    return pair32_sum(x);
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct alignas(16) U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 ld16(const void* p) { return *reinterpret_cast<const U4*>(p); }

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Explicitly global (address space 1) and LDS (address space 3) accesses: keep the compiler
// from falling back to flat instructions, which also count against the LDS wait counter.
#define PA_GLOBAL __attribute__((address_space(1)))
#define PA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ U4 gld16(const void* p) {
    const u32x4v v = *(const PA_GLOBAL u32x4v*)p;
    return U4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ int gld_i32(const int32_t* p) { return *(const PA_GLOBAL int32_t*)p; }
__device__ __forceinline__ uint32_t gld_u8(const void* p) { return *(const PA_GLOBAL uint8_t*)p; }
__device__ __forceinline__ uint2 gld8(const void* p) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v v = *(const PA_GLOBAL u32x2v*)p;
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float gld_f32(const float* p) { return *(const PA_GLOBAL float*)p; }
template <typename T>
__device__ __forceinline__ void gst(T* p, T v) { *(PA_GLOBAL T*)p = v; }
__device__ __forceinline__ void lds_st16(PA_LDS unsigned char* p, const U4& v) {
    *(PA_LDS u32x4v*)p = u32x4v{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ U4 lds_ld16(const PA_LDS unsigned char* p) {
    const u32x4v v = *(const PA_LDS u32x4v*)p;
    return U4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint32_t lds_addr(const PA_LDS unsigned char* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Global -> LDS without registers: every lane's 16 bytes at sbase + voff (non-temporal) land at
// LDS byte address m0 + 16 * lane.  Issued from inline assembly so that the compiler, which
// cannot tell the ring's stages apart, does not drain every load before each LDS read; the
// waits are placed by hand (wait_vmem).  Each use is preceded by the LDS reads of the stage it
// overwrites having completed (lgkmcnt(0)).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\tglobal_load_lds_dwordx4 %0, %1 nt" :: "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
// the same with a 64-bit address per lane
__device__ __forceinline__ void dma16_lane(const void* addr, uint32_t m0) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\tglobal_load_lds_dwordx4 %0, off nt" :: "v"(addr), "{m0}"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Rescale threshold of the online softmax, in log2 units: a wave keeps a reference maximum
// and only rescales its state when a score exceeds it by more than this, so exponentials
// stay <= 2^8 and most passes need no cross-lane maximum at all.
constexpr float kRescaleThreshold = 8.0f;

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef short i16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// float32 -> bf16 bits, round to nearest even (finite, non-negative inputs: softmax weights).
__device__ __forceinline__ uint32_t weight_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 8 fp8 codes (two dwords) -> 8 bf16 values, exact (every E4M3FN value is a bf16 number).
__device__ __forceinline__ void e4m3x8_to_bf16(uint32_t w0, uint32_t w1, uint32_t (&o)[4]) {
    // gfx950's scaled pair conversion with a scale of 1: one instruction per two values
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), 1.0f, true));
}

// ------------------------------------------------------------------ MXFP4 (OCP microscaling, 4-bit)

// E8M0 scale byte -> its float32 value 2^(byte - 127) (0xFF gives infinity, so the block
// decodes to infinities and NaNs).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
    return __uint_as_float(code == 0 ? 0x00400000u : code << 23);
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times their block's scale -> 8 bf16
// values (four dwords, element 0 first).  gfx950's scaled pair conversion; exact, since every
// E2M1 value times 2^-127 .. 2^125 is a bfloat16 number.
__device__ __forceinline__ U4 e2m1x8_to_bf16(uint32_t w, float scale) {
    return U4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
}

}  // namespace
