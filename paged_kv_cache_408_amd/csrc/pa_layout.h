// LDS layouts of the K/V tiles, shared by the kernels and by the host-side layout check
// (tests/lds_layout_dump.cpp).  LDS has 64 banks of 4 bytes; a 16-byte chunk of a tile row
// is placed at a slot that depends on the row, so that the lanes of one LDS instruction
// touch different banks.
#pragma once

#include <hip/hip_runtime.h>

// Decode: slot of bf16 chunk c (16 bytes = 8 dims) in row `row` of a wave's V tile (D / 8
// chunks per row): c XOR a per-row mask m.  m / 2 runs through every value on any 8
// consecutive rows that share banks, so the transpose reads (2 chunks of 4 rows per 16 lanes,
// 8 rows per 32) never collide; m % 4 (D = 128) or m % 2 (D = 64, where rows r and r + 2 share
// banks) differs between the rows one write instruction covers, so the fp8 tile writes (2 rows
// x 8 chunks) and the 4-bit ones (4 rows x 4 chunks) do not collide either.
template <int D>
__host__ __device__ constexpr int vt_slot(int row, int c) {
    return D == 128 ? c ^ ((2 * (row & 7)) ^ ((row ^ (row >> 1)) & 1)) : c ^ ((row & 7) ^ ((row >> 1) & 1));
}

// Prefill: chunk c of K/V tile row R (D / 8 chunks per row) sits at slot c ^ prefill_swz(R).
// The K operand reads one chunk of 32 consecutive rows: 16 consecutive rows must land on
// different banks (D = 128: every row covers all banks once, so a bijection of R % 16; D = 64:
// rows of equal parity share banks, so a bijection of (R / 2) % 8).  The transpose reads of V
// take 4 chunks (32 dims) of 4 consecutive rows per 32 lanes: those chunk groups must be
// disjoint among rows that share banks.
template <int D>
__host__ __device__ constexpr int prefill_swz(int row) {
    return D == 128 ? ((row & 3) << 2) | ((row >> 2) & 3) : (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
