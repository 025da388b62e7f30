// Layout of the stored score gradient dS for the two-pass backward that
// keeps dS (gfx950; shared by the dK/dV kernels that write it and the dQ
// kernel that reads it).
//
// The dK/dV pass (KV-major) forms dS_ij = P_ij (dP_ij - delta_i) for every
// visible pair anyway; storing it (bf16, the rounding the dQ product takes)
// lets the dQ pass (Q-major) compute dQ_i = scale * sum_j dS_ij k_j without
// forming S and dP a second time.  The gate gradient's row sums
// sum_j dS_ij cannot come from the bf16 values (their rounding moves dg by
// percents), so the dK/dV pass also stores them in fp32, summed over each
// 16-key block; the dQ pass adds the blocks of a row in a fixed order.
//
// Units: query rows in 32-row tiles, keys in 16-key blocks, both counted
// from the start of their sequence.  Row tile rt of sequence n has the
// global number rtb(n) + rt, rtb(n) = floor(cu[n] / 32) + n (no two
// sequences share a number: rtb(n+1) - rtb(n) >= ceil(L_n / 32)).  Key block
// kb is visible to row tile rt iff kb_lo(rt) <= kb <= kb_hi(rt):
//   kb_lo(rt) = (W > 0 ? max(0, 32 rt - W + 1) : 0) / 16,
//   kb_hi(rt) = min(2 rt + 1, (L - 1) / 16),
// and lives in slot kb - kb_lo(rt) < nslot, where
//   nslot = W > 0 ? min(2 + (W + 14) / 16, 2 RT) : 2 RT,  RT = ceil(max_seqlen / 32).
// One 1 KB tile per (query head h, global row tile, slot), key-major inside:
// key k of the block holds 64 bytes, rows 0-15 and 16-31 in its two 32-byte
// halves, swapped for keys 4-7 and 12-15 (ds_off), so that the transposed
// reads of the dQ pass (two lane groups: keys 0-3 and 4-7 of the same rows)
// fall on different LDS banks.  The row partials use the same numbering with
// 32 floats per tile.
#pragma once
#include "common.h"

namespace attn {

constexpr int kDsRows = 32;     // query rows per dS tile
constexpr int kDsKeys = 16;     // keys per dS tile
constexpr int kDsTileBytes = kDsRows * kDsKeys * 2;

__host__ __device__ inline long ds_row_tiles(long T, int num_seqs) { return T / kDsRows + num_seqs + 1; }

__host__ __device__ inline int ds_slots(int max_seqlen, int window) {
  // in 64-bit: max_seqlen + 31 and window + 14 overflow int near INT_MAX
  const long rt = ((long)max_seqlen + kDsRows - 1) / kDsRows;
  const long full = 2 * rt;
  if (window <= 0) return (int)full;
  const long w = 2 + ((long)window + 14) / 16;
  return (int)(w < full ? w : full);
}

__host__ __device__ inline int ds_kb_lo(int rt, int window) {
  const int first = window > 0 ? kDsRows * rt - window + 1 : 0;
  return (first > 0 ? first : 0) / kDsKeys;
}

__host__ __device__ inline int ds_kb_hi(int rt, int L) {
  const int a = 2 * rt + 1, b = (L - 1) / kDsKeys;
  return a < b ? a : b;
}

// global number of row tile rt of the sequence that starts at token cu_n
__host__ __device__ inline long ds_grt(int cu_n, int n, int rt) { return (long)(cu_n / kDsRows) + n + rt; }

// byte offset of (key k, row r) inside a tile
__host__ __device__ inline int ds_off(int k, int r) {
  return k * 64 + (((r >> 4) ^ ((k >> 2) & 1)) << 5) + (r & 15) * 2;
}

// tile index (times kDsTileBytes for the byte offset, times 32 for the
// partials' float offset)
__host__ __device__ inline long ds_tile(int h, long grt, int slot, long nrt, int nslot) {
  return ((long)h * nrt + grt) * nslot + slot;
}

}  // namespace attn
