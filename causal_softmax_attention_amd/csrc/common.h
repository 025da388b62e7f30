// Device helpers shared by the gfx950 attention kernels.
//
// Matrix-core lane layouts used throughout (checked on gfx950 with an
// in-bounds probe; l = lane 0..63):
//   v_mfma_f32_16x16x32_bf16: A[m][k]: m = l%16, k = 8*(l/16)+e (e = 0..7)
//                             B[k][n]: n = l%16, k = 8*(l/16)+e
//                             C[m][n]: n = l%16, m = 4*(l/16)+i (i = 0..3)
//   v_mfma_f32_16x16x16_bf16: as above with k = 4*(l/16)+e (e = 0..3)
//   ds_read_b64_tr_b16: within each group of 16 lanes, result lane i,
//                       element j (0..3) is element i%4 of the 8 bytes
//                       addressed by lane 4*j + i/4 of the same group.
//   ds_read_b64_tr_b8:  result lane i, byte j (0..7) is byte i%8 of the
//                       8 bytes addressed by lane 2*j + i/8 of its group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf in running maxima: exp2(x - kNegBig) is 0 for
// every finite score, and kNegBig - kNegBig = 0 avoids inf - inf.
constexpr float kNegBig = -1.0e30f;
// Lazy-rescale slack (log2 units): a running max is raised only when a new
// score exceeds it by more than this, so probabilities stay below 2^8 and
// the accumulators are rescaled rarely.  Numerator and denominator share the
// same stale max, so the result is unchanged.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
      __builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 8 contiguous bf16 read from LDS as one 16-byte access.
__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// Transposed 4 x bf16 read (see the layout note at the top).
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS i16x4*)(LDS_AS void*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}
// Transposed 8 x byte read.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (LDS_AS i32x2*)(LDS_AS void*)(const_cast<uint8_t*>(p)));
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Round-to-nearest-even float -> bf16 (the compiler emits the gfx950
// hardware conversion for this cast).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// Max / sum across the four 16-lane groups that hold the same column n
// (lanes l, l^16, l^32, l^48), with the gfx950 lane swaps
// v_permlane32_swap (lane l <-> l^32 between two registers) and
// v_permlane16_swap (odd 16-lane rows <-> even rows): two VALU steps, no
// LDS round trip.
__device__ __forceinline__ float xgroup_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xgroup_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two OCP e4m3fn bytes (low or high half of a 32-bit word) -> two floats.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(int word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles filled by direct global->LDS loads.
//
// A tile of rows of RB bytes is stored without padding; the 16-byte chunk c
// of row r sits at chunk position c ^ swz(r).  With RB >= 256 the swizzle
// 2*(r%8) + (r/8)%2 makes both access patterns used by the kernels free of
// bank conflicts: 16 lanes reading the same logical chunk of 16 consecutive
// rows (MFMA operand rows), and ds_read_b64_tr_b16 reading two adjacent
// chunks of 4 consecutive rows.  128-byte rows use (r/2)%8.
template <int RB>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (RB >= 256) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (r >> 1) & (RB / 16 - 1);
}
// LDS byte offset of logical byte `b` (within its row) of row r.
template <int RB>
__device__ __forceinline__ int tile_off(int r, int b) {
  return r * RB + ((((b >> 4) ^ tile_swz<RB>(r)) << 4) | (b & 15));
}

// Direct loads of rows row0 .. row0+ROWS-1 of a row-major global matrix
// (gstride bytes between rows, RB bytes used per row) into a swizzled LDS
// tile.  Each of the 4 waves of the workgroup issues every 4th 1 KB block;
// lane l of a block writes LDS bytes [16 l, 16 l + 16).  The per-lane source
// offsets inside a tile are fixed, so they are computed once.  Rows at or
// past `nrows` re-read row nrows-1 (in range and finite; the kernels mask
// those keys).  Completion is awaited with s_waitcnt vmcnt before a barrier.
template <int RB, int ROWS>
struct TileDma {
  static constexpr int NI = ROWS * RB / 1024;
  static constexpr int PW = NI / 4;          // blocks per wave
  static_assert(NI % 4 == 0 && NI * 1024 == ROWS * RB, "tile must split into 4 x k 1 KB blocks");
  int row[PW];                               // tile row of this lane's chunk
  int col[PW];                               // byte offset of the chunk in that row
  int off[PW];                               // row * gstride + col
  __device__ __forceinline__ void init(long gstride, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int o = (wave + 4 * j) * 1024 + lane * 16;
      row[j] = o / RB;
      col[j] = (((o % RB) >> 4) ^ tile_swz<RB>(row[j])) << 4;
      off[j] = (int)(row[j] * gstride) + col[j];
    }
  }
  __device__ __forceinline__ void issue(const uint8_t* gbase, long gstride, int row0, int nrows,
                                        uint8_t* lds, int wave) const {
    const uint8_t* tb = gbase + row0 * gstride;
    const bool tail = row0 + ROWS > nrows;   // uniform: only the last tile clamps
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const uint8_t* src = tail ? gbase + min(row0 + row[j], nrows - 1) * gstride + col[j] : tb + off[j];
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void LDS_AS*)(lds + (wave + 4 * j) * 1024), 16, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace attn
