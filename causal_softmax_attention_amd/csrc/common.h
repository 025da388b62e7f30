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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
// The same read from a pointer already in the LDS address space (lets the
// compiler fold constant parts of the address into the offset field).
__device__ __forceinline__ bf16x4 lds_tr16(const LDS_AS uint8_t* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p));
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
// Maximum of two or three floats as one v_max / v_max3.  fmaxf makes the
// compiler quiet possible signalling NaNs first (a self-max per operand it
// cannot prove canonical, e.g. lane-swap results); operands here are
// arithmetic results or -inf, never signalling NaNs, and for quiet NaNs the
// instruction already returns the other operand as fmaxf does.  Only for
// operands written by ordinary VALU instructions: the compiler does not
// insert the wait states an MFMA result needs before an inline-asm read.
__device__ __forceinline__ float max_nq(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nq(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float xgroup_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = max_nq(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max_nq(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xgroup_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Workgroup index x of n -> logical index: consecutive logical indices land on
// the same XCD (workgroups are dealt round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int x, int n) {
  if (n % 8 != 0) return x;
  return (x % 8) * (n / 8) + x / 8;
}

// x of another lane of the same 16-lane row through a DPP move (CTRL: a
// quad_perm, row_mirror 0x140 or row_half_mirror 0x141; every lane has a
// source in these patterns).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Coefficient pairs for split_lo, (-1, 0) and (0, -1) as bf16 pairs.  They
// must reach v_dot2_f32_bf16 from registers: as an inline constant the
// compiler encodes (-1, 0) as the f32 constant -1.0, whose bf16 halves the
// hardware reads as (0, -1).  Made once per kernel; the empty asm keeps the
// compiler from folding them back into constants.
struct SplitCoef {
  bf16x2 c0, c1;
};
__device__ __forceinline__ SplitCoef split_coef() {
  unsigned c0, c1;
  asm("s_mov_b32 %0, 0x0000bf80" : "=s"(c0));
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(c1));
  return SplitCoef{__builtin_bit_cast(bf16x2, c0), __builtin_bit_cast(bf16x2, c1)};
}

// x - h[0] and y - h[1] for h = (x, y) rounded to bf16: one v_dot2_f32_bf16
// each (h . (-1, 0) + x); the difference of a float and its bf16 rounding is
// exact in fp32.
__device__ __forceinline__ f32x2 split_lo(bf16x2 h, float x, float y, SplitCoef k) {
  return f32x2{__builtin_amdgcn_fdot2_f32_bf16(h, k.c0, x, false), __builtin_amdgcn_fdot2_f32_bf16(h, k.c1, y, false)};
}

// Two OCP e4m3fn bytes (low or high half of a 32-bit word) -> two floats.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(int word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
}

// ---------------------------------------------------------------------------
// Direct global->LDS copies (global_load_lds) issued through inline asm.
//
// Lane l of a copy reads sbase + voff (saddr form: a wave-uniform 64-bit base
// in SGPRs plus a 32-bit per-lane offset) and writes its 16 (or 4) bytes at
// LDS address m0 + 16 l (or 4 l).  The compiler does not see these copies;
// had they been issued through the builtin, it would make every later LDS
// read (and every barrier) wait for all copies in flight, which serialises
// a prefetch ring.  Kernels therefore wait for them explicitly with
// wait_vm<N>() (N = copies issued after the ones needed) and must not rely
// on compiler-inserted waits for LDS data written this way.  M0 is used by
// nothing else in these kernels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}
// A wave-uniform pointer pinned to scalar registers (for the copy bases above
// when the compiler has computed a uniform value in vector registers).
template <typename T>
__device__ __forceinline__ const T* sgpr_ptr(const T* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier for kernels that manage their own waits: LDS accesses
// of this wave are complete, and the compiler moves no memory access across.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Inclusive scan of L values by one 256-thread workgroup, in scan order
// q = 0 .. L-1 (load(q) / store(q, v) map q to memory).  Rounds of 4096
// values, 16 consecutive ones per thread held in registers, so that each
// round costs one memory latency rather than one per value; the chunk totals
// are scanned in LDS.  Summation order is fixed (deterministic).
template <typename Load, typename Store>
__device__ __forceinline__ void block_scan_256(int L, Load load, Store store) {
  __shared__ float part[256];
  const int tid = threadIdx.x;
  float carry = 0.f;
  for (int base = 0; base < L; base += 4096) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = base + 16 * tid + j;
      v[j] = q < L ? load(q) : 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // Hillis-Steele inclusive scan
      const float x = tid >= off ? part[tid - off] : 0.f;
      __syncthreads();
      part[tid] += x;
      __syncthreads();
    }
    float run = carry + part[tid] - s;            // exclusive prefix of this chunk
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = base + 16 * tid + j;
      run += v[j];
      if (q < L) store(q, run);
    }
    carry += part[255];
    __syncthreads();                              // part is reused by the next round
  }
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles: a tile of rows of RB bytes is stored without padding;
// the 16-byte chunk c of row r sits at chunk position c ^ swz(r).  The
// kernels read a tile in two ways: MFMA operand rows (ds_read_b128: 16 lanes
// read the same logical chunk of 16 consecutive rows, 4 lane groups read 4
// adjacent chunks) and transposed reads (ds_read_b64_tr_b16: each lane group
// reads two adjacent chunks of 4 consecutive rows).  Measured on gfx950 with
// the bank-conflict counter, ds_read_b128 is served 32 lanes at a time over
// 512 bytes of banks and the transposed read 32 lanes at a time over 256
// bytes.  Under that model these swizzles are free of conflicts for both
// reads (confirmed by the counter): 256-byte rows XOR the chunk with
// 2*(r%8) ^ 2*((r/8)%2); 128-byte rows with 2*(((r/2)%4) ^ ((r/8)%2)).
// (The more obvious 2*(r%8)+(r/8)%2 conflicts 2-way on the row reads, and
// r%16 2-way on the transposed ones.)  Rows of 512 bytes or more use the
// 256-byte rule on the low chunk bits (measured faster there than the rule
// the model suggests for them, so the model is incomplete for wide rows).
template <int RB>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (RB >= 256) return ((r & 7) << 1) ^ (((r >> 3) & 1) << 1);
  else return (((r >> 1) & 3) ^ ((r >> 3) & 1)) << 1;
}
// LDS byte offset of logical byte `b` (within its row) of row r.
template <int RB>
__device__ __forceinline__ int tile_off(int r, int b) {
  return r * RB + ((((b >> 4) ^ tile_swz<RB>(r)) << 4) | (b & 15));
}

}  // namespace attn
