// Device helpers shared by the gfx950 kernels: bf16 conversion, lane
// reductions through DPP, and 16x16 MFMA block products.
//
// MFMA fragment convention used by every kernel (wave64, 16x16 blocks,
// lane = 16*grp + col, grp in 0..3, col in 0..15), for a contraction slab of
// 16 along the summed index:
//   A fragment (16 rows x 16 k):  lane holds A[row = col][k = 4*grp + q], q = 0..3
//   B fragment (16 k x 16 cols):  lane holds B[k = 4*grp + q][n = col]
//   C/D block  (16 x 16):         lane holds D[row = 4*grp + q][n = col]
// So a D block is, with no data movement, the B fragment of the same matrix
// and the A fragment of its transpose.  bf16 slabs use one
// v_mfma_f32_16x16x16_bf16; fp32 slabs use four v_mfma_f32_16x16x4_f32, the
// q-th of which carries k = 4*grp + q in every lane group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16 with round to nearest even (NaN stays NaN), by the
// hardware conversion v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {  // a in the low half
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// Split x into hi + lo, both bf16: hi = rne(x), lo = rne(x - hi).  |x - hi - lo| <= 2^-17 |x|.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}
// The same for a pair: hi and lo packed two to a word, a in the low halves.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// ---------------------------------------------------------------- DPP lane reductions
// Row = 16 lanes.  Butterfly sums over groups of 2, 4, 8 or 16 consecutive lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_lanes2(float x) { return x + dpp<0xB1>(x); }       // quad_perm 1,0,3,2
__device__ __forceinline__ float sum_lanes4(float x) {
  x = sum_lanes2(x);
  return x + dpp<0x4E>(x);  // quad_perm 2,3,0,1
}
__device__ __forceinline__ float sum_lanes8(float x) {
  x = sum_lanes4(x);
  return x + dpp<0x141>(x);  // row_half_mirror: joins the two quads of each 8-lane half
}
__device__ __forceinline__ float sum_lanes16(float x) {
  x = sum_lanes8(x);
  return x + dpp<0x140>(x);  // row_mirror: joins the two halves of the row
}
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N == 1) return x;
  else if constexpr (N == 2) return sum_lanes2(x);
  else if constexpr (N == 4) return sum_lanes4(x);
  else if constexpr (N == 8) return sum_lanes8(x);
  else return sum_lanes16(x);
}

// ---------------------------------------------------------------- MFMA block products
// bf16 operand fragment: 4 values, packed as a short vector for the builtin.
struct bfrag {
  s4 v;
};
// hi/lo split of an fp32 fragment.
struct sfrag {
  s4 hi, lo;
};

__device__ __forceinline__ s4 pack4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
  s4 r;
  r[0] = short(a);
  r[1] = short(b);
  r[2] = short(c);
  r[3] = short(d);
  return r;
}

__device__ __forceinline__ sfrag split4(f4 x) {
  uint16_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split_bf16(x[i], h[i], l[i]);
  sfrag r;
  r.hi = pack4(h[0], h[1], h[2], h[3]);
  r.lo = pack4(l[0], l[1], l[2], l[3]);
  return r;
}

__device__ __forceinline__ f4 mma_bf(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// exact-bf16 A times split B: A*Bhi + A*Blo
__device__ __forceinline__ f4 mma_e_s(s4 a, const sfrag& b, f4 c) {
  c = mma_bf(a, b.hi, c);
  return mma_bf(a, b.lo, c);
}
// split A times split B: Ahi*Bhi + Ahi*Blo + Alo*Bhi (the lo*lo term is below 2^-16 relative)
__device__ __forceinline__ f4 mma_s_s(const sfrag& a, const sfrag& b, f4 c) {
  c = mma_bf(a.lo, b.hi, c);
  c = mma_bf(a.hi, b.lo, c);
  return mma_bf(a.hi, b.hi, c);
}
// fp32 slab: four 16x16x4 products, the q-th using k = 4*grp + q.
__device__ __forceinline__ f4 mma_f32(f4 a, f4 b, f4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- K = 32 slabs
// Same convention with a contraction slab of 32: the A fragment lane holds
// A[row = col][k = 8*grp + q] and the B fragment lane holds
// B[k = 8*grp + q][n = col], q = 0..7; the D block layout is unchanged.  bf16
// slabs are one v_mfma_f32_16x16x32_bf16 on 8 packed bf16 (a uint4); fp32
// slabs are eight v_mfma_f32_16x16x4_f32, the q-th carrying k = 8*grp + q.
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

struct f8 {  // eight fp32 operand values of one lane
  f4 a, b;
};

__device__ __forceinline__ f4 mma32(uint4 a, uint4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma32(const f8& a, const f8& b, f4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[0], b.a[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[1], b.a[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[2], b.a[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[3], b.a[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[0], b.b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[1], b.b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[2], b.b[2], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[3], b.b[3], c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return uint32_t(lo) | (uint32_t(hi) << 16); }

// Round 4 fp32 to bf16 (8 bytes) and, optionally, the rounding residues (8 bytes).
__device__ __forceinline__ uint2 bf16x4(f4 x) { return uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])}; }
__device__ __forceinline__ void split_bf16x4(f4 x, uint2& hi, uint2& lo) {
  split_bf16x2(x[0], x[1], hi.x, lo.x);
  split_bf16x2(x[2], x[3], hi.y, lo.y);
}
__device__ __forceinline__ void split_bf16x8(const f8& x, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split_bf16x4(x.a, h0, l0);
  split_bf16x4(x.b, h1, l1);
  hi = uint4{h0.x, h0.y, h1.x, h1.y};
  lo = uint4{l0.x, l0.y, l1.x, l1.y};
}

// ---------------------------------------------------------------- io element access
template <typename IO>
struct io_traits;
template <>
struct io_traits<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float x) { *p = x; }
};
template <>
struct io_traits<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float x) { *p = f2bf(x); }
};

// Clamp a sequence's [bos, eos) to [0, T] so malformed offsets cannot index out of bounds.
__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int T, int& bos, int& eos) {
  int a = cu[n], b = cu[n + 1];
  a = a < 0 ? 0 : (a > T ? T : a);
  b = b < a ? a : (b > T ? T : b);
  bos = a;
  eos = b;
}

}  // namespace gdn
