// Grouped expert GEMM on 4-bit group-affine weights.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Dequantize the weights during the matrix multiplication": each weight is a
// 4-bit code, each group of 64 weights shares a bf16 scale and bias, and the
// matrix unit consumes bf16, so the weights are rebuilt in bf16 one small tile
// at a time, kept on chip while they multiply the routed activation rows, and
// never written out whole; accumulation is fp32 and the output bf16.  The
// ablation there rebuilds the whole bf16 matrix in memory first and reads it
// back.  Both are built here: Q4 = true rebuilds in registers, Q4 = false
// reads a bf16 matrix that dequant_q4_kernel wrote.
//
// y[r] = W_e x[r] for the rows r of expert e (rows grouped by expert through
// expert_offsets).  W_e is [N, K]: weight (n, k) = bf16(scale * code + bias)
// with the code in nibble k % 2 of byte k / 2 of row n (even k low) and the
// scale and bias of group k / 64; the product and the sum are formed by one
// fp32 fma and rounded once to bf16 (nearest even).
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_bf16): a workgroup of four waves
// owns one expert and a block of BN = 128 output columns, and walks all of
// that expert's rows in passes of up to RT row tiles of 16.  Wave w owns 32
// columns (two 16-column tiles): per 32-wide slab of k it rebuilds its two B
// fragments once (one dword of eight codes per lane: two mask operations,
// eight byte conversions, eight fma and four bf16 packs) and multiplies them
// by the pass's A fragments (16 bytes of one activation row per lane), so
// each weight is rebuilt once per pass and up to RT row tiles reuse it.  The
// next slab's codes and activations are loaded while the current one
// computes.
#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {
constexpr int BN = 128;  // output columns per workgroup
constexpr int RT = 8;    // row tiles (of 16) per pass
constexpr int GROUP = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// byte j of x as a float (the compiler emits v_cvt_f32_ubyte<j>)
template <int J>
__device__ __forceinline__ float ubyte(uint32_t x) { return float((x >> (8 * J)) & 0xFFu); }

// Eight rebuilt weights (k = 8 grp .. 8 grp + 7 of one column) from one dword
// of codes: byte j holds k = 2 j (low nibble) and 2 j + 1 (high nibble).
__device__ __forceinline__ uint4 rebuild8(uint32_t d, float s, float b) {
  const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
  const float w0 = fmaf(s, ubyte<0>(lo), b), w1 = fmaf(s, ubyte<0>(hi), b);
  const float w2 = fmaf(s, ubyte<1>(lo), b), w3 = fmaf(s, ubyte<1>(hi), b);
  const float w4 = fmaf(s, ubyte<2>(lo), b), w5 = fmaf(s, ubyte<2>(hi), b);
  const float w6 = fmaf(s, ubyte<3>(lo), b), w7 = fmaf(s, ubyte<3>(hi), b);
  return uint4{pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5), pack_bf16x2(w6, w7)};
}
}  // namespace

// The ablation's separate pass: the whole bf16 matrix [E, N, K] in memory.
// One thread per dword of codes (eight weights, one 16-byte store).
__global__ __launch_bounds__(256) void dequant_q4_kernel(size_t n_dwords, int k, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases, uint4* __restrict__ w) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_dwords) return;
  const size_t row = i / size_t(k / 8), kk = (i % size_t(k / 8)) * 8;  // row = e * N + n
  const size_t gi = row * size_t(k / GROUP) + kk / GROUP;
  w[i] = rebuild8(codes[i], bf16_bits_to_f32(scales[gi]), bf16_bits_to_f32(biases[gi]));
}

template <bool Q4>
__global__ __launch_bounds__(256) void moe_gemm_kernel(int n_exp, int m, int n, int k, const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ offsets,
                                                       const uint8_t* __restrict__ wsrc,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint16_t* __restrict__ biases, uint16_t* __restrict__ y) {
  const int ncb = n / BN;
  const int e = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  int r_lo = offsets[e], r_hi = offsets[e + 1];
  r_lo = r_lo < 0 ? 0 : (r_lo > m ? m : r_lo);  // malformed offsets cannot index out of bounds
  r_hi = r_hi < r_lo ? r_lo : (r_hi > m ? m : r_hi);
  if (r_hi == r_lo) return;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = cb * BN + 32 * wave;  // this wave's 32 columns
  const int ngroups = k / GROUP;
  // per lane: columns n0 + col and n0 + 16 + col; k offset 8 grp within a slab
  const size_t wrow0 = size_t(e) * n + n0 + col, wrow1 = wrow0 + 16;

  for (int p0 = r_lo; p0 < r_hi; p0 += 16 * RT) {
    const int nt = min(RT, (r_hi - p0 + 15) / 16);  // row tiles in this pass
    f4 acc[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t][0] = acc[t][1] = zero4();
    // A rows of this lane in each tile (rows past the expert read its last row; their results are dropped)
    const uint16_t* xrow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) xrow[t] = x + size_t(min(p0 + 16 * t + col, r_hi - 1)) * k + 8 * grp;

    auto load_b = [&](uint32_t (&d)[2], uint4 (&wb)[2], int k0) __attribute__((always_inline)) {
      if constexpr (Q4) {
        d[0] = *reinterpret_cast<const uint32_t*>(wsrc + wrow0 * (k / 2) + k0 / 2 + 4 * grp);
        d[1] = *reinterpret_cast<const uint32_t*>(wsrc + wrow1 * (k / 2) + k0 / 2 + 4 * grp);
      } else {
        const uint16_t* wb16 = reinterpret_cast<const uint16_t*>(wsrc);
        wb[0] = *reinterpret_cast<const uint4*>(wb16 + wrow0 * k + k0 + 8 * grp);
        wb[1] = *reinterpret_cast<const uint4*>(wb16 + wrow1 * k + k0 + 8 * grp);
      }
    };
    auto load_a = [&](uint4 (&a)[RT], int k0) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
        if (t < nt) a[t] = *reinterpret_cast<const uint4*>(xrow[t] + k0);
    };

    uint32_t dc[2], dn[2];
    uint4 wc[2], wn[2], ac[RT], an[RT];
    float s0 = 0.f, b0 = 0.f, s1 = 0.f, b1 = 0.f;
    load_b(dc, wc, 0);
    load_a(ac, 0);
    for (int k0 = 0; k0 < k; k0 += 32) {
      if constexpr (Q4) {
        if ((k0 & (GROUP - 1)) == 0) {  // a new group: its scale and bias for both columns
          const int g = k0 / GROUP;
          s0 = bf16_bits_to_f32(scales[wrow0 * ngroups + g]), b0 = bf16_bits_to_f32(biases[wrow0 * ngroups + g]);
          s1 = bf16_bits_to_f32(scales[wrow1 * ngroups + g]), b1 = bf16_bits_to_f32(biases[wrow1 * ngroups + g]);
        }
      }
      const int kn = min(k0 + 32, k - 32);  // the next slab (the last one reloads itself)
      load_b(dn, wn, kn);
      load_a(an, kn);
      uint4 bf0, bf1;
      if constexpr (Q4) {
        bf0 = rebuild8(dc[0], s0, b0);
        bf1 = rebuild8(dc[1], s1, b1);
      } else {
        bf0 = wc[0], bf1 = wc[1];
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < nt) {
          acc[t][0] = mma32(ac[t], bf0, acc[t][0]);
          acc[t][1] = mma32(ac[t], bf1, acc[t][1]);
        }
      }
      dc[0] = dn[0], dc[1] = dn[1], wc[0] = wn[0], wc[1] = wn[1];
#pragma unroll
      for (int t = 0; t < RT; ++t) ac[t] = an[t];
    }
    // D block: lane holds rows 4 grp .. 4 grp + 3 of the tile, column col
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (t < nt) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int r = p0 + 16 * t + 4 * grp + qq;
          if (r < r_hi) {
            y[size_t(r) * n + n0 + col] = f2bf(acc[t][0][qq]);
            y[size_t(r) * n + n0 + 16 + col] = f2bf(acc[t][1][qq]);
          }
        }
      }
    }
  }
}

hipError_t launch_moe_gemm(int n_exp, int m, int n, int k, const void* x, const int32_t* offsets,
                           const void* weights, const void* scales, const void* biases, void* y, bool q4,
                           hipStream_t st) {
  const unsigned blocks = unsigned(n_exp) * unsigned(n / BN);
  if (blocks == 0 || m == 0) return hipSuccess;
  Prof prof(q4 ? "moe_gemm_q4" : "moe_gemm_bf16", st);
  if (q4)
    hipLaunchKernelGGL(moe_gemm_kernel<true>, dim3(blocks), dim3(256), 0, st, n_exp, m, n, k,
                       static_cast<const uint16_t*>(x), offsets, static_cast<const uint8_t*>(weights),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(biases),
                       static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(moe_gemm_kernel<false>, dim3(blocks), dim3(256), 0, st, n_exp, m, n, k,
                       static_cast<const uint16_t*>(x), offsets, static_cast<const uint8_t*>(weights), nullptr,
                       nullptr, static_cast<uint16_t*>(y));
  return hipGetLastError();
}

hipError_t launch_dequant_q4(int n_exp, int n, int k, const void* codes, const void* scales, const void* biases,
                             void* w, hipStream_t st) {
  const size_t n_dwords = size_t(n_exp) * n * (k / 8);
  if (n_dwords == 0) return hipSuccess;
  Prof prof("dequant_q4", st);
  hipLaunchKernelGGL(dequant_q4_kernel, dim3(unsigned((n_dwords + 255) / 256)), dim3(256), 0, st, n_dwords, k,
                     static_cast<const uint32_t*>(codes), static_cast<const uint16_t*>(scales),
                     static_cast<const uint16_t*>(biases), static_cast<uint4*>(w));
  return hipGetLastError();
}

}  // namespace gdn
