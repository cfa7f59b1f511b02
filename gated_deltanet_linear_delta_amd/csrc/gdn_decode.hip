// Decode step of the gated delta rule: one token per sequence.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Decode: minimize bytes moved per token": at batch 1 a decode step is bound
// by the bytes it moves.  Here those bytes are almost all the fp32 state
// (2 * d_v * d_k * 4 per head), so the kernel reads every state row once and
// writes it once, fully coalesced, with the two dot products S.k and S.q
// reduced across lanes by DPP instead of LDS.  The update is the rank-one
// form of the gated delta rule:
//   p = S k,  u = beta (v - alpha p),  S' = alpha S + u k^T,
//   o = S' q = alpha (S q) + u (k . q),      alpha = exp(g).
//
// Layout: a state row (fixed value index i) is d_k contiguous floats.  LPR =
// d_k / 8 lanes share a row, each holding 8 floats as two float4 at column
// offsets 4*l and d_k/2 + 4*l, so every load instruction covers contiguous
// 16*LPR-byte runs.  A workgroup holds 16 rows (16 * LPR threads).
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

template <typename IO>
__device__ __forceinline__ void load4(const IO* p, float* x) {
  if constexpr (sizeof(IO) == 4) {
    f4 t = *reinterpret_cast<const f4*>(p);
    x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
  } else {
    uint2 t = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(t.x << 16);
    x[1] = __uint_as_float(t.x & 0xffff0000u);
    x[2] = __uint_as_float(t.y << 16);
    x[3] = __uint_as_float(t.y & 0xffff0000u);
  }
}

// RPL rows per lane group: each lane keeps 2 * RPL float4 loads of the state
// in flight, enough bytes per wave to keep HBM busy at large batch.
template <typename IO, int DK, int RPL>
__global__ __launch_bounds__(16 * (DK / 8)) void decode_kernel(
    int total_rows, int h_qk, int h_v, int d_v, const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const float* s_in, IO* __restrict__ out, float* s_out) {
  constexpr int LPR = DK / 8;
  const int l = threadIdx.x % LPR;
  // 16 * RPL consecutive rows per workgroup; d_v is a multiple of 16 * RPL, so
  // they all belong to one (sequence, head)
  const int row0 = (blockIdx.x * 16 + threadIdx.x / LPR) * RPL;
  if (row0 >= total_rows) return;  // whole row groups leave together
  const int bh = row0 / d_v;  // b * h_v + h
  const int h = bh % h_v;
  const int b = bh / h_v;
  const int j = h / (h_v / h_qk);
  const int c0 = 4 * l, c1 = DK / 2 + 4 * l;

  f4 sa[RPL], sb[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float* sr = s_in + size_t(row0 + r) * DK;
    sa[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(sr + c0));
    sb[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(sr + c1));
  }
  const IO* kp = k + (size_t(b) * h_qk + j) * DK;
  const IO* qp = q + (size_t(b) * h_qk + j) * DK;
  float kv[8], qv[8];
  load4(kp + c0, kv);
  load4(kp + c1, kv + 4);
  load4(qp + c0, qv);
  load4(qp + c1, qv + 4);
  const float alpha = expf(g[bh]);
  const float bt = beta[bh];
  float vi[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) vi[r] = io_traits<IO>::load(v + size_t(row0 + r));
  float kq0 = 0.f, kq1 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kq0 = fmaf(kv[e], qv[e], kq0);
    kq1 = fmaf(kv[e + 4], qv[e + 4], kq1);
  }
  const float kq = sum_lanes<LPR>(kq0 + kq1);
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    float s[8] = {sa[r][0], sa[r][1], sa[r][2], sa[r][3], sb[r][0], sb[r][1], sb[r][2], sb[r][3]};
    float p0 = 0.f, p1 = 0.f, r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p0 = fmaf(s[e], kv[e], p0);
      p1 = fmaf(s[e + 4], kv[e + 4], p1);
      r0 = fmaf(s[e], qv[e], r0);
      r1 = fmaf(s[e + 4], qv[e + 4], r1);
    }
    const float p = sum_lanes<LPR>(p0 + p1);
    const float rq = sum_lanes<LPR>(r0 + r1);
    const float u = bt * (vi[r] - alpha * p);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = fmaf(alpha, s[e], u * kv[e]);
    float* so = s_out + size_t(row0 + r) * DK;
    __builtin_nontemporal_store(f4{s[0], s[1], s[2], s[3]}, reinterpret_cast<f4*>(so + c0));
    __builtin_nontemporal_store(f4{s[4], s[5], s[6], s[7]}, reinterpret_cast<f4*>(so + c1));
    if (l == 0) io_traits<IO>::store(out + size_t(row0 + r), fmaf(alpha, rq, u * kq));
  }
}

// ---------------------------------------------------------------- fused step
// The same step with the work on either side of it folded in (section
// "Reduce state and intermediate traffic": the decode path fuses the
// preparation of queries and keys, and the recurrent update with its
// normalisation, so that no intermediate goes through memory):
//   q = q_raw / sqrt(|q_raw|^2 + qk_eps),  k likewise        (fp32, not rounded)
//   alpha = exp(-scale_h softplus(g_raw + bias_h)),  beta = sigmoid(beta_raw)
//   o = S' q as above,  out = o / sqrt(mean_dv(o^2) + norm_eps) * w
// The norm spans all d_v rows of a head, so a workgroup owns one (sequence,
// head): d_v / RPL lane groups of LPR lanes, RPL rows each (rows rg,
// rg + d_v / RPL, ...), at least one full wave.  The unnormalised o
// goes through LDS; every wave then sums the squares in the same order, so
// all of them derive the same scale without a second barrier.
// The products with the state are formed from the raw q and k and scaled by
// 1/|q|, 1/|k| afterwards (S k_raw / |k| = S k), so they run beside the norm
// reductions instead of after them; the scalar activations and inverse
// square roots use the hardware exp2, log2, rcp and rsq (about 1e-6
// relative error, far below the fp32 tolerance).
struct FusedArgs {
  const float* gate_bias;   // [h_v] or null
  const float* gate_scale;  // [h_v] or null
  const float* norm_w;      // [d_v] or null
  float qk_eps, norm_eps;
};

__device__ __forceinline__ float wave_sum64(float x) {
  x = sum_lanes16(x);  // each row's sum in all its lanes; the four rows read out as scalars
  auto rd = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return (rd(0) + rd(16)) + (rd(32) + rd(48));
}

template <typename IO, int DK, int NQ, int RPL>
__global__ __launch_bounds__(1024) void decode_fused_kernel(
    int h_qk, int h_v, int d_v, const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ g_raw, const float* __restrict__ b_raw, FusedArgs fa, const float* s_in,
    IO* __restrict__ out, float* s_out) {
  constexpr int LPR = DK / (4 * NQ);  // lanes per row
  constexpr int NV = 4 * NQ;          // state values per lane and row
  __shared__ float so[128];
  const int bh = blockIdx.x;  // b * h_v + h
  const int h = bh % h_v;
  const int b = bh / h_v;
  const int j = h / (h_v / h_qk);
  const int l = threadIdx.x % LPR;
  const int rg = threadIdx.x / LPR;
  const int ngrp = d_v / RPL;
  const bool act = rg < ngrp;  // lane groups past the rows (blocks padded to a wave) only join the sum
  auto cof = [&](int m) { return 4 * l + m * (DK / NQ); };  // column of the lane's m-th float4

  f4 sv[RPL][NQ];
  int row[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    row[r] = min(rg, ngrp - 1) + r * ngrp;
    const float* sr = s_in + (size_t(bh) * d_v + row[r]) * DK;
#pragma unroll
    for (int m = 0; m < NQ; ++m) sv[r][m] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(sr + cof(m)));
  }
  const IO* kp = k + (size_t(b) * h_qk + j) * DK;
  const IO* qp = q + (size_t(b) * h_qk + j) * DK;
  float kv[NV], qv[NV];
#pragma unroll
  for (int m = 0; m < NQ; ++m) load4(kp + cof(m), kv + 4 * m), load4(qp + cof(m), qv + 4 * m);
  const float x = g_raw[bh] + (fa.gate_bias ? fa.gate_bias[h] : 0.f);
  constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
  // softplus ln(1 + e^x) through the hardware exp2 and log2 (x past 20: ln(1 + e^x) = x in fp32)
  const float sp = x > 20.f ? x : __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(x * LOG2E)) * LN2;
  const float alpha = __builtin_amdgcn_exp2f(-(fa.gate_scale ? fa.gate_scale[h] : 1.f) * sp * LOG2E);
  const float bt = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b_raw[bh] * LOG2E));
  // v and the norm weight of the lane's rows with the other inputs, so that
  // no load waits at the end of the step
  float vi[RPL], nw[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    vi[r] = io_traits<IO>::load(v + size_t(bh) * d_v + row[r]);
    nw[r] = fa.norm_w ? fa.norm_w[row[r]] : 1.f;
  }

  float kk0 = 0.f, kk1 = 0.f, qq0 = 0.f, qq1 = 0.f, kq0 = 0.f, kq1 = 0.f;
#pragma unroll
  for (int e = 0; e < NV / 2; ++e) {
    kk0 = fmaf(kv[e], kv[e], kk0);
    kk1 = fmaf(kv[e + NV / 2], kv[e + NV / 2], kk1);
    qq0 = fmaf(qv[e], qv[e], qq0);
    qq1 = fmaf(qv[e + NV / 2], qv[e + NV / 2], qq1);
    kq0 = fmaf(kv[e], qv[e], kq0);
    kq1 = fmaf(kv[e + NV / 2], qv[e + NV / 2], kq1);
  }
  const float rk = __builtin_amdgcn_rsqf(sum_lanes<LPR>(kk0 + kk1) + fa.qk_eps);
  const float rq = __builtin_amdgcn_rsqf(sum_lanes<LPR>(qq0 + qq1) + fa.qk_eps);
  const float kq = sum_lanes<LPR>(kq0 + kq1) * rk * rq;

  float o[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    float s[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) s[e] = sv[r][e / 4][e % 4];
    float p0 = 0.f, p1 = 0.f, r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int e = 0; e < NV / 2; ++e) {
      p0 = fmaf(s[e], kv[e], p0);
      p1 = fmaf(s[e + NV / 2], kv[e + NV / 2], p1);
      r0 = fmaf(s[e], qv[e], r0);
      r1 = fmaf(s[e + NV / 2], qv[e + NV / 2], r1);
    }
    const float p = sum_lanes<LPR>(p0 + p1) * rk;
    const float sq = sum_lanes<LPR>(r0 + r1) * rq;
    const float u = bt * (vi[r] - alpha * p);
    const float uk = u * rk;
#pragma unroll
    for (int e = 0; e < NV; ++e) s[e] = fmaf(alpha, s[e], uk * kv[e]);
    if (act) {
      float* so_row = s_out + (size_t(bh) * d_v + row[r]) * DK;
#pragma unroll
      for (int m = 0; m < NQ; ++m)
        __builtin_nontemporal_store(f4{s[4 * m], s[4 * m + 1], s[4 * m + 2], s[4 * m + 3]},
                                    reinterpret_cast<f4*>(so_row + cof(m)));
    }
    o[r] = fmaf(alpha, sq, u * kq);
    if (act && l == 0) so[row[r]] = o[r];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
  for (int i = lane; i < d_v; i += 64) ss = fmaf(so[i], so[i], ss);
  const float scale = __builtin_amdgcn_rsqf(wave_sum64(ss) / float(d_v) + fa.norm_eps);
  if (act && l == 0) {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      io_traits<IO>::store(out + size_t(bh) * d_v + row[r], o[r] * scale * nw[r]);
  }
}

template <typename IO, int DK>
static hipError_t launch_decode_fused_t(const Dims& d, const void* q, const void* k, const void* v,
                                        const float* g_raw, const float* b_raw, const FusedArgs& fa,
                                        const float* s_in, void* out, float* s_out, hipStream_t st) {
  const int blocks = d.num_seqs * d.h_v;
  if (blocks == 0) return hipSuccess;
  Prof prof("decode_fused", st);
  // Two shapes, chosen by the number of (sequence, head) workgroups.  With
  // few heads (below 512 workgroups, e.g. B = 1) the step is the latency of
  // one workgroup: each lane holds 16 values of a state row (NQ = 4 float4),
  // so a row needs d_k / 16 lanes and every reduction one DPP step less, and
  // a workgroup has at most 512 lanes.  With enough heads to fill the GPU
  // (B = 32) the step is the stream of all heads: each lane holds 8 values
  // (NQ = 2) and a workgroup up to 1024 lanes, so each lane's serial work per
  // row is short.  Measured at d = 128: B = 1 3.77 -> 3.59 us against one
  // shape for both, B = 32 26.1 -> 24.3 us against 512-lane workgroups.
  // RPL = 1, 2, 4 or 8 rows per lane group keep the workgroup within its cap
  // (each lane then has NQ RPL state loads in flight).
  auto launch = [&](auto nq_c, auto maxl_c) {
    constexpr int NQ = decltype(nq_c)::value, MAXL = decltype(maxl_c)::value;
    constexpr int LPR = DK / (4 * NQ);
    const int lanes = d.d_v * LPR;
    const int rpl = lanes <= MAXL ? 1 : lanes / MAXL;
    auto go = [&](auto rc) {
      constexpr int RPL = decltype(rc)::value;
      hipLaunchKernelGGL((decode_fused_kernel<IO, DK, NQ, RPL>), dim3(blocks),
                         dim3(lanes / RPL < 64 ? 64 : lanes / RPL), 0, st, d.h_qk, d.h_v, d.d_v,
                         static_cast<const IO*>(q), static_cast<const IO*>(k), static_cast<const IO*>(v), g_raw,
                         b_raw, fa, s_in, static_cast<IO*>(out), s_out);
      return hipGetLastError();
    };
    constexpr int RMAX = 128 * LPR / MAXL;  // rows per lane group at d_v = 128
    if constexpr (RMAX >= 8) if (rpl == 8) return go(std::integral_constant<int, 8>());
    if constexpr (RMAX >= 4) if (rpl == 4) return go(std::integral_constant<int, 4>());
    if constexpr (RMAX >= 2) if (rpl == 2) return go(std::integral_constant<int, 2>());
    return go(std::integral_constant<int, 1>());
  };
  if (blocks >= 512) return launch(std::integral_constant<int, 2>(), std::integral_constant<int, 1024>());
  return launch(std::integral_constant<int, 4>(), std::integral_constant<int, 512>());
}

hipError_t launch_decode_fused(const Dims& d, const void* q, const void* k, const void* v, const float* g_raw,
                               const float* b_raw, const float* gate_bias, const float* gate_scale,
                               const float* norm_weight, float qk_eps, float norm_eps, const float* s_in,
                               void* out, float* s_out, hipStream_t st) {
  const FusedArgs fa{gate_bias, gate_scale, norm_weight, qk_eps, norm_eps};
#define GDN_DECF(IO, DK) return launch_decode_fused_t<IO, DK>(d, q, k, v, g_raw, b_raw, fa, s_in, out, s_out, st)
  if (d.bf16) {
    switch (d.d_k) {
      case 16: GDN_DECF(uint16_t, 16);
      case 32: GDN_DECF(uint16_t, 32);
      case 64: GDN_DECF(uint16_t, 64);
      case 128: GDN_DECF(uint16_t, 128);
    }
  } else {
    switch (d.d_k) {
      case 16: GDN_DECF(float, 16);
      case 32: GDN_DECF(float, 32);
      case 64: GDN_DECF(float, 64);
      case 128: GDN_DECF(float, 128);
    }
  }
#undef GDN_DECF
  return hipErrorInvalidValue;
}

// Large batches use 4 rows per lane group (more bytes in flight per wave);
// small ones 1, to spread the few rows over more compute units.
template <typename IO, int DK>
static hipError_t launch_decode_t(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const float* s_in, void* out, float* s_out,
                                  hipStream_t st) {
  const int rows = d.num_seqs * d.h_v * d.d_v;
  if (rows == 0) return hipSuccess;
  dim3 block(16 * (DK / 8));
  Prof prof("decode", st);
  if (rows >= 65536 && d.d_v % 64 == 0) {
    hipLaunchKernelGGL((decode_kernel<IO, DK, 4>), dim3((rows + 63) / 64), block, 0, st, rows, d.h_qk, d.h_v,
                       d.d_v, static_cast<const IO*>(q), static_cast<const IO*>(k), static_cast<const IO*>(v), g,
                       beta, s_in, static_cast<IO*>(out), s_out);
  } else {
    hipLaunchKernelGGL((decode_kernel<IO, DK, 1>), dim3((rows + 15) / 16), block, 0, st, rows, d.h_qk, d.h_v,
                       d.d_v, static_cast<const IO*>(q), static_cast<const IO*>(k), static_cast<const IO*>(v), g,
                       beta, s_in, static_cast<IO*>(out), s_out);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* s_in, void* out, float* s_out, hipStream_t st) {
#define GDN_DEC(IO, DK) return launch_decode_t<IO, DK>(d, q, k, v, g, beta, s_in, out, s_out, st)
  if (d.bf16) {
    switch (d.d_k) {
      case 16: GDN_DEC(uint16_t, 16);
      case 32: GDN_DEC(uint16_t, 32);
      case 64: GDN_DEC(uint16_t, 64);
      case 128: GDN_DEC(uint16_t, 128);
    }
  } else {
    switch (d.d_k) {
      case 16: GDN_DEC(float, 16);
      case 32: GDN_DEC(float, 32);
      case 64: GDN_DEC(float, 64);
      case 128: GDN_DEC(float, 128);
    }
  }
#undef GDN_DEC
  return hipErrorInvalidValue;
}

}  // namespace gdn
