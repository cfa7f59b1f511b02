// Prefill by direct token scan, with the state held in registers.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Keeping the recurrent state on chip": the state matrix is split among the
// lanes of a SIMD group, loaded into registers once, carried through the
// whole scan with partial sums exchanged by cross-lane operations rather than
// shared memory, and written back once at the end.  On gfx950 a state row
// (fixed value index) lives in LPR = d_k / 8 lanes, 8 fp32 per lane; the two
// dot products per token are reduced with DPP.  Rows are independent given
// the token stream (the delta rule couples only the key index), so a
// workgroup owns 16 rows of one (sequence, value head) and needs no
// communication besides the shared token tiles.
//
// Per token:  p = S k,  u = beta (v - alpha p),  S <- alpha S + u k^T,
//             o = alpha (S_old q) + u (k . q),   alpha = exp(g).
// Token data (k, q, alpha, beta, k.q and the workgroup's 16 v values) is
// staged in LDS in tiles of TT tokens; outputs are staged and written per
// tile.
//
// The same section measures the alternative, a blockwise scan that keeps the
// state in memory and moves it there and back every block, with the
// cooperating threads meeting at barriers.  BLOCKWISE = true builds that
// ablation: every `sblock` tokens each lane stores its state to s_out, the
// workgroup meets at a barrier, and the lane reads the state back, so the
// arithmetic and its rounding are those of the resident scan.
#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {
constexpr int TT = 64;  // tokens per LDS tile

template <typename IO>
__device__ __forceinline__ void lds_load4(const IO* p, float* x) {
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
}  // namespace

template <typename IO, int DK, bool BLOCKWISE>
__global__ __launch_bounds__(16 * (DK / 8)) void scan_kernel(
    int T, int h_qk, int h_v, int d_v, const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const float* s_in, IO* __restrict__ out, float* s_out, int sblock) {
  constexpr int LPR = DK / 8;
  constexpr int NT = 16 * LPR;            // threads
  constexpr int E16 = 16 / sizeof(IO);    // io elements per 16 bytes
  __shared__ __attribute__((aligned(16))) IO sk[TT][DK];
  __shared__ __attribute__((aligned(16))) IO sq[TT][DK];
  __shared__ float sa[TT], sb[TT], skq[TT];
  __shared__ float sv[TT][16];
  __shared__ float so[TT][16];

  const int nrb = d_v / 16;
  const int rb = blockIdx.x % nrb;
  const int nh = blockIdx.x / nrb;
  const int h = nh % h_v;
  const int n = nh / h_v;
  const int j = h / (h_v / h_qk);
  const int tid = threadIdx.x;
  const int l = tid % LPR;
  const int lr = tid / LPR;  // local row 0..15
  const int i = rb * 16 + lr;
  const int c0 = 4 * l, c1 = DK / 2 + 4 * l;
  const size_t srow = (size_t(nh) * d_v + i) * DK;

  int bos, eos;
  seq_range(cu, n, T, bos, eos);
  if (bos == eos && s_in == s_out) return;  // no tokens and the state already in place

  float s[8];
  if (s_in) {
    f4 a = *reinterpret_cast<const f4*>(s_in + srow + c0);
    f4 b = *reinterpret_cast<const f4*>(s_in + srow + c1);
    s[0] = a[0]; s[1] = a[1]; s[2] = a[2]; s[3] = a[3];
    s[4] = b[0]; s[5] = b[1]; s[6] = b[2]; s[7] = b[3];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
  }

  int left = sblock;  // tokens before the next round trip through memory (blockwise only)
  for (int t0 = bos; t0 < eos; t0 += TT) {
    const int nt = min(TT, eos - t0);
    // ---- stage the tile
    for (int x = tid; x < nt * (DK / E16); x += NT) {
      const int r = x / (DK / E16), cc = (x % (DK / E16)) * E16;
      const size_t off = (size_t(t0 + r) * h_qk + j) * DK + cc;
      *reinterpret_cast<uint4*>(&sk[r][cc]) = *reinterpret_cast<const uint4*>(k + off);
      *reinterpret_cast<uint4*>(&sq[r][cc]) = *reinterpret_cast<const uint4*>(q + off);
    }
    for (int x = tid; x < nt; x += NT) {
      sa[x] = expf(g[size_t(t0 + x) * h_v + h]);
      sb[x] = beta[size_t(t0 + x) * h_v + h];
    }
    for (int x = tid; x < nt * 16; x += NT) {
      const int r = x / 16, cc = x % 16;
      sv[r][cc] = io_traits<IO>::load(v + (size_t(t0 + r) * h_v + h) * d_v + rb * 16 + cc);
    }
    __syncthreads();
    // k . q per token: LPR lanes per token, 8 elements each
    for (int r = lr; r < nt; r += 16) {
      float kv[8], qv[8];
      lds_load4(&sk[r][c0], kv);
      lds_load4(&sk[r][c1], kv + 4);
      lds_load4(&sq[r][c0], qv);
      lds_load4(&sq[r][c1], qv + 4);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(kv[e], qv[e], a);
      a = sum_lanes<LPR>(a);
      if (l == 0) skq[r] = a;
    }
    __syncthreads();
    // ---- walk the tile
    for (int r = 0; r < nt; ++r) {
      if constexpr (BLOCKWISE) {
        if (left == 0) {  // the same count in every lane: the barrier is uniform
          *reinterpret_cast<f4*>(s_out + srow + c0) = f4{s[0], s[1], s[2], s[3]};
          *reinterpret_cast<f4*>(s_out + srow + c1) = f4{s[4], s[5], s[6], s[7]};
          __syncthreads();
          const f4 a = *reinterpret_cast<const f4*>(s_out + srow + c0);
          const f4 b = *reinterpret_cast<const f4*>(s_out + srow + c1);
          s[0] = a[0]; s[1] = a[1]; s[2] = a[2]; s[3] = a[3];
          s[4] = b[0]; s[5] = b[1]; s[6] = b[2]; s[7] = b[3];
          left = sblock;
        }
        --left;
      }
      float kv[8], qv[8];
      lds_load4(&sk[r][c0], kv);
      lds_load4(&sk[r][c1], kv + 4);
      lds_load4(&sq[r][c0], qv);
      lds_load4(&sq[r][c1], qv + 4);
      const float alpha = sa[r], bt = sb[r], kq = skq[r], vi = sv[r][lr];
      float p0 = 0.f, p1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0 = fmaf(s[e], kv[e], p0);
        p1 = fmaf(s[e + 4], kv[e + 4], p1);
        q0 = fmaf(s[e], qv[e], q0);
        q1 = fmaf(s[e + 4], qv[e + 4], q1);
      }
      const float p = sum_lanes<LPR>(p0 + p1);
      const float rq = sum_lanes<LPR>(q0 + q1);
      const float u = bt * (vi - alpha * p);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = fmaf(alpha, s[e], u * kv[e]);
      if (l == 0) so[r][lr] = fmaf(alpha, rq, u * kq);
    }
    __syncthreads();
    for (int x = tid; x < nt * 16; x += NT) {
      const int r = x / 16, cc = x % 16;
      io_traits<IO>::store(out + (size_t(t0 + r) * h_v + h) * d_v + rb * 16 + cc, so[r][cc]);
    }
    // the next tile's staging writes sk/sq/sv/sa/sb only after every thread
    // passed this point
    __syncthreads();
  }
  *reinterpret_cast<f4*>(s_out + srow + c0) = f4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<f4*>(s_out + srow + c1) = f4{s[4], s[5], s[6], s[7]};
}

template <typename IO, int DK>
static hipError_t launch_scan_t(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu, const float* s_in, void* out,
                                float* s_out, int sblock, hipStream_t st) {
  const int blocks = d.num_seqs * d.h_v * (d.d_v / 16);
  if (blocks == 0) return hipSuccess;
  if (sblock > 0) {
    Prof prof("scan_blockwise", st);
    hipLaunchKernelGGL((scan_kernel<IO, DK, true>), dim3(blocks), dim3(16 * (DK / 8)), 0, st, d.total_tokens,
                       d.h_qk, d.h_v, d.d_v, static_cast<const IO*>(q), static_cast<const IO*>(k),
                       static_cast<const IO*>(v), g, beta, cu, s_in, static_cast<IO*>(out), s_out, sblock);
  } else {
    Prof prof("scan", st);
    hipLaunchKernelGGL((scan_kernel<IO, DK, false>), dim3(blocks), dim3(16 * (DK / 8)), 0, st, d.total_tokens,
                       d.h_qk, d.h_v, d.d_v, static_cast<const IO*>(q), static_cast<const IO*>(k),
                       static_cast<const IO*>(v), g, beta, cu, s_in, static_cast<IO*>(out), s_out, 0);
  }
  return hipGetLastError();
}

hipError_t launch_scan(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const int32_t* cu, const float* s_in, void* out, float* s_out,
                       hipStream_t st, int sblock) {
#define GDN_SCAN(IO, DK) return launch_scan_t<IO, DK>(d, q, k, v, g, beta, cu, s_in, out, s_out, sblock, st)
  if (d.bf16) {
    switch (d.d_k) {
      case 16: GDN_SCAN(uint16_t, 16);
      case 32: GDN_SCAN(uint16_t, 32);
      case 64: GDN_SCAN(uint16_t, 64);
      case 128: GDN_SCAN(uint16_t, 128);
    }
  } else {
    switch (d.d_k) {
      case 16: GDN_SCAN(float, 16);
      case 32: GDN_SCAN(float, 32);
      case 64: GDN_SCAN(float, 64);
      case 128: GDN_SCAN(float, 128);
    }
  }
#undef GDN_SCAN
  return hipErrorInvalidValue;
}

}  // namespace gdn
