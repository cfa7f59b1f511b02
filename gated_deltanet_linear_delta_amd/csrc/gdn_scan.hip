// Prefill by direct token scan, with the state held in registers.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Keeping the recurrent state on chip": the state matrix is split among the
// lanes of a SIMD group, loaded into registers once, carried through the
// whole scan with partial sums exchanged by cross-lane operations rather than
// shared memory, and written back once at the end.  On gfx950 a state row
// (fixed value index) lives in LPR = d_k / 8 lanes, 8 fp32 per lane; dot
// products are reduced with DPP.  Rows are independent given the token
// stream (the delta rule couples only the key index), so a workgroup owns 16
// rows of one (sequence, value head) and needs no communication besides the
// shared token tiles.
//
// Per token the recurrence is  p = S k,  u = beta (v - alpha p),
// S <- alpha S + u k^T,  o = S q.  Walking it one token at a time puts a load,
// a dot product, a cross-lane reduction and the update on the critical path
// of every token.  The tokens are instead walked in blocks of NBK = 4 with the
// same arithmetic regrouped.  With S the state before the block, G_j the
// block's running sum of g, a_j = exp(G_j) and u_i already known for i < j:
//   p_j = a_{j-1} (S k_j) + sum_{i<j} exp(G_{j-1} - G_i) (k_i . k_j) u_i
//   o_j = a_j (S q_j)     + sum_{i<=j} exp(G_j - G_i)   (k_i . q_j) u_i
//   S  <- a_3 S + sum_i exp(G_3 - G_i) u_i k_i^T
// (a_{-1} = 1).  The eight dot products S k_j, S q_j of a block are
// independent, so their reductions overlap; the scalar weights are the same
// for every row and are formed once per tile.  Token data (k and q in fp32,
// g, beta, and the workgroup's 16 v values) is staged in LDS in tiles of TT
// tokens, zero past the sequence's end, so a short last block adds nothing.
//
// The same section measures the alternative, a blockwise scan that keeps the
// state in memory and moves it there and back every block, with the
// cooperating threads meeting at barriers.  BLOCKWISE = true builds that
// ablation: every `sblock` tokens (a multiple of NBK) each lane stores its
// state to s_out, the workgroup meets at a barrier, and the lane reads the
// state back, so the arithmetic and its rounding are those of the resident
// scan.
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {
constexpr int TT = 32;         // tokens per LDS tile
constexpr int NBK = 4;         // tokens per lookahead block
constexpr int NBT = TT / NBK;  // blocks per tile
// Per-block scalars: a_j, c_j = exp(G_3 - G_j), the six k.k weights (i < j),
// the ten k.q weights (i <= j), beta_j, beta_j alpha_j.
constexpr int SB_A = 0, SB_C = 4, SB_W = 8, SB_WQ = 14, SB_B = 24, SB_BA = 28, SB_N = 32;
// pair e of the 16 weighted dot products of a block: e < 6 are k_i . k_j
// (i < j), the rest k_i . q_j (i <= j), in row-major order
__device__ __forceinline__ constexpr int pair_i(int e) {
  return e < 6 ? (e < 3 ? 0 : (e < 5 ? 1 : 2)) : (e < 10 ? 0 : (e < 13 ? 1 : (e < 15 ? 2 : 3)));
}
__device__ __forceinline__ constexpr int pair_j(int e) {
  return e < 6 ? (e < 3 ? e + 1 : (e < 5 ? e - 1 : 3)) : (e < 10 ? e - 6 : (e < 13 ? e - 9 : (e < 15 ? e - 11 : 3)));
}

template <typename IO>
__device__ __forceinline__ void to_f32(const uint4& raw, float* x) {
  if constexpr (sizeof(IO) == 4) {
    x[0] = __uint_as_float(raw.x), x[1] = __uint_as_float(raw.y);
    x[2] = __uint_as_float(raw.z), x[3] = __uint_as_float(raw.w);
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) x[2 * i] = __uint_as_float(w[i] << 16), x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) d = fmaf(a[e], b[e], d);
  return d;
}
__device__ __forceinline__ void lds8(const float* row, int c0, int c1, float* x) {
  const f4 a = *reinterpret_cast<const f4*>(row + c0), b = *reinterpret_cast<const f4*>(row + c1);
  x[0] = a[0], x[1] = a[1], x[2] = a[2], x[3] = a[3], x[4] = b[0], x[5] = b[1], x[6] = b[2], x[7] = b[3];
}
}  // namespace

template <typename IO, int DK, bool BLOCKWISE, bool PREFETCH>
__global__ __launch_bounds__(16 * (DK / 8)) void scan_kernel(
    int T, int h_qk, int h_v, int d_v, const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const float* s_in, IO* __restrict__ out, float* s_out, int sblock) {
  constexpr int LPR = DK / 8;
  constexpr int NT = 16 * LPR;          // threads
  constexpr int E16 = 16 / sizeof(IO);  // io elements per 16 bytes
  __shared__ __attribute__((aligned(16))) float sk[TT][DK];
  __shared__ __attribute__((aligned(16))) float sq[TT][DK];
  __shared__ __attribute__((aligned(16))) float sv[16][TT];  // v of the workgroup's rows, token fastest
  __shared__ __attribute__((aligned(16))) float so[TT][16];
  __shared__ __attribute__((aligned(16))) float sblk[NBT][SB_N];
  __shared__ float sg[TT], sb[TT];

  const int nrb = d_v / 16;
  const int rb = blockIdx.x % nrb;
  const int nh = blockIdx.x / nrb;
  const int h = nh % h_v;
  const int n = nh / h_v;
  const int j_qk = h / (h_v / h_qk);
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
    lds8(s_in + srow, c0, c1, s);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
  }

  int left = sblock;  // tokens before the next round trip through memory (blockwise only)
  for (int t0 = bos; t0 < eos; t0 += TT) {
    const int nt = min(TT, eos - t0);
    // ---- stage the tile: k and q in fp32, zero past the end
    for (int x = tid; x < TT * (DK / E16); x += NT) {
      const int r = x / (DK / E16), cc = (x % (DK / E16)) * E16;
      float kf[E16], qf[E16];
      if (r < nt) {
        const size_t off = (size_t(t0 + r) * h_qk + j_qk) * DK + cc;
        to_f32<IO>(*reinterpret_cast<const uint4*>(k + off), kf);
        to_f32<IO>(*reinterpret_cast<const uint4*>(q + off), qf);
      } else {
#pragma unroll
        for (int e = 0; e < E16; ++e) kf[e] = qf[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E16; e += 4) {
        *reinterpret_cast<f4*>(&sk[r][cc + e]) = f4{kf[e], kf[e + 1], kf[e + 2], kf[e + 3]};
        *reinterpret_cast<f4*>(&sq[r][cc + e]) = f4{qf[e], qf[e + 1], qf[e + 2], qf[e + 3]};
      }
    }
    for (int x = tid; x < TT; x += NT) {
      sg[x] = x < nt ? g[size_t(t0 + x) * h_v + h] : 0.f;  // past the end: alpha = 1, beta = 0
      sb[x] = x < nt ? beta[size_t(t0 + x) * h_v + h] : 0.f;
    }
    for (int x = tid; x < TT * 16; x += NT) {
      const int r = x / 16, cc = x % 16;
      sv[cc][r] = r < nt ? io_traits<IO>::load(v + (size_t(t0 + r) * h_v + h) * d_v + rb * 16 + cc) : 0.f;
    }
    __syncthreads();

    // ---- per-block scalars: row group lr forms half of block lr / 2's
    // sixteen weighted dot products (all its lanes get the sums); lane m of
    // the group then scales entry m by its exponential, so each lane takes
    // one exponential
    {
      const int bk = lr >> 1, half = lr & 1, tb = bk * NBK;
      float G[NBK];
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < NBK; ++jj) G[jj] = acc += sg[tb + jj];
      float dots[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int e = half * 8 + m;  // which pair: the same in all lanes of the group
        const int pi = pair_i(e), pj = pair_j(e);
        float ka[8], kb[8];
        lds8(&sk[tb + pi][0], c0, c1, ka);
        lds8(e < 6 ? &sk[tb + pj][0] : &sq[tb + pj][0], c0, c1, kb);
        dots[m] = sum_lanes<LPR>(dot8(ka, kb));
      }
#pragma unroll
      for (int m0 = 0; m0 < 8; m0 += LPR) {
        const int m = m0 + l;  // this lane's entry (lanes past 8 have none)
        if (m < 8) {
          const int e = half * 8 + m;
          float d = dots[0], gi = G[0], gj = G[0];
#pragma unroll
          for (int mm = 1; mm < 8; ++mm) d = m == mm ? dots[mm] : d;
          // e < 6: exp(G_{j-1} - G_i), else exp(G_j - G_i)
          const int pi = pair_i(e), pj = pair_j(e) - (e < 6 ? 1 : 0);
#pragma unroll
          for (int jj = 1; jj < NBK; ++jj) {
            gi = pi == jj ? G[jj] : gi;
            gj = pj == jj ? G[jj] : gj;
          }
          const int slot = e < 6 ? SB_W + e : SB_WQ + e - 6;  // pairs are stored in the same order
          sblk[bk][slot] = d * expf(gj - gi);
        }
      }
      if (half == 1) {
        // lanes 0..15 of the group: entry jj = l % 4 of a_j, c_j, beta_j, beta_j alpha_j
#pragma unroll
        for (int x0 = 0; x0 < 4 * NBK; x0 += LPR) {
          const int x = x0 + l;
          if (x < 4 * NBK) {
            const int jj = x & 3, kind = x >> 2;
            float gj = G[0];
#pragma unroll
            for (int t = 1; t < NBK; ++t) gj = jj == t ? G[t] : gj;
            const float gt = sg[tb + jj], bt = sb[tb + jj];
            const float ex = kind == 0 ? gj : (kind == 1 ? G[NBK - 1] - gj : gt);
            const float ev = expf(ex);
            sblk[bk][kind == 0 ? SB_A + jj : (kind == 1 ? SB_C + jj : (kind == 2 ? SB_B + jj : SB_BA + jj))] =
                kind == 2 ? bt : (kind == 3 ? bt * ev : ev);
          }
        }
      }
    }
    __syncthreads();

    // ---- walk the tile's blocks.  With PREFETCH, k and q of the next block
    // are read from LDS while the current one computes (two register sets,
    // the loop unrolled by two so that neither is indexed at run time); that
    // hides LDS latency when each SIMD runs one or two waves, and costs
    // occupancy when there are enough workgroups to fill the CUs.
    const int nbk = (nt + NBK - 1) / NBK;
    auto load_kq = [&](float (&kb)[NBK][8], float (&qb)[NBK][8], int bk) __attribute__((always_inline)) {
      const int tb = min(bk, NBT - 1) * NBK;  // past the tile: a valid block, unused
#pragma unroll
      for (int jj = 0; jj < NBK; ++jj) {
        lds8(&sk[tb + jj][0], c0, c1, kb[jj]);
        lds8(&sq[tb + jj][0], c0, c1, qb[jj]);
      }
    };
    auto step = [&](float (&kv)[NBK][8], float (&qv)[NBK][8], float (&kn)[NBK][8], float (&qn)[NBK][8], int bk)
                    __attribute__((always_inline)) {
      if constexpr (BLOCKWISE) {
        if (left == 0) {  // the same count in every lane: the barrier is uniform
          *reinterpret_cast<f4*>(s_out + srow + c0) = f4{s[0], s[1], s[2], s[3]};
          *reinterpret_cast<f4*>(s_out + srow + c1) = f4{s[4], s[5], s[6], s[7]};
          __syncthreads();
          lds8(s_out + srow, c0, c1, s);
          left = sblock;
        }
        left -= NBK;
      }
      const int tb = bk * NBK;
      const f4* sp = reinterpret_cast<const f4*>(&sblk[bk][0]);
      const f4 A = sp[0], Cw = sp[1], W0 = sp[2], W1 = sp[3], W2 = sp[4], W3 = sp[5], Bt = sp[6], BA = sp[7];
      const f4 vv = *reinterpret_cast<const f4*>(&sv[lr][tb]);
      if constexpr (!PREFETCH) load_kq(kv, qv, bk);
      float pk[NBK], pq[NBK];
#pragma unroll
      for (int jj = 0; jj < NBK; ++jj) pk[jj] = dot8(s, kv[jj]), pq[jj] = dot8(s, qv[jj]);
      if constexpr (PREFETCH) load_kq(kn, qn, bk + 1);
#pragma unroll
      for (int jj = 0; jj < NBK; ++jj) pk[jj] = sum_lanes<LPR>(pk[jj]), pq[jj] = sum_lanes<LPR>(pq[jj]);
      // W: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3) in W0[0..3], W1[0..1]; WQ in W1[2..3], W2, W3
      const float u0 = fmaf(-BA[0], pk[0], Bt[0] * vv[0]);
      const float p1 = fmaf(W0[0], u0, A[0] * pk[1]);
      const float u1 = fmaf(-BA[1], p1, Bt[1] * vv[1]);
      const float p2 = fmaf(W0[3], u1, fmaf(W0[1], u0, A[1] * pk[2]));
      const float u2 = fmaf(-BA[2], p2, Bt[2] * vv[2]);
      const float p3 = fmaf(W1[1], u2, fmaf(W0[2], u0, fmaf(W1[0], u1, A[2] * pk[3])));
      const float u3 = fmaf(-BA[3], p3, Bt[3] * vv[3]);
      // WQ: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
      const float o0 = fmaf(W1[2], u0, A[0] * pq[0]);
      const float o1 = fmaf(W2[2], u1, fmaf(W1[3], u0, A[1] * pq[1]));
      const float o2 = fmaf(W3[1], u2, fmaf(W2[3], u1, fmaf(W2[0], u0, A[2] * pq[2])));
      const float o3 = fmaf(W3[3], u3, fmaf(W3[2], u2, fmaf(W3[0], u1, fmaf(W2[1], u0, A[3] * pq[3]))));
      const float cu0 = Cw[0] * u0, cu1 = Cw[1] * u1, cu2 = Cw[2] * u2, cu3 = Cw[3] * u3;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        s[e] = fmaf(cu3, kv[3][e], fmaf(cu2, kv[2][e], fmaf(cu1, kv[1][e], fmaf(cu0, kv[0][e], A[3] * s[e]))));
      if (l == 0) {
        so[tb + 0][lr] = o0;
        so[tb + 1][lr] = o1;
        so[tb + 2][lr] = o2;
        so[tb + 3][lr] = o3;
      }
    };
    if constexpr (PREFETCH) {
      float kA[NBK][8], qA[NBK][8], kB[NBK][8], qB[NBK][8];
      load_kq(kA, qA, 0);
      for (int bk = 0; bk < nbk; bk += 2) {
        step(kA, qA, kB, qB, bk);
        if (bk + 1 < nbk) step(kB, qB, kA, qA, bk + 1);
      }
    } else {
      float kA[NBK][8], qA[NBK][8];
      for (int bk = 0; bk < nbk; ++bk) step(kA, qA, kA, qA, bk);
    }
    __syncthreads();
    for (int x = tid; x < nt * 16; x += NT) {
      const int r = x / 16, cc = x % 16;
      io_traits<IO>::store(out + (size_t(t0 + r) * h_v + h) * d_v + rb * 16 + cc, so[r][cc]);
    }
    // the next tile's staging writes the tiles only after every thread passed this point
    __syncthreads();
  }
  *reinterpret_cast<f4*>(s_out + srow + c0) = f4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<f4*>(s_out + srow + c1) = f4{s[4], s[5], s[6], s[7]};
}

// Up to about four workgroups per CU (256 CUs) the scan prefetches each
// block's k and q; past that the CUs are full and occupancy matters more.
constexpr int kPrefetchMaxBlocks = 1024;

template <typename IO, int DK>
static hipError_t launch_scan_t(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu, const float* s_in, void* out,
                                float* s_out, int sblock, hipStream_t st) {
  const int blocks = d.num_seqs * d.h_v * (d.d_v / 16);
  if (blocks == 0) return hipSuccess;
  auto go = [&](auto bw, auto pf) {
    constexpr bool BW = decltype(bw)::value, PF = decltype(pf)::value;
    Prof prof(BW ? "scan_blockwise" : "scan", st);
    hipLaunchKernelGGL((scan_kernel<IO, DK, BW, PF>), dim3(blocks), dim3(16 * (DK / 8)), 0, st, d.total_tokens,
                       d.h_qk, d.h_v, d.d_v, static_cast<const IO*>(q), static_cast<const IO*>(k),
                       static_cast<const IO*>(v), g, beta, cu, s_in, static_cast<IO*>(out), s_out, sblock);
    return hipGetLastError();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  const bool pf = blocks <= kPrefetchMaxBlocks;
  if (sblock > 0) return pf ? go(T_(), T_()) : go(T_(), F_());
  return pf ? go(F_(), T_()) : go(F_(), F_());
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
