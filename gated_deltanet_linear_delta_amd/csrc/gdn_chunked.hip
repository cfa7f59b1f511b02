// Chunked prefill of the gated delta rule on gfx950 MFMA.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Qwen creates three distinct workload shapes": instead of walking tokens,
// prefill may regroup the recurrent updates into blocks that expose matrix
// operations and token-level parallelism while computing the same result.
// The pages print no block formula; the one used here follows from unrolling
// the recurrence over a block of n <= C tokens that starts from state S0
// (rows of K, Q, V are the block's tokens):
//
//   G_r = sum_{i<=r} g_i,  gamma_r = exp(G_r),  dec_r = exp(G_{n-1} - G_r)
//   A_ri = beta_r exp(G_r - G_i) (k_r . k_i)  (i < r),   T = (I + A)^{-1}
//   QKm_ri = exp(G_r - G_i) (q_r . k_i)       (i <= r)
//   Y   = diag(beta) V - diag(beta gamma) (K S0^T)
//   U   = T Y
//   O   = diag(gamma) (Q S0^T) + QKm U
//   S1^T = gamma_{n-1} S0^T + K^T diag(dec) U
//
// Decays are always formed as exp of a non-positive difference of fp64
// partial sums, so nothing overflows and nothing but true decay underflows.
//
// Three launches:
//   1. chunk_offsets_kernel: chunk_off[n] = chunks before sequence n.
//   2. chunk_prep_kernel, one workgroup per (chunk, value head), fully
//      parallel: stages the block's K and Q in LDS, forms the Gram products
//      on MFMA, the gate prefix sums, A, and T = (I + A)^{-1} (16x16 diagonal
//      blocks by forward substitution in registers, off-diagonal blocks by
//      fp32 MFMA block products), and writes T, QKm and the per-token scalars
//      to the workspace as ready-to-use MFMA A fragments.
//   3. chunk_sweep_kernel, one workgroup per (sequence, value head, 16 rows of
//      the state): walks the chunks in order with its 16 x d_k slice of the
//      fp32 state held in MFMA accumulators.  State rows are independent
//      given the block's T, so the 16-row slices of one head never talk to
//      each other.
//
// Precision.  bf16 inputs (K, Q, V) enter MFMA exactly.  Every derived fp32
// operand (S, Y, U, dec*U, T, QKm) is split into hi + lo bf16 halves, so the
// block products keep about 16 mantissa bits per operand and fp32
// accumulation.  fp32 inputs use fp32 MFMA throughout.
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

template <int C>
struct Geom {
  static constexpr int NB = C / 16;                 // 16-token blocks per chunk
  static constexpr int NBLK = NB * (NB + 1) / 2;    // lower-triangular 16x16 blocks
  static constexpr size_t FRAG = 64 * 16;           // one 16x16 fragment: 64 lanes x 16 bytes
  static constexpr size_t T_OFF = 0;
  static constexpr size_t QK_OFF = NBLK * FRAG;
  static constexpr size_t SCAL_OFF = 2 * NBLK * FRAG;
  static constexpr size_t BYTES = SCAL_OFF + 4 * C * sizeof(float);  // per (chunk, value head)
  static_assert(BYTES % 256 == 0, "keep per-chunk blocks 256-byte aligned");
};

__device__ __forceinline__ int blk_index(int r, int i) { return r * (r + 1) / 2 + i; }

__device__ __forceinline__ void blk_decode(int p, int& r, int& i) {
  r = 0;
  while ((r + 1) * (r + 2) / 2 <= p) ++r;
  i = p - r * (r + 1) / 2;
}

// 16-byte fragment in its workspace / LDS form: split bf16 (hi, lo) or fp32.
template <bool BF>
__device__ __forceinline__ uint4 pack_frag(f4 x) {
  if constexpr (BF) {
    sfrag s = split4(x);
    uint4 r;
    r.x = uint32_t(uint16_t(s.hi[0])) | (uint32_t(uint16_t(s.hi[1])) << 16);
    r.y = uint32_t(uint16_t(s.hi[2])) | (uint32_t(uint16_t(s.hi[3])) << 16);
    r.z = uint32_t(uint16_t(s.lo[0])) | (uint32_t(uint16_t(s.lo[1])) << 16);
    r.w = uint32_t(uint16_t(s.lo[2])) | (uint32_t(uint16_t(s.lo[3])) << 16);
    return r;
  } else {
    uint4 r;
    r.x = __float_as_uint(x[0]);
    r.y = __float_as_uint(x[1]);
    r.z = __float_as_uint(x[2]);
    r.w = __float_as_uint(x[3]);
    return r;
  }
}

__device__ __forceinline__ sfrag as_sfrag(uint4 u) {
  sfrag s;
  s.hi = pack4(uint16_t(u.x), uint16_t(u.x >> 16), uint16_t(u.y), uint16_t(u.y >> 16));
  s.lo = pack4(uint16_t(u.z), uint16_t(u.z >> 16), uint16_t(u.w), uint16_t(u.w >> 16));
  return s;
}
__device__ __forceinline__ f4 as_f4(uint4 u) {
  return f4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}

// derived (split) x derived (split)
template <bool BF>
__device__ __forceinline__ f4 mma_dd(uint4 a, uint4 b, f4 c) {
  if constexpr (BF) return mma_s_s(as_sfrag(a), as_sfrag(b), c);
  else return mma_f32(as_f4(a), as_f4(b), c);
}

// Four consecutive io elements from LDS as an exact operand fragment.
template <typename IO>
struct ExactFrag;
template <>
struct ExactFrag<uint16_t> {
  s4 v;
  __device__ __forceinline__ void load_row(const uint16_t* p) { v = *reinterpret_cast<const s4*>(p); }
  __device__ __forceinline__ void load_col(const uint16_t* p, int stride) {
    v = pack4(p[0], p[stride], p[2 * stride], p[3 * stride]);
  }
  // exact x derived
  __device__ __forceinline__ f4 mma(uint4 b, f4 c) const { return mma_e_s(v, as_sfrag(b), c); }
  __device__ __forceinline__ f4 mma_exact(const ExactFrag& b, f4 c) const { return mma_bf(v, b.v, c); }
};
template <>
struct ExactFrag<float> {
  f4 v;
  __device__ __forceinline__ void load_row(const float* p) { v = *reinterpret_cast<const f4*>(p); }
  __device__ __forceinline__ void load_col(const float* p, int stride) {
    v = f4{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
  __device__ __forceinline__ f4 mma(uint4 b, f4 c) const { return mma_f32(v, as_f4(b), c); }
  __device__ __forceinline__ f4 mma_exact(const ExactFrag& b, f4 c) const { return mma_f32(v, b.v, c); }
};

// Stage rows [t0, t0 + nc) of head j of a [T, h, DK] tensor into LDS rows of
// KP elements; rows nc..C-1 are zero-filled.
template <typename IO, int DK, int C, int KP, int NT>
__device__ __forceinline__ void stage_rows(IO* dst, const IO* __restrict__ src, int t0, int nc, int heads, int j,
                                           int tid) {
  constexpr int E16 = 16 / sizeof(IO);
  constexpr int PER_ROW = DK / E16;
  for (int x = tid; x < C * PER_ROW; x += NT) {
    const int r = x / PER_ROW, cc = (x % PER_ROW) * E16;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < nc) val = *reinterpret_cast<const uint4*>(src + (size_t(t0 + r) * heads + j) * DK + cc);
    *reinterpret_cast<uint4*>(dst + r * KP + cc) = val;
  }
}

template <typename IO, int DK, int C>
struct PrepLds {
  static constexpr int E16 = 16 / sizeof(IO);
  static constexpr int KP = DK + E16;  // padded row, elements
  static constexpr int AP = C + 4;     // padded fp32 row of A and T
  static constexpr size_t KQ_BYTES = 2 * size_t(C) * KP * sizeof(IO);
  static constexpr size_t T_BYTES = size_t(C) * AP * sizeof(float);
  static constexpr size_t R0 = KQ_BYTES > T_BYTES ? KQ_BYTES : T_BYTES;  // K, Q; later T
  static constexpr size_t A_OFF = R0;
  static constexpr size_t G_OFF = A_OFF + T_BYTES;  // fp64 prefix sums
  static constexpr size_t B_OFF = G_OFF + C * sizeof(double);
  static constexpr size_t BYTES = B_OFF + C * sizeof(float);
};

template <typename IO, int DK, int C>
struct SweepLds {
  static constexpr int NB = C / 16, KB = DK / 16;
  static constexpr int E16 = 16 / sizeof(IO);
  static constexpr int KP = DK + E16;
  static constexpr size_t Q_OFF = size_t(C) * KP * sizeof(IO);
  static constexpr size_t S_OFF = 2 * Q_OFF;
  static constexpr size_t Y_OFF = S_OFF + KB * 1024;
  static constexpr size_t U_OFF = Y_OFF + NB * 1024;
  static constexpr size_t UD_OFF = U_OFF + NB * 1024;
  static constexpr size_t SC_OFF = UD_OFF + NB * 1024;
  static constexpr size_t BYTES = SC_OFF + 4 * C * sizeof(float);
};

}  // namespace

// chunk_off[n] = number of C-token chunks in sequences 0..n-1; chunk_off[N] = total.
__global__ __launch_bounds__(256) void chunk_offsets_kernel(int N, int T, int C, const int32_t* __restrict__ cu,
                                                            int32_t* __restrict__ chunk_off) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256;
  const int lo = min(N, tid * per), hi = min(N, lo + per);
  int sum = 0;
  for (int n = lo; n < hi; ++n) {
    int b, e;
    seq_range(cu, n, T, b, e);
    sum += (e - b + C - 1) / C;
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int n = lo; n < hi; ++n) {
    chunk_off[n] = run;
    int b, e;
    seq_range(cu, n, T, b, e);
    run += (e - b + C - 1) / C;
  }
  if (tid == 255) chunk_off[N] = part[255];
}

template <typename IO, int DK, int C>
__global__ __launch_bounds__(256) void chunk_prep_kernel(int N, int T, int h_qk, int h_v,
                                                         const IO* __restrict__ q, const IO* __restrict__ k,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ beta,
                                                         const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ chunk_off,
                                                         uint8_t* __restrict__ ws) {
  using Geo = Geom<C>;
  using Lds = PrepLds<IO, DK, C>;
  constexpr int NB = Geo::NB, NBLK = Geo::NBLK, KB = DK / 16;
  constexpr bool BF = sizeof(IO) == 2;
  constexpr int KP = Lds::KP, AP = Lds::AP;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  IO* sK = reinterpret_cast<IO*>(smem);
  IO* sQ = sK + C * KP;
  float* sT = reinterpret_cast<float*>(smem);  // reuses the K/Q region after the Gram products
  float* sA = reinterpret_cast<float*>(smem + Lds::A_OFF);
  double* sG = reinterpret_cast<double*>(smem + Lds::G_OFF);
  float* sBeta = reinterpret_cast<float*>(smem + Lds::B_OFF);

  const int gc = blockIdx.x, h = blockIdx.y;
  if (gc >= chunk_off[N]) return;
  int lo = 0, hi = N - 1;  // last sequence whose first chunk is <= gc
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= gc) lo = mid;
    else hi = mid - 1;
  }
  int bos, eos;
  seq_range(cu, lo, T, bos, eos);
  const int t0 = bos + (gc - chunk_off[lo]) * C;
  const int nc = min(C, eos - t0);
  if (nc <= 0) return;
  const int j = h / (h_v / h_qk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  uint8_t* wsb = ws + (size_t(gc) * h_v + h) * Geo::BYTES;

  stage_rows<IO, DK, C, KP, 256>(sK, k, t0, nc, h_qk, j, tid);
  stage_rows<IO, DK, C, KP, 256>(sQ, q, t0, nc, h_qk, j, tid);
  if (wave == 0) {
    double gl = 0.0;
    float bl = 0.f;
    if (lane < nc) {
      gl = g[size_t(t0 + lane) * h_v + h];
      bl = beta[size_t(t0 + lane) * h_v + h];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(gl, off);
      if (lane >= off) gl += y;
    }
    const double glast = __shfl(gl, nc - 1);
    if (lane < C) {
      sG[lane] = gl;
      sBeta[lane] = bl;
      const float gam = lane < nc ? float(exp(gl)) : 0.f;
      const float dec = lane < nc ? float(exp(glast - gl)) : 0.f;
      float* sc = reinterpret_cast<float*>(wsb + Geo::SCAL_OFF);
      sc[lane] = bl;
      sc[C + lane] = bl * gam;
      sc[2 * C + lane] = gam;
      sc[3 * C + lane] = dec;
    }
  }
  __syncthreads();

  // Gram blocks.  p < NBLK: K K^T block (r, i) -> A (strictly lower, scaled) in LDS.
  // p >= NBLK: K Q^T block (i, r), whose D layout is the A fragment of QK^T
  // block (r, i) -> masked, decayed, written to the workspace.
  for (int p = wave; p < 2 * NBLK; p += 4) {
    const bool isA = p < NBLK;
    int r, i;
    blk_decode(isA ? p : p - NBLK, r, i);
    const int ra = isA ? r : i;
    const IO* bsrc = isA ? sK + (16 * i + col) * KP : sQ + (16 * r + col) * KP;
    const IO* asrc = sK + (16 * ra + col) * KP;
    f4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KB; ++s) {
      ExactFrag<IO> a, b;
      a.load_row(asrc + 16 * s + 4 * grp);
      b.load_row(bsrc + 16 * s + 4 * grp);
      acc = a.mma_exact(b, acc);
    }
    if (isA) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * r + 4 * grp + e, cl = 16 * i + col;
        float val = 0.f;
        if (cl < row) val = sBeta[row] * expf(float(sG[row] - sG[cl])) * acc[e];
        sA[row * AP + cl] = val;
      }
    } else {
      f4 m;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * r + col, cl = 16 * i + 4 * grp + e;
        m[e] = cl <= row ? expf(float(sG[row] - sG[cl])) * acc[e] : 0.f;
      }
      *reinterpret_cast<uint4*>(wsb + Geo::QK_OFF + blk_index(r, i) * Geo::FRAG + lane * 16) = pack_frag<BF>(m);
    }
  }
  __syncthreads();  // A complete; K and Q are dead, their space becomes T

  // Diagonal blocks: T_bb = (I + A_bb)^{-1}.  Lane 4c+s owns column c and the
  // rows congruent to s mod 4; each row is one quad reduction.
  if (wave < NB) {
    const int b = wave, c = lane >> 2, s = lane & 3;
    float a[16][4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int m = 0; m < 4; ++m) a[rr][m] = sA[(16 * b + rr) * AP + 16 * b + 4 * m + s];
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float part = a[rr][0] * t[0] + a[rr][1] * t[1] + a[rr][2] * t[2] + a[rr][3] * t[3];
      const float val = (rr == c ? 1.f : 0.f) - sum_lanes4(part);
      if (s == (rr & 3)) t[rr >> 2] = val;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) sT[(16 * b + 4 * m + s) * AP + 16 * b + c] = t[m];
  }
  __syncthreads();

  // Off-diagonal blocks, one block row at a time:
  //   T(i, jj) = -T(i, i) * sum_{kk = jj}^{i-1} A(i, kk) T(kk, jj)
  for (int i = 1; i < NB; ++i) {
    if (wave < i) {
      const int jj = wave;
      f4 P = zero4();
      for (int kk = jj; kk < i; ++kk) {
        const f4 a = *reinterpret_cast<const f4*>(&sA[(16 * i + col) * AP + 16 * kk + 4 * grp]);
        f4 bt;
#pragma unroll
        for (int e = 0; e < 4; ++e) bt[e] = sT[(16 * kk + 4 * grp + e) * AP + 16 * jj + col];
        P = mma_f32(a, bt, P);
      }
      const f4 tii = *reinterpret_cast<const f4*>(&sT[(16 * i + col) * AP + 16 * i + 4 * grp]);
      const f4 R = mma_f32(tii, P, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * grp + e) * AP + 16 * jj + col] = -R[e];
    }
    __syncthreads();
  }

  for (int p = wave; p < NBLK; p += 4) {
    int r, i;
    blk_decode(p, r, i);
    const f4 x = *reinterpret_cast<const f4*>(&sT[(16 * r + col) * AP + 16 * i + 4 * grp]);
    *reinterpret_cast<uint4*>(wsb + Geo::T_OFF + blk_index(r, i) * Geo::FRAG + lane * 16) = pack_frag<BF>(x);
  }
}

template <typename IO, int DK, int C>
__global__ __launch_bounds__(256) void chunk_sweep_kernel(int N, int T, int h_qk, int h_v, int d_v, int max_chunks,
                                                          const IO* __restrict__ q, const IO* __restrict__ k,
                                                          const IO* __restrict__ v, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ chunk_off,
                                                          const uint8_t* __restrict__ ws, const float* s_in,
                                                          IO* __restrict__ out, float* s_out) {
  using Geo = Geom<C>;
  using Lds = SweepLds<IO, DK, C>;
  constexpr int NB = Geo::NB, KB = DK / 16, KP = Lds::KP;
  constexpr int SB = (KB + 3) / 4;  // state blocks per wave
  constexpr bool BF = sizeof(IO) == 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  IO* sK = reinterpret_cast<IO*>(smem);
  IO* sQ = reinterpret_cast<IO*>(smem + Lds::Q_OFF);
  uint4* sS = reinterpret_cast<uint4*>(smem + Lds::S_OFF);
  uint4* sY = reinterpret_cast<uint4*>(smem + Lds::Y_OFF);
  uint4* sU = reinterpret_cast<uint4*>(smem + Lds::U_OFF);
  uint4* sUd = reinterpret_cast<uint4*>(smem + Lds::UD_OFF);
  float* sSc = reinterpret_cast<float*>(smem + Lds::SC_OFF);

  // Workgroups are dealt to the 8 XCDs round-robin; give the 16-row slices of
  // one head consecutive chain numbers on one XCD so they share its L2.
  const int ntile = d_v / 16;
  const int nchain = N * h_v * ntile;
  const int per = (nchain + 7) / 8;
  const int L = int(blockIdx.x & 7) * per + int(blockIdx.x >> 3);
  if (L >= nchain) return;
  const int tl = L % ntile, nh = L / ntile, h = nh % h_v, n = nh / h_v;
  const int j = h / (h_v / h_qk);
  const int dv0 = 16 * tl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, col = lane & 15;

  f4 st[SB];
#pragma unroll
  for (int bi = 0; bi < SB; ++bi) {
    const int b = wave + 4 * bi;
    if (b < KB) {
      st[bi] = s_in ? *reinterpret_cast<const f4*>(s_in + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp)
                    : zero4();
      sS[b * 64 + lane] = pack_frag<BF>(st[bi]);
    }
  }
  int bos, eos;
  seq_range(cu, n, T, bos, eos);
  const int nchunk = (eos - bos + C - 1) / C;
  const int gc0 = chunk_off[n];

  for (int cc = 0; cc < nchunk; ++cc) {
    const int gc = gc0 + cc;
    if (gc >= max_chunks) break;
    const int t0 = bos + cc * C;
    const int nc = min(C, eos - t0);
    const uint8_t* wsb = ws + (size_t(gc) * h_v + h) * Geo::BYTES;

    // (a) stage the chunk; fetch this wave's T and QKm fragments and V values
    stage_rows<IO, DK, C, KP, 256>(sK, k, t0, nc, h_qk, j, tid);
    stage_rows<IO, DK, C, KP, 256>(sQ, q, t0, nc, h_qk, j, tid);
    for (int x = tid; x < 4 * C; x += 256) sSc[x] = reinterpret_cast<const float*>(wsb + Geo::SCAL_OFF)[x];
    uint4 tf[NB], qf[NB];
    float vv[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave < NB) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i <= wave) {
          tf[i] = *reinterpret_cast<const uint4*>(wsb + Geo::T_OFF + blk_index(wave, i) * Geo::FRAG + lane * 16);
          qf[i] = *reinterpret_cast<const uint4*>(wsb + Geo::QK_OFF + blk_index(wave, i) * Geo::FRAG + lane * 16);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * wave + 4 * grp + e;
        if (tok < nc) vv[e] = io_traits<IO>::load(v + (size_t(t0 + tok) * h_v + h) * d_v + dv0 + col);
      }
    }
    __syncthreads();

    // (b) X = K S^T and Z = Q S^T for token block r = wave; Y = beta V - beta gamma X
    f4 z = zero4();
    if (wave < NB) {
      const int r = wave;
      f4 x = zero4();
#pragma unroll
      for (int s = 0; s < KB; ++s) {
        const uint4 sb = sS[s * 64 + lane];
        ExactFrag<IO> ak, aq;
        ak.load_row(sK + (16 * r + col) * KP + 16 * s + 4 * grp);
        aq.load_row(sQ + (16 * r + col) * KP + 16 * s + 4 * grp);
        x = ak.mma(sb, x);
        z = aq.mma(sb, z);
      }
      f4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * r + 4 * grp + e;
        y[e] = sSc[tok] * vv[e] - sSc[C + tok] * x[e];
      }
      sY[r * 64 + lane] = pack_frag<BF>(y);
    }
    __syncthreads();

    // (c) U = T Y for block row r; also dec * U for the state update
    if (wave < NB) {
      const int r = wave;
      f4 u = zero4();
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i <= r) u = mma_dd<BF>(tf[i], sY[i * 64 + lane], u);
      sU[r * 64 + lane] = pack_frag<BF>(u);
      f4 ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) ud[e] = sSc[3 * C + 16 * r + 4 * grp + e] * u[e];
      sUd[r * 64 + lane] = pack_frag<BF>(ud);
    }
    __syncthreads();

    // (d) O = gamma Z + QKm U for block row r; S^T <- gamma_last S^T + K^T (dec U)
    if (wave < NB) {
      const int r = wave;
      f4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sSc[2 * C + 16 * r + 4 * grp + e] * z[e];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i <= r) o = mma_dd<BF>(qf[i], sU[i * 64 + lane], o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * r + 4 * grp + e;
        if (tok < nc) io_traits<IO>::store(out + (size_t(t0 + tok) * h_v + h) * d_v + dv0 + col, o[e]);
      }
    }
    const float glast = sSc[2 * C + nc - 1];
#pragma unroll
    for (int bi = 0; bi < SB; ++bi) {
      const int b = wave + 4 * bi;
      if (b < KB) {
        f4 acc = st[bi] * glast;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          ExactFrag<IO> a;
          a.load_col(sK + (16 * i + 4 * grp) * KP + 16 * b + col, KP);
          acc = a.mma(sUd[i * 64 + lane], acc);
        }
        st[bi] = acc;
        sS[b * 64 + lane] = pack_frag<BF>(acc);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int bi = 0; bi < SB; ++bi) {
    const int b = wave + 4 * bi;
    if (b < KB) *reinterpret_cast<f4*>(s_out + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp) = st[bi];
  }
}

// ---------------------------------------------------------------- host side

size_t chunked_max_chunks(const Dims& d, int chunk) {
  // sum_n ceil(L_n / C) <= (T + N (C - 1)) / C
  return (size_t(d.total_tokens) + size_t(d.num_seqs) * size_t(chunk - 1)) / size_t(chunk);
}

static size_t chunk_bytes(int chunk) {
  switch (chunk) {
    case 16: return Geom<16>::BYTES;
    case 32: return Geom<32>::BYTES;
    case 64: return Geom<64>::BYTES;
  }
  return 0;
}

static size_t offsets_bytes(const Dims& d) { return (size_t(d.num_seqs + 1) * 4 + 255) / 256 * 256; }

size_t chunked_workspace_bytes(const Dims& d, int chunk) {
  const size_t cb = chunk_bytes(chunk);
  if (cb == 0) return 0;
  return offsets_bytes(d) + chunked_max_chunks(d, chunk) * size_t(d.h_v) * cb;
}

template <typename IO, int DK, int C>
static hipError_t launch_chunked_t(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const int32_t* cu, const float* s_in, void* out,
                                   float* s_out, void* workspace, hipStream_t st) {
  int32_t* chunk_off = static_cast<int32_t*>(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace) + offsets_bytes(d);
  const size_t max_chunks = chunked_max_chunks(d, C);
  {
    Prof prof("chunk_offsets", st);
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, d.num_seqs, d.total_tokens, C, cu,
                       chunk_off);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (max_chunks > 0) {
    constexpr size_t lds = PrepLds<IO, DK, C>::BYTES;
    if (lds > 65536) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prep_kernel<IO, DK, C>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
    Prof prof("chunk_prep", st);
    hipLaunchKernelGGL((chunk_prep_kernel<IO, DK, C>), dim3(unsigned(max_chunks), unsigned(d.h_v)), dim3(256), lds,
                       st, d.num_seqs, d.total_tokens, d.h_qk, d.h_v, static_cast<const IO*>(q),
                       static_cast<const IO*>(k), g, beta, cu, chunk_off, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nchain = d.num_seqs * d.h_v * (d.d_v / 16);
  if (nchain == 0) return hipSuccess;
  const int per = (nchain + 7) / 8;
  constexpr size_t lds = SweepLds<IO, DK, C>::BYTES;
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_sweep_kernel<IO, DK, C>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  Prof prof("chunk_sweep", st);
  hipLaunchKernelGGL((chunk_sweep_kernel<IO, DK, C>), dim3(8 * per), dim3(256), lds, st, d.num_seqs,
                     d.total_tokens, d.h_qk, d.h_v, d.d_v, int(max_chunks), static_cast<const IO*>(q),
                     static_cast<const IO*>(k), static_cast<const IO*>(v), cu, chunk_off, ws, s_in,
                     static_cast<IO*>(out), s_out);
  return hipGetLastError();
}

template <typename IO, int DK>
static hipError_t launch_chunked_c(const Dims& d, int chunk, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu, const float* s_in,
                                   void* out, float* s_out, void* ws, hipStream_t st) {
  switch (chunk) {
    case 16: return launch_chunked_t<IO, DK, 16>(d, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
    case 32: return launch_chunked_t<IO, DK, 32>(d, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
    case 64: return launch_chunked_t<IO, DK, 64>(d, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
static hipError_t launch_chunked_k(const Dims& d, int chunk, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu, const float* s_in,
                                   void* out, float* s_out, void* ws, hipStream_t st) {
  switch (d.d_k) {
    case 16: return launch_chunked_c<IO, 16>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
    case 32: return launch_chunked_c<IO, 32>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
    case 64: return launch_chunked_c<IO, 64>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
    case 128: return launch_chunked_c<IO, 128>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, ws, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunked(const Dims& d, int chunk, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu, const float* s_in, void* out, float* s_out,
                          void* workspace, hipStream_t st) {
  if (d.bf16) return launch_chunked_k<uint16_t>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, workspace, st);
  return launch_chunked_k<float>(d, chunk, q, k, v, g, beta, cu, s_in, out, s_out, workspace, st);
}

}  // namespace gdn
