// Decode attention over a grouped-query KV cache.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", sections
// "Pack query heads to reuse KV rows" and "Switch attention layouts at long
// contexts": in a decode step of a full-attention layer every query head reads
// the whole KV cache of its KV head, and the query heads of one group (eight
// in the model described there) read the same rows.  Packing several query
// heads into one workgroup loads each KV row once for all of them; the
// fixed-block layout splits each context into equal parts that run in
// parallel and are merged afterwards.  Neither changes the result.
//
// o[b, h] = sum_t softmax_t(scale q[b, h] . k[b, j, t]) v[b, j, t] over the
// first context_lens[b] positions, j = h / (h_q / h_kv).
//
// One workgroup of four waves serves HP query heads of one KV head over a
// range of positions (the whole context in the general layout, one of nb
// equal parts in the fixed-block layout).  Wave w takes the 16-position tiles
// w, w + 4, ... of that range, and loads the next tile's key and value rows
// while it works on the current one.  Per tile, all on the matrix unit
// except the softmax bookkeeping:
//   * scores S[16 positions, 16 columns] = K_tile Q^T, four-wide bf16
//     v_mfma_f32_16x16x32_bf16 slabs: the key rows are the A fragments,
//     loaded straight from memory (lane = 16 grp + row holds 8 consecutive
//     values of one key row per 32-wide slab); the HP queries are the B
//     fragments, held in registers for the whole range (columns past HP are
//     zero and their rows of the output are dropped);
//   * an online softmax per head in base 2 (scores times scale * log2 e): the
//     running maximum m, the rescale factor 2^(m_old - m_new) applied to the
//     output rows when it is not 1, the probabilities p and a per-lane sum l;
//   * O[heads, columns] += P V_tile with v_mfma_f32_16x16x16_bf16: the score
//     block's lane layout (head = col, positions 4 grp + r) is already the A
//     fragment of P, split into a bf16 high part and a bf16 residue so that
//     p reaches the product to 2^-17 relative; the value tile goes through a
//     per-wave LDS buffer (rows padded by 8 bytes, so that the four row groups
//     a fragment read touches fall on disjoint banks) and each B fragment
//     lane reads four positions of one column.
// The waves' (m, l, O) are merged through LDS at the end.  The general layout
// divides by l and writes bf16; the fixed-block layout writes the part's
// (m, l, O) in fp32 and attn_combine_kernel merges the parts of each head.
// Every head's arithmetic is the same whatever HP is (its column of the score
// block and its row of the output block are computed independently of the
// others), so packed and unpacked launches give the same bytes.
#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kWaves = 4;  // waves per workgroup of the decode kernel (8 measured no faster)
constexpr int kTile = 16;  // positions per wave step

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint16_t* q;     // [B, h_q, DK]
  const uint16_t* k;     // [B, h_kv, t_max, DK]
  const uint16_t* v;     // [B, h_kv, t_max, DK]
  const int32_t* lens;   // [B]
  uint16_t* out;         // [B, h_q, DK]         (general layout)
  float* part_o;         // [B, h_q, nb, DK]     (fixed-block layout)
  float* part_ml;        // [B, h_q, nb, 2]
  int h_q, h_kv, t_max, group, packs, nb;
  float c;               // scale * log2(e)
};

__device__ __forceinline__ f4 mfma_kq(v4u a, v4u b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0,
                                                 0);
}

// LDS written by some lanes of a wave and read by others of the same wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DK, int HP, bool PARTIAL>
__global__ __launch_bounds__(64 * kWaves) void attn_decode_kernel(AttnArgs a) {
  static_assert(DK == 64 || DK == 128 || DK == 256, "head size");
  static_assert(HP == 1 || HP == 2 || HP == 4 || HP == 8, "heads per workgroup");
  constexpr int KS = DK / 32;          // 32-wide slabs of the score product
  constexpr int CB = DK / 16;          // 16-column blocks of the output
  constexpr int VS = DK + 4;           // LDS row stride of a value tile (bf16): 4 rows apart -> 32 bytes of banks apart
  constexpr int CPR = DK / 8;          // 16-byte chunks per value row
  constexpr int RPI = 64 / CPR;        // value rows per load instruction
  constexpr int VLD = kTile / RPI;     // value load instructions per tile

  // the value tiles during the loop, the waves' outputs after it
  constexpr int kVtBytes = kWaves * kTile * VS * 2, kSoBytes = kWaves * HP * DK * 4;
  __shared__ __align__(16) unsigned char lds_raw[kVtBytes > kSoBytes ? kVtBytes : kSoBytes];
  __shared__ float sm[kWaves][HP], sl[kWaves][HP];
  auto vt = reinterpret_cast<uint16_t(*)[kTile * VS]>(lds_raw);
  auto so = reinterpret_cast<float(*)[HP][DK]>(lds_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int wg = blockIdx.x;
  const int blk = wg % a.nb;
  wg /= a.nb;
  const int pk = wg % a.packs;
  wg /= a.packs;
  const int j = wg % a.h_kv, b = wg / a.h_kv;
  const int h0 = j * a.group + pk * HP;

  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.t_max ? a.t_max : len);
  int start = 0, end = len;
  if (PARTIAL) {
    const int part = ((len + a.nb - 1) / a.nb + kTile - 1) / kTile * kTile;
    start = min(blk * part, len);
    end = min(start + part, len);
  }
  const size_t kv_off = (size_t(b) * a.h_kv + j) * size_t(a.t_max) * DK;
  const uint16_t* kb = a.k + kv_off;
  const uint16_t* vb = a.v + kv_off;

  const int col = lane & 15, grp = lane >> 4;          // fragment coordinates
  const int vrow = lane / CPR, vch = lane % CPR;       // value-load coordinates

  v4u qf[KS];
  {
    const uint16_t* qp = a.q + (size_t(b) * a.h_q + h0 + (col < HP ? col : 0)) * DK + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = col < HP ? *reinterpret_cast<const v4u*>(qp + 32 * kk) : v4u{0, 0, 0, 0};
  }

  f4 o[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) o[c] = zero4();
  float m_run = -INFINITY, l_run = 0.f;

  // Rows past the range are clamped to its last row (read, then masked).
  auto load_k = [&](int t0, v4u (&kf)[KS]) {
    const uint16_t* kp = kb + size_t(min(t0 + col, end - 1)) * DK + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = *reinterpret_cast<const v4u*>(kp + 32 * kk);
  };
  auto load_v = [&](int t0, v4u (&vr)[VLD]) {
#pragma unroll
    for (int i = 0; i < VLD; ++i)
      vr[i] = *reinterpret_cast<const v4u*>(vb + size_t(min(t0 + RPI * i + vrow, end - 1)) * DK + 8 * vch);
  };

  v4u kf[KS], vr[VLD];
  uint16_t* vw = &vt[wave][0];
  if (start + wave * kTile < end) {
    load_k(start + wave * kTile, kf);
    load_v(start + wave * kTile, vr);
  }
  for (int t0 = start + wave * kTile; t0 < end; t0 += kWaves * kTile) {
    // this tile's value rows to LDS, the next tile's rows in flight
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(vw + (RPI * i + vrow) * VS + 8 * vch);
      *reinterpret_cast<v2u*>(dst) = v2u{vr[i].x, vr[i].y};
      *reinterpret_cast<v2u*>(dst + 2) = v2u{vr[i].z, vr[i].w};
    }
    v4u kn[KS];
    load_k(t0 + kWaves * kTile, kn);
    load_v(t0 + kWaves * kTile, vr);

    f4 s = zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = mfma_kq(kf[kk], qf[kk], s);

    // lane (col, grp) holds the scores of head col at positions t0 + 4 grp + r
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = t0 + 4 * grp + r < end ? s[r] * a.c : -INFINITY;
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float al = exp2_(m_run - m_use);
    f4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2_(x[r] - m_use);
    l_run = l_run * al + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    // p is the A fragment of P (rows = heads, k = positions 4 grp + r); hi + lo bf16 carry it to 2^-17
    const sfrag ps = split4(p);

    // rescale the output rows (head 4 grp + r) by their heads' factors, unless all are 1
    if (__any(al != 1.f)) {
      float ah[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ah[r] = __shfl(al, 4 * grp + r);
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] *= ah[r];
    }
    wave_sync();
    // O[head, 16 c + col] += sum_positions P[head, pos] V[pos, 16 c + col]; the B fragment
    // lane (col, grp) holds V[4 grp + r][16 c + col]
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const uint16_t* vp = vw + 4 * grp * VS + 16 * c + col;
      const s4 vf = pack4(vp[0], vp[VS], vp[2 * VS], vp[3 * VS]);
      o[c] = mma_bf(ps.lo, vf, o[c]);
      o[c] = mma_bf(ps.hi, vf, o[c]);
    }
    wave_sync();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = kn[kk];
  }

  // per-wave totals: l over the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (col < HP && grp == 0) {
    sm[wave][col] = m_run;
    sl[wave][col] = l_run;
  }
  __syncthreads();  // every wave is done with its value tile before the outputs overwrite them
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * grp + r < HP) so[wave][4 * grp + r][16 * c + col] = o[c][r];
  __syncthreads();

  constexpr int LPT = DK / 4;
  for (int idx = tid; idx < HP * LPT; idx += 64 * kWaves) {
    const int h = idx / LPT, c4 = idx % LPT;
    float mx = sm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm[w][h]);
    float L = 0.f;
    f4 O = zero4();
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = exp2_(sm[w][h] - mx);
        L += wt * sl[w][h];
        const f4 ow = *reinterpret_cast<const f4*>(&so[w][h][4 * c4]);
        O += wt * ow;
      }
    }
    const size_t row = size_t(b) * a.h_q + h0 + h;
    if (PARTIAL) {
      const size_t pr = row * a.nb + blk;
      *reinterpret_cast<f4*>(a.part_o + pr * DK + 4 * c4) = O;
      if (c4 == 0) *reinterpret_cast<f2v*>(a.part_ml + pr * 2) = f2v{mx, L};
    } else {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      *reinterpret_cast<v2u*>(a.out + row * DK + 4 * c4) =
          v2u{pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv)};
    }
  }
}

// Merge the nb parts of each (sequence, query head): workgroup (row, chunk)
// owns 64 output columns of one row, in sixteen slices of parts (16 lanes x 4
// columns each).  A slice merges its parts c = slice, slice + 16, ... in
// registers, online (running maximum, rescaled sum and output), with the
// loads of eight parts issued before their merge; the sixteen slices are then
// merged through LDS.  The order is fixed, so the result is deterministic.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* part_o, const float* part_ml, uint16_t* out,
                                                           int nb, int dk) {
  constexpr int kAhead = 8;  // parts per slice whose loads are in flight together
  __shared__ float cm[16], cl[16];
  __shared__ __align__(16) float co[16][64];
  const int tid = threadIdx.x;
  const int chunks = dk / 64;
  const size_t row = blockIdx.x / chunks;
  const int c0 = (blockIdx.x % chunks) * 64;
  const int slice = tid >> 4, c4 = tid & 15;
  const float* pml = part_ml + row * nb * 2;
  const float* po = part_o + row * nb * size_t(dk) + c0 + 4 * c4;

  float M = -INFINITY, L = 0.f;
  f4 O = zero4();
  for (int base = slice; base < nb; base += 16 * kAhead) {
    f2v ml[kAhead];
    f4 x[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int c = base + 16 * i;
      ml[i] = c < nb ? *reinterpret_cast<const f2v*>(pml + 2 * c) : f2v{-INFINITY, 0.f};
      x[i] = c < nb ? *reinterpret_cast<const f4*>(po + size_t(c) * dk) : zero4();
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (ml[i][0] == -INFINITY) continue;  // an empty part (or past the last)
      const float mn = fmaxf(M, ml[i][0]);
      const float a1 = exp2_(M - mn), a2 = exp2_(ml[i][0] - mn);
      L = L * a1 + ml[i][1] * a2;
      O = O * a1 + x[i] * a2;
      M = mn;
    }
  }
  if (c4 == 0) {
    cm[slice] = M;
    cl[slice] = L;
  }
  *reinterpret_cast<f4*>(&co[slice][4 * c4]) = O;
  __syncthreads();
  if (tid < 16) {
    float mx = cm[0];
#pragma unroll
    for (int sl = 1; sl < 16; ++sl) mx = fmaxf(mx, cm[sl]);
    float Lt = 0.f;
    f4 Ot = zero4();
    if (mx != -INFINITY) {
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) {
        const float wt = exp2_(cm[sl] - mx);
        Lt += wt * cl[sl];
        Ot += wt * *reinterpret_cast<const f4*>(&co[sl][4 * tid]);
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    *reinterpret_cast<v2u*>(out + row * dk + c0 + 4 * tid) =
        v2u{pack_bf16x2(Ot[0] * inv, Ot[1] * inv), pack_bf16x2(Ot[2] * inv, Ot[3] * inv)};
  }
}

template <int DK, int HP>
hipError_t launch_attn_t(const AttnDims& d, const AttnArgs& a, bool fixed_block, hipStream_t st) {
  const unsigned blocks = unsigned(size_t(d.batch) * d.h_kv * a.packs * a.nb);
  if (fixed_block) {
    {
      Prof prof("attn_decode_parts", st);
      hipLaunchKernelGGL((attn_decode_kernel<DK, HP, true>), dim3(blocks), dim3(64 * kWaves), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    Prof prof("attn_combine", st);
    hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(size_t(d.batch) * d.h_q * (DK / 64))), dim3(256), 0, st,
                       a.part_o, a.part_ml, a.out, a.nb, DK);
    return hipGetLastError();
  }
  Prof prof("attn_decode", st);
  hipLaunchKernelGGL((attn_decode_kernel<DK, HP, false>), dim3(blocks), dim3(64 * kWaves), 0, st, a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_attn_dk(const AttnDims& d, const AttnArgs& a, int hp, bool fixed_block, hipStream_t st) {
  switch (hp) {
    case 1: return launch_attn_t<DK, 1>(d, a, fixed_block, st);
    case 2: return launch_attn_t<DK, 2>(d, a, fixed_block, st);
    case 4: return launch_attn_t<DK, 4>(d, a, fixed_block, st);
    default: return launch_attn_t<DK, 8>(d, a, fixed_block, st);
  }
}

}  // namespace

size_t attn_workspace_bytes(const AttnDims& d, int nb) {
  const size_t rows = size_t(d.batch) * d.h_q * size_t(nb);
  const size_t o_bytes = (rows * d.head_dim * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * 2 * sizeof(float);
}

hipError_t launch_attn_decode(const AttnDims& d, float scale, bool fixed_block, int hp, int nb, const void* q,
                              const void* k, const void* v, const int32_t* lens, void* out, void* workspace,
                              hipStream_t st) {
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lens = lens;
  a.out = static_cast<uint16_t*>(out);
  a.h_q = d.h_q;
  a.h_kv = d.h_kv;
  a.t_max = d.t_max;
  a.group = d.h_q / d.h_kv;
  a.packs = a.group / hp;
  a.nb = fixed_block ? nb : 1;
  a.c = scale * 1.4426950408889634f;
  if (fixed_block) {
    const size_t rows = size_t(d.batch) * d.h_q * size_t(nb);
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (rows * d.head_dim * sizeof(float) + 255) / 256 * 256);
  } else {
    a.part_o = a.part_ml = nullptr;
  }
  switch (d.head_dim) {
    case 64: return launch_attn_dk<64>(d, a, hp, fixed_block, st);
    case 128: return launch_attn_dk<128>(d, a, hp, fixed_block, st);
    default: return launch_attn_dk<256>(d, a, hp, fixed_block, st);
  }
}

}  // namespace gdn
