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
//   O   = diag(gamma) (Q S0^T) + R Y,          R  = QKm T
//   S1^T = gamma_{n-1} S0^T + K^T (T' Y),      T' = diag(dec) T
//
// (U = T Y is the block's matrix of delta updates; folding T into R and T'
// leaves two block products between one state and the next.)  Decays are
// always formed as exp of a non-positive difference of fp64 partial sums, so
// nothing overflows and nothing but true decay underflows.
//
// Workspace slots: chunk j of sequence n uses slot (bos_n + n (C - 1)) / C + j
// (bos_n = its first token).  Consecutive sequences get disjoint slot ranges
// and every slot is below (T + N (C - 1)) / C, so no prefix sum over
// sequences is needed to place a chunk.
//
// Launches:
//   1. chunk_table_kernel (only for more than one sequence): per slot, the
//      chunk's (first token, length), or (0, 0) for an unused slot.  With one
//      sequence slot j is simply tokens [j C, min(T, j C + C)).
//   2. chunk_prep_kernel, one workgroup per (chunk, value head), fully
//      parallel: Gram products on MFMA, gate prefix sums, A, T = (I + A)^{-1}
//      (16x16 diagonal blocks by forward substitution in registers,
//      off-diagonal blocks by fp32 MFMA block products), R = QKm T, and the
//      per-token scalars, written to the workspace as MFMA A fragments.
//   3. chunk_sweep_kernel, one workgroup per (sequence, value head, 16 rows of
//      the state): walks the chunks in order with its 16 x d_k slice of the
//      fp32 state in MFMA accumulators.  State rows are independent given the
//      block's T, so slices of one head never talk to each other.  Chunk c+1's
//      inputs are fetched into registers while chunk c is computed, and the
//      barriers wait only for LDS traffic.
//
// All block products use 16x16x32 fragments (see gdn_common.hpp).  Precision:
// bf16 inputs (K, Q, V) enter MFMA exactly.  Y and T'Y are split into hi + lo
// bf16 halves, as is R; the state (in K S^T, Q S^T) and T' enter rounded
// once to bf16: their error reaches the outputs damped by the block decay
// and stays well below the output's own bf16 rounding.  Every product
// accumulates in fp32.  fp32 inputs use fp32 MFMA throughout.
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

struct sp8 {  // hi + lo bf16 halves of eight fp32 values
  uint4 hi, lo;
};

// Products on one 32-wide slab.  Split operands feed two accumulators (the
// hi part and the small corrections) so that consecutive products do not
// wait on each other.
__device__ __forceinline__ void mm_es(uint4 a, const sp8& b, f4& ch, f4& cl) {
  ch = mma32(a, b.hi, ch);
  cl = mma32(a, b.lo, cl);
}
__device__ __forceinline__ void mm_es(const f8& a, const f8& b, f4& ch, f4&) { ch = mma32(a, b, ch); }
__device__ __forceinline__ void mm_ss(const sp8& a, const sp8& b, f4& ch, f4& cl) {
  ch = mma32(a.hi, b.hi, ch);
  cl = mma32(a.hi, b.lo, cl);
  cl = mma32(a.lo, b.hi, cl);
}
__device__ __forceinline__ void mm_ss(const f8& a, const f8& b, f4& ch, f4&) { ch = mma32(a, b, ch); }

template <bool BF>
struct Types {
  using E = uint4;  // exact or once-rounded operand: 8 bf16
  using S = sp8;    // split operand
  using IO = uint16_t;
};
template <>
struct Types<false> {
  using E = f8;
  using S = f8;
  using IO = float;
};

__device__ __forceinline__ void zero(uint4& x) { x = uint4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void zero(f8& x) { x.a = zero4(), x.b = zero4(); }
__device__ __forceinline__ void zero(sp8& x) { zero(x.hi), zero(x.lo); }
__device__ __forceinline__ void zero(float& x) { x = 0.f; }
__device__ __forceinline__ void zero(uint16_t& x) { x = 0; }

// 8 consecutive elements of an LDS/global row as an operand.
__device__ __forceinline__ void ld8(uint4& d, const uint16_t* p) { d = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void ld8(f8& d, const float* p) {
  d.a = *reinterpret_cast<const f4*>(p);
  d.b = *reinterpret_cast<const f4*>(p + 4);
}
// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group,
// result lane i, element m is element i % 4 of the 8 bytes addressed by lane
// 4 m + i / 4 of the group.  So if lane 4 m + a addresses row m, columns
// 4 a .. 4 a + 3 of a row-major bf16 tile, lane i receives rows 0..3 of
// column i: four consecutive rows of one column, as an operand wants them.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4v lds_s4v;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(p)));
}

// 8 elements of a column (stride apart) as an operand.
__device__ __forceinline__ void ld8col(uint4& d, const uint16_t* p, int stride) {
  d = uint4{pack2(p[0], p[stride]), pack2(p[2 * stride], p[3 * stride]), pack2(p[4 * stride], p[5 * stride]),
            pack2(p[6 * stride], p[7 * stride])};
}
__device__ __forceinline__ void ld8col(f8& d, const float* p, int stride) {
  d.a = f4{p[0], p[stride], p[2 * stride], p[3 * stride]};
  d.b = f4{p[4 * stride], p[5 * stride], p[6 * stride], p[7 * stride]};
}

// Row stride (bytes) of an LDS tile read by 16-byte fragment rows (lane
// col of each 16-lane group reads row col): strides of 32 mod 128 bytes keep
// those ds_read_b128 free of bank conflicts on gfx950 (measured: 288 B rows
// run at about 205 B/clk per CU, 272 B rows at 128).
constexpr int frag_row_stride(int row_bytes) { return (row_bytes + 95) / 128 * 128 + 32; }

// Exchange buffers: [16 rows][K + pad] arrays with K contiguous, written from
// D blocks (4 consecutive k per lane) and read as B fragments (8 consecutive
// k per lane).  bf16 buffers hold either the rounded value (single) or the
// hi and lo halves in two planes; fp32 buffers hold the value.
template <bool BF, int K>
struct XBuf {
  using El = std::conditional_t<BF, uint16_t, float>;
  static constexpr int LD = frag_row_stride(K * int(sizeof(El))) / int(sizeof(El));  // row stride, elements
  static constexpr size_t PLANE = 16 * LD * sizeof(El);
};

template <bool BF, int K>
__device__ __forceinline__ void xb_write_single(uint8_t* buf, int n, int k0, f4 v) {
  using X = XBuf<BF, K>;
  if constexpr (BF) *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(buf) + n * X::LD + k0) = bf16x4(v);
  else *reinterpret_cast<f4*>(reinterpret_cast<float*>(buf) + n * X::LD + k0) = v;
}
template <bool BF, int K>
__device__ __forceinline__ void xb_write_split(uint8_t* buf, int n, int k0, f4 v) {
  using X = XBuf<BF, K>;
  if constexpr (BF) {
    uint2 h, l;
    split_bf16x4(v, h, l);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(buf) + n * X::LD + k0) = h;
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(buf + X::PLANE) + n * X::LD + k0) = l;
  } else {
    *reinterpret_cast<f4*>(reinterpret_cast<float*>(buf) + n * X::LD + k0) = v;
  }
}
template <bool BF, int K>
__device__ __forceinline__ void xb_read_single(typename Types<BF>::E& d, const uint8_t* buf, int n, int k0) {
  using X = XBuf<BF, K>;
  ld8(d, reinterpret_cast<const typename X::El*>(buf) + n * X::LD + k0);
}
template <bool BF, int K>
__device__ __forceinline__ void xb_read_split(typename Types<BF>::S& d, const uint8_t* buf, int n, int k0) {
  using X = XBuf<BF, K>;
  if constexpr (BF) {
    ld8(d.hi, reinterpret_cast<const uint16_t*>(buf) + n * X::LD + k0);
    ld8(d.lo, reinterpret_cast<const uint16_t*>(buf + X::PLANE) + n * X::LD + k0);
  } else {
    ld8(d, reinterpret_cast<const float*>(buf) + n * X::LD + k0);
  }
}
template <bool BF, int K>
constexpr size_t xb_bytes_split() {
  return (BF ? 2 : 1) * XBuf<BF, K>::PLANE;
}

// Workspace block of one (chunk, value head).  A fragments of 16 rows x 32
// columns of the lower-triangular C x C matrices T' and R: fragment (r, s),
// r = row block, s = 32-wide column slab, exists for s <= r / 2.  A fragment
// is one (single) or two (split / fp32) planes of 64 lanes x 16 bytes.
template <bool BF, int C>
struct Geom {
  static constexpr int NB = C / 16;  // 16-token row blocks
  static constexpr int NF = NB == 1 ? 1 : (NB == 2 ? 2 : 6);
  static constexpr int TPL = BF ? 1 : 2;  // planes of a T' fragment
  static constexpr size_t PLANE = 1024;
  static constexpr size_t T_OFF = 0;
  static constexpr size_t R_OFF = T_OFF + size_t(NF) * TPL * PLANE;
  static constexpr size_t SCAL_OFF = R_OFF + size_t(NF) * 2 * PLANE;
  static constexpr size_t BYTES = SCAL_OFF + 4 * C * sizeof(float);
  static_assert(BYTES % 256 == 0, "keep per-chunk blocks 256-byte aligned");
};
// Q of one (chunk, query/key head) laid out as the sweep's A fragments: for
// each 16-row block r and 32-column slab s, 64 lanes x 8 values (one 1 KiB
// plane in bf16, two in fp32), so that the sweep loads them as contiguous
// 1 KiB rows instead of 16 rows of 64 bytes a power-of-two stride apart.
__host__ __device__ constexpr size_t qfrag_bytes(int dk, int c, bool bf) {
  return size_t(c / 16) * size_t((dk < 32 ? 32 : dk) / 32) * (bf ? 1 : 2) * 1024;
}

// first fragment of row block r: sum over r' < r of (r' / 2 + 1)
__device__ __forceinline__ constexpr int frag_base(int r) { return r == 0 ? 0 : (r == 1 ? 1 : (r == 2 ? 2 : 4)); }
// row of the p-th block of a lower-triangular block matrix (blocks (r, i), i <= r, row-major)
__device__ __forceinline__ constexpr int tri_row(int p) { return p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3)); }

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS (and scalar)
// traffic only, so global loads and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// exp(x) by the hardware base-2 exponential; relative error about |x| 2^-24
// from rounding x log2(e), far inside what the decays need.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }


template <typename IO, int DK, int C>
struct PrepLds {
  static constexpr int E16 = 16 / sizeof(IO);
  static constexpr int NB = C / 16;
  static constexpr int CP = C < 32 ? 32 : C;     // token rows, padded to a 32 slab
  static constexpr int DKP = DK < 32 ? 32 : DK;  // key columns, padded to a 32 slab
  static constexpr int KP = DKP + E16;           // row stride, elements (16-byte pad)
  // A, QKm, T and R are lower block triangular: only their NBLK nonzero
  // 16 x 16 blocks are stored, block (r, i) at index r (r + 1) / 2 + i, rows
  // BP floats apart (BP = 20 keeps fragment reads and D-layout writes free
  // of bank conflicts).  All three share the K/Q tile space once the Gram
  // products are in registers; R later reuses A.
  static constexpr int NBLK = NB * (NB + 1) / 2;
  static constexpr int BP = 20;
  static constexpr size_t KQ_BYTES = 2 * size_t(CP) * KP * sizeof(IO);
  static constexpr size_t M_BYTES = size_t(NBLK) * 16 * BP * sizeof(float);
  static constexpr size_t U_BYTES = KQ_BYTES > 3 * M_BYTES ? KQ_BYTES : 3 * M_BYTES;
  static constexpr size_t A_OFF = 0, QK_OFF = M_BYTES, T_OFF = 2 * M_BYTES;
  static constexpr size_t GB_OFF = U_BYTES;           // fp64 prefix sum before each 16-token block
  static constexpr size_t GL_OFF = GB_OFF + 8 * 4;    // fp32 prefix sum within the token's block
  static constexpr size_t B_OFF = GL_OFF + C * sizeof(float);
  static constexpr size_t D_OFF = B_OFF + C * sizeof(float);
  static constexpr size_t BYTES = D_OFF + C * sizeof(float);
};

template <typename IO, int DK, int C>
struct SweepLds {
  static constexpr bool BF = sizeof(IO) == 2;
  static constexpr int ESZ = int(sizeof(IO));
  static constexpr int E16 = 16 / ESZ;
  static constexpr int CP = C < 32 ? 32 : C;     // token rows of the staged K tile
  static constexpr int DKP = DK < 32 ? 32 : DK;  // its columns
  static constexpr int KP = frag_row_stride(DKP * ESZ) / ESZ;  // row stride, elements
  static constexpr size_t KBUF = size_t(CP) * KP * ESZ;
  static constexpr size_t VBUF = size_t(C) * 16 * ESZ;                       // V slice: C tokens x 16 values
  static constexpr size_t TBUF = size_t(Geom<BF, C>::NF) * Geom<BF, C>::TPL * Geom<BF, C>::PLANE;  // T' fragments
  static constexpr size_t SCBUF = 4 * C * sizeof(float);                     // beta, beta gamma, gamma, dec
  // K, Q, V and T' have one buffer each: a chunk's copies are written after
  // the last read of the previous chunk's (the second barrier of a step).
  // The scalars are read until the end of a step and have two (chunk parity).
  static constexpr size_t K_OFF = 0;
  static constexpr size_t V_OFF = K_OFF + KBUF;
  static constexpr size_t T_OFF = V_OFF + VBUF;
  static constexpr size_t SC_OFF = T_OFF + TBUF;
  static constexpr size_t S_OFF = SC_OFF + 2 * SCBUF;  // state (B fragments of S^T)
  static constexpr size_t Y_OFF = S_OFF + XBuf<BF, DKP>::PLANE;
  static constexpr size_t UD_OFF = Y_OFF + xb_bytes_split<BF, CP>();
  static constexpr size_t BYTES = UD_OFF + xb_bytes_split<BF, CP>();
  static_assert(BYTES % 16 == 0, "zeroed in 16-byte pieces");
};

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Raw buffer resources (stride 0): a load whose bytes lie at or past `bytes`
// returns zeros and such a store is dropped, per dword.
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return uint4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void bload_op(uint4& d, Rsrc r, uint32_t off) { d = bload16(r, off); }
__device__ __forceinline__ void bload_op(f8& d, Rsrc r, uint32_t off) {
  const uint4 a = bload16(r, off), b = bload16(r, off + 16);
  d.a = f4{__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)};
  d.b = f4{__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
}
template <typename IO>
__device__ __forceinline__ IO bload_el(Rsrc r, uint32_t off) {
  if constexpr (sizeof(IO) == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <typename IO>
__device__ __forceinline__ void bstore_el(Rsrc r, uint32_t off, float x) {
  if constexpr (sizeof(IO) == 2) __builtin_amdgcn_raw_buffer_store_b16(f2bf(x), r, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
__device__ __forceinline__ float io_val(uint16_t x) { return bf2f(x); }
__device__ __forceinline__ float io_val(float x) { return x; }
// A split (bf16 hi + lo, two planes `plane` bytes apart) or fp32 operand from global memory.
__device__ __forceinline__ void ld_split(sp8& d, const uint8_t* p, int plane) {
  d.hi = *reinterpret_cast<const uint4*>(p);
  d.lo = *reinterpret_cast<const uint4*>(p + plane);
}
__device__ __forceinline__ void ld_split(f8& d, const uint8_t* p, int plane) {
  d.a = *reinterpret_cast<const f4*>(p);
  d.b = *reinterpret_cast<const f4*>(p + plane);
}

}  // namespace

// Slot table: tab[slot] = (first token, length) of the chunk in that slot,
// (0, 0) for slots no chunk uses.  Thread n % 256 fills the slots from
// sequence n's first slot up to the next sequence's first slot.
__device__ __forceinline__ int first_slot(int bos, int n, int C) { return (bos + n * (C - 1)) / C; }

__global__ __launch_bounds__(256) void chunk_table_kernel(int N, int T, int C, int max_chunks,
                                                          const int32_t* __restrict__ cu, int2* __restrict__ tab) {
  for (int n = threadIdx.x; n < N; n += 256) {
    int b, e;
    seq_range(cu, n, T, b, e);
    const int s0 = first_slot(b, n, C);
    const int s1 = min(first_slot(e, n + 1, C), max_chunks);
    int t = b;
    for (int sl = max(s0, 0); sl < s1; ++sl, t += C) tab[sl] = t < e ? make_int2(t, min(C, e - t)) : make_int2(0, 0);
  }
  int bN, eN;
  seq_range(cu, N - 1, T, bN, eN);
  for (int sl = max(first_slot(eN, N, C), 0) + int(threadIdx.x); sl < max_chunks; sl += 256) tab[sl] = make_int2(0, 0);
}

template <typename IO, int DK, int C>
__global__ __launch_bounds__(512) void chunk_prep_kernel(int h_qk, int h_v, const IO* __restrict__ q,
                                                         const IO* __restrict__ k, const float* __restrict__ g,
                                                         const float* __restrict__ beta, int num_seqs, int T,
                                                         const int2* __restrict__ tab, uint8_t* __restrict__ ws,
                                                         uint8_t* __restrict__ qf) {
  constexpr bool BF = sizeof(IO) == 2;
  using Geo = Geom<BF, C>;
  using Lds = PrepLds<IO, DK, C>;
  using E = typename Types<BF>::E;
  constexpr int NB = Geo::NB, E16 = Lds::E16, KP = Lds::KP, BP = Lds::BP;
  constexpr int NKS = Lds::DKP / 32;
  constexpr int NBLK = NB * (NB + 1) / 2;
  constexpr int NW = 8;                     // waves per workgroup
  constexpr int NGP = (NBLK + NW - 1) / NW;  // Gram blocks per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  IO* sK = reinterpret_cast<IO*>(smem);
  IO* sQ = sK + Lds::CP * KP;
  float* sA = reinterpret_cast<float*>(smem + Lds::A_OFF);   // after the Gram products
  float* sR = sA;                                            // after the inverse
  float* sQK = reinterpret_cast<float*>(smem + Lds::QK_OFF);
  float* sT = reinterpret_cast<float*>(smem + Lds::T_OFF);
  double* sGb = reinterpret_cast<double*>(smem + Lds::GB_OFF);
  float* sGl = reinterpret_cast<float*>(smem + Lds::GL_OFF);
  float* sBeta = reinterpret_cast<float*>(smem + Lds::B_OFF);
  float* sDec = reinterpret_cast<float*>(smem + Lds::D_OFF);

  const int gc = blockIdx.x, h = blockIdx.y;
  const int2 ch = num_seqs == 1 ? make_int2(gc * C, min(C, T - gc * C)) : tab[gc];
  const int t0 = ch.x, nc = ch.y;
  if (nc <= 0) return;
  const int j = h / (h_v / h_qk);
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = wave_id();
  // element (row, c), c <= row rounded to blocks, of a stored lower block-triangular matrix
  auto lt = [&](float* m, int row, int c) {
    const int rb = row >> 4, cb = c >> 4;
    return m + (rb * (rb + 1) / 2 + cb) * 16 * BP + (row & 15) * BP + (c & 15);
  };
  uint8_t* wsb = ws + (size_t(gc) * h_v + h) * Geo::BYTES;

  // K and Q rows of the chunk (rows >= nc and columns >= DK are zero)
  constexpr int PER_ROW = Lds::DKP / E16;
  for (int x = tid; x < Lds::CP * PER_ROW; x += 64 * NW) {
    const int r = x / PER_ROW, c16 = (x % PER_ROW) * E16;
    uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (r < nc && c16 < DK) {
      const size_t off = (size_t(t0 + r) * h_qk + j) * DK + c16;
      kv = *reinterpret_cast<const uint4*>(k + off);
      qv = *reinterpret_cast<const uint4*>(q + off);
    }
    *reinterpret_cast<uint4*>(sK + r * KP + c16) = kv;
    *reinterpret_cast<uint4*>(sQ + r * KP + c16) = qv;
  }
  // Gate prefix sums in fp64: G_t = sum_{i<=t} g_i.  Kept as the sum before
  // each 16-token block (fp64) plus the part within the block (fp32, small),
  // so that every decay exp(G_r - G_i) is formed from a short fp32 argument.
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
    const double gbase = __shfl(gl, max((lane & ~15) - 1, 0));  // sum before the token's block
    const double gb = lane >= 16 ? gbase : 0.0;
    if (lane < C) {
      const float gam = lane < nc ? fast_exp(float(gl)) : 0.f;
      const float dec = lane < nc ? fast_exp(float(glast - gl)) : 0.f;
      if ((lane & 15) == 0) sGb[lane >> 4] = gb;
      sGl[lane] = float(gl - gb);
      sBeta[lane] = bl;
      sDec[lane] = dec;
      float* sc = reinterpret_cast<float*>(wsb + Geo::SCAL_OFF);
      sc[lane] = bl;
      sc[C + lane] = bl * gam;
      sc[2 * C + lane] = gam;
      sc[3 * C + lane] = dec;
    }
  }
  lds_barrier();

  // Gram blocks (r, i), i <= r, dealt round-robin to the waves: each wave
  // computes K K^T (-> A) and Q K^T (-> QKm) of the same block, which share
  // the decays.  Products stay in registers until every wave is done with
  // the K and Q tiles.
  f4 gk[NGP], gq[NGP];
#pragma unroll
  for (int n = 0; n < NGP; ++n) {
    const int pb = wave + NW * n;
    gk[n] = zero4(), gq[n] = zero4();
    if (pb < NBLK) {
      const int r = tri_row(pb), i = pb - r * (r + 1) / 2;
      const IO* ksrc = sK + (16 * r + col) * KP + 8 * grp;
      const IO* qsrc = sQ + (16 * r + col) * KP + 8 * grp;
      const IO* bsrc = sK + (16 * i + col) * KP + 8 * grp;
      f4 k1 = zero4(), q1 = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        E ak, aq, b;
        ld8(ak, ksrc + 32 * s);
        ld8(aq, qsrc + 32 * s);
        ld8(b, bsrc + 32 * s);
        if (s & 1) {
          k1 = mma32(ak, b, k1);
          q1 = mma32(aq, b, q1);
        } else {
          gk[n] = mma32(ak, b, gk[n]);
          gq[n] = mma32(aq, b, gq[n]);
        }
      }
      gk[n] = gk[n] + k1;
      gq[n] = gq[n] + q1;
    }
  }
  // the first value head of each query/key group stores Q as fragments
  if (h % (h_v / h_qk) == 0) {
    constexpr int NQF = NB * NKS;
    uint8_t* qb = qf + (size_t(gc) * h_qk + j) * qfrag_bytes(DK, C, BF);
    for (int p = wave; p < NQF; p += NW) {
      const int rq = p / NKS, sq = p % NKS;
      const IO* src = sQ + (16 * rq + col) * KP + 32 * sq + 8 * grp;
      if constexpr (BF) {
        *reinterpret_cast<uint4*>(qb + size_t(p) * 1024 + lane * 16) = *reinterpret_cast<const uint4*>(src);
      } else {
        *reinterpret_cast<f4*>(qb + size_t(p) * 2048 + lane * 16) = *reinterpret_cast<const f4*>(src);
        *reinterpret_cast<f4*>(qb + size_t(p) * 2048 + 1024 + lane * 16) = *reinterpret_cast<const f4*>(src + 4);
      }
    }
  }
  lds_barrier();  // K and Q are dead; their space becomes A and QKm
#pragma unroll
  for (int n = 0; n < NGP; ++n) {
    const int pb = wave + NW * n;
    if (pb < NBLK) {
      const int r = tri_row(pb), i = pb - r * (r + 1) / 2;
      const float dblk = float(sGb[r] - sGb[i]);
      const f4 glr = *reinterpret_cast<const f4*>(sGl + 16 * r + 4 * grp);
      const f4 btr = *reinterpret_cast<const f4*>(sBeta + 16 * r + 4 * grp);
      const float glc = sGl[16 * i + col];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * r + 4 * grp + e, cl = 16 * i + col;
        const float dcy = fast_exp(cl <= row ? dblk + glr[e] - glc : 0.f);
        *lt(sA, row, cl) = cl < row ? btr[e] * dcy * gk[n][e] : 0.f;
        *lt(sQK, row, cl) = cl <= row ? dcy * gq[n][e] : 0.f;
      }
    }
  }
  lds_barrier();

  // Diagonal blocks: T_bb = (I + A_bb)^{-1}.  Lane 4c+s owns column c and the
  // rows congruent to s mod 4; each row is one quad reduction.
  if (wave < NB) {
    const int b = wave, c = lane >> 2, s = lane & 3;
    float a[16][4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int m = 0; m < 4; ++m) a[rr][m] = *lt(sA, 16 * b + rr, 16 * b + 4 * m + s);
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float part = a[rr][0] * t[0] + a[rr][1] * t[1] + a[rr][2] * t[2] + a[rr][3] * t[3];
      const float val = (rr == c ? 1.f : 0.f) - sum_lanes4(part);
      if (s == (rr & 3)) t[rr >> 2] = val;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) *lt(sT, 16 * b + 4 * m + s, 16 * b + c) = t[m];
  }
  lds_barrier();

  // Off-diagonal blocks in two rounds, T being block lower triangular:
  //   T(i, i-1) = -T(i, i) A(i, i-1) T(i-1, i-1)             (i odd)
  // then, with the 32 x 32 halves T1 (blocks 0-1) and T2 (blocks 2-3),
  //   X = -T2 A21 T1,  X(i, j) = -sum_{l=2}^{i} T(i, l) M(l, j),
  //   M(l, j) = sum_{k=j}^{1} A(l, k) T(k, j),
  // each X block by one wave with M in registers.
  auto tcol = [&](int kk, int jj) {  // B operand: block (kk, jj) of T, rows 4 grp .., column col
    f4 bt;
#pragma unroll
    for (int e = 0; e < 4; ++e) bt[e] = *lt(sT, 16 * kk + 4 * grp + e, 16 * jj + col);
    return bt;
  };
  auto arow = [&](float* m, int ii, int kk) {  // A operand: block (ii, kk), row col, columns 4 grp ..
    return *reinterpret_cast<const f4*>(lt(m, 16 * ii + col, 16 * kk + 4 * grp));
  };
  if (NB >= 2 && wave < NB / 2) {
    const int i = 2 * wave + 1;
    const f4 P = mma_f32(arow(sA, i, i - 1), tcol(i - 1, i - 1), zero4());
    const f4 Rr = mma_f32(arow(sT, i, i), P, zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) *lt(sT, 16 * i + 4 * grp + e, 16 * (i - 1) + col) = -Rr[e];
  }
  lds_barrier();
  if (NB == 4 && wave < 4) {
    const int i = 2 + (wave >> 1), jj = wave & 1;
    auto mlj = [&](int l) {
      f4 m = mma_f32(arow(sA, l, 1), tcol(1, jj), zero4());
      if (jj == 0) m = mma_f32(arow(sA, l, 0), tcol(0, 0), m);
      return m;
    };
    f4 X = mma_f32(arow(sT, i, 2), mlj(2), zero4());
    if (i == 3) X = mma_f32(arow(sT, 3, 3), mlj(3), X);
#pragma unroll
    for (int e = 0; e < 4; ++e) *lt(sT, 16 * i + 4 * grp + e, 16 * jj + col) = -X[e];
  }
  if (NB == 4) lds_barrier();

  // R = QKm T, lower-triangular blocks R(r, i) = sum_{k=i}^{r} QKm(r, k) T(k, i), in fp32.
  for (int p = wave; p < NBLK; p += NW) {
    int r = 0;
    while ((r + 1) * (r + 2) / 2 <= p) ++r;
    const int i = p - r * (r + 1) / 2;
    f4 acc = zero4();
    for (int kk = i; kk <= r; ++kk) {
      acc = mma_f32(arow(sQK, r, kk), tcol(kk, i), acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) *lt(sR, 16 * r + 4 * grp + e, 16 * i + col) = acc[e];
  }
  lds_barrier();

  // Fragments (r, s), s <= r / 2, of T' = diag(dec) T and R, lower-triangular
  // (entries above the diagonal and beyond C are zero).
  for (int p = wave; p < Geo::NF; p += NW) {
    int r = 0;
    while (r + 1 < NB && frag_base(r + 1) <= p) ++r;
    const int s = p - frag_base(r);
    const int row = 16 * r + col, k0 = 32 * s + 8 * grp;
    f8 tv, rv;
    zero(tv), zero(rv);
    if (k0 < C && (k0 >> 4) <= r) {  // blocks above the diagonal are zero and not stored
      tv.a = *reinterpret_cast<const f4*>(lt(sT, row, k0));
      tv.b = *reinterpret_cast<const f4*>(lt(sT, row, k0 + 4));
      rv.a = *reinterpret_cast<const f4*>(lt(sR, row, k0));
      rv.b = *reinterpret_cast<const f4*>(lt(sR, row, k0 + 4));
    }
    const float dr = sDec[row];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ka = k0 + e <= row, kb = k0 + 4 + e <= row;
      tv.a[e] = ka ? dr * tv.a[e] : 0.f;
      tv.b[e] = kb ? dr * tv.b[e] : 0.f;
      rv.a[e] = ka ? rv.a[e] : 0.f;
      rv.b[e] = kb ? rv.b[e] : 0.f;
    }
    uint8_t* tp = wsb + Geo::T_OFF + size_t(p) * Geo::TPL * Geo::PLANE + lane * 16;
    uint8_t* rp = wsb + Geo::R_OFF + size_t(p) * 2 * Geo::PLANE + lane * 16;
    if constexpr (BF) {
      uint4 th, tl, rh, rl;
      split_bf16x8(tv, th, tl);
      split_bf16x8(rv, rh, rl);
      *reinterpret_cast<uint4*>(tp) = th;
      *reinterpret_cast<uint4*>(rp) = rh;
      *reinterpret_cast<uint4*>(rp + Geo::PLANE) = rl;
    } else {
      *reinterpret_cast<f4*>(tp) = tv.a;
      *reinterpret_cast<f4*>(tp + Geo::PLANE) = tv.b;
      *reinterpret_cast<f4*>(rp) = rv.a;
      *reinterpret_cast<f4*>(rp + Geo::PLANE) = rv.b;
    }
  }
}

template <typename IO, int DK, int C>
__global__ __launch_bounds__(512) void chunk_sweep_kernel(int N, int T, int h_qk, int h_v, int d_v, int max_chunks,
                                                          const IO* __restrict__ q, const IO* __restrict__ k,
                                                          const IO* __restrict__ v, const int32_t* __restrict__ cu,
                                                          const uint8_t* __restrict__ ws, const uint8_t* __restrict__ qf,
                                                          const float* s_in, IO* __restrict__ out, float* s_out) {
  constexpr bool BF = sizeof(IO) == 2;
  using Geo = Geom<BF, C>;
  using Lds = SweepLds<IO, DK, C>;
  using E = typename Types<BF>::E;
  using Sp = typename Types<BF>::S;
  constexpr int NB = Geo::NB, KB = DK / 16, CP = Lds::CP, DKP = Lds::DKP, KP = Lds::KP, E16 = Lds::E16;
  constexpr int ESZ = Lds::ESZ;
  constexpr int NKS = DKP / 32, NTS = CP / 32;  // 32-wide slabs along d_k and along the chunk
  constexpr int SB = (KB + 3) / 4;              // state blocks per chain wave
  constexpr int NTF = (NB + 1) / 2;             // T' / R fragments per row block, at most
  constexpr int PER_ROW = DK / E16;             // 16-byte pieces per K row
  constexpr int NKP = (C * PER_ROW + 255) / 256;                                 // K pieces per helper lane
  constexpr int NVP = int(Lds::VBUF / 16), NTP = int(Lds::TBUF / 16), NSP = int(Lds::SCBUF / 16);
  constexpr int NVT = (NVP + NTP + NSP + 255) / 256;                             // other pieces per helper lane
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sS = smem + Lds::S_OFF;
  uint8_t* sY = smem + Lds::Y_OFF;
  uint8_t* sUd = smem + Lds::UD_OFF;

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
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = wave_id();
  const int r = wave & 3;                    // row block (and state-block group) of this wave
  const bool rowblk = NB >= 4 || r < NB;

  int bos, eos;
  seq_range(cu, n, T, bos, eos);
  int nchunk = (eos - bos + C - 1) / C;
  const int gc0 = first_slot(bos, n, C);
  nchunk = max(0, min(nchunk, max_chunks - gc0));  // malformed offsets cannot run past the workspace
  const int kstride = h_qk * DK;  // elements between consecutive tokens of q / k
  const int vstride = h_v * d_v;  // and of v
  auto chunk_t0 = [&](int cc) { return bos + cc * C; };
  auto chunk_nc = [&](int cc) { return min(C, eos - chunk_t0(cc)); };

  // zero LDS once: K rows / columns past C or d_k, and exchange columns past
  // C or d_k, are read as zeros
  for (int x = tid; x < int(Lds::BYTES / 16); x += 512) reinterpret_cast<uint4*>(smem)[x] = uint4{0u, 0u, 0u, 0u};
  lds_barrier();

  if (wave < 4) {
    // ============================================================ chain waves
    // The recurrence proper: per chunk X = K S^T, Y, T'Y and the state
    // update, touching only LDS and the matrix cores.
    f4 st[SB];
#pragma unroll
    for (int bi = 0; bi < SB; ++bi) {
      const int b = r + 4 * bi;
      st[bi] = zero4();
      if (b < KB) {
        if (s_in) st[bi] = *reinterpret_cast<const f4*>(s_in + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp);
        xb_write_single<BF, DKP>(sS, col, 16 * b + 4 * grp, st[bi]);
      }
    }
    lds_barrier();  // chunk 0 staged, state written

    const int arow = col * KP + 8 * grp;                       // A fragment rows of the K tile
    const int tcol = 8 * grp * KP + col;                       // K^T fragment, element reads
    const int trow = (8 * grp + col / 4) * KP + 4 * (col % 4);  // K^T fragment, transpose reads
    for (int cc = 0; cc < nchunk; ++cc) {
      const int buf = cc & 1, nc = chunk_nc(cc);
      const IO* sK = reinterpret_cast<const IO*>(smem + Lds::K_OFF);
      const IO* sV = reinterpret_cast<const IO*>(smem + Lds::V_OFF);
      const uint8_t* sTp = smem + Lds::T_OFF;
      const float* sSc = reinterpret_cast<const float*>(smem + Lds::SC_OFF + buf * Lds::SCBUF);

      // (1) X = K S^T for token block r; Y = beta V - beta gamma X
      if (rowblk) {
        f4 x = zero4(), x1 = zero4();
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          E ak, bs;
          ld8(ak, sK + 16 * r * KP + arow + 32 * s);
          xb_read_single<BF, DKP>(bs, sS, col, 32 * s + 8 * grp);
          if (s & 1) x1 = mma32(ak, bs, x1);
          else x = mma32(ak, bs, x);
        }
        x = x + x1;
        float vv[4];
        if constexpr (BF) {
          // rows 16 r + 4 grp .. + 3 of column col by one transpose read
          const uint2 t = lds_tr16(sV + (16 * r + 4 * grp + col / 4) * 16 + 4 * (col % 4));
          vv[0] = __uint_as_float(t.x << 16), vv[1] = __uint_as_float(t.x & 0xffff0000u);
          vv[2] = __uint_as_float(t.y << 16), vv[3] = __uint_as_float(t.y & 0xffff0000u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = sV[(16 * r + 4 * grp + e) * 16 + col];
        }
        f4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = 16 * r + 4 * grp + e;
          const float b = sSc[tok], bg = sSc[C + tok];
          y[e] = tok < nc ? b * vv[e] - bg * x[e] : 0.f;
        }
        xb_write_split<BF, CP>(sY, col, 16 * r + 4 * grp, y);
      }
      lds_barrier();

      // (2) Ud = T' Y for token block r; K^T fragments for (3)
      if (rowblk) {
        const uint8_t* tf = sTp + size_t(frag_base(r)) * Geo::TPL * Geo::PLANE + lane * 16;
        f4 uh = zero4(), ul = zero4();
#pragma unroll
        for (int s = 0; s < NTF; ++s) {
          if (2 * s <= r) {
            Sp yb;
            E tv;
            xb_read_split<BF, CP>(yb, sY, col, 32 * s + 8 * grp);
            if constexpr (BF) {
              tv = *reinterpret_cast<const uint4*>(tf + s * Geo::PLANE);
            } else {
              tv.a = *reinterpret_cast<const f4*>(tf + s * 2 * Geo::PLANE);
              tv.b = *reinterpret_cast<const f4*>(tf + s * 2 * Geo::PLANE + Geo::PLANE);
            }
            mm_es(tv, yb, uh, ul);
          }
        }
        xb_write_split<BF, CP>(sUd, col, 16 * r + 4 * grp, uh + ul);
      }
      E kt[SB][NTS];
#pragma unroll
      for (int bi = 0; bi < SB; ++bi) {
        const int b = r + 4 * bi;
        if (b < KB) {
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            if constexpr (BF) {
              const uint2 lo = lds_tr16(sK + 32 * s * KP + trow + 16 * b);
              const uint2 hi = lds_tr16(sK + 32 * s * KP + 4 * KP + trow + 16 * b);
              kt[bi][s] = uint4{lo.x, lo.y, hi.x, hi.y};
            } else {
              ld8col(kt[bi][s], sK + 32 * s * KP + tcol + 16 * b, KP);
            }
          }
        }
      }
      lds_barrier();

      // (3) S^T <- gamma_last S^T + K^T Ud for the owned state blocks
      const float glast = sSc[2 * C + nc - 1];
#pragma unroll
      for (int bi = 0; bi < SB; ++bi) {
        const int b = r + 4 * bi;
        if (b < KB) {
          f4 ah = st[bi] * glast, al = zero4();
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            Sp ub;
            xb_read_split<BF, CP>(ub, sUd, col, 32 * s + 8 * grp);
            mm_es(kt[bi][s], ub, ah, al);
          }
          st[bi] = ah + al;
          xb_write_single<BF, DKP>(sS, col, 16 * b + 4 * grp, st[bi]);
        }
      }
      lds_barrier();
    }

#pragma unroll
    for (int bi = 0; bi < SB; ++bi) {
      const int b = r + 4 * bi;
      if (b < KB) *reinterpret_cast<f4*>(s_out + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp) = st[bi];
    }
  } else {
    // ============================================================ helper waves
    // Everything off the recurrence: fetch chunk c+1 while chunk c runs and
    // stage it in the other LDS buffers, and compute and store the output
    // O = gamma (Q S^T) + R Y of token block r.
    const int ht = tid - 256;  // 0..255
    // per-lane byte offsets relative to a chunk's first token row
    uint32_t koff[NKP];
#pragma unroll
    for (int it = 0; it < NKP; ++it) {
      const int x = ht + 256 * it;
      koff[it] = x < C * PER_ROW ? uint32_t(((x / PER_ROW) * kstride + (x % PER_ROW) * E16) * ESZ) : 0x80000000u;
    }
    uint32_t ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ooff[e] = uint32_t(((16 * r + 4 * grp + e) * vstride + col) * ESZ);
    const uint32_t kq_tail = uint32_t(DK * ESZ), v_tail = uint32_t(16 * ESZ);

    // Staged inputs (K tile, V slice, T' fragments, scalars) are fetched two
    // chunks ahead into registers and written to LDS one chunk ahead, so the
    // loads have a whole chunk to land; the Q and R fragments of the next
    // chunk stay in registers.  Loads are spread over the three windows so
    // that no window waits behind a full memory queue.
    struct Staged {
      uint4 kp[NKP];  // K rows, 16-byte pieces
      uint4 vt[NVT];  // V slice, T' fragments and scalars, 16-byte pieces
    };
    struct Frags {
      E aq[NKS];   // Q rows of block r (A fragments, stored in that order by the prep kernel)
      Sp rf[NTF];  // R fragments of block r
    };
    auto fetch_k = [&](Staged& P, int cc) {
      const int t0 = chunk_t0(cc), nc = chunk_nc(cc);
      const Rsrc rk = make_rsrc(k + (size_t(t0) * h_qk + j) * DK, uint32_t((nc - 1) * kstride * ESZ) + kq_tail);
#pragma unroll
      for (int it = 0; it < NKP; ++it) P.kp[it] = bload16(rk, koff[it]);
    };
    auto fetch_vt = [&](Staged& P, int cc) {
      // one plain load per piece, its address chosen per lane: V rows past
      // the chunk's end are clamped to its last row (those tokens are masked
      // where V is used)
      const int t0 = chunk_t0(cc), nc = chunk_nc(cc);
      const IO* vb = v + (size_t(t0) * h_v + h) * d_v + dv0;
      const uint8_t* wsb = ws + (size_t(gc0 + cc) * h_v + h) * Geo::BYTES;
      constexpr int PPT = 16 / E16;  // pieces per token row of the V slice
#pragma unroll
      for (int it = 0; it < NVT; ++it) {
        const int x = min(ht + 256 * it, NVP + NTP + NSP - 1);
        const int tok = min(x / PPT, nc - 1);
        const uint8_t* src = x < NVP ? reinterpret_cast<const uint8_t*>(vb + tok * vstride + (x % PPT) * E16)
                           : x < NVP + NTP ? wsb + Geo::T_OFF + size_t(x - NVP) * 16
                                           : wsb + Geo::SCAL_OFF + size_t(x - NVP - NTP) * 16;
        P.vt[it] = *reinterpret_cast<const uint4*>(src);
      }
    };
    auto fetch_qfrags = [&](Frags& F, int cc) {
      const int rb = rowblk ? r : 0;
      const uint8_t* qp = qf + (size_t(gc0 + cc) * h_qk + j) * qfrag_bytes(DK, C, BF) + lane * 16;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        if constexpr (BF) {
          F.aq[s] = *reinterpret_cast<const uint4*>(qp + size_t(rb * NKS + s) * 1024);
        } else {
          F.aq[s].a = *reinterpret_cast<const f4*>(qp + size_t(rb * NKS + s) * 2048);
          F.aq[s].b = *reinterpret_cast<const f4*>(qp + size_t(rb * NKS + s) * 2048 + 1024);
        }
      }
    };
    auto fetch_rfrags = [&](Frags& F, int cc) {
      // every helper wave issues the same loads (a lane whose fragment is not
      // needed reads one shared line instead)
      const int rb = rowblk ? r : 0;
      const uint8_t* rp = ws + (size_t(gc0 + cc) * h_v + h) * Geo::BYTES + Geo::R_OFF +
                          size_t(frag_base(rb)) * 2 * Geo::PLANE;
#pragma unroll
      for (int s = 0; s < NTF; ++s) {
        const bool need = rowblk && 2 * s <= r;
        ld_split(F.rf[s], rp + (need ? s * 2 * Geo::PLANE + lane * 16 : 0), need ? Geo::PLANE : 0);
      }
    };
    auto commit = [&](const Staged& P, int buf) {
      IO* sK = reinterpret_cast<IO*>(smem + Lds::K_OFF);
#pragma unroll
      for (int it = 0; it < NKP; ++it) {
        const int x = ht + 256 * it;
        if (x < C * PER_ROW) *reinterpret_cast<uint4*>(sK + (x / PER_ROW) * KP + (x % PER_ROW) * E16) = P.kp[it];
      }
#pragma unroll
      for (int it = 0; it < NVT; ++it) {
        const int x = ht + 256 * it;
        uint8_t* dst = x < NVP ? smem + Lds::V_OFF + size_t(x) * 16
                     : x < NVP + NTP ? smem + Lds::T_OFF + size_t(x - NVP) * 16
                                     : smem + Lds::SC_OFF + buf * Lds::SCBUF + size_t(x - NVP - NTP) * 16;
        if (x < NVP + NTP + NSP) *reinterpret_cast<uint4*>(dst) = P.vt[it];
      }
    };

    // S_c = staged inputs of chunk c (in registers until committed), F = Q / R fragments
    Staged SA, SB;
    Frags F, Fn;
    if (nchunk > 0) {
      fetch_k(SA, 0);
      fetch_vt(SA, 0);
      fetch_qfrags(F, 0);
      fetch_rfrags(F, 0);
      fetch_k(SB, min(1, nchunk - 1));
      fetch_vt(SB, min(1, nchunk - 1));
      commit(SA, 0);
    }
    lds_barrier();  // chunk 0 staged, state written

    auto step = [&](int cc, Staged& next, Staged& after) {
      // next = chunk cc+1 (loaded, not yet committed); after = free, receives chunk cc+2
      const int buf = cc & 1, nc = chunk_nc(cc);
      const float* sSc = reinterpret_cast<const float*>(smem + Lds::SC_OFF + buf * Lds::SCBUF);

      // (1) Z = Q S^T of block r (S is the chunk's initial state); K, V, T'
      // and scalars of chunk cc+2, Q fragments of chunk cc+1
      f4 z = zero4();
      if (rowblk) {
        f4 z1 = zero4();
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          E bs;
          xb_read_single<BF, DKP>(bs, sS, col, 32 * s + 8 * grp);
          if (s & 1) z1 = mma32(F.aq[s], bs, z1);
          else z = mma32(F.aq[s], bs, z);
        }
        z = z + z1;
      }
      const int c2 = min(cc + 2, nchunk - 1), c1 = min(cc + 1, nchunk - 1);  // past the end: harmless refetch
      fetch_k(after, c2);
      fetch_vt(after, c2);
      fetch_qfrags(Fn, c1);
      lds_barrier();

      // (2) O = gamma Z + R Y for block r, stored straight from the D layout
      if (rowblk) {
        f4 oh, ol = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) oh[e] = sSc[2 * C + 16 * r + 4 * grp + e] * z[e];
#pragma unroll
        for (int s = 0; s < NTF; ++s) {
          if (2 * s <= r) {
            Sp yb;
            xb_read_split<BF, CP>(yb, sY, col, 32 * s + 8 * grp);
            mm_ss(F.rf[s], yb, oh, ol);
          }
        }
        const f4 o = oh + ol;
        const int t0 = chunk_t0(cc);
        const Rsrc ro = make_rsrc(out + (size_t(t0) * h_v + h) * d_v + dv0, uint32_t((nc - 1) * vstride * ESZ) + v_tail);
#pragma unroll
        for (int e = 0; e < 4; ++e) bstore_el<IO>(ro, ooff[e], o[e]);
      }
      lds_barrier();

      // (3) R fragments of chunk cc+1; stage chunk cc+1 in the LDS buffers
      fetch_rfrags(Fn, c1);
      commit(next, buf ^ 1);  // after the last chunk this fills buffers nobody reads
      F = Fn;
      lds_barrier();
    };
    for (int cc = 0; cc < nchunk; cc += 2) {
      step(cc, SB, SA);
      if (cc + 1 < nchunk) step(cc + 1, SA, SB);
    }
  }
}

// ---------------------------------------------------------------- host side

size_t chunked_max_chunks(const Dims& d, int chunk) {
  // sum_n ceil(L_n / C) <= (T + N (C - 1)) / C
  return (size_t(d.total_tokens) + size_t(d.num_seqs) * size_t(chunk - 1)) / size_t(chunk);
}

static size_t chunk_bytes(bool bf16, int chunk) {
  switch (chunk) {
    case 16: return bf16 ? Geom<true, 16>::BYTES : Geom<false, 16>::BYTES;
    case 32: return bf16 ? Geom<true, 32>::BYTES : Geom<false, 32>::BYTES;
    case 64: return bf16 ? Geom<true, 64>::BYTES : Geom<false, 64>::BYTES;
  }
  return 0;
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }
static size_t table_bytes(const Dims& d, int chunk) { return round256(chunked_max_chunks(d, chunk) * 8); }

static size_t blocks_bytes(const Dims& d, int chunk) {
  return chunked_max_chunks(d, chunk) * size_t(d.h_v) * chunk_bytes(d.bf16, chunk);
}

size_t chunked_workspace_bytes(const Dims& d, int chunk) {
  if (chunk_bytes(d.bf16, chunk) == 0) return 0;
  return table_bytes(d, chunk) + blocks_bytes(d, chunk) +
         chunked_max_chunks(d, chunk) * size_t(d.h_qk) * qfrag_bytes(d.d_k, chunk, d.bf16);
}

template <typename IO, int DK, int C>
static hipError_t launch_chunked_t(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const int32_t* cu, const float* s_in, void* out,
                                   float* s_out, void* workspace, hipStream_t st) {
  uint8_t* base = static_cast<uint8_t*>(workspace);
  int2* tab = reinterpret_cast<int2*>(base);
  uint8_t* ws = base + table_bytes(d, C);
  uint8_t* qf = ws + blocks_bytes(d, C);
  const size_t max_chunks = chunked_max_chunks(d, C);
  hipError_t e = hipSuccess;
  if (d.num_seqs > 1) {
    Prof prof("chunk_table", st);
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, st, d.num_seqs, d.total_tokens, C,
                       int(max_chunks), cu, tab);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (max_chunks > 0) {
    constexpr size_t lds = PrepLds<IO, DK, C>::BYTES;
    if (lds > 65536) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prep_kernel<IO, DK, C>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
    Prof prof("chunk_prep", st);
    hipLaunchKernelGGL((chunk_prep_kernel<IO, DK, C>), dim3(unsigned(max_chunks), unsigned(d.h_v)), dim3(512), lds,
                       st, d.h_qk, d.h_v, static_cast<const IO*>(q), static_cast<const IO*>(k), g, beta, d.num_seqs,
                       d.total_tokens, tab, ws, qf);
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
  hipLaunchKernelGGL((chunk_sweep_kernel<IO, DK, C>), dim3(8 * per), dim3(512), lds, st, d.num_seqs,
                     d.total_tokens, d.h_qk, d.h_v, d.d_v, int(max_chunks), static_cast<const IO*>(q),
                     static_cast<const IO*>(k), static_cast<const IO*>(v), cu, ws, qf, s_in,
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
