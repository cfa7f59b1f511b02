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
//   O   = diag(gamma) (Q S0^T) + R Y,          R = QKm T
//   S1^T = gamma_{n-1} S0^T + P Y,              P = K^T diag(dec) T
//
// (T Y is the block's matrix of delta updates; folding T into R and P, which
// do not depend on the state, leaves two block products between one state
// and the next: Y from S0, then S1 from Y.)  Decays are always formed as exp
// of a non-positive difference of fp64 partial sums, so nothing overflows and
// nothing but true decay underflows.
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
//   2. chunk_prep_kernel, one workgroup per (chunk, value head) (each XCD a
//      contiguous range of them, so value heads sharing K and Q meet in its
//      L2), fully
//      parallel: Gram products on MFMA, gate prefix sums, A, T = (I + A)^{-1}
//      (16x16 diagonal blocks by forward substitution in registers,
//      off-diagonal blocks by fp32 MFMA block products), R = QKm T, P, and the
//      per-token scalars, written to the workspace as MFMA A fragments; the
//      first value head of each query/key group also writes Q and K as
//      fragments.
//   3. chunk_sweep_kernel, one workgroup per (sequence, value head, 16 rows of
//      the state): walks the chunks in order with its 16 x d_k slice of the
//      fp32 state in MFMA accumulators.  State rows are independent given the
//      block's P, so slices of one head never talk to each other.  Four
//      waves run the recurrence (Y, then the state update); four others form
//      the output and stage inputs ahead.
//
// All block products use 16x16x32 fragments (see gdn_common.hpp).  Precision:
// bf16 inputs (K, Q, V) enter MFMA exactly.  Y, R and the state (in K S^T and
// Q S^T) are split into hi + lo bf16 halves, as is diag(dec) T when P is
// formed; with gates near 1, Q S^T carries most of an output, so the state
// rounded once would put its bf16 error there undamped.  P enters rounded once:
// its error enters each chunk's state update (about 1e-3 relative on the final
// state).  Every product accumulates in fp32.  fp32 inputs use fp32 MFMA
// throughout.
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
__device__ __forceinline__ void mm_se(const sp8& a, uint4 b, f4& ch, f4& cl) {
  ch = mma32(a.hi, b, ch);
  cl = mma32(a.lo, b, cl);
}
__device__ __forceinline__ void mm_se(const f8& a, const f8& b, f4& ch, f4&) { ch = mma32(a, b, ch); }
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

__device__ __forceinline__ void zero(f8& x) { x.a = zero4(), x.b = zero4(); }

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

// 8 fp32 elements of a column (stride apart) as an operand.
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
// k per lane).  bf16 buffers hold the hi and lo halves in two planes; fp32
// buffers hold the value.
template <bool BF, int K>
struct XBuf {
  using El = std::conditional_t<BF, uint16_t, float>;
  static constexpr int LD = frag_row_stride(K * int(sizeof(El))) / int(sizeof(El));  // row stride, elements
  static constexpr size_t PLANE = 16 * LD * sizeof(El);
};

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

// Fragment counts.  An operand fragment covers 16 rows x 32 columns: 64
// lanes x 8 values, stored as one 1 KiB plane per 8 bf16 (a bf16 value rounded
// once) or two planes (hi + lo bf16 halves of a split value, or fp32).
__host__ __device__ constexpr int dk_pad(int dk) { return dk < 32 ? 32 : dk; }
__host__ __device__ constexpr int c_pad(int c) { return c < 32 ? 32 : c; }
// fragments (r, s), s <= r / 2, of a lower-triangular C x C matrix
__host__ __device__ constexpr int tri_frags(int c) { return c == 16 ? 1 : (c == 32 ? 2 : 6); }
// Workspace block of one (chunk, value head): P = K^T diag(dec) T as d_k / 16
// row blocks x 32-token slabs (rounded once), R = QKm T as its
// lower-triangular fragments (split), then beta, beta gamma and gamma per
// token.
__host__ __device__ constexpr size_t p_off(bool, int, int) { return 0; }
__host__ __device__ constexpr size_t r_off(bool bf, int dk, int c) {
  return size_t(dk / 16) * (c_pad(c) / 32) * (bf ? 1 : 2) * 1024;
}
__host__ __device__ constexpr size_t scal_off(bool bf, int dk, int c) { return r_off(bf, dk, c) + size_t(tri_frags(c)) * 2 * 1024; }
__host__ __device__ constexpr size_t chunk_block_bytes(bool bf, int dk, int c) {
  return (scal_off(bf, dk, c) + 3 * size_t(c) * sizeof(float) + 255) / 256 * 256;
}
// Block of one (chunk, query/key head): Q, then K, as A fragments (C / 16 row
// blocks x d_k / 32 slabs), so that the sweep loads them as contiguous 1 KiB
// rows.
__host__ __device__ constexpr size_t k_frap_off(int dk, int c, bool bf) {
  return size_t(c / 16) * (dk_pad(dk) / 32) * (bf ? 1 : 2) * 1024;
}
__host__ __device__ constexpr size_t qk_frag_bytes(int dk, int c, bool bf) { return 2 * k_frap_off(dk, c, bf); }
template <bool BF, int DK, int C>
struct Geom {
  static constexpr int NB = C / 16;  // 16-token row blocks
  static constexpr int NF = tri_frags(C);
  static constexpr int TPL = BF ? 1 : 2;  // planes of a rounded-once fragment
  static constexpr size_t PLANE = 1024;
  static constexpr size_t P_OFF = p_off(BF, DK, C);
  static constexpr size_t R_OFF = r_off(BF, DK, C);
  static constexpr size_t SCAL_OFF = scal_off(BF, DK, C);
  static constexpr size_t BYTES = chunk_block_bytes(BF, DK, C);
  static_assert(SCAL_OFF % 256 == 0 && BYTES % 256 == 0, "keep per-chunk blocks 256-byte aligned");
};

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

// fp64 lane data movement on the two 32-bit halves: a DPP move (lanes the
// pattern leaves without a source, or rows outside ROWMASK, read 0) and a
// read of one lane.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, ROWMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, ROWMASK, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l), __builtin_amdgcn_readlane(__double2loint(x), l));
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within rows
// of 16 lanes, then the last lane of row 0 (of row 2) is added to row 1 (row
// 3), then the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ double wave_prefix_sum(double x) {
  x += dpp_f64<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31
  return x;
}


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
  // After R, T' = diag(dec) T is kept as the split B fragments of P's
  // products (2 KiB each, as many as R has fragments): in QKm's space when it
  // fits, else after T.
  static constexpr size_t TF_BYTES = size_t(tri_frags(C)) * 2048;
  static constexpr bool TF_IN_QK = TF_BYTES <= M_BYTES;
  static constexpr size_t U_MIN = 3 * M_BYTES + (TF_IN_QK ? 0 : TF_BYTES);
  static constexpr size_t U_BYTES = KQ_BYTES > U_MIN ? KQ_BYTES : U_MIN;
  static constexpr size_t A_OFF = 0, QK_OFF = M_BYTES, T_OFF = 2 * M_BYTES;
  static constexpr size_t TF_OFF = TF_IN_QK ? QK_OFF : 3 * M_BYTES;
  static constexpr size_t GB_OFF = U_BYTES;           // fp64 prefix sum before each 16-token block
  static constexpr size_t GL_OFF = GB_OFF + 8 * 4;    // fp32 prefix sum within the token's block
  static constexpr size_t B_OFF = GL_OFF + C * sizeof(float);   // beta
  static constexpr size_t D_OFF = B_OFF + C * sizeof(float);    // dec
  static constexpr size_t BYTES = D_OFF + C * sizeof(float);
  // at the end the whole region [0, U_BYTES) holds P^T in K's layout
  static_assert(KQ_BYTES / 2 <= U_BYTES, "P tile fits the union");
};

template <typename IO, int DK, int C>
struct SweepLds {
  static constexpr bool BF = sizeof(IO) == 2;
  static constexpr int ESZ = int(sizeof(IO));
  static constexpr int E16 = 16 / ESZ;
  static constexpr int CP = c_pad(C);    // token rows of the exchange buffer
  static constexpr int DKP = dk_pad(DK);  // key columns of the state buffer
  static constexpr size_t VBUF = size_t(C) * 16 * ESZ;    // V slice: C tokens x 16 values
  static constexpr size_t SCBUF = 3 * C * sizeof(float);  // beta, beta gamma, gamma
  // S (B fragments of S^T, split: hi and lo planes) and Y have one buffer each.  The V slice and the
  // scalars are written two chunks ahead: V has two buffers (chunk parity),
  // the scalars, read until the end of a step, four.
  static constexpr size_t S_OFF = 0;
  static constexpr size_t Y_OFF = S_OFF + xb_bytes_split<BF, DKP>();
  static constexpr size_t V_OFF = Y_OFF + xb_bytes_split<BF, CP>();
  static constexpr size_t SC_OFF = V_OFF + 2 * VBUF;
  static constexpr size_t BYTES = SC_OFF + 4 * SCBUF;
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
// Four consecutive values of one row (8 bytes in bf16, 16 in fp32).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <typename IO>
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t off, f4 x) {
  if constexpr (sizeof(IO) == 2) {
    const uint2 v = bf16x4(x);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, r, off, 0, 0);
  }
}
// 16 bytes of a per-chunk operand into the workspace, written through the
// XCD's L2 (agent scope: cache-policy bit 4, sc1, on this chip).  Only the
// next kernel reads them, so held dirty in L2 they would take space from the
// prep's own loads and wait there to be written back; written through, they
// still reach the sweep as fast as before (non-temporal stores, by contrast,
// send its reads to HBM).  Measured at 4096 tokens: prep 31.0 -> 28.9 us,
// the sweep unchanged.
constexpr int kStoreThroughL2 = 16;
__device__ __forceinline__ void ws_store16(Rsrc r, uint32_t off, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, kStoreThroughL2);
}
__device__ __forceinline__ u32x4 bits(uint4 x) { return u32x4{x.x, x.y, x.z, x.w}; }
__device__ __forceinline__ u32x4 bits(f4 x) {
  return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
}
// A split (bf16 hi + lo, two planes `plane` bytes apart) or fp32 operand from global memory.
__device__ __forceinline__ void ld_split(sp8& d, const uint8_t* p, int plane) {
  d.hi = *reinterpret_cast<const uint4*>(p);
  d.lo = *reinterpret_cast<const uint4*>(p + plane);
}
__device__ __forceinline__ void ld_split(f8& d, const uint8_t* p, int plane) {
  d.a = *reinterpret_cast<const f4*>(p);
  d.b = *reinterpret_cast<const f4*>(p + plane);
}
// A rounded-once (bf16: one plane) or fp32 (two planes) operand from global memory.
__device__ __forceinline__ void ld_e(uint4& d, const uint8_t* p, int) { d = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void ld_e(f8& d, const uint8_t* p, int plane) { ld_split(d, p, plane); }

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

// One prep item p = chunk slot * h_v + value head, by the 512 lanes of a
// workgroup whose LDS is `smem`.
template <typename IO, int DK, int C>
__device__ __forceinline__ void prep_item(int h_qk, int h_v, const IO* __restrict__ q, const IO* __restrict__ k,
                                          const float* __restrict__ g, const float* __restrict__ beta, int num_seqs,
                                          int T, int num_items, const int2* __restrict__ tab, uint8_t* __restrict__ ws,
                                          uint8_t* __restrict__ qf, const int p, uint8_t* smem) {
  constexpr bool BF = sizeof(IO) == 2;
  using Geo = Geom<BF, DK, C>;
  using Lds = PrepLds<IO, DK, C>;
  using E = typename Types<BF>::E;
  using Sp = typename Types<BF>::S;
  constexpr int NB = Geo::NB, E16 = Lds::E16, KP = Lds::KP, BP = Lds::BP;
  constexpr int NKS = Lds::DKP / 32, KB = DK / 16, NTS = Lds::CP / 32;
  constexpr int NBLK = NB * (NB + 1) / 2;
  constexpr int NW = 8;                      // waves per workgroup
  constexpr int GW = NW - 1;                 // the gate wave; waves 0 .. GW-1 form the Gram blocks
  constexpr int NGP = (NBLK + GW - 1) / GW;  // Gram blocks per wave
  constexpr int WPK = NW / KB;               // waves per 16-key block of P
  constexpr int NRW = (NB + WPK - 1) / WPK;  // token blocks of P per wave
  IO* sK = reinterpret_cast<IO*>(smem);
  IO* sQ = sK + Lds::CP * KP;
  float* sA = reinterpret_cast<float*>(smem + Lds::A_OFF);  // after the Gram products
  float* sR = sA;                                           // after the inverse
  float* sQK = reinterpret_cast<float*>(smem + Lds::QK_OFF);
  uint8_t* sTf = smem + Lds::TF_OFF;                        // after R: T' as split B fragments
  float* sT = reinterpret_cast<float*>(smem + Lds::T_OFF);
  IO* sP = reinterpret_cast<IO*>(smem);  // at the end: P^T (tokens x keys) in K's layout
  double* sGb = reinterpret_cast<double*>(smem + Lds::GB_OFF);
  float* sGl = reinterpret_cast<float*>(smem + Lds::GL_OFF);
  float* sBeta = reinterpret_cast<float*>(smem + Lds::B_OFF);
  float* sDec = reinterpret_cast<float*>(smem + Lds::D_OFF);

  if (p >= num_items) return;
  const int gc = p / h_v, h = p % h_v;
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
  // row `row`, columns k0 .. k0 + 7 of a stored lower block-triangular
  // matrix whose diagonal blocks are exactly zero above the diagonal (R: the
  // product of two such blocks); blocks above the diagonal and past C read
  // as zero
  auto row8 = [&](float* m, int row, int k0) {
    f8 x;
    zero(x);
    if (k0 < C && (k0 >> 4) <= (row >> 4)) {
      x.a = *reinterpret_cast<const f4*>(lt(m, row, k0));
      x.b = *reinterpret_cast<const f4*>(lt(m, row, k0 + 4));
    }
    return x;
  };
  // fragment p of the lower-triangular fragment set: row block and slab
  auto frag_rs = [&](int p, int& r, int& s) {
    r = 0;
    while (r + 1 < NB && frag_base(r + 1) <= p) ++r;
    s = p - frag_base(r);
  };
  // two planes at byte `off` of the workspace block: hi, lo (fp32: a, b)
  auto store_split = [&](Rsrc r, uint32_t off, const f8& x) {
    if constexpr (BF) {
      uint4 hi, lo;
      split_bf16x8(x, hi, lo);
      ws_store16(r, off, bits(hi));
      ws_store16(r, off + Geo::PLANE, bits(lo));
    } else {
      ws_store16(r, off, bits(x.a));
      ws_store16(r, off + Geo::PLANE, bits(x.b));
    }
  };
  uint8_t* wsb = ws + (size_t(gc) * h_v + h) * Geo::BYTES;
  const Rsrc rws = make_rsrc(wsb, Geo::BYTES);

  // gate and beta of the chunk's tokens, for the gate wave (used after the barrier)
  float g_ld = 0.f, b_ld = 0.f;
  if (wave == GW && lane < nc) {
    g_ld = g[size_t(t0 + lane) * h_v + h];
    b_ld = beta[size_t(t0 + lane) * h_v + h];
  }
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
  lds_barrier();

  // Gate prefix sums in fp64: G_t = sum_{i<=t} g_i.  Kept, in base 2 (times
  // log2 e), as the sum before each 16-token block (fp64) plus the part within
  // the block (fp32, small), so that every decay exp(G_r - G_i) is one exp2
  // of a short fp32 argument.  One wave computes them while the others form
  // the Gram blocks.
  if (wave == GW) {
    const double gl = wave_prefix_sum(double(g_ld));
    const double glast = readlane_f64(gl, nc - 1);
    const int blk = lane >> 4;  // sum before the token's 16-token block: the scan at lane 16 blk - 1
    const double s15 = readlane_f64(gl, 15), s31 = readlane_f64(gl, 31), s47 = readlane_f64(gl, 47);
    const double gb = blk == 0 ? 0.0 : (blk == 1 ? s15 : (blk == 2 ? s31 : s47));
    if (lane < C) {
      const float gam = lane < nc ? fast_exp(float(gl)) : 0.f;
      const float dec = lane < nc ? fast_exp(float(glast - gl)) : 0.f;
      if ((lane & 15) == 0) sGb[blk] = gb * 1.4426950408889634;
      sGl[lane] = float((gl - gb) * 1.4426950408889634);
      sBeta[lane] = b_ld;
      sDec[lane] = dec;
      float* sc = reinterpret_cast<float*>(wsb + Geo::SCAL_OFF);
      sc[lane] = b_ld;
      sc[C + lane] = b_ld * gam;
      sc[2 * C + lane] = gam;
    }
  }

  // Gram blocks (r, i), i <= r, dealt round-robin to waves 0 .. GW-1: each wave
  // computes K K^T (-> A) and Q K^T (-> QKm) of the same block, which share
  // the decays.  Products stay in registers until every wave is done with
  // the K and Q tiles.
  f4 gk[NGP], gq[NGP];
#pragma unroll
  for (int n = 0; n < NGP; ++n) {
    const int pb = wave < GW ? wave + GW * n : NBLK;
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
  // the first value head of each query/key group stores Q and K as fragments
  if (h % (h_v / h_qk) == 0) {
    constexpr int NQF = NB * NKS;
    const Rsrc rqb = make_rsrc(qf + (size_t(gc) * h_qk + j) * qk_frag_bytes(DK, C, BF), qk_frag_bytes(DK, C, BF));
    for (int p = wave; p < 2 * NQF; p += NW) {
      const int rq = (p % NQF) / NKS, sq = p % NKS;
      const IO* src = (p < NQF ? sQ : sK) + (16 * rq + col) * KP + 32 * sq + 8 * grp;
      const uint32_t off = uint32_t(p * Geo::TPL * Geo::PLANE + lane * 16);
      if constexpr (BF) {
        ws_store16(rqb, off, bits(*reinterpret_cast<const uint4*>(src)));
      } else {
        ws_store16(rqb, off, bits(*reinterpret_cast<const f4*>(src)));
        ws_store16(rqb, off + Geo::PLANE, bits(*reinterpret_cast<const f4*>(src + 4)));
      }
    }
  }
  // K^T operand of this wave's 16-key block of P (rows = keys, k = tokens),
  // read by LDS transpose reads while the K tile is still there and kept in
  // registers until P is formed
  const int wkb = wave % KB;
  E ktw[NTS];
#pragma unroll
  for (int s = 0; s < NTS; ++s) {
    if constexpr (BF) {
      const IO* src = sK + (32 * s + 8 * grp + col / 4) * KP + 16 * wkb + 4 * (col % 4);
      const uint2 lo = lds_tr16(src), hi = lds_tr16(src + 4 * KP);
      ktw[s] = uint4{lo.x, lo.y, hi.x, hi.y};
    } else {
      ld8col(ktw[s], sK + (32 * s + 8 * grp) * KP + 16 * wkb + col, KP);
    }
  }
  lds_barrier();  // K and Q are dead; their space becomes A, QKm and T
  // Scale the Gram blocks by their decays into A and QKm.  The lane's
  // elements of block (r, i) are (4 grp + e, col), BP floats apart; only the
  // diagonal blocks need the causal mask.
#pragma unroll
  for (int n = 0; n < NGP; ++n) {
    const int pb = wave < GW ? wave + GW * n : NBLK;
    if (pb < NBLK) {
      const int r = tri_row(pb), i = pb - r * (r + 1) / 2;
      float* pa = sA + pb * 16 * BP + 4 * grp * BP + col;
      float* pq = sQK + pb * 16 * BP + 4 * grp * BP + col;
      const f4 glr = *reinterpret_cast<const f4*>(sGl + 16 * r + 4 * grp);
      const f4 btr = *reinterpret_cast<const f4*>(sBeta + 16 * r + 4 * grp);
      const float cb = float(sGb[r] - sGb[i]) - sGl[16 * i + col];  // base 2, with glr: <= 0 below the diagonal
      if (i < r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dcy = __builtin_amdgcn_exp2f(cb + glr[e]);
          pa[e * BP] = btr[e] * dcy * gk[n][e];
          pq[e * BP] = dcy * gq[n][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * grp + e;  // row within the block
          const float dcy = __builtin_amdgcn_exp2f(col <= rr ? cb + glr[e] : 0.f);
          pa[e * BP] = col < rr ? btr[e] * dcy * gk[n][e] : 0.f;
          pq[e * BP] = col <= rr ? dcy * gq[n][e] : 0.f;
        }
      }
    }
  }
  lds_barrier();

  // Diagonal blocks: T_bb = (I + A_bb)^{-1}.  Lane 4c+s owns column c and the
  // rows congruent to s mod 4; each row is one quad reduction.
  if (wave < NB) {
    const int b = wave, c = lane >> 2, s = lane & 3;
    // a[rr][m] = A(rr, 4 m + s) of the block; columns 4 m .. 4 m + 3 >= rr
    // are zero (A is strictly lower triangular) and are neither read nor used
    float a[16][4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int m = 0; m < 4; ++m) a[rr][m] = 4 * m < rr ? *lt(sA, 16 * b + rr, 16 * b + 4 * m + s) : 0.f;
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (4 * m < rr) part += a[rr][m] * t[m];
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
    const int r = tri_row(p), i = p - r * (r + 1) / 2;
    f4 acc = zero4();
    for (int kk = i; kk <= r; ++kk) acc = mma_f32(arow(sQK, r, kk), tcol(kk, i), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) *lt(sR, 16 * r + 4 * grp + e, 16 * i + col) = acc[e];
  }
  lds_barrier();

  // R as split fragments.
  for (int p = wave; p < Geo::NF; p += NW) {
    int r, s;
    frag_rs(p, r, s);
    store_split(rws, uint32_t(Geo::R_OFF + p * 2 * Geo::PLANE + lane * 16), row8(sR, 16 * r + col, 32 * s + 8 * grp));
  }
  // T' = diag(dec) T as the B operands of P's products, split once here:
  // fragment (r, s), s >= r / 2, holds column 16 r + col of T' at rows
  // 32 s + 8 grp .. + 7 (hi plane, then lo plane; fp32: rows + 0..3, then
  // + 4..7).  Block (jb, ib) of T' fills half jb % 2 of fragment (ib, jb / 2);
  // the halves above the diagonal (odd ib, jb = ib - 1) and past C (C = 16)
  // are written as zeros.
  auto tfrag = [&](int r, int s) { return (r < 2 ? r * NTS : 2 * NTS + (r - 2) * (NTS - 1)) + (s - r / 2); };
  constexpr int NZB = NB / 2 + (NB == 1 ? 1 : 0);
  for (int pb = wave; pb < NBLK + NZB; pb += NW) {
    int jb, ib;
    f4 t = zero4();
    if (pb < NBLK) {
      jb = tri_row(pb), ib = pb - jb * (jb + 1) / 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jr = 16 * jb + 4 * grp + e;
        t[e] = sDec[jr] * *lt(sT, jr, 16 * ib + col);
      }
    } else {
      ib = NB == 1 ? 0 : 2 * (pb - NBLK) + 1;
      jb = NB == 1 ? 1 : ib - 1;
    }
    // lane 16 (2 (jb % 2) + grp / 2) + col of the fragment, its values 4 (grp % 2) ..
    uint8_t* dst = sTf + tfrag(ib, jb / 2) * 2048 + ((2 * (jb & 1) + (grp >> 1)) * 16 + col) * 16;
    if constexpr (BF) {
      uint2 h, l;
      split_bf16x4(t, h, l);
      *reinterpret_cast<uint2*>(dst + 8 * (grp & 1)) = h;
      *reinterpret_cast<uint2*>(dst + 1024 + 8 * (grp & 1)) = l;
    } else {
      *reinterpret_cast<f4*>(dst + 1024 * (grp & 1)) = t;
    }
  }
  lds_barrier();

  // P blocks (key block wkb, token block r) = sum_s K^T(wkb, slab s) T'(slab s, r)
  // over the slabs reaching the diagonal (s >= r / 2).
  f4 pacc[NRW];
#pragma unroll
  for (int ri = 0; ri < NRW; ++ri) {
    const int r = wave / KB + WPK * ri;
    pacc[ri] = zero4();
    if (r < NB) {
      f4 cl = zero4();
#pragma unroll
      for (int s = 0; s < NTS; ++s) {
        if (2 * s + 1 >= r) {
          Sp tb;
          ld_split(tb, sTf + tfrag(r, s) * 2048 + lane * 16, 1024);
          mm_es(ktw[s], tb, pacc[ri], cl);
        }
      }
      pacc[ri] = pacc[ri] + cl;
    }
  }
  lds_barrier();  // A, R and T are dead; the region becomes the P^T tile
#pragma unroll
  for (int ri = 0; ri < NRW; ++ri) {
    const int r = wave / KB + WPK * ri;
    if (r < NB) {  // D block: P rows = keys 16 wkb + 4 grp .., column = token 16 r + col
      IO* dst = sP + (16 * r + col) * KP + 16 * wkb + 4 * grp;
      if constexpr (BF) *reinterpret_cast<uint2*>(dst) = bf16x4(pacc[ri]);
      else *reinterpret_cast<f4*>(dst) = pacc[ri];
    }
  }
  lds_barrier();
  // P as A fragments (b, s): rows = keys 16 b .., k = tokens 32 s + 8 grp ..
  // (tokens past C zero)
  for (int p = wave; p < KB * NTS; p += NW) {
    const int b = p / NTS, s = p % NTS;
    const bool live = 32 * s + 8 * grp < C;
    const uint32_t off = uint32_t(Geo::P_OFF + p * Geo::TPL * Geo::PLANE + lane * 16);
    if constexpr (BF) {
      const IO* src = sP + (32 * s + 8 * grp + col / 4) * KP + 16 * b + 4 * (col % 4);
      const uint2 lo = lds_tr16(src), hi = lds_tr16(src + 4 * KP);
      ws_store16(rws, off, live ? u32x4{lo.x, lo.y, hi.x, hi.y} : u32x4{0u, 0u, 0u, 0u});
    } else {
      f8 t;
      ld8col(t, sP + (32 * s + 8 * grp) * KP + 16 * b + col, KP);
      ws_store16(rws, off, bits(live ? t.a : zero4()));
      ws_store16(rws, off + Geo::PLANE, bits(live ? t.b : zero4()));
    }
  }
}

// items p = chunk * h_v + value head, the items of XCD x (workgroups i with
// i % 8 == x) contiguous: value heads of one query/key head run on one XCD
// back to back and share its L2 for their K and Q tiles
template <typename IO, int DK, int C>
__global__ __launch_bounds__(512) void chunk_prep_kernel(int h_qk, int h_v, const IO* __restrict__ q,
                                                         const IO* __restrict__ k, const float* __restrict__ g,
                                                         const float* __restrict__ beta, int num_seqs, int T,
                                                         int num_items, const int2* __restrict__ tab,
                                                         uint8_t* __restrict__ ws, uint8_t* __restrict__ qf) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int per = int(gridDim.x) >> 3;
  const int p = int(blockIdx.x & 7) * per + int(blockIdx.x >> 3);
  prep_item<IO, DK, C>(h_qk, h_v, q, k, g, beta, num_seqs, T, num_items, tab, ws, qf, p, smem);
}

// LATE_P: the chain waves load the next chunk's P after their products with
// Y (second window) instead of with their LDS reads (first window).  That
// evens out the vector-memory instructions issued per window (32 and 32 per
// compute unit instead of 48 and 16), which shortens the first window, whose
// loads queue behind each other, when the operands come from the memory-side
// cache (about 4 % faster sweep at 4096 tokens); with operands from HBM the later
// issue leaves too little time to cover the latency, so large working sets
// keep the early issue.
template <typename IO, int DK, int C, bool LATE_P>
__global__ __launch_bounds__(512) void chunk_sweep_kernel(int N, int T, int h_qk, int h_v, int d_v, int max_chunks,
                                                          const IO* __restrict__ v, const int32_t* __restrict__ cu,
                                                          const uint8_t* __restrict__ ws, const uint8_t* __restrict__ qf,
                                                          const float* s_in, IO* __restrict__ out, float* s_out,
                                                          int pfd) {
  constexpr bool BF = sizeof(IO) == 2;
  using Geo = Geom<BF, DK, C>;
  using Lds = SweepLds<IO, DK, C>;
  using E = typename Types<BF>::E;
  using Sp = typename Types<BF>::S;
  constexpr int NB = Geo::NB, KB = DK / 16, CP = Lds::CP, DKP = Lds::DKP, E16 = Lds::E16;
  constexpr int ESZ = Lds::ESZ, TPL = Geo::TPL;
  constexpr size_t PL = Geo::PLANE;
  constexpr int NKS = DKP / 32, NTS = CP / 32;  // 32-wide slabs along d_k and along the chunk
  constexpr int SB = (KB + 3) / 4;              // state blocks per chain wave
  constexpr int NTF = (NB + 1) / 2;             // R fragments per row block, at most
  constexpr size_t QKF = qk_frag_bytes(DK, C, BF), KF = k_frap_off(DK, C, BF);
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sS = smem + Lds::S_OFF;
  uint8_t* sY = smem + Lds::Y_OFF;

  // Workgroups are dealt to the 8 XCDs round-robin (workgroup i to XCD i % 8).
  // A unit is the h_v / h_qk value heads that share one query/key head, each
  // in d_v / 16 row slices; units are dealt to the XCDs round-robin, so the
  // chains of a unit share one L2 (the same Q and K, and each head's P and R),
  // and every sequence's heads spread over all XCDs, which keeps a ragged
  // batch's XCDs evenly loaded.
  const int ntile = d_v / 16;
  const int U = (h_v / h_qk) * ntile;  // chains per unit
  const int i_x = int(blockIdx.x >> 3);
  const int unit = int(blockIdx.x & 7) + 8 * (i_x / U);
  if (unit >= N * h_qk) return;
  const int uidx = i_x % U;  // chain index within the unit
  const int L = unit * U + uidx;
  const int tl = L % ntile, nh = L / ntile, h = nh % h_v, n = nh / h_v;
  const int j = h / (h_v / h_qk);
  const int dv0 = 16 * tl;
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = wave_id();
  const int r = wave & 3;                    // row block (and state-block group) of this wave
  const bool rowblk = NB >= 4 || r < NB;
  const int rb = rowblk ? r : 0;             // row block whose fragments this wave loads

  int bos, eos;
  seq_range(cu, n, T, bos, eos);
  int nchunk = (eos - bos + C - 1) / C;
  const int gc0 = first_slot(bos, n, C);
  nchunk = max(0, min(nchunk, max_chunks - gc0));  // malformed offsets cannot run past the workspace
  if (nchunk == 0 && s_in == s_out) return;  // no tokens and the state already in place
  const int vstride = h_v * d_v;  // elements between consecutive tokens of v
  auto chunk_t0 = [&](int cc) { return bos + cc * C; };
  auto chunk_nc = [&](int cc) { return min(C, eos - chunk_t0(cc)); };
  auto wsb = [&](int cc) { return ws + (size_t(gc0 + cc) * h_v + h) * Geo::BYTES; };
  auto qfb = [&](int cc) { return qf + (size_t(gc0 + cc) * h_qk + j) * QKF; };
  // A fragments of row block rb from a Q or K set (d_k / 32 slabs)
  auto fetch_rows = [&](E (&d)[NKS], const uint8_t* set) __attribute__((always_inline)) {
    const uint8_t* p = set + size_t(rb * NKS) * TPL * PL + lane * 16;
#pragma unroll
    for (int s = 0; s < NKS; ++s) ld_e(d[s], p + s * TPL * PL, int(PL));
  };

  // zero LDS once: exchange columns past C or d_k are read as zeros
  for (int x = tid; x < int(Lds::BYTES / 16); x += 512) reinterpret_cast<uint4*>(smem)[x] = uint4{0u, 0u, 0u, 0u};
  lds_barrier();

  if (wave < 4) {
    // ============================================================ chain waves
    // The recurrence proper: per chunk X = K S^T and Y for token block r,
    // then S^T <- gamma_last S^T + P Y for the owned state blocks.  K and P
    // fragments are loaded two chunks ahead into registers.
    f4 st[SB];
#pragma unroll
    for (int bi = 0; bi < SB; ++bi) {
      const int b = r + 4 * bi;
      st[bi] = zero4();
      if (b < KB) {
        if (s_in) st[bi] = *reinterpret_cast<const f4*>(s_in + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp);
        xb_write_split<BF, DKP>(sS, col, 16 * b + 4 * grp, st[bi]);
      }
    }
    auto fetch_p = [&](E (&pf)[SB][NTS], int cc) __attribute__((always_inline)) {
      const uint8_t* p = wsb(cc) + Geo::P_OFF + lane * 16;
#pragma unroll
      for (int bi = 0; bi < SB; ++bi) {
        const int b = min(r + 4 * bi, KB - 1);  // a wave without this block loads a valid one and ignores it
#pragma unroll
        for (int s = 0; s < NTS; ++s) ld_e(pf[bi][s], p + size_t(b * NTS + s) * TPL * PL, int(PL));
      }
    };
    E kA[NKS], kB[NKS], pA[SB][NTS], pB[SB][NTS];
    if (nchunk > 0) {
      fetch_rows(kA, qfb(0) + KF);
      fetch_rows(kB, qfb(min(1, nchunk - 1)) + KF);
      fetch_p(pA, 0);
    }
    lds_barrier();  // state written, chunks 0 and 1 staged

    // kf, pf: fragments of chunk cc; pn: the other P set, loaded here with
    // chunk cc+1.  Each window issues its LDS reads first and its global
    // loads next, so that a load waiting for the memory queue overlaps the
    // LDS latency instead of delaying the barrier.
    auto step = [&](int cc, E (&kf)[NKS], E (&pf)[SB][NTS], E (&pn)[SB][NTS]) __attribute__((always_inline)) {
      const int nc = chunk_nc(cc);
      const float* sSc = reinterpret_cast<const float*>(smem + Lds::SC_OFF + (cc & 3) * Lds::SCBUF);

      // (1) X = K S^T for token block r (S split: the rounding of the state
      // would otherwise enter every later chunk); Y = beta V - beta gamma X
      Sp bs[NKS];
      uint2 vt;
      f4 bt, bg;
      if (rowblk) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) xb_read_split<BF, DKP>(bs[s], sS, col, 32 * s + 8 * grp);
        bt = *reinterpret_cast<const f4*>(sSc + 16 * r + 4 * grp);
        bg = *reinterpret_cast<const f4*>(sSc + C + 16 * r + 4 * grp);
        if constexpr (BF) {
          // rows 16 r + 4 grp .. + 3 of column col by one transpose read
          const IO* sV = reinterpret_cast<const IO*>(smem + Lds::V_OFF + (cc & 1) * Lds::VBUF);
          vt = lds_tr16(sV + (16 * r + 4 * grp + col / 4) * 16 + 4 * (col % 4));
        }
      }
      if constexpr (!LATE_P) fetch_p(pn, min(cc + 1, nchunk - 1));  // past the end: harmless refetch
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
      if (rowblk) {
        f4 x = zero4(), x1 = zero4(), xl = zero4(), xl1 = zero4();
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          if (s & 1) mm_es(kf[s], bs[s], x1, xl1);
          else mm_es(kf[s], bs[s], x, xl);
        }
        x = (x + x1) + (xl + xl1);
        float vv[4];
        if constexpr (BF) {
          vv[0] = __uint_as_float(vt.x << 16), vv[1] = __uint_as_float(vt.x & 0xffff0000u);
          vv[2] = __uint_as_float(vt.y << 16), vv[3] = __uint_as_float(vt.y & 0xffff0000u);
        } else {
          const IO* sV = reinterpret_cast<const IO*>(smem + Lds::V_OFF + (cc & 1) * Lds::VBUF);
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = sV[(16 * r + 4 * grp + e) * 16 + col];
        }
        f4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = bt[e] * vv[e] - bg[e] * x[e];
        if (nc < C) {  // tokens past the end of a partial chunk
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * r + 4 * grp + e >= nc) y[e] = 0.f;
        }
        xb_write_split<BF, CP>(sY, col, 16 * r + 4 * grp, y);
      }
      lds_barrier();

      // (2) S^T <- gamma_last S^T + P Y for the owned state blocks
      Sp yb[NTS];
#pragma unroll
      for (int s = 0; s < NTS; ++s) xb_read_split<BF, CP>(yb[s], sY, col, 32 * s + 8 * grp);
      const float glast = sSc[2 * C + nc - 1];
      fetch_rows(kf, qfb(min(cc + 2, nchunk - 1)) + KF);
      __builtin_amdgcn_sched_barrier(0);
      f4 ah[SB], al[SB];
#pragma unroll
      for (int bi = 0; bi < SB; ++bi) ah[bi] = st[bi] * glast, al[bi] = zero4();
#pragma unroll
      for (int s = 0; s < NTS; ++s)
#pragma unroll
        for (int bi = 0; bi < SB; ++bi)
          if (r + 4 * bi < KB) mm_es(pf[bi][s], yb[s], ah[bi], al[bi]);
      if constexpr (LATE_P) {
        __builtin_amdgcn_sched_barrier(0);
        fetch_p(pn, min(cc + 1, nchunk - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int bi = 0; bi < SB; ++bi) {
        const int b = r + 4 * bi;
        if (b < KB) {
          st[bi] = ah[bi] + al[bi];
          xb_write_split<BF, DKP>(sS, col, 16 * b + 4 * grp, st[bi]);
        }
      }
      lds_barrier();
    };
    // Pairs of steps, the first pair peeled, so that every path into the
    // loop has issued the same memory operations in the same order (the
    // memory-counter waits then stay exact); an odd last chunk runs after
    // the loop.
    int cc = 0;
    if (nchunk >= 2) {
      step(0, kA, pA, pB);
      step(1, kB, pB, pA);
      for (cc = 2; cc + 1 < nchunk; cc += 2) {
        step(cc, kA, pA, pB);
        step(cc + 1, kB, pB, pA);
      }
    }
    if (cc < nchunk) step(cc, kA, pA, pB);

#pragma unroll
    for (int bi = 0; bi < SB; ++bi) {
      const int b = r + 4 * bi;
      if (b < KB) *reinterpret_cast<f4*>(s_out + (size_t(nh) * d_v + dv0 + col) * DK + 16 * b + 4 * grp) = st[bi];
    }
  } else {
    // ============================================================ helper waves
    // Everything off the recurrence, for token block r: Z = Q S^T, the
    // output O = gamma Z + R Y, and the staging of V slices and scalars two
    // chunks ahead.  Both products are formed transposed (the operands swap
    // roles, same registers), so that each lane holds four consecutive values
    // of one output row and stores them at once.  Q and R fragments are
    // loaded two chunks ahead into registers.
    const int ht = tid - 256;  // 0..255
    float pf_sink = 0.f;        // keeps the prefetch loads alive
    constexpr int NVP = int(Lds::VBUF / 16);      // 16-byte pieces of a chunk's V slice
    constexpr int NSP = int(Lds::SCBUF / 16);      // and of its scalars
    constexpr int NST = (NVP + NSP + 255) / 256;   // pieces per helper lane
    const uint32_t ooff = uint32_t(((16 * r + col) * vstride + 4 * grp) * ESZ);
    const uint32_t v_tail = uint32_t(16 * ESZ);

    auto fetch_stg = [&](u32x4 (&P)[NST], int cc) __attribute__((always_inline)) {
      // one plain load per piece, its address chosen per lane: V rows past
      // the chunk's end are clamped to its last row (those tokens are masked
      // where V is used)
      const int t0 = chunk_t0(cc), nc = chunk_nc(cc);
      const IO* vb = v + (size_t(t0) * h_v + h) * d_v + dv0;
      const uint8_t* sc = wsb(cc) + Geo::SCAL_OFF;
      constexpr int PPT = 16 / E16;  // pieces per token row of the V slice
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        const int x = min(ht + 256 * it, NVP + NSP - 1);
        const int tok = min(x / PPT, nc - 1);
        const uint8_t* src = x < NVP ? reinterpret_cast<const uint8_t*>(vb + size_t(tok) * vstride + (x % PPT) * E16)
                                     : sc + size_t(x - NVP) * 16;
        P[it] = *reinterpret_cast<const u32x4*>(src);
      }
    };
    auto commit_stg = [&](const u32x4 (&P)[NST], int cc) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        const int x = ht + 256 * it;
        uint8_t* dst = x < NVP ? smem + Lds::V_OFF + (cc & 1) * Lds::VBUF + size_t(x) * 16
                               : smem + Lds::SC_OFF + (cc & 3) * Lds::SCBUF + size_t(x - NVP) * 16;
        if (x < NVP + NSP) *reinterpret_cast<u32x4*>(dst) = P[it];
      }
    };

    // One loop per fragment count, so that each wave issues only the loads
    // it needs and every path through a loop issues the same ones.
    auto run = [&](auto nr_c) __attribute__((always_inline)) {
      constexpr int NR = decltype(nr_c)::value;  // R fragments of block r (0: no token block)
      constexpr int NRA = NR > 0 ? NR : 1;
      auto fetch_r = [&](Sp (&d)[NRA], int cc) __attribute__((always_inline)) {
        const uint8_t* p = wsb(cc) + Geo::R_OFF + size_t(frag_base(r)) * 2 * PL + lane * 16;
#pragma unroll
        for (int s = 0; s < NR; ++s) ld_split(d[s], p + s * 2 * PL, int(PL));
      };
      E aqA[NKS], aqB[NKS];
      Sp rA[NRA], rB[NRA];
      // staged pieces (V slice and scalars) of one chunk, as native vectors so
      // that the copies stay in registers
      u32x4 s0[NST], s1[NST];
      if (nchunk > 0) {
        const int c1 = min(1, nchunk - 1);
        fetch_stg(s0, 0);
        fetch_stg(s1, c1);
        if constexpr (NR > 0) {
          fetch_rows(aqA, qfb(0));
          fetch_rows(aqB, qfb(c1));
          fetch_r(rA, 0);
        }
        commit_stg(s0, 0);
        commit_stg(s1, 1);
        fetch_stg(s0, min(2, nchunk - 1));
      }
      lds_barrier();  // state written, chunks 0 and 1 staged

      // aq, rf: fragments of chunk cc; stg: staged chunk cc+2.  rn and sn,
      // the other sets, are loaded here with R of chunk cc+1 and the staged
      // pieces of chunk cc+3, in the first window, where these waves wait.
      // L2 prefetch of chunk cc, pfd chunks ahead (pfd past the last chunk: no
      // prefetch, for operands and V small enough to stay in the memory-side
      // cache between the prep and this launch): each chain touches one dword of its share of the 128-byte
      // lines (the unit's chains share the K and Q sets, a value head's slices
      // its per-chunk block and V rows), so the loads of a few steps later
      // find them in the XCD's L2 instead of waiting for HBM.
      auto prefetch = [&](int cc) __attribute__((always_inline)) -> float {
        constexpr int LN = 128;
        constexpr int NQK = int(QKF / LN), NWS = int(Geo::BYTES / LN);
        const int vrow_lines = (d_v * ESZ + LN - 1) / LN;
        const int nv = (chunk_nc(cc) * vrow_lines - tl + ntile - 1) / ntile;
        const int nqk = (NQK - uidx + U - 1) / U, nws = (NWS - tl + ntile - 1) / ntile;
        int m = ht;
        const uint8_t* a = nullptr;
        if (m < nv) {
          const int ln = tl + ntile * m;
          a = reinterpret_cast<const uint8_t*>(v + (size_t(chunk_t0(cc) + ln / vrow_lines) * h_v + h) * d_v) +
              size_t(ln % vrow_lines) * LN;
        } else if ((m -= nv) < nqk) {
          a = qfb(cc) + size_t(uidx + U * m) * LN;
        } else if ((m -= nqk) < nws) {
          a = wsb(cc) + size_t(tl + ntile * m) * LN;
        }
        return a ? *reinterpret_cast<const float*>(a) : 0.f;
      };
      float pf_prev = 0.f;

      auto step = [&](int cc, E (&aq)[NKS], Sp (&rf)[NRA], Sp (&rn)[NRA], u32x4 (&stg)[NST],
                      u32x4 (&sn)[NST]) __attribute__((always_inline)) {
        const int nc = chunk_nc(cc);
        const float* sSc = reinterpret_cast<const float*>(smem + Lds::SC_OFF + (cc & 3) * Lds::SCBUF);
        pf_sink += pf_prev;  // consume the previous step's prefetch (issued a whole step ago)
        pf_prev = cc + pfd < nchunk ? prefetch(cc + pfd) : 0.f;

        // (1) Z^T = S Q^T for token block r (S is the chunk's initial state,
        // split: with slow decay S Q^T carries most of the output)
        Sp bs[NKS];
        if constexpr (NR > 0) {
#pragma unroll
          for (int s = 0; s < NKS; ++s) xb_read_split<BF, DKP>(bs[s], sS, col, 32 * s + 8 * grp);
          fetch_r(rn, min(cc + 1, nchunk - 1));
        }
        fetch_stg(sn, min(cc + 3, nchunk - 1));
        __builtin_amdgcn_sched_barrier(0);
        f4 z = zero4();
        if constexpr (NR > 0) {
          f4 z1 = zero4(), zl = zero4(), zl1 = zero4();
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
            if (s & 1) mm_se(bs[s], aq[s], z1, zl1);
            else mm_se(bs[s], aq[s], z, zl);
          }
          z = (z + z1) + (zl + zl1);
          fetch_rows(aq, qfb(min(cc + 2, nchunk - 1)));
        }
        lds_barrier();

        // (2) O^T = Z^T diag(gamma) + Y^T R^T for token block r: lane holds
        // values 4 grp .. + 3 of output row 16 r + col; stage chunk cc+2
        if constexpr (NR > 0) {
          Sp yb[NRA];
#pragma unroll
          for (int s = 0; s < NR; ++s) xb_read_split<BF, CP>(yb[s], sY, col, 32 * s + 8 * grp);
          f4 oh = z * sSc[2 * C + 16 * r + col], ol = zero4();
#pragma unroll
          for (int s = 0; s < NR; ++s) mm_ss(yb[s], rf[s], oh, ol);
          const Rsrc ro = make_rsrc(out + (size_t(chunk_t0(cc)) * h_v + h) * d_v + dv0,
                                    uint32_t((nc - 1) * vstride * ESZ) + v_tail);
          bstore4<IO>(ro, ooff, oh + ol);  // rows past the chunk's end are dropped
        }
        commit_stg(stg, cc + 2);  // after the last chunk this fills buffers nobody reads
        lds_barrier();
      };
      int cc = 0;  // pairs of steps, the first pair peeled (as for the chain waves)
      if (nchunk >= 2) {
        step(0, aqA, rA, rB, s0, s1);
        step(1, aqB, rB, rA, s1, s0);
        for (cc = 2; cc + 1 < nchunk; cc += 2) {
          step(cc, aqA, rA, rB, s0, s1);
          step(cc + 1, aqB, rB, rA, s1, s0);
        }
      }
      if (cc < nchunk) step(cc, aqA, rA, rB, s0, s1);
    };
    if (!rowblk) run(std::integral_constant<int, 0>());
    else if (NTF == 1 || r < 2) run(std::integral_constant<int, 1>());
    else run(std::integral_constant<int, NTF>());
    if (T < 0) s_out[tid] = pf_sink;  // never true (T >= 0): the sink only has to look used
  }
}

// ---------------------------------------------------------------- host side

size_t chunked_max_chunks(const Dims& d, int chunk) {
  // sum_n ceil(L_n / C) <= (T + N (C - 1)) / C
  return (size_t(d.total_tokens) + size_t(d.num_seqs) * size_t(chunk - 1)) / size_t(chunk);
}

static size_t chunk_bytes(const Dims& d, int chunk) {
  if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
  return chunk_block_bytes(d.bf16, d.d_k, chunk);
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }
static size_t table_bytes(const Dims& d, int chunk) { return round256(chunked_max_chunks(d, chunk) * 8); }

static size_t blocks_bytes(const Dims& d, int chunk) {
  return chunked_max_chunks(d, chunk) * size_t(d.h_v) * chunk_bytes(d, chunk);
}

static size_t qf_bytes(const Dims& d, int chunk) {
  return chunked_max_chunks(d, chunk) * size_t(d.h_qk) * qk_frag_bytes(d.d_k, chunk, d.bf16);
}

size_t chunked_workspace_bytes(const Dims& d, int chunk) {
  if (chunk_bytes(d, chunk) == 0) return 0;
  return table_bytes(d, chunk) + blocks_bytes(d, chunk) + qf_bytes(d, chunk);
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
    const size_t items = max_chunks * size_t(d.h_v);
    hipLaunchKernelGGL((chunk_prep_kernel<IO, DK, C>), dim3(unsigned((items + 7) / 8 * 8)), dim3(512), lds,
                       st, d.h_qk, d.h_v, static_cast<const IO*>(q), static_cast<const IO*>(k), g, beta, d.num_seqs,
                       d.total_tokens, int(items), tab, ws, qf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // eight XCDs, each dealt ceil(units / 8) units of U chains (see the kernel)
  const int units = d.num_seqs * d.h_qk, U = (d.h_v / d.h_qk) * (d.d_v / 16);
  if (units == 0) return hipSuccess;
  const int per = (units + 7) / 8 * U;
  constexpr size_t lds = SweepLds<IO, DK, C>::BYTES;
  if (lds > 65536) {
    for (const void* f : {reinterpret_cast<const void*>(&chunk_sweep_kernel<IO, DK, C, false>),
                          reinterpret_cast<const void*>(&chunk_sweep_kernel<IO, DK, C, true>)}) {
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
  }
  // Prefetch six chunks ahead when the operands and V (per launch) exceed
  // what the 256 MiB memory-side cache keeps between the two launches.
  const size_t v_bytes = size_t(d.total_tokens) * d.h_v * d.d_v * (d.bf16 ? 2 : 4);
  const bool large = blocks_bytes(d, C) + qf_bytes(d, C) + v_bytes > (size_t(192) << 20);
  const int pfd = large ? 6 : (1 << 30);
  Prof prof("chunk_sweep", st);
  if (large)
    hipLaunchKernelGGL((chunk_sweep_kernel<IO, DK, C, false>), dim3(8 * per), dim3(512), lds, st, d.num_seqs,
                       d.total_tokens, d.h_qk, d.h_v, d.d_v, int(max_chunks), static_cast<const IO*>(v), cu, ws, qf,
                       s_in, static_cast<IO*>(out), s_out, pfd);
  else
    hipLaunchKernelGGL((chunk_sweep_kernel<IO, DK, C, true>), dim3(8 * per), dim3(512), lds, st, d.num_seqs,
                       d.total_tokens, d.h_qk, d.h_v, d.d_v, int(max_chunks), static_cast<const IO*>(v), cu, ws, qf,
                       s_in, static_cast<IO*>(out), s_out, pfd);
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
