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
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_bf16).  The rows of each expert
// are cut into blocks of BM = 64 (the last one short); block b of expert e is
// slot first_slot(e) + b with first_slot(e) = (offset_e + e (BM - 1)) / BM, so
// the grid needs no table: a workgroup stages the expert offsets in LDS and
// finds its expert by binary search.  A workgroup of four waves owns one row
// block and BN = 128 output columns; wave w owns 32 of them (two 16-column
// tiles) for all four row tiles.  The contraction runs in super-slabs of 128
// k, each four MFMA slabs of 32; within a super-slab lane group grp takes
// k = 32 grp + 8 j + (0..7) in slab j, the same for the activations and the
// weights (a sum over k does not care about the order), so one 16-byte load
// per lane and column brings the codes of all four slabs, all in one group of
// 64 (one scale and bias per lane and column).  The codes are loaded two
// super-slabs ahead, the activations one slab ahead; each weight is rebuilt
// once per row block (two mask operations, eight byte conversions, eight fma
// and four bf16 packs per eight weights).
//
// Packed codes.  In the row-major layout one 16-byte load per lane and column
// makes an instruction touch 16 weight rows k / 2 bytes apart, 64 bytes each
// (a power-of-two stride when k is); the compute unit's load path takes that
// shape slowly.  gdn_moe_pack_q4 rewrites the codes once (at weight-load time)
// so that the 16 rows x 64 bytes of one 16-row tile and super-slab that one
// such load instruction needs are one contiguous 1 KiB block, in lane order:
// block ((e * n / 16 + t) * k / 128 + u), lane 16 g + c at byte 16 lane holds
// bytes 64 u + 16 g .. + 15 of row 16 t + c (the codes of k = 128 u + 32 g ..
// + 31).  The packed GEMM reads those blocks; its arithmetic is the same.
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {
constexpr int BN = 128;  // output columns per workgroup
constexpr int BM = 64;   // rows per block (four row tiles of 16)
constexpr int GROUP = 64;
constexpr int KS = 128;  // k per super-slab

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// staged pieces as native vectors, so that arrays of them stay in registers
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

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

// One thread per 16-byte piece of the packed layout (64 pieces per block).
__global__ __launch_bounds__(256) void pack_q4_kernel(size_t n_pieces, int n, int k, const uint4* __restrict__ codes,
                                                      uint4* __restrict__ packed) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_pieces) return;
  const size_t blk = i >> 6;
  const int lane = int(i & 63), g = lane >> 4, c = lane & 15;
  const size_t nu = size_t(k / KS), nt = size_t(n / 16);
  const size_t u = blk % nu, t = (blk / nu) % nt, e = blk / (nu * nt);
  const size_t row = e * size_t(n) + 16 * t + c;  // row of the [E * n, k / 2] byte matrix
  packed[i] = codes[(row * size_t(k / 2) + 64 * u + 16 * g) / 16];
}

__device__ __forceinline__ int first_slot(int off, int e) { return (off + e * (BM - 1)) / BM; }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its global loads (__syncthreads would also drain the
// codes and activations prefetched for later super-slabs).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS: the expert offsets, then two buffers of the row block's activations for
// one super-slab, [BM rows][KS k] bf16 with rows AS bytes apart (32 mod 128,
// so the 16-lane fragment reads of 16 rows are free of bank conflicts), then
// two buffers of the block's scales and biases for a window of four
// super-slabs (eight groups), [2 arrays][BN columns][8 groups] bf16.
constexpr int AS = KS * 2 + 32;
constexpr int ABUF = BM * AS;
constexpr int WIN = 4;                        // super-slabs per scale/bias window
constexpr int WG_GROUPS = WIN * KS / GROUP;  // groups per window (8)
constexpr int SBBUF = 2 * BN * WG_GROUPS * 2;
__host__ __device__ constexpr size_t moe_lds_bytes(int n_exp) {
  return (size_t(n_exp + 1) * 4 + 15) / 16 * 16 + 2 * ABUF + 2 * SBBUF;
}

template <bool Q4, bool PACKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void moe_gemm_kernel(
    int n_exp, int m, int n, int k, const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
    const uint8_t* __restrict__ wsrc, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* soff = reinterpret_cast<int*>(smem);
  uint8_t* sa = smem + (size_t(n_exp + 1) * 4 + 15) / 16 * 16;
  uint8_t* ssb = sa + 2 * ABUF;
  // Workgroups reach the eight XCDs round-robin (workgroup i on XCD i % 8).
  // XCD x takes the contiguous slots [x S8, x S8 + S8) (S8 = slots / 8, the
  // slot count being a multiple of 8), in order, each with its ncb column
  // blocks together: the column blocks share the slot's activation rows, and
  // the row blocks of one expert, adjacent slots, share its codes, through
  // that XCD's L2.  Workgroup i is column block (i / 8) % ncb of slot
  // (i % 8) S8 + (i / 8) / ncb.
  const int ncb = n / BN;
  const int S8 = int(gridDim.x) / (8 * ncb);
  const int xi = int(blockIdx.x >> 3);
  const int slot = int(blockIdx.x & 7) * S8 + xi / ncb, cb = xi % ncb;
  for (int i = threadIdx.x; i <= n_exp; i += 256) {
    int o = offsets[i];
    soff[i] = o < 0 ? 0 : (o > m ? m : o);  // malformed offsets cannot index out of bounds
  }
  __syncthreads();
  // the expert whose slots contain this one: the largest e with first_slot(e) <= slot
  int lo = 0, hi = n_exp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first_slot(soff[mid], mid) <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int e_lo = soff[e], e_hi = max(soff[e + 1], e_lo);
  const int fs = first_slot(e_lo, e);
  if (slot < fs) return;  // only with malformed (decreasing) offsets
  const int r_lo = e_lo + (slot - fs) * BM;
  if (r_lo >= e_hi) return;  // a spare slot of this expert
  const int r_hi = min(r_lo + BM, e_hi);

  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = cb * BN + 32 * wave;  // this wave's 32 columns
  const int ngroups = k / GROUP;
  const size_t wrow0 = size_t(e) * n + n0 + col, wrow1 = wrow0 + 16;

  // The k loop, for NT row tiles that hold rows (1..4, the same in the whole
  // workgroup): only those tiles are staged, read and multiplied.
  auto run = [&](auto nt_c) __attribute__((always_inline)) {
    constexpr int NT = decltype(nt_c)::value;
    constexpr int NP = NT;  // 16-byte pieces per thread: NT * 16 rows * 16 pieces / 256 threads
    // staging of one super-slab of activations: thread tid moves pieces
    // tid + 256 i (row p / 16, 16 bytes at k = 8 (p % 16)); rows past the
    // block repeat its last row (their results are dropped)
    uint32_t goff[NP], loff[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + 256 * i, r = p >> 4, c = p & 15;
      goff[i] = uint32_t(min(r_lo + r, r_hi - 1)) * uint32_t(k) + 8 * c;
      loff[i] = uint32_t(r * AS + 16 * c);
    }
    auto fetch_a = [&](v4u (&st)[NP], int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NP; ++i) st[i] = *reinterpret_cast<const v4u*>(x + goff[i] + ks);
    };
    auto commit_a = [&](const v4u (&st)[NP], int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NP; ++i) *reinterpret_cast<v4u*>(sa + buf * ABUF + loff[i]) = st[i];
    };
    // codes of one super-slab for both columns: 16 bytes each (Q4); packed,
    // the wave's two 16-row tiles are consecutive tile rows, k / KS blocks apart
    const size_t pblk0 = (size_t(e) * (n / 16) + size_t(n0 / 16)) * size_t(k / KS);
    auto load_w = [&](uint4 (&c)[2], int ks) __attribute__((always_inline)) {
      if constexpr (Q4 && PACKED) {
        const size_t b0 = pblk0 + size_t(ks / KS);
        c[0] = *reinterpret_cast<const uint4*>(wsrc + (b0 << 10) + lane * 16);
        c[1] = *reinterpret_cast<const uint4*>(wsrc + ((b0 + size_t(k / KS)) << 10) + lane * 16);
      } else if constexpr (Q4) {
        c[0] = *reinterpret_cast<const uint4*>(wsrc + wrow0 * (k / 2) + ks / 2 + 16 * grp);
        c[1] = *reinterpret_cast<const uint4*>(wsrc + wrow1 * (k / 2) + ks / 2 + 16 * grp);
      }
    };
    // scales and biases of window w (8 groups) for the block's 128 columns:
    // thread t loads array t / 128, column t % 128, as four 4-byte pieces
    // (a scattered 2-byte load per lane and super-slab costs far more), and
    // the window goes to LDS at the barrier before it is used
    const int sb_arr = tid >> 7, sb_col = tid & (BN - 1);
    const uint16_t* sb_row =
        Q4 ? (sb_arr ? biases : scales) + (size_t(e) * n + size_t(cb) * BN + sb_col) * ngroups : nullptr;
    auto fetch_sb = [&](uint32_t (&r)[4], int w) __attribute__((always_inline)) {
      if constexpr (Q4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int g = WG_GROUPS * w + 2 * i;
          r[i] = g < ngroups ? *reinterpret_cast<const uint32_t*>(sb_row + g) : 0u;
        }
      }
    };
    auto commit_sb = [&](const uint32_t (&r)[4], int w) __attribute__((always_inline)) {
      if constexpr (Q4)
        *reinterpret_cast<uint4*>(ssb + (w & 1) * SBBUF + (sb_arr * BN + sb_col) * (WG_GROUPS * 2)) =
            uint4{r[0], r[1], r[2], r[3]};
    };

    f4 acc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = zero4();
    uint4 c0[2], c1[2], c2[2];
    v4u stg[NP];
    uint32_t sbr[4];
    const int nks = k / KS, nwin = (nks + WIN - 1) / WIN;
    load_w(c0, 0);
    load_w(c1, min(KS, k - KS));
    fetch_sb(sbr, 0);
    fetch_a(stg, 0);
    commit_sb(sbr, 0);
    commit_a(stg, 0);
    lds_barrier();
    for (int si = 0; si < nks; ++si) {
      const int ks = si * KS, buf = si & 1;
      // the next super-slab's activations first, then the codes two ahead, so
      // that waiting for the activations leaves the codes in flight; both
      // unconditional (the end reloads the last) so the memory waits stay exact
      const int w = si / WIN;
      fetch_a(stg, min(ks + KS, k - KS));
      load_w(c2, min(ks + 2 * KS, k - KS));
      if (si % WIN == 0 && w + 1 < nwin) fetch_sb(sbr, w + 1);  // the next window, committed at this one's end
      float s0 = 0.f, b0 = 0.f, s1 = 0.f, b1 = 0.f;
      if constexpr (Q4) {
        // group of the lane's k in this super-slab: 2 (si % WIN) + grp / 2 within the window
        const uint16_t* sbw = reinterpret_cast<const uint16_t*>(ssb + (w & 1) * SBBUF);
        const int gl = 2 * (si % WIN) + (grp >> 1), c0l = 32 * wave + col;
        s0 = bf16_bits_to_f32(sbw[c0l * WG_GROUPS + gl]);
        b0 = bf16_bits_to_f32(sbw[(BN + c0l) * WG_GROUPS + gl]);
        s1 = bf16_bits_to_f32(sbw[(c0l + 16) * WG_GROUPS + gl]);
        b1 = bf16_bits_to_f32(sbw[(BN + c0l + 16) * WG_GROUPS + gl]);
      }
      const uint32_t d0[4] = {c0[0].x, c0[0].y, c0[0].z, c0[0].w}, d1[4] = {c0[1].x, c0[1].y, c0[1].z, c0[1].w};
      const uint8_t* abase = sa + buf * ABUF + col * AS + 64 * grp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = ks + 8 * j;
        uint4 bf0, bf1;
        if constexpr (Q4) {
          bf0 = rebuild8(d0[j], s0, b0);
          bf1 = rebuild8(d1[j], s1, b1);
        } else {
          const uint16_t* wb16 = reinterpret_cast<const uint16_t*>(wsrc);
          bf0 = *reinterpret_cast<const uint4*>(wb16 + wrow0 * k + kk + 32 * grp);
          bf1 = *reinterpret_cast<const uint4*>(wb16 + wrow1 * k + kk + 32 * grp);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 a = *reinterpret_cast<const uint4*>(abase + 16 * t * AS + 16 * j);
          acc[t][0] = mma32(a, bf0, acc[t][0]);
          acc[t][1] = mma32(a, bf1, acc[t][1]);
        }
      }
      commit_a(stg, buf ^ 1);  // the other buffer: its last readers passed the previous barrier
      if (si % WIN == WIN - 1 && w + 1 < nwin) commit_sb(sbr, w + 1);  // likewise for window w - 1's buffer
      lds_barrier();
      c0[0] = c1[0], c0[1] = c1[1], c1[0] = c2[0], c1[1] = c2[1];
    }
    // D block: lane holds rows 4 grp .. 4 grp + 3 of the tile, column col
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int r = r_lo + 16 * t + 4 * grp + qq;
        if (r < r_hi) {
          y[size_t(r) * n + n0 + col] = f2bf(acc[t][0][qq]);
          y[size_t(r) * n + n0 + 16 + col] = f2bf(acc[t][1][qq]);
        }
      }
    }
  };
  const int nt = (r_hi - r_lo + 15) / 16;  // row tiles that hold rows, 1..4
  if (nt == 1) run(std::integral_constant<int, 1>());
  else if (nt == 2) run(std::integral_constant<int, 2>());
  else if (nt == 3) run(std::integral_constant<int, 3>());
  else run(std::integral_constant<int, 4>());
}

hipError_t launch_moe_gemm(int n_exp, int m, int n, int k, const void* x, const int32_t* offsets,
                           const void* weights, const void* scales, const void* biases, void* y, bool q4,
                           bool packed, hipStream_t st) {
  // row-block slots: sum_e ceil(m_e / BM) <= (m + E (BM - 1)) / BM, rounded up
  // to a multiple of 8 for the XCD mapping (the spare slots return at once)
  const size_t slots = ((size_t(m) + size_t(n_exp) * (BM - 1)) / BM + 7) / 8 * 8;
  const unsigned blocks = unsigned(slots * size_t(n / BN));
  if (blocks == 0 || m == 0) return hipSuccess;
  Prof prof(q4 ? (packed ? "moe_gemm_q4_packed" : "moe_gemm_q4") : "moe_gemm_bf16", st);
  const size_t lds = moe_lds_bytes(n_exp);
  auto go = [&](auto kern, const void* sc, const void* bi) {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, st, n_exp, m, n, k, static_cast<const uint16_t*>(x),
                       offsets, static_cast<const uint8_t*>(weights), static_cast<const uint16_t*>(sc),
                       static_cast<const uint16_t*>(bi), static_cast<uint16_t*>(y));
    return hipGetLastError();
  };
  if (!q4) return go(moe_gemm_kernel<false, false>, nullptr, nullptr);
  if (packed) return go(moe_gemm_kernel<true, true>, scales, biases);
  return go(moe_gemm_kernel<true, false>, scales, biases);
}

hipError_t launch_pack_q4(int n_exp, int n, int k, const void* codes, void* packed, hipStream_t st) {
  const size_t n_pieces = size_t(n_exp) * n * (k / 32);
  if (n_pieces == 0) return hipSuccess;
  Prof prof("pack_q4", st);
  hipLaunchKernelGGL(pack_q4_kernel, dim3(unsigned((n_pieces + 255) / 256)), dim3(256), 0, st, n_pieces, n, k,
                     static_cast<const uint4*>(codes), static_cast<uint4*>(packed));
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
