"""GPU parity of the grouped expert GEMM on 4-bit group-affine weights
(gdn_moe_gemm_q4) and of the pages' ablation (gdn_dequant_q4 then
gdn_moe_gemm_bf16) against the fp64 oracle.

Perplexity's "Optimizing on-device inference for Apple Silicon", section
"Dequantize the weights during the matrix multiplication": 4-bit codes, a bf16
scale and bias per group of 64 weights, the weights rebuilt in bf16, fp32
accumulation, bf16 output.  Checks:

- the rebuilt bf16 weights equal the oracle's bit for bit (both round the
  exact scale * code + bias once);
- the fused and the two-pass forms give the same y bit for bit;
- y against the oracle per (expert, column block) slice, relative Frobenius,
  3e-3 (bf16 output; the products are exact, the fp32 sums differ in order);
- the hand-worked fixture, whose sums are exact in fp32, equals the oracle's
  values rounded to bf16 exactly.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import make_moe
from oracle import dequantize_q4, grouped_gemm_q4, round_bf16

from helpers import TOL, Errors, seq_errors, host

pytestmark = pytest.mark.gpu


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def dev(m):
    return dict(x=bf(m.x), expert_offsets=torch.from_numpy(m.expert_offsets.astype(np.int32)).cuda(),
                codes=torch.from_numpy(m.codes).cuda(), scales=bf(m.scales), biases=bf(m.biases))


def max_rel_rows(y, r, off):
    """Largest relative Frobenius error over experts' row blocks."""
    worst = 0.0
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            den = np.linalg.norm(r[a:b])
            worst = max(worst, np.linalg.norm(y[a:b] - r[a:b]) / den if den > 0 else np.linalg.norm(y[a:b]))
    return worst


def test_dequant_bit_exact():
    m = make_moe(64, num_experts=3, top_k=2, k=256, n=128, seed=11)
    d = dev(m)
    w = gdn.dequant_q4(d["codes"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    ref = dequantize_q4(m.codes, m.scales, m.biases)
    np.testing.assert_array_equal(host(w), ref)


@pytest.mark.parametrize("tokens,E,top_k,K,N", [
    (64, 4, 2, 128, 128),
    (200, 8, 3, 256, 256),
    (300, 16, 8, 512, 128),     # experts with hundreds of rows: several 64-row blocks
    (40, 64, 4, 128, 384),      # many empty experts
])
def test_moe_gemm_parity(tokens, E, top_k, K, N):
    m = make_moe(tokens, num_experts=E, top_k=top_k, k=K, n=N, seed=tokens + E)
    d = dev(m)
    y = gdn.moe_gemm_q4(**d)
    w = gdn.dequant_q4(d["codes"], d["scales"], d["biases"])
    y2 = gdn.moe_gemm_bf16(d["x"], d["expert_offsets"], w)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # the ablation computes exactly the same
    ref = grouped_gemm_q4(m.x, m.codes, m.scales, m.biases, m.expert_offsets)
    err = max_rel_rows(host(y), ref, m.expert_offsets)
    counts = np.diff(m.expert_offsets)
    print(f"moe q4 tokens={tokens} E={E} K={K} N={N} rows/expert {counts.min()}..{counts.max()}: err={err:.3e}",
          flush=True)
    assert err <= TOL["bf16"]


def test_moe_gemm_golden_fixture():
    # the hand-worked case (2 experts, 2 columns, K = 128) in columns 0-1 of a 128-column problem
    from test_oracle import load_q4_fixture
    f = load_q4_fixture()
    E, N, K = 2, 128, 128
    codes = np.zeros((E, N, K // 2), np.uint8)
    scales = np.zeros((E, N, K // 64))
    biases = np.zeros((E, N, K // 64))
    codes[:, :2], scales[:, :2], biases[:, :2] = f["codes"], f["scales"], f["biases"]
    y = gdn.moe_gemm_q4(bf(f["x"]), torch.from_numpy(f["offsets"].astype(np.int32)).cuda(),
                        torch.from_numpy(codes).cuda(), bf(scales), bf(biases))
    torch.cuda.synchronize()
    yh = host(y)
    np.testing.assert_array_equal(yh[:, :2], round_bf16(f["y"]))  # 706 rounds to 704 in bf16
    np.testing.assert_array_equal(yh[:, 2:], 0.0)


def test_moe_gemm_full_size_all_experts():
    # 2048 tokens routed to 8 of 256 experts, K = 2048, N = 1024: the oracle
    # checks every expert (one call per expert keeps its fp64 weights small),
    # on the three measures over each expert's rows (rows as tokens)
    m = make_moe(2048, num_experts=256, top_k=8, k=2048, n=1024, seed=2048)
    d = dev(m)
    y = gdn.moe_gemm_q4(**d)
    torch.cuda.synchronize()
    yh = host(y)
    worst = Errors()
    for e in range(len(m.expert_offsets) - 1):
        a, b = int(m.expert_offsets[e]), int(m.expert_offsets[e + 1])
        if b == a:
            continue
        sub_off = np.array([0, b - a])
        ref = grouped_gemm_q4(m.x[a:b], m.codes[e:e + 1], m.scales[e:e + 1], m.biases[e:e + 1], sub_off)
        worst = worst.merge(seq_errors(yh[a:b, None, :], ref[:, None, :]))
    print(f"moe full size, all 256 experts: {worst}", flush=True)
    assert worst.ok("bf16"), worst


def test_moe_gemm_empty_batch():
    m = make_moe(16, num_experts=4, top_k=1, k=128, n=128, seed=1)
    d = dev(m)
    x0 = d["x"][:0]
    off0 = torch.zeros(5, dtype=torch.int32, device="cuda")
    y = gdn.moe_gemm_q4(x0, off0, d["codes"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def pack_reference(codes):
    """The packed code layout by reshapes: 1 KiB block (e, t, u) holds, at lane
    16 g + c, bytes 64 u + 16 g .. + 15 of row 16 t + c of expert e."""
    E, N, KB = codes.shape
    t = codes.reshape(E, N // 16, 16, 2 * KB // 128, 4, 16)  # [e, t, c, u, g, byte]
    return np.ascontiguousarray(t.transpose(0, 1, 3, 4, 2, 5)).reshape(E, N, KB)


@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (3, 256, 384), (2, 128, 2048)])
def test_pack_layout(E, N, K):
    codes = np.random.default_rng(E * 1000 + K).integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    packed = gdn.moe_pack_q4(torch.from_numpy(codes).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(packed), pack_reference(codes))


@pytest.mark.parametrize("tokens,E,top_k,k,n", [
    (64, 8, 2, 256, 256),
    (300, 16, 4, 384, 128),
    (16, 64, 1, 128, 256),          # most experts empty
    (2048, 256, 8, 2048, 1024),     # the bench shape
])
def test_packed_gemm_equals_unpacked(tokens, E, top_k, k, n):
    # the packed layout changes where the codes are read from, not the arithmetic
    m = make_moe(tokens, num_experts=E, top_k=top_k, k=k, n=n, seed=7 * tokens + E)
    d = dev(m)
    y = gdn.moe_gemm_q4(**d)
    packed = gdn.moe_pack_q4(d["codes"])
    y2 = gdn.moe_gemm_q4_packed(d["x"], d["expert_offsets"], packed, d["scales"], d["biases"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
