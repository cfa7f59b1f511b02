"""GPU parity of decode attention over a grouped-query KV cache
(gdn_attention_decode) against the fp64 oracle.

Perplexity's "Optimizing on-device inference for Apple Silicon", sections
"Pack query heads to reuse KV rows" and "Switch attention layouts at long
contexts": query heads of one group share a KV head (16 query and 2 KV heads,
256 values per head in the model described there); packing query heads into
one workgroup gives identical output bytes; the fixed-block layout splits the
cache into equal parts for contexts of 32K and more.  Checks:

- every (sequence, query head) output against the oracle, relative Frobenius
  3e-3 (bf16 output; scores and sums in fp32), for both layouts, every pack
  size, head sizes 64 / 128 / 256, group sizes 1 to 16, ragged and empty
  contexts, more parts than positions;
- packed and unpacked launches give the same bytes, for both layouts;
- positions past a context are never read (NaN there changes nothing);
- the hand-worked fixture (its keys rounded to bf16) and the pages' long
  contexts, 32K and 128K positions, on every head.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import attention_device, make_attention, round_to_bf16
from oracle import decode_attention

from helpers import TOL, seq_errors, host

pytestmark = pytest.mark.gpu


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def dev(inp):
    return (bf(inp.q), bf(inp.k_cache), bf(inp.v_cache),
            torch.from_numpy(np.asarray(inp.context_lens, dtype=np.int32)).cuda())


def max_rel_heads(o, ref):
    """Largest relative Frobenius error over (sequence, head) rows; rows whose
    reference is zero must be exactly zero."""
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            den = np.linalg.norm(ref[b, h])
            err = np.linalg.norm(o[b, h] - ref[b, h])
            if den == 0:
                assert err == 0, (b, h)
            else:
                worst = max(worst, err / den)
    return worst


CASES = [
    # lens, h_q, h_kv, d, max_context
    ([1000], 16, 2, 256, None),
    ([1, 700, 0, 1500], 16, 2, 256, 1600),
    ([33, 257, 1024], 8, 2, 128, None),
    ([500, 17], 4, 4, 64, 600),          # one query head per KV head
    ([900], 16, 1, 128, None),           # a group of 16: two packs of 8
    ([300, 301], 12, 2, 256, None),      # a group of 6: packs of 2
]


@pytest.mark.parametrize("lens,h_q,h_kv,d,T", CASES)
@pytest.mark.parametrize("layout,nb", [("general", 0), ("fixed_block", 0), ("fixed_block", 3), ("fixed_block", 64)])
def test_attention_parity(lens, h_q, h_kv, d, T, layout, nb):
    inp = make_attention(lens, h_q, h_kv, d, T, seed=sum(lens) + d)
    q, k, v, cl = dev(inp)
    T_max = k.shape[2]
    nb = min(nb, T_max)
    o = gdn.attention_decode(q, k, v, cl, inp.scale, layout=layout, num_blocks=nb)
    torch.cuda.synchronize()
    ref = decode_attention(inp.q, inp.k_cache, inp.v_cache, inp.context_lens, inp.scale)
    err = max_rel_heads(host(o), ref)
    print(f"attention lens={lens} h_q={h_q} h_kv={h_kv} d={d} {layout} nb={nb}: err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("layout", ["general", "fixed_block"])
def test_attention_packing_same_bytes(layout):
    inp = make_attention([777, 64, 1], 16, 2, 256, None, seed=3)
    q, k, v, cl = dev(inp)
    outs = [gdn.attention_decode(q, k, v, cl, inp.scale, layout=layout, heads_per_group=hp, num_blocks=8)
            for hp in (1, 2, 4, 8)]
    torch.cuda.synchronize()
    for hp, o in zip((2, 4, 8), outs[1:]):
        assert torch.equal(o, outs[0]), hp


def test_attention_layouts_agree_and_auto():
    inp = make_attention([4096, 2500], 16, 2, 256, None, seed=4)
    q, k, v, cl = dev(inp)
    ref = decode_attention(inp.q, inp.k_cache, inp.v_cache, inp.context_lens, inp.scale)
    for layout, nb in [("general", 0), ("fixed_block", 1), ("fixed_block", 16), ("fixed_block", 256), ("auto", 0)]:
        o = gdn.attention_decode(q, k, v, cl, inp.scale, layout=layout, num_blocks=nb)
        torch.cuda.synchronize()
        err = max_rel_heads(host(o), ref)
        print(f"attention 4096 {layout} nb={nb}: err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]


def test_attention_positions_past_context_not_read():
    inp = make_attention([100, 37], 8, 2, 128, 256, seed=5)
    q, k, v, cl = dev(inp)
    o1 = gdn.attention_decode(q, k, v, cl, inp.scale, layout="fixed_block", num_blocks=4)
    o2 = gdn.attention_decode(q, k, v, cl, inp.scale, layout="general")
    k2, v2 = k.clone(), v.clone()
    for b, n in enumerate((100, 37)):
        k2[b, :, n:] = float("nan")
        v2[b, :, n:] = float("inf")
    o3 = gdn.attention_decode(q, k2, v2, cl, inp.scale, layout="fixed_block", num_blocks=4)
    o4 = gdn.attention_decode(q, k2, v2, cl, inp.scale, layout="general")
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(o2, o4)


def test_attention_empty_and_single_position():
    inp = make_attention([0, 1, 0], 16, 2, 256, 64, seed=6)
    q, k, v, cl = dev(inp)
    for layout in ("general", "fixed_block"):
        o = gdn.attention_decode(q, k, v, cl, inp.scale, layout=layout)
        torch.cuda.synchronize()
        oh = host(o)
        assert np.all(oh[0] == 0) and np.all(oh[2] == 0)
        # one position: the weight is exactly 1, so the output is that position's value (already bf16)
        np.testing.assert_array_equal(oh[1], np.repeat(inp.v_cache[1, :, 0], 8, axis=0))


def test_attention_sharp_scores():
    # scale 4 makes the scores span hundreds: only the running maximum keeps exp in range
    inp = make_attention([2000], 16, 2, 256, None, seed=7)
    q, k, v, cl = dev(inp)
    for layout in ("general", "fixed_block"):
        o = gdn.attention_decode(q, k, v, cl, 4.0, layout=layout)
        torch.cuda.synchronize()
        ref = decode_attention(inp.q, inp.k_cache, inp.v_cache, inp.context_lens, 4.0)
        err = max_rel_heads(host(o), ref)
        print(f"attention sharp {layout}: err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]


def test_attention_golden_fixture():
    # the hand-worked case in the first two of 64 columns; the fixture's keys
    # are logs, which bf16 cannot hold, so the reference is the oracle on the
    # rounded keys and the fixture's exact values are met to bf16 accuracy
    from test_oracle import load_attention_fixture
    f = load_attention_fixture()
    d = 64
    q = np.zeros((2, 4, d))
    k = np.zeros((2, 2, 3, d))
    v = np.zeros((2, 2, 3, d))
    q[..., :2], k[..., :2], v[..., :2] = f["q"], round_to_bf16(f["k"].astype(np.float32)), f["v"]
    cl = torch.tensor(f["lens"], dtype=torch.int32).cuda()
    for layout in ("general", "fixed_block"):
        o = gdn.attention_decode(bf(q), bf(k), bf(v), cl, f["scale"], layout=layout, heads_per_group=1)
        torch.cuda.synchronize()
        oh = host(o)
        ref = decode_attention(q, k, v, f["lens"], f["scale"])
        assert max_rel_heads(oh, ref) <= TOL["bf16"]
        np.testing.assert_allclose(oh[..., :2], f["out"], rtol=2e-2, atol=2e-2)
        assert np.all(oh[..., 2:] == 0)


@pytest.mark.parametrize("T,layout", [(32768, "general"), (32768, "auto"), (131072, "auto")])
def test_attention_long_context_all_heads(T, layout):
    # the pages' shape at their long contexts: 16 query heads on 2 KV heads,
    # 256 values; the oracle on every query head, each output row checked on
    # the three measures (the 16 heads' output rows taken as the rows of one slice)
    q, k, v, cl, scale = attention_device([T], seed=T)
    o = gdn.attention_decode(q, k, v, cl, scale, layout=layout)
    torch.cuda.synchronize()
    oh = host(o)
    ref = decode_attention(host(q), host(k), host(v), np.array([T]), scale)
    err = max_rel_heads(oh, ref)
    e = seq_errors(oh[0][:, None, :], ref[0][:, None, :])
    print(f"attention T={T} {layout} all 16 heads: frob {err:.3e}; {e}", flush=True)
    assert err <= TOL["bf16"] and e.ok("bf16"), (err, e)


def test_attention_context_lengths_clamped():
    # context lengths are clamped on the device to [0, max_context]: a negative
    # one reads nothing (zero output), one past the cache reads the whole cache
    inp = make_attention([300, 300], 8, 2, 128, 300, seed=8)
    q, k, v, _ = dev(inp)
    for layout in ("general", "fixed_block"):
        o_bad = gdn.attention_decode(q, k, v, torch.tensor([-5, 10**6], dtype=torch.int32, device="cuda"),
                                     inp.scale, layout=layout)
        o_ref = gdn.attention_decode(q, k, v, torch.tensor([0, 300], dtype=torch.int32, device="cuda"),
                                     inp.scale, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(o_bad, o_ref)
        assert bool((o_bad[0] == 0).all())
