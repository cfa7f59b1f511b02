"""GPU parity: the HIP kernels behind the C ABI against the fp64 oracle.

Every test calls libgdn.so through the Python binding and compares with the
oracle on the same seeded inputs, per (sequence, value head) slice, on three
measures (metrics.py): relative Frobenius error within 1e-5 (fp32 inputs) or
3e-3 (bf16 inputs, fp32 state), the largest elementwise error against the
slice's largest element, and a per-token bound that a single wrong token
cannot pass.  Shapes are those of Perplexity's "Optimizing on-device
inference for Apple Silicon" recurrent layer as configured here (16
query/key heads shared by 32 value heads, d = 128, chunk 64), plus small
shapes that span several chunks and ragged tails.  At the long and ragged
workloads every head and sequence is compared, with the oracle spread over
the host's cores (oracle_pool.py).
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import (decode_1000_steps, make_decode, make_prefill, prefill_4096, prefill_131072,
                                                     ragged_32_then_decode, tiny_fp32_prefill)
from oracle import gated_delta_decode_step, gated_delta_recurrence

from helpers import TOL, Errors, dev_prefill, f32, host, max_rel_out, max_rel_state, out_errors, state_errors, torch_io
from oracle_pool import check_prefill_item, host_workers, pool_map

pytestmark = pytest.mark.gpu

PREFILL = {"scan": gdn.prefill_scan, "chunked": gdn.prefill_chunked}


def run_prefill(kind, d, chunk=64, **kw):
    if kind == "chunked":
        return gdn.prefill_chunked(**d, chunk_size=chunk, **kw)
    return gdn.prefill_scan(**d, **kw)


def check_prefill(inp, kind, chunk=None, tol=None):
    d = dev_prefill(inp)
    o, s = run_prefill(kind, d, chunk or inp.chunk_size)
    torch.cuda.synchronize()
    o_ref, s_ref = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.state_in)
    eo, es = out_errors(host(o), o_ref, inp.cu_seqlens), state_errors(host(s), s_ref)
    print(f"{kind} chunk={chunk} out: {eo}; state: {es}", flush=True)
    if tol is None:
        assert eo.ok(inp.io_dtype) and es.ok(inp.io_dtype), (eo, es)
    else:
        assert eo.frob <= tol and es.frob <= tol, (eo, es)
    return eo, es


# ---------------------------------------------------------------- small shapes first
@pytest.mark.parametrize("kind", ["scan", "chunked"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_small_single_sequence(kind, io):
    inp = make_prefill([150], 2, 4, 32, 32, io, 2.0, 0.3, seed=21, chunk_size=32)
    check_prefill(inp, kind, 32)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
def test_chunked_sizes(chunk, dk, dv):
    inp = make_prefill([chunk * 3 + 5], 2, 4, dk, dv, "f32", 0.0, 0.5, seed=dk + dv + chunk)
    check_prefill(inp, "chunked", chunk)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
def test_scan_sizes(dk, dv):
    inp = make_prefill([77], 2, 4, dk, dv, "f32", 0.0, 0.5, seed=dk * dv)
    check_prefill(inp, "scan")


@pytest.mark.parametrize("kind", ["scan", "chunked"])
def test_ragged_tails_and_empty(kind):
    lens = [1, 15, 16, 17, 0, 63, 64, 65, 130, 0]
    inp = make_prefill(lens, 2, 4, 64, 64, "bf16", 2.0, 0.05, seed=5)
    check_prefill(inp, kind, 64)
    d = dev_prefill(inp)
    _, s = run_prefill(kind, d, 64)
    torch.cuda.synchronize()
    # zero-length sequences pass their state through unchanged
    for n in (4, 9):
        assert torch.equal(s[n], d["state_in"][n])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("h_qk,h_v", [(2, 2), (2, 6), (1, 4), (2, 16)])
def test_chunked_group_sizes(h_qk, h_v, io):
    # 1, 3, 4 and 8 value heads per query/key head: every value head of a
    # group reads its query/key head's rows and fragments
    args = ("f32", 0.0, 0.5) if io == "f32" else ("bf16", 2.0, 0.05)
    inp = make_prefill([200, 70], h_qk, h_v, 64, 64, *args, seed=70 + h_v)
    check_prefill(inp, "chunked", 64)


# ---------------------------------------------------------------- the named workloads
def test_tiny_fp32():
    inp = tiny_fp32_prefill()
    check_prefill(inp, "chunked", 16)
    check_prefill(inp, "scan")


def test_decode_1000_steps():
    dec = decode_1000_steps()
    steps = dec.q.shape[0]
    state = f32(dec.state)
    outs = []
    q, k, v = (torch_io(x, "bf16") for x in (dec.q, dec.k, dec.v))
    g, beta = f32(dec.g), f32(dec.beta)
    for t in range(steps):
        o, state = gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], state, state_out=state)
        outs.append(o)
    torch.cuda.synchronize()
    o_gpu = host(torch.stack(outs))  # [steps, 1, Hv, dv]
    S = dec.state.astype(np.float64)
    o_ref = np.zeros(o_gpu.shape)
    for t in range(steps):
        o_ref[t], S = gated_delta_decode_step(dec.q[t], dec.k[t], dec.v[t], dec.g[t], dec.beta[t], S)
    eo = out_errors(o_gpu[:, 0], o_ref[:, 0], [0, steps])
    es = state_errors(host(state), S)
    print(f"decode 1000 steps out: {eo}; state: {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16"), (eo, es)


@pytest.mark.parametrize("kind", ["chunked", "scan"])
def test_prefill_4096(kind):
    check_prefill(prefill_4096(), kind, 64)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def test_long_prefill_131072_all_heads():
    """T = 131072: the chunked kernel over all 32 value heads, and the oracle
    on every head (one item per query/key head and its two value heads, in a
    pool of host processes): all tokens and the final state."""
    inp = prefill_131072()
    d = dev_prefill(inp)
    o, s = gdn.prefill_chunked(**d, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    o_h, s_h = o.float().cpu().numpy(), s.cpu().numpy()
    del d, o, s
    G = inp.v.shape[1] // inp.q.shape[1]

    def items():
        for j in range(inp.q.shape[1]):
            hs = slice(G * j, G * j + G)
            yield {"q": _f32(inp.q[:, j:j + 1]), "k": _f32(inp.k[:, j:j + 1]), "v": _f32(inp.v[:, hs]),
                   "g": _f32(inp.g[:, hs]), "beta": _f32(inp.beta[:, hs]), "o": _f32(o_h[:, hs]),
                   "s": _f32(s_h[:, hs]), "tag": f"heads {G * j}-{G * j + G - 1}"}

    print(f"oracle on {host_workers()} host processes", flush=True)
    eo, es = Errors(), Errors()
    for res in pool_map(check_prefill_item, items()):
        print(f"T=131072 {res['tag']}: out {res['out']}; state {res['state']}", flush=True)
        eo, es = eo.merge(res["out"]), es.merge(res["state"])
    print(f"T=131072 all heads: out {eo}; state {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16"), (eo, es)


@pytest.mark.parametrize("kind", ["chunked", "scan"])
def test_ragged_32_then_decode(kind):
    """32 ragged sequences with their own initial state, then 256 decode
    steps at B=32 carried from the prefill state.  The oracle runs on every
    sequence, all heads, the prefill and all 256 decode steps (one item per
    sequence in a pool of host processes)."""
    pre, dec = ragged_32_then_decode()
    d = dev_prefill(pre)
    o, s = run_prefill(kind, d, 64)
    steps = dec.q.shape[0]
    q, k, v = (torch_io(x, "bf16") for x in (dec.q, dec.k, dec.v))
    g, beta = f32(dec.g), f32(dec.beta)
    state = s.clone()
    outs = []
    for t in range(steps):
        od, state = gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], state, state_out=state)
        outs.append(od)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs).float().cpu().numpy()
    o_h, s_h, sd_h = o.float().cpu().numpy(), s.cpu().numpy(), state.cpu().numpy()
    cu = pre.cu_seqlens

    def items():
        for n in range(len(cu) - 1):
            a, b = int(cu[n]), int(cu[n + 1])
            yield {"q": _f32(pre.q[a:b]), "k": _f32(pre.k[a:b]), "v": _f32(pre.v[a:b]), "g": _f32(pre.g[a:b]),
                   "beta": _f32(pre.beta[a:b]), "state_in": _f32(pre.state_in[n:n + 1]), "o": _f32(o_h[a:b]),
                   "s": _f32(s_h[n:n + 1]), "tag": f"seq {n} (len {b - a})",
                   "dec": {"q": _f32(dec.q[:, n:n + 1]), "k": _f32(dec.k[:, n:n + 1]), "v": _f32(dec.v[:, n:n + 1]),
                           "g": _f32(dec.g[:, n:n + 1]), "beta": _f32(dec.beta[:, n:n + 1]),
                           "o": _f32(o_dec[:, n]), "s": _f32(sd_h[n:n + 1])}}

    worst = {key: Errors() for key in ("out", "state", "dec_out", "dec_state")}
    for res in pool_map(check_prefill_item, items()):
        print(f"{kind} {res['tag']}: prefill out {res['out']}; state {res['state']}; "
              f"decode out {res['dec_out']}; state {res['dec_state']}"
              + (f"; wrong: {res['bad_tokens']}" if "bad_tokens" in res else ""), flush=True)
        for key in worst:
            worst[key] = worst[key].merge(res[key])
    print(f"{kind} all 32 sequences: " + "; ".join(f"{key} {e}" for key, e in worst.items()), flush=True)
    assert all(e.ok("bf16") for e in worst.values()), worst


# ---------------------------------------------------------------- properties
@pytest.mark.parametrize("kind", ["scan", "chunked"])
def test_delta_invariant_q_equals_k(kind):
    """beta = 1, unit keys, q = k: each output is exactly the written value."""
    inp = make_prefill([100], 2, 2, 64, 64, "f32", 0.0, 0.5, seed=31)
    inp.q = inp.k.copy()
    inp.beta = np.ones_like(inp.beta)
    d = dev_prefill(inp)
    o, _ = run_prefill(kind, d, 32)
    torch.cuda.synchronize()
    err = np.max(np.abs(host(o) - inp.v)) / np.max(np.abs(inp.v))
    print(f"{kind} q=k beta=1: max err {err:.3e}", flush=True)
    assert err < 1e-5


@pytest.mark.parametrize("kind", ["scan", "chunked", "decode"])
def test_constancy_beta0_alpha1(kind):
    inp = make_prefill([40], 2, 4, 32, 32, "f32", 0.0, 0.5, seed=41)
    inp.beta[:] = 0
    inp.g[:] = 0
    d = dev_prefill(inp)
    if kind == "decode":
        st = d["state_in"].expand(1, -1, -1, -1).contiguous()
        _, s = gdn.decode_step(d["q"][:1], d["k"][:1], d["v"][:1], d["g"][:1], d["beta"][:1], st)
    else:
        _, s = run_prefill(kind, d, 16)
    torch.cuda.synchronize()
    assert torch.equal(s, d["state_in"])


@pytest.mark.parametrize("kind", ["scan", "chunked"])
def test_split_and_carry(kind):
    """Running T tokens at once equals running T1, then T - T1 from the carried state."""
    inp = make_prefill([200], 2, 4, 64, 64, "bf16", 2.0, 0.05, seed=51)
    d = dev_prefill(inp)
    o, s = run_prefill(kind, d, 64)
    cut = 77
    d1 = {kk: (vv[:cut] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in d.items()}
    d1["cu_seqlens"] = torch.tensor([0, cut], dtype=torch.int32, device="cuda")
    o1, s1 = run_prefill(kind, d1, 64)
    d2 = {kk: (vv[cut:].contiguous() if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in d.items()}
    d2["cu_seqlens"] = torch.tensor([0, 200 - cut], dtype=torch.int32, device="cuda")
    d2["state_in"] = s1
    o2, s2 = run_prefill(kind, d2, 64)
    torch.cuda.synchronize()
    eo = max_rel_out(host(torch.cat([o1, o2])), host(o), [0, 200])
    es = max_rel_state(host(s2), host(s))
    print(f"{kind} split/carry: out {eo:.3e} state {es:.3e}", flush=True)
    assert eo < 2e-3 and es < 1e-4


@pytest.mark.parametrize("kind", ["scan", "chunked"])
def test_deterministic_and_in_place(kind):
    inp = make_prefill([300, 45], 2, 4, 128, 128, "bf16", 2.0, 0.05, seed=61)
    d = dev_prefill(inp)
    o1, s1 = run_prefill(kind, d, 64)
    o2, s2 = run_prefill(kind, d, 64)
    st = d["state_in"].clone()
    d3 = dict(d, state_in=st)
    o3, s3 = run_prefill(kind, d3, 64, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)


def test_decode_in_place_and_batch_equivalence():
    dec = make_decode(3, 5, 2, 4, 64, 128, "bf16", 0.0, 0.1, seed=71)
    q, k, v = (torch_io(x, "bf16") for x in (dec.q, dec.k, dec.v))
    g, beta = f32(dec.g), f32(dec.beta)
    s0 = f32(dec.state)
    o_a, s_a = gdn.decode_step(q[0], k[0], v[0], g[0], beta[0], s0)
    s_in = s0.clone()
    o_b, s_b = gdn.decode_step(q[0], k[0], v[0], g[0], beta[0], s_in, state_out=s_in)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)
    # decode steps == prefill over the same tokens
    pre_q, pre_k, pre_v = q[:, 2].contiguous(), k[:, 2].contiguous(), v[:, 2].contiguous()
    cu = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    o_p, s_p = gdn.prefill_scan(pre_q, pre_k, pre_v, g[:, 2].contiguous(), beta[:, 2].contiguous(), cu,
                                s0[2:3].contiguous())
    st = s0.clone()
    outs = []
    for t in range(3):
        o, st = gdn.decode_step(q[t], k[t], v[t], g[t], beta[t], st, state_out=st)
        outs.append(o[2])
    torch.cuda.synchronize()
    assert max_rel_out(host(torch.stack(outs)), host(o_p), [0, 3]) < TOL["bf16"]
    assert max_rel_state(host(st[2:3]), host(s_p)) < 1e-5
