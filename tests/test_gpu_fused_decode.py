"""GPU parity of the fused decode step (gdn_decode_step_fused) against the
fp64 oracle's gated_delta_decode_fused.

The step folds the q/k L2 normalisation, the gate and beta activations and a
per-head RMS norm of the output into the recurrent update, the fusion that
Perplexity's "Optimizing on-device inference for Apple Silicon" describes in
section "Reduce state and intermediate traffic".  Errors are per (sequence,
value head) slice, relative Frobenius: 1e-5 for fp32 inputs, 3e-3 for bf16.
Shapes cover the 16/32-head d = 128 layer at batch 1 and 32 (one workgroup
per head; the step has one shape below 512 workgroups and another from 512
on, both covered), the small sizes (workgroups padded to a full wave) and
every d_k.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import make_decode_raw
from oracle import gated_delta_decode_fused

from helpers import f32, host, out_errors, state_errors, torch_io

pytestmark = pytest.mark.gpu


def dev(r, with_params=True):
    d = dict(q_raw=torch_io(r.q_raw, r.io_dtype), k_raw=torch_io(r.k_raw, r.io_dtype), v=torch_io(r.v, r.io_dtype),
             g_raw=f32(r.g_raw), beta_raw=f32(r.beta_raw), state_in=f32(r.state))
    if with_params:
        d.update(gate_bias=f32(r.gate_bias), gate_scale=f32(r.gate_scale), norm_weight=f32(r.norm_weight))
    return d


def oracle(r, with_params=True, **eps):
    kw = dict(gate_bias=r.gate_bias, gate_scale=r.gate_scale, norm_weight=r.norm_weight) if with_params else {}
    return gated_delta_decode_fused(r.q_raw, r.k_raw, r.v, r.g_raw, r.beta_raw, r.state, **kw, **eps)


def errors(o, s, o_ref, s_ref):
    B = o_ref.shape[0]
    return out_errors(host(o), o_ref, np.arange(B + 1)), state_errors(host(s), s_ref)


@pytest.mark.parametrize("B,h_qk,h_v,d_k,d_v,io", [
    (1, 16, 32, 128, 128, "bf16"),
    (32, 16, 32, 128, 128, "bf16"),
    (3, 2, 4, 16, 16, "f32"),
    (2, 2, 4, 32, 64, "f32"),
    (4, 1, 2, 64, 128, "f32"),
    (2, 4, 4, 128, 32, "f32"),
    (5, 2, 4, 128, 128, "f32"),
    (128, 2, 4, 64, 64, "f32"),   # 512 workgroups and more: the large-batch shape at smaller d_k
    (256, 1, 2, 32, 128, "f32"),
])
def test_fused_decode_parity(B, h_qk, h_v, d_k, d_v, io):
    r = make_decode_raw(B, h_qk, h_v, d_k, d_v, io, state_std=0.1, seed=300 + B + d_k + d_v)
    o, s = gdn.decode_step_fused(**dev(r), qk_eps=1e-6, norm_eps=1e-5)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(r, qk_eps=1e-6, norm_eps=1e-5)
    eo, es = errors(o, s, o_ref, s_ref)
    print(f"fused decode B={B} {h_qk}/{h_v} d={d_k}/{d_v} {io}: out {eo}; state {es}", flush=True)
    assert eo.ok(io) and es.ok(io), (eo, es)


def test_fused_decode_defaults_and_in_place():
    r = make_decode_raw(4, 16, 32, 128, 128, "bf16", state_std=0.05, seed=411)
    d = dev(r, with_params=False)
    o, s = gdn.decode_step_fused(**d)  # params NULL: no bias, no scale, no weight, eps 1e-6
    s_in = d["state_in"].clone()
    o2, s2 = gdn.decode_step_fused(**dict(d, state_in=s_in), state_out=s_in)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)
    o_ref, s_ref = oracle(r, with_params=False)
    eo, es = errors(o, s, o_ref, s_ref)
    print(f"fused decode defaults: out {eo}; state {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16"), (eo, es)


def test_fused_decode_64_carried_steps():
    # the state carried through 64 fused steps at batch 2 stays within tolerance
    rng = np.random.default_rng(77)
    r0 = make_decode_raw(2, 16, 32, 128, 128, "bf16", state_std=0.02, rng=rng)
    state = f32(r0.state)
    S = r0.state.astype(np.float64)
    params = dict(gate_bias=f32(r0.gate_bias), gate_scale=f32(r0.gate_scale), norm_weight=f32(r0.norm_weight))
    outs, refs = [], []
    for _ in range(64):
        r = make_decode_raw(2, 16, 32, 128, 128, "bf16", state_std=0.0, rng=rng)
        o, state = gdn.decode_step_fused(torch_io(r.q_raw, "bf16"), torch_io(r.k_raw, "bf16"), torch_io(r.v, "bf16"),
                                         f32(r.g_raw), f32(r.beta_raw), state, state_out=state, **params)
        outs.append(o)
        o_ref, S = gated_delta_decode_fused(r.q_raw, r.k_raw, r.v, r.g_raw, r.beta_raw, S, gate_bias=r0.gate_bias,
                                            gate_scale=r0.gate_scale, norm_weight=r0.norm_weight)
        refs.append(o_ref)
    torch.cuda.synchronize()
    o_gpu, o_ref = host(torch.stack(outs)), np.stack(refs)  # [64, 2, 32, 128]
    eo = out_errors(o_gpu[:, 0], o_ref[:, 0], [0, 64]).merge(out_errors(o_gpu[:, 1], o_ref[:, 1], [0, 64]))
    es = state_errors(host(state), S)
    print(f"fused decode 64 steps: out {eo}; state {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16"), (eo, es)


def test_fused_decode_extreme_gates():
    # softplus past its cut-over (g_raw + bias > 20: alpha ~ 0) and far below it (alpha ~ 1); beta at both ends
    r = make_decode_raw(2, 2, 4, 64, 64, "f32", state_std=0.5, seed=5)
    r.g_raw[0] = np.array([30.0, 19.5, -30.0, 0.0], np.float32)
    r.beta_raw[0] = np.array([40.0, -40.0, 0.0, 3.0], np.float32)
    o, s = gdn.decode_step_fused(**dev(r))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(r)
    eo, es = errors(o, s, o_ref, s_ref)
    print(f"fused decode extreme gates: out {eo}; state {es}", flush=True)
    assert eo.ok("f32") and es.ok("f32"), (eo, es)
