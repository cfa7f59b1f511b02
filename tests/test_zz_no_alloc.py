"""The allocation-free segmented prefill (gdn_prefill_segmented_noalloc).

It runs the kernels of gdn_prefill_segmented with the workspace in the
library's static device scratch, so its results must equal that entry point's
bit for bit.  Two calls in a row, the second with a smaller input, check that
what the first call leaves in the shared scratch does not leak into the
second.  Sizes beyond the scratch are refused on the host.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import make_prefill

from helpers import dev_prefill, host, out_errors, state_errors
from oracle import gated_delta_recurrence

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk,L", [(64, 1024), (64, 2048), (32, 512), (0, 1000)])
def test_noalloc_equals_segmented_two_calls(chunk, L):
    first = make_prefill([1000, 3000, 77], 16, 32, 128, 128, "bf16", 2.0, 0.02, seed=91)
    second = make_prefill([500, 90], 16, 32, 128, 128, "bf16", 2.0, 0.02, seed=92)
    for inp in (first, second):
        d = dev_prefill(inp)
        o_ref, s_ref = gdn.prefill_segmented(**d, chunk_size=chunk, segment_tokens=L)
        o, s = gdn.prefill_segmented_noalloc(**d, chunk_size=chunk, segment_tokens=L)
        torch.cuda.synchronize()
        print(f"noalloc chunk={chunk} L={L} T={inp.q.shape[0]}: equal out {torch.equal(o, o_ref)}, "
              f"state {torch.equal(s, s_ref)}", flush=True)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    # and the second call against the oracle
    r_o, r_s = gated_delta_recurrence(second.q, second.k, second.v, second.g, second.beta, second.cu_seqlens,
                                      second.state_in)
    eo, es = out_errors(host(o), r_o, second.cu_seqlens), state_errors(host(s), r_s)
    print(f"noalloc vs oracle: out {eo}; state {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16")


def test_noalloc_refuses_segments_beyond_the_scratch():
    inp = make_prefill([300], 16, 32, 128, 128, "bf16", 2.0, None, seed=93)
    d = dev_prefill(inp)
    need = gdn.segmented_workspace_bytes(1, 300, 16, 32, 128, 128, gdn.GDN_DTYPE_BF16, 64, 8192)
    # 300 tokens fit any segment; the check uses min(total, segment) tokens
    assert need < gdn.STATIC_SCRATCH_BYTES
    big = make_prefill([6000], 16, 32, 128, 128, "bf16", 2.0, None, seed=94)
    db = dev_prefill(big)
    assert gdn.segmented_workspace_bytes(1, 6000, 16, 32, 128, 128, gdn.GDN_DTYPE_BF16, 64,
                                         4096) > gdn.STATIC_SCRATCH_BYTES
    out = torch.full((6000, 32, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as err:
        gdn.prefill_segmented_noalloc(**db, out=out, chunk_size=64, segment_tokens=4096)
    assert err.value.status == gdn.GDN_ERR_INVALID and "static scratch" in str(err.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was enqueued
    o, _ = gdn.prefill_segmented_noalloc(**d, chunk_size=64, segment_tokens=8192)
    torch.cuda.synchronize()
    assert np.isfinite(host(o)).all()
