"""Entry points called on a side stream (the binding's `stream` argument).

The binding allocates workspaces and default outputs on the stream the
kernels run on, so the caching allocator cannot hand their memory to other
work while the kernels still read it.  Each case launches on a side stream
with an internally allocated workspace, at once fills fresh allocations of
the same size on the current stream, and compares the result, after the side
stream is synchronised, with the same call on the current stream, bit for
bit.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import attention_device, make_prefill

from helpers import dev_prefill

pytestmark = pytest.mark.gpu


def _scribble(nbytes):
    # allocations on the current stream while the side stream still runs
    bufs = [torch.full((nbytes // 4 + 64,), float("nan"), device="cuda") for _ in range(3)]
    return bufs


@pytest.mark.parametrize("kind", ["chunked", "segmented"])
def test_prefill_on_side_stream(kind):
    inp = make_prefill([3000, 500, 1], 16, 32, 128, 128, "bf16", 2.0, 0.02, seed=81)
    d = dev_prefill(inp)
    call = (lambda **kw: gdn.prefill_chunked(**d, chunk_size=64, **kw)) if kind == "chunked" else \
        (lambda **kw: gdn.prefill_segmented(**d, chunk_size=64, segment_tokens=1024, **kw))
    o_ref, s_ref = call()
    torch.cuda.synchronize()
    need = gdn.chunked_workspace_bytes(3, 3501, 16, 32, 128, 128)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o, s = call(stream=side)
        junk = _scribble(need)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        del junk


def test_attention_on_side_stream():
    q, k, v, cl, scale = attention_device([20000, 7000], seed=9)
    o_ref = gdn.attention_decode(q, k, v, cl, scale, layout="fixed_block")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = gdn.attention_decode_workspace_bytes(2, 16, 2, 256, int(k.shape[2]), scale, "fixed_block")
    for _ in range(3):
        o = gdn.attention_decode(q, k, v, cl, scale, layout="fixed_block", stream=side)
        junk = _scribble(max(need, 1 << 20))
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        del junk
    assert np.isfinite(o.float().cpu().numpy()).all()
