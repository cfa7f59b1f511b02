"""Shared test helpers: moving generated inputs to the GPU (the error
measures live in metrics.py)."""
import numpy as np
import torch

from metrics import (TOL, TOL_MAX, TOL_TOK, Errors, max_rel_out, max_rel_state, out_errors,  # noqa: F401
                     seq_errors, state_errors)


def torch_io(x: np.ndarray, io_dtype: str, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if io_dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are bf16-representable
    return t.to(device)


def f32(x: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def dev_prefill(inp, device="cuda"):
    return dict(
        q=torch_io(inp.q, inp.io_dtype, device),
        k=torch_io(inp.k, inp.io_dtype, device),
        v=torch_io(inp.v, inp.io_dtype, device),
        g=f32(inp.g, device),
        beta=f32(inp.beta, device),
        cu_seqlens=torch.from_numpy(np.asarray(inp.cu_seqlens, dtype=np.int32)).to(device),
        state_in=None if inp.state_in is None else f32(inp.state_in, device),
    )


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
