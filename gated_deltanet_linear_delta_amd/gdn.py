"""Python binding of libgdn.so: argument marshalling only.

Every function takes torch tensors on the GPU, checks their dtypes, shapes and
contiguity, and passes raw device pointers and the current HIP stream to the
C ABI declared in include/gdn.h.  All arithmetic runs in the library's HIP
kernels; there is no fallback.  If libgdn.so is missing or does not load,
every entry point raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GDN_LIB", os.path.join(_PKG, "libgdn.so"))

GDN_OK, GDN_ERR_INVALID, GDN_ERR_UNSUPPORTED, GDN_ERR_LAUNCH = 0, 1, 2, 3
GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
EXPORTS = ("gdn_prefill_scan", "gdn_prefill_scan_blockwise", "gdn_prefill_chunked", "gdn_prefill_chunked_workspace",
           "gdn_prefill_segmented", "gdn_prefill_segmented_workspace", "gdn_prefill_segmented_noalloc",
           "gdn_decode_step", "gdn_decode_step_fused",
           "gdn_moe_gemm_q4", "gdn_moe_pack_q4", "gdn_moe_gemm_q4_packed", "gdn_dequant_q4", "gdn_moe_gemm_bf16", "gdn_attention_decode",
           "gdn_attention_decode_workspace", "gdn_profile_enable", "gdn_profile_collect", "gdn_status_string",
           "gdn_last_error")
GDN_ATTN_AUTO, GDN_ATTN_GENERAL, GDN_ATTN_FIXED_BLOCK = 0, 1, 2
ATTN_LAYOUTS = {"auto": GDN_ATTN_AUTO, "general": GDN_ATTN_GENERAL, "fixed_block": GDN_ATTN_FIXED_BLOCK}


class GdnShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int)]


class GdnFusedParams(ctypes.Structure):
    _fields_ = [("gate_bias", ctypes.c_void_p), ("gate_scale", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("qk_eps", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class GdnMoeShape(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("rows", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n", ctypes.c_int32)]


class GdnAttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_context", ctypes.c_int32)]


class GdnAttnParams(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("layout", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load libgdn.so once and declare its signatures; raises if it is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} not found: build it with `python -m gated_deltanet_linear_delta_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    shp = ctypes.POINTER(GdnShape)
    lib.gdn_prefill_scan.argtypes = [shp, vp, vp, vp, f, f, vp, f, vp, f, vp]
    lib.gdn_prefill_scan.restype = ctypes.c_int
    lib.gdn_prefill_chunked.argtypes = [shp, vp, vp, vp, f, f, vp, f, vp, f, i32, vp, ctypes.c_size_t, vp]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_scan_blockwise.argtypes = [shp, vp, vp, vp, f, f, vp, f, vp, f, i32, vp]
    lib.gdn_prefill_scan_blockwise.restype = ctypes.c_int
    lib.gdn_prefill_segmented.argtypes = [shp, vp, vp, vp, f, f, vp, f, vp, f, i32, i32, vp, ctypes.c_size_t, vp]
    lib.gdn_prefill_segmented.restype = ctypes.c_int
    lib.gdn_prefill_segmented_noalloc.argtypes = [shp, vp, vp, vp, f, f, vp, f, vp, f, i32, i32, vp]
    lib.gdn_prefill_segmented_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_segmented_workspace.argtypes = [shp, i32, i32]
    lib.gdn_prefill_segmented_workspace.restype = ctypes.c_size_t
    lib.gdn_prefill_chunked_workspace.argtypes = [shp, i32]
    lib.gdn_prefill_chunked_workspace.restype = ctypes.c_size_t
    lib.gdn_decode_step.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, vp, vp, vp, f, f, f, vp, f, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step_fused.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, vp, vp, vp, f, f,
                                          ctypes.POINTER(GdnFusedParams), f, vp, f, vp]
    lib.gdn_decode_step_fused.restype = ctypes.c_int
    mshp = ctypes.POINTER(GdnMoeShape)
    lib.gdn_moe_gemm_q4.argtypes = [mshp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_moe_gemm_q4.restype = ctypes.c_int
    lib.gdn_moe_pack_q4.argtypes = [mshp, vp, vp, vp]
    lib.gdn_moe_pack_q4.restype = ctypes.c_int
    lib.gdn_moe_gemm_q4_packed.argtypes = [mshp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_moe_gemm_q4_packed.restype = ctypes.c_int
    lib.gdn_dequant_q4.argtypes = [mshp, vp, vp, vp, vp, vp]
    lib.gdn_dequant_q4.restype = ctypes.c_int
    lib.gdn_moe_gemm_bf16.argtypes = [mshp, vp, vp, vp, vp, vp]
    lib.gdn_moe_gemm_bf16.restype = ctypes.c_int
    ashp, apar = ctypes.POINTER(GdnAttnShape), ctypes.POINTER(GdnAttnParams)
    lib.gdn_attention_decode_workspace.argtypes = [ashp, apar]
    lib.gdn_attention_decode_workspace.restype = ctypes.c_size_t
    lib.gdn_attention_decode.argtypes = [ashp, apar, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_attention_decode.restype = ctypes.c_int
    lib.gdn_profile_enable.argtypes = [ctypes.c_int]
    lib.gdn_profile_enable.restype = ctypes.c_int
    lib.gdn_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                        ctypes.c_int]
    lib.gdn_profile_collect.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != GDN_OK:
        lib = load_library()
        name = lib.gdn_status_string(status).decode()
        raise GdnError(status, f"{name}: {lib.gdn_last_error().decode()}")


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, not {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate on the stream the kernels run on.  torch's caching allocator
    hands a freed block only to later allocations on the stream it was
    allocated on, so a workspace (or output) allocated under `stream` cannot
    be reused by other work while the kernels still read it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in):
    io = _io_dtype(q)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _need(q, "q", q.dtype, (T, h_qk, d_k))
    _need(k, "k", q.dtype, (T, h_qk, d_k))
    _need(v, "v", q.dtype, (T, h_v, d_v))
    _need(g, "g", torch.float32, (T, h_v))
    _need(beta, "beta", torch.float32, (T, h_v))
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (N, h_v, d_v, d_k))
    return GdnShape(N, T, h_qk, h_v, d_k, d_v, io)


def _outputs(shape: GdnShape, like, out, state_out):
    if out is None:
        out = torch.empty((shape.total_tokens, shape.h_v, shape.d_v), dtype=like.dtype, device=like.device)
    else:
        _need(out, "out", like.dtype, (shape.total_tokens, shape.h_v, shape.d_v))
    sshape = (shape.num_seqs, shape.h_v, shape.d_v, shape.d_k)
    if state_out is None:
        state_out = torch.empty(sshape, dtype=torch.float32, device=like.device)
    else:
        _need(state_out, "state_out", torch.float32, sshape)
    return out, state_out


def prefill_scan(q, k, v, g, beta, cu_seqlens, state_in=None, out=None, state_out=None, stream=None):
    """Direct token scan (gdn_prefill_scan).  Returns (out, state_out)."""
    lib = load_library()
    with _on(stream):
        shape = _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in)
        out, state_out = _outputs(shape, q, out, state_out)
        _check(lib.gdn_prefill_scan(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(cu_seqlens), _ptr(state_in), _ptr(out), _ptr(state_out), _stream(stream)))
        return out, state_out


def prefill_scan_blockwise(q, k, v, g, beta, cu_seqlens, state_in=None, out=None, state_out=None, state_block=32,
                           stream=None):
    """The blockwise-scan ablation (gdn_prefill_scan_blockwise): the direct
    scan with its state moved to state_out and back every ``state_block``
    tokens.  Returns (out, state_out)."""
    lib = load_library()
    with _on(stream):
        shape = _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in)
        out, state_out = _outputs(shape, q, out, state_out)
        _check(lib.gdn_prefill_scan_blockwise(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                              _ptr(cu_seqlens), _ptr(state_in), _ptr(out), _ptr(state_out),
                                              int(state_block), _stream(stream)))
        return out, state_out


def chunked_workspace_bytes(num_seqs, total_tokens, h_qk, h_v, d_k, d_v, io_dtype=GDN_DTYPE_BF16, chunk_size=64):
    lib = load_library()
    shape = GdnShape(num_seqs, total_tokens, h_qk, h_v, d_k, d_v, io_dtype)
    return int(lib.gdn_prefill_chunked_workspace(ctypes.byref(shape), chunk_size))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    return torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)


def _aligned_ptr(ws: torch.Tensor):
    p = ws.data_ptr()
    return (p + 255) // 256 * 256, ws.numel() - ((p + 255) // 256 * 256 - p)


def prefill_chunked(q, k, v, g, beta, cu_seqlens, state_in=None, out=None, state_out=None, chunk_size=64,
                    workspace=None, stream=None):
    """Chunked prefill (gdn_prefill_chunked).  Returns (out, state_out).
    ``workspace`` is a uint8 device tensor from alloc_workspace (allocated
    here if None)."""
    lib = load_library()
    with _on(stream):
        shape = _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in)
        out, state_out = _outputs(shape, q, out, state_out)
        need = int(lib.gdn_prefill_chunked_workspace(ctypes.byref(shape), int(chunk_size)))
        if workspace is None:
            workspace = alloc_workspace(need, q.device)
        if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
            raise TypeError("workspace must be a uint8 GPU tensor")
        wp, wn = _aligned_ptr(workspace)
        _check(lib.gdn_prefill_chunked(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(cu_seqlens), _ptr(state_in), _ptr(out), _ptr(state_out), int(chunk_size),
                                       ctypes.c_void_p(wp), ctypes.c_size_t(max(wn, 0)), _stream(stream)))
        return out, state_out


def segmented_workspace_bytes(num_seqs, total_tokens, h_qk, h_v, d_k, d_v, io_dtype=GDN_DTYPE_BF16, chunk_size=64,
                              segment_tokens=8192):
    lib = load_library()
    shape = GdnShape(num_seqs, total_tokens, h_qk, h_v, d_k, d_v, io_dtype)
    return int(lib.gdn_prefill_segmented_workspace(ctypes.byref(shape), int(chunk_size), int(segment_tokens)))


def prefill_segmented(q, k, v, g, beta, cu_seqlens, state_in=None, out=None, state_out=None, chunk_size=64,
                      segment_tokens=8192, workspace=None, stream=None):
    """Prefill in windows of ``segment_tokens`` packed tokens with the state
    carried between them (gdn_prefill_segmented); chunk_size 0 runs the
    direct scan in each window.  Returns (out, state_out)."""
    lib = load_library()
    with _on(stream):
        shape = _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in)
        out, state_out = _outputs(shape, q, out, state_out)
        need = int(lib.gdn_prefill_segmented_workspace(ctypes.byref(shape), int(chunk_size), int(segment_tokens)))
        if workspace is None:
            workspace = alloc_workspace(need, q.device)
        if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
            raise TypeError("workspace must be a uint8 GPU tensor")
        wp, wn = _aligned_ptr(workspace)
        _check(lib.gdn_prefill_segmented(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(cu_seqlens), _ptr(state_in), _ptr(out), _ptr(state_out), int(chunk_size),
                                         int(segment_tokens), ctypes.c_void_p(wp), ctypes.c_size_t(max(wn, 0)),
                                         _stream(stream)))
        return out, state_out


STATIC_SCRATCH_BYTES = 64 << 20  # GDN_STATIC_SCRATCH_BYTES in include/gdn.h


def prefill_segmented_noalloc(q, k, v, g, beta, cu_seqlens, state_in=None, out=None, state_out=None, chunk_size=64,
                              segment_tokens=2048, stream=None):
    """gdn_prefill_segmented with the workspace in the library's static
    device scratch (gdn_prefill_segmented_noalloc): the library allocates
    nothing; out and state_out are allocated here only when not given.
    Returns (out, state_out)."""
    lib = load_library()
    with _on(stream):
        shape = _prefill_shape(q, k, v, g, beta, cu_seqlens, state_in)
        out, state_out = _outputs(shape, q, out, state_out)
        _check(lib.gdn_prefill_segmented_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                                 _ptr(cu_seqlens), _ptr(state_in), _ptr(out), _ptr(state_out),
                                                 int(chunk_size), int(segment_tokens), _stream(stream)))
        return out, state_out


def decode_step(q, k, v, g, beta, state_in, out=None, state_out=None, stream=None):
    """One recurrent step per sequence (gdn_decode_step).  q, k [B, h_qk, d_k];
    v [B, h_v, d_v]; g, beta [B, h_v]; state_in [B, h_v, d_v, d_k].
    ``state_out`` may be ``state_in`` for an in-place update.  Returns
    (out, state_out)."""
    lib = load_library()
    with _on(stream):
        io = _io_dtype(q)
        B, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1], v.shape[2]
        _need(k, "k", q.dtype, (B, h_qk, d_k))
        _need(q, "q", q.dtype, (B, h_qk, d_k))
        _need(v, "v", q.dtype, (B, h_v, d_v))
        _need(g, "g", torch.float32, (B, h_v))
        _need(beta, "beta", torch.float32, (B, h_v))
        _need(state_in, "state_in", torch.float32, (B, h_v, d_v, d_k))
        if out is None:
            out = torch.empty((B, h_v, d_v), dtype=q.dtype, device=q.device)
        else:
            _need(out, "out", q.dtype, (B, h_v, d_v))
        if state_out is None:
            state_out = torch.empty_like(state_in)
        else:
            _need(state_out, "state_out", torch.float32, (B, h_v, d_v, d_k))
        _check(lib.gdn_decode_step(B, h_qk, h_v, d_k, d_v, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(state_in), _ptr(out), _ptr(state_out), _stream(stream)))
        return out, state_out


def decode_step_fused(q_raw, k_raw, v, g_raw, beta_raw, state_in, gate_bias=None, gate_scale=None,
                      norm_weight=None, qk_eps=1e-6, norm_eps=1e-6, out=None, state_out=None, stream=None):
    """Decode step with the q/k L2 norms, the gate and beta activations and
    the per-head RMS output norm in the same kernel (gdn_decode_step_fused).
    q_raw, k_raw [B, h_qk, d_k]; v [B, h_v, d_v]; g_raw, beta_raw [B, h_v];
    state_in [B, h_v, d_v, d_k]; gate_bias, gate_scale [h_v] and norm_weight
    [d_v] fp32 or None.  Returns (out, state_out)."""
    lib = load_library()
    with _on(stream):
        io = _io_dtype(q_raw)
        B, h_qk, d_k = q_raw.shape
        h_v, d_v = v.shape[1], v.shape[2]
        _need(q_raw, "q_raw", q_raw.dtype, (B, h_qk, d_k))
        _need(k_raw, "k_raw", q_raw.dtype, (B, h_qk, d_k))
        _need(v, "v", q_raw.dtype, (B, h_v, d_v))
        _need(g_raw, "g_raw", torch.float32, (B, h_v))
        _need(beta_raw, "beta_raw", torch.float32, (B, h_v))
        _need(state_in, "state_in", torch.float32, (B, h_v, d_v, d_k))
        for t, name, n in ((gate_bias, "gate_bias", h_v), (gate_scale, "gate_scale", h_v),
                           (norm_weight, "norm_weight", d_v)):
            if t is not None:
                _need(t, name, torch.float32, (n,))
        if out is None:
            out = torch.empty((B, h_v, d_v), dtype=q_raw.dtype, device=q_raw.device)
        else:
            _need(out, "out", q_raw.dtype, (B, h_v, d_v))
        if state_out is None:
            state_out = torch.empty_like(state_in)
        else:
            _need(state_out, "state_out", torch.float32, (B, h_v, d_v, d_k))
        params = GdnFusedParams(_ptr(gate_bias), _ptr(gate_scale), _ptr(norm_weight), float(qk_eps), float(norm_eps))
        _check(lib.gdn_decode_step_fused(B, h_qk, h_v, d_k, d_v, io, _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_raw),
                                         _ptr(beta_raw), ctypes.byref(params), _ptr(state_in), _ptr(out),
                                         _ptr(state_out), _stream(stream)))
        return out, state_out


def _moe_shape(x, expert_offsets, codes_or_weights, packed):
    E, N = codes_or_weights.shape[0], codes_or_weights.shape[1]
    K = codes_or_weights.shape[2] * (2 if packed else 1)
    M = x.shape[0]
    _need(x, "x", torch.bfloat16, (M, K))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    return GdnMoeShape(E, M, K, N)


def moe_gemm_q4(x, expert_offsets, codes, scales, biases, y=None, stream=None):
    """Grouped expert GEMM on 4-bit group-affine weights (gdn_moe_gemm_q4).
    x [M, K] bf16 grouped by expert; expert_offsets [E + 1] int32; codes
    [E, N, K / 2] uint8; scales, biases [E, N, K / 64] bf16.  Returns y [M, N]
    bf16."""
    lib = load_library()
    with _on(stream):
        shape = _moe_shape(x, expert_offsets, codes, True)
        E, N, K = shape.num_experts, shape.n, shape.k
        _need(codes, "codes", torch.uint8, (E, N, K // 2))
        _need(scales, "scales", torch.bfloat16, (E, N, K // 64))
        _need(biases, "biases", torch.bfloat16, (E, N, K // 64))
        if y is None:
            y = torch.empty((shape.rows, N), dtype=torch.bfloat16, device=x.device)
        else:
            _need(y, "y", torch.bfloat16, (shape.rows, N))
        _check(lib.gdn_moe_gemm_q4(ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(codes), _ptr(scales),
                                   _ptr(biases), _ptr(y), _stream(stream)))
        return y


def moe_pack_q4(codes, packed=None, stream=None):
    """Codes [E, N, K / 2] uint8 rewritten in the tiled layout that
    moe_gemm_q4_packed reads (gdn_moe_pack_q4); the result has the same shape
    and size, its bytes in the packed order."""
    lib = load_library()
    with _on(stream):
        E, N, K = codes.shape[0], codes.shape[1], codes.shape[2] * 2
        _need(codes, "codes", torch.uint8, (E, N, K // 2))
        if packed is None:
            packed = torch.empty_like(codes)
        else:
            _need(packed, "packed", torch.uint8, (E, N, K // 2))
        shape = GdnMoeShape(E, 0, K, N)
        _check(lib.gdn_moe_pack_q4(ctypes.byref(shape), _ptr(codes), _ptr(packed), _stream(stream)))
        return packed


def moe_gemm_q4_packed(x, expert_offsets, packed_codes, scales, biases, y=None, stream=None):
    """moe_gemm_q4 on codes from moe_pack_q4 (gdn_moe_gemm_q4_packed); the
    same y bit for bit."""
    lib = load_library()
    with _on(stream):
        shape = _moe_shape(x, expert_offsets, packed_codes, True)
        E, N, K = shape.num_experts, shape.n, shape.k
        _need(packed_codes, "packed_codes", torch.uint8, (E, N, K // 2))
        _need(scales, "scales", torch.bfloat16, (E, N, K // 64))
        _need(biases, "biases", torch.bfloat16, (E, N, K // 64))
        if y is None:
            y = torch.empty((shape.rows, N), dtype=torch.bfloat16, device=x.device)
        else:
            _need(y, "y", torch.bfloat16, (shape.rows, N))
        _check(lib.gdn_moe_gemm_q4_packed(ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(packed_codes),
                                          _ptr(scales), _ptr(biases), _ptr(y), _stream(stream)))
        return y


def dequant_q4(codes, scales, biases, weights=None, stream=None):
    """The whole bf16 weight matrix [E, N, K] rebuilt from 4-bit codes
    (gdn_dequant_q4, the ablation's separate pass)."""
    lib = load_library()
    with _on(stream):
        E, N, K = codes.shape[0], codes.shape[1], codes.shape[2] * 2
        _need(codes, "codes", torch.uint8, (E, N, K // 2))
        _need(scales, "scales", torch.bfloat16, (E, N, K // 64))
        _need(biases, "biases", torch.bfloat16, (E, N, K // 64))
        if weights is None:
            weights = torch.empty((E, N, K), dtype=torch.bfloat16, device=codes.device)
        else:
            _need(weights, "weights", torch.bfloat16, (E, N, K))
        shape = GdnMoeShape(E, 0, K, N)
        _check(lib.gdn_dequant_q4(ctypes.byref(shape), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(weights),
                                  _stream(stream)))
        return weights


def moe_gemm_bf16(x, expert_offsets, weights, y=None, stream=None):
    """The same grouped GEMM on bf16 weights [E, N, K] (gdn_moe_gemm_bf16)."""
    lib = load_library()
    with _on(stream):
        shape = _moe_shape(x, expert_offsets, weights, False)
        _need(weights, "weights", torch.bfloat16, (shape.num_experts, shape.n, shape.k))
        if y is None:
            y = torch.empty((shape.rows, shape.n), dtype=torch.bfloat16, device=x.device)
        else:
            _need(y, "y", torch.bfloat16, (shape.rows, shape.n))
        _check(lib.gdn_moe_gemm_bf16(ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(weights), _ptr(y),
                                     _stream(stream)))
        return y


def _attn_params(head_dim, scale, layout, heads_per_group, num_blocks):
    if layout not in ATTN_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(ATTN_LAYOUTS)}")
    sc = 1.0 / head_dim ** 0.5 if scale is None else float(scale)
    return GdnAttnParams(sc, ATTN_LAYOUTS[layout], int(heads_per_group), int(num_blocks))


def attention_decode_workspace_bytes(batch, h_q, h_kv, head_dim, max_context, scale=None, layout="auto",
                                     heads_per_group=0, num_blocks=0):
    lib = load_library()
    shape = GdnAttnShape(batch, h_q, h_kv, head_dim, max_context)
    params = _attn_params(head_dim, scale, layout, heads_per_group, num_blocks)
    return int(lib.gdn_attention_decode_workspace(ctypes.byref(shape), ctypes.byref(params)))


def attention_decode(q, k_cache, v_cache, context_lens, scale=None, layout="auto", heads_per_group=0, num_blocks=0,
                     out=None, workspace=None, stream=None):
    """Decode attention over a grouped-query KV cache (gdn_attention_decode).
    q [B, h_q, d] bf16; k_cache, v_cache [B, h_kv, T_max, d] bf16;
    context_lens [B] int32.  ``layout`` is "auto", "general" or
    "fixed_block"; scale None means 1 / sqrt(d).  Returns out [B, h_q, d]
    bf16."""
    lib = load_library()
    with _on(stream):
        if k_cache.dim() != 4 or q.dim() != 3:
            raise ValueError("q must be [B, h_q, d] and k_cache [B, h_kv, T_max, d]")
        B, h_kv, T, d = k_cache.shape
        h_q = q.shape[1]
        _need(q, "q", torch.bfloat16, (B, h_q, d))
        _need(k_cache, "k_cache", torch.bfloat16, (B, h_kv, T, d))
        _need(v_cache, "v_cache", torch.bfloat16, (B, h_kv, T, d))
        _need(context_lens, "context_lens", torch.int32, (B,))
        if out is None:
            out = torch.empty((B, h_q, d), dtype=torch.bfloat16, device=q.device)
        else:
            _need(out, "out", torch.bfloat16, (B, h_q, d))
        shape = GdnAttnShape(B, h_q, h_kv, d, T)
        params = _attn_params(d, scale, layout, heads_per_group, num_blocks)
        need = int(lib.gdn_attention_decode_workspace(ctypes.byref(shape), ctypes.byref(params)))
        wp, wn = 0, 0
        if need > 0:
            if workspace is None:
                workspace = alloc_workspace(need, q.device)
            if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
                raise TypeError("workspace must be a uint8 GPU tensor")
            wp, wn = _aligned_ptr(workspace)
        _check(lib.gdn_attention_decode(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(context_lens), _ptr(out), ctypes.c_void_p(wp),
                                        ctypes.c_size_t(max(wn, 0)), _stream(stream)))
        return out


def profile_enable(enabled: bool = True):
    """Bracket every kernel the library enqueues with HIP events on its stream."""
    _check(load_library().gdn_profile_enable(1 if enabled else 0))


def profile_collect(cap: int = 1 << 16):
    """[(kernel name, elapsed ms)] for the kernels recorded since the last
    collect, in launch order; the caller synchronises first."""
    lib = load_library()
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib.gdn_profile_collect(names, ms, cap)
    if n < 0:
        raise GdnError(GDN_ERR_LAUNCH, "gdn_profile_collect: an event query failed")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]
