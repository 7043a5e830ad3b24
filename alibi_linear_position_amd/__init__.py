"""Python binding of libalibi, the gfx950 causal ALiBi attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/alibi.h. PyTorch provides device memory and
the current stream. There is no fallback: if libalibi.so has not been built,
or a call returns an error status, these functions raise.

    slopes(H)                          -> float32 CPU tensor (host generator)
    attn_fwd(q, k, v, slopes, causal)  -> bf16 (B, H, N, d)
    attn_fwd_f32(q, k, v, slopes, causal)
    attn_fwd_ex(q, k, v, slopes, causal, clamp=, log_distance=, softcap=,
                q_offset=, k_offset=)     -> mitigations / position offsets,
                                             bf16 or fp32 by q's dtype
    slopes_recipe(recipe, H, log_distance) -> float32 CPU tensor
    attn_fwd_train(q, k, v, slopes, causal) -> (out, lse)
    attn_bwd(q, k, v, out, dout, lse, slopes, causal) -> (dq, dk, dv)
    attn_decode(q, kcache, vcache, slopes)  -> bf16 (B, H, d)
    decode_ws_bytes(B, H, L, d), attn_decode_ws(q, kcache, vcache, ws, slopes)
                                           -> the decode with a caller-owned workspace
    attn_weights_f32(q, k, slopes, causal)  -> fp32 (B, H, N, N), test only
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ALIBI_LIBRARY names another build of the same library (e.g. an instrumented
# test build); by default the in-tree libalibi.so.
LIB_PATH = os.environ.get("ALIBI_LIBRARY") or os.path.join(HERE, "libalibi.so")

ALIBI_OK = 0
_STATUS = {0: "ALIBI_OK", -1: "ALIBI_EINVAL", -2: "ALIBI_ENOTSUP", -3: "ALIBI_EHIP", -4: "ALIBI_ENOMEM"}

# (name, argtypes) of every entry point declared in include/alibi.h
_P = ctypes.c_void_p
_I = ctypes.c_int
EXPORTS = {
    "alibi_slopes": [_I, _P],
    "alibi_attn_fwd": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P],
    "alibi_attn_fwd_f32": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P],
    "alibi_attn_decode": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
    "alibi_attn_weights_f32": [_P, _P, _P, _I, _I, _I, _I, _P, _I, _P],
    "alibi_attn_fwd_ex": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P],
    "alibi_attn_fwd_ex_f32": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P],
    "alibi_slopes_recipe": [_I, _I, _I, _P],
    "alibi_debug_schedule": [_I, _I, _I, _P],
    "alibi_debug_fwd_waves": [_I],
    "alibi_debug_fwd_split": [_I],
    "alibi_debug_bwd_query_blocks": [_I],
    "alibi_debug_fwd_form": [_I, _I, _I, _I, _I, _I, _I, _I, _P],
    "alibi_debug_stream_read": [_P, ctypes.c_longlong, _P, _I, _P],
    "alibi_debug_mfma_rate": [_P, _I, _I, _P, _I, _P],
    "alibi_attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P],
    "alibi_attn_bwd_ex": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P, _P],
    "alibi_status_string": [_I],
    "alibi_release": [],
    "alibi_decode_ws_bytes": [_I, _I, _I, _I],
    "alibi_attn_decode_ws": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, ctypes.c_size_t, _P],
    "alibi_debug_fail_allocations": [_I],
    "alibi_attn_decode_noalloc": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
    "alibi_attn_decode_ex": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P],
    "alibi_key_norm_max": [_P, _I, _I, _I, _I, _P, _P],
}
_RESTYPES = {"alibi_status_string": ctypes.c_char_p, "alibi_decode_ws_bytes": ctypes.c_size_t}

# mitigation bits of alibi_fwd_opts.flags and the slope recipes (include/alibi.h)
CLAMP, LOG_DISTANCE, SOFTCAP, SKIP_UNDERFLOW, WINDOW = 1, 2, 4, 8, 16
RECIPES = {"default": 0, "steep": 1, "safe": 2, "wide": 3, "explicit": 4}


class FwdOpts(ctypes.Structure):
    """Mirror of struct alibi_fwd_opts."""
    _fields_ = [("flags", ctypes.c_int), ("clamp_min", ctypes.c_float), ("softcap", ctypes.c_float),
                ("q_offset", ctypes.c_int), ("k_offset", ctypes.c_int), ("lse", ctypes.c_void_p),
                ("window", ctypes.c_void_p)]


class DecodeOpts(ctypes.Structure):
    """Mirror of struct alibi_decode_opts."""
    _fields_ = [("flags", ctypes.c_int), ("key_norm_max", ctypes.c_void_p)]


_lib = None


class AlibiError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with {_STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libalibi.so (once) and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m alibi_linear_position_amd.build`")
    lib = ctypes.CDLL(path)
    for name, argtypes in EXPORTS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    _lib = lib
    return lib


def _check(fn_name, status):
    if status != ALIBI_OK:
        msg = load_library().alibi_status_string(status).decode()
        raise AlibiError(fn_name, status, msg)


def status_string(status: int) -> str:
    return load_library().alibi_status_string(int(status)).decode()


def slopes(H: int):
    """Per-head slopes from the library's host generator (float32 CPU tensor)."""
    import torch
    out = torch.empty(int(H), dtype=torch.float32)
    _check("alibi_slopes", load_library().alibi_slopes(int(H), ctypes.c_void_p(out.data_ptr())))
    return out


def slopes_recipe(recipe: str, H: int, log_distance: bool = False):
    """Slopes from target blindness distances (float32 CPU tensor); see alibi_slopes_recipe."""
    import torch
    out = torch.empty(int(H), dtype=torch.float32)
    if recipe not in RECIPES:
        raise ValueError(f"unknown recipe {recipe!r}; one of {sorted(RECIPES)}")
    st = load_library().alibi_slopes_recipe(RECIPES[recipe], int(H), int(bool(log_distance)),
                                            ctypes.c_void_p(out.data_ptr()))
    _check("alibi_slopes_recipe", st)
    return out


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, ndim, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _slopes_dev(slopes_t, H, device):
    import torch
    if slopes_t is None:
        slopes_t = slopes(H)
    s = slopes_t.to(device=device, dtype=torch.float32).contiguous()
    if s.numel() != H:
        raise ValueError(f"expected {H} slopes, got {s.numel()}")
    return s


def _fwd(entry, dtype, q, k, v, slopes_t, causal, out):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, dtype, 4, n)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have one shape (B, H, N, d)")
    B, H, N, d = q.shape
    s = _slopes_dev(slopes_t, H, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, dtype, 4, "out")
    with torch.cuda.device(q.device):
        st = getattr(load_library(), entry)(
            _P(q.data_ptr()), _P(k.data_ptr()), _P(v.data_ptr()), _P(out.data_ptr()),
            B, H, N, d, _P(s.data_ptr()), int(bool(causal)), _stream_handle(q.device))
    _check(entry, st)
    return out


def attn_fwd(q, k, v, slopes=None, causal=True, out=None):
    """Fused ALiBi attention forward, bf16 (B, H, N, d) device tensors."""
    import torch
    return _fwd("alibi_attn_fwd", torch.bfloat16, q, k, v, slopes, causal, out)


def attn_fwd_f32(q, k, v, slopes=None, causal=True, out=None):
    """fp32 ALiBi attention forward (generic kernel)."""
    import torch
    return _fwd("alibi_attn_fwd_f32", torch.float32, q, k, v, slopes, causal, out)


def attn_fwd_ex(q, k, v, slopes=None, causal=True, clamp=None, log_distance=False, softcap=None,
                q_offset=0, k_offset=0, skip_underflow=False, out=None, lse=None, window=None):
    """Forward with mitigations, position offsets and an optional hard window.

    q: (B, H, Nq, d); k, v: (B, H, Nk, d); bf16 (MFMA / generic kernel) or fp32
    (generic kernel), by q's dtype. clamp: bias floor or None; log_distance:
    ln(D + 1) distances; softcap: z or None; query row r sits at position
    q_offset + r, key row c at k_offset + c. skip_underflow: exact skipping of
    key tiles whose weights all round to zero (bit-identical output). lse: an
    fp32 (B, H, Nq) device tensor that receives each row's log-sum-exp.
    window: None or H per-head windows in tokens (causal, no mitigation): query
    r sees key c when 0 <= pos(r) - pos(c) < window[h].
    """
    import torch
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, dtype, 4, n)
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("expected q (B, H, Nq, d) and k, v (B, H, Nk, d)")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    s = _slopes_dev(slopes, H, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, dtype, 4, "out")
    o = FwdOpts()
    o.flags = (CLAMP if clamp is not None else 0) | (LOG_DISTANCE if log_distance else 0) | \
        (SOFTCAP if softcap is not None else 0) | (SKIP_UNDERFLOW if skip_underflow else 0)
    o.clamp_min = float(clamp) if clamp is not None else 0.0
    o.softcap = float(softcap) if softcap is not None else 0.0
    o.q_offset = int(q_offset)
    o.k_offset = int(k_offset)
    if lse is not None:
        _need(lse, torch.float32, 3, "lse")
        if tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be (B, H, Nq)")
        o.lse = lse.data_ptr()
    wt = None
    if window is not None:
        wt = torch.as_tensor(window, dtype=torch.int32).reshape(-1).to(q.device).contiguous()
        if wt.numel() != H:
            raise ValueError(f"expected {H} windows, got {wt.numel()}")
        o.flags |= WINDOW
        o.window = wt.data_ptr()
    entry = "alibi_attn_fwd_ex" if dtype == torch.bfloat16 else "alibi_attn_fwd_ex_f32"
    with torch.cuda.device(q.device):
        st = getattr(load_library(), entry)(
            _P(q.data_ptr()), _P(k.data_ptr()), _P(v.data_ptr()), _P(out.data_ptr()),
            B, H, Nq, Nk, d, _P(s.data_ptr()), int(bool(causal)), ctypes.byref(o),
            _stream_handle(q.device))
    _check(entry, st)
    return out


def attn_fwd_train(q, k, v, slopes=None, causal=True):
    """Forward that also returns the row log-sum-exp the backward needs: (out, lse)."""
    import torch
    B, H, N, _ = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    out = attn_fwd_ex(q, k, v, slopes, causal, lse=lse)
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, slopes=None, causal=True, clamp=None, log_distance=False,
             skip_underflow=False, softcap=None):
    """Gradients (dq, dk, dv), bf16 (B, H, N, d), of the plain forward, or of the
    forward with the clamp, the log-distance bias and/or the soft cap z (lse from
    attn_fwd_ex with the same settings). skip_underflow: exact skipping of the
    query-key tiles whose every P rounds to zero (plain form;
    bit-identical gradients)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, torch.bfloat16, 4, n)
        if t.shape != q.shape:
            raise ValueError(f"{n} must have q's shape")
    _need(lse, torch.float32, 3, "lse")
    B, H, N, d = q.shape
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be (B, H, N)")
    s = _slopes_dev(slopes, H, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    o = None
    if clamp is not None or log_distance or skip_underflow or softcap is not None:
        o = FwdOpts()
        o.flags = ((CLAMP if clamp is not None else 0) | (LOG_DISTANCE if log_distance else 0)
                   | (SKIP_UNDERFLOW if skip_underflow else 0) | (SOFTCAP if softcap is not None else 0))
        o.clamp_min = float(clamp) if clamp is not None else 0.0
        o.softcap = float(softcap) if softcap is not None else 0.0
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_bwd_ex(
            _P(q.data_ptr()), _P(k.data_ptr()), _P(v.data_ptr()), _P(out.data_ptr()),
            _P(dout.data_ptr()), _P(lse.data_ptr()), _P(dq.data_ptr()), _P(dk.data_ptr()),
            _P(dv.data_ptr()), B, H, N, d, _P(s.data_ptr()), int(bool(causal)),
            None if o is None else ctypes.byref(o), _stream_handle(q.device))
    _check("alibi_attn_bwd_ex", st)
    return dq, dk, dv


def attn_decode(q, kcache, vcache, slopes=None, out=None):
    """Single-query decode: q (B, H, d), caches (B, H, L, d), bf16 device tensors."""
    import torch
    _need(q, torch.bfloat16, 3, "q")
    _need(kcache, torch.bfloat16, 4, "kcache")
    _need(vcache, torch.bfloat16, 4, "vcache")
    B, H, L, d = kcache.shape
    if vcache.shape != kcache.shape or tuple(q.shape) != (B, H, d):
        raise ValueError("expected q (B, H, d) and caches (B, H, L, d)")
    s = _slopes_dev(slopes, H, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, torch.bfloat16, 3, "out")
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_decode(
            _P(q.data_ptr()), _P(kcache.data_ptr()), _P(vcache.data_ptr()), _P(out.data_ptr()),
            B, H, L, d, _P(s.data_ptr()), _stream_handle(q.device))
    _check("alibi_attn_decode", st)
    return out


def key_norm_max(kcache):
    """max_j |k_j| per (b, h) of a bf16 cache (B, H, L, d), d in {64, 128}:
    fp32 (B, H) on the cache's device (the bound attn_decode_ex skips with)."""
    import torch
    _need(kcache, torch.bfloat16, 4, "kcache")
    B, H, L, d = kcache.shape
    out = torch.empty((B, H), dtype=torch.float32, device=kcache.device)
    with torch.cuda.device(kcache.device):
        st = load_library().alibi_key_norm_max(_P(kcache.data_ptr()), B, H, L, d, _P(out.data_ptr()),
                                               _stream_handle(kcache.device))
    _check("alibi_key_norm_max", st)
    return out


def attn_decode_ex(q, kcache, vcache, slopes=None, skip_underflow=False, key_norm_max=None, out=None):
    """attn_decode with options: skip_underflow=True skips, exactly, the cached
    keys whose weights round to zero, given key_norm_max (fp32 (B, H) on the
    device: an upper bound of every key norm of each (b, h), e.g. from
    key_norm_max(kcache))."""
    import torch
    _need(q, torch.bfloat16, 3, "q")
    _need(kcache, torch.bfloat16, 4, "kcache")
    _need(vcache, torch.bfloat16, 4, "vcache")
    B, H, L, d = kcache.shape
    if vcache.shape != kcache.shape or tuple(q.shape) != (B, H, d):
        raise ValueError("expected q (B, H, d) and caches (B, H, L, d)")
    s = _slopes_dev(slopes, H, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, torch.bfloat16, 3, "out")
    opts = DecodeOpts()
    opts.flags = 0
    opts.key_norm_max = None
    if skip_underflow:
        if key_norm_max is None:
            raise ValueError("skip_underflow needs key_norm_max")
        if key_norm_max.dtype != torch.float32 or key_norm_max.device != q.device or \
                tuple(key_norm_max.shape) != (B, H) or not key_norm_max.is_contiguous():
            raise ValueError("key_norm_max must be a contiguous fp32 (B, H) tensor on q's device")
        opts.flags = SKIP_UNDERFLOW
        opts.key_norm_max = key_norm_max.data_ptr()
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_decode_ex(
            _P(q.data_ptr()), _P(kcache.data_ptr()), _P(vcache.data_ptr()), _P(out.data_ptr()),
            B, H, L, d, _P(s.data_ptr()), ctypes.byref(opts), _stream_handle(q.device))
    _check("alibi_attn_decode_ex", st)
    return out


def attn_decode_noalloc(q, kcache, vcache, slopes_dev, out):
    """attn_decode through the entry point that allocates nothing: slopes_dev (H
    fp32 on q's device) and out (bf16 (B, H, d)) are passed in, so this call
    allocates no device memory either."""
    import torch
    _need(q, torch.bfloat16, 3, "q")
    _need(kcache, torch.bfloat16, 4, "kcache")
    _need(vcache, torch.bfloat16, 4, "vcache")
    _need(out, torch.bfloat16, 3, "out")
    B, H, L, d = kcache.shape
    if vcache.shape != kcache.shape or tuple(q.shape) != (B, H, d) or tuple(out.shape) != (B, H, d):
        raise ValueError("expected q, out (B, H, d) and caches (B, H, L, d)")
    if not (isinstance(slopes_dev, torch.Tensor) and slopes_dev.device == q.device and
            slopes_dev.dtype == torch.float32 and slopes_dev.is_contiguous() and slopes_dev.numel() == H):
        raise ValueError("slopes_dev must be H contiguous fp32 values on q's device")
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_decode_noalloc(
            _P(q.data_ptr()), _P(kcache.data_ptr()), _P(vcache.data_ptr()), _P(out.data_ptr()),
            B, H, L, d, _P(slopes_dev.data_ptr()), _stream_handle(q.device))
    _check("alibi_attn_decode_noalloc", st)
    return out


def fwd_form(B, H, Nq, Nk, d, causal=True, flags=0, delta=0):
    """The form a bf16 forward call with these sizes launches (host only): 0 = the
    generic kernel, 4 or 8 = MFMA waves per workgroup, 2 = the key-range split."""
    form = ctypes.c_int(-1)
    st = load_library().alibi_debug_fwd_form(int(B), int(H), int(Nq), int(Nk), int(d), int(bool(causal)),
                                             int(flags), int(delta), ctypes.byref(form))
    _check("alibi_debug_fwd_form", st)
    return form.value


def decode_ws_bytes(B, H, L, d):
    """Bytes of device workspace attn_decode_ws needs for this shape (0: none)."""
    return int(load_library().alibi_decode_ws_bytes(int(B), int(H), int(L), int(d)))


def attn_decode_ws(q, kcache, vcache, ws, slopes=None, out=None):
    """attn_decode with a caller-owned workspace: ws, a device tensor of at least
    decode_ws_bytes(...) bytes (or None when that is 0)."""
    import torch
    _need(q, torch.bfloat16, 3, "q")
    _need(kcache, torch.bfloat16, 4, "kcache")
    _need(vcache, torch.bfloat16, 4, "vcache")
    B, H, L, d = kcache.shape
    if vcache.shape != kcache.shape or tuple(q.shape) != (B, H, d):
        raise ValueError("expected q (B, H, d) and caches (B, H, L, d)")
    s = _slopes_dev(slopes, H, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, torch.bfloat16, 3, "out")
    if ws is not None and (not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous device tensor")
    ptr, nbytes = (0, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_decode_ws(
            _P(q.data_ptr()), _P(kcache.data_ptr()), _P(vcache.data_ptr()), _P(out.data_ptr()),
            B, H, L, d, _P(s.data_ptr()), _P(ptr), ctypes.c_size_t(nbytes), _stream_handle(q.device))
    _check("alibi_attn_decode_ws", st)
    return out


def attn_weights_f32(q, k, slopes=None, causal=True):
    """Test-only: materialised fp32 weights (B, H, N, N) of the fp32 forward."""
    import torch
    _need(q, torch.float32, 4, "q")
    _need(k, torch.float32, 4, "k")
    B, H, N, d = q.shape
    s = _slopes_dev(slopes, H, q.device)
    w = torch.empty((B, H, N, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = load_library().alibi_attn_weights_f32(
            _P(q.data_ptr()), _P(k.data_ptr()), _P(w.data_ptr()), B, H, N, d,
            _P(s.data_ptr()), int(bool(causal)), _stream_handle(q.device))
    _check("alibi_attn_weights_f32", st)
    return w


def release():
    _check("alibi_release", load_library().alibi_release())
