"""MonarchAttention forward pass on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of include/monarch_attn.h.  It only
marshals arguments: PyTorch supplies device memory and the current stream,
and every step of the method runs in the HIP kernels of libmonarch_attn.so.
There is no fallback: without the built library (or on a tensor that is not
on a HIP device) the calls raise.

    import structured_sub_quadratic_amd as ma
    y = ma.forward(q, k, v, b1=128, b2=128)               # [B,H,N,d] on cuda
    y, ex = ma.forward(q, k, v, 630, 52, layout="fh_w", fhw=(21, 30, 52),
                       c1=2, c2=2, exports=("L", "R", "lse", "objective"))
"""

import ctypes

from . import _lib
from ._lib import (MonarchAttnError, LAYOUTS, MA_FLAG_FORCE_STAGED, MA_FLAG_FAST_AGGREGATE,
                   MA_FLAG_FORCE_FUSED, MA_FLAG_PRECISE_AGGREGATE, MA_FLAG_PAD_FRONT,
                   MA_FLAG_REUSE_FORWARD_STATE)

__all__ = ["forward", "forward_timed", "forward_noalloc", "backward", "make_problem",
           "workspace_size",
           "backward_workspace_size", "num_launches", "launch_names", "Event",
           "MonarchAttnError", "LAYOUTS", "library_path", "version"]


def library_path():
    return _lib.LIB_PATH


def version():
    return _lib.load().monarch_attn_version().decode()


def _dtype_code(dtype):
    import torch
    if dtype == torch.float32:
        return _lib.MA_F32
    if dtype == torch.bfloat16:
        return _lib.MA_BF16
    raise TypeError(f"unsupported dtype {dtype}")


def make_problem(batch, heads, seq_len, head_dim, b1, b2, steps=1, c1=1, c2=1, scale=None,
                 dtype="bf16", layout="flat", fhw=None, flags=0, kv_heads=0, causal=0):
    """Build the C problem descriptor.  dtype: "f32"/"bf16" or a torch dtype.
    kv_heads: heads of K and V (0: heads); grouped-query attention when
    smaller.  causal: 0, or g grid blocks per causal unit (block-causal use,
    see ma_problem.causal)."""
    if not isinstance(dtype, int):
        dtype = {"f32": _lib.MA_F32, "bf16": _lib.MA_BF16}.get(dtype, None) \
            if isinstance(dtype, str) else _dtype_code(dtype)
        if dtype is None:
            raise TypeError("dtype must be 'f32' or 'bf16'")
    f, h, w = fhw if fhw is not None else (0, 0, 0)
    return _lib.MAProblem(batch, heads, seq_len, head_dim, b1, b2, c1, c2, steps,
                          0.0 if scale is None else float(scale), dtype, LAYOUTS[layout],
                          f, h, w, flags, kv_heads, causal)


def workspace_size(problem):
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().monarch_attn_workspace_size(ctypes.byref(problem), ctypes.byref(n)),
               "monarch_attn_workspace_size")
    return n.value


def backward_workspace_size(problem):
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().monarch_attn_backward_workspace_size(ctypes.byref(problem),
                                                                ctypes.byref(n)),
               "monarch_attn_backward_workspace_size")
    return n.value


def num_launches(problem):
    return _lib.load().monarch_attn_num_launches(ctypes.byref(problem))


def launch_names(problem):
    lib = _lib.load()
    return [lib.monarch_attn_launch_name(ctypes.byref(problem), j).decode()
            for j in range(num_launches(problem))]


class Event:
    """A hipEvent_t owned by the library's helper functions (diagnostics)."""

    def __init__(self):
        self.ptr = ctypes.c_void_p()
        _lib.check(_lib.load().monarch_attn_event_create(ctypes.byref(self.ptr)),
                   "monarch_attn_event_create")

    def elapsed_ms(self, later):
        ms = ctypes.c_float()
        _lib.check(_lib.load().monarch_attn_event_elapsed_ms(self.ptr, later.ptr, ctypes.byref(ms)),
                   "monarch_attn_event_elapsed_ms")
        return ms.value

    def __del__(self):
        try:
            if self.ptr:
                _lib.load().monarch_attn_event_destroy(self.ptr)
        except Exception:
            pass


def _prepare(q, k, v, b1, b2, steps, c1, c2, scale, layout, fhw, exports, workspace, out,
             force_staged, fast_aggregate, force_fused=False, precise_aggregate=False,
             pad="post", causal=0):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a HIP device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [batch, heads, seq_len, head_dim] tensor")
    if k.shape != v.shape or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("k and v must share shape, and q, k, v their dtype")
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, D) or Hkv < 1 or H % Hkv:
        raise ValueError("k, v must be [batch, kv_heads, seq_len, head_dim] with kv_heads | heads")
    flags = (MA_FLAG_FORCE_STAGED if force_staged else 0) | \
        (MA_FLAG_FAST_AGGREGATE if fast_aggregate else 0) | \
        (MA_FLAG_FORCE_FUSED if force_fused else 0) | \
        (MA_FLAG_PRECISE_AGGREGATE if precise_aggregate else 0)
    if pad not in ("pre", "post"):
        raise ValueError("pad must be 'pre' or 'post'")
    if pad == "pre":
        flags |= MA_FLAG_PAD_FRONT
    prob = make_problem(B, H, N, D, b1, b2, steps, c1, c2, scale, q.dtype, layout, fhw, flags,
                        kv_heads=Hkv, causal=causal)
    ws_bytes = workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    ex = {}
    exports = tuple(exports or ())
    if "L" in exports:
        ex["L"] = torch.empty((B, H, b2, b1, b1 * c2), dtype=torch.float32, device=q.device)
    if "R" in exports:
        ex["R"] = torch.empty((B, H, b1, b2, c1, b2), dtype=torch.float32, device=q.device)
    if "lse" in exports:
        ex["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if "objective" in exports:
        ex["objective"] = torch.empty((B * H,), dtype=torch.float64, device=q.device)
    cex = _lib.MAExports(*(ex[n].data_ptr() if n in ex else None
                           for n in ("L", "R", "lse", "objective")))
    return prob, workspace, out, ex, cex


def forward(q, k, v, b1, b2, steps=1, c1=1, c2=1, scale=None, layout="flat", fhw=None,
            exports=(), workspace=None, out=None, force_staged=False, fast_aggregate=False,
            force_fused=False, precise_aggregate=False, pad="post", causal=0):
    """MonarchAttention forward on the current stream.  Returns Y, or (Y, dict
    of exports) when exports (a subset of "L", "R", "lse", "objective") is
    non-empty.  Shapes of the exports are documented in monarch_attn.h.
    A flat sequence with seq_len < b1*b2 is padded to the grid, after its
    tokens (pad="post") or before them (pad="pre"; see MA_FLAG_PAD_FRONT).
    fast_aggregate / precise_aggregate: bf16 only, force the plain or the
    split precision of the c = R K path (default: plain for T = 1, split for
    T > 1; see MA_FLAG_FAST_AGGREGATE).  force_fused / force_staged: T = 1 as
    one cooperative launch / as separate stage launches.  causal: 0
    (bidirectional) or g >= 1, block-causal use: query block l attends to
    key block k iff floor(k/g) <= floor(l/g) (ma_problem.causal)."""
    import torch
    prob, workspace, out, ex, cex = _prepare(q, k, v, b1, b2, steps, c1, c2, scale, layout, fhw,
                                             exports, workspace, out, force_staged,
                                             fast_aggregate, force_fused, precise_aggregate, pad,
                                             causal)
    st = torch.cuda.current_stream(q.device).cuda_stream
    status = _lib.load().monarch_attn_forward(
        ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        ctypes.byref(cex), workspace.data_ptr(), workspace.numel(), st)
    _lib.check(status, "monarch_attn_forward")
    return (out, ex) if exports else out


def forward_timed(q, k, v, b1, b2, events, steps=1, c1=1, c2=1, scale=None, layout="flat",
                  fhw=None, workspace=None, out=None, force_staged=False, fast_aggregate=False,
                  force_fused=False, precise_aggregate=False, pad="post", causal=0):
    """forward() that also records the start and end of kernel launch j into
    events[2j] and events[2j+1] (Event objects) on the current stream."""
    import torch
    prob, workspace, out, ex, cex = _prepare(q, k, v, b1, b2, steps, c1, c2, scale, layout, fhw,
                                             (), workspace, out, force_staged, fast_aggregate,
                                             force_fused, precise_aggregate, pad, causal)
    st = torch.cuda.current_stream(q.device).cuda_stream
    arr = (ctypes.c_void_p * len(events))(*[e.ptr.value for e in events])
    status = _lib.load().monarch_attn_forward_timed(
        ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        ctypes.byref(cex), workspace.data_ptr(), workspace.numel(), st, arr, len(events))
    _lib.check(status, "monarch_attn_forward_timed")
    return out


def forward_noalloc(q, k, v, b1, b2, out, steps=1, c1=1, c2=1, scale=None, layout="flat",
                    fhw=None, exports=None, fast_aggregate=False, precise_aggregate=False,
                    pad="post", causal=0):
    """forward() through monarch_attn_forward_noalloc: no workspace argument
    and no allocation (the library's own per-device scratch array serves as
    the workspace; problems whose workspace exceeds
    MONARCH_ATTN_SCRATCH_BYTES raise MonarchAttnError).  The caller passes
    the output `out` (shaped like q) and, optionally, `exports`, a dict of
    preallocated export tensors ("L", "R", "lse", "objective", shaped as in
    forward()).  Calls that overlap on one device share that array."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d HIP device tensor")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be shaped and typed like q")
    B, H, N, D = q.shape
    flags = (MA_FLAG_FAST_AGGREGATE if fast_aggregate else 0) | \
        (MA_FLAG_PRECISE_AGGREGATE if precise_aggregate else 0) | \
        (MA_FLAG_PAD_FRONT if pad == "pre" else 0)
    prob = make_problem(B, H, N, D, b1, b2, steps, c1, c2, scale, q.dtype, layout, fhw, flags,
                        kv_heads=k.shape[1], causal=causal)
    ex = exports or {}
    cex = _lib.MAExports(*(ex[n].data_ptr() if n in ex else None
                           for n in ("L", "R", "lse", "objective")))
    st = torch.cuda.current_stream(q.device).cuda_stream
    status = _lib.load().monarch_attn_forward_noalloc(
        ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        ctypes.byref(cex), st)
    _lib.check(status, "monarch_attn_forward_noalloc")
    return out


def backward(q, k, v, dy, b1, b2, steps=1, c1=1, c2=1, scale=None, layout="flat", fhw=None,
             workspace=None, out=None, pad="post", reuse_forward_state=False, y=None, causal=0):
    """Gradients (dq, dk, dv) of <dy, forward(q, k, v, ...)> on the current
    stream.  Covers what monarch_attn_backward documents (blocks of at most
    128 keys, any b1; k, v may have fewer heads; pad, tiles c1, c2 and
    causal as in forward, at any T; bf16 at head_dim 128 with T > 1 keeps to
    b2 <= 64).
    out: optional (dq, dk, dv) tensors to write.
    reuse_forward_state (T = 1): `workspace` holds the state a forward call
    of the same inputs left there (that call was given this workspace, of at
    least backward_workspace_size bytes); the backward does not rebuild it.
    y: optional forward output for these inputs; long stage-2 columns then
    take their softmax-gradient row sums from dy . y instead of a pass over
    their keys."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("dy", dy)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a HIP device tensor")
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous 4-d tensor typed like q")
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    if dy.shape != q.shape or k.shape != v.shape or (k.shape[0], k.shape[2], k.shape[3]) != (B, N, D) \
            or H % Hkv:
        raise ValueError("dy must be shaped like q, and k, v [batch, kv_heads, seq_len, head_dim]")
    if pad not in ("pre", "post"):
        raise ValueError("pad must be 'pre' or 'post'")
    if y is not None and (not y.is_cuda or y.shape != q.shape or y.dtype != q.dtype
                          or not y.is_contiguous()):
        raise ValueError("y must be a contiguous device tensor shaped and typed like q")
    flags = (MA_FLAG_PAD_FRONT if pad == "pre" else 0) | \
        (MA_FLAG_REUSE_FORWARD_STATE if reuse_forward_state else 0)
    prob = make_problem(B, H, N, D, b1, b2, steps, c1, c2, scale, q.dtype, layout, fhw, flags,
                        kv_heads=Hkv, causal=causal)
    ws_bytes = backward_workspace_size(prob)
    if reuse_forward_state and workspace is None:
        raise ValueError("reuse_forward_state needs the workspace the forward call used")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k),
                                              torch.empty_like(v))
    st = torch.cuda.current_stream(q.device).cuda_stream
    status = _lib.load().monarch_attn_backward(
        ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
        y.data_ptr() if y is not None else None, dy.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(), st)
    _lib.check(status, "monarch_attn_backward")
    return dq, dk, dv
