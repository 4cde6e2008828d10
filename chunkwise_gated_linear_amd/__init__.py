"""Chunkwise gated linear attention forward on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libgla.so`` (declared in
``include/gla.h``).  It only marshals arguments: torch provides device memory
and the current HIP stream, every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing,
importing the binding still works but every call raises.

    o, ht = gla_fwd(q, k, v, g, h0=None, cu_seqlens=None, scale=None,
                    chunk=64, output_final_state=False)
    dq, dk, dv, dg, dh0 = gla_bwd(q, k, v, g, do, h0=None, dht=None,
                                  cu_seqlens=None, scale=None)

K and V are multiples of 16 in [16, 256], for the forward and the backward.

Shapes are time-major: q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T, HV, K]
(a decay per key) or [B, T, HV] (one per value head); h0, ht [N, HV, K, V]
float32; cu_seqlens int32 [N+1] for packed sequences (B == 1).  HV = H is the
plain method; HV a multiple of H groups value heads on key heads (value head
hv reads key head hv // (HV // H)).
Defaults follow page "fla/ops/gla/fused_chunk.py" (fused_chunk_gla: scale
defaults to K^-0.5, the final state is returned only on request) and page
"fla/ops/ttt/fused_chunk.py" (fused_chunk_ttt_linear: a given scale must be
positive, packed inputs need a batch of one and one initial state per
sequence).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["gla_fwd", "gla_bwd", "gla_fwd_noalloc", "wy_fwd", "bwd_workspace_bytes", "GlaCall", "GlaBwdCall",
           "WyProblem", "WyCall", "workspace_bytes", "library_path", "load_library", "GlaError",
           "STATUS", "Problem", "STATUS_WAIT_EXHAUSTED", "read_status"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgla.so")
_lib = None

STATUS = {
    0: "GLA_OK", 1: "GLA_ERR_NULL_ARG", 2: "GLA_ERR_BAD_SHAPE", 3: "GLA_ERR_BAD_DTYPE",
    4: "GLA_ERR_BAD_SCALE", 5: "GLA_ERR_UNSUPPORTED", 6: "GLA_ERR_WORKSPACE", 7: "GLA_ERR_HIP",
}
GLA_F32, GLA_BF16 = 0, 1
GATE_PER_KEY, GATE_PER_HEAD = 0, 1
CHUNK = 64
STATUS_WAIT_EXHAUSTED = 1  # bit of the workspace status word: a bounded wait between waves ran out


class GlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("segment_chunks", ctypes.c_int32), ("packed", ctypes.c_int32),
                ("value_tile", ctypes.c_int32), ("wait_limit", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("gate", ctypes.c_int32), ("schedule", ctypes.c_int32)]


class WyProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("chunk", ctypes.c_int32), ("packed", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first (python -m "
                           "chunkwise_gated_linear_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    lib.gla_fwd_workspace_bytes.argtypes = [ctypes.POINTER(Problem)]
    lib.gla_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gla_fwd.argtypes = [ctypes.POINTER(Problem), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                            ctypes.c_size_t, vp]
    lib.gla_fwd.restype = ctypes.c_int
    lib.gla_fwd_noalloc.argtypes = [ctypes.POINTER(Problem), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gla_fwd_noalloc.restype = ctypes.c_int
    lib.gla_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Problem)]
    lib.gla_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gla_bwd.argtypes = [ctypes.POINTER(Problem)] + [vp] * 14 + [ctypes.c_size_t, vp]
    lib.gla_bwd.restype = ctypes.c_int
    lib.gla_wy_fwd_workspace_bytes.argtypes = [ctypes.POINTER(WyProblem)]
    lib.gla_wy_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gla_wy_fwd.argtypes = [ctypes.POINTER(WyProblem)] + [vp] * 9 + [ctypes.c_size_t, vp]
    lib.gla_wy_fwd.restype = ctypes.c_int
    lib.gla_status_str.argtypes = [ctypes.c_int]
    lib.gla_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_msg(lib, code: int) -> str:
    return lib.gla_status_str(code).decode()


def make_problem(B, T, H, K, V, dtype_code, n_seqs, chunk=CHUNK, scale=1.0,
                 segment_chunks=0, packed=False, value_tile=0, wait_limit=0, HV=0,
                 gate=GATE_PER_KEY, schedule=0) -> Problem:
    return Problem(int(B), int(T), int(H), int(K), int(V), int(dtype_code), int(n_seqs),
                   int(chunk), float(scale), int(segment_chunks), 1 if packed else 0,
                   int(value_tile), int(wait_limit), int(HV), int(gate), int(schedule))


def workspace_bytes(problem: Problem) -> int:
    lib = load_library()
    n = lib.gla_fwd_workspace_bytes(ctypes.byref(problem))
    if n == ctypes.c_size_t(-1).value:
        raise GlaError(2, "invalid problem")
    return int(n)


def bwd_workspace_bytes(problem: Problem) -> int:
    lib = load_library()
    n = lib.gla_bwd_workspace_bytes(ctypes.byref(problem))
    if n == ctypes.c_size_t(-1).value:
        raise GlaError(5, "invalid problem for the backward")
    return int(n)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _new_workspace(nbytes: int, dev):
    """Workspace of nbytes; zeroed, so that its status word starts clear."""
    import torch
    return torch.zeros(nbytes, dtype=torch.uint8, device=dev)


def read_status(workspace) -> int:
    """The sticky status word (first 4 bytes) of a workspace; synchronises with the device."""
    import torch
    return int(workspace[:4].cpu().view(torch.int32).item()) & 0xFFFFFFFF


def gla_fwd(q, k, v, g, h0=None, cu_seqlens=None, scale: Optional[float] = None,
            chunk: int = CHUNK, output_final_state: bool = False, segment_chunks: int = 0,
            workspace=None, out=None, value_tile: int = 0,
            wait_limit: int = 0, schedule: int = 0) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Gated linear attention forward through libgla.so.

    Returns (o, ht): o has v's shape and dtype; ht is [N, H, K, V] float32 when
    ``output_final_state`` else None.  Inputs must be contiguous tensors on one
    HIP device; the call is asynchronous on torch's current stream.  A given
    ``workspace`` (uint8, zeroed before its first use) is used when it is large
    enough; its status word can then be read with ``read_status``.
    """
    import torch

    lib = load_library()
    prob, N, dev = _problem_for(q, k, v, g, h0, cu_seqlens, out, scale, chunk, segment_chunks,
                                value_tile, wait_limit, schedule)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    with torch.cuda.device(dev):
        ws = lib.gla_fwd_workspace_bytes(ctypes.byref(prob))
        if ws == ctypes.c_size_t(-1).value:
            code_v = lib.gla_fwd(ctypes.byref(prob), None, None, None, None, None, None, None, None,
                                 None, 0, None)
            raise GlaError(code_v, _status_msg(lib, code_v))
        o = out if out is not None else torch.empty_like(v)
        if out is not None and (out.shape != v.shape or out.dtype != v.dtype):
            raise ValueError("out must match v's shape and dtype")
        ht = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev) if output_final_state else None
        if workspace is None or workspace.numel() * workspace.element_size() < ws:
            workspace = _new_workspace(ws, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.gla_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0),
                         _ptr(cu_seqlens), _ptr(o), _ptr(ht), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), stream)
    if rc != 0:
        raise GlaError(rc, _status_msg(lib, rc))
    return o, ht


def gla_fwd_noalloc(q, k, v, g, o, h0=None, cu_seqlens=None, ht=None, scale: Optional[float] = None,
                    status=None, chunk: int = CHUNK, segment_chunks: int = 0, value_tile: int = 0,
                    schedule: int = 0) -> None:
    """The forward through the library's no-allocation entry point (gla_fwd_noalloc).

    The caller provides o (v's shape and dtype) and, when wanted, ht ([N, H, K, V]
    float32) and a device int32 status word (zeroed; receives GLA_STATUS_* bits).
    Nothing is allocated on the device; problems whose workspace would exceed the
    library's 64 MiB scratch raise GlaError(GLA_ERR_WORKSPACE).  Asynchronous on
    torch's current stream.
    """
    import torch

    lib = load_library()
    prob, N, dev = _problem_for(q, k, v, g, h0, cu_seqlens, o, scale, chunk, segment_chunks, value_tile, 0,
                                schedule)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if o.shape != v.shape or o.dtype != v.dtype:
        raise ValueError("o must match v's shape and dtype")
    if ht is not None and (tuple(ht.shape) != (N, HV, K, V) or ht.dtype != torch.float32 or ht.device != dev
                           or not ht.is_contiguous()):
        raise ValueError(f"ht must be a contiguous float32 [{N}, {HV}, {K}, {V}] tensor on {dev}")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1 or status.device != dev):
        raise ValueError("status must be an int32 device tensor")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.gla_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0),
                                 _ptr(cu_seqlens), _ptr(o), _ptr(ht), _ptr(status), stream)
    if rc != 0:
        raise GlaError(rc, _status_msg(lib, rc))


def gla_bwd(q, k, v, g, do, h0=None, dht=None, cu_seqlens=None, scale: Optional[float] = None,
            chunk: int = CHUNK, need_dh0: Optional[bool] = None, workspace=None, schedule: int = 0,
            wait_limit: int = 0):
    """Gradients of the forward through libgla.so's gla_bwd.

    ``do`` is the gradient of o (v's shape and dtype), ``dht`` that of the final
    state ([N, HV, K, V] float32) or None.  Returns (dq, dk, dv, dg, dh0): dq, dk
    like q, dv like v, dg like g (float32), dh0 [N, HV, K, V] float32 when
    ``need_dh0`` (default: h0 was given) else None.  Asynchronous on torch's
    current stream; a given ``workspace`` (uint8, zeroed before its first use) is
    used when large enough.  ``schedule``: 0 automatic, 1 a separate scan
    launch, 2 the scan chained into the summary kernel, 3 the summary kernel
    walking whole chains; ``wait_limit`` bounds the chained scan's waits as
    for gla_fwd.
    """
    import torch

    lib = load_library()
    prob, N, dev = _problem_for(q, k, v, g, h0, cu_seqlens, None, scale, chunk, 0, 0, wait_limit, schedule)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if do.shape != v.shape or do.dtype != v.dtype or do.device != dev or not do.is_contiguous():
        raise ValueError("do must be a contiguous tensor of v's shape and dtype on v's device")
    if dht is not None and (tuple(dht.shape) != (N, HV, K, V) or dht.dtype != torch.float32
                            or dht.device != dev or not dht.is_contiguous()):
        raise ValueError(f"dht must be a contiguous float32 [{N}, {HV}, {K}, {V}] tensor on {dev}")
    if need_dh0 is None:
        need_dh0 = h0 is not None
    with torch.cuda.device(dev):
        ws = lib.gla_bwd_workspace_bytes(ctypes.byref(prob))
        if ws == ctypes.c_size_t(-1).value:
            rc = lib.gla_bwd(ctypes.byref(prob), *([None] * 14), 0, None)
            raise GlaError(rc, _status_msg(lib, rc))
        dq, dk = torch.empty_like(q), torch.empty_like(k)
        dv = torch.empty_like(v)
        dg = torch.empty_like(g)
        dh0 = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev) if need_dh0 else None
        if workspace is None or workspace.numel() * workspace.element_size() < ws:
            # every byte past the status header is written before it is read
            workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
            workspace[:256].zero_()
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.gla_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(cu_seqlens),
                         _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh0),
                         _ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    if rc != 0:
        raise GlaError(rc, _status_msg(lib, rc))
    return dq, dk, dv, dg, dh0


def _problem_for(q, k, v, g, h0, cu_seqlens, out, scale, chunk, segment_chunks, value_tile, wait_limit,
                 schedule=0):
    """Checks the tensors of a call and builds its gla_problem (page defaults for scale)."""
    import torch

    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [B, T, H, K] and v [B, T, HV, V]")
    HV = v.shape[2]
    if HV % q.shape[2] != 0:
        raise ValueError(f"value heads ({HV}) must be a multiple of key heads ({q.shape[2]})")
    if g.shape == (*v.shape[:3], q.shape[3]):
        gate = GATE_PER_KEY
    elif g.shape == v.shape[:3]:
        gate = GATE_PER_HEAD
    else:
        raise ValueError("g must be [B, T, HV, K] (a decay per key) or [B, T, HV] (one per value head)")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    if q.dtype == torch.bfloat16:
        code = GLA_BF16
    elif q.dtype == torch.float32:
        code = GLA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if g.dtype != torch.float32:
        raise ValueError("g must be float32")
    tensors = [q, k, v, g] + [t for t in (h0, cu_seqlens, out) if t is not None]
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on the same GPU")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError(f"packed sequences need a batch of one, got B={B}")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if h0 is not None:
        if h0.dtype != torch.float32 or tuple(h0.shape) != (N, HV, K, V):
            raise ValueError(f"initial state must be float32 [{N}, {HV}, {K}, {V}], "
                             f"got {tuple(h0.shape)} {h0.dtype}")
    if scale is None:
        scale = K ** -0.5
    elif not (scale > 0):
        raise ValueError("scale must be positive")
    prob = make_problem(B, T, H, K, V, code, N, chunk, scale, segment_chunks, cu_seqlens is not None,
                        value_tile, wait_limit, HV, gate, schedule)
    return prob, N, dev


class GlaCall:
    """A prepared forward: validates once, allocates o, ht and the workspace once,
    and then enqueues the same C ABI call on every ``__call__`` (for timing loops
    and stream capture).  ``stream`` defaults to torch's current stream at call time."""

    def __init__(self, q, k, v, g, h0=None, cu_seqlens=None, scale=None, chunk: int = CHUNK,
                 output_final_state: bool = False, segment_chunks: int = 0, value_tile: int = 0,
                 wait_limit: int = 0, schedule: int = 0):
        import torch

        self.lib = load_library()
        self.problem, N, self.device = _problem_for(q, k, v, g, h0, cu_seqlens, None, scale, chunk,
                                                    segment_chunks, value_tile, wait_limit, schedule)
        ws = workspace_bytes(self.problem)
        self.workspace = _new_workspace(ws, self.device)
        self.ws_bytes = ws
        # validation and allocation of o and ht through the same path as gla_fwd
        o, ht = gla_fwd(q, k, v, g, h0=h0, cu_seqlens=cu_seqlens, scale=scale, chunk=chunk,
                        output_final_state=output_final_state, segment_chunks=segment_chunks,
                        workspace=self.workspace, value_tile=value_tile, wait_limit=wait_limit,
                        schedule=schedule)
        self.o, self.ht = o, ht
        self._args = (q, k, v, g, h0, cu_seqlens)

    def __call__(self, stream=None):
        import torch
        q, k, v, g, h0, cu = self._args
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.gla_fwd(ctypes.byref(self.problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0),
                              _ptr(cu), _ptr(self.o), _ptr(self.ht), self.workspace.data_ptr(),
                              self.ws_bytes, s)
        if rc != 0:
            raise GlaError(rc, _status_msg(self.lib, rc))
        return self.o, self.ht

    def status(self) -> int:
        """Sticky status word of this call's workspace (GLA_STATUS_* bits); synchronises."""
        return read_status(self.workspace)


class GlaBwdCall:
    """A prepared backward: validates once, allocates dq, dk, dv, dg, dh0 and the
    workspace once, then enqueues the same gla_bwd call on every ``__call__``."""

    def __init__(self, q, k, v, g, do, h0=None, dht=None, cu_seqlens=None, scale=None, chunk: int = CHUNK,
                 need_dh0: Optional[bool] = None, schedule: int = 0):
        import torch

        self.lib = load_library()
        self.problem, N, self.device = _problem_for(q, k, v, g, h0, cu_seqlens, None, scale, chunk, 0, 0, 0,
                                                    schedule)
        self.ws_bytes = bwd_workspace_bytes(self.problem)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.workspace[:256].zero_()
        dq, dk, dv, dg, dh0 = gla_bwd(q, k, v, g, do, h0=h0, dht=dht, cu_seqlens=cu_seqlens, scale=scale,
                                      chunk=chunk, need_dh0=need_dh0, workspace=self.workspace,
                                      schedule=schedule)
        self.out = (dq, dk, dv, dg, dh0)
        self._args = (q, k, v, g, h0, cu_seqlens, do, dht)

    def __call__(self, stream=None):
        import torch
        q, k, v, g, h0, cu, do, dht = self._args
        dq, dk, dv, dg, dh0 = self.out
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.gla_bwd(ctypes.byref(self.problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(cu),
                              _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dh0),
                              self.workspace.data_ptr(), self.ws_bytes, s)
        if rc != 0:
            raise GlaError(rc, _status_msg(self.lib, rc))
        return self.out

    def status(self) -> int:
        """Sticky status word of this call's workspace (GLA_STATUS_* bits); synchronises."""
        return read_status(self.workspace)


def _wy_problem(k, v, beta, A, g, cu_seqlens):
    """Checks the tensors of a WY call and builds its gla_wy_problem."""
    import torch

    if k.dim() != 4 or v.dim() != 4 or v.shape[:2] != k.shape[:2] or v.shape[2] % k.shape[2] != 0:
        raise ValueError("expected k [B, T, H, K] and v [B, T, HV, V] with HV a multiple of H")
    B, T, H, K = k.shape
    HV, V = v.shape[2], v.shape[3]
    if tuple(A.shape) != (B, T, HV, CHUNK) or tuple(beta.shape) != (B, T, HV):
        raise ValueError(f"A must be [{B}, {T}, {HV}, {CHUNK}] and beta [{B}, {T}, {HV}]")
    if g is not None and tuple(g.shape) != (B, T, HV):
        raise ValueError(f"g must be [{B}, {T}, {HV}]")
    if not (k.dtype == v.dtype == A.dtype) or k.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k, v and A must share a dtype, bfloat16 or float32")
    if beta.dtype != torch.float32 or (g is not None and g.dtype != torch.float32):
        raise ValueError("beta and g must be float32")
    tensors = [k, v, beta, A] + [t for t in (g, cu_seqlens) if t is not None]
    dev = k.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors) or not all(t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous and on the same GPU")
    if cu_seqlens is not None:
        if B != 1 or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("packed sequences need B == 1 and int32 cu_seqlens")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    prob = WyProblem(B, T, H, HV, K, V, GLA_BF16 if k.dtype == torch.bfloat16 else GLA_F32, N, CHUNK,
                     1 if cu_seqlens is not None else 0)
    return prob, dev


class WyCall:
    """A prepared WY forward: validates once, allocates w, u and the workspace
    once, then enqueues the same gla_wy_fwd call on every ``__call__``."""

    def __init__(self, k, v, beta, A, g=None, cu_seqlens=None):
        import torch

        self.lib = load_library()
        self.problem, self.device = _wy_problem(k, v, beta, A, g, cu_seqlens)
        n = self.lib.gla_wy_fwd_workspace_bytes(ctypes.byref(self.problem))
        if n == ctypes.c_size_t(-1).value:
            raise GlaError(2, "invalid problem")
        self.ws_bytes = int(n)
        self.workspace = _new_workspace(self.ws_bytes, self.device)
        B, T, H, K = k.shape
        self.w = torch.empty((B, T, v.shape[2], K), dtype=k.dtype, device=self.device)
        self.u = torch.empty_like(v)
        self._args = (k, v, beta, A, g, cu_seqlens)
        self()

    def __call__(self, stream=None):
        import torch
        k, v, beta, A, g, cu = self._args
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.gla_wy_fwd(ctypes.byref(self.problem), _ptr(k), _ptr(v), _ptr(beta), _ptr(A), _ptr(g),
                                 _ptr(cu), _ptr(self.w), _ptr(self.u), self.workspace.data_ptr(), self.ws_bytes, s)
        if rc != 0:
            raise GlaError(rc, _status_msg(self.lib, rc))
        return self.w, self.u


def wy_fwd(k, v, beta, A, g=None, cu_seqlens=None, workspace=None):
    """WY-representation forward of the gated delta rule through libgla.so's gla_wy_fwd.

    k [B, T, H, K], v [B, T, HV, V], A [B, T, HV, 64] in one dtype (bf16 or
    fp32); beta [B, T, HV] and g [B, T, HV] (base-2 log gate, optional) float32;
    cu_seqlens int32 [N+1] for packed sequences.  Returns (w [B, T, HV, K],
    u [B, T, HV, V]) in the input dtype.  Asynchronous on torch's current stream.
    """
    import torch

    lib = load_library()
    prob, dev = _wy_problem(k, v, beta, A, g, cu_seqlens)
    B, T, H, K = k.shape
    HV = v.shape[2]
    with torch.cuda.device(dev):
        ws = lib.gla_wy_fwd_workspace_bytes(ctypes.byref(prob))
        if ws == ctypes.c_size_t(-1).value:
            rc = lib.gla_wy_fwd(ctypes.byref(prob), *([None] * 9), 0, None)
            raise GlaError(rc, _status_msg(lib, rc))
        w = torch.empty((B, T, HV, K), dtype=k.dtype, device=dev)
        u = torch.empty_like(v)
        if workspace is None or workspace.numel() * workspace.element_size() < ws:
            workspace = _new_workspace(ws, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.gla_wy_fwd(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(beta), _ptr(A), _ptr(g),
                            _ptr(cu_seqlens), _ptr(w), _ptr(u), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), stream)
    if rc != 0:
        raise GlaError(rc, _status_msg(lib, rc))
    return w, u
