"""Thin ctypes binding of libocc.so (the C ABI in include/occ.h).

Argument marshalling only: every function checks the tensors it is handed
(device, dtype, shape, contiguity), passes their device addresses and the
current HIP stream to the C entry point of the same name, and raises
``OccError`` on a non-OK status.  All computation happens in the library's
kernels; when the library is missing this module raises instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .workloads import Workload

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libocc.so")

OCC_OK, OCC_ERR_INVALID_ARG, OCC_ERR_UNSUPPORTED, OCC_ERR_WORKSPACE, OCC_ERR_HIP = range(5)
OCC_F32, OCC_BF16 = 0, 1
OCC_PRUNE_OFF, OCC_PRUNE_TRAVERSE, OCC_PRUNE_GROUPSUM, OCC_PRUNE_SIMILARITY = 0, 1, 2, 3
OCC_FLAG_TRAIN = 1
OCC_FLAG_DETERMINISTIC = 2
OCC_NOALLOC_SCRATCH_BYTES = 128 << 20
BSTAGES = ["dispatch", "dgrad_down", "dgrad_up", "shared", "combine", "wgrad_down", "wgrad_up",
           "route"]
OCC_BSTAGE_COUNT = len(BSTAGES)
STAGES = ["route", "brim", "dispatch", "shared_up", "shared_down", "gemm_up", "gemm_down_first",
          "gemm_down_rest", "combine"]
OCC_STAGE_COUNT = len(STAGES)

EXPORTED = ["occ_status_string", "occ_workspace_size", "occ_route",
            "occ_similarity_accumulate", "occ_similarity_rank", "occ_route_similarity",
            "occ_build_brim", "occ_moe_forward", "occ_moe_forward_routed", "occ_gate",
            "occ_moe_forward_gated", "occ_moe_backward", "occ_forward_views",
            "occ_coactivation_stats", "occ_place_experts", "occ_events_create",
            "occ_events_destroy", "occ_event_elapsed_ms", "occ_moe_forward_noalloc"]


class OccError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "Ne", "k", "Nd", "F", "n_shared", "F_shared", "prune_rule",
                 "prune_groups", "dtype", "flags")]


class Brim(ctypes.Structure):
    _fields_ = [("brim0", ctypes.c_void_p), ("sfd_off", ctypes.c_void_p),
                ("epd_off", ctypes.c_void_p), ("epd_src", ctypes.c_void_p),
                ("epd_w", ctypes.c_void_p), ("tok_epd", ctypes.c_void_p),
                ("brim1", ctypes.c_void_p), ("down_rows", ctypes.c_void_p),
                ("first_cnt", ctypes.c_void_p), ("tile_off", ctypes.c_void_p)]


class ForwardView(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("ids", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("brim", Brim),
                ("x_sfd", ctypes.c_void_p), ("epd", ctypes.c_void_p),
                ("sfd_out", ctypes.c_void_p), ("h_shared", ctypes.c_void_p),
                ("y_shared", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OccError(OCC_ERR_HIP, f"{LIB_PATH} is missing; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(LayerDesc)
        sigs = {
            "occ_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "occ_workspace_size": ([dp, ctypes.POINTER(sz)], ctypes.c_int),
            "occ_route": ([dp, vp, vp, vp, vp, vp], ctypes.c_int),
            "occ_similarity_accumulate": ([i32, i32, vp, vp, vp], ctypes.c_int),
            "occ_similarity_rank": ([i32, vp, vp, vp, vp], ctypes.c_int),
            "occ_route_similarity": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "occ_build_brim": ([dp, vp, vp, vp, ctypes.c_int, vp, sz, ctypes.POINTER(Brim), vp],
                               ctypes.c_int),
            "occ_moe_forward": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp],
                                ctypes.c_int),
            "occ_moe_forward_noalloc": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
                                        ctypes.c_int),
            "occ_moe_forward_routed": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                        vp, vp], ctypes.c_int),
            "occ_gate": ([dp, vp, vp, vp, vp], ctypes.c_int),
            "occ_moe_backward": ([dp] + [vp] * 20 + [sz, vp, vp], ctypes.c_int),
            "occ_moe_forward_gated": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp],
                                      ctypes.c_int),
            "occ_forward_views": ([dp, vp, ctypes.POINTER(ForwardView)], ctypes.c_int),
            "occ_coactivation_stats": ([dp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "occ_place_experts": ([vp, i32, i32, vp], ctypes.c_int),
            "occ_events_create": ([i32, vp], ctypes.c_int),
            "occ_events_destroy": ([i32, vp], ctypes.c_int),
            "occ_event_elapsed_ms": ([vp, vp, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().occ_status_string(status).decode()
    except OccError:
        return f"status {status}"


def _check(status: int, what: str):
    if status != OCC_OK:
        raise OccError(status, what)


def desc_of(w: Workload, **over) -> LayerDesc:
    f = dict(T=w.T, d=w.d, Ne=w.Ne, k=w.k, Nd=w.Nd, F=w.F, n_shared=w.n_shared,
             F_shared=w.F_shared, prune_rule=w.prune_rule, prune_groups=w.prune_groups,
             dtype=w.dtype, flags=0)
    f.update(over)
    return LayerDesc(**f)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor | None, name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _host_i32(a, name: str, shape=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {a.shape}")
    return a


def _hp(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def occ_workspace_size(desc: LayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().occ_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "occ_workspace_size")
    return n.value


def alloc_workspace(desc: LayerDesc, device="cuda") -> torch.Tensor:
    """A device byte tensor of occ_workspace_size bytes (torch allocations are 256-aligned)."""
    return torch.empty(occ_workspace_size(desc), dtype=torch.uint8, device=device)


def occ_route(desc: LayerDesc, logits, placement, ids, w, stream=None):
    T, Ne, k = desc.T, desc.Ne, desc.k
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    _check(lib().occ_route(ctypes.byref(desc), _dev(logits, "logits", torch.float32, (T, Ne)),
                           _hp(L), _dev(ids, "ids", torch.int32, (T, k)),
                           _dev(w, "w", torch.float32, (T, k)), _stream(stream)), "occ_route")


def occ_similarity_accumulate(logits, gram, stream=None):
    """gram (Ne x Ne fp64) += logits^T logits, one batch (appendix A.3)."""
    T, Ne = logits.shape
    _check(lib().occ_similarity_accumulate(
        T, Ne, _dev(logits, "logits", torch.float32, (T, Ne)),
        _dev(gram, "gram", torch.float64, (Ne, Ne)), _stream(stream)), "occ_similarity_accumulate")


def occ_similarity_rank(gram, rank, t2=None, stream=None):
    """Squared cosine table (optional t2) and per-row ranking from a Gram matrix."""
    Ne = gram.shape[0]
    _check(lib().occ_similarity_rank(
        Ne, _dev(gram, "gram", torch.float64, (Ne, Ne)),
        _dev(t2, "t2", torch.float64, (Ne, Ne)), _dev(rank, "rank", torch.int32, (Ne, Ne)),
        _stream(stream)), "occ_similarity_rank")


def occ_route_similarity(desc: LayerDesc, logits, placement, sim_rank, ids, w, stream=None):
    T, Ne, k = desc.T, desc.Ne, desc.k
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    _check(lib().occ_route_similarity(
        ctypes.byref(desc), _dev(logits, "logits", torch.float32, (T, Ne)), _hp(L),
        _dev(sim_rank, "sim_rank", torch.int32, (Ne, Ne)), _dev(ids, "ids", torch.int32, (T, k)),
        _dev(w, "w", torch.float32, (T, k)), _stream(stream)), "occ_route_similarity")


def occ_build_brim(desc: LayerDesc, ids, w, placement, workspace, dense_brim1=True,
                   stream=None) -> Brim:
    T, k = desc.T, desc.k
    L = _host_i32(placement, "placement", (desc.Nd, desc.Ne // desc.Nd))
    out = Brim()
    _check(lib().occ_build_brim(ctypes.byref(desc), _dev(ids, "ids", torch.int32, (T, k)),
                                _dev(w, "w", torch.float32, (T, k)), _hp(L), int(dense_brim1),
                                _dev(workspace, "workspace", torch.uint8),
                                workspace.numel(), ctypes.byref(out), _stream(stream)),
           "occ_build_brim")
    return out


def occ_moe_forward(desc: LayerDesc, x, logits, placement, w_gate, w_up, w_down, ws_gate, ws_up,
                    ws_down, y, workspace, stage_events=None, stream=None):
    T, d, Ne, F = desc.T, desc.d, desc.Ne, desc.F
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    nsh, Fsh = desc.n_shared, desc.F_shared
    sh = [None, None, None]
    if nsh > 0:
        sh = [_dev(ws_gate, "ws_gate", dt, (nsh, Fsh, d)), _dev(ws_up, "ws_up", dt, (nsh, Fsh, d)),
              _dev(ws_down, "ws_down", dt, (nsh, d, Fsh))]
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (OCC_STAGE_COUNT + 1))(*stage_events)
    _check(lib().occ_moe_forward(
        ctypes.byref(desc), _dev(x, "x", dt, (T, d)),
        _dev(logits, "logits", torch.float32, (T, Ne)), _hp(L),
        _dev(w_gate, "w_gate", dt, (Ne, F, d)), _dev(w_up, "w_up", dt, (Ne, F, d)),
        _dev(w_down, "w_down", dt, (Ne, d, F)), *sh, _dev(y, "y", dt, (T, d)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)),
        "occ_moe_forward")


def occ_moe_forward_noalloc(desc: LayerDesc, x, logits, placement, w_gate, w_up, w_down, ws_gate,
                            ws_up, ws_down, y, stage_events=None, stream=None):
    """occ_moe_forward with the library's static per-GPU scratch array as the
    workspace (nothing allocated; shapes up to OCC_NOALLOC_SCRATCH_BYTES of
    workspace; calls on one GPU must not overlap)."""
    T, d, Ne, F = desc.T, desc.d, desc.Ne, desc.F
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    nsh, Fsh = desc.n_shared, desc.F_shared
    sh = [None, None, None]
    if nsh > 0:
        sh = [_dev(ws_gate, "ws_gate", dt, (nsh, Fsh, d)), _dev(ws_up, "ws_up", dt, (nsh, Fsh, d)),
              _dev(ws_down, "ws_down", dt, (nsh, d, Fsh))]
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (OCC_STAGE_COUNT + 1))(*stage_events)
    _check(lib().occ_moe_forward_noalloc(
        ctypes.byref(desc), _dev(x, "x", dt, (T, d)),
        _dev(logits, "logits", torch.float32, (T, Ne)), _hp(L),
        _dev(w_gate, "w_gate", dt, (Ne, F, d)), _dev(w_up, "w_up", dt, (Ne, F, d)),
        _dev(w_down, "w_down", dt, (Ne, d, F)), *sh, _dev(y, "y", dt, (T, d)),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)),
        "occ_moe_forward_noalloc")


def occ_moe_forward_routed(desc: LayerDesc, x, ids, w, placement, w_gate, w_up, w_down, ws_gate,
                           ws_up, ws_down, y, workspace, stage_events=None, stream=None):
    T, d, Ne, F, k = desc.T, desc.d, desc.Ne, desc.F, desc.k
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    nsh, Fsh = desc.n_shared, desc.F_shared
    sh = [None, None, None]
    if nsh > 0:
        sh = [_dev(ws_gate, "ws_gate", dt, (nsh, Fsh, d)), _dev(ws_up, "ws_up", dt, (nsh, Fsh, d)),
              _dev(ws_down, "ws_down", dt, (nsh, d, Fsh))]
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (OCC_STAGE_COUNT + 1))(*stage_events)
    _check(lib().occ_moe_forward_routed(
        ctypes.byref(desc), _dev(x, "x", dt, (T, d)), _dev(ids, "ids", torch.int32, (T, k)),
        _dev(w, "w", torch.float32, (T, k)), _hp(L),
        _dev(w_gate, "w_gate", dt, (Ne, F, d)), _dev(w_up, "w_up", dt, (Ne, F, d)),
        _dev(w_down, "w_down", dt, (Ne, d, F)), *sh, _dev(y, "y", dt, (T, d)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)),
        "occ_moe_forward_routed")


def occ_gate(desc: LayerDesc, x, w_router, logits, stream=None):
    T, d, Ne = desc.T, desc.d, desc.Ne
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    _check(lib().occ_gate(ctypes.byref(desc), _dev(x, "x", dt, (T, d)),
                          _dev(w_router, "w_router", dt, (Ne, d)),
                          _dev(logits, "logits", torch.float32, (T, Ne)), _stream(stream)),
           "occ_gate")


def occ_moe_forward_gated(desc: LayerDesc, x, w_router, placement, w_gate, w_up, w_down, ws_gate,
                          ws_up, ws_down, y, workspace, stage_events=None, stream=None):
    T, d, Ne, F = desc.T, desc.d, desc.Ne, desc.F
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    nsh, Fsh = desc.n_shared, desc.F_shared
    sh = [None, None, None]
    if nsh > 0:
        sh = [_dev(ws_gate, "ws_gate", dt, (nsh, Fsh, d)), _dev(ws_up, "ws_up", dt, (nsh, Fsh, d)),
              _dev(ws_down, "ws_down", dt, (nsh, d, Fsh))]
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (OCC_STAGE_COUNT + 1))(*stage_events)
    _check(lib().occ_moe_forward_gated(
        ctypes.byref(desc), _dev(x, "x", dt, (T, d)), _dev(w_router, "w_router", dt, (Ne, d)),
        _hp(L), _dev(w_gate, "w_gate", dt, (Ne, F, d)), _dev(w_up, "w_up", dt, (Ne, F, d)),
        _dev(w_down, "w_down", dt, (Ne, d, F)), *sh, _dev(y, "y", dt, (T, d)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)),
        "occ_moe_forward_gated")


def occ_moe_backward(desc: LayerDesc, dy, x, logits, placement, w_gate, w_up, w_down, ws_gate,
                     ws_up, ws_down, dx, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down,
                     dw, dlogits, workspace, stage_events=None, stream=None):
    """Backward pass; the workspace must hold a training forward's state."""
    T, d, Ne, F, k = desc.T, desc.d, desc.Ne, desc.F, desc.k
    dt = torch.bfloat16 if desc.dtype == OCC_BF16 else torch.float32
    f32 = torch.float32
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    nsh, Fsh = desc.n_shared, desc.F_shared
    sh = [None] * 6
    if nsh > 0:
        sh = [_dev(ws_gate, "ws_gate", dt, (nsh, Fsh, d)), _dev(ws_up, "ws_up", dt, (nsh, Fsh, d)),
              _dev(ws_down, "ws_down", dt, (nsh, d, Fsh)),
              _dev(dws_gate, "dws_gate", f32, (nsh, Fsh, d)),
              _dev(dws_up, "dws_up", f32, (nsh, Fsh, d)),
              _dev(dws_down, "dws_down", f32, (nsh, d, Fsh))]
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * (OCC_BSTAGE_COUNT + 1))(*stage_events)
    _check(lib().occ_moe_backward(
        ctypes.byref(desc), _dev(dy, "dy", dt, (T, d)), _dev(x, "x", dt, (T, d)),
        _dev(logits, "logits", f32, (T, Ne)), _hp(L),
        _dev(w_gate, "w_gate", dt, (Ne, F, d)), _dev(w_up, "w_up", dt, (Ne, F, d)),
        _dev(w_down, "w_down", dt, (Ne, d, F)), *sh[:3], _dev(dx, "dx", dt, (T, d)),
        _dev(dw_gate, "dw_gate", f32, (Ne, F, d)), _dev(dw_up, "dw_up", f32, (Ne, F, d)),
        _dev(dw_down, "dw_down", f32, (Ne, d, F)), *sh[3:], _dev(dw, "dw", f32, (T, k)),
        _dev(dlogits, "dlogits", f32, (T, Ne)), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None,
        _stream(stream)), "occ_moe_backward")


def occ_forward_views(desc: LayerDesc, workspace) -> ForwardView:
    out = ForwardView()
    _check(lib().occ_forward_views(ctypes.byref(desc), _dev(workspace, "workspace", torch.uint8),
                                   ctypes.byref(out)), "occ_forward_views")
    return out


def occ_coactivation_stats(desc: LayerDesc, ids, placement, C, P, n_sfd, ct, intra, stream=None):
    T, k, Ne = desc.T, desc.k, desc.Ne
    L = _host_i32(placement, "placement", (desc.Nd, Ne // desc.Nd))
    _check(lib().occ_coactivation_stats(
        ctypes.byref(desc), _dev(ids, "ids", torch.int32, (T, k)), _hp(L),
        _dev(C, "C", torch.int32, (Ne, Ne)), _dev(P, "P", torch.float32, (Ne, Ne)),
        _dev(n_sfd, "n_sfd", torch.int64, (1,)), _dev(ct, "ct", torch.float64, (1,)),
        _dev(intra, "intra", torch.float64, (1,)), _stream(stream)), "occ_coactivation_stats")


def occ_place_experts(C, Nd: int) -> np.ndarray:
    """Algorithm 1 on host counts C (Ne x Ne); returns the (Nd, Ne/Nd) placement."""
    Cc = np.ascontiguousarray(C, dtype=np.int32)
    Ne = Cc.shape[0]
    if Cc.shape != (Ne, Ne):
        raise ValueError("C must be square")
    L = np.empty((Nd, Ne // max(Nd, 1)), np.int32)
    _check(lib().occ_place_experts(_hp(Cc), Ne, Nd, _hp(L)), "occ_place_experts")
    return L


class StageEvents:
    """stages+1 HIP events for a call's stage timing (occ_moe_forward's by
    default; OCC_BSTAGE_COUNT for occ_moe_backward)."""

    def __init__(self, stages: int = OCC_STAGE_COUNT):
        self.n = stages + 1
        self.arr = (ctypes.c_void_p * self.n)()
        _check(lib().occ_events_create(self.n, self.arr), "occ_events_create")

    @property
    def handles(self):
        return list(self.arr)

    def elapsed_ms(self) -> list[float]:
        out = []
        for i in range(self.n - 1):
            ms = ctypes.c_float(0)
            _check(lib().occ_event_elapsed_ms(self.arr[i], self.arr[i + 1], ctypes.byref(ms)),
                   "occ_event_elapsed_ms")
            out.append(ms.value)
        return out

    def close(self):
        if self.arr is not None:
            lib().occ_events_destroy(self.n, self.arr)
            self.arr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ws_view(workspace: torch.Tensor, ptr: int, shape, dtype: torch.dtype) -> torch.Tensor:
    """A torch view of a buffer the library placed inside `workspace` (a device
    address returned by occ_build_brim / occ_forward_views)."""
    off = int(ptr) - workspace.data_ptr()
    numel = int(np.prod(shape)) if len(shape) else 1
    nbytes = numel * torch.empty(0, dtype=dtype).element_size()
    if off < 0 or off + nbytes > workspace.numel():
        raise ValueError("address outside the workspace")
    return workspace[off:off + nbytes].view(dtype).view(*shape)
