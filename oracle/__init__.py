"""CPU oracle for Occult's MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``occ_oracle.c`` (plain C, fp64), compiled with gcc
into ``liboracle.so``; this module only marshals numpy arrays.  Float inputs
are passed as fp32 arrays or as bf16 bit patterns (uint16), and the C code
widens every element exactly to fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "occ_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
PRUNE_OFF, PRUNE_TRAVERSE, PRUNE_GROUPSUM, PRUNE_SIMILARITY = 0, 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = ctypes.CDLL(LIB)
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _float_arg(a):
    """(array, dtype code) for an fp32 array or a bf16 bit-pattern array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype in (np.uint16, np.int16):
        return a.view(np.uint16), BF16
    raise TypeError(f"oracle takes fp32 or bf16 bit patterns, got {a.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def route(logits: np.ndarray, k: int, placement: np.ndarray, prune_rule: int = PRUNE_OFF,
          prune_groups: int = 0):
    """Top-k softmax routing (Eq. 2) with optional pruning (section 3.3).

    Returns ids (T, k) int32 in routing-score order and w (T, k) float64."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, Ne = lg.shape
    L = _i32(placement)
    Nd = L.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().orc_route(T, Ne, k, _p(lg), Nd, _p(L), prune_rule, prune_groups, _p(ids), _p(w))
    _check(rc, "route")
    return ids, w


def sim_accumulate(logits: np.ndarray, gram: np.ndarray | None = None) -> np.ndarray:
    """Eq. 6-8's Gram matrix of the logit columns, fp64, one more batch added
    (tokens in ascending order) to `gram` (a fresh zero matrix if None)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, Ne = lg.shape
    g = np.zeros((Ne, Ne), np.float64) if gram is None else np.array(gram, np.float64, order="C")
    _check(_load().orc_sim_accumulate(T, Ne, _p(lg), _p(g)), "sim_accumulate")
    return g


def sim_rank(gram: np.ndarray):
    """Squared cosine similarity table (Eq. 7/8) and each row's ranking:
    returns (t2 (Ne, Ne) float64, rank (Ne, Ne) int32)."""
    g = np.ascontiguousarray(gram, dtype=np.float64)
    Ne = g.shape[0]
    t2 = np.empty((Ne, Ne), np.float64)
    rank = np.empty((Ne, Ne), np.int32)
    _check(_load().orc_sim_rank(Ne, _p(g), _p(t2), _p(rank)), "sim_rank")
    return t2, rank


def route_similarity(logits: np.ndarray, k: int, placement: np.ndarray, prune_groups: int,
                     rank: np.ndarray):
    """Expert-similarity-based collaboration pruning (section 3.3): ids (T, k)
    int32 and w (T, k) float64."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, Ne = lg.shape
    L = _i32(placement)
    Nd = L.shape[0]
    r = _i32(rank)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().orc_route_similarity(T, Ne, k, _p(lg), Nd, _p(L), prune_groups, _p(r),
                                      _p(ids), _p(w))
    _check(rc, "route_similarity")
    return ids, w


def gate(rows, x, w_router) -> np.ndarray:
    """Router logits g(x) = x W_r^T (section 2.1) of the listed rows, fp64:
    (len(rows), Ne)."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    xa, dt = _float_arg(x)
    wa, dw = _float_arg(w_router)
    if dt != dw:
        raise TypeError("x and w_router must share a dtype")
    d = xa.shape[1]
    Ne = wa.shape[0]
    out = np.empty((len(rows), Ne), np.float64)
    _check(_load().orc_gate(len(rows), _p(rows), d, Ne, dt, _p(xa), _p(wa), _p(out)), "gate")
    return out


def brim0(ids: np.ndarray, Ne: int, placement: np.ndarray):
    """BRIM_0 of Algorithm 3: (Nd, T) int32 and sfd_off (Nd+1) int64."""
    ids = _i32(ids)
    T, k = ids.shape
    L = _i32(placement)
    Nd = L.shape[0]
    b0 = np.empty((Nd, T), np.int32)
    off = np.empty(Nd + 1, np.int64)
    _check(_load().orc_brim0(T, k, _p(ids), Ne, Nd, _p(L), _p(b0), _p(off)), "brim0")
    return b0, off


def brim1(ids: np.ndarray, w: np.ndarray, Ne: int, placement: np.ndarray, b0=None, sfd_off=None):
    """BRIM_1 of Algorithm 5 per group plus its condensed (CSR) form.

    Returns dict: brim1 (flat, group g's n x N_g block at n*sfd_off[g]),
    epd_off (Ne+1), epd_src (T*k), epd_w (T*k), brim0, sfd_off."""
    ids = _i32(ids)
    T, k = ids.shape
    L = _i32(placement)
    Nd = L.shape[0]
    n = Ne // Nd
    if b0 is None:
        b0, sfd_off = brim0(ids, Ne, L)
    wv = np.ascontiguousarray(w, dtype=np.float64)
    N_sfd = int(sfd_off[-1])
    b1 = np.empty(max(n * N_sfd, 1), np.int32)
    epd_off = np.empty(Ne + 1, np.int64)
    epd_src = np.empty(max(T * k, 1), np.int64)
    epd_w = np.empty(max(T * k, 1), np.float64)
    b0c = _i32(b0)
    offc = np.ascontiguousarray(sfd_off, dtype=np.int64)
    rc = _load().orc_brim1(T, k, _p(ids), _p(wv), Ne, Nd, _p(L), _p(b0c), _p(offc), _p(b1),
                           _p(epd_off), _p(epd_src), _p(epd_w))
    _check(rc, "brim1")
    return dict(brim1=b1[: n * N_sfd], epd_off=epd_off, epd_src=epd_src[: T * k],
                epd_w=epd_w[: T * k], brim0=b0c, sfd_off=offc)


def _opt(a, T):
    if a is None:
        return None, None
    arr, _ = _float_arg(a)
    return arr, _p(arr)


def moe_rows(rows, x, ids, w, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
             nthreads: int = 0):
    """Eq. 1 output rows (float64) for the given token rows."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    xa, dt = _float_arg(x)
    T, d = xa.shape
    ids = _i32(ids)
    k = ids.shape[1]
    wv = np.ascontiguousarray(w, dtype=np.float64)
    g, _ = _float_arg(w_gate)
    u, _ = _float_arg(w_up)
    dn, _ = _float_arg(w_down)
    F = g.shape[1]
    n_sh, F_sh = 0, 0
    sg = su = sd = None
    if ws_gate is not None:
        sg, _ = _float_arg(ws_gate)
        su, _ = _float_arg(ws_up)
        sd, _ = _float_arg(ws_down)
        n_sh, F_sh = sg.shape[0], sg.shape[1]
    y = np.empty((len(rows), d), np.float64)
    nul = ctypes.c_void_p(0)
    rc = _load().orc_moe_rows(len(rows), _p(rows), d, k, F, n_sh, F_sh, dt, _p(xa), _p(ids),
                              _p(wv), _p(g), _p(u), _p(dn),
                              _p(sg) if sg is not None else nul,
                              _p(su) if su is not None else nul,
                              _p(sd) if sd is not None else nul, nthreads, _p(y))
    _check(rc, "moe_rows")
    return y


def moe_backward(x, ids, w, dy, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
                 logits=None) -> dict:
    """Gradients of Eq. 1 (routing ids fixed) for upstream gradient dy (T, d):
    dx, dW_gate, dW_up, dW_down (and the shared experts'), dw (T, k) and,
    when logits are given, dlogits through the full softmax.  fp64."""
    xa, dt = _float_arg(x)
    T, d = xa.shape
    ids = _i32(ids)
    k = ids.shape[1]
    wv = np.ascontiguousarray(w, dtype=np.float64)
    dyv = np.ascontiguousarray(dy, dtype=np.float64)
    g, _ = _float_arg(w_gate)
    u, _ = _float_arg(w_up)
    dn, _ = _float_arg(w_down)
    Ne, F = g.shape[0], g.shape[1]
    n_sh, F_sh = 0, 0
    sg = su = sd = None
    if ws_gate is not None:
        sg, _ = _float_arg(ws_gate)
        su, _ = _float_arg(ws_up)
        sd, _ = _float_arg(ws_down)
        n_sh, F_sh = sg.shape[0], sg.shape[1]
    out = dict(dx=np.empty((T, d)), dW_gate=np.empty((Ne, F, d)), dW_up=np.empty((Ne, F, d)),
               dW_down=np.empty((Ne, d, F)), dw=np.empty((T, k)))
    if n_sh:
        out.update(dWs_gate=np.empty((n_sh, F_sh, d)), dWs_up=np.empty((n_sh, F_sh, d)),
                   dWs_down=np.empty((n_sh, d, F_sh)))
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    if lg is not None:
        out["dlogits"] = np.empty((T, Ne))
    nul = ctypes.c_void_p(0)
    opt = lambda a: _p(a) if a is not None else nul
    rc = _load().orc_moe_backward(
        T, d, Ne, k, F, n_sh, F_sh, dt, _p(xa), _p(ids), _p(wv), opt(lg), _p(g), _p(u), _p(dn),
        opt(sg), opt(su), opt(sd), _p(dyv), _p(out["dx"]), _p(out["dW_gate"]), _p(out["dW_up"]),
        _p(out["dW_down"]), opt(out.get("dWs_gate")), opt(out.get("dWs_up")),
        opt(out.get("dWs_down")), _p(out["dw"]), opt(out.get("dlogits")))
    _check(rc, "moe_backward")
    return out


def moe_backward_rows(rows, x, ids, w, dy, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                      ws_down=None, logits=None) -> dict:
    """The per-token parts of moe_backward for the listed rows: dx, dw and
    (with logits) dlogits rows."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    xa, dt = _float_arg(x)
    T, d = xa.shape
    ids = _i32(ids)
    k = ids.shape[1]
    g, _ = _float_arg(w_gate)
    u, _ = _float_arg(w_up)
    dn, _ = _float_arg(w_down)
    Ne, F = g.shape[0], g.shape[1]
    n_sh, F_sh = 0, 0
    sg = su = sd = None
    if ws_gate is not None:
        sg, _ = _float_arg(ws_gate)
        su, _ = _float_arg(ws_up)
        sd, _ = _float_arg(ws_down)
        n_sh, F_sh = sg.shape[0], sg.shape[1]
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    out = dict(dx=np.empty((len(rows), d)), dw=np.empty((len(rows), k)))
    if lg is not None:
        out["dlogits"] = np.empty((len(rows), Ne))
    nul = ctypes.c_void_p(0)
    opt = lambda a: _p(a) if a is not None else nul
    rc = _load().orc_moe_backward_rows(
        len(rows), _p(rows), d, Ne, k, F, n_sh, F_sh, dt, _p(xa), _p(ids),
        _p(np.ascontiguousarray(w, dtype=np.float64)), opt(lg), _p(g), _p(u), _p(dn), opt(sg),
        opt(su), opt(sd), _p(np.ascontiguousarray(dy, dtype=np.float64)), _p(out["dx"]),
        _p(out["dw"]), opt(out.get("dlogits")))
    _check(rc, "moe_backward_rows")
    return out


def moe_wgrad_rows(x, ids, w, dy, w_gate, w_up, w_down, e: int, f_rows, n_rows) -> dict:
    """Rows f_rows of dW_gate[e], dW_up[e] and rows n_rows of dW_down[e]."""
    xa, dt = _float_arg(x)
    T, d = xa.shape
    ids = _i32(ids)
    k = ids.shape[1]
    g, _ = _float_arg(w_gate)
    u, _ = _float_arg(w_up)
    dn, _ = _float_arg(w_down)
    F = g.shape[1]
    fs, ns = _i32(f_rows), _i32(n_rows)
    out = dict(dW_gate=np.empty((len(fs), d)), dW_up=np.empty((len(fs), d)),
               dW_down=np.empty((len(ns), F)))
    rc = _load().orc_moe_wgrad_rows(
        T, d, k, F, dt, _p(xa), _p(ids), _p(np.ascontiguousarray(w, dtype=np.float64)), _p(g),
        _p(u), _p(dn), _p(np.ascontiguousarray(dy, dtype=np.float64)), int(e), len(fs), _p(fs),
        len(ns), _p(ns), _p(out["dW_gate"]), _p(out["dW_up"]), _p(out["dW_down"]))
    _check(rc, "moe_wgrad_rows")
    return out


def threads(nthreads: int = 0) -> int:
    """How many threads moe_rows runs with for this request."""
    return int(_load().orc_threads(nthreads))


def occult_replay(x, ids, w, placement, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                  ws_down=None):
    """The BRIM-driven ORI->SFD->EPD->SFD->ORI pipeline of Algorithm 2, fp64."""
    xa, dt = _float_arg(x)
    T, d = xa.shape
    ids = _i32(ids)
    k = ids.shape[1]
    L = _i32(placement)
    Nd = L.shape[0]
    wv = np.ascontiguousarray(w, dtype=np.float64)
    g, _ = _float_arg(w_gate)
    u, _ = _float_arg(w_up)
    dn, _ = _float_arg(w_down)
    Ne, F = g.shape[0], g.shape[1]
    n_sh, F_sh = 0, 0
    sg = su = sd = None
    nul = ctypes.c_void_p(0)
    if ws_gate is not None:
        sg, _ = _float_arg(ws_gate)
        su, _ = _float_arg(ws_up)
        sd, _ = _float_arg(ws_down)
        n_sh, F_sh = sg.shape[0], sg.shape[1]
    y = np.empty((T, d), np.float64)
    rc = _load().orc_occult_replay(T, d, Ne, k, Nd, F, n_sh, F_sh, dt, _p(xa), _p(ids), _p(wv),
                                   _p(L), _p(g), _p(u), _p(dn),
                                   _p(sg) if sg is not None else nul,
                                   _p(su) if su is not None else nul,
                                   _p(sd) if sd is not None else nul, _p(y))
    _check(rc, "occult_replay")
    return y


def coact(ids: np.ndarray, Ne: int, placement: np.ndarray):
    """Eq. 3-4 and section 2.2: C (int64), P (fp32), n_sfd, CT, intra share."""
    ids = _i32(ids)
    T, k = ids.shape
    L = _i32(placement)
    Nd = L.shape[0]
    C = np.empty((Ne, Ne), np.int64)
    P = np.empty((Ne, Ne), np.float32)
    n_sfd = ctypes.c_int64(0)
    ct = ctypes.c_double(0)
    intra = ctypes.c_double(0)
    rc = _load().orc_coact(T, k, _p(ids), Ne, Nd, _p(L), _p(C), _p(P), ctypes.byref(n_sfd),
                           ctypes.byref(ct), ctypes.byref(intra))
    _check(rc, "coact")
    return dict(C=C, P=P, n_sfd=n_sfd.value, ct=ct.value, intra=intra.value)


def placement(C: np.ndarray, Nd: int) -> np.ndarray:
    """Algorithm 1 on the integer co-activation counts: (Nd, Ne/Nd) int32."""
    Cc = np.ascontiguousarray(C, dtype=np.int64)
    Ne = Cc.shape[0]
    L = np.empty((Nd, Ne // Nd), np.int32)
    _check(_load().orc_placement(Ne, Nd, _p(Cc), _p(L)), "placement")
    return L
