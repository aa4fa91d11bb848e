"""Seeded synthetic inputs for the MoE layer.

Shared by the tests, the benchmark and the smoke check; holds none of the
layer's arithmetic.  Every tensor gets its own CPU generator seeded with
seed_base + j:

  j=0  latent cluster of each token, uniform over n_c clusters
  j=1  router-logit noise N(0, 1) in fp32; the cluster's experts
       (expert e is in cluster e mod n_c) get +bonus
  j=2  tokens x ~ N(0, 1)
  j=3  routed expert weights ~ N(0, 0.02^2), drawn expert by expert in index
       order: gate (F x d), up (F x d), down (d x F)
  j=4  shared expert weights, drawn the same way
  j=5, j=6  a profiling batch of router logits drawn like j=0 and j=1 (the
       input of the expert similarity table)
  j=7  router (gate projection) weights W_r ~ N(0, 1/d), Ne x d, for the
       workloads that compute their logits as x W_r^T

Values are drawn in fp32 and rounded to the workload's dtype (round to nearest
even, torch's conversion).  Logits stay fp32.  Weight layouts follow
nn.Linear (out, in): the reduction dimension is contiguous.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import DTYPE_BF16, Workload

WEIGHT_STD = 0.02


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32


def _gen(w: Workload, j: int) -> torch.Generator:
    return torch.Generator().manual_seed(w.seed_base + j)


def _logits(w: Workload, T: int, j_cluster: int, j_noise: int) -> torch.Tensor:
    cluster = torch.randint(w.n_c, (T,), generator=_gen(w, j_cluster))
    noise = torch.randn(T, w.Ne, generator=_gen(w, j_noise), dtype=torch.float32)
    member = (torch.arange(w.Ne)[None, :] % w.n_c) == cluster[:, None]
    return (noise + w.bonus * member.to(torch.float32)).contiguous()


def make_logits(w: Workload, T: int | None = None) -> torch.Tensor:
    return _logits(w, w.T if T is None else T, 0, 1)


def make_profile_logits(w: Workload, T: int = 16384) -> torch.Tensor:
    """A profiling batch from the same distribution, drawn independently."""
    return _logits(w, T, 5, 6)


def make_x(w: Workload, T: int | None = None) -> torch.Tensor:
    T = w.T if T is None else T
    x = torch.randn(T, w.d, generator=_gen(w, 2), dtype=torch.float32)
    return x.to(torch_dtype(w)).contiguous()


def _expert_weights(w: Workload, n_exp: int, F: int, j: int):
    dt = torch_dtype(w)
    g = _gen(w, j)
    gate = torch.empty(n_exp, F, w.d, dtype=dt)
    up = torch.empty(n_exp, F, w.d, dtype=dt)
    down = torch.empty(n_exp, w.d, F, dtype=dt)
    for e in range(n_exp):
        gate[e] = (torch.randn(F, w.d, generator=g) * WEIGHT_STD).to(dt)
        up[e] = (torch.randn(F, w.d, generator=g) * WEIGHT_STD).to(dt)
        down[e] = (torch.randn(w.d, F, generator=g) * WEIGHT_STD).to(dt)
    return gate, up, down


def make_weights(w: Workload):
    """Routed (Ne, F, d), (Ne, F, d), (Ne, d, F) in the workload dtype."""
    return _expert_weights(w, w.Ne, w.F, 3)


def make_shared_weights(w: Workload):
    """Shared (n_shared, F_shared, d) x2 and (n_shared, d, F_shared), or Nones."""
    if w.n_shared == 0:
        return None, None, None
    return _expert_weights(w, w.n_shared, w.F_shared, 4)


def make_router_weights(w: Workload) -> torch.Tensor:
    """Gate projection W_r (Ne, d) in the workload dtype: logits x W_r^T then
    have unit variance for x ~ N(0, 1)."""
    wr = torch.randn(w.Ne, w.d, generator=_gen(w, 7), dtype=torch.float32) / np.sqrt(w.d)
    return wr.to(torch_dtype(w)).contiguous()


def contiguous_placement(w: Workload) -> np.ndarray:
    """Group g holds experts g*n .. g*n+n-1, in that order."""
    return np.arange(w.Ne, dtype=np.int32).reshape(w.Nd, w.n)


def make_all(w: Workload, T: int | None = None) -> dict:
    gate, up, down = make_weights(w)
    sg, su, sd = make_shared_weights(w)
    return dict(logits=make_logits(w, T), x=make_x(w, T), w_gate=gate, w_up=up, w_down=down,
                ws_gate=sg, ws_up=su, ws_down=sd, placement=contiguous_placement(w),
                w_router=make_router_weights(w) if w.gated else None)


def sample_rows(T: int, count: int, seed: int = 99) -> np.ndarray:
    """A sorted, seeded sample of distinct token rows (always holding 0 and T-1)."""
    if count >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    rows = rng.choice(T, size=count, replace=False)
    rows[0], rows[-1] = 0, T - 1
    return np.unique(rows).astype(np.int64)
