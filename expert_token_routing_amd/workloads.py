"""The five synthetic MoE-layer workloads the layer is tested and measured on.

Shapes follow the models the Occult paper evaluates (Table 2 of "Occult:
Optimizing Collaborative Communication across Experts for Accelerated Parallel
MoE Training and Inference" gives k and the expert count Ne for OLMoE,
Qwen1.5-MoE and DeepSeek-MoE).  Hidden size d, FFN width F and the shared
experts are the usual published shapes of those models.  Router logits are
synthetic: unit Gaussian noise plus a bonus on the experts of one latent
cluster per token, clusters strided over the expert index (expert e belongs to
cluster e mod n_c), which spreads each cluster over every contiguous group.

This module holds sizes and seeds only; no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field

PRUNE_OFF = 0
PRUNE_TRAVERSE = 1  # groups gathered by walking the top-k list (paper, section 3.3)
PRUNE_GROUPSUM = 2  # groups ranked by the sum of their top-k logits
PRUNE_SIMILARITY = 3  # TRAVERSE's groups, other experts replaced by the most similar (A.3 table)

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the workload list; fixes the seeds
    T: int              # tokens in the batch (ORI rows)
    d: int              # hidden size
    Ne: int             # routed experts
    k: int              # top-k
    Nd: int             # expert groups (the devices of expert parallelism)
    F: int              # routed expert FFN width
    n_shared: int = 0   # shared (always-on) experts
    F_shared: int = 0
    dtype: int = DTYPE_BF16
    n_c: int = 8        # latent clusters of the synthetic logits
    bonus: float = 1.5  # logit bonus on the token's cluster
    prune_rule: int = PRUNE_OFF
    prune_groups: int = 0
    gated: bool = False  # logits computed on the device as x W_r^T (gate projection)
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def n(self) -> int:
        return self.Ne // self.Nd

    @property
    def seed_base(self) -> int:
        return 1234 + 100 * self.index

    @property
    def dtype_name(self) -> str:
        return "f32" if self.dtype == DTYPE_F32 else "bf16"

    def flops_per_token(self) -> int:
        """Algorithmic FLOPs per token: k SwiGLU experts plus the shared ones."""
        return 2 * self.k * self.d * 3 * self.F + 2 * self.n_shared * self.d * 3 * self.F_shared


TINY_F32 = Workload("tiny_fp32_t256", 1, T=256, d=128, Ne=8, k=2, Nd=2, F=256,
                    dtype=DTYPE_F32, n_c=2, bonus=2.0)
OLMOE = Workload("olmoe_t8192", 2, T=8192, d=2048, Ne=64, k=8, Nd=8, F=1024,
                 n_c=8, bonus=1.5)
DEEPSEEK = Workload("deepseek_t16384", 3, T=16384, d=2048, Ne=64, k=6, Nd=8, F=1408,
                    n_shared=2, F_shared=1408, n_c=16, bonus=1.5)
OLMOE_PRUNED = Workload("olmoe_pruned2_t32768", 4, T=32768, d=2048, Ne=64, k=8, Nd=8, F=1024,
                        n_c=8, bonus=1.5, prune_rule=PRUNE_GROUPSUM, prune_groups=2)
QWEN = Workload("qwen_t65536", 5, T=65536, d=2048, Ne=60, k=4, Nd=4, F=1408,
                n_shared=1, F_shared=5632, n_c=10, bonus=1.0)

# The pruned OLMoE shape under expert-similarity-based pruning (section 3.3);
# its table is built from a separate profiling batch (synth.make_profile_logits).
OLMOE_SIM = Workload("olmoe_sim2_t32768", 6, T=32768, d=2048, Ne=64, k=8, Nd=8, F=1024,
                     n_c=8, bonus=1.5, prune_rule=PRUNE_SIMILARITY, prune_groups=2)

# Decode regime: one step of a batch of 512 concurrent requests (the decoding
# batch of the paper's Figure 10) through the OLMoE-shaped layer, its router
# logits computed from the tokens by the gate projection.
OLMOE_DECODE = Workload("olmoe_decode_t512", 7, T=512, d=2048, Ne=64, k=8, Nd=8, F=1024,
                        n_c=8, bonus=1.5, gated=True)

ALL = [TINY_F32, OLMOE, DEEPSEEK, OLMOE_PRUNED, QWEN, OLMOE_SIM, OLMOE_DECODE]
BY_NAME = {w.name: w for w in ALL}


def scaled(w: Workload, T: int, name: str | None = None, **over) -> Workload:
    """Same layer shape and seeds with a different token count (or fields)."""
    kw = dict(w.__dict__)
    kw.pop("extra", None)
    kw.update(T=T, name=name or f"{w.name}_T{T}")
    kw.update(over)
    return Workload(**kw)


# The pruned OLMoE batch again under the TRAVERSE rule (same inputs).
OLMOE_PRUNED_TRAVERSE = scaled(OLMOE_PRUNED, OLMOE_PRUNED.T, name=OLMOE_PRUNED.name + "_traverse",
                               prune_rule=PRUNE_TRAVERSE)
BY_NAME[OLMOE_PRUNED_TRAVERSE.name] = OLMOE_PRUNED_TRAVERSE
