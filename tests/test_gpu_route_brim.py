"""GPU parity of the integer steps against the oracle, bit for bit: routing
ids (with both pruning rules), BRIM_0 / BRIM_1 and their condensed form, the
co-activation counts C, P, N_sfd, CT and the intra share.  The BRIM and the
statistics are built on the oracle's routing, so every expected value comes
from the oracle alone.  Full workload
sizes (the sizes the benchmark runs) plus ragged and degenerate shapes."""
import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import W_RTOL, inputs, oracle_route, weight_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def gpu_route(wl, logits, placement):
    desc = occ.desc_of(wl, T=logits.shape[0])
    ids = torch.empty(logits.shape[0], wl.k, dtype=torch.int32, device="cuda")
    w = torch.empty(logits.shape[0], wl.k, dtype=torch.float32, device="cuda")
    occ.occ_route(desc, logits.cuda(), placement, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


FULL = [W.TINY_F32, W.OLMOE, W.DEEPSEEK, W.OLMOE_PRUNED, W.QWEN]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_route_full_size(wl):
    logits = synth.make_logits(wl)
    L = synth.contiguous_placement(wl)
    ids, w = gpu_route(wl, logits, L)
    ids_o, w_o = oracle.route(logits.numpy(), wl.k, L, wl.prune_rule, wl.prune_groups)
    assert np.array_equal(ids, ids_o)
    np.testing.assert_allclose(w, w_o, rtol=W_RTOL, atol=0)
    # and within the error bound of the device's fp32 softmax arithmetic
    assert np.all(np.abs(w - w_o) <= weight_bound(logits.numpy(), ids_o) * w_o)
    if wl.prune_rule:
        grp = np.repeat(np.arange(wl.Nd), wl.n)
        spans = np.array([len(set(grp[r].tolist())) for r in ids])
        assert spans.max() <= wl.prune_groups  # CT's bound under pruning


@pytest.mark.parametrize("rule", [W.PRUNE_TRAVERSE, W.PRUNE_GROUPSUM])
@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_route_pruning(rule, G):
    wl = W.scaled(W.OLMOE, 4099, prune_rule=rule, prune_groups=G)
    logits = synth.make_logits(wl)
    L = np.random.default_rng(G).permutation(64).astype(np.int32).reshape(8, 8)
    ids, w = gpu_route(wl, logits, L)
    ids_o, w_o = oracle.route(logits.numpy(), wl.k, L, rule, G)
    assert np.array_equal(ids, ids_o)
    np.testing.assert_allclose(w, w_o, rtol=W_RTOL)


def test_route_signed_zeros_and_infinities():
    # -0 and +0 compare equal (ties to the lower index); infinities order
    # like any other value
    vals = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)
    for Ne, k, Nd in [(64, 8, 8), (200, 6, 8)]:
        wl = W.Workload(f"zeros_{Ne}", 9, T=513, d=64, Ne=Ne, k=k, Nd=Nd, F=64)
        pick = np.random.default_rng(Ne).integers(0, len(vals), (513, Ne))
        logits = torch.from_numpy(vals[pick])
        L = synth.contiguous_placement(wl)
        ids, _ = gpu_route(wl, logits, L)
        ids_o, _ = oracle.route(logits.numpy(), k, L)
        assert np.array_equal(ids, ids_o), Ne


@pytest.mark.parametrize("Ne,k,rule", [(64, 8, W.PRUNE_OFF), (60, 4, W.PRUNE_OFF),
                                       (64, 8, W.PRUNE_GROUPSUM), (200, 6, W.PRUNE_OFF)])
def test_route_nan_logits_rank_last(Ne, k, rule):
    """A NaN logit ranks as -inf: the ids are those of the logits with every
    NaN replaced by -inf (ties to the lower index), so they stay distinct and
    in range; the weights are unspecified then."""
    wl = W.Workload(f"nan_{Ne}", 9, T=1031, d=64, Ne=Ne, k=k, Nd=4, F=64,
                    prune_rule=rule, prune_groups=2 if rule else 0)
    rng = np.random.default_rng(Ne + k)
    lg = rng.standard_normal((1031, Ne)).astype(np.float32)
    lg[rng.random((1031, Ne)) < 0.2] = np.nan
    lg[:7] = np.nan                        # rows of NaN only
    lg[7:11, : Ne // 2] = -np.inf          # -inf beside NaN
    lg[7:11, Ne // 2:] = np.nan
    L = synth.contiguous_placement(wl)
    ids, _ = gpu_route(wl, torch.from_numpy(lg), L)
    ids_o, _ = oracle.route(np.where(np.isnan(lg), -np.inf, lg).astype(np.float32), k, L, rule,
                            wl.prune_groups)
    assert np.array_equal(ids, ids_o)


def test_route_ties_and_wide_expert_counts():
    # integer-valued logits: many exact ties, broken toward the lower index
    # Ne <= 64 without pruning takes the 16-lanes-per-token kernel (k up to
    # 32: two recorded rounds per lane), the others the wave kernel
    for Ne, k, Nd in [(8, 2, 2), (8, 8, 2), (12, 5, 3), (64, 8, 8), (60, 17, 4), (256, 8, 16),
                      (130, 5, 10), (32, 32, 4)]:
        wl = W.Workload(f"ties_{Ne}", 9, T=777, d=64, Ne=Ne, k=k, Nd=Nd, F=64)
        g = torch.Generator().manual_seed(Ne)
        logits = torch.randint(-3, 4, (777, Ne), generator=g).float()
        L = synth.contiguous_placement(wl)
        ids, w = gpu_route(wl, logits, L)
        ids_o, w_o = oracle.route(logits.numpy(), k, L)
        assert np.array_equal(ids, ids_o), (Ne, k)
        np.testing.assert_allclose(w, w_o, rtol=W_RTOL)
        for rule in (W.PRUNE_TRAVERSE, W.PRUNE_GROUPSUM):
            G = max(1, -(-k // (Ne // Nd)))
            wlp = W.scaled(wl, 777, prune_rule=rule, prune_groups=G)
            ids, _ = gpu_route(wlp, logits, L)
            ids_o, _ = oracle.route(logits.numpy(), k, L, rule, G)
            assert np.array_equal(ids, ids_o), (Ne, k, rule)


def gpu_brim(wl, ids_t, w_t, placement, dense=True):
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    b = occ.occ_build_brim(desc, ids_t.cuda(), w_t.cuda(), placement, ws, dense)
    torch.cuda.synchronize()
    v = lambda p, shape, dt=torch.int32: occ.ws_view(ws, p, shape, dt).cpu().numpy()
    T, k, Nd, Ne = wl.T, wl.k, wl.Nd, wl.Ne
    sfd_off = v(b.sfd_off, (Nd + 1,))
    N_sfd = int(sfd_off[-1])
    return dict(brim0=v(b.brim0, (Nd, T)), sfd_off=sfd_off, epd_off=v(b.epd_off, (Ne + 1,)),
                epd_src=v(b.epd_src, (T * k,)), epd_w=v(b.epd_w, (T * k,), torch.float32),
                tok_epd=v(b.tok_epd, (T, k)), tile_off=v(b.tile_off, (Ne + 1,)),
                down_rows=v(b.down_rows, (T * k,)), first_cnt=v(b.first_cnt, (Ne,)),
                brim1=v(b.brim1, (wl.n * N_sfd,)) if dense else None)


def tile_schedule(wl, loads, bm):
    """The grouped GEMMs' row tiles per expert: ceil(rows / bm), and on the
    320-row build, extra tiles until the up-projection's tiles (ceil(F / 128)
    column tiles per row tile) fill their last round of the CUs: one at a
    time, at most 64, each to the expert whose tiles hold the most rows
    (ties to the lower placement position) among those whose tiles could
    still lose a 16-row block."""
    from fractions import Fraction
    vt = (loads + bm - 1) // bm
    if bm != 320:
        return vt
    cols = -(-wl.F // 128)
    slots = torch.cuda.get_device_properties(0).multi_processor_count
    t0 = int(vt.sum())
    rounds = -(-t0 * cols // slots)
    for _ in range(min(rounds * slots // cols - t0, 64)):
        cand = [p for p in range(len(vt)) if 0 < vt[p] < -(-loads[p] // 16)]
        if not cand:
            break
        best = max(cand, key=lambda p: (Fraction(int(loads[p]), int(vt[p])), -p))
        vt[best] += 1
    return vt


def check_brim(wl, placement, ids_g=None, w_g=None):
    """The device's BRIM from the oracle's routing (ids, fp32 weights)
    against the oracle's literal counter loops on the same routing."""
    if ids_g is None:
        ids_g, w_g = oracle.route(synth.make_logits(wl).numpy(), wl.k, placement, wl.prune_rule,
                                  wl.prune_groups)
    w_g = np.asarray(w_g, dtype=np.float32)
    b = gpu_brim(wl, torch.from_numpy(ids_g), torch.from_numpy(w_g), placement)
    r = oracle.brim1(ids_g, w_g.astype(np.float64), wl.Ne, placement)
    assert np.array_equal(b["brim0"], r["brim0"])
    assert np.array_equal(b["sfd_off"], r["sfd_off"])
    assert np.array_equal(b["epd_off"], r["epd_off"])
    assert np.array_equal(b["epd_src"], r["epd_src"])
    assert np.array_equal(b["epd_w"].astype(np.float64), r["epd_w"])  # a copy of w
    assert np.array_equal(b["brim1"], r["brim1"])
    # tok_epd is the inverse map: EPD row of (t, j) carries t's SFD row for that group
    T, k = wl.T, wl.k
    rows = b["tok_epd"].reshape(-1)
    assert np.array_equal(np.sort(rows), np.arange(T * k))
    grp = np.empty(wl.Ne, np.int64)
    for g, row in enumerate(placement):
        grp[row] = g
    tt = np.repeat(np.arange(T), k)
    assert np.array_equal(b["epd_src"][rows], b["brim0"][grp[ids_g.reshape(-1)], tt])
    # the library's row-tile capacity: 32 for fp32; bf16 takes 128-row tiles
    # when the experts average fewer than 96 rows, else tiles of up to 320
    bm = (32 if wl.dtype != W.DTYPE_BF16 else 128 if wl.T * wl.k < 96 * wl.Ne else 320)
    loads = np.diff(b["epd_off"])
    assert np.array_equal(np.diff(b["tile_off"]), tile_schedule(wl, loads, bm))
    # merge order: per expert, the EPD rows that are the first (lowest-slot)
    # contributor to their SFD row, then the others, each in token order
    pos = np.empty(wl.Ne, np.int64)
    pos[placement.reshape(-1)] = np.arange(wl.Ne)
    p_of = pos[ids_g]                                   # T x k placement positions
    g_of = p_of // wl.n
    lower_same = (g_of[:, :, None] == g_of[:, None, :]) & (p_of[:, None, :] < p_of[:, :, None])
    is_first = ~lower_same.any(2)
    erow = b["tok_epd"]
    for p in range(wl.Ne):
        lo, hi = b["epd_off"][p], b["epd_off"][p + 1]
        mine = p_of == p
        firsts = np.sort(erow[mine & is_first])
        rest = np.sort(erow[mine & ~is_first])
        assert b["first_cnt"][p] == len(firsts)
        assert np.array_equal(b["down_rows"][lo:hi], np.concatenate([firsts, rest]))
    # every SFD row has exactly one first contributor
    assert int(is_first.sum()) == int(b["sfd_off"][-1])
    return b


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_brim_full_size(wl):
    check_brim(wl, synth.contiguous_placement(wl))


def test_brim_rescheduled_placement():
    wl = W.OLMOE
    logits = synth.make_logits(wl)
    L0 = synth.contiguous_placement(wl)
    ids_o, _ = oracle.route(logits.numpy(), wl.k, L0)
    L1 = oracle.placement(oracle.coact(ids_o, wl.Ne, L0)["C"], wl.Nd)
    b0 = check_brim(wl, L0)
    b1 = check_brim(wl, L1)
    assert b1["sfd_off"][-1] < b0["sfd_off"][-1]  # rescheduling lowers CT here


@pytest.mark.parametrize("shape", [
    dict(T=1), dict(T=5), dict(T=1023), dict(T=1025), dict(T=3000, Nd=1),
    # batches of up to 512 tokens and 1024 routing entries take the
    # one-workgroup BRIM: its edges and its largest tables
    dict(T=128, k=8), dict(T=129, k=8), dict(T=512, k=2), dict(T=513, k=1),
    dict(T=512, Ne=256, Nd=64, k=32), dict(T=32, Ne=256, Nd=64, k=32),
    dict(T=64, Ne=256, Nd=1, k=3), dict(T=200, Ne=130, Nd=10, k=5, F=1408),
    dict(T=500, Ne=8, Nd=2, k=2, F=1408),  # 320-row tiles: the schedule takes extra row tiles
    dict(T=2000, Ne=16, Nd=16, k=4), dict(T=1500, k=1), dict(T=999, Ne=256, Nd=64, k=8),
    dict(T=1100, Ne=60, Nd=4, k=4),
    # schedules that take extra row tiles, with several experts per lane
    dict(T=9000, Ne=256, Nd=64, k=8, F=1024), dict(T=20000, Ne=130, Nd=10, k=5, F=1408),
])
def test_brim_ragged_and_degenerate(shape):
    base = dict(Ne=64, Nd=8, k=8, F=64)
    base.update(shape)
    wl = W.Workload("brim_edge", 11, d=64, n_c=4, **base)
    check_brim(wl, synth.contiguous_placement(wl))


def test_brim_expert_and_group_with_no_tokens():
    wl = W.Workload("starved", 12, T=2000, d=64, Ne=16, k=2, Nd=4, F=64, n_c=2)
    logits = synth.make_logits(wl)
    logits[:, 4:8] = -50.0   # group 1 never chosen
    logits[:, 13] = -50.0    # nor expert 13
    L = synth.contiguous_placement(wl)
    ids, w = oracle.route(logits.numpy(), wl.k, L)
    assert not np.isin(ids, [4, 5, 6, 7, 13]).any()
    b = check_brim(wl, L, ids, w)
    assert b["sfd_off"][1] == b["sfd_off"][2]
    assert b["epd_off"][13] == b["epd_off"][14]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_coactivation_stats(wl):
    logits = synth.make_logits(wl)
    L = synth.contiguous_placement(wl)
    ids, _ = oracle.route(logits.numpy(), wl.k, L, wl.prune_rule, wl.prune_groups)
    desc = occ.desc_of(wl)
    C = torch.empty(wl.Ne, wl.Ne, dtype=torch.int32, device="cuda")
    P = torch.empty(wl.Ne, wl.Ne, dtype=torch.float32, device="cuda")
    n_sfd = torch.empty(1, dtype=torch.int64, device="cuda")
    ct = torch.empty(1, dtype=torch.float64, device="cuda")
    intra = torch.empty(1, dtype=torch.float64, device="cuda")
    for _ in range(2):  # a second call must start from zero again
        occ.occ_coactivation_stats(desc, torch.from_numpy(ids).cuda(), L, C, P, n_sfd, ct, intra)
    torch.cuda.synchronize()
    st = oracle.coact(ids, wl.Ne, L)
    assert np.array_equal(C.cpu().numpy(), st["C"])
    assert np.array_equal(P.cpu().numpy(), st["P"])
    assert int(n_sfd.item()) == st["n_sfd"]
    assert float(ct.item()) == st["ct"]
    assert float(intra.item()) == st["intra"]
    lo = -(-wl.k * wl.Nd // wl.Ne)
    assert lo <= st["ct"] <= min(wl.k, wl.Nd)


def test_coactivation_wide_expert_count_uses_global_histogram():
    wl = W.Workload("wide", 13, T=3000, d=64, Ne=128, k=6, Nd=8, F=64, n_c=16)
    logits = synth.make_logits(wl)
    L = synth.contiguous_placement(wl)
    ids, _ = oracle.route(logits.numpy(), wl.k, L)
    desc = occ.desc_of(wl)
    C = torch.empty(128, 128, dtype=torch.int32, device="cuda")
    P = torch.empty(128, 128, dtype=torch.float32, device="cuda")
    n_sfd = torch.empty(1, dtype=torch.int64, device="cuda")
    ct = torch.empty(1, dtype=torch.float64, device="cuda")
    intra = torch.empty(1, dtype=torch.float64, device="cuda")
    occ.occ_coactivation_stats(desc, torch.from_numpy(ids).cuda(), L, C, P, n_sfd, ct, intra)
    torch.cuda.synchronize()
    st = oracle.coact(ids, 128, L)
    assert np.array_equal(C.cpu().numpy(), st["C"]) and np.array_equal(P.cpu().numpy(), st["P"])
    assert float(ct.item()) == st["ct"]
