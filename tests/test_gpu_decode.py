"""GPU parity of the decode path: the gate projection g(x) (paper section
2.1) against the fp64 oracle within fp32 accumulation's error bound, routing
on the device's own logits bit for bit, the gated layer to the layer
tolerance, and both GEMM tile sizes around the point where the library
switches between them (128-row tiles when T*k < 96*Ne)."""
import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import (TOL, W_RTOL, bits, forward, inputs, oracle_rows, routed_to_counts,
                        row_err, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def gpu_gate(wl, x, wr):
    desc = occ.desc_of(wl, T=x.shape[0])
    lg = torch.empty(x.shape[0], wl.Ne, dtype=torch.float32, device="cuda")
    occ.occ_gate(desc, x.cuda(), wr.cuda(), lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy()


def check_gate(wl, T):
    x = synth.make_x(wl, T)
    wr = synth.make_router_weights(wl)
    got = gpu_gate(wl, x, wr)
    ref = oracle.gate(np.arange(T), bits(x), bits(wr))
    # fp32 accumulation of d exact products: |err| <= d u / (1 - d u) sum |x_i w_i|
    u = 2.0 ** -24
    mag = np.abs(x.double().numpy()) @ np.abs(wr.double().numpy()).T
    bound = wl.d * u / (1 - wl.d * u) * mag
    assert np.all(np.abs(got - ref) <= bound)
    return x, wr, got


@pytest.mark.parametrize("wl,T", [
    (W.OLMOE_DECODE, 512),
    (W.OLMOE_DECODE, 37),                                            # ragged token block
    (W.scaled(W.QWEN, 100, name="qwen_gate_T100", gated=True), 100),  # Ne = 60
    (W.scaled(W.OLMOE, 50, name="ne256_gate_T50", Ne=256, Nd=16, gated=True), 50),
    (W.scaled(W.TINY_F32, 70, name="tiny_gate_T70", gated=True), 70),  # fp32 path
], ids=["decode512", "ragged37", "ne60", "ne256", "fp32"])
def test_gate_matches_oracle(wl, T):
    check_gate(wl, T)


def gated_forward(wl, dev, L):
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=synth.torch_dtype(wl), device="cuda")
    occ.occ_moe_forward_gated(desc, dev["x"], dev["w_router"], L, dev["w_gate"], dev["w_up"],
                              dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    torch.cuda.synchronize()
    v = occ.occ_forward_views(desc, ws)
    lg = occ.ws_view(ws, v.logits, (wl.T, wl.Ne), torch.float32).cpu().numpy()
    ids = occ.ws_view(ws, v.ids, (wl.T, wl.k), torch.int32).cpu().numpy()
    w = occ.ws_view(ws, v.w, (wl.T, wl.k), torch.float32).cpu().numpy()
    return y, lg, ids, w


def gate_error_bound(x, wr, d):
    """Per (token, expert) bound on |device fp32 logit - exact logit|: fp32
    accumulation of d exact bf16 products, d u / (1 - d u) sum |x_i w_i|."""
    u = 2.0 ** -24
    mag = np.abs(x.double().numpy()) @ np.abs(wr.double().numpy()).T
    return d * u / (1 - d * u) * mag


@pytest.mark.parametrize("wl", [W.OLMOE_DECODE, W.scaled(W.DEEPSEEK, 261)],
                         ids=["olmoe_decode", "deepseek_shared"])
def test_gated_forward_matches_oracle(wl):
    """The gated layer against the oracle's own pipeline: its fp64 gate
    rounded to fp32, its router, its Eq. 1.  The device's logits differ from
    the oracle's by at most E = (fp32 accumulation bound) + (the oracle's
    fp32 rounding) per entry, so a token's ids must equal the oracle's bit
    for bit unless two of its logits that decide the ordered top-k (the
    k+1 largest) lie within 2E of each other; there the device's list must
    still be a valid ordered top-k under that bound.  y and w are compared
    on the tokens whose ids equal the oracle's."""
    inp = inputs(wl)  # the DeepSeek case shares the plain forward tests' tensors
    if inp["w_router"] is None:
        inp = dict(inp, w_router=synth.make_router_weights(wl))
    dev = to_dev(inp)
    L = inp["placement"]
    y, lg, ids, w = gated_forward(wl, dev, L)
    # the logits in the workspace are occ_gate's
    assert np.array_equal(lg, gpu_gate(wl, inp["x"], inp["w_router"]))
    # the oracle's routing on its own logits
    lg_o = oracle.gate(np.arange(wl.T), bits(inp["x"]), bits(inp["w_router"]))
    ids_o, w_o = oracle.route(lg_o.astype(np.float32), wl.k, L)
    E = gate_error_bound(inp["x"], inp["w_router"], wl.d) + 2.0 ** -24 * np.abs(lg_o)
    Et = E.max(1)
    srt = -np.sort(-lg_o, axis=1)[:, :wl.k + 1]
    close = (srt[:, :-1] - srt[:, 1:] <= 2 * Et[:, None]).any(1)
    same = (ids == ids_o).all(1)
    # a differing token must be one whose deciding logits are within 2E
    assert np.all(same | close), np.flatnonzero(~(same | close))[:10]
    for t in np.flatnonzero(~same):
        sel = ids[t].astype(np.int64)
        assert len(set(sel.tolist())) == wl.k
        l = lg_o[t]
        # ordered within the bound, and no unselected expert clearly above
        assert np.all(l[sel[:-1]] >= l[sel[1:]] - 2 * Et[t])
        rest = np.setdiff1d(np.arange(wl.Ne), sel)
        assert l[sel].min() >= l[rest].max() - 2 * Et[t]
    print(f"{wl.name}: {(~same).sum()} of {wl.T} tokens route differently from the oracle "
          f"({close.sum()} within the bound)")
    assert same.mean() >= 0.99, same.mean()
    rows = np.flatnonzero(same)
    # weights: the fp32 softmax bound plus the logit error, |dw/w| <= 2 max E
    rel = np.abs(w[rows] - w_o[rows]) / w_o[rows]
    assert np.all(rel <= W_RTOL + 2 * Et[rows, None]), rel.max()
    ref = oracle_rows(wl, inp, rows, ids_o[rows], w_o[rows])
    assert row_err(y.float().cpu().numpy().astype(np.float64)[rows], ref).max() <= TOL[wl.dtype]
    # the same layer through occ_moe_forward on the device's logits:
    # identical routing, equal output up to the order of the fp32 atomic adds
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    y2 = torch.empty_like(y)
    occ.occ_moe_forward(desc, dev["x"], torch.from_numpy(lg).cuda(), L, dev["w_gate"],
                        dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"],
                        y2, ws)
    torch.cuda.synchronize()
    assert row_err(y2.float().cpu().numpy(), y.float().cpu().numpy()).max() <= 1e-2


@pytest.mark.parametrize("T", [767, 768], ids=["m128_tiles", "m320_tiles"])
def test_forward_on_both_sides_of_the_tile_switch(T):
    """OLMoE shape: T*k < 96*Ne below 768 tokens (128-row tiles), not at 768
    (tiles of up to 320 rows); both against the oracle on sampled rows."""
    wl = W.scaled(W.OLMOE, T)
    inp = inputs(wl)
    dev = to_dev(inp)
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], inp["placement"], dev["w_gate"],
                        dev["w_up"], dev["w_down"], None, None, None, y, ws)
    torch.cuda.synchronize()
    v = occ.occ_forward_views(desc, ws)
    ids = occ.ws_view(ws, v.ids, (wl.T, wl.k), torch.int32).cpu().numpy()
    w = occ.ws_view(ws, v.w, (wl.T, wl.k), torch.float32).cpu().numpy()
    ids_o, w_o = oracle.route(inp["logits"].numpy(), wl.k, inp["placement"])
    assert np.array_equal(ids, ids_o)
    np.testing.assert_allclose(w, w_o, rtol=W_RTOL, atol=0)
    tile_off = occ.ws_view(ws, v.brim.tile_off, (wl.Ne + 1,), torch.int32).cpu().numpy()
    epd_off = occ.ws_view(ws, v.brim.epd_off, (wl.Ne + 1,), torch.int32).cpu().numpy()
    bm = 128 if T * wl.k < 96 * wl.Ne else 320  # tile capacity in rows
    assert np.array_equal(np.diff(tile_off), (np.diff(epd_off) + bm - 1) // bm)
    rows = synth.sample_rows(wl.T, 128, seed=T)
    ref = oracle_rows(wl, inp, rows, ids_o, w_o)
    assert row_err(y.float().cpu().numpy()[rows], ref).max() <= TOL[wl.dtype]


def test_small_tile_split_edges():
    """Small batches (T*k < 96*Ne: 128-row tiles, and with the atomic merge
    one down-projection launch into rows the dispatch zeroed): experts whose
    row counts straddle one MFMA block (15-17), half a tile (63-65), one tile
    (127-129) and two (255-257, shared out over three tiles), besides no rows
    and 1 -- row by row against the oracle under both merges."""
    counts = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 2, 35]
    wl = W.Workload("small_tile_edges", 22, T=sum(counts) // 2, d=256, Ne=16, k=2, Nd=4, F=256,
                    n_c=4, bonus=1.5)
    assert wl.T * wl.k < 96 * wl.Ne
    inp = synth.make_all(wl)
    inp["logits"] = routed_to_counts(counts, wl.k, seed=22)
    ids, w = oracle.route(inp["logits"].numpy(), wl.k, inp["placement"])
    assert np.array_equal(np.bincount(ids.reshape(-1), minlength=wl.Ne), counts)
    ref = oracle_rows(wl, inp, np.arange(wl.T), ids, w)
    dev = to_dev(inp)
    for flags in (0, occ.OCC_FLAG_DETERMINISTIC):
        y, ws, v, _ = forward(wl, inp, dev=dev, flags=flags)
        tile_off = occ.ws_view(ws, v.brim.tile_off, (wl.Ne + 1,), torch.int32).cpu().numpy()
        epd_off = occ.ws_view(ws, v.brim.epd_off, (wl.Ne + 1,), torch.int32).cpu().numpy()
        assert np.array_equal(np.diff(tile_off), (np.diff(epd_off) + 127) // 128)
        err = row_err(y, ref)
        assert err.max() <= TOL[wl.dtype], f"flags {flags}: max per-row rel err {err.max():.3e}"
