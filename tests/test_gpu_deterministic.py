"""The deterministic merge (OCC_FLAG_DETERMINISTIC: every EPD row's fp32
down-projection result stored, each SFD row summed over its group's experts
in ascending placement position, no atomic adds; the paper's serial
aggregation over local experts, appendix A.2).  Parity with the oracle at the
usual tolerances, and bitwise identity of every output across runs, across a
graph replay and across the two merge schedules that the atomic path would
use (one launch for small batches, first/rest otherwise)."""
import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import TOL, W_RTOL, bits, oracle_rows, row_err, to_dev

pytestmark = pytest.mark.gpu

DET = occ.OCC_FLAG_DETERMINISTIC


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def run_forward(wl, inp, dev, flags=DET, L=None):
    desc = occ.desc_of(wl, flags=flags)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=synth.torch_dtype(wl), device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], inp["placement"] if L is None else L,
                        dev["w_gate"], dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"],
                        dev["ws_down"], y, ws)
    torch.cuda.synchronize()
    return y, ws, desc


@pytest.mark.parametrize("wl", [
    W.scaled(W.OLMOE, 1100, name="det_olmoe_T1100"),              # first/rest regime
    W.scaled(W.OLMOE, 300, name="det_olmoe_T300"),                # one-launch regime
    W.scaled(W.DEEPSEEK, 261, name="det_deepseek_T261"),          # shared experts, F = 1408
    W.Workload("det_ragged", 31, T=333, d=192, Ne=16, k=5, Nd=4, F=320, n_c=4, bonus=1.5),
    W.scaled(W.TINY_F32, 500, name="det_tiny_f32"),               # fp32 path
], ids=lambda w: w.name)
def test_deterministic_forward_matches_oracle_and_repeats_bitwise(wl):
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    y0, ws0, desc = run_forward(wl, inp, dev)
    y1, _, _ = run_forward(wl, inp, dev)
    assert torch.equal(y0, y1)
    ids, w = oracle.route(inp["logits"].numpy(), wl.k, inp["placement"])
    ref = oracle_rows(wl, inp, np.arange(wl.T), ids, w)
    err = row_err(y0.float().cpu().numpy(), ref)
    assert err.max() <= TOL[wl.dtype], err.max()
    # stage one is materialised: the SFD rows, added in ascending group order
    # in fp32 (plus the shared experts) and cast once, give y bit for bit
    v = occ.occ_forward_views(desc, ws0)
    sfd_off = occ.ws_view(ws0, v.brim.sfd_off, (wl.Nd + 1,), torch.int32).cpu().numpy()
    n_sfd = int(sfd_off[-1])
    sfd = occ.ws_view(ws0, v.sfd_out, (n_sfd, wl.d), torch.float32).cpu()
    b0 = occ.ws_view(ws0, v.brim.brim0, (wl.Nd, wl.T), torch.int32).cpu().numpy()
    acc = torch.zeros(wl.T, wl.d, dtype=torch.float32)
    for gi in range(wl.Nd):
        sel = np.nonzero(b0[gi] >= 0)[0]
        acc[sel] = acc[sel] + sfd[b0[gi][sel]]
    if wl.n_shared:
        acc = acc + occ.ws_view(ws0, v.y_shared, (wl.T, wl.d), torch.float32).cpu()
    assert torch.equal(acc.to(y0.dtype), y0.cpu())
    # the merged SFD rows agree with the atomic path's up to summation order
    ya, _, _ = run_forward(wl, inp, dev, flags=0)
    assert row_err(ya.float().cpu().numpy(), y0.float().cpu().numpy().astype(np.float64)).max() \
        <= TOL[wl.dtype]


def test_deterministic_full_size_and_graph_replay():
    """OLMoE-shaped layer at T = 8192 with the Algorithm 1 placement: sampled
    rows against the oracle, then a captured HIP graph replayed three times
    with eager work in between, every replay bitwise equal to the eager run."""
    wl = W.OLMOE
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    ids0, _ = oracle.route(inp["logits"].numpy(), wl.k, inp["placement"])
    L = oracle.placement(oracle.coact(ids0, wl.Ne, inp["placement"])["C"], wl.Nd)
    y0, _, desc = run_forward(wl, inp, dev, L=L)
    rows = synth.sample_rows(wl.T, 48, seed=5)
    ids, w = oracle.route(inp["logits"].numpy(), wl.k, L)
    ref = oracle_rows(wl, inp, rows, ids, w)
    assert row_err(y0.float().cpu().numpy()[rows], ref).max() <= TOL[wl.dtype]

    ws = occ.alloc_workspace(desc)
    y = torch.empty_like(y0)
    stream = torch.cuda.Stream()
    args = (desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"], dev["w_down"], None,
            None, None, y, ws)
    with torch.cuda.stream(stream):
        occ.occ_moe_forward(*args)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        occ.occ_moe_forward(*args)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
        _ = (dev["x"].float() * 2).sum().item()  # unrelated eager work between replays


def test_deterministic_backward_matches_oracle_and_repeats_bitwise():
    wl = W.Workload("det_bwd", 32, T=900, d=256, Ne=16, k=4, Nd=4, F=256, n_shared=1,
                    F_shared=256, n_c=4, bonus=1.5)
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | DET)
    dt = torch.bfloat16
    f32 = dict(dtype=torch.float32, device="cuda")
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(4)) * 0.5).to(dt).cuda()

    def once():
        ws = occ.alloc_workspace(desc)
        y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
        occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                            dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
        out = dict(dx=torch.empty(wl.T, wl.d, dtype=dt, device="cuda"),
                   dWg=torch.empty(wl.Ne, wl.F, wl.d, **f32), dWu=torch.empty(wl.Ne, wl.F, wl.d, **f32),
                   dWd=torch.empty(wl.Ne, wl.d, wl.F, **f32),
                   dWsg=torch.empty(1, wl.F_shared, wl.d, **f32),
                   dWsu=torch.empty(1, wl.F_shared, wl.d, **f32),
                   dWsd=torch.empty(1, wl.d, wl.F_shared, **f32),
                   dw=torch.empty(wl.T, wl.k, **f32), dl=torch.empty(wl.T, wl.Ne, **f32))
        occ.occ_moe_backward(desc, dy, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                             dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"],
                             out["dx"], out["dWg"], out["dWu"], out["dWd"], out["dWsg"],
                             out["dWsu"], out["dWsd"], out["dw"], out["dl"], ws)
        torch.cuda.synchronize()
        v = occ.occ_forward_views(desc, ws)
        ids = occ.ws_view(ws, v.ids, (wl.T, wl.k), torch.int32).cpu().numpy()
        wts = occ.ws_view(ws, v.w, (wl.T, wl.k), torch.float32).cpu().numpy()
        return y, out, ids, wts

    y0, g0, ids, wts = once()
    y1, g1, _, _ = once()
    assert torch.equal(y0, y1)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key
    # the training forward against the oracle: ids bit for bit, weights, y
    ids_o, w_o = oracle.route(inp["logits"].numpy(), wl.k, L)
    assert np.array_equal(ids, ids_o)
    np.testing.assert_allclose(wts, w_o, rtol=W_RTOL, atol=0)
    ref_y = oracle_rows(wl, inp, np.arange(wl.T), ids_o, w_o)
    assert row_err(y0.float().cpu().numpy(), ref_y).max() <= TOL[wl.dtype]
    # the oracle's backward on the oracle's own routing
    ref = oracle.moe_backward(bits(inp["x"]), ids_o, w_o, dy.double().cpu().numpy(),
                              bits(inp["w_gate"]), bits(inp["w_up"]), bits(inp["w_down"]),
                              bits(inp["ws_gate"]), bits(inp["ws_up"]), bits(inp["ws_down"]),
                              logits=inp["logits"].numpy())
    assert row_err(g0["dx"].float().cpu().numpy(), ref["dx"]).max() <= 2e-2
    for key, rk in (("dWg", "dW_gate"), ("dWu", "dW_up"), ("dWd", "dW_down"),
                    ("dWsg", "dWs_gate"), ("dWsu", "dWs_up"), ("dWsd", "dWs_down"),
                    ("dw", "dw"), ("dl", "dlogits")):
        a, b = g0[key].cpu().numpy(), ref[rk]
        assert np.linalg.norm(a - b) / np.linalg.norm(b) <= 2e-2, key
