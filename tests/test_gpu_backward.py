"""GPU parity of the backward pass (occ_moe_backward after a training
forward) against the oracle's fp64 gradients: dx, the routed and shared
expert weight gradients, the routing-weight and logit gradients.  Shapes
cover both merge schedules (one launch after a zero-fill, first/rest),
dimensions that are not multiples of the 256-wide tiles, shared experts and
the OLMoE expert shape.

Tolerances: dy, x and the weights are exact bf16 values; the device rounds
the saved pre-activations g, u, the modulated state h and the SwiGLU
gradients dg, du to bf16 (2^-9 relative each) and accumulates in fp32, and
dx is rounded to bf16 once.  Each gradient therefore carries a few 2^-9 of
relative error: 2e-2, measured normwise (per row for dx and per expert
matrix for the weights, where single elements of a cancelling sum are
meaningless) and 5e-2 of the tensor's scale element-wise."""
import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import TOL, W_RTOL, bits, oracle_rows, routed_to_counts, row_err, to_dev

pytestmark = pytest.mark.gpu

NORM_TOL = 2e-2
ELEM_TOL = 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def shape(name, T, d, F, Ne=8, k=2, Nd=4, n_shared=0, F_shared=0, index=11):
    return W.Workload(name, index, T=T, d=d, Ne=Ne, k=k, Nd=Nd, F=F, n_shared=n_shared,
                      F_shared=F_shared, n_c=2, bonus=1.0)


def run(wl, placement=None, with_logits=True, inp=None, flags=occ.OCC_FLAG_TRAIN):
    inp = inp or synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"] if placement is None else placement
    desc = occ.desc_of(wl, flags=flags)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    ids, w = check_train_forward(wl, inp, L, desc, ws, y)
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(wl.index)) * 0.5).to(dt)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = dict(dx=torch.empty(wl.T, wl.d, dtype=dt, device="cuda"),
               dW_gate=torch.empty(wl.Ne, wl.F, wl.d, **f32),
               dW_up=torch.empty(wl.Ne, wl.F, wl.d, **f32),
               dW_down=torch.empty(wl.Ne, wl.d, wl.F, **f32),
               dw=torch.empty(wl.T, wl.k, **f32),
               dlogits=torch.empty(wl.T, wl.Ne, **f32) if with_logits else None)
    sh = dict(dWs_gate=None, dWs_up=None, dWs_down=None)
    if wl.n_shared:
        sh = dict(dWs_gate=torch.empty(wl.n_shared, wl.F_shared, wl.d, **f32),
                  dWs_up=torch.empty(wl.n_shared, wl.F_shared, wl.d, **f32),
                  dWs_down=torch.empty(wl.n_shared, wl.d, wl.F_shared, **f32))
    out.update(sh)
    occ.occ_moe_backward(desc, dy.cuda(), dev["x"], dev["logits"] if with_logits else None, L,
                         dev["w_gate"], dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"],
                         dev["ws_down"], out["dx"], out["dW_gate"], out["dW_up"], out["dW_down"],
                         out["dWs_gate"], out["dWs_up"], out["dWs_down"], out["dw"],
                         out["dlogits"], ws)
    torch.cuda.synchronize()
    got = {k2: (None if t is None else t.float().cpu().numpy()) for k2, t in out.items()}
    ref = oracle.moe_backward(bits(inp["x"]), ids, w, dy.double().numpy(), bits(inp["w_gate"]),
                              bits(inp["w_up"]), bits(inp["w_down"]), bits(inp["ws_gate"]),
                              bits(inp["ws_up"]), bits(inp["ws_down"]),
                              logits=inp["logits"].numpy() if with_logits else None)
    return got, ref


def check_train_forward(wl, inp, L, desc, ws, y, rows=None):
    """The training forward (OCC_FLAG_TRAIN: pre-activations kept, its own
    workspace layout) against the oracle: routing ids bit for bit, routing
    weights within W_RTOL, y within the layer tolerance of Eq. 1 on `rows`
    (all rows by default).  Returns the oracle's own routing, which seeds
    the oracle's backward."""
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(inp["logits"].numpy(), wl.k, L, wl.prune_rule, wl.prune_groups)
    v = occ.occ_forward_views(desc, ws)
    ids = occ.ws_view(ws, v.ids, (wl.T, wl.k), torch.int32).cpu().numpy()
    w = occ.ws_view(ws, v.w, (wl.T, wl.k), torch.float32).cpu().numpy()
    assert np.array_equal(ids, ids_o), "training forward: routing ids differ from the oracle"
    np.testing.assert_allclose(w, w_o, rtol=W_RTOL, atol=0)
    rows = np.arange(wl.T) if rows is None else rows
    ref = oracle_rows(wl, inp, rows, ids_o, w_o)
    err = row_err(y.float().cpu().numpy().astype(np.float64)[rows], ref)
    assert err.max() <= TOL[wl.dtype], f"training forward: max per-row rel err {err.max():.3e}"
    return ids_o, w_o


def normwise(a, b):
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def check(got, ref, keys):
    assert row_err(got["dx"], ref["dx"]).max() <= NORM_TOL
    for key in keys:
        g, r = got[key], ref[key]
        for e in range(r.shape[0]):       # per expert matrix
            assert normwise(g[e], r[e]) <= NORM_TOL, (key, e, normwise(g[e], r[e]))
            scale = np.abs(r[e]).max()
            assert np.abs(g[e] - r[e]).max() <= ELEM_TOL * scale, (key, e)
    for key in ("dw", "dlogits"):
        if got.get(key) is None:
            continue
        assert normwise(got[key], ref[key]) <= NORM_TOL, (key, normwise(got[key], ref[key]))
        assert np.abs(got[key] - ref[key]).max() <= ELEM_TOL * np.abs(ref[key]).max(), key


ROUTED = ["dW_gate", "dW_up", "dW_down"]
SHARED = ["dWs_gate", "dWs_up", "dWs_down"]


@pytest.mark.parametrize("wl", [
    shape("bwd_one_launch", T=300, d=256, F=256),              # T*k < 128*Ne: zero-fill merge
    shape("bwd_two_phase", T=1100, d=256, F=256, index=12),    # first / rest merge
    shape("bwd_ragged", T=700, d=384, F=320, k=3, Nd=2, index=13),  # overlapping tiles
], ids=lambda w: w.name)
def test_backward_matches_oracle(wl):
    got, ref = run(wl)
    check(got, ref, ROUTED)


@pytest.mark.parametrize("flags", [occ.OCC_FLAG_TRAIN,
                                   occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC],
                         ids=["atomic", "deterministic"])
def test_backward_row_tile_split_edges(flags):
    """Experts whose row counts straddle the input-gradient GEMMs' 320-row
    tiles (319-321, 639-641) and the weight-gradient GEMMs' 64-deep K slices
    and 256-row steps (255-257, 511-513), besides no rows, 1 and 15-17."""
    counts = [0, 1, 15, 16, 17, 255, 256, 257, 319, 320, 321, 511, 512, 513, 639, 640, 641, 3]
    wl = shape("bwd_split_edges", T=sum(counts) // 2, d=256, F=256, Ne=18, k=2, Nd=6, index=16)
    inp = synth.make_all(wl)
    inp["logits"] = routed_to_counts(counts, wl.k, seed=16)
    got, ref = run(wl, inp=inp, flags=flags)
    check(got, ref, ROUTED)


def test_backward_long_expert_segments():
    """Experts of 8191-8193 and 16385 rows: the weight-gradient GEMMs keep
    a gathered operand's row indices in LDS windows of 8192 rows, so these
    segments fill one window exactly, leave one row for a second window, or
    span three; deterministic merge."""
    counts = [8191, 8192, 8193, 16385, 12000, 3]
    wl = shape("bwd_long_segments", T=sum(counts) // 2, d=256, F=256, Ne=6, k=2, Nd=2, index=19)
    inp = synth.make_all(wl)
    inp["logits"] = routed_to_counts(counts, wl.k, seed=19)
    got, ref = run(wl, inp=inp, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    check(got, ref, ROUTED)


def test_backward_with_shared_experts():
    wl = shape("bwd_shared", T=500, d=256, F=256, n_shared=2, F_shared=320, index=14)
    got, ref = run(wl)
    check(got, ref, ROUTED + SHARED)


def test_backward_shared_experts_split_k():
    """Shared experts over 4096 tokens: their weight gradients (K = all T
    rows against a 256 x 320 or 640 x 256 output, a few tiles) are summed
    in 4 chunks of 1024 rows, added in chunk order.  Every gradient against
    the oracle, and bitwise equal across two runs."""
    wl = shape("bwd_shared_splitk", T=4096, d=256, F=256, n_shared=2, F_shared=320, index=18)
    inp = synth.make_all(wl)
    got, ref = run(wl, inp=inp, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    check(got, ref, ROUTED + SHARED)
    again, _ = run(wl, inp=inp, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    for key in SHARED + ["dx"]:
        assert np.array_equal(again[key], got[key]), key


def test_backward_olmoe_expert_shape():
    """d = 2048, F = 1024 (32 K slices in the input gradients, full-width
    weight tiles), fewer experts so that the fp64 oracle stays small."""
    wl = shape("bwd_olmoe_dims", T=256, d=2048, F=1024, Ne=8, k=2, Nd=4, index=15)
    got, ref = run(wl)
    check(got, ref, ROUTED)


def test_backward_rescheduled_placement_and_no_logits():
    wl = shape("bwd_placement", T=900, d=256, F=256, Ne=16, k=4, Nd=4, index=16)
    L = np.random.default_rng(3).permutation(16).astype(np.int32).reshape(4, 4)
    got, ref = run(wl, placement=L, with_logits=False)
    check(got, ref, ROUTED)


@pytest.mark.parametrize("flags", [occ.OCC_FLAG_TRAIN,
                                   occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC],
                         ids=["atomic", "deterministic"])
def test_backward_full_size_sampled(flags):
    """The OLMoE-shaped layer at the size bench.py runs (T = 8192), training
    forward + backward in the benchmark's launch configuration (either
    merge); sampled dx, dw and dlogits rows and sampled rows of two experts'
    weight gradients against the oracle computed one by one."""
    from gpu_common import inputs
    wl = W.OLMOE
    inp = inputs(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=flags)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], None, None, None, y, ws)
    rows = synth.sample_rows(wl.T, 32, seed=21)
    ids, w = check_train_forward(wl, inp, L, desc, ws, y, rows=synth.sample_rows(wl.T, 96, seed=22))
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(8)) * 0.5).to(dt)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    dWg = torch.empty(wl.Ne, wl.F, wl.d, **f32)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(wl.Ne, wl.d, wl.F, **f32)
    dw = torch.empty(wl.T, wl.k, **f32)
    dl = torch.empty(wl.T, wl.Ne, **f32)
    occ.occ_moe_backward(desc, dy.cuda(), dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                         dev["w_down"], None, None, None, dx, dWg, dWu, dWd, None, None, None, dw,
                         dl, ws)
    torch.cuda.synchronize()
    dyd = dy.double().numpy()
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                 bits(inp["w_up"]), bits(inp["w_down"]),
                                 logits=inp["logits"].numpy())
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL
    for key, got in (("dw", dw), ("dlogits", dl)):
        g = got.cpu().numpy()[rows]
        assert normwise(g, r[key]) <= NORM_TOL, key
        assert np.abs(g - r[key]).max() <= ELEM_TOL * np.abs(r[key]).max(), key
    fs, ns = np.array([0, 517, wl.F - 1]), np.array([0, 1000, wl.d - 1])
    for e in (5, 60):
        q = oracle.moe_wgrad_rows(bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                  bits(inp["w_up"]), bits(inp["w_down"]), e, fs, ns)
        for key, got, sel in (("dW_gate", dWg, fs), ("dW_up", dWu, fs), ("dW_down", dWd, ns)):
            g = got[e].cpu().numpy()[sel]
            for i in range(len(sel)):
                assert normwise(g[i], q[key][i]) <= NORM_TOL, (key, e, sel[i])
                assert np.abs(g[i] - q[key][i]).max() <= ELEM_TOL * np.abs(q[key][i]).max()


def test_backward_full_size_shared_experts_sampled():
    """The DeepSeek-shaped layer at full size (T = 16384, two shared experts
    of F = 1408), training forward + backward under the deterministic merge
    as the benchmark runs it; the shared experts' weight gradients, which
    sum over all T tokens in 8 and 4 ordered chunks, on sampled rows of both
    experts, and sampled dx rows.  A shared expert is an expert that every
    token selects with weight 1 (Eq. 1), so the oracle's per-expert gradient
    rows give its gradients."""
    from gpu_common import inputs
    wl = W.DEEPSEEK
    inp = inputs(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    ids, w = check_train_forward(wl, inp, L, desc, ws, y, rows=synth.sample_rows(wl.T, 48, seed=23))
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(9)) * 0.5).to(dt)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    dWg = torch.empty(wl.Ne, wl.F, wl.d, **f32)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(wl.Ne, wl.d, wl.F, **f32)
    nsh, Fs = wl.n_shared, wl.F_shared
    dWsg = torch.empty(nsh, Fs, wl.d, **f32)
    dWsu = torch.empty_like(dWsg)
    dWsd = torch.empty(nsh, wl.d, Fs, **f32)
    occ.occ_moe_backward(desc, dy.cuda(), dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                         dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], dx, dWg, dWu,
                         dWd, dWsg, dWsu, dWsd, None, None, ws)
    torch.cuda.synchronize()
    dyd = dy.double().numpy()
    rows = synth.sample_rows(wl.T, 24, seed=24)
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                 bits(inp["w_up"]), bits(inp["w_down"]), bits(inp["ws_gate"]),
                                 bits(inp["ws_up"]), bits(inp["ws_down"]))
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL
    all_tok = np.zeros((wl.T, 1), np.int32)
    ones = np.ones((wl.T, 1), np.float64)
    fs, ns = np.array([0, 700, Fs - 1]), np.array([0, 1001, wl.d - 1])
    for sx in range(nsh):
        q = oracle.moe_wgrad_rows(bits(inp["x"]), all_tok, ones, dyd, bits(inp["ws_gate"][sx:sx + 1]),
                                  bits(inp["ws_up"][sx:sx + 1]), bits(inp["ws_down"][sx:sx + 1]),
                                  0, fs, ns)
        for key, got, sel in (("dW_gate", dWsg, fs), ("dW_up", dWsu, fs), ("dW_down", dWsd, ns)):
            g = got[sx].cpu().numpy()[sel]
            for i in range(len(sel)):
                assert normwise(g[i], q[key][i]) <= NORM_TOL, (key, sx, sel[i])
                assert np.abs(g[i] - q[key][i]).max() <= ELEM_TOL * np.abs(q[key][i]).max()


def test_backward_shared_input_gradient_pipelined_build():
    """A batch long enough (T = 32768, d = 2048: 128 x 8 tiles of 256 x 256,
    four rounds of the CUs) that the shared experts' input gradient
    dg W_g + du W_u runs on the pipelined dense build, over the transposed
    shared weights; sampled dx rows against the oracle."""
    wl = shape("bwd_shared_pipe", T=32768, d=2048, F=256, n_shared=1, F_shared=512, index=19)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert (wl.T // 256) * (wl.d // 256) >= 4 * cus
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    ids, w = check_train_forward(wl, inp, L, desc, ws, y, rows=synth.sample_rows(wl.T, 32, seed=25))
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(10)) * 0.5).to(dt)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    dWg = torch.empty(wl.Ne, wl.F, wl.d, **f32)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(wl.Ne, wl.d, wl.F, **f32)
    dWsg = torch.empty(1, wl.F_shared, wl.d, **f32)
    dWsu = torch.empty_like(dWsg)
    dWsd = torch.empty(1, wl.d, wl.F_shared, **f32)
    occ.occ_moe_backward(desc, dy.cuda(), dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                         dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], dx, dWg, dWu,
                         dWd, dWsg, dWsu, dWsd, None, None, ws)
    torch.cuda.synchronize()
    rows = synth.sample_rows(wl.T, 24, seed=26)
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dy.double().numpy(),
                                 bits(inp["w_gate"]), bits(inp["w_up"]), bits(inp["w_down"]),
                                 bits(inp["ws_gate"]), bits(inp["ws_up"]), bits(inp["ws_down"]))
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL


def test_backward_full_size_qwen_sampled():
    """The Qwen-shaped layer at the size bench.py times its training step
    (T = 65536, 60 experts of F = 1408, top-4, one shared expert of
    F = 5632), deterministic merge: sampled dx, dw and dlogits rows, sampled
    rows of two routed experts' weight gradients, against the oracle
    computed one by one.  (The shared expert's weight gradients sum over all
    65536 tokens, each needing the expert's full 5632-feature backward in
    fp64: they are checked at T = 16384 and on the long dense shapes.)"""
    from gpu_common import inputs
    wl = W.QWEN
    inp = inputs(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    ids, w = check_train_forward(wl, inp, L, desc, ws, y, rows=synth.sample_rows(wl.T, 32, seed=27))
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(11)) * 0.5).to(dt)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    dWg = torch.empty(wl.Ne, wl.F, wl.d, **f32)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(wl.Ne, wl.d, wl.F, **f32)
    Fs = wl.F_shared
    dWsg = torch.empty(1, Fs, wl.d, **f32)
    dWsu = torch.empty_like(dWsg)
    dWsd = torch.empty(1, wl.d, Fs, **f32)
    dw = torch.empty(wl.T, wl.k, **f32)
    dl = torch.empty(wl.T, wl.Ne, **f32)
    occ.occ_moe_backward(desc, dy.cuda(), dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                         dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], dx, dWg, dWu,
                         dWd, dWsg, dWsu, dWsd, dw, dl, ws)
    torch.cuda.synchronize()
    del ws
    dyd = dy.double().numpy()
    rows = synth.sample_rows(wl.T, 24, seed=28)
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                 bits(inp["w_up"]), bits(inp["w_down"]), bits(inp["ws_gate"]),
                                 bits(inp["ws_up"]), bits(inp["ws_down"]),
                                 logits=inp["logits"].numpy())
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL
    for key, got in (("dw", dw), ("dlogits", dl)):
        g = got.cpu().numpy()[rows]
        assert normwise(g, r[key]) <= NORM_TOL, key
        assert np.abs(g - r[key]).max() <= ELEM_TOL * np.abs(r[key]).max(), key
    fs, ns = np.array([0, 703, wl.F - 1]), np.array([0, 1001, wl.d - 1])
    for e in (7, 52):
        q = oracle.moe_wgrad_rows(bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                  bits(inp["w_up"]), bits(inp["w_down"]), e, fs, ns)
        for key, got, sel in (("dW_gate", dWg, fs), ("dW_up", dWu, fs), ("dW_down", dWd, ns)):
            g = got[e].cpu().numpy()[sel]
            for i in range(len(sel)):
                assert normwise(g[i], q[key][i]) <= NORM_TOL, (key, e, sel[i])
                assert np.abs(g[i] - q[key][i]).max() <= ELEM_TOL * np.abs(q[key][i]).max()
