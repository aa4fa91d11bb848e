"""GPU parity of the shared experts' large dense products.  A dense product
that fills at least 4 rounds of the CUs with 256 x 256 tiles (T x output
width >= 4 x 256 x 65,536 on 256 CUs) takes the four-wave, software-
pipelined GEMM build; these shapes reach that size while driving the
pipelined loop's edge cases: one, two, three and four 64-deep K slices, a
ragged last row tile (T not a multiple of 256), a partial last column tile,
three shared experts laid end to end along K, and the training forward
(pre-activations kept) with its backward.  Checked against the oracle on
sampled rows (the first and last rows, rows on both sides of row-tile
edges, random rows): the layer output y (Eq. 1), the shared experts' own
fp32 output (the oracle with every routing weight zero), and in training,
dx rows and rows of the shared weight gradients (a shared expert is an
expert every token selects with weight 1)."""
import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import TOL, bits, forward, oracle_rows, row_err, to_dev

pytestmark = pytest.mark.gpu

NORM_TOL = 2e-2   # the backward tests' gradient tolerance (see test_gpu_backward)
ELEM_TOL = 5e-2
T_RAGGED = 65_573  # 256 full row tiles and one of 37 rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def shape(name, index, d, F_shared, n_shared=1, T=T_RAGGED):
    return W.Workload(name, index, T=T, d=d, Ne=4, k=1, Nd=2, F=256, n_shared=n_shared,
                      F_shared=F_shared, n_c=2, bonus=1.0)


def pipelined(M, cols):
    """Whether the library's size rule sends a dense product to the
    pipelined build on this GPU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return -(-M // 256) * -(-cols // 256) >= 4 * cus


def sample(T, seed):
    edges = [0, 1, 255, 256, 257, 511, 512, T // 2, T - 38, T - 37, T - 36, T - 2, T - 1]
    return np.unique(np.concatenate([edges, synth.sample_rows(T, 64, seed=seed)]))


def check_shared_out(wl, inp, views, ws, rows):
    """y_shared (T x d fp32: the shared experts' sum) against the oracle's
    layer with every routing weight zero."""
    ysh = occ.ws_view(ws, views.y_shared, (wl.T, wl.d), torch.float32)
    got = ysh.cpu().numpy().astype(np.float64)[rows]
    ids = np.zeros((wl.T, wl.k), np.int32)
    ref = oracle_rows(wl, inp, rows, ids, np.zeros((wl.T, wl.k)))
    err = row_err(got, ref)
    assert err.max() <= TOL[wl.dtype], f"{wl.name}: shared output, max per-row rel err {err.max():.3e}"


CASES = [
    # up-projection pipelined: K = d = 64 (one slice), 2176 output columns (a
    # 64-feature last column tile); the down-projection (width 64) is not
    shape("dense_up_k64", 31, d=64, F_shared=1088),
    # down-projection pipelined: K = 128 (two slices), width 2112 (a 64-wide
    # last column tile)
    shape("dense_down_k128", 32, d=2112, F_shared=128),
    # down-projection over three shared experts' blocks of 64 (three slices)
    shape("dense_down_3x64", 33, d=2112, F_shared=64, n_shared=3),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_large_dense_products(wl):
    up_cols, down_cols = 2 * wl.n_shared * wl.F_shared, wl.d
    assert pipelined(wl.T, up_cols) or pipelined(wl.T, down_cols), "shape below the size rule"
    inp = synth.make_all(wl)
    rows = sample(wl.T, wl.index)
    ids_o, w_o = oracle.route(inp["logits"].numpy(), wl.k, inp["placement"], wl.prune_rule,
                              wl.prune_groups)
    ref = oracle_rows(wl, inp, rows, ids_o, w_o)
    for flags in (0, occ.OCC_FLAG_DETERMINISTIC):
        y, ws, v, _ = forward(wl, inp, flags=flags)
        err = row_err(y[rows], ref)
        assert err.max() <= TOL[wl.dtype], f"{wl.name} flags {flags}: max per-row rel err {err.max():.3e}"
        check_shared_out(wl, inp, v, ws, rows)
        del ws


def test_large_dense_training():
    """The training forward keeps the shared expert's gate and up
    pre-activations from the pipelined up-projection's epilogue (K = d = 256,
    four slices; 2048 output columns); the backward reads them back."""
    wl = shape("dense_train", 34, d=256, F_shared=1024)
    assert pipelined(wl.T, 2 * wl.F_shared)
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    torch.cuda.synchronize()
    ids, w = oracle.route(inp["logits"].numpy(), wl.k, L, wl.prune_rule, wl.prune_groups)
    rows = sample(wl.T, wl.index)
    err = row_err(y.float().cpu().numpy().astype(np.float64)[rows], oracle_rows(wl, inp, rows, ids, w))
    assert err.max() <= TOL[wl.dtype], f"training forward: max per-row rel err {err.max():.3e}"
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(wl.index)) * 0.5).to(dt)
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
    dyd = dy.double().numpy()
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                 bits(inp["w_up"]), bits(inp["w_down"]), bits(inp["ws_gate"]),
                                 bits(inp["ws_up"]), bits(inp["ws_down"]))
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL
    fs, ns = np.array([0, 517, wl.F_shared - 1]), np.array([0, 130, wl.d - 1])
    q = oracle.moe_wgrad_rows(bits(inp["x"]), np.zeros((wl.T, 1), np.int32), np.ones((wl.T, 1)),
                              dyd, bits(inp["ws_gate"]), bits(inp["ws_up"]), bits(inp["ws_down"]),
                              0, fs, ns)
    for key, got, sel in (("dW_gate", dWsg, fs), ("dW_up", dWsu, fs), ("dW_down", dWsd, ns)):
        g = got[0].cpu().numpy()[sel]
        for i in range(len(sel)):
            den = np.linalg.norm(q[key][i])
            assert np.linalg.norm(g[i] - q[key][i]) / (den if den > 0 else 1.0) <= NORM_TOL, (key, sel[i])
            assert np.abs(g[i] - q[key][i]).max() <= ELEM_TOL * np.abs(q[key][i]).max(), (key, sel[i])


def test_large_dense_training_two_shared_experts():
    """Two shared experts and a batch long enough that their input gradient
    dx_sh = sum of dg W_g + du W_u (one product over both experts' blocks of
    transposed weights, K = 2 x 2 x 256) runs on the pipelined build
    (257 x 4 tiles); sampled dx rows, including the ragged last row tile,
    and sampled rows of both experts' weight gradients."""
    wl = shape("dense_train_2sh", 35, d=1024, F_shared=256, n_shared=2)
    assert pipelined(wl.T, wl.d)
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN | occ.OCC_FLAG_DETERMINISTIC)
    ws = occ.alloc_workspace(desc)
    dt = torch.bfloat16
    y = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                        dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
    torch.cuda.synchronize()
    ids, w = oracle.route(inp["logits"].numpy(), wl.k, L, wl.prune_rule, wl.prune_groups)
    rows = sample(wl.T, wl.index)
    err = row_err(y.float().cpu().numpy().astype(np.float64)[rows], oracle_rows(wl, inp, rows, ids, w))
    assert err.max() <= TOL[wl.dtype], f"training forward: max per-row rel err {err.max():.3e}"
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(wl.index)) * 0.5).to(dt)
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
    r = oracle.moe_backward_rows(rows, bits(inp["x"]), ids, w, dyd, bits(inp["w_gate"]),
                                 bits(inp["w_up"]), bits(inp["w_down"]), bits(inp["ws_gate"]),
                                 bits(inp["ws_up"]), bits(inp["ws_down"]))
    assert row_err(dx.float().cpu().numpy()[rows], r["dx"]).max() <= NORM_TOL
    fs, ns = np.array([0, 100, Fs - 1]), np.array([0, 517, wl.d - 1])
    for sx in range(nsh):
        q = oracle.moe_wgrad_rows(bits(inp["x"]), np.zeros((wl.T, 1), np.int32),
                                  np.ones((wl.T, 1)), dyd, bits(inp["ws_gate"][sx:sx + 1]),
                                  bits(inp["ws_up"][sx:sx + 1]), bits(inp["ws_down"][sx:sx + 1]),
                                  0, fs, ns)
        for key, got, sel in (("dW_gate", dWsg, fs), ("dW_up", dWsu, fs), ("dW_down", dWsd, ns)):
            g = got[sx].cpu().numpy()[sel]
            for i in range(len(sel)):
                den = np.linalg.norm(q[key][i])
                assert np.linalg.norm(g[i] - q[key][i]) / (den if den > 0 else 1.0) <= NORM_TOL, \
                    (key, sx, sel[i])
