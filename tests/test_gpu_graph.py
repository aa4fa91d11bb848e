"""The layer captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches on the capturing stream) and replayed several times, with eager
calls and synchronisations in between, against the eager result: the
forward at the benchmark's size, the decode step with its gate projection,
and a training forward + backward.  No launch records a memset (zeroing is
a fill kernel), so every replay must reproduce the eager values up to the
order of the fp32 atomic adds."""
import numpy as np
import pytest
import torch

from expert_token_routing_amd import occ, synth, workloads as W

from gpu_common import inputs, row_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    occ.lib()


def check_replays(step, outputs, replays=3):
    step()
    torch.cuda.synchronize()
    eager = [o.float().cpu().numpy() for o in outputs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the stream once outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(replays):
        for o in outputs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            got = o.float().cpu().numpy().reshape(e.shape[0], -1)
            assert row_err(got, e.reshape(e.shape[0], -1)).max() <= 1e-2, i
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_forward_graph_replays():
    wl = W.OLMOE
    inp = inputs(wl)
    dev = to_dev(inp)
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    L = inp["placement"]
    check_replays(lambda: occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"],
                                              dev["w_up"], dev["w_down"], None, None, None, y,
                                              ws), [y])


def test_decode_graph_replays():
    wl = W.OLMOE_DECODE
    inp = inputs(wl)
    dev = to_dev(inp)
    desc = occ.desc_of(wl)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    L = inp["placement"]
    check_replays(lambda: occ.occ_moe_forward_gated(desc, dev["x"], dev["w_router"], L,
                                                    dev["w_gate"], dev["w_up"], dev["w_down"],
                                                    None, None, None, y, ws), [y])


def test_training_step_graph_replays():
    wl = W.Workload("graph_train", 18, T=1100, d=256, Ne=8, k=2, Nd=4, F=256, n_shared=1,
                    F_shared=256, n_c=2, bonus=1.0)
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN)
    ws = occ.alloc_workspace(desc)
    L = inp["placement"]
    f32 = dict(dtype=torch.float32, device="cuda")
    y = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    dy = torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    dx = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    gr = [torch.empty(wl.Ne, wl.F, wl.d, **f32), torch.empty(wl.Ne, wl.F, wl.d, **f32),
          torch.empty(wl.Ne, wl.d, wl.F, **f32), torch.empty(1, wl.F_shared, wl.d, **f32),
          torch.empty(1, wl.F_shared, wl.d, **f32), torch.empty(1, wl.d, wl.F_shared, **f32)]
    dw = torch.empty(wl.T, wl.k, **f32)
    dl = torch.empty(wl.T, wl.Ne, **f32)

    def step():
        occ.occ_moe_forward(desc, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                            dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)
        occ.occ_moe_backward(desc, dy, dev["x"], dev["logits"], L, dev["w_gate"], dev["w_up"],
                             dev["w_down"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], dx, *gr,
                             dw, dl, ws)
    check_replays(step, [y, dx, dw, dl] + gr)


@pytest.mark.parametrize("flags", [0, occ.OCC_FLAG_DETERMINISTIC], ids=["atomic", "deterministic"])
def test_shared_expert_graph_replays_follow_new_inputs(flags):
    """A layer with shared experts, which run on a side stream forked from
    the capturing stream, captured once and replayed on new token values
    written into the same input buffer, the workspace cleared before each
    replay: every replay must equal an eager run on the same values, so the
    side stream's launches are part of the graph (not run once at capture)."""
    wl = W.scaled(W.DEEPSEEK, 700, name="graph_shared_T700")
    inp = synth.make_all(wl)
    dev = to_dev(inp)
    L = inp["placement"]
    desc = occ.desc_of(wl, flags=flags)
    ws = occ.alloc_workspace(desc)
    y = torch.empty(wl.T, wl.d, dtype=torch.bfloat16, device="cuda")
    x = dev["x"].clone()

    def step():
        occ.occ_moe_forward(desc, x, dev["logits"], L, dev["w_gate"], dev["w_up"], dev["w_down"],
                            dev["ws_gate"], dev["ws_up"], dev["ws_down"], y, ws)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the stream once outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        x_new = torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(300 + i))
        x.copy_(x_new.to(torch.bfloat16).cuda())
        ws.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        y_graph = y.clone()
        ws.zero_()
        step()
        torch.cuda.synchronize()
        if flags & occ.OCC_FLAG_DETERMINISTIC:
            assert torch.equal(y_graph, y), i
        else:
            assert row_err(y_graph.float().cpu().numpy(), y.float().cpu().numpy()).max() <= 1e-2, i
