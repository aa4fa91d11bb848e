"""Benchmark of the Occult MoE layer on one MI355X.

One step = one occ_moe_forward call (route -> BRIM -> dispatch -> shared
experts -> SwiGLU grouped GEMM -> intra-group merge -> cross-group combine)
over one batch, inputs resident in HBM.  The headline workload is the
largest one that fits one GPU: the Qwen-MoE-shaped long-prefill layer
(T = 65536 tokens, d = 2048, 60 experts of F = 1408, top-4, 4 groups of 15,
one shared expert of width 5632, bf16).  The expert placement is the
rescheduled one (Algorithm 1 on the batch's co-activation counts, built with
the library's own calls, untimed); the contiguous placement is timed beside
it.  The step uses the deterministic merge of Algorithm 8 (every EPD row's
fp32 result stored, each SFD row summed in slot order, the combine in the
same pass); the atomic-add merge is timed beside it (`--atomic` swaps the
two).  `value` is the rate of the step replayed from a HIP graph (the
launches captured once); the eager rate, with HIP events between the
stages, is reported beside it.  A training step (forward keeping the
backward's state, then the backward pass) is timed too.

After the headline, the other workloads (tiny fp32, OLMoE-shaped, DeepSeek-
shaped, the pruned OLMoE shape under GROUPSUM and under TRAVERSE) are each
measured the same way and reported under `configs` (`--only` skips them).

Prints one JSON line.  `roofline` is for the dominant kernel (the SwiGLU
up-projection GEMM, launched once for the shared expert and once for the
routed experts, 3.02 TFLOP each at the headline shape): algorithmic FLOPs
per launch over its average duration, measured with HIP events recorded
around it on the layer's stream during the timed steps.  `stage_roofline`
puts every stage against its own bound with the method's algorithmic work
(each operand moved once, stage one's fp32 SFD rows written once);
`design_traffic` gives the HBM bytes the kernels really move, from the
committed counter profiles, over those algorithmic bytes.  `hbm_copy` is a
plain 1 GiB device-to-device copy (the runtime's) timed on this GPU, read +
write bytes per second, reported beside the 8 TB/s peak.  `cpu_baseline`
times the oracle on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU + % of bf16 MFMA / HBM roofline; CT"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3  # fp32 vector / MFMA
HEADLINE = "qwen_t65536"

# The pages' own figures (Occult paper: abstract, section 3.2 and Table 1,
# section 4.1): 4 NVIDIA RTX A6000 over PCIe, bf16 data with fp32
# atomic_add, Triton kernels, real OLMoE routing on 2^14 prompt tokens.
# Quoted as context beside the measurement; not a target.
CONTEXT = {
    "hardware": "4x NVIDIA RTX A6000 (48 GB) over PCIe, bf16 data, fp32 atomic_add, "
                "Triton kernels (paper section 4.1)",
    "speedup": ">1.5x over the compared MoE systems across tasks and models (abstract)",
    "ct_cut_from_rescheduling": "~20% (section 3.2); Table 1, OLMoE prefill of 2^14 tokens: "
                                "E(CT) 3.68 -> 3.02 (-17.9%), latency 15.93 s -> 12.53 s (-21.3%)",
    "note": "context, not a target: real routing on other hardware; the measured CT cut "
            "below is on seeded synthetic routing",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true",
                    help="measure the chosen workload only (no per-config records)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (headline)")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="the same for each of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contiguous", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--atomic", action="store_true",
                    help="time the atomic-add merge as the main step (default: the "
                         "deterministic merge)")
    ap.add_argument("--one-merge", action="store_true",
                    help="skip timing the other merge beside the main one")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training step (forward with saved state + backward)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    return ap.parse_args()


def merge_name(flags):
    from expert_token_routing_amd import occ
    return "deterministic" if flags & occ.OCC_FLAG_DETERMINISTIC else "atomic"


def name_stages(st, flags):
    """The forward's stage times under names that fit the merge in use: the
    deterministic merge's eighth stage is the merge together with the combine."""
    from expert_token_routing_amd import occ
    st = dict(st)
    if flags & occ.OCC_FLAG_DETERMINISTIC:
        st["gemm_down"] = st.pop("gemm_down_first")
        st["merge_and_combine"] = st.pop("gemm_down_rest")
        st.pop("combine")
    return st


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's "
              "expert groups stand in for devices on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    from expert_token_routing_amd import workloads as W

    wl = W.BY_NAME[args.workload]
    out = measure(args, wl, headline=True)
    if not args.only and wl.name == HEADLINE:
        cfgs = {}
        for w in (W.TINY_F32, W.OLMOE, W.DEEPSEEK, W.OLMOE_PRUNED, W.OLMOE_PRUNED_TRAVERSE):
            cfgs[w.name] = measure(args, w, headline=False)
        out["configs"] = cfgs
    out["hbm_copy"] = copy_bandwidth()
    out["context"] = dict(CONTEXT, measured_ct_cut={
        k: v["ct_cut"] for k, v in [(out["config"]["workload"], out)] + list(
            out.get("configs", {}).items()) if v.get("ct_cut") is not None})
    print(json.dumps(out), flush=True)


def measure(args, wl, headline):
    """Time one workload; the full JSON record for the headline, a shorter
    one (no other merge, no training step, a shorter oracle sample) for the
    other workloads."""
    import numpy as np
    import torch

    from expert_token_routing_amd import occ, profiling, synth, workloads as W

    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name}: generating inputs")
    inp = synth.make_all(wl)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    desc = occ.desc_of(wl)
    main_flags = 0 if args.atomic else occ.OCC_FLAG_DETERMINISTIC
    desc_main = occ.desc_of(wl, flags=main_flags)
    ws_main = occ.alloc_workspace(desc_main, dev)
    dt = synth.torch_dtype(wl)
    y = torch.empty(wl.T, wl.d, dtype=dt, device=dev)
    stream = torch.cuda.current_stream()

    sim = wl.prune_rule == W.PRUNE_SIMILARITY
    sim_rank, table_ms = None, None
    if sim:
        # --- expert similarity table (appendix A.3; offline, timed on its own)
        prof = synth.make_profile_logits(wl).to(dev)
        gram = torch.zeros(wl.Ne, wl.Ne, dtype=torch.float64, device=dev)
        sim_rank = torch.empty(wl.Ne, wl.Ne, dtype=torch.int32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        occ.occ_similarity_accumulate(prof, gram)
        occ.occ_similarity_rank(gram, sim_rank)
        e1.record(stream)
        torch.cuda.synchronize()
        table_ms = e0.elapsed_time(e1)
        log(f"[bench] similarity table from {prof.shape[0]} profiled tokens: {table_ms:.3f} ms")

    if wl.gated:
        # decode path: the logits come from the tokens (gate projection)
        g["logits"] = torch.empty(wl.T, wl.Ne, dtype=torch.float32, device=dev)
        occ.occ_gate(desc, g["x"], g["w_router"], g["logits"])

    # --- placement (offline step, untimed): Algorithm 1 on this batch's counts
    L_contig = inp["placement"]
    ids = torch.empty(wl.T, wl.k, dtype=torch.int32, device=dev)
    wts = torch.empty(wl.T, wl.k, dtype=torch.float32, device=dev)
    if sim:
        occ.occ_route_similarity(desc, g["logits"], L_contig, sim_rank, ids, wts)
    else:
        occ.occ_route(desc, g["logits"], L_contig, ids, wts)
    C = torch.empty(wl.Ne, wl.Ne, dtype=torch.int32, device=dev)
    P = torch.empty(wl.Ne, wl.Ne, dtype=torch.float32, device=dev)
    n_sfd = torch.empty(1, dtype=torch.int64, device=dev)
    ct = torch.empty(1, dtype=torch.float64, device=dev)
    intra = torch.empty(1, dtype=torch.float64, device=dev)
    occ.occ_coactivation_stats(desc, ids, L_contig, C, P, n_sfd, ct, intra)
    torch.cuda.synchronize()
    ct_contig, intra_contig = float(ct.item()), float(intra.item())
    L_alg1 = occ.occ_place_experts(C.cpu().numpy(), wl.Nd)
    # pruned routing depends on the placement: route again under Algorithm 1's
    if sim:
        occ.occ_route_similarity(desc, g["logits"], L_alg1, sim_rank, ids, wts)
    else:
        occ.occ_route(desc, g["logits"], L_alg1, ids, wts)
    occ.occ_coactivation_stats(desc, ids, L_alg1, C, P, n_sfd, ct, intra)
    torch.cuda.synchronize()
    ct_alg1, nsfd_alg1, intra_alg1 = float(ct.item()), int(n_sfd.item()), float(intra.item())
    active = int((torch.diagonal(C) > 0).sum().item())

    r_ids = torch.empty(wl.T, wl.k, dtype=torch.int32, device=dev)
    r_w = torch.empty(wl.T, wl.k, dtype=torch.float32, device=dev)

    def run(L, steps, events=None, route_events=None, mode=None):
        desc, ws = mode or (desc_main, ws_main)
        for i in range(steps):
            ev = events[i].handles if events is not None else None
            if wl.gated:
                occ.occ_moe_forward_gated(desc, g["x"], g["w_router"], L, g["w_gate"], g["w_up"],
                                          g["w_down"], g["ws_gate"], g["ws_up"], g["ws_down"], y,
                                          ws, stage_events=ev)
                continue
            if not sim:
                occ.occ_moe_forward(desc, g["x"], g["logits"], L, g["w_gate"], g["w_up"],
                                    g["w_down"], g["ws_gate"], g["ws_up"], g["ws_down"], y, ws,
                                    stage_events=ev)
                continue
            # similarity-pruned routing, then the layer on that routing
            if route_events is not None:
                route_events[i][0].record(stream)
            occ.occ_route_similarity(desc, g["logits"], L, sim_rank, r_ids, r_w)
            if route_events is not None:
                route_events[i][1].record(stream)
            occ.occ_moe_forward_routed(desc, g["x"], r_ids, r_w, L, g["w_gate"], g["w_up"],
                                       g["w_down"], g["ws_gate"], g["ws_up"], g["ws_down"], y,
                                       ws, stage_events=ev)

    def timed(L, label, mode=None):
        log(f"[bench] {wl.name} {label}: warmup {args.warmup}")
        run(L, args.warmup, mode=mode)
        torch.cuda.synchronize()
        events = [occ.StageEvents() for _ in range(args.steps)]
        rev = None
        if sim:
            rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        run(L, args.steps, events, rev, mode=mode)
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(stop) / args.steps
        stages = np.array([e.elapsed_ms() for e in events])  # steps x stages
        for e in events:
            e.close()
        st = {s: float(v) for s, v in zip(occ.STAGES, stages.mean(0))}
        if sim:
            # the routed forward's route stage is the copy of the given routing
            st["route_copy"] = st.pop("route")
            st = {"route_similarity": float(np.mean([a.elapsed_time(b) for a, b in rev])), **st}
        log(f"[bench] {wl.name} {label}: {ms:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})")
        return ms, st

    def graph_timed(L, label, mode=None):
        """One step captured in a HIP graph (no stage events), replayed."""
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run(L, 1, mode=mode)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            run(L, 1, mode=mode)
        for _ in range(args.warmup):
            gr.replay()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            gr.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        gms = start.elapsed_time(stop) / args.steps
        log(f"[bench] {wl.name} {label}: graph replay {gms:.4f} ms/step")
        del gr
        return gms

    ms_eager, stages = timed(L_alg1, "alg1 placement")
    ms_graph = None if args.no_graph else graph_timed(L_alg1, "alg1 placement")
    # the layer launched from a HIP graph is how a serving or training loop
    # runs it; the eager rate is reported beside it
    ms = ms_graph if ms_graph is not None else ms_eager
    tokens_per_s = wl.T / (ms / 1e3)
    res_other = None
    if headline and not args.one_merge:
        # the other merge strategy: same layer, same placement
        other_flags = occ.OCC_FLAG_DETERMINISTIC if args.atomic else 0
        desc_o = occ.desc_of(wl, flags=other_flags)
        mode_o = (desc_o, occ.alloc_workspace(desc_o, dev))
        label = merge_name(other_flags) + " merge"
        ms_o, stages_o = timed(L_alg1, label, mode=mode_o)
        ms_og = None if args.no_graph else graph_timed(L_alg1, label, mode=mode_o)
        res_other = {"merge": merge_name(other_flags), "value": wl.T / ((ms_og or ms_o) / 1e3),
                     "ms_per_step": ms_og or ms_o, "eager_ms_per_step": ms_o,
                     "stages_ms": name_stages(stages_o, other_flags)}
        del mode_o
    res_contig = None
    if not args.no_contiguous:
        ms_c, stages_c = timed(L_contig, "contiguous placement")
        res_contig = {"value": wl.T / (ms_c / 1e3), "ms_per_step": ms_c, "ct": ct_contig,
                      "intra": intra_contig, "stages_ms": name_stages(stages_c, main_flags)}

    if args.copy_calibration and headline:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    sroof, design = stage_rooflines(wl, stages, ms, main_flags, nsfd_alg1, active, profiling)
    roofline = dominant_roofline(wl, stages, nsfd_alg1, active, profiling)
    if res_other is not None:
        # the other merge's stages against the same algorithmic work (its
        # combine is the separate pass of Algorithm 9 under the atomic merge)
        res_other["stage_roofline"] = stage_rooflines(
            wl, stages_o, res_other["ms_per_step"], other_flags, nsfd_alg1, active, profiling)[0]

    # --- training step: forward keeping the backward's state, then backward
    train = None
    if (headline and not args.no_train and wl.dtype == W.DTYPE_BF16 and not sim
            and not wl.gated and wl.d >= 256 and wl.F >= 256
            and (wl.n_shared == 0 or wl.F_shared >= 256)):
        train = train_leg(args, wl, g, L_alg1, stream)

    # --- CPU baseline: the oracle on a bounded sample of this workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, L_alg1, args.cpu_seconds if headline else
                           args.config_cpu_seconds,
                           None if sim_rank is None else sim_rank.cpu().numpy())

    out = {}
    if headline:
        out = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s",
               "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "bf16" if wl.dtype == W.DTYPE_BF16 else "f32",
               "data": "synthetic"}
    else:
        out = {"value": round(tokens_per_s, 1), "unit": "tokens/s", "ms_per_step": round(ms, 5),
               "dtype": "bf16" if wl.dtype == W.DTYPE_BF16 else "f32"}
    out.update({
        "launch": "hip_graph" if ms_graph is not None else "eager",
        "eager_ms_per_step": round(ms_eager, 5),
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "Ne": wl.Ne, "k": wl.k,
                   "Nd": wl.Nd, "F": wl.F, "n_shared": wl.n_shared, "F_shared": wl.F_shared,
                   "placement": "alg1", "merge": merge_name(main_flags)},
        "ct": ct_alg1, "n_sfd": nsfd_alg1, "intra": intra_alg1,
        "ct_bounds": [-(-wl.k * wl.Nd // wl.Ne), min(wl.k, wl.Nd)],
        "ct_contiguous": ct_contig,
        "ct_cut": round(1.0 - ct_alg1 / ct_contig, 4) if ct_contig > 0 else None,
        "roofline": roofline, "cpu_baseline": cpu, "stage_roofline": sroof,
        "design_traffic": design,
        "stages_ms": {s: round(v, 5) for s, v in name_stages(stages, main_flags).items()},
        "contiguous": res_contig,
    })
    if wl.prune_rule in (W.PRUNE_TRAVERSE, W.PRUNE_GROUPSUM):
        out["config"]["pruning"] = (("traverse" if wl.prune_rule == W.PRUNE_TRAVERSE
                                     else "groupsum") + f", {wl.prune_groups} groups")
    if headline:
        out["other_merge"] = res_other
        if train is not None:
            out["train"] = train
    if sim:
        out["config"]["pruning"] = f"similarity, {wl.prune_groups} groups"
        out["similarity_table_ms"] = round(table_ms, 4)
    del ws_main, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def copy_bandwidth():
    """A plain 1 GiB device-to-device copy (the runtime's), timed: bytes read
    plus written per second, beside the 8 TB/s peak.  (The dispatch kernel's
    row copies run faster than this copy, so it is a measured reference, not
    a ceiling.)"""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    gbs = 2 * n / (ms / 1e3) / 1e9
    return {"bytes": 2 * n, "ms": round(ms, 4), "GB_per_s": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def algorithmic_work(wl, n_sfd, active):
    """The method's own work per stage, (flops, HBM bytes): every operand
    moved once, stage one's fp32 SFD rows written once (bf16 s = 2 bytes)."""
    from expert_token_routing_amd import workloads as W

    es = 2 if wl.dtype == W.DTYPE_BF16 else 4
    T, d, k, F, Ne = wl.T, wl.d, wl.k, wl.F, wl.Ne
    w = {
        "route": (0.0, T * (4 * Ne + 8 * k)),
        # gather: x read once, each SFD replica written once
        "dispatch": (0.0, (T + n_sfd) * d * es),
        # GEMM1: the SFD rows read once, the active experts' gate and up
        # weights, the EPD hidden states written
        "gemm_up": (2.0 * T * k * d * 2 * F, (n_sfd * d + active * 2 * F * d + T * k * F) * es),
        # GEMM2: the EPD rows, the down weights, one fp32 write of each SFD row
        "gemm_down": (2.0 * T * k * F * d, (T * k * F + active * d * F) * es + n_sfd * d * 4),
        # combine: the fp32 SFD rows read, y written (+ the shared output)
        "combine": (0.0, n_sfd * d * 4 + T * d * es + (T * d * 4 if wl.n_shared else 0)),
    }
    if wl.n_shared:
        fs = wl.n_shared * wl.F_shared
        w["shared_up"] = (2.0 * T * d * 2 * fs, (T * d + 2 * fs * d + T * fs) * es)
        w["shared_down"] = (2.0 * T * fs * d, (T * fs + fs * d) * es + T * d * 4)
    return w


def stage_rooflines(wl, stages, ms, flags, n_sfd, active, profiling):
    """Every stage against its own bound, t_roof = max(flops / peak, algorithmic
    bytes / HBM peak); the layer's fraction is the stages' t_roof summed over
    the step time (the BRIM is latency-bound and counts zero).  Also the
    kernels' measured HBM traffic over the algorithmic bytes, where a counter
    profile of this workload is committed and still matches the source."""
    from expert_token_routing_amd import occ, workloads as W

    es = 2 if wl.dtype == W.DTYPE_BF16 else 4
    peak_f = (PEAK_BF16_TFLOPS if es == 2 else PEAK_F32_TFLOPS) * 1e12
    work = algorithmic_work(wl, n_sfd, active)
    st = name_stages(stages, flags)
    det = bool(flags & occ.OCC_FLAG_DETERMINISTIC)
    measured = {
        "route": st.get("route", st.get("route_copy", 0.0)),
        "dispatch": st["dispatch"],
        "gemm_up": st["gemm_up"],
        # deterministic: one launch storing every row; atomic: first + rest
        "gemm_down": st["gemm_down"] if det else st["gemm_down_first"] + st["gemm_down_rest"],
        "combine": st["merge_and_combine"] if det else st["combine"],
    }
    if wl.n_shared:
        measured["shared_up"] = st["shared_up"]
        measured["shared_down"] = st["shared_down"]
    out = {}
    for name, (fl, by) in work.items():
        t_f, t_b = fl / peak_f, by / (PEAK_HBM_GBS * 1e9)
        t = max(t_f, t_b)
        m = max(measured[name], 1e-9)
        out[name] = {"ms": round(m, 5), "bound": "mfma" if t_f >= t_b else "hbm",
                     "roof_ms": round(t * 1e3, 5), "frac": round(t * 1e3 / m, 4),
                     "flops": fl, "bytes": by}
    if det:
        out["combine"]["note"] = ("the deterministic merge pass: sums the stored EPD rows into "
                                  "their SFD rows and does the combine")
    roof_sum = sum(v["roof_ms"] for v in out.values())
    out["layer"] = {"ms": round(ms, 5), "roof_ms": round(roof_sum, 5),
                    "frac": round(roof_sum / ms, 4),
                    "note": "sum of the stages' roofline times over the step time; the BRIM "
                            "is latency-bound and counted at zero"}
    # the design's real traffic over the algorithmic bytes (counter profiles)
    design = {}
    src = {"k_dispatch": "rows.hip", "k_merge_slots": "rows.hip"}
    alg = {"k_dispatch": work["dispatch"][1], "k_merge_slots": work["combine"][1]}
    # k_gemm_up and k_gemm_down launch once for the routed experts and once
    # for the shared ones, unless the shared product is large enough for the
    # pipelined k_gemm_*_dense: the counters are averaged per launch
    for gemm, cols in (("up", 2 * wl.n_shared * wl.F_shared), ("down", wl.d)):
        kern = f"k_gemm_{gemm}"
        launches = [work[f"gemm_{gemm}"][1]]
        if wl.n_shared:
            sh = work[f"shared_{gemm}"][1]
            if dense_pipelined(wl.T, cols):
                alg[f"{kern}_dense"], src[f"{kern}_dense"] = sh, "gemm_bf16.hip"
            else:
                launches.append(sh)
        alg[kern], src[kern] = sum(launches) / len(launches), "gemm_bf16.hip"
    for kern, a in alg.items():
        tb = profiling.traffic_bytes(kern, wl.name, src[kern])
        if tb is not None:
            design[kern] = {"traffic_bytes": tb, "algorithmic_bytes": a,
                            "ratio": round(tb / a, 3)}
    return out, design


def dense_pipelined(M, cols):
    """The library's size rule: a dense product (the shared experts) of at
    least 4 rounds of 256 x 256 tiles on the GPU's CUs runs on the pipelined
    four-wave build (kernels k_gemm_*_dense)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return -(-M // 256) * -(-cols // 256) >= 4 * cus


def dominant_roofline(wl, stages, n_sfd, active, profiling):
    """The up-projection GEMM kernel that takes the most time per step: its
    launches' algorithmic FLOPs over their average duration (HIP events on
    the layer's stream).  The routed up-projection is k_gemm_up (k_gemm_up_m128
    in the decode regime); the shared experts' runs on the same kernel
    (then the figures are per launch, averaged over the two) unless it is
    large enough for the pipelined k_gemm_up_dense."""
    from expert_token_routing_amd import workloads as W

    es = 2 if wl.dtype == W.DTYPE_BF16 else 4
    work = algorithmic_work(wl, n_sfd, active)
    small = wl.T * wl.k < 96 * wl.Ne and es == 2
    routed = "k_gemm_up_m128" if small else "k_gemm_up"
    if es != 2:
        routed = "k_gemm_up_f32"
    kernels = {routed: [("gemm_up", work["gemm_up"])]}
    if wl.n_shared:
        shared = routed
        if es == 2 and not small and dense_pipelined(wl.T, 2 * wl.n_shared * wl.F_shared):
            shared = "k_gemm_up_dense"
        kernels.setdefault(shared, []).append(("shared_up", work["shared_up"]))
    kernel, launches = max(kernels.items(), key=lambda kv: sum(stages[s] for s, _ in kv[1]))
    n = len(launches)
    avg_ms = sum(stages[s] for s, _ in launches) / n
    flops = sum(f for _, (f, _b) in launches) / n
    nbytes = sum(b for _, (_f, b) in launches) / n
    traffic = profiling.traffic_bytes(kernel, wl.name,
                                      "gemm_bf16.hip" if es == 2 else "gemm_f32.hip")
    # fp32 layers multiply on the vector ALUs, not the matrix cores
    peak = PEAK_BF16_TFLOPS if es == 2 else PEAK_F32_TFLOPS
    if flops / nbytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / (avg_ms / 1e3) / 1e12
        r = {"bound": "mfma" if es == 2 else "alu", "achieved": round(achieved, 2),
             "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / (avg_ms / 1e3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    r.update({"traffic": traffic, "kernel": kernel, "launches_per_step": n,
              "avg_ms": round(avg_ms, 5), "flops_per_launch": flops, "bytes_per_launch": nbytes})
    return r


def train_leg(args, wl, g, L, stream):
    """Time forward (OCC_FLAG_TRAIN) + backward steps on the same inputs; the
    backward GEMMs' achieved TFLOP/s from HIP events around each stage."""
    import numpy as np
    import torch

    from expert_token_routing_amd import occ

    dev = torch.device("cuda:0")
    desc = occ.desc_of(wl, flags=occ.OCC_FLAG_TRAIN |
                       (0 if args.atomic else occ.OCC_FLAG_DETERMINISTIC))
    ws = occ.alloc_workspace(desc, dev)
    dt = torch.bfloat16
    f32 = dict(dtype=torch.float32, device=dev)
    y = torch.empty(wl.T, wl.d, dtype=dt, device=dev)
    dy = (torch.randn(wl.T, wl.d, generator=torch.Generator().manual_seed(77)) * 0.5).to(dt).to(dev)
    dx = torch.empty(wl.T, wl.d, dtype=dt, device=dev)
    dWg = torch.empty(wl.Ne, wl.F, wl.d, **f32)
    dWu = torch.empty_like(dWg)
    dWd = torch.empty(wl.Ne, wl.d, wl.F, **f32)
    dws = [None, None, None]
    if wl.n_shared:
        dws = [torch.empty(wl.n_shared, wl.F_shared, wl.d, **f32),
               torch.empty(wl.n_shared, wl.F_shared, wl.d, **f32),
               torch.empty(wl.n_shared, wl.d, wl.F_shared, **f32)]
    dw = torch.empty(wl.T, wl.k, **f32)
    dl = torch.empty(wl.T, wl.Ne, **f32)

    def step(fev=None, bev=None):
        occ.occ_moe_forward(desc, g["x"], g["logits"], L, g["w_gate"], g["w_up"], g["w_down"],
                            g["ws_gate"], g["ws_up"], g["ws_down"], y, ws, stage_events=fev)
        occ.occ_moe_backward(desc, dy, g["x"], g["logits"], L, g["w_gate"], g["w_up"],
                             g["w_down"], g["ws_gate"], g["ws_up"], g["ws_down"], dx, dWg, dWu,
                             dWd, *dws, dw, dl, ws, stage_events=bev)

    log(f"[bench] {wl.name} training step: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fev = [occ.StageEvents() for _ in range(args.steps)]
    bev = [occ.StageEvents(occ.OCC_BSTAGE_COUNT) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(fev[i].handles, bev[i].handles)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    fst = np.array([e.elapsed_ms() for e in fev]).mean(0)
    bst = np.array([e.elapsed_ms() for e in bev]).mean(0)
    for e in fev + bev:
        e.close()
    bstages = {s: float(v) for s, v in zip(occ.BSTAGES, bst)}
    rows = wl.T * wl.k
    flops = {"dgrad_down": 2.0 * rows * wl.d * wl.F, "dgrad_up": 2.0 * rows * 2 * wl.F * wl.d,
             "wgrad_down": 2.0 * rows * wl.d * wl.F, "wgrad_up": 2.0 * rows * 2 * wl.F * wl.d}
    gemms = {k: {"ms": round(bstages[k], 5),
                 "tflops": round(f / (bstages[k] / 1e3) / 1e12, 1),
                 "frac": round(f / (bstages[k] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
             for k, f in flops.items()}
    if wl.n_shared:
        fs = wl.n_shared * wl.F_shared
        f_sh = 2.0 * wl.T * wl.d * 3 * fs * 2  # dgrad and wgrad of the three products
        gemms["shared"] = {"ms": round(bstages["shared"], 5),
                           "tflops": round(f_sh / (bstages["shared"] / 1e3) / 1e12, 1),
                           "frac": round(f_sh / (bstages["shared"] / 1e3) / 1e12
                                         / PEAK_BF16_TFLOPS, 4)}
    log(f"[bench] {wl.name} training step: {ms:.4f} ms (forward {fst.sum():.4f}, "
        f"backward {bst.sum():.4f})")
    out = {"ms_per_step": round(ms, 5), "tokens_per_s": round(wl.T / (ms / 1e3), 1),
           "forward_ms": round(float(fst.sum()), 5), "backward_ms": round(float(bst.sum()), 5),
           "backward_stages_ms": {k: round(v, 5) for k, v in bstages.items()},
           "backward_gemms": gemms}
    del ws, dWg, dWu, dWd, dws
    return out


def cpu_baseline(wl, inp, placement, seconds, sim_rank=None):
    """Time the oracle (route, BRIM, stats on the full batch; Eq. 1 rows on a
    sample sized to about `seconds`) and scale to tokens/s."""
    import numpy as np
    import torch

    import oracle
    from expert_token_routing_amd import synth

    log(f"[bench] {wl.name} cpu baseline: oracle route/BRIM/stats on the full batch")
    t0 = time.perf_counter()
    logits = inp["logits"].numpy()
    if wl.gated:
        xb = inp["x"].contiguous().view(torch.int16).numpy().view(np.uint16)
        wb = inp["w_router"].contiguous().view(torch.int16).numpy().view(np.uint16)
        logits = oracle.gate(np.arange(wl.T), xb, wb).astype(np.float32)
    if sim_rank is not None:
        ids, w = oracle.route_similarity(logits, wl.k, placement, wl.prune_groups, sim_rank)
    else:
        ids, w = oracle.route(logits, wl.k, placement, wl.prune_rule, wl.prune_groups)
    oracle.brim1(ids, w, wl.Ne, placement)
    oracle.coact(ids, wl.Ne, placement)
    t_index = time.perf_counter() - t0

    bits = lambda t: None if t is None else t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if inp["x"].dtype == torch.float32:
        bits = lambda t: None if t is None else t.contiguous().numpy()
    args = (bits(inp["x"]), ids, w, bits(inp["w_gate"]), bits(inp["w_up"]), bits(inp["w_down"]),
            bits(inp["ws_gate"]), bits(inp["ws_up"]), bits(inp["ws_down"]))
    threads = oracle.threads(0)
    probe = synth.sample_rows(wl.T, max(threads, 4), seed=5)
    t0 = time.perf_counter()
    oracle.moe_rows(probe, *args)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(min(wl.T, max(len(probe), seconds / max(per_row, 1e-9))))
    rows = synth.sample_rows(wl.T, n, seed=6)
    log(f"[bench] {wl.name} cpu baseline: Eq. 1 on {len(rows)} sampled rows with {threads} "
        "threads")
    t0 = time.perf_counter()
    oracle.moe_rows(rows, *args)
    t_rows = time.perf_counter() - t0
    per_token = t_rows / len(rows) + t_index / wl.T
    return {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"Eq. 1 output for {len(rows)} of {wl.T} tokens (seeded sample) in "
                       f"{t_rows:.1f} s plus route/BRIM/co-activation on all {wl.T} tokens in "
                       f"{t_index:.2f} s, fp64, {threads} threads")}


if __name__ == "__main__":
    main()
