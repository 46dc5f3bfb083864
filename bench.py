"""Benchmark of the MoE-FFN decode hot path on one MI355X.

Default workload (one step = one token through the whole stack): a 60-layer stack of MoE layers,
each with 512 routed + 1 shared q4 expert (H=4096, I=1024, group 64, bf16 scale/bias) and an fp32
router (E=512, top-4), all resident in HBM (218.4 GB, generated on the device from the seeded
generator).  Tokens are decoded autoregressively at batch 1: every layer consumes RMSNorm of its
input and adds its MoE output to the residual, and token t+1 starts from RMSNorm of token t's
stack output.  One token is one launch of the persistent decode kernel (which runs all layers);
with --stack-mode kernels, one token's three-kernels-per-layer launches are captured into a HIP
graph and replayed.

Prints one JSON line (rank 0): tokens/s, achieved HBM GB/s over the algorithmic bytes
(2,629,632,000 B per token), the roofline of the dominant launch, and the fp64 CPU oracle timed on a
bounded sample of the same workload (at one thread and at all cores), together with a one-layer
parity check of the decode chain taken from the GPU's own layer state after the timed tokens.

Other workloads (one JSON line each, same keys):
    --workload layer --bits 4|2   one token through one MoE layer (512 + 1 experts), rotated over
                                  --layers resident copies so that nothing is served from the
                                  last-level cache
    --workload expert             one expert FFN call (gate/up/SwiGLU/down) rotated over the 512
                                  routed experts of a resident layer
    --workload prefill | oproj | gdn | copy

    python bench.py [--gpus 1] [--steps 256] [--warmup 16] [--layers 60] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "MoE-FFN decode tokens/s and achieved HBM GB/s (% of peak), 60-layer q4, 1 GPU"
SEED_W = 20260301  # weights of layer L use stream keys (SEED_W, L, slot, tensor)
SEED_X = 777       # token inputs use (SEED_X, token)
EPS = 1e-6


def layer_bytes(bits: int, H: int, I: int, E: int, k: int) -> int:
    """Algorithmic bytes one decode layer-token must move: k routed + 1 shared expert records,
    the router matrix and shared-gate vector, the input and the output vector."""
    import synth
    return ((k + 1) * synth.expert_bytes(bits, H, I) + E * H * 4 + H * 4 + 2 * H * 4)


def code_hash(src: bytes) -> str:
    """sha256 of a C++ source with comments and whitespace removed (comment edits keep it)."""
    import hashlib
    import re
    t = src.decode()
    t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
    t = re.sub(r"//[^\n]*", "", t)
    return hashlib.sha256("".join(t.split()).encode()).hexdigest()


def stack_traffic(n_layers: int):
    """HBM bytes per persist_kernel launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by the same counters on a plain 1 GiB copy), if the record in profiles/
    was taken on the current kernel source and the same layers per launch; otherwise None."""
    rec_path = os.path.join(ROOT, "profiles", "persist_kernel_stack60_traffic.json")
    try:
        rec = json.load(open(rec_path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if code_hash(src) != rec["source_code_sha256"]:
        return None
    if rec["layers_per_dispatch"] != min(n_layers, 64):
        return None
    return rec["traffic_bytes_per_dispatch"]


def build_stack(n_layers: int, bits: int, dev, dev_err=None):
    """n_layers resident layers of 512 routed + 1 shared expert (device-generated from the
    seeded generator; layer L uses weight key L), each with its fp32 router, shared-gate vector
    and column-blocked router copy.  dev_err (int32 device word) goes into every descriptor."""
    import torch
    import group_quantized_expert_amd as moe
    import synth
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    n_slots = E + 1
    slot_bytes = synth.expert_bytes(bits, H, I)
    keep = []
    descs = []
    for L in range(n_layers):
        buf = torch.empty(n_slots * slot_bytes, dtype=torch.uint8, device=dev)
        synth.gpu_fill_experts(buf.data_ptr(), slot_bytes, 0, n_slots, SEED_W, L, bits,
                               stream=torch.cuda.current_stream().cuda_stream)
        wr = torch.from_numpy(synth.router_weights(SEED_W, L, E, H)).to(dev)
        wsg = torch.from_numpy(synth.shared_gate_weights(SEED_W, L, H)).to(dev)
        wr_cb = torch.empty_like(wr)
        moe.moe_pack_router(wr, E, H, wr_cb, torch.cuda.current_stream().cuda_stream)
        keep += [buf, wr, wsg, wr_cb]
        descs.append(moe.layer(moe.experts(buf, bits, H, I, n_slots, slot_bytes, dev_err=dev_err),
                               wr, wsg, E, k, E, w_router_cb=wr_cb))
    torch.cuda.synchronize()
    return descs, keep


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle_layer(bits, experts, wr, wsg, budget_s, max_tokens, min_tokens=2):
    import oracle
    import synth
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    times = []
    t_start = time.perf_counter()
    tok = 0
    while (time.perf_counter() - t_start < budget_s and tok < max_tokens) or tok < min_tokens:
        x = synth.activations(SEED_X, tok)
        t0 = time.perf_counter()
        oracle.layer(x, wr, wsg, experts.__getitem__, bits, k, E, H, I, synth.GROUP,
                     norm_input=True, eps=EPS)
        times.append(time.perf_counter() - t0)
        tok += 1
    return float(np.median(times)), len(times)


def cpu_baseline(bits: int, n_layers_model: int, budget_s: float = 10.0,
                 budget_1t_s: float = 4.0) -> dict:
    """fp64 oracle on a bounded sample: decode tokens through layer 0 of the stack (all 513
    experts pre-generated in host memory, so only the oracle's arithmetic is timed) until the
    time budget is spent, at all cores and then at one thread; the median layer-token time is
    extrapolated to tokens/s of the n_layers_model-layer stack."""
    import oracle
    import synth
    H, E = synth.HIDDEN, synth.N_EXPERTS
    experts = [synth.expert(SEED_W, 0, s, bits) for s in range(E + 1)]
    wr = synth.router_weights(SEED_W, 0, E, H)
    wsg = synth.shared_gate_weights(SEED_W, 0, H)
    cores = len(os.sched_getaffinity(0))
    threads = min(int(os.environ.get("OMP_NUM_THREADS", cores)), cores)
    oracle.set_num_threads(threads)
    per_layer, n_all = _time_oracle_layer(bits, experts, wr, wsg, budget_s, 4096)
    oracle.set_num_threads(1)
    per_layer_1t, n_1t = _time_oracle_layer(bits, experts, wr, wsg, budget_1t_s, 256)
    oracle.set_num_threads(threads)
    n = n_layers_model
    what = f"extrapolated x{n} layers" if n > 1 else "one layer-token per token"
    return {
        "value": 1.0 / (per_layer * n),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n_all} tokens through layer 0 of the stack (fp64 oracle, all 513 "
                   f"experts resident in host memory), median {per_layer * 1e3:.2f} ms per "
                   f"layer-token at {threads} threads, {what}"),
        "value_1thread": 1.0 / (per_layer_1t * n),
        "sample_1thread": f"{n_1t} tokens, median {per_layer_1t * 1e3:.1f} ms per layer-token",
        "cpu_model": cpu_model(),
    }


def stack_parity_sample(descs, x_tok, layer_idx: int, bits: int, flags: int) -> dict:
    """One-step parity of the decode chain at (the token after the timed ones, layer_idx),
    starting from the GPU's own layer input: the GPU runs layers 0 .. layer_idx - 1 from the
    chain's current token input, then layer layer_idx alone (the same kernel and arithmetic as
    inside the one-launch stack); the fp64 oracle runs that layer on the GPU's layer input.
    Routed ids must match unless the oracle's 4th/5th logit gap is below 1e-3, where every GPU
    id's oracle logit must be within 1e-4 of the 4th; outputs within relative L2 1e-4 and
    max-abs 1e-3 * max|ref|."""
    import torch
    import group_quantized_expert_amd as moe
    import oracle
    import synth
    H, I, E, k, G = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K, synth.GROUP
    dev = x_tok.device
    x_in = x_tok.clone()
    x_l = torch.empty(H, dtype=torch.float32, device=dev)
    out = torch.empty(H, dtype=torch.float32, device=dev)
    trace = torch.empty(1, k, dtype=torch.int32, device=dev)
    wsb = moe.moe_stack_workspace_bytes(descs[:1])
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    if layer_idx > 0:
        moe.moe_decode_stack(descs[:layer_idx], x_in, x_l, None, EPS, None, ws, wsb, flags=flags)
    else:
        x_l.copy_(x_in)
    moe.moe_decode_stack(descs[layer_idx:layer_idx + 1], x_l, out, None, EPS, trace, ws, wsb,
                         flags=flags)
    torch.cuda.synchronize()
    xl = x_l.cpu().numpy().astype(np.float64)
    got = out.cpu().numpy().astype(np.float64)
    gids = sorted(int(v) for v in trace.cpu().numpy()[0])
    wr = synth.router_weights(SEED_W, layer_idx, E, H)
    wsg = synth.shared_gate_weights(SEED_W, layer_idx, H)
    ref = oracle.layer(xl, wr, wsg, lambda s: synth.expert(SEED_W, layer_idx, s, bits), bits, k,
                       E, H, I, G, norm_input=True, eps=EPS)
    lg = np.sort(ref["logits"])[::-1]
    gap = float(lg[k - 1] - lg[k])
    ids_match = gids == sorted(int(v) for v in ref["ids"])
    near_tie = gap < 1e-3
    ids_ok = ids_match or (near_tie and all(ref["logits"][e] >= lg[k - 1] - 1e-4 for e in gids))
    rel = float(np.linalg.norm(got - ref["out"]) / np.linalg.norm(ref["out"]))
    mx = float(np.max(np.abs(got - ref["out"])) / np.max(np.abs(ref["out"])))
    ok = ids_ok and (not ids_match or (rel <= 1e-4 and mx <= 1e-3))
    return {"layer": layer_idx, "ids_match": ids_match, "oracle_gap": gap, "near_tie": near_tie,
            "rel_l2": rel, "max_abs_over_max_ref": mx, "ok": bool(ok)}


def _events_time(step, steps: int, warmup: int, stream=None) -> float:
    """ms per step over `steps` calls after `warmup`, from HIP events recorded on the stream
    the kernels are launched on."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s = stream or torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def layer_bench(args) -> dict:
    """One token through one MoE layer (512 routed + 1 shared expert, q4 or q2, H 4096, I 1024):
    step i runs layer copy i mod --layers on token input i mod 64 (distinct routings), so that
    neither the experts nor the router and shared expert are served from the 256 MB last-level
    cache (20 q4 copies hold 308 MB of router + shared-expert bytes alone).  By default the
    three-kernel layer decode runs, a graph replay covering all copies once; --exec persistent
    runs the persistent kernel with one layer per launch (its cooperative launch costs ~17 us
    per call that back-to-back one-layer calls cannot hide)."""
    import torch
    import group_quantized_expert_amd as moe
    import synth
    dev = torch.device("cuda:0")
    bits = args.bits
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    n = args.layers
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    descs, keep = build_stack(n, bits, dev, dev_err=err)
    nx = 64
    X = torch.from_numpy(np.stack([synth.activations(SEED_X, t) for t in range(nx)])).to(dev)
    out = torch.empty(nx, H, dtype=torch.float32, device=dev)
    persistent = args.exec == "persistent"
    stream = torch.cuda.current_stream()
    if persistent:
        flags = moe.STACK_PERSISTENT | (moe.STACK_PLAIN_LAUNCH if args.plain_launch else 0)
        arrs = [(moe.MoeLayer * 1)(d) for d in descs]
        wsb = moe.moe_stack_workspace_bytes(descs[:1])
        ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
        ctr = [0]

        def step():
            i = ctr[0]
            ctr[0] += 1
            moe.moe_decode_stack(arrs[i % n], X[i % nx], out[i % nx], None, EPS, None, ws, wsb,
                                 stream, flags=flags)

        ms = _events_time(step, args.steps, args.warmup, stream)
        kernel = "persist_kernel (one layer per launch)"
        dtype = "f32 (q4 codes as exact integer dot products)"
    else:
        wsb = moe.moe_layer_workspace_bytes(descs[0])
        ws = [torch.zeros(wsb, dtype=torch.uint8, device=dev) for _ in range(n)]

        def all_layers():
            for i in range(n):
                moe.moe_layer_decode(descs[i], X[i % nx], 0, EPS, out[i % nx], None, None, None,
                                     ws[i], wsb)

        ms = graph_time(all_layers, max(1, args.steps // n), max(1, args.warmup // n)) / n
        kernel = "k1 + k2 + k3 per layer (graph replay)"
        dtype = "f32"
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item())} after the timed layers")
    assert torch.isfinite(out).all().item(), "non-finite layer output"
    lb = layer_bytes(bits, H, I, E, k)
    gbs = lb / ms / 1e6
    res = {"metric": f"MoE-FFN decode tokens/s and achieved HBM GB/s, one q{bits} layer, 1 GPU",
           "value": round(1e3 / ms, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
           "config": {"workload": f"one q{bits} MoE layer decode, batch 1 (512 + 1 experts, "
                                  f"{n} resident copies rotated)",
                      "bits": bits, "layers_rotated": n, "hidden": H, "intermediate": I,
                      "experts": E, "top_k": k, "shared_experts": 1, "group": synth.GROUP},
           "us_per_layer_token": round(ms * 1e3, 3),
           "hbm_gb_s": round(gbs, 1), "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": None, "bytes_per_launch": lb,
                        "avg_launch_us": round(ms * 1e3, 3)}}
    if not args.no_cpu_baseline:
        del keep, ws
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(bits, 1)
    return res


def expert_bench(args) -> dict:
    """One expert FFN for one token (gate/up dequant GEMVs, SwiGLU, down GEMV; q4, H 4096,
    I 1024) through moe_expert_ffn_q4: a graph replay calls it for each of the 512 routed
    experts of a resident layer (3.6 GB, far above the last-level cache), one expert per call."""
    import torch
    import group_quantized_expert_amd as moe
    import oracle
    import synth
    dev = torch.device("cuda:0")
    H, I, E = synth.HIDDEN, synth.INTER, synth.N_EXPERTS
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    descs, keep = build_stack(1, 4, dev, dev_err=err)
    ex = descs[0].experts
    ids = torch.arange(E, dtype=torch.int32, device=dev)
    x = torch.from_numpy(synth.activations(SEED_X, 0)).to(dev)
    y = torch.empty(E, H, dtype=torch.float32, device=dev)
    h = torch.empty(E, I, dtype=torch.float32, device=dev)

    def all_experts():
        for e in range(E):
            moe.moe_expert_ffn_q4(ex, x, ids[e:e + 1], 1, y[e], h[e])

    ms_all = graph_time(all_experts, max(1, args.steps // 32), max(1, args.warmup // 32))
    ms = ms_all / E
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item())}")
    unit = synth.expert_bytes(4) + 2 * H * 4
    gbs = unit / ms / 1e6
    res = {"metric": "single expert SwiGLU FFN calls/s and achieved HBM GB/s, q4, 1 GPU",
           "value": round(1e3 / ms, 1), "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "single q4 expert SwiGLU FFN, one token, rotated over the 512 "
                                  "experts of a resident layer", "hidden": H, "intermediate": I,
                      "group": synth.GROUP, "bits": 4},
           "us_per_call": round(ms * 1e3, 3), "hbm_gb_s": round(gbs, 1),
           "roofline": {"bound": "hbm", "kernel": "k2 (gate/up + SwiGLU) + k3 (down), graph",
                        "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "bytes_per_launch": unit, "avg_launch_us": round(ms * 1e3, 3)}}
    if not args.no_cpu_baseline:
        rec = synth.expert(SEED_W, 0, 0, 4)
        xh = synth.activations(SEED_X, 0)
        cores = len(os.sched_getaffinity(0))
        threads = min(int(os.environ.get("OMP_NUM_THREADS", cores)), cores)
        timed = {}
        for nt, budget in ((threads, 8.0), (1, 4.0)):
            oracle.set_num_threads(nt)
            ts, t0 = [], time.perf_counter()
            while time.perf_counter() - t0 < budget or len(ts) < 2:
                a = time.perf_counter()
                oracle.expert_ffn(4, H, I, synth.GROUP, rec, xh)
                ts.append(time.perf_counter() - a)
            timed[nt] = (float(np.median(ts)), len(ts))
        oracle.set_num_threads(threads)
        res["cpu_baseline"] = {
            "value": 1.0 / timed[threads][0], "unit": "calls/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{timed[threads][1]} calls of one expert (fp64 oracle), median "
                      f"{timed[threads][0] * 1e3:.2f} ms at {threads} threads",
            "value_1thread": 1.0 / timed[1][0],
            "sample_1thread": f"{timed[1][1]} calls, median {timed[1][0] * 1e3:.1f} ms",
            "cpu_model": cpu_model()}
    return res


def batch_bench(args) -> dict:
    """Small-batch decode: B tokens per step through the --layers-layer q4 stack (three kernels per
    layer for all B tokens at once, graph-replayed), every token fed back through RMSNorm of its
    stack output as in the single-token decode."""
    import torch
    import group_quantized_expert_amd as moe
    import synth
    dev = torch.device("cuda:0")
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    B = args.tokens
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    descs, keep = build_stack(args.layers, 4, dev, dev_err=err)
    arr = (moe.MoeLayer * len(descs))(*descs)
    wsb = moe.moe_stack_batch_workspace_bytes(descs, B)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    x = torch.from_numpy(np.stack([synth.activations(SEED_X, t) for t in range(B)])).to(dev)
    x_out = torch.empty(B, H, dtype=torch.float32, device=dev)

    def step():
        moe.moe_decode_stack_batch(arr, x, B, x_out, x, EPS, None, ws, wsb)

    ms = graph_time(step, args.steps, args.warmup)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item())}")
    assert torch.isfinite(x_out).all().item(), "non-finite stack output"
    distinct = E * (1 - (1 - k / E) ** B) + 1  # expected distinct experts a layer-step reads
    step_bytes = args.layers * (distinct * synth.expert_bytes(4) + E * H * 4 + H * 4 + 2 * B * H * 4)
    gbs = step_bytes / ms / 1e6
    return {"metric": "MoE-FFN small-batch decode tokens/s, 60-layer q4, 1 GPU",
            "value": round(B * 1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": f"{args.layers}-layer q4 MoE-FFN stack decode, {B} tokens per "
                                   f"step", "layers": args.layers, "tokens_per_step": B,
                       "hidden": H, "intermediate": I, "experts": E, "top_k": k},
            "us_per_layer_step": round(ms * 1e3 / args.layers, 3),
            "expected_bytes_per_step": round(step_bytes),
            "hbm_gb_s_expected_bytes": round(gbs, 1)}


def prefill_bench(args) -> dict:
    """One q4 layer (512 + 1 experts) over a chunk of T tokens: time moe_prefill_q4."""
    import torch
    import group_quantized_expert_amd as moe
    import synth
    dev = torch.device("cuda:0")
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    T = args.tokens
    descs, keep = build_stack(1, 4, dev)
    L = descs[0]
    X = np.stack([synth.activations(SEED_X, t) for t in range(T)])
    d_x = torch.from_numpy(X).to(dev)
    out = torch.empty(T, H, dtype=torch.float32, device=dev)
    wsb = moe.moe_prefill_workspace_bytes(L, T)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        moe.moe_prefill_q4(L, d_x, T, out, None, None, None, ws, wsb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        moe.moe_prefill_q4(L, d_x, T, out, None, None, None, ws, wsb)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    wbytes = (E + 1) * synth.expert_bytes(4) + E * H * 4 + H * 4 + 2 * T * H * 4
    flops = 2 * T * E * H + 2 * T * H + (T * k + T) * 3 * 2 * H * I
    return {"metric": "MoE-FFN prefill tokens/s, one q4 layer, 1 GPU", "value": round(T / ms * 1e3, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16x2-mfma/f32", "data": "synthetic",
            "config": {"workload": f"prefill chunk of {T} tokens through one q4 MoE layer",
                       "tokens": T, "hidden": H, "intermediate": I, "experts": E, "top_k": k},
            "hbm_gb_s": round(wbytes / ms / 1e6, 1),
            "useful_tflops": round(flops / ms / 1e9, 2)}


def graph_time(fn, steps: int, warmup: int) -> float:
    """ms per replay of a HIP graph holding the launches `fn` makes (captured once, so host
    launch cost is not timed), over `steps` replays after `warmup` untimed ones."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for _ in range(warmup):
        graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def gdn_bench(args) -> dict:
    """The GatedDeltaNet state update of the linear-attention layers for one token: 45 layers of
    64 heads x 128 x 128 fp32 state, each layer its own state.  Four tokens' worth of distinct
    states (4 x 45 x 4 MiB = 755 MB, above the last-level cache) are updated in one replay, so
    every update reads its state from HBM as it would between the expert reads of a real step."""
    import torch
    import group_quantized_expert_amd as moe
    dev = torch.device("cuda:0")
    nh, dk, dv, n, rot = 64, 128, 128, 45, 4
    g = torch.Generator(device=dev)
    g.manual_seed(SEED_W)
    S = [0.1 * torch.randn(nh, dv, dk, generator=g, device=dev) for _ in range(n * rot)]
    q = torch.nn.functional.normalize(torch.randn(n, nh, dk, generator=g, device=dev), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(n, nh, dk, generator=g, device=dev), dim=-1)
    v = torch.randn(n, nh, dv, generator=g, device=dev)
    alpha = torch.rand(n, nh, generator=g, device=dev) * 0.5 + 0.5
    beta = torch.rand(n, nh, generator=g, device=dev)
    out = torch.empty(n, nh, dv, device=dev)

    def tokens():
        for j in range(n * rot):
            l = j % n
            moe.moe_gdn_step(S[j], q[l], k[l], v[l], alpha[l], beta[l], nh, dk, dv, out[l])

    ms = graph_time(tokens, args.steps, args.warmup) / rot
    launch_ms = ms / n
    step_bytes = 2 * nh * dv * dk * 4 + (2 * nh * dk + 2 * nh * dv + 2 * nh) * 4
    gbs = step_bytes / launch_ms / 1e6
    return {"metric": "GatedDeltaNet state update decode tokens/s, 1 GPU",
            "value": round(1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "GatedDeltaNet state update, 45 layers x 64 heads x 128x128, "
                                   "batch 1", "layers": n, "heads": nh, "dk": dk, "dv": dv},
            "roofline": {"bound": "hbm", "kernel": "gdn_step_kernel", "achieved": round(gbs, 1),
                         "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                         "traffic": None, "us_per_launch": round(launch_ms * 1e3, 3),
                         "bytes_per_launch": step_bytes}}


def oproj_bench(args) -> dict:
    """The dense q4 attention output projection (8192 -> 4096, group 64) and the standalone
    RMSNorm that follow each other before the router, for one token through `--layers` layers,
    each with its own weights (1.13 GB for 60 layers, far above the last-level cache).  The
    projection's own launches are also timed alone, back to back, for its roofline."""
    import torch
    import group_quantized_expert_amd as moe
    dev = torch.device("cuda:0")
    R, C, n = 4096, 8192, args.layers
    rec_bytes = R * C // 2 + 2 * 2 * R * (C // 64)
    g = torch.Generator(device=dev)
    g.manual_seed(SEED_W)
    recs = []
    for _ in range(n):  # codes uniform 0..15 in both nibbles; scale ~ U(0.01, 0.03); bias -8 scale
        codes = torch.randint(0, 256, (R * C // 2,), generator=g, device=dev, dtype=torch.uint8)
        scale = (torch.rand(R * (C // 64), generator=g, device=dev, dtype=torch.float64) * 0.02
                 + 0.01).to(torch.bfloat16)
        recs.append(torch.cat([codes, scale.view(torch.uint8), (-8 * scale).view(torch.uint8)]))
    assert all(r.numel() == rec_bytes for r in recs)
    mats = [moe.qmatrix(r, 4, R, C) for r in recs]
    a = torch.randn(n, C, generator=g, device=dev, dtype=torch.float32)
    y = torch.empty(n, R, dtype=torch.float32, device=dev)
    xn = torch.empty_like(y)

    def step():
        for l in range(n):
            moe.moe_qgemv(mats[l], a[l], y[l])
            moe.moe_rmsnorm(y[l], 1, R, 1e-6, xn[l])

    def proj_only():
        for l in range(n):
            moe.moe_qgemv(mats[l], a[l], y[l])

    ms = graph_time(step, args.steps, args.warmup)
    proj_ms = graph_time(proj_only, args.steps, args.warmup) / n
    wbytes = rec_bytes + C * 4 + R * 4          # per projection: record, input, output
    norm_bytes = 2 * R * 4                      # per norm: read and write 4096 floats
    gbs = wbytes / proj_ms / 1e6
    return {"metric": "o_proj q4 GEMV + RMSNorm decode tokens/s, 1 GPU",
            "value": round(1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"o_proj [4096 x 8192] q4 GEMV + RMSNorm, {n} layers, batch 1",
                       "layers": n, "rows": R, "cols": C, "group": 64},
            "us_per_layer": round(ms * 1e3 / n, 3),
            "hbm_gb_s": round(n * (wbytes + norm_bytes) / ms / 1e6, 1),
            "roofline": {"bound": "hbm", "kernel": "qgemv_kernel<4, 8192>",
                         "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbs / 8000.0, 4), "traffic": None,
                         "us_per_launch": round(proj_ms * 1e3, 3), "bytes_per_launch": wbytes}}


def copy_bench(args) -> dict:
    """A plain device-to-device copy of 1 GiB (reads 1 GiB, writes 1 GiB) per step: the
    reference for turning the FETCH_SIZE / WRITE_SIZE counters into HBM bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(args.warmup, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"workload": "copy", "bytes_read": n, "bytes_written": n, "ms_per_copy": round(ms, 4),
            "gb_s_read_plus_write": round(2 * n / ms / 1e6, 1)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=None,
                    help="stack depth (default 60), or layer copies rotated by --workload layer "
                         "(default 20)")
    ap.add_argument("--workload", choices=["stack", "layer", "expert", "batch", "prefill", "copy",
                                           "oproj", "gdn"], default="stack",
                    help="copy: a plain 1 GiB device copy, the reference the HBM counters "
                         "(FETCH_SIZE, WRITE_SIZE) are scaled by")
    ap.add_argument("--bits", type=int, choices=[2, 4], default=4,
                    help="code width of the stack and layer workloads (the headline is q4)")
    ap.add_argument("--exec", choices=["kernels", "persistent"], default="kernels",
                    help="layer workload: three kernels per layer (default: the faster way to run "
                         "one layer per call) or the persistent kernel with one layer per launch")
    ap.add_argument("--tokens", type=int, default=None,
                    help="prefill chunk size (default 2048) or tokens per batch step (default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stack-mode", choices=["auto", "kernels", "persistent"], default="auto",
                    help="decode stack execution: persistent one-launch-per-token kernel (auto "
                         "where supported) or three kernels per layer")
    ap.add_argument("--plain-launch", action="store_true",
                    help="issue the persistent kernel with an ordinary launch (for profilers "
                         "that cannot follow cooperative launches)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode stack (218 GB) fits one MI355X and the "
              "data-parallel path needs no exchange; run with --gpus 1.", file=sys.stderr)
        return 2
    if args.layers is None:
        args.layers = 20 if args.workload == "layer" else 60
    if args.tokens is None:
        args.tokens = 4 if args.workload == "batch" else 2048
    other = {"prefill": prefill_bench, "copy": copy_bench, "oproj": oproj_bench,
             "gdn": gdn_bench, "layer": layer_bench, "expert": expert_bench, "batch": batch_bench}
    if args.workload in other:
        print(json.dumps(other[args.workload](args)), flush=True)
        return 0

    import torch
    import group_quantized_expert_amd as moe
    import synth

    dev = torch.device("cuda:0")
    bits = args.bits
    H, I, E, k = synth.HIDDEN, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    t_setup = time.perf_counter()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    descs, keep = build_stack(args.layers, bits, dev, dev_err=err)
    print(f"# stack of {args.layers} layers resident ({args.layers * (E + 1) * synth.expert_bytes(bits) / 1e9:.1f} GB experts) "
          f"in {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    arr = (moe.MoeLayer * len(descs))(*descs)
    ws_bytes = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    x_tok = torch.from_numpy(synth.activations(SEED_X, 0)).to(dev)  # token input, overwritten
    x_out = torch.empty(H, dtype=torch.float32, device=dev)

    mode = {"auto": moe.STACK_AUTO, "kernels": moe.STACK_KERNELS,
            "persistent": moe.STACK_PERSISTENT}[args.stack_mode]
    flags = mode | (moe.STACK_PLAIN_LAUNCH if args.plain_launch else 0)
    stream = torch.cuda.current_stream()
    if mode == moe.STACK_KERNELS:
        # three kernels per layer: capture one token (all layers) into a graph and replay it
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            moe.moe_decode_stack(arr, x_tok, x_out, x_tok, EPS, None, ws, ws_bytes, side,
                                 flags=flags)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe.moe_decode_stack(arr, x_tok, x_out, x_tok, EPS, None, ws, ws_bytes, None,
                                 flags=flags)
        step = graph.replay
    else:
        # one cooperative launch per token; x_tok receives RMSNorm(x_out) for the next token
        def step():
            moe.moe_decode_stack(arr, x_tok, x_out, x_tok, EPS, None, ws, ws_bytes, stream,
                                 flags=flags)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup {args.warmup} tokens done", file=sys.stderr, flush=True)

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_tok_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = total_ms / args.steps
    tok_s = 1000.0 / ms_per_step
    bytes_tok = args.layers * layer_bytes(bits, H, I, E, k)
    gbs = bytes_tok * tok_s / 1e9
    dev_err = int(err.item())
    if dev_err != 0:
        print(f"# device error word {dev_err} after the timed tokens (2: a persistent wait timed "
              f"out, 4: workgroups not placed one per CU across the 8 XCDs); outputs undefined",
              file=sys.stderr, flush=True)
        return 1
    assert torch.isfinite(x_out).all().item(), "non-finite stack output"
    print(f"# {args.steps} tokens: {ms_per_step * 1e3:.1f} us/token (median "
          f"{np.median(per_tok_ms) * 1e3:.1f}, p99 {np.percentile(per_tok_ms, 99) * 1e3:.1f}), "
          f"{gbs:.0f} GB/s, wall {wall:.2f} s, device error word 0", file=sys.stderr, flush=True)

    persistent = mode != moe.STACK_KERNELS
    launches = -(-args.layers // 64) if persistent else 1
    bytes_launch = bytes_tok / launches
    avg_launch_s = ms_per_step / 1e3 / launches
    achieved = bytes_launch / avg_launch_s / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": stack_traffic(args.layers) if persistent and bits == 4 else None,
        "kernel": ("persist_kernel (one launch decodes up to 64 layers of one token)" if persistent
                   else "three kernels per layer, one graph replay per token"),
        "bytes_per_launch": round(bytes_launch), "launches_per_token": launches,
        "avg_launch_us": round(avg_launch_s * 1e6, 2),
    }
    result = {
        "metric": METRIC if bits == 4 else METRIC.replace("q4", "q2"), "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.layers}-layer q{bits} MoE-FFN stack decode, batch 1",
                   "layers": args.layers, "hidden": H, "intermediate": I, "experts": E,
                   "top_k": k, "shared_experts": 1, "group": synth.GROUP, "bits": bits,
                   "tokens": args.steps, "resident_bytes": args.layers * (
                       (E + 1) * synth.expert_bytes(bits) + E * H * 4 + H * 4)},
        "hbm_gb_s": round(gbs, 1), "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "us_per_token_median": round(float(np.median(per_tok_ms)) * 1e3, 2),
        "us_per_token_p99": round(float(np.percentile(per_tok_ms, 99)) * 1e3, 2),
        "device_error_word": dev_err,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        # the oracle leg: a one-layer parity sample of the chain (the token after the timed
        # ones, the deepest layer, from the GPU's own layer input), then the oracle's timing
        parity = stack_parity_sample(descs, x_tok, args.layers - 1, bits, flags)
        if int(err.item()) != 0 or not parity["ok"]:
            print(f"# parity sample failed: {parity}, device error word {int(err.item())}",
                  file=sys.stderr, flush=True)
            return 1
        del keep, ws
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(bits, args.layers)
        result["cpu_baseline"]["parity_sample"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
