"""Per-phase timeline of the persistent decode kernel (an instrumentation build of libmoe).

    python -m group_quantized_expert_amd.phase_timeline --build   # on any host: hipcc, gfx950
    python -m group_quantized_expert_amd.phase_timeline           # on the GPU

--build compiles libmoe_stamps.so beside libmoe.so from the same sources with
-DMOE_PHASE_STAMPS, which makes one lane of the wave that reaches each phase boundary of each
layer write the GPU's 100 MHz real-time counter (s_memrealtime) to a device buffer.  The run
decodes tokens through a resident 60-layer q4 stack (the bench's synthetic weights), once with
the stamps off (the instrumented kernel's own token time) and then token by token with the
stamps on, and prints, for each event, its time after the layer's start (the median over the
256 workgroups of exchange wave 0's loop start), as medians and 90th percentiles over
workgroups and the layers 2..57.  The stamps cost a few stores per layer; the timed run with
them off shows how close the instrumented kernel stays to libmoe.so.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
OUT = os.path.join(_HERE, "libmoe_stamps.so")
N_EVENTS = 32  # stamps per (layer, workgroup), as laid out by the kernel
N_WG = 256
MAX_LAYERS = 64

# event -> (who writes it, what it marks); the order of a layer's phases
EVENTS = {
    0: ("x0", "layer start (exchange wave 0 enters the layer)"),
    1: ("x0", "router hop 1 done (XCD-local slice sums)"),
    2: ("x0", "router hop 2 done (slice sums across XCDs)"),
    3: ("x0", "router hop 3 done (whole logit vector read)"),
    4: ("x0", "top-4 done, ids flag set"),
    15: ("x2", "layer input gathered into LDS"),
    5: ("c0", "compute wave 0 has issued its gate/up rows"),
    16: ("x2", "input digit planes written"),
    6: ("c0", "compute wave 0 sees the digit planes"),
    7: ("c0", "gate/up partial sums done"),
    8: ("c0", "SwiGLU outputs published; at barrier E"),
    9: ("x0", "down rows loaded"),
    10: ("x0", "SwiGLU outputs of all workgroups gathered"),
    11: ("x0", "past barrier E"),
    12: ("c0", "routed down products done, next layer's prefetch issued; at barrier F"),
    13: ("x0", "past barrier F (shared slot's down rows done)"),
    14: ("x0", "output rows and next layer's router partials published"),
}


def build(verbose: bool = False) -> str:
    from group_quantized_expert_amd import build as b
    cmd = [b.HIPCC, *b.FLAGS, "-DMOE_PHASE_STAMPS",
           *[os.path.join(b.CSRC, s) for s in b.SOURCES], "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, cwd=b.CSRC, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "is not a recognized feature" not in l)
        raise RuntimeError(f"hipcc failed:\n{msgs}")
    os.replace(OUT + ".tmp", OUT)
    return OUT


def run(n_layers: int, tokens: int) -> None:
    import numpy as np
    import torch
    if _ROOT not in sys.path:
        sys.path.insert(0, _ROOT)
    import group_quantized_expert_amd as moe
    if not os.path.exists(OUT):
        raise RuntimeError(f"{OUT} is missing: run this module with --build first")
    moe.LIB_PATH = OUT
    L_ = moe.lib()
    L_.moe_phase_stamps.argtypes = [ctypes.c_void_p]
    L_.moe_phase_stamps.restype = None
    import bench
    import synth

    dev = torch.device("cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    descs, keep = bench.build_stack(n_layers, 4, dev, dev_err=err)
    arr = (moe.MoeLayer * n_layers)(*descs)
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    x = torch.from_numpy(synth.activations(bench.SEED_X, 0)).to(dev)
    xo = torch.empty_like(x)
    stamps = torch.zeros(MAX_LAYERS * N_WG * N_EVENTS, dtype=torch.int64, device=dev)

    def token():
        moe.moe_decode_stack(arr, x, xo, x, 1e-6, None, ws, wsb, flags=moe.STACK_PERSISTENT)

    print(f"# {n_layers}-layer q4 stack resident; instrumented library {OUT}", flush=True)
    for _ in range(5):
        token()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        token()
    e1.record()
    torch.cuda.synchronize()
    print(f"# stamps off: {e0.elapsed_time(e1) / 20 * 1e3:.1f} us per token (20 tokens)", flush=True)

    L_.moe_phase_stamps(stamps.data_ptr())
    rel = {ev: [] for ev in EVENTS}
    periods, tok_us = [], []
    inner = range(2, n_layers - 2)
    for _ in range(tokens):
        stamps.zero_()
        e0.record()
        token()
        e1.record()
        torch.cuda.synchronize()
        tok_us.append(e0.elapsed_time(e1) * 1e3)
        T = stamps.cpu().numpy().reshape(MAX_LAYERS, N_WG, N_EVENTS)[:n_layers].astype(np.float64)
        T *= 1e-2  # 100 MHz ticks -> us
        start = np.median(T[:, :, 0], axis=1)
        periods += list(np.diff(start)[1:-1])
        for ev in EVENTS:
            rel[ev].append(np.concatenate([T[l, :, ev] - start[l] for l in inner]))
    L_.moe_phase_stamps(None)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item())}")
    print(f"# stamps on: {np.median(tok_us):.1f} us per token (median of {tokens} single tokens); "
          f"layer period median {np.median(periods):.2f} us "
          f"(p10 {np.percentile(periods, 10):.2f}, p90 {np.percentile(periods, 90):.2f})")
    print(f"# events: us after the layer's start, over {N_WG} workgroups x layers "
          f"{inner.start}..{inner.stop - 1} x {tokens} tokens; device error word 0")
    print("| event | wave | median | p90 |")
    print("|---|---|---|---|")
    for ev, (who, what) in sorted(EVENTS.items(), key=lambda kv: np.median(np.concatenate(rel[kv[0]]))):
        d = np.concatenate(rel[ev])
        print(f"| {what} | {who} | {np.median(d):.2f} | {np.percentile(d, 90):.2f} |")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--build", action="store_true", help="compile libmoe_stamps.so and exit")
    ap.add_argument("--layers", type=int, default=60)
    ap.add_argument("--tokens", type=int, default=3)
    args = ap.parse_args()
    if args.build:
        print(build(verbose=True))
        return
    if not 6 <= args.layers <= MAX_LAYERS:
        raise SystemExit(f"--layers must be in 6..{MAX_LAYERS}")
    run(args.layers, args.tokens)


if __name__ == "__main__":
    main()
