"""Full-size parity of the 60-layer q4 decode stack (marked gpu).

The benchmark workload: 60 resident layers of 512 routed + 1 shared q4 experts (218 GB), decoded
autoregressively at batch 1 with the per-layer RMSNorm and the token-to-token feedback.  The oracle
runs its own fp64 chain from the same token input and never takes a value from the GPU; it
regenerates on the host only the experts its routing selects.

Token 0: every layer's routed expert set matches and the 60-layer output is within relative L2 1e-4
and max-abs 1e-3 * max|ref|.

Token 1 starts from RMSNorm of token 0's output, and its trajectory amplifies perturbations: run
through the oracle alone, a 1e-7 relative perturbation of its input grows to ~4e-3 after 60 layers,
so no fp32 computation can match the fp64 chain to 1e-4 over all 60 layers.  It is therefore checked
(a) in 6-layer windows that the GPU runs from the oracle's own layer states, each within the 1e-4
bar, and (b) as the GPU-chained continuation the benchmark times: the same routed expert set at
every layer, and the output within 5e-2 relative L2 of the oracle chain.  In (b) a layer may
select differently only where the oracle's 4th and 5th logits are closer than the chain's own
rounding drift can reach at that depth (the token-1 input's deviation, grown by the measured
4e4 over 60 layers, times 10); both selections are then correct, the chains part there, and the
comparison stops at that layer.

Later tokens (4, 12 and 24 of the chain the benchmark decodes, every token fed back through
RMSNorm of the previous output): one-step parity at every layer from the GPU's own layer input.
The token's 60 layers are re-run as 60 one-layer launches (bitwise the same as the one 60-layer
launch, which is checked), and each layer's output is compared with the oracle's layer step on the
same input at the 1e-4 bar.  Routed sets must match where the oracle's 4th/5th logit gap is at
least 1e-3; below that (a near-tie the generator cannot exclude for computed inputs) every GPU id's
oracle logit must be within 1e-4 of the 4th, and the layer is counted and reported.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED_W, SEED_X, LAYERS, EPS, WINDOW = 20260301, 777, 60, 1e-6, 6


ERR = None


@pytest.fixture(scope="module")
def stack(gpu_available):
    global ERR
    free, total = torch.cuda.mem_get_info()
    need = LAYERS * (gu.E + 1) * synth.expert_bytes(4)
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    ERR = torch.zeros(1, dtype=torch.int32, device="cuda")
    layers = [gu.Layer(SEED_W, L, 4, dev_err=ERR) for L in range(LAYERS)]
    yield layers
    del layers
    torch.cuda.empty_cache()


def _gpu_stack(layers, x_in_np, trace=None):
    descs = [l.L for l in layers]
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x_in = torch.from_numpy(np.ascontiguousarray(x_in_np, dtype=np.float32)).cuda()
    x_out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    xn = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    moe.moe_decode_stack(descs, x_in, x_out, xn, EPS, trace, ws, wsb)
    torch.cuda.synchronize()
    assert int(ERR.item()) == 0, "persistent kernel reported a device error"
    return x_out.cpu().numpy(), xn.cpu().numpy()


def _oracle_chain(layers, x0):
    trace = []
    out = oracle.stack_token(np.asarray(x0, dtype=np.float64),
                             [(l.wr, l.wsg, l.expert_cpu) for l in layers], 4, gu.K, gu.E, gu.H,
                             gu.I, 64, eps=EPS, trace=trace)
    return out, trace


def test_stack_token0_full_chain(stack):
    x0 = synth.activations(SEED_X, 0)
    trace = torch.empty(LAYERS, gu.K, dtype=torch.int32, device="cuda")
    out, xn = _gpu_stack(stack, x0, trace)
    ref, otrace = _oracle_chain(stack, x0)
    got = trace.cpu().numpy()
    for L, r in enumerate(otrace):
        gu.assert_same_routing(got[L], None, r["ids"], None, ("token 0", L))
    gu.assert_close(out, ref, "token 0 stack output")
    gu.assert_close(xn, oracle.rmsnorm(ref, EPS), "token 0 normalised output")


def test_stack_token1_windows_and_continuation(stack):
    x0 = synth.activations(SEED_X, 0)
    ref0, _ = _oracle_chain(stack, x0)
    x1 = oracle.rmsnorm(ref0, EPS)  # the oracle's own token-1 input
    ref1, otrace = _oracle_chain(stack, x1)
    states = [x1] + [r["out"] for r in otrace]  # oracle layer states x_0 .. x_60 of token 1
    # (a) 6-layer windows run on the GPU from the oracle's states (perturbations of this
    # trajectory grow about 5x per 6 layers, so each window stays far inside the bar)
    for L0 in range(0, LAYERS, WINDOW):
        win = stack[L0:L0 + WINDOW]
        trace = torch.empty(len(win), gu.K, dtype=torch.int32, device="cuda")
        out, _ = _gpu_stack(win, states[L0].astype(np.float32), trace)
        got = trace.cpu().numpy()
        for j, r in enumerate(otrace[L0:L0 + WINDOW]):
            gu.assert_same_routing(got[j], None, r["ids"], None, ("token 1 window", L0 + j))
        gu.assert_close(out, states[L0 + len(win)], f"token 1 layers {L0}..{L0 + len(win) - 1}")
    # (b) the GPU-chained continuation (what the benchmark decodes)
    _, xn0 = _gpu_stack(stack, x0)
    trace = torch.empty(LAYERS, gu.K, dtype=torch.int32, device="cuda")
    out1, _ = _gpu_stack(stack, xn0, trace)
    got = trace.cpu().numpy()
    assert np.all(np.isfinite(out1))
    drift0 = max(gu.rel_l2(xn0, x1), 1e-7)
    part = gu.chained_routing(got, otrace, drift0, gu.K, LAYERS, "token 1 chained")
    if part is not None:
        return  # the chains part at a near-tie: later layers and the output are not comparable
    assert gu.rel_l2(out1, ref1) <= 5e-2


def test_stack_later_tokens_one_step_parity(stack):
    descs = [l.L for l in stack]
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x_tok = torch.from_numpy(synth.activations(SEED_X, 0)).cuda()
    x_out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    sampled = {4: None, 12: None, 24: None}
    for t in range(max(sampled) + 1):
        if t in sampled:
            sampled[t] = x_tok.clone()
        moe.moe_decode_stack(descs, x_tok, x_out, x_tok, EPS, None, ws, wsb)
        if t in sampled:
            sampled[t] = (sampled[t], x_out.clone())
    torch.cuda.synchronize()
    assert int(ERR.item()) == 0
    near_ties = []
    one = torch.empty(1, gu.K, dtype=torch.int32, device="cuda")
    for t, (x_in, x_full) in sampled.items():
        state = x_in.clone()
        nxt = torch.empty_like(state)
        for L, lay in enumerate(stack):
            moe.moe_decode_stack([lay.L], state, nxt, None, EPS, one, ws, wsb)
            torch.cuda.synchronize()
            xin = state.cpu().numpy().astype(np.float64)
            got = nxt.cpu().numpy()
            ids = sorted(int(v) for v in one.cpu().numpy()[0])
            ref = lay.oracle_layer(xin, norm_input=True)
            lg = np.sort(ref["logits"])[::-1]
            gap = lg[gu.K - 1] - lg[gu.K]
            if ids != sorted(int(v) for v in ref["ids"]):
                assert gap < 1e-3, (t, L, ids, ref["ids"], gap)
                assert all(ref["logits"][e] >= lg[gu.K - 1] - 1e-4 for e in ids), (t, L)
                near_ties.append((t, L, float(gap)))
            else:
                gu.assert_close(got, ref["out"], f"token {t} layer {L}")
            state, nxt = nxt, state
        assert np.array_equal(state.cpu().numpy(), x_full.cpu().numpy()), \
            f"token {t}: 60 one-layer launches differ from the one-launch stack"
    assert int(ERR.item()) == 0
    print(f"later-token one-step parity: {3 * LAYERS} layer-tokens, near-ties with a different "
          f"(valid) set: {near_ties}")
