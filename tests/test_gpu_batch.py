"""Small-batch decode and few-slot launch shapes (marked gpu).

moe_layer_decode_batch / moe_decode_stack_batch run T tokens through the same three kernels as the
single-token calls; each token's result must be bitwise the single-token call's (same arithmetic,
only the grid differs) and match the fp64 oracle per token: ids bit-exact on gap-enforced inputs,
outputs within relative L2 1e-4 and max-abs 1e-3 * max|ref|.  The expert FFN with one, two and
three slots uses smaller blocks (so that the grid still covers the chip); it is checked against the
oracle per slot.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, EPS = 4711, 1e-6


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.fixture(scope="module")
def q4(gpu_available):
    return gu.Layer(SEED, 0, 4)


@pytest.fixture(scope="module")
def q2(gpu_available):
    return gu.Layer(SEED, 1, 2)


def _tokens(lay, T, norm):
    xs, t = [], 0
    for _ in range(T):
        t, x = gu.gap_enforced_x(SEED + 9, lay.wr, gu.K, start=t, norm_input=bool(norm))
        xs.append(x)
        t += 1
    return np.stack(xs)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("T,norm", [(2, 0), (3, 1), (4, 0), (8, 1), (33, 0)])
def test_layer_batch(q4, q2, bits, T, norm):
    lay = q4 if bits == 4 else q2
    X = _tokens(lay, T, norm)
    wsb = moe.moe_layer_batch_workspace_bytes(lay.L, T)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(T, gu.H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, gu.K + 1, dtype=torch.int32, device="cuda")
    w = torch.empty(T, gu.K, dtype=torch.float32, device="cuda")
    sg = torch.empty(T, dtype=torch.float32, device="cuda")
    moe.moe_layer_decode_batch(lay.L, _dev(X), T, norm, EPS, out, ids, w, sg, ws, wsb)
    torch.cuda.synchronize()
    got, gids, gw, gsg = out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), sg.cpu().numpy()
    wsb1 = moe.moe_layer_workspace_bytes(lay.L)
    ws1 = torch.zeros(wsb1, dtype=torch.uint8, device="cuda")
    o1 = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    i1 = torch.empty(gu.K + 1, dtype=torch.int32, device="cuda")
    w1 = torch.empty(gu.K, dtype=torch.float32, device="cuda")
    s1 = torch.empty(1, dtype=torch.float32, device="cuda")
    for t in range(T):
        moe.moe_layer_decode(lay.L, _dev(X[t]), norm, EPS, o1, i1, w1, s1, ws1, wsb1)
        torch.cuda.synchronize()
        assert np.array_equal(got[t], o1.cpu().numpy()), (bits, T, t)
        assert np.array_equal(gids[t], i1.cpu().numpy()) and np.array_equal(gw[t], w1.cpu().numpy())
        assert gsg[t] == s1.cpu().numpy()[0]
        ref = lay.oracle_layer(X[t], norm_input=bool(norm))
        assert gids[t][gu.K] == gu.E
        gu.assert_same_routing(gids[t][:gu.K], gw[t], ref["ids"], ref["weights"], (bits, T, t))
        gu.assert_close(got[t], ref["out"], f"batch q{bits} T={T} token {t}")


@pytest.mark.parametrize("bits", [4, 2])
def test_stack_batch_equals_single_token_stacks(gpu_available, bits):
    T, NL, E = 4, 3, 16
    layers = [gu.Layer(SEED + 3, L, bits, n_experts=E) for L in range(NL)]
    descs = [l.L for l in layers]
    X = np.stack([synth.activations(SEED + 3, t) for t in range(T)])
    wsb = moe.moe_stack_batch_workspace_bytes(descs, T)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x_in = _dev(X)
    x_out = torch.empty(T, gu.H, dtype=torch.float32, device="cuda")
    trace = torch.empty(NL, T, gu.K, dtype=torch.int32, device="cuda")
    moe.moe_decode_stack_batch(descs, x_in, T, x_out, x_in, EPS, trace, ws, wsb)  # xn aliases x_in
    torch.cuda.synchronize()
    got, xn, tr = x_out.cpu().numpy(), x_in.cpu().numpy(), trace.cpu().numpy()
    wsb1 = moe.moe_stack_workspace_bytes(descs)
    ws1 = torch.zeros(wsb1, dtype=torch.uint8, device="cuda")
    for t in range(T):
        a = _dev(X[t])
        o = torch.empty(gu.H, dtype=torch.float32, device="cuda")
        n = torch.empty(gu.H, dtype=torch.float32, device="cuda")
        tt = torch.empty(NL, gu.K, dtype=torch.int32, device="cuda")
        moe.moe_decode_stack(descs, a, o, n, EPS, tt, ws1, wsb1, flags=moe.STACK_KERNELS)
        torch.cuda.synchronize()
        assert np.array_equal(got[t], o.cpu().numpy()) and np.array_equal(xn[t], n.cpu().numpy())
        assert np.array_equal(tr[:, t, :], tt.cpu().numpy())
        otrace = []
        ref = oracle.stack_token(X[t].astype(np.float64), [(l.wr, l.wsg, l.expert_cpu) for l in layers],
                                 bits, gu.K, E, gu.H, gu.I, 64, eps=EPS, trace=otrace)
        for L, r in enumerate(otrace):
            gu.assert_same_routing(tr[L, t], None, r["ids"], None, (t, L))
        gu.assert_close(got[t], ref, f"q{bits} stack batch token {t}")


@pytest.mark.parametrize("n", [1, 2, 3])
def test_expert_ffn_few_slots(q4, n):
    """One to three slots run on smaller blocks (k2) and more waves per slot (k3)."""
    lay = q4
    x = synth.activations(SEED, 21)
    slots = [300, 512, 7][:n]
    ids = torch.tensor(slots, dtype=torch.int32, device="cuda")
    y = torch.empty(n, gu.H, dtype=torch.float32, device="cuda")
    h = torch.empty(n, gu.I, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn_q4(lay.desc, _dev(x), ids, n, y, h)
    torch.cuda.synchronize()
    for j, s in enumerate(slots):
        _, _, h_ref, y_ref = oracle.expert_ffn(4, gu.H, gu.I, 64, lay.expert_cpu(s), x)
        gu.assert_close(h.cpu().numpy()[j], h_ref, f"h slot {s}")
        gu.assert_close(y.cpu().numpy()[j], y_ref, f"y slot {s}")


def test_batch_validation(q4):
    T = 2
    x = torch.zeros(T, gu.H, dtype=torch.float32, device="cuda")
    wsb = moe.moe_layer_batch_workspace_bytes(q4.L, T)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:  # out overlaps x
        moe.moe_layer_decode_batch(q4.L, x, T, 0, EPS, x, None, None, None, ws, wsb)
    assert e.value.status == moe.MOE_E_SHAPE
    assert moe.moe_layer_batch_workspace_bytes(q4.L, 65) == 0
    assert moe.moe_layer_batch_workspace_bytes(q4.L, 0) == 0
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_decode_batch(q4.L, x, T, 0, EPS, torch.empty_like(x), None, None, None, ws,
                                   wsb - 1)
    assert e.value.status == moe.MOE_E_WORKSPACE
