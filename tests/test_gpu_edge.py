"""GPU checks of the packer and of the routing edge cases (marked gpu).

Packer: canonical expert records (gate | up | down, each codes | scale | bias) placed into the
resident slot array by moe_pack, at a slot stride larger than the record, must hold the records
byte for byte, leave the padding untouched, and decode to bitwise the same layer output as slots
filled directly by the generator (the arithmetic only sees the records).

Routing: exact ties between router logits go to the lower expert index and a NaN logit is never
selected, as the oracle does (its tie and NaN rules are pinned by the CPU tests).  The crafted
routers give three clearly leading experts, then two experts whose router rows are identical (so
their logits are bitwise equal on any summation order) competing for the fourth place, and one
expert whose row would lead by far but holds a NaN.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, EPS = 8642, 1e-6
LEAD = {300: 0.30, 7: 0.25, 100: 0.20}   # experts and their share of the input direction
TIE = (50, 20)                           # identical rows: 20 must win the fourth place
TIE_C = 0.15
NAN_E = 400                              # 0.5 of the input direction, and one NaN weight


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _crafted_router(wr, direction):
    """Small random rows (logits ~ N(0, 0.8^2) for a norm-64 input), then the lead, tie and
    NaN rows along the unit vector `direction`."""
    w = (0.1 * wr).astype(np.float32)
    for e, c in LEAD.items():
        w[e] = (c * direction).astype(np.float32)
    for e in TIE:
        w[e] = (TIE_C * direction).astype(np.float32)
    w[NAN_E] = (0.5 * direction).astype(np.float32)
    w[NAN_E, 1234] = np.nan
    return w


EXPECT_IDS = [300, 7, 100, 20]


# ------------------------------------------------------------------------------------------
# packer
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 2])
def test_pack_host_records_into_strided_slots(gpu_available, bits):
    """16 routed + 1 shared expert generated on the host, uploaded back to back and packed in
    two calls into slots 272 bytes wider than a record; then a layer decode of the packed slots
    equals the decode of generator-filled slots bit for bit."""
    E = 16
    n = E + 1
    rec = synth.expert_bytes(bits)
    stride = rec + 272
    host = np.concatenate([synth.expert(SEED, 2, s, bits) for s in range(n)])
    canon = _dev(host)
    slots = torch.full((n * stride,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = moe.experts(slots, bits, gu.H, gu.I, n, stride)
    moe.moe_pack(canon[:10 * rec], 10, 0, dst)
    moe.moe_pack(canon[10 * rec:], n - 10, 10, dst)
    torch.cuda.synchronize()
    got = slots.cpu().numpy().reshape(n, stride)
    for s in range(n):
        assert np.array_equal(got[s, :rec], host[s * rec:(s + 1) * rec]), s
        assert np.all(got[s, rec:] == 0xA5), s
    ref = gu.Layer(SEED, 2, bits, n_experts=E)
    packed = moe.layer(dst, ref.d_wr, ref.d_wsg, E, gu.K, E)
    x = _dev(synth.activations(SEED, 3))
    outs = []
    for L in (packed, ref.L):
        wsb = moe.moe_layer_workspace_bytes(L)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
        ids = torch.empty(gu.K + 1, dtype=torch.int32, device="cuda")
        moe.moe_layer_decode(L, x, 1, EPS, out, ids, None, None, ws, wsb)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), ids.cpu().numpy()))
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][0], outs[1][0])
    res = ref.oracle_layer(synth.activations(SEED, 3), norm_input=True)
    gu.assert_close(outs[0][0], res["out"], f"packed q{bits} layer")


def test_pack_full_layer_persistent_decode(gpu_available):
    """All 513 q4 records of a full-size layer, canonical back to back on the device, packed
    into strided slots: the persistent stack decode of the packed layer equals that of the
    generator-filled layer bit for bit, and sampled slots equal the host generator's bytes."""
    bits, E = 4, gu.E
    n = E + 1
    rec = synth.expert_bytes(bits)
    stride = rec + 4096
    canon = torch.empty(n * rec, dtype=torch.uint8, device="cuda")
    synth.gpu_fill_experts(canon.data_ptr(), rec, 0, n, SEED, 5, bits, stream=gu.stream_handle())
    slots = torch.zeros(n * stride, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dst = moe.experts(slots, bits, gu.H, gu.I, n, stride, dev_err=err)
    moe.moe_pack(canon, n, 0, dst)
    torch.cuda.synchronize()
    del canon
    for s in (0, 1, 255, 511, 512):
        got = slots[s * stride:s * stride + rec].cpu().numpy()
        assert np.array_equal(got, synth.expert(SEED, 5, s, bits)), s
    ref = gu.Layer(SEED, 5, bits, dev_err=err)
    packed = moe.layer(dst, ref.d_wr, ref.d_wsg, E, gu.K, E, w_router_cb=ref.d_wr_cb)
    x = _dev(synth.activations(SEED, 6))
    outs = []
    for L in (packed, ref.L):
        wsb = moe.moe_stack_workspace_bytes([L])
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
        trace = torch.empty(1, gu.K, dtype=torch.int32, device="cuda")
        moe.moe_decode_stack([L], x, out, None, EPS, trace, ws, wsb, flags=moe.STACK_PERSISTENT)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), trace.cpu().numpy()))
    assert int(err.item()) == 0
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][0], outs[1][0])


# ------------------------------------------------------------------------------------------
# routing: exact ties and NaN logits
# ------------------------------------------------------------------------------------------

def test_router_topk_tie_and_nan(gpu_available):
    rng = np.random.default_rng(5)
    T = 3
    X = rng.standard_normal((T, gu.H)).astype(np.float32)
    base = synth.router_weights(SEED, 0)
    ids = torch.empty(T, gu.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, gu.K, dtype=torch.float32, device="cuda")
    wsb = moe.moe_router_workspace_bytes(T, gu.E)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for t in range(T):
        d = X[t].astype(np.float64) / np.linalg.norm(X[t])
        wr = _crafted_router(base, d)
        moe.moe_router_topk(_dev(X[t]), 1, _dev(wr), None, gu.H, gu.E, gu.K, ids[t], gu.K, w[t],
                            None, ws, wsb)
        torch.cuda.synchronize()
        logits = oracle.router_logits(wr, X[t])
        assert np.isnan(logits[NAN_E]) and logits[TIE[0]] == logits[TIE[1]]
        rid, rw = oracle.topk(logits, gu.K)
        assert rid.tolist() == EXPECT_IDS
        got = ids.cpu().numpy()[t]
        assert got.tolist() == EXPECT_IDS, got  # order too: descending logit, ties to lower id
        np.testing.assert_allclose(w.cpu().numpy()[t], rw, rtol=1e-5, atol=1e-7)


def test_persistent_topk_tie_and_nan(gpu_available):
    """The same crafted router in a full-size q4 layer through the persistent kernel (whose
    top-4 runs on the all-reduced K-split logits of the normalised input); the whole layer
    output is compared with the oracle too."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lay = gu.Layer(SEED, 9, 4, dev_err=err)
    x = synth.activations(SEED, 10)
    xn = oracle.rmsnorm(x, EPS)
    wr = _crafted_router(lay.wr, xn / np.linalg.norm(xn))
    lay.wr = wr
    lay.d_wr.copy_(torch.from_numpy(wr))
    moe.moe_pack_router(lay.d_wr, gu.E, gu.H, lay.d_wr_cb)
    for L in (lay.L, lay.L_plain):  # blocked router copy and plain router layout
        wsb = moe.moe_stack_workspace_bytes([L])
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
        trace = torch.empty(1, gu.K, dtype=torch.int32, device="cuda")
        moe.moe_decode_stack([L], _dev(x), out, None, EPS, trace, ws, wsb,
                             flags=moe.STACK_PERSISTENT)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert trace.cpu().numpy()[0].tolist() == EXPECT_IDS
        ref = lay.oracle_layer(x, norm_input=True)
        assert ref["ids"].tolist() == EXPECT_IDS and np.isnan(ref["logits"][NAN_E])
        gu.assert_close(out.cpu().numpy(), ref["out"], "persistent layer, crafted router")
