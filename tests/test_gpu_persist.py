"""GPU parity of the persistent stack decode (one cooperative launch per token; marked gpu).

Full-size q4 and q2 layers (512 routed + 1 shared expert, H 4096, I 1024) so that the persistent
kernel is the one that runs.  Checks: routed expert sets and outputs against the fp64 oracle chain;
agreement with the kernel-per-step path; the same bits with and without the column-blocked
router copy, and that copy's layout; bitwise run-to-run determinism across repeated launches
(the exchange tags advance every launch); the split of stacks longer than 64 layers into several
launches, which must equal running the pieces one after the other; the device error word stays 0.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, SEED_X, NL, EPS = 97531, 4242, 3, 1e-6


@pytest.fixture(scope="module", params=[4, 2], ids=["q4", "q2"])
def layers(request, gpu_available):
    bits = request.param
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ls = [gu.Layer(SEED, L, bits, dev_err=err) for L in range(NL)]
    yield ls, err, bits
    del ls
    torch.cuda.empty_cache()


def _run(descs, x_np, mode, n_trace=None):
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x_in = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
    x_out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    xn = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    trace = torch.full((len(descs), gu.K), -7, dtype=torch.int32, device="cuda")
    moe.moe_decode_stack(descs, x_in, x_out, xn, EPS, trace, ws, wsb, flags=mode)
    torch.cuda.synchronize()
    return x_out.cpu().numpy(), xn.cpu().numpy(), trace.cpu().numpy()


def test_persist_matches_oracle(layers):
    ls, err, bits = layers
    x0 = synth.activations(SEED_X, 0)
    out, xn, trace = _run([l.L for l in ls], x0, moe.STACK_PERSISTENT)
    assert int(err.item()) == 0
    otrace = []
    ref = oracle.stack_token(np.asarray(x0, np.float64), [(l.wr, l.wsg, l.expert_cpu) for l in ls],
                             bits, gu.K, gu.E, gu.H, gu.I, 64, eps=EPS, trace=otrace)
    for L, r in enumerate(otrace):
        gu.assert_same_routing(trace[L], None, r["ids"], None, ("layer", L))
    gu.assert_close(out, ref, "persistent stack output")
    gu.assert_close(xn, oracle.rmsnorm(ref, EPS), "persistent normalised output")


def test_persist_matches_kernel_path(layers):
    ls, err, bits = layers
    descs = [l.L for l in ls]
    for t in range(3):
        x = synth.activations(SEED_X, 100 + t)
        a, an, ta = _run(descs, x, moe.STACK_PERSISTENT)
        b, bn, tb = _run(descs, x, moe.STACK_KERNELS)
        for L in range(NL):
            gu.assert_same_routing(ta[L], None, tb[L], None, ("token", t, "layer", L))
        gu.assert_close(a, b, f"token {t}: persistent vs kernel path")
        gu.assert_close(an, bn, f"token {t}: normalised")
    assert int(err.item()) == 0


def test_pack_router_layout(layers):
    ls, _, _ = layers
    l = ls[0]
    want = l.wr.reshape(gu.E, gu.H // 16, 16).transpose(1, 0, 2)
    assert np.array_equal(l.d_wr_cb.cpu().numpy().reshape(gu.H // 16, gu.E, 16), want)
    # a small odd shape through the grid-stride loop
    w = torch.arange(7 * 48, dtype=torch.float32, device="cuda").reshape(7, 48)
    d = torch.full_like(w, -1.0)
    moe.moe_pack_router(w, 7, 48, d)
    torch.cuda.synchronize()
    ref = w.cpu().numpy().reshape(7, 3, 16).transpose(1, 0, 2)
    assert np.array_equal(d.cpu().numpy().reshape(3, 7, 16), ref)


def test_persist_router_copy_same_bits(layers):
    """The blocked router copy changes only where the next layer's router columns are read
    from, not the arithmetic: outputs and routing are bitwise those of the plain layout."""
    ls, err, bits = layers
    for t in range(2):
        x = synth.activations(SEED_X, 200 + t)
        a, an, ta = _run([l.L for l in ls], x, moe.STACK_PERSISTENT)
        b, bn, tb = _run([l.L_plain for l in ls], x, moe.STACK_PERSISTENT)
        assert np.array_equal(ta, tb)
        assert np.array_equal(a, b) and np.array_equal(an, bn)
    assert int(err.item()) == 0


def test_persist_autoregressive_deterministic(layers):
    """Four tokens fed back through one workspace (xn_out aliases x_in), twice from the same
    start: every launch advances the exchange epoch, the results must not change."""
    ls, err, bits = layers
    descs = [l.L for l in ls]
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x_tok = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    x_out = torch.empty(gu.H, dtype=torch.float32, device="cuda")
    runs = []
    for _ in range(2):
        x_tok.copy_(torch.from_numpy(synth.activations(SEED_X, 7)))
        outs = []
        for _t in range(4):
            moe.moe_decode_stack(descs, x_tok, x_out, x_tok, EPS, None, ws, wsb,
                                 flags=moe.STACK_PERSISTENT)
            outs.append(x_out.clone())
        torch.cuda.synchronize()
        runs.append(torch.stack(outs).cpu().numpy())
    assert np.array_equal(runs[0], runs[1])
    assert np.all(np.isfinite(runs[0]))
    assert int(err.item()) == 0


def test_persist_long_stack_is_split(layers):
    """70 layers (the 3 resident layers repeated) exceed one launch's 64: the result must equal
    running layers 0..63 and then 64..69 as two calls."""
    ls, err, bits = layers
    descs = [ls[i % NL].L for i in range(70)]
    x = synth.activations(SEED_X, 11)
    out, xn, trace = _run(descs, x, moe.STACK_PERSISTENT)
    a, _, ta = _run(descs[:64], x, moe.STACK_PERSISTENT)
    # the second piece starts from the raw output of the first (each layer normalises its input)
    b, bn, tb = _run(descs[64:], a, moe.STACK_PERSISTENT)
    assert np.array_equal(out, b) and np.array_equal(xn, bn)
    assert np.array_equal(trace[:64], ta) and np.array_equal(trace[64:], tb)
    assert int(err.item()) == 0
