"""Pins for the fp64 CPU oracle (CPU only).

Each test checks the oracle against something other than itself: values derived by hand from the
pages' definitions (tests/golden/*.json), closed forms of special cases, invariants, library
routines (scipy / torch CPU) for textbook functions, and exact rational arithmetic.  Each is
chosen so that a plausible mistake (swapped nibbles, transposed scale planes, a dropped bias,
swapped SwiGLU operands, a missing renormalisation, a sum instead of a mean) fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from tests import qpack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _golden_record(fx):
    rows = []
    for r in range(fx["rows"]):
        row = []
        for hexbyte, count in fx["codes_bytes"][f"row{r}"]:
            row += [int(hexbyte, 16)] * count
        rows.append(row)
    codes = np.array(rows, dtype=np.uint8).reshape(-1)
    s = np.array([[int(h, 16) for h in r] for r in fx["scale_bf16_hex"]], dtype=np.uint16)
    b = np.array([[int(h, 16) for h in r] for r in fx["bias_bf16_hex"]], dtype=np.uint16)
    return np.concatenate([codes, s.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)])


def _golden_x(name, C):
    if name == "ones":
        return np.ones(C)
    if name == "iota":
        return np.arange(C, dtype=np.float64)
    if name.startswith("onehot"):
        x = np.zeros(C)
        x[int(name[6:])] = 1.0
        return x
    raise ValueError(name)


# --------------------------------------------------------------------------------------------
# layout (P0)
# --------------------------------------------------------------------------------------------

def test_expert_record_sizes_match_pages():
    # a2a-mcp.org deep dive 1 and the kitpa.org news item give ~6.75 MB per 4-bit expert;
    # the damoang.net repost gives ~3.9 MB per expert, which is the 2-bit record.
    q4 = oracle.expert_bytes(4, 4096, 1024, 64)
    q2 = oracle.expert_bytes(2, 4096, 1024, 64)
    assert q4 == 7_077_888 == int(6.75 * 2 ** 20)
    assert q2 == 3_932_160 and round(q2 / 1e6, 1) == 3.9
    assert synth.expert_bytes(4) == q4 and synth.expert_bytes(2) == q2


# --------------------------------------------------------------------------------------------
# dequant matvec (P1-P5)
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["q4_tiny_matvec.json", "q2_tiny_matvec.json"])
def test_golden_matvec(name):
    fx = _golden(name)
    rec = _golden_record(fx)
    bits, R, C, G = fx["bits"], fx["rows"], fx["cols"], fx["group"]
    for case in fx["cases"]:
        x = _golden_x(case["x"], C)
        for fn in (oracle.qmatvec, oracle.qmatvec_fma_form, oracle.qmatvec_xsum_form):
            y = fn(bits, R, C, G, rec, x)
            assert y.tolist() == case["y"], (fn.__name__, case)


@pytest.mark.parametrize("bits", [4, 2])
def test_zero_codes_give_bias_times_group_sum(bits):
    rng = np.random.default_rng(1)
    R, C, G = 16, 4096, 64
    Q = np.zeros((R, C), dtype=np.uint8)
    s = qpack.random_bf16(rng, (R, C // G), 0.01, 0.03)
    b = qpack.random_bf16(rng, (R, C // G), 0.05, 0.3, signed=True)
    rec = qpack.record(bits, Q, s, b)
    x = rng.standard_normal(C)
    Xg = x.reshape(C // G, G).sum(axis=1)
    expect = qpack.bf16_bits_to_f64(b) @ Xg
    y = oracle.qmatvec(bits, R, C, G, rec, x)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [4, 2])
def test_onehot_selects_one_dequantized_column(bits):
    rng = np.random.default_rng(2)
    R, C, G = 8, 256, 64
    Q = rng.integers(0, 1 << bits, size=(R, C), dtype=np.uint8)
    s = qpack.random_bf16(rng, (R, C // G), 0.01, 0.5)
    b = qpack.random_bf16(rng, (R, C // G), 0.01, 0.5, signed=True)
    rec = qpack.record(bits, Q, s, b)
    sf, bf = qpack.bf16_bits_to_f64(s), qpack.bf16_bits_to_f64(b)
    for j in [0, 1, 2, 3, 63, 64, 65, 130, 255]:
        x = np.zeros(C)
        x[j] = 1.0
        y = oracle.qmatvec(bits, R, C, G, rec, x)
        expect = Q[:, j] * sf[:, j // G] + bf[:, j // G]
        assert np.array_equal(y, expect), j


@pytest.mark.parametrize("bits", [4, 2])
def test_zero_scale_and_bias_give_zero(bits):
    rng = np.random.default_rng(3)
    R, C, G = 4, 128, 64
    Q = rng.integers(0, 1 << bits, size=(R, C), dtype=np.uint8)
    z = np.zeros((R, C // G), dtype=np.uint16)
    y = oracle.qmatvec(bits, R, C, G, qpack.record(bits, Q, z, z), rng.standard_normal(C))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("bits", [4, 2])
def test_ones_input_gives_integer_code_sums(bits):
    rng = np.random.default_rng(4)
    R, C, G = 8, 512, 64
    Q = rng.integers(0, 1 << bits, size=(R, C), dtype=np.uint8)
    s = qpack.random_bf16(rng, (R, C // G), 0.01, 0.03)
    b = qpack.random_bf16(rng, (R, C // G), 0.05, 0.3, signed=True)
    rec = qpack.record(bits, Q, s, b)
    qsum = Q.reshape(R, C // G, G).astype(np.int64).sum(axis=2)
    expect = (qpack.bf16_bits_to_f64(s) * qsum + G * qpack.bf16_bits_to_f64(b)).sum(axis=1)
    y = oracle.qmatvec(bits, R, C, G, rec, np.ones(C))
    np.testing.assert_allclose(y, expect, rtol=1e-14)


def _frac_bf16(bits16):
    f = float(qpack.bf16_bits_to_f64(np.array([bits16], dtype=np.uint16))[0])
    return Fraction(f)


@pytest.mark.parametrize("bits,C", [(4, 64), (4, 128), (2, 64), (2, 128)])
def test_rearranged_forms_are_exact_identities(bits, C):
    """Naive dequant-then-dot, the fma(code, s*x, b*x) form and the per-group x-sum form agree
    exactly in rational arithmetic, and the oracle's fp64 results sit within 1e-12 of it."""
    rng = np.random.default_rng(5 + C + bits)
    R, G = 4, 64
    nq = 1 << bits
    Q = (np.arange(R * C).reshape(R, C) * 7 + rng.integers(0, nq, size=(R, C))) % nq
    Q = Q.astype(np.uint8)
    for r in range(R):  # every code value appears in every group of every row
        for g in range(C // G):
            Q[r, g * G:g * G + nq] = np.arange(nq)
    s = qpack.random_bf16(rng, (R, C // G), 0.01, 0.06)
    b = qpack.random_bf16(rng, (R, C // G), 0.01, 0.5, signed=True)
    x = rng.standard_normal(C).astype(np.float32).astype(np.float64)
    rec = qpack.record(bits, Q, s, b)
    xf = [Fraction(float(v)) for v in x]
    for r in range(R):
        naive = Fraction(0)
        fmaf = Fraction(0)
        xsum = Fraction(0)
        for g in range(C // G):
            sg, bg = _frac_bf16(s[r, g]), _frac_bf16(b[r, g])
            qx = Fraction(0)
            xs = Fraction(0)
            for c in range(g * G, (g + 1) * G):
                q = int(Q[r, c])
                naive += (q * sg + bg) * xf[c]
                fmaf += q * (sg * xf[c]) + bg * xf[c]
                qx += q * xf[c]
                xs += xf[c]
            xsum += sg * qx + bg * xs
        assert naive == fmaf == xsum
        scale = max(1.0, abs(float(naive)))
        for fn in (oracle.qmatvec, oracle.qmatvec_fma_form, oracle.qmatvec_xsum_form):
            y = fn(bits, R, C, G, rec, x)
            assert abs(y[r] - float(naive)) <= 1e-12 * scale, fn.__name__


def test_matvec_is_linear_in_x():
    rng = np.random.default_rng(6)
    R, C, G = 8, 1024, 64
    rec = qpack.record(4, *qpack.random_matrix(rng, 4, R, C, G))
    x1, x2 = rng.standard_normal(C), rng.standard_normal(C)
    y = oracle.qmatvec(4, R, C, G, rec, x1 + x2)
    np.testing.assert_allclose(y, oracle.qmatvec(4, R, C, G, rec, x1) +
                               oracle.qmatvec(4, R, C, G, rec, x2), rtol=1e-11, atol=1e-11)


def test_dequant_matches_matvec_against_library_matmul():
    rng = np.random.default_rng(7)
    R, C, G = 32, 512, 64
    rec = qpack.record(2, *qpack.random_matrix(rng, 2, R, C, G))
    W = oracle.dequant(2, R, C, G, rec)
    x = rng.standard_normal(C)
    np.testing.assert_allclose(oracle.qmatvec(2, R, C, G, rec, x), W @ x, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------------
# router, softmax, top-k, shared gate (P6-P8)
# --------------------------------------------------------------------------------------------

def test_golden_router():
    fx = _golden("router_tiny.json")
    W = np.array(fx["w_router"], dtype=np.float32)
    logits = oracle.router_logits(W, fx["x"])
    assert logits.tolist() == fx["logits"]
    ids, w = oracle.topk(logits, fx["k"])
    assert ids.tolist() == fx["ids"]
    np.testing.assert_allclose(w, fx["weights"], rtol=1e-15)


def test_router_onehot_is_column():
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((512, 4096)) / 8).astype(np.float32)
    for j in [0, 17, 4095]:
        x = np.zeros(4096)
        x[j] = 1.0
        assert np.array_equal(oracle.router_logits(W, x), W[:, j].astype(np.float64))


def test_softmax_matches_library_and_is_stable():
    rng = np.random.default_rng(9)
    l = rng.standard_normal(512) * 8
    np.testing.assert_allclose(oracle.softmax(l), scipy.special.softmax(l), rtol=1e-13)
    big = np.array([1000.0, 999.0, -1000.0])
    p = oracle.softmax(big)
    assert np.all(np.isfinite(p))
    np.testing.assert_allclose(p, scipy.special.softmax(big), rtol=1e-13)


def test_topk_closed_form_weights():
    l = np.full(512, -50.0)
    l[[10, 300, 7, 99]] = [3.0, 2.0, 1.0, 0.0]
    ids, w = oracle.topk(l, 4)
    assert ids.tolist() == [10, 300, 7, 99]
    e = np.exp([3.0, 2.0, 1.0, 0.0])
    np.testing.assert_allclose(w, e / e.sum(), rtol=1e-14)
    # renormalised weights do not depend on the other logits nor on a common shift
    l2 = l.copy()
    l2[[0, 1, 2]] = [-1.0, -2.0, -0.5]
    ids2, w2 = oracle.topk(l2 + 123.0, 4)
    assert ids2.tolist() == ids.tolist()
    np.testing.assert_allclose(w2, w, rtol=1e-12)


def test_topk_ties_go_to_lower_index_and_nan_is_never_chosen():
    l = np.zeros(16)
    l[[3, 9, 12]] = 5.0
    l[5] = np.nan
    ids, w = oracle.topk(l, 4)
    assert ids.tolist() == [3, 9, 12, 0]
    np.testing.assert_allclose(w.sum(), 1.0, rtol=1e-15)
    assert 5 not in ids.tolist()


def test_topk_matches_library_sort_bruteforce():
    rng = np.random.default_rng(10)
    for trial in range(200):
        E = int(rng.integers(4, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        l = rng.integers(-3, 4, size=E).astype(np.float64)  # many ties
        ids, w = oracle.topk(l, k)
        order = np.lexsort((np.arange(E), -l))[:k]
        assert ids.tolist() == order.tolist()
        p = scipy.special.softmax(l)[order]
        np.testing.assert_allclose(w, p / p.sum(), rtol=1e-13)


def test_shared_gate_sigmoid():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(4096)
    assert oracle.shared_gate(np.zeros(4096, dtype=np.float32), x) == 0.5
    w = np.zeros(4096, dtype=np.float32)
    w[5] = 0.75
    xo = np.zeros(4096)
    xo[5] = 2.0
    assert oracle.shared_gate(w, xo) == pytest.approx(scipy.special.expit(1.5), rel=1e-15)
    w2 = (rng.standard_normal(4096) / 8).astype(np.float32)
    a = float(w2.astype(np.float64) @ x)
    assert oracle.shared_gate(w2, x) == pytest.approx(scipy.special.expit(a), rel=1e-13)


# --------------------------------------------------------------------------------------------
# expert FFN, SwiGLU, combine, RMSNorm (P9-P10)
# --------------------------------------------------------------------------------------------

def _const_matrix(bits, R, C, G, code, scale_bits, bias_bits):
    Q = np.full((R, C), code, dtype=np.uint8)
    s = np.full((R, C // G), scale_bits, dtype=np.uint16)
    b = np.full((R, C // G), bias_bits, dtype=np.uint16)
    return Q, s, b


def test_swiglu_operand_order_and_down_projection():
    """gate, up and down built so g, u, h and y are known: h = silu(g) * u, y = W_down h."""
    bits, H, I, G = 4, 128, 64, 64
    # gate: every weight 1.5*1 + 0 = 1.5 -> g = 1.5 * sum(x); up: 0.5*2 - 2 = -1 -> u = -sum(x)
    gate = _const_matrix(bits, I, H, G, 1, 0x3FC0, 0x0000)   # s=1.5, b=0
    up = _const_matrix(bits, I, H, G, 2, 0x3F00, 0xC000)     # s=0.5, b=-2
    rng = np.random.default_rng(12)
    down = qpack.random_matrix(rng, bits, H, I, G)
    rec = qpack.expert_record(bits, gate, up, down)
    x = np.zeros(H)
    x[[3, 70]] = [0.5, 0.25]  # sum = 0.75
    g, u, h, y = oracle.expert_ffn(bits, H, I, G, rec, x)
    assert np.all(g == 1.125) and np.all(u == -0.75)
    silu = torch.nn.functional.silu(torch.tensor(1.125, dtype=torch.float64)).item()
    np.testing.assert_allclose(h, silu * -0.75, rtol=1e-15)
    Wd = oracle.dequant(bits, H, I, G, qpack.record(bits, *down))
    np.testing.assert_allclose(y, Wd @ h, rtol=1e-12, atol=1e-14)


def test_zero_gate_gives_zero_output():
    bits, H, I, G = 2, 128, 64, 64
    rng = np.random.default_rng(13)
    zero = _const_matrix(bits, I, H, G, 0, 0x0000, 0x0000)
    rec = qpack.expert_record(bits, zero, qpack.random_matrix(rng, bits, I, H, G),
                              qpack.random_matrix(rng, bits, H, I, G))
    g, u, h, y = oracle.expert_ffn(bits, H, I, G, rec, rng.standard_normal(H))
    assert np.all(g == 0) and np.all(h == 0) and np.all(y == 0)


def test_combine_closed_form_and_permutation_invariance():
    H, k = 8, 4
    x = np.arange(H, dtype=np.float64)
    y = np.zeros((k + 1, H))
    for j in range(k + 1):
        y[j, j] = 10.0 * (j + 1)
    w = np.array([0.4, 0.3, 0.2, 0.1])
    out = oracle.combine(x, y, w, 0.5)
    expect = x.copy()
    expect[:4] += [4.0, 6.0, 6.0, 4.0]
    expect[4] += 25.0
    np.testing.assert_allclose(out, expect, rtol=1e-15)
    perm = [2, 0, 3, 1]
    yp = np.concatenate([y[perm], y[k:]])
    np.testing.assert_allclose(oracle.combine(x, yp, w[perm], 0.5), out, rtol=1e-15)


def test_rmsnorm_constant_vector_and_scale():
    for c in [1.0, -3.0, 1e-3]:
        out = oracle.rmsnorm(np.full(4096, c), 1e-6)
        np.testing.assert_allclose(out, c / np.sqrt(c * c + 1e-6), rtol=1e-12)
    rng = np.random.default_rng(14)
    x = rng.standard_normal(4096)
    np.testing.assert_allclose(oracle.rmsnorm(7.0 * x, 0.0), oracle.rmsnorm(x, 0.0), rtol=1e-13)
    assert np.sqrt(np.mean(oracle.rmsnorm(x, 0.0) ** 2)) == pytest.approx(1.0, rel=1e-14)


# --------------------------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------------------------

def _tiny_layer(rng, bits, H, I, G, E, zero_experts=False):
    experts = {}
    for e in range(E + 1):
        if zero_experts:
            mats = [_const_matrix(bits, I, H, G, 5, 0, 0), _const_matrix(bits, I, H, G, 5, 0, 0),
                    _const_matrix(bits, H, I, G, 5, 0, 0)]
        else:
            mats = [qpack.random_matrix(rng, bits, I, H, G), qpack.random_matrix(rng, bits, I, H, G),
                    qpack.random_matrix(rng, bits, H, I, G)]
        experts[e] = qpack.expert_record(bits, *mats)
    wr = (rng.standard_normal((E, H)) / 8).astype(np.float32)
    wsg = (rng.standard_normal(H) / 8).astype(np.float32)
    return experts, wr, wsg


def test_layer_with_zero_experts_returns_residual():
    rng = np.random.default_rng(15)
    H, I, G, E = 128, 64, 64, 8
    experts, wr, wsg = _tiny_layer(rng, 4, H, I, G, E, zero_experts=True)
    x = rng.standard_normal(H)
    res = oracle.layer(x, wr, wsg, experts.__getitem__, 4, 2, E, H, I, G)
    assert np.array_equal(res["out"], x)


def test_layer_composes_the_pinned_steps():
    rng = np.random.default_rng(16)
    H, I, G, E, k = 128, 64, 64, 8, 2
    experts, wr, wsg = _tiny_layer(rng, 4, H, I, G, E)
    x = rng.standard_normal(H)
    res = oracle.layer(x, wr, wsg, experts.__getitem__, 4, k, E, H, I, G, norm_input=True)
    xn = x / np.sqrt(np.mean(x * x) + 1e-6)
    np.testing.assert_allclose(res["xin"], xn, rtol=1e-14)
    logits = wr.astype(np.float64) @ xn
    order = np.lexsort((np.arange(E), -logits))[:k]
    assert res["ids"].tolist() == order.tolist()
    ys = []
    for e in list(order) + [E]:
        W = [oracle.dequant(4, I, H, G, experts[e][:oracle.matrix_bytes(4, I, H, G)]),
             oracle.dequant(4, I, H, G, experts[e][oracle.matrix_bytes(4, I, H, G):
                                                   2 * oracle.matrix_bytes(4, I, H, G)]),
             oracle.dequant(4, H, I, G, experts[e][2 * oracle.matrix_bytes(4, I, H, G):])]
        g, u = W[0] @ xn, W[1] @ xn
        h = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
        ys.append(W[2] @ h)
    p = scipy.special.softmax(logits)[order]
    p = p / p.sum()
    sg = scipy.special.expit(float(wsg.astype(np.float64) @ xn))
    expect = x + sum(p[j] * ys[j] for j in range(k)) + sg * ys[k]
    np.testing.assert_allclose(res["out"], expect, rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------------------------
# layer without a shared expert, and the layer stack (reading H11/H12: every layer consumes a
# unit-gain RMSNorm of its own input, the residual carries the un-normalised vector, and the
# stack passes each layer's raw output to the next)
# --------------------------------------------------------------------------------------------

def test_layer_without_shared_expert_is_zero_shared_expert():
    """shared_slot=None must equal a layer whose shared expert is all zeros (codes, scale and
    bias), whatever its gate, and the combine of the routed outputs with a zero row and gate."""
    rng = np.random.default_rng(21)
    H, I, G, E, k = 128, 64, 64, 8, 2
    experts, wr, wsg = _tiny_layer(rng, 4, H, I, G, E)
    zero = qpack.expert_record(4, _const_matrix(4, I, H, G, 0, 0, 0),
                               _const_matrix(4, I, H, G, 0, 0, 0),
                               _const_matrix(4, H, I, G, 0, 0, 0))
    with_zero = dict(experts)
    with_zero[E] = zero
    x = rng.standard_normal(H)
    for norm in (False, True):
        a = oracle.layer(x, wr, wsg, experts.__getitem__, 4, k, None, H, I, G, norm_input=norm)
        b = oracle.layer(x, wr, wsg, with_zero.__getitem__, 4, k, E, H, I, G, norm_input=norm)
        assert a["ids"].tolist() == b["ids"].tolist()
        assert np.array_equal(a["weights"], b["weights"])
        assert np.array_equal(b["y"][k], np.zeros(H)) and b["sg"] > 0.0
        assert np.array_equal(a["out"], b["out"])
        assert a["h"].shape == (k, I) and a["sg"] == 0.0
        routed = np.stack([oracle.expert_ffn(4, H, I, G, experts[int(e)], a["xin"])[3]
                           for e in a["ids"]] + [np.zeros(H)])
        assert np.array_equal(a["out"], oracle.combine(x, routed, a["weights"], 0.0))


def _stack(x, layers, **kw):
    H, I, G, E, k = 128, 64, 64, 8, 2
    return oracle.stack_token(x, layers, 4, k, E, H, I, G, **kw)


def test_stack_of_zero_layers_returns_its_input_exactly():
    """Zero experts add exactly nothing, so any depth returns the raw input bit for bit: the
    stack carries the un-normalised residual, not the normalised layer input."""
    rng = np.random.default_rng(22)
    H, I, G, E = 128, 64, 64, 8
    zl = []
    for _ in range(3):
        experts, wr, wsg = _tiny_layer(rng, 4, H, I, G, E, zero_experts=True)
        zl.append((wr, wsg, experts.__getitem__))
    x = 3.0 * rng.standard_normal(H)
    for depth in (1, 2, 3):
        trace = []
        out = _stack(x, zl[:depth], trace=trace)
        assert np.array_equal(out, x)
        assert len(trace) == depth
        for r in trace:  # each layer still normalised its own input before routing
            np.testing.assert_allclose(r["xin"], x / np.sqrt(np.mean(x * x) + 1e-6), rtol=1e-14)


def test_stack_composes_layers_on_raw_outputs():
    """A stack of distinct layers equals the pinned layer step applied in order, each on the
    previous layer's raw output with its own input norm; a zero layer anywhere is the
    identity."""
    rng = np.random.default_rng(23)
    H, I, G, E, k = 128, 64, 64, 8, 2
    mk = lambda zero=False: (lambda t: (t[1], t[2], t[0].__getitem__))(
        _tiny_layer(rng, 4, H, I, G, E, zero_experts=zero))
    n1, n2, n3, z = mk(), mk(), mk(), mk(True)
    x = rng.standard_normal(H)

    def by_hand(v, layers):
        for wr, wsg, get in layers:
            v = oracle.layer(v, wr, wsg, get, 4, k, E, H, I, G, norm_input=True)["out"]
        return v

    trace = []
    out = _stack(x, [n1, n2, n3], trace=trace)
    assert np.array_equal(out, by_hand(x, [n1, n2, n3]))
    assert np.array_equal(trace[1]["out"], by_hand(x, [n1, n2]))
    assert not np.array_equal(out, by_hand(x, [n3, n2, n1]))  # the order matters
    assert np.array_equal(_stack(x, [z, n1, z, n2]), _stack(x, [n1, n2]))


def test_stack_layer_sees_only_the_direction_of_its_input():
    """With eps = 0 a layer's experts see input / rms(input), so scaling the input of a
    one-layer stack by 4 (a power of two: the norm scales exactly) leaves the normalised input,
    the routing and every expert output bit for bit unchanged and only scales the residual:
    stack(4x) - 4x equals stack(x) - x up to the fp64 rounding of the residual add.  A stack
    that forgot the per-layer norm, or normalised the residual, fails this."""
    rng = np.random.default_rng(24)
    H, I, G, E = 128, 64, 64, 8
    experts, wr, wsg = _tiny_layer(rng, 4, H, I, G, E)
    n1 = (wr, wsg, experts.__getitem__)
    x = rng.standard_normal(H)
    t1, t4 = [], []
    a = _stack(x, [n1], eps=0.0, trace=t1) - x
    b = _stack(4.0 * x, [n1], eps=0.0, trace=t4) - 4.0 * x
    assert np.array_equal(t1[0]["xin"], t4[0]["xin"])
    assert t1[0]["ids"].tolist() == t4[0]["ids"].tolist()
    assert np.array_equal(t1[0]["y"], t4[0]["y"])
    assert np.max(np.abs(a)) > 0.1
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
