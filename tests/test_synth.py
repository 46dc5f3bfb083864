"""CPU checks of the seeded input generator (SplitMix64 counter streams, bf16 rounding,
distributions of the synthetic workloads)."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # published reference sequence of SplitMix64 started from state 1234567
    expect = [6457827717110365317, 3203168211198807973, 9817491932198370423,
              4593380528125082431, 16408922859458223821]
    assert [synth.draw(1234567, i) for i in range(5)] == expect


def test_bf16_round_to_nearest_even():
    one = 1.0
    assert synth.f64_to_bf16(one) == 0x3F80
    assert synth.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80           # tie -> even
    assert synth.f64_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82       # tie -> even (up)
    assert synth.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81  # above the tie
    assert synth.f64_to_bf16(0.02) == 0x3CA4
    assert synth.f64_to_bf16(-2.0) == 0xC000
    assert synth.f64_to_bf16(1.0 - 2 ** -9) == 0x3F80           # mantissa carry into exponent


def test_expert_record_composition_and_determinism():
    H, I, G = 256, 128, 64
    e1 = synth.expert(11, 3, 5, 4, H, I, G)
    e2 = synth.expert(11, 3, 5, 4, H, I, G)
    assert np.array_equal(e1, e2)
    mg = synth.matrix_bytes(4, I, H, G)
    gate = synth.matrix(11, 3, 5, synth.T_GATE_CODES, synth.T_GATE_SCALE, 4, I, H, G)
    down = synth.matrix(11, 3, 5, synth.T_DOWN_CODES, synth.T_DOWN_SCALE, 4, H, I, G)
    assert np.array_equal(e1[:mg], gate) and np.array_equal(e1[2 * mg:], down)
    assert not np.array_equal(synth.expert(11, 3, 6, 4, H, I, G), e1)
    assert not np.array_equal(synth.expert(11, 4, 5, 4, H, I, G), e1)


def _planes(rec, bits, R, C, G):
    nc = R * C * bits // 8
    nm = R * (C // G)
    codes = rec[:nc]
    s = rec[nc:nc + 2 * nm].view(np.uint16)
    b = rec[nc + 2 * nm:nc + 4 * nm].view(np.uint16)
    return codes, s, b


def _f(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def test_q4_distribution():
    rec = synth.matrix(1, 0, 0, synth.T_GATE_CODES, synth.T_GATE_SCALE, 4, 1024, 4096, 64)
    codes, s, b = _planes(rec, 4, 1024, 4096, 64)
    nib = np.concatenate([codes & 15, codes >> 4])
    hist = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(hist - 1 / 16) < 2e-3)
    sf = _f(s)
    ulp = 2.0 ** -8  # bf16 rounding of the interval ends
    assert sf.min() >= 0.01 * (1 - ulp) and sf.max() <= 0.03 * (1 + ulp)
    assert abs(sf.mean() - 0.02) < 1e-3
    assert np.array_equal(_f(b), -8.0 * sf)


def test_q2_distribution():
    rec = synth.matrix(1, 0, 0, synth.T_DOWN_CODES, synth.T_DOWN_SCALE, 2, 4096, 1024, 64)
    codes, s, b = _planes(rec, 2, 4096, 1024, 64)
    crumbs = np.concatenate([(codes >> (2 * j)) & 3 for j in range(4)])
    hist = np.bincount(crumbs, minlength=4) / crumbs.size
    assert np.all(np.abs(hist - 0.25) < 2e-3)
    sf = _f(s)
    ulp = 2.0 ** -8
    assert sf.min() >= 0.02 * (1 - ulp) and sf.max() <= 0.06 * (1 + ulp)
    assert abs(sf.mean() - 0.04) < 2e-3
    # bias = -1.5 s rounded to bf16 (nearest even); -1.5 s itself is exact in fp32
    t = (-1.5 * sf).astype(np.float32).view(np.uint32)
    rne = ((t + 0x7FFF + ((t >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(b, rne)
    assert np.all(np.abs(_f(b) / (-1.5 * sf) - 1) <= 2.0 ** -8)
    # the four codes sit symmetric about zero: dequantized weights have mean ~0
    assert abs(1.5 + float(np.mean(_f(b) / sf))) < 1e-2


def test_normals():
    x = synth.activations(3, 0)
    assert x.dtype == np.float32 and x.size == 4096
    assert abs(x.mean()) < 0.06 and abs(x.std() - 1.0) < 0.05
    w = synth.router_weights(3, 1)
    assert w.shape == (512, 4096) and abs(w.std() - 0.125) < 1e-3
    assert not np.array_equal(synth.activations(3, 1), x)
