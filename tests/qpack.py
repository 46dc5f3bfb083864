"""Test-side helpers that build canonical quantized records from explicit integer codes.

The canonical record of an [R x C] matrix is codes | scale bf16 [R][C/G] | bias bf16 [R][C/G]; q4
keeps element c in byte c/2 (even c in the low nibble), q2 keeps element c at bits 2*(c%4) of byte
c/4.  These helpers write that layout from numpy arrays so tests can craft inputs with known
values.  They contain no MoE arithmetic.
"""
import numpy as np


def pack_codes(bits: int, Q: np.ndarray) -> np.ndarray:
    Q = np.asarray(Q, dtype=np.uint8)
    R, C = Q.shape
    if bits == 4:
        assert Q.max(initial=0) < 16
        return (Q[:, 0::2] | (Q[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    assert bits == 2 and Q.max(initial=0) < 4
    return (Q[:, 0::4] | (Q[:, 1::4] << 2) | (Q[:, 2::4] << 4) | (Q[:, 3::4] << 6)).astype(
        np.uint8).reshape(-1)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Exact conversion: the inputs must already be bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def random_bf16(rng, shape, lo: float, hi: float, signed: bool = False) -> np.ndarray:
    """bf16 bit patterns of values uniform in magnitude [lo, hi) (rounded down to bf16)."""
    v = rng.uniform(lo, hi, size=shape).astype(np.float32)
    if signed:
        v *= rng.choice([-1.0, 1.0], size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def record(bits: int, Q, s_bits, b_bits) -> np.ndarray:
    """Canonical matrix record from codes Q [R][C] and bf16 bit planes [R][C/G]."""
    codes = pack_codes(bits, Q)
    s = np.ascontiguousarray(s_bits, dtype=np.uint16).reshape(-1)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16).reshape(-1)
    return np.concatenate([codes, s.view(np.uint8), b.view(np.uint8)])


def expert_record(bits, gate, up, down) -> np.ndarray:
    """gate/up/down are (Q, s_bits, b_bits) triples."""
    return np.concatenate([record(bits, *gate), record(bits, *up), record(bits, *down)])


def random_matrix(rng, bits: int, R: int, C: int, G: int):
    """Random codes and bf16 scale/bias planes of the benchmark distributions."""
    Q = rng.integers(0, 1 << bits, size=(R, C), dtype=np.uint8)
    s = random_bf16(rng, (R, C // G), 0.01, 0.03)
    zp = 8 if bits == 4 else 2
    b = f32_to_bf16_bits(-zp * bf16_bits_to_f64(s).astype(np.float32))
    return Q, s, b
