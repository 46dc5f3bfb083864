"""Seeded synthetic inputs for the MoE decode/prefill workloads (test and bench input only).

The draw definitions live in ``synth.h``; ``libsynth_cpu.so`` (gcc) writes them on the host and
``libsynth_gpu.so`` (hipcc, gfx950) writes the same bytes in device memory.  Nothing here computes
any part of the MoE layer: this module only produces codes, bf16 scales/biases and fp32 normals.

Workload distributions (q4 / q2 experts, N(0,1) activations, N(0,1/64) router and shared-gate
weights) follow the benchmark configurations: q4 codes uniform 0..15 with scale ~ U(0.01, 0.03)
and bias = -8*scale; q2 codes uniform 0..3 with scale ~ U(0.02, 0.06) and bias = bf16(-1.5*scale)
(codes symmetric about zero; with -2*scale every q2 weight has mean -scale/2, and a stack of such
layers drives the SwiGLU into saturation after one layer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

# tensor ids inside a stream key (mirror of synth.h)
T_GATE_CODES, T_GATE_SCALE, T_UP_CODES, T_UP_SCALE, T_DOWN_CODES, T_DOWN_SCALE = range(6)
T_ROUTER = 16
T_SHARED_GATE = 17
T_X = 32

# per-bit-width code distribution: (scale lo, scale hi, zero point)
QPARAMS = {4: (0.01, 0.03, 8.0), 2: (0.02, 0.06, 1.5)}

# model shape of the benchmark workloads
HIDDEN, INTER, GROUP, N_EXPERTS, TOP_K = 4096, 1024, 64, 512, 4
SHARED_SLOT = N_EXPERTS  # slot 512 holds the always-on shared expert
ROUTER_SIGMA = 0.125      # N(0, 1/64)


def build(verbose: bool = False) -> None:
    """Compile libsynth_cpu.so (gcc) and libsynth_gpu.so (hipcc, gfx950)."""
    cpu = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
           os.path.join(_HERE, "synth_cpu.c"), "-o", CPU_LIB, "-lm"]
    gpu = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth_gpu.hip"), "-o", GPU_LIB]
    for cmd in (cpu, gpu):
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True, cwd=_HERE,
                       stdout=None if verbose else subprocess.DEVNULL,
                       stderr=subprocess.STDOUT if not verbose else None)


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            raise RuntimeError(f"{CPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(CPU_LIB)
        u64, i32, f64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_fill_matrix.argtypes = [vp, u64, i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                          f64, f64]
        lib.synth_fill_expert.argtypes = [vp, u64, i32, i32, i32, i32, i32, i32, f64, f64, f64]
        lib.synth_fill_normal.argtypes = [vp, u64, u64, i32, i32, i32, f64]
        lib.synth_expert_nbytes.argtypes = [i32, i32, i32, i32]
        lib.synth_expert_nbytes.restype = u64
        lib.synth_key_export.argtypes = [u64, u64, u64, u64]
        lib.synth_key_export.restype = u64
        lib.synth_draw_export.argtypes = [u64, u64]
        lib.synth_draw_export.restype = u64
        lib.synth_f64_to_bf16_export.argtypes = [f64]
        lib.synth_f64_to_bf16_export.restype = ctypes.c_uint16
        _cpu = lib
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        u64, i32, f64, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_gpu_fill_experts.argtypes = [vp, u64, i32, i32, u64, i32, i32, i32, i32, i32,
                                               f64, f64, f64, vp]
        lib.synth_gpu_fill_experts.restype = i32
        _gpu = lib
    return _gpu


def matrix_bytes(bits: int, rows: int, cols: int, group: int) -> int:
    return rows * cols * bits // 8 + 4 * rows * (cols // group)


def expert_bytes(bits: int, hidden: int = HIDDEN, inter: int = INTER, group: int = GROUP) -> int:
    return int(_cpu_lib().synth_expert_nbytes(bits, hidden, inter, group))


def key(seed: int, layer: int, slot: int, tensor: int) -> int:
    return int(_cpu_lib().synth_key_export(seed, layer, slot, tensor))


def draw(k: int, i: int) -> int:
    return int(_cpu_lib().synth_draw_export(k, i))


def f64_to_bf16(v: float) -> int:
    return int(_cpu_lib().synth_f64_to_bf16_export(v))


def expert(seed: int, layer: int, slot: int, bits: int, hidden: int = HIDDEN,
           inter: int = INTER, group: int = GROUP) -> np.ndarray:
    """One canonical expert record (gate | up | down) as uint8."""
    lo, hi, zp = QPARAMS[bits]
    out = np.empty(expert_bytes(bits, hidden, inter, group), dtype=np.uint8)
    _cpu_lib().synth_fill_expert(out.ctypes.data, seed, layer, slot, bits, hidden, inter, group,
                                 lo, hi, zp)
    return out


def matrix(seed: int, layer: int, slot: int, codes_tensor: int, scale_tensor: int, bits: int,
           rows: int, cols: int, group: int) -> np.ndarray:
    """One canonical [rows x cols] matrix record (codes | scale | bias) as uint8."""
    lo, hi, zp = QPARAMS[bits]
    out = np.empty(matrix_bytes(bits, rows, cols, group), dtype=np.uint8)
    _cpu_lib().synth_fill_matrix(out.ctypes.data, seed, layer, slot, codes_tensor, scale_tensor,
                                 bits, rows, cols, group, lo, hi, zp)
    return out


def normal(n: int, seed: int, layer: int, slot: int, tensor: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _cpu_lib().synth_fill_normal(out.ctypes.data, n, seed, layer, slot, tensor, sigma)
    return out


def router_weights(seed: int, layer: int, n_experts: int = N_EXPERTS,
                   hidden: int = HIDDEN) -> np.ndarray:
    """Router W fp32 [E][H] ~ N(0, 1/64)."""
    return normal(n_experts * hidden, seed, layer, 0, T_ROUTER, ROUTER_SIGMA).reshape(
        n_experts, hidden)


def shared_gate_weights(seed: int, layer: int, hidden: int = HIDDEN) -> np.ndarray:
    """Shared-expert gate vector fp32 [H] ~ N(0, 1/64)."""
    return normal(hidden, seed, layer, 0, T_SHARED_GATE, ROUTER_SIGMA)


def activations(seed: int, token: int, hidden: int = HIDDEN) -> np.ndarray:
    """Token activation fp32 [H] ~ N(0, 1)."""
    return normal(hidden, seed, token, 0, T_X, 1.0)


def gpu_fill_experts(base_ptr: int, slot_bytes: int, slot0: int, nslots: int, seed: int,
                     layer: int, bits: int, hidden: int = HIDDEN, inter: int = INTER,
                     group: int = GROUP, stream: int = 0) -> None:
    """Fill device slots [slot0, slot0+nslots) of one layer with the same bytes expert() writes."""
    lo, hi, zp = QPARAMS[bits]
    rc = _gpu_lib().synth_gpu_fill_experts(base_ptr, slot_bytes, slot0, nslots, seed, layer, bits,
                                           hidden, inter, group, lo, hi, zp, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_experts failed with code {rc}")
