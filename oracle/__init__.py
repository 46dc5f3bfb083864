"""Plain fp64 CPU oracle for the group-quantized MoE FFN block -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It never imports the GPU library and shares no code with it.  The arithmetic lives
in ``moe_oracle.c`` (plain loops, fp64); this module marshals numpy arrays and composes the steps
of one MoE layer in the order the pages give them:

* router logits, softmax, top-k, renormalised weights (Flash-MoE wiki summary,
  jeongsk-2ndbrain.pages.dev, "Per-layer pipeline": routing logits on the GPU, softmax + top-K on
  the CPU);
* per selected expert and the shared expert: gate/up dequant matvec, SwiGLU, down matvec
  (a2a-mcp.org "What is Flash-MoE", deep dives 2 and 3);
* combine + residual + sigmoid-gated shared expert (same page, deep dive 3);
* for the layer stack, a unit-gain RMSNorm of each layer's input (deep dive 3, two-pass RMSNorm;
  wiki "Per-layer pipeline": CMD3 = expert forward + combine + norm);
* the GatedDeltaNet state update of the linear-attention layers (``gdn_step``, numpy fp64; wiki
  technique 4, "Accelerate BLAS linear attention").

Every function is pinned by the CPU tests (closed forms, hand-derived fixtures under
``tests/golden/``, invariants, exact rational arithmetic).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Callable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> None:
    """Compile liboracle.so with gcc (fp64, OpenMP over output rows)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
           os.path.join(_HERE, "moe_oracle.c"), "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=_HERE)


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        i32, i64, f64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.orc_matrix_bytes.argtypes = [i32, i32, i32, i32]
        lib.orc_matrix_bytes.restype = i64
        lib.orc_expert_bytes.argtypes = [i32, i32, i32, i32]
        lib.orc_expert_bytes.restype = i64
        for name in ("orc_qmatvec", "orc_qmatvec_fma_form", "orc_qmatvec_xsum_form"):
            getattr(lib, name).argtypes = [i32, i32, i32, i32, vp, vp, vp]
        lib.orc_dequant.argtypes = [i32, i32, i32, i32, vp, vp]
        lib.orc_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        lib.orc_router_logits.argtypes = [i32, i32, vp, vp, vp]
        lib.orc_softmax.argtypes = [i32, vp, vp]
        lib.orc_topk.argtypes = [i32, i32, vp, vp, vp]
        lib.orc_shared_gate.argtypes = [i32, vp, vp]
        lib.orc_shared_gate.restype = f64
        lib.orc_combine.argtypes = [i32, i32, vp, vp, vp, f64, vp]
        lib.orc_rmsnorm.argtypes = [i32, f64, vp, vp]
        lib.orc_set_num_threads.argtypes = [i32]
        lib.orc_set_num_threads.restype = None
        lib.orc_max_threads.restype = i32
        _lib = lib
    return _lib


def set_num_threads(n: int) -> None:
    """OpenMP threads of the row loops (results do not depend on it)."""
    _L().orc_set_num_threads(int(n))


def max_threads() -> int:
    return int(_L().orc_max_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint8)


def matrix_bytes(bits: int, rows: int, cols: int, group: int) -> int:
    return int(_L().orc_matrix_bytes(bits, rows, cols, group))


def expert_bytes(bits: int, hidden: int, inter: int, group: int) -> int:
    return int(_L().orc_expert_bytes(bits, hidden, inter, group))


def dequant(bits: int, rows: int, cols: int, group: int, rec) -> np.ndarray:
    rec = _u8(rec)
    assert rec.size >= matrix_bytes(bits, rows, cols, group)
    W = np.empty((rows, cols), dtype=np.float64)
    _L().orc_dequant(bits, rows, cols, group, rec.ctypes.data, W.ctypes.data)
    return W


def _matvec(fn, bits, rows, cols, group, rec, x):
    rec, x = _u8(rec), _f64(x)
    assert rec.size >= matrix_bytes(bits, rows, cols, group) and x.size == cols
    y = np.empty(rows, dtype=np.float64)
    fn(bits, rows, cols, group, rec.ctypes.data, x.ctypes.data, y.ctypes.data)
    return y


def qmatvec(bits, rows, cols, group, rec, x) -> np.ndarray:
    """Naive dequantize-then-dot."""
    return _matvec(_L().orc_qmatvec, bits, rows, cols, group, rec, x)


def qmatvec_fma_form(bits, rows, cols, group, rec, x) -> np.ndarray:
    return _matvec(_L().orc_qmatvec_fma_form, bits, rows, cols, group, rec, x)


def qmatvec_xsum_form(bits, rows, cols, group, rec, x) -> np.ndarray:
    return _matvec(_L().orc_qmatvec_xsum_form, bits, rows, cols, group, rec, x)


def expert_ffn(bits: int, hidden: int, inter: int, group: int, expert, x):
    """Returns (g, u, h, y) of one expert FFN with SwiGLU."""
    expert, x = _u8(expert), _f64(x)
    assert expert.size >= expert_bytes(bits, hidden, inter, group) and x.size == hidden
    g = np.empty(inter)
    u = np.empty(inter)
    h = np.empty(inter)
    y = np.empty(hidden)
    _L().orc_expert_ffn(bits, hidden, inter, group, expert.ctypes.data, x.ctypes.data,
                        g.ctypes.data, u.ctypes.data, h.ctypes.data, y.ctypes.data)
    return g, u, h, y


def router_logits(w_router, x) -> np.ndarray:
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    x = _f64(x)
    E, H = w.shape
    assert x.size == H
    out = np.empty(E)
    _L().orc_router_logits(E, H, w.ctypes.data, x.ctypes.data, out.ctypes.data)
    return out


def softmax(logits) -> np.ndarray:
    l = _f64(logits)
    p = np.empty_like(l)
    _L().orc_softmax(l.size, l.ctypes.data, p.ctypes.data)
    return p


def topk(logits, k: int):
    """(ids int32[k], weights fp64[k]) in descending-logit order, ties to the lower index."""
    l = _f64(logits)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k)
    _L().orc_topk(l.size, k, l.ctypes.data, ids.ctypes.data, w.ctypes.data)
    return ids, w


def shared_gate(w_sg, x) -> float:
    w = np.ascontiguousarray(w_sg, dtype=np.float32)
    x = _f64(x)
    return float(_L().orc_shared_gate(x.size, w.ctypes.data, x.ctypes.data))


def combine(residual, y, weights, sg: float) -> np.ndarray:
    """out = residual + sum_j w_j y_j + sg * y[k]; y is [k+1][H] with the shared row last."""
    r = _f64(residual)
    y = _f64(y)
    w = _f64(weights)
    k = w.size
    assert y.shape == (k + 1, r.size)
    out = np.empty_like(r)
    _L().orc_combine(r.size, k, r.ctypes.data, y.ctypes.data, w.ctypes.data, float(sg),
                     out.ctypes.data)
    return out


def rmsnorm(x, eps: float) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    _L().orc_rmsnorm(x.size, float(eps), x.ctypes.data, out.ctypes.data)
    return out


def gdn_step(state, q, k, v, alpha, beta):
    """One decode step of the gated delta rule, per head, in fp64 (numpy, no C part).

    The Flash-MoE wiki (jeongsk-2ndbrain.pages.dev, technique 4, "Accelerate BLAS linear attention") runs the
    GatedDeltaNet recurrence of 64 heads with 128x128 state each as a scale, a matrix-vector
    product and a rank-one update per head.  The pages print no formula; the reading taken is the
    published gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", 2024) in its
    one-token form, whose steps are exactly those three calls, followed by the read-out:
        S <- alpha * S                  (decay gate)
        u  = S k                        (what the state currently recalls for key k)
        S <- S + beta * (v - u) k^T     (delta-rule correction toward v)
        o  = S q                        (read-out with the query)
    state [n_heads][dv][dk]; q, k [n_heads][dk]; v [n_heads][dv]; alpha, beta [n_heads].
    Returns (new state, o [n_heads][dv]); the inputs are not modified.
    """
    S = _f64(state).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha).reshape(-1), _f64(beta).reshape(-1)
    nh, dv, dk = S.shape
    assert q.shape == (nh, dk) and k.shape == (nh, dk) and v.shape == (nh, dv)
    o = np.empty((nh, dv))
    for h in range(nh):
        S[h] *= alpha[h]
        u = S[h] @ k[h]
        S[h] += beta[h] * np.outer(v[h] - u, k[h])
        o[h] = S[h] @ q[h]
    return S, o


def layer(x, w_router, w_sg, get_expert: Callable[[int], np.ndarray], bits: int, k: int,
          shared_slot: int, hidden: int, inter: int, group: int, norm_input: bool = False,
          eps: float = 1e-6) -> dict:
    """One MoE layer for one token.

    ``get_expert(slot)`` returns the canonical record of an expert slot; ``shared_slot`` None means
    the layer has no shared expert.  With ``norm_input`` the
    router and the experts see RMSNorm(x) while the residual stays x (layer-stack reading); without
    it they see x itself.  ``w_sg`` None means the shared expert enters with weight 1.
    """
    x = _f64(x)
    xin = rmsnorm(x, eps) if norm_input else x
    logits = router_logits(w_router, xin)
    ids, w = topk(logits, k)
    sg = shared_gate(w_sg, xin) if w_sg is not None else 1.0
    ys = []
    hs = []
    slots = list(ids) + ([shared_slot] if shared_slot is not None else [])
    for e in slots:
        _, _, h, y = expert_ffn(bits, hidden, inter, group, get_expert(int(e)), xin)
        ys.append(y)
        hs.append(h)
    if shared_slot is None:  # no shared expert: its row and gate are zero
        ys.append(np.zeros(hidden))
        sg = 0.0
    Y = np.stack(ys)
    out = combine(x, Y, w, sg)
    return dict(logits=logits, ids=ids, weights=w, sg=sg, h=np.stack(hs), y=Y, out=out,
                xin=xin)


def stack_token(x0, layers: Sequence, bits: int, k: int, shared_slot: int, hidden: int,
                inter: int, group: int, eps: float = 1e-6, trace: Optional[list] = None):
    """Decode one token through a stack of layers.

    ``layers[L]`` is a tuple ``(w_router, w_sg, get_expert)``.  Each layer consumes RMSNorm of its
    input, and adds its MoE output to the un-normalised input.  Returns the stack output.
    """
    x = _f64(x0)
    for L, (wr, wsg, get) in enumerate(layers):
        res = layer(x, wr, wsg, get, bits, k, shared_slot, hidden, inter, group, norm_input=True,
                    eps=eps)
        if trace is not None:
            trace.append(res)
        x = res["out"]
    return x
