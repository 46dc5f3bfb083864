"""Python binding of libmoe, the MI355X (gfx950) group-quantized MoE FFN hot path.

Thin ctypes marshalling over the C ABI declared in ``include/moe.h``: every function here has
the name of the C entry point, converts tensors to device pointers and the stream to a handle,
calls the library and raises :class:`MoeError` on a non-zero status.  All computation runs in
the HIP kernels of ``libmoe.so``; there is no fallback path.  PyTorch only provides device
memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_E_NULL, MOE_E_SHAPE, MOE_E_ALIGN, MOE_E_BITS, MOE_E_WORKSPACE, MOE_E_HIP = range(7)

EXPORTS = [
    "moe_status_string", "moe_version", "moe_router_workspace_bytes", "moe_router_topk",
    "moe_expert_ffn_q4", "moe_expert_ffn_q2", "moe_combine", "moe_layer_workspace_bytes",
    "moe_layer_decode", "moe_stack_workspace_bytes", "moe_decode_stack",
    "moe_prefill_workspace_bytes", "moe_prefill_q4", "moe_qgemv", "moe_rmsnorm", "moe_pack",
    "moe_set_stack_mode", "moe_pack_router", "moe_gdn_step",
]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class MoeExperts(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("bits", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("slot_bytes", ctypes.c_int64),
                ("dev_err", ctypes.c_void_p)]


class MoeQMatrix(ctypes.Structure):
    _fields_ = [("rec", ctypes.c_void_p), ("bits", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("group", ctypes.c_int32)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("experts", MoeExperts), ("w_router", ctypes.c_void_p),
                ("w_sg", ctypes.c_void_p), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("shared_slot", ctypes.c_int32),
                ("w_router_cb", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libmoe.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        P = ctypes.POINTER
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_version.restype = ctypes.c_char_p
        L.moe_router_workspace_bytes.argtypes = [i32, i32]
        L.moe_router_workspace_bytes.restype = sz
        L.moe_router_topk.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, sz, vp]
        for n in ("moe_expert_ffn_q4", "moe_expert_ffn_q2"):
            getattr(L, n).argtypes = [P(MoeExperts), vp, vp, i32, vp, vp, vp]
        L.moe_combine.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, i32, vp]
        L.moe_layer_workspace_bytes.argtypes = [P(MoeLayer)]
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_decode.argtypes = [P(MoeLayer), vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_stack_workspace_bytes.argtypes = [P(MoeLayer), i32]
        L.moe_stack_workspace_bytes.restype = sz
        L.moe_decode_stack.argtypes = [P(MoeLayer), i32, vp, vp, vp, f32, vp, vp, sz, vp]
        L.moe_set_stack_mode.argtypes = [i32]
        L.moe_set_stack_mode.restype = None
        L.moe_prefill_workspace_bytes.argtypes = [P(MoeLayer), i32]
        L.moe_prefill_workspace_bytes.restype = sz
        L.moe_prefill_q4.argtypes = [P(MoeLayer), vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_qgemv.argtypes = [P(MoeQMatrix), vp, vp, vp]
        L.moe_rmsnorm.argtypes = [vp, i32, i32, f32, vp, vp]
        L.moe_gdn_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
        L.moe_pack.argtypes = [vp, i32, i32, P(MoeExperts), vp]
        L.moe_pack_router.argtypes = [vp, i32, i32, vp, vp]
        for n in EXPORTS:
            if getattr(L, n).restype is ctypes.c_int or n in (
                    "moe_router_topk", "moe_expert_ffn_q4", "moe_expert_ffn_q2", "moe_combine",
                    "moe_layer_decode", "moe_decode_stack", "moe_prefill_q4", "moe_qgemv",
                    "moe_rmsnorm", "moe_pack", "moe_pack_router", "moe_gdn_step"):
                getattr(L, n).restype = i32
        _lib = L
    return _lib


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _ptr(t) -> int | None:
    """Device pointer of a tensor (or an int address); None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != MOE_OK:
        raise MoeError(fn, st, lib().moe_status_string(st).decode())


def status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def version() -> str:
    return lib().moe_version().decode()


def experts(base, bits: int, hidden: int, inter: int, n_slots: int, slot_bytes: int,
            group: int = 64, dev_err=None) -> MoeExperts:
    return MoeExperts(_ptr(base), bits, hidden, inter, group, n_slots, slot_bytes, _ptr(dev_err))


def layer(experts_desc: MoeExperts, w_router, w_sg, n_experts: int, top_k: int,
          shared_slot: int, w_router_cb=None) -> MoeLayer:
    return MoeLayer(experts_desc, _ptr(w_router), _ptr(w_sg), n_experts, top_k, shared_slot,
                    _ptr(w_router_cb))


def qmatrix(rec, bits: int, rows: int, cols: int, group: int = 64) -> MoeQMatrix:
    return MoeQMatrix(_ptr(rec), bits, rows, cols, group)


# ---------------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------------

def moe_router_workspace_bytes(T: int, E: int) -> int:
    return int(lib().moe_router_workspace_bytes(T, E))


def moe_router_topk(x, T, w_router, w_sg, H, E, k, ids, ld_ids, weights, shared_gate, ws,
                    ws_bytes, stream=None) -> None:
    _check("moe_router_topk", lib().moe_router_topk(
        _ptr(x), T, _ptr(w_router), _ptr(w_sg), H, E, k, _ptr(ids), ld_ids, _ptr(weights),
        _ptr(shared_gate), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn_q4(w: MoeExperts, x, ids, n, y, h, stream=None) -> None:
    _check("moe_expert_ffn_q4", lib().moe_expert_ffn_q4(
        ctypes.byref(w), _ptr(x), _ptr(ids), n, _ptr(y), _ptr(h), _stream(stream)))


def moe_expert_ffn_q2(w: MoeExperts, x, ids, n, y, h, stream=None) -> None:
    _check("moe_expert_ffn_q2", lib().moe_expert_ffn_q2(
        ctypes.byref(w), _ptr(x), _ptr(ids), n, _ptr(y), _ptr(h), _stream(stream)))


def moe_combine(residual, y, weights, k, shared_gate, out, out_norm, eps, H, stream=None) -> None:
    _check("moe_combine", lib().moe_combine(
        _ptr(residual), _ptr(y), _ptr(weights), k, _ptr(shared_gate), _ptr(out), _ptr(out_norm),
        eps, H, _stream(stream)))


def moe_layer_workspace_bytes(L: MoeLayer) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(L)))


def moe_layer_decode(L: MoeLayer, x, norm_input, eps, out, ids_out, weights_out, sg_out, ws,
                     ws_bytes, stream=None) -> None:
    _check("moe_layer_decode", lib().moe_layer_decode(
        ctypes.byref(L), _ptr(x), int(norm_input), eps, _ptr(out), _ptr(ids_out),
        _ptr(weights_out), _ptr(sg_out), _ptr(ws), ws_bytes, _stream(stream)))


def _layer_array(layers):
    arr = (MoeLayer * len(layers))(*layers)
    return arr


def moe_stack_workspace_bytes(layers) -> int:
    arr = _layer_array(layers)
    return int(lib().moe_stack_workspace_bytes(arr, len(layers)))


def moe_decode_stack(layers, x_in, x_out, xn_out, eps, ids_trace, ws, ws_bytes,
                     stream=None) -> None:
    arr = layers if isinstance(layers, ctypes.Array) else _layer_array(layers)
    _check("moe_decode_stack", lib().moe_decode_stack(
        arr, len(arr), _ptr(x_in), _ptr(x_out), _ptr(xn_out), eps, _ptr(ids_trace), _ptr(ws),
        ws_bytes, _stream(stream)))


STACK_AUTO, STACK_KERNELS, STACK_PERSISTENT = 0, 1, 2


def moe_set_stack_mode(mode: int) -> None:
    """Process-wide moe_decode_stack execution: STACK_AUTO, STACK_KERNELS or STACK_PERSISTENT."""
    lib().moe_set_stack_mode(int(mode))


def moe_prefill_workspace_bytes(L: MoeLayer, T: int) -> int:
    return int(lib().moe_prefill_workspace_bytes(ctypes.byref(L), T))


def moe_prefill_q4(L: MoeLayer, x, T, out, ids_out, weights_out, sg_out, ws, ws_bytes,
                   stream=None) -> None:
    _check("moe_prefill_q4", lib().moe_prefill_q4(
        ctypes.byref(L), _ptr(x), T, _ptr(out), _ptr(ids_out), _ptr(weights_out), _ptr(sg_out),
        _ptr(ws), ws_bytes, _stream(stream)))


def moe_pack_router(w_router, n_experts: int, hidden: int, dst, stream=None) -> None:
    _check("moe_pack_router", lib().moe_pack_router(_ptr(w_router), n_experts, hidden, _ptr(dst),
                                                    _stream(stream)))


def moe_qgemv(m: MoeQMatrix, x, y, stream=None) -> None:
    _check("moe_qgemv", lib().moe_qgemv(ctypes.byref(m), _ptr(x), _ptr(y), _stream(stream)))


def moe_rmsnorm(x, T: int, H: int, eps: float, out, stream=None) -> None:
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(x), T, H, eps, _ptr(out), _stream(stream)))


def moe_gdn_step(state, q, k, v, alpha, beta, n_heads: int, dk: int, dv: int, out,
                 stream=None) -> None:
    _check("moe_gdn_step", lib().moe_gdn_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                              _ptr(beta), n_heads, dk, dv, _ptr(out),
                                              _stream(stream)))


def moe_pack(canonical, n, slot0, dst: MoeExperts, stream=None) -> None:
    _check("moe_pack", lib().moe_pack(_ptr(canonical), n, slot0, ctypes.byref(dst),
                                      _stream(stream)))
