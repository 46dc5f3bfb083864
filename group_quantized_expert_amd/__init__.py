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
    "moe_pack_router", "moe_gdn_step", "moe_decode_stack_static",
    "moe_layer_batch_workspace_bytes", "moe_layer_decode_batch",
    "moe_stack_batch_workspace_bytes", "moe_decode_stack_batch",
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
        L.moe_decode_stack.argtypes = [P(MoeLayer), i32, vp, vp, vp, f32, vp, i32, vp, sz, vp]
        L.moe_decode_stack_static.argtypes = [P(MoeLayer), i32, vp, vp, vp, f32, vp, i32, vp]
        L.moe_layer_batch_workspace_bytes.argtypes = [P(MoeLayer), i32]
        L.moe_layer_batch_workspace_bytes.restype = sz
        L.moe_layer_decode_batch.argtypes = [P(MoeLayer), vp, i32, i32, f32, vp, vp, vp, vp, vp,
                                             sz, vp]
        L.moe_stack_batch_workspace_bytes.argtypes = [P(MoeLayer), i32, i32]
        L.moe_stack_batch_workspace_bytes.restype = sz
        L.moe_decode_stack_batch.argtypes = [P(MoeLayer), i32, vp, i32, vp, vp, f32, vp, vp, sz,
                                             vp]
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
                    "moe_rmsnorm", "moe_pack", "moe_pack_router", "moe_gdn_step",
                    "moe_decode_stack_static", "moe_layer_decode_batch",
                    "moe_decode_stack_batch"):
                getattr(L, n).restype = i32
        _lib = L
    return _lib


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _ptr(t, name: str = "tensor", dtype=None, numel: int = 0):
    """Device pointer of a tensor argument, after checking that the kernels can use it.

    A torch tensor must live on a GPU, be contiguous, have ``dtype`` (when given) and hold at
    least ``numel`` elements: the kernels index it as a dense array of that type and size, so
    anything else would make them read or write outside the allocation.  ``None`` passes NULL
    (the library decides whether NULL is allowed).  A plain int is taken as a raw device
    address and cannot be checked."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: expected a GPU tensor, got {type(t).__name__} on "
                         f"{getattr(t, 'device', '?')}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _f32(t, name, numel):
    import torch
    return _ptr(t, name, torch.float32, numel)


def _i32(t, name, numel):
    import torch
    return _ptr(t, name, torch.int32, numel)


def _u8(t, name, numel):
    import torch
    return _ptr(t, name, torch.uint8, numel)


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


def _matrix_bytes(bits: int, rows: int, cols: int, group: int = 64) -> int:
    return rows * cols * bits // 8 + 4 * rows * (cols // group)


def _expert_bytes(bits: int, hidden: int, inter: int, group: int = 64) -> int:
    return 2 * _matrix_bytes(bits, inter, hidden, group) + _matrix_bytes(bits, hidden, inter, group)


def experts(base, bits: int, hidden: int, inter: int, n_slots: int, slot_bytes: int,
            group: int = 64, dev_err=None) -> MoeExperts:
    """Descriptor of n_slots resident expert records (uint8 device buffer of n_slots *
    slot_bytes bytes; the last slot needs only its record).  The tensors must outlive every
    call that uses the descriptor."""
    last = (n_slots - 1) * slot_bytes + _expert_bytes(bits, hidden, inter, group) if n_slots > 0 else 0
    return MoeExperts(_u8(base, "experts.base", last), bits, hidden, inter, group, n_slots,
                      slot_bytes, _i32(dev_err, "experts.dev_err", 1))


def layer(experts_desc: MoeExperts, w_router, w_sg, n_experts: int, top_k: int,
          shared_slot: int, w_router_cb=None) -> MoeLayer:
    H = experts_desc.hidden
    return MoeLayer(experts_desc, _f32(w_router, "w_router", n_experts * H),
                    _f32(w_sg, "w_sg", H), n_experts, top_k, shared_slot,
                    _f32(w_router_cb, "w_router_cb", n_experts * H))


def qmatrix(rec, bits: int, rows: int, cols: int, group: int = 64) -> MoeQMatrix:
    return MoeQMatrix(_u8(rec, "rec", _matrix_bytes(bits, rows, cols, group)), bits, rows, cols,
                      group)


# ---------------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------------

def moe_router_workspace_bytes(T: int, E: int) -> int:
    return int(lib().moe_router_workspace_bytes(T, E))


def moe_router_topk(x, T, w_router, w_sg, H, E, k, ids, ld_ids, weights, shared_gate, ws,
                    ws_bytes, stream=None) -> None:
    _check("moe_router_topk", lib().moe_router_topk(
        _f32(x, "x", T * H), T, _f32(w_router, "w_router", E * H), _f32(w_sg, "w_sg", H), H, E,
        k, _i32(ids, "ids", (T - 1) * ld_ids + k), ld_ids, _f32(weights, "weights", T * k),
        _f32(shared_gate, "shared_gate", T), _u8(ws, "ws", ws_bytes), ws_bytes, _stream(stream)))


def _expert_ffn(fn: str, w: MoeExperts, x, ids, n, y, h, stream) -> None:
    _check(fn, getattr(lib(), fn)(
        ctypes.byref(w), _f32(x, "x", w.hidden), _i32(ids, "ids", n), n,
        _f32(y, "y", n * w.hidden), _f32(h, "h", n * w.inter), _stream(stream)))


def moe_expert_ffn_q4(w: MoeExperts, x, ids, n, y, h, stream=None) -> None:
    _expert_ffn("moe_expert_ffn_q4", w, x, ids, n, y, h, stream)


def moe_expert_ffn_q2(w: MoeExperts, x, ids, n, y, h, stream=None) -> None:
    _expert_ffn("moe_expert_ffn_q2", w, x, ids, n, y, h, stream)


def moe_combine(residual, y, weights, k, shared_gate, out, out_norm, eps, H, stream=None) -> None:
    _check("moe_combine", lib().moe_combine(
        _f32(residual, "residual", H), _f32(y, "y", (k + 1) * H), _f32(weights, "weights", k), k,
        _f32(shared_gate, "shared_gate", 1), _f32(out, "out", H), _f32(out_norm, "out_norm", H),
        eps, H, _stream(stream)))


def moe_layer_workspace_bytes(L: MoeLayer) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(L)))


def moe_layer_decode(L: MoeLayer, x, norm_input, eps, out, ids_out, weights_out, sg_out, ws,
                     ws_bytes, stream=None) -> None:
    H, k = L.experts.hidden, L.top_k
    _check("moe_layer_decode", lib().moe_layer_decode(
        ctypes.byref(L), _f32(x, "x", H), int(norm_input), eps, _f32(out, "out", H),
        _i32(ids_out, "ids_out", k + (1 if L.shared_slot >= 0 else 0)),
        _f32(weights_out, "weights_out", k), _f32(sg_out, "sg_out", 1), _u8(ws, "ws", ws_bytes),
        ws_bytes, _stream(stream)))


def _layer_array(layers):
    arr = (MoeLayer * len(layers))(*layers)
    return arr


def moe_stack_workspace_bytes(layers) -> int:
    arr = _layer_array(layers)
    return int(lib().moe_stack_workspace_bytes(arr, len(layers)))


STACK_AUTO, STACK_KERNELS, STACK_PERSISTENT, STACK_PLAIN_LAUNCH = 0, 1, 2, 16


def moe_decode_stack(layers, x_in, x_out, xn_out, eps, ids_trace, ws, ws_bytes,
                     stream=None, flags: int = STACK_AUTO) -> None:
    """flags: STACK_AUTO, STACK_KERNELS or STACK_PERSISTENT, optionally | STACK_PLAIN_LAUNCH
    (chosen per call; the library keeps no mode between calls)."""
    arr = layers if isinstance(layers, ctypes.Array) else _layer_array(layers)
    H, k = arr[0].experts.hidden, arr[0].top_k
    _check("moe_decode_stack", lib().moe_decode_stack(
        arr, len(arr), _f32(x_in, "x_in", H), _f32(x_out, "x_out", H), _f32(xn_out, "xn_out", H),
        eps, _i32(ids_trace, "ids_trace", len(arr) * k), int(flags), _u8(ws, "ws", ws_bytes),
        ws_bytes, _stream(stream)))


def moe_decode_stack_static(layers, x_in, x_out, xn_out, eps, ids_trace, stream=None,
                            flags: int = STACK_AUTO) -> None:
    """moe_decode_stack with the library's own per-GPU scratch instead of a workspace (no
    allocation in any call; calls on one GPU must not overlap)."""
    arr = layers if isinstance(layers, ctypes.Array) else _layer_array(layers)
    H, k = arr[0].experts.hidden, arr[0].top_k
    _check("moe_decode_stack_static", lib().moe_decode_stack_static(
        arr, len(arr), _f32(x_in, "x_in", H), _f32(x_out, "x_out", H), _f32(xn_out, "xn_out", H),
        eps, _i32(ids_trace, "ids_trace", len(arr) * k), int(flags), _stream(stream)))


def moe_layer_batch_workspace_bytes(L: MoeLayer, T: int) -> int:
    return int(lib().moe_layer_batch_workspace_bytes(ctypes.byref(L), T))


def moe_layer_decode_batch(L: MoeLayer, x, T: int, norm_input, eps, out, ids_out, weights_out,
                           sg_out, ws, ws_bytes, stream=None) -> None:
    H, k = L.experts.hidden, L.top_k
    _check("moe_layer_decode_batch", lib().moe_layer_decode_batch(
        ctypes.byref(L), _f32(x, "x", T * H), T, int(norm_input), eps, _f32(out, "out", T * H),
        _i32(ids_out, "ids_out", T * (k + (1 if L.shared_slot >= 0 else 0))),
        _f32(weights_out, "weights_out", T * k), _f32(sg_out, "sg_out", T),
        _u8(ws, "ws", ws_bytes), ws_bytes, _stream(stream)))


def moe_stack_batch_workspace_bytes(layers, T: int) -> int:
    arr = _layer_array(layers)
    return int(lib().moe_stack_batch_workspace_bytes(arr, len(layers), T))


def moe_decode_stack_batch(layers, x_in, T: int, x_out, xn_out, eps, ids_trace, ws, ws_bytes,
                           stream=None) -> None:
    arr = layers if isinstance(layers, ctypes.Array) else _layer_array(layers)
    H, k = arr[0].experts.hidden, arr[0].top_k
    _check("moe_decode_stack_batch", lib().moe_decode_stack_batch(
        arr, len(arr), _f32(x_in, "x_in", T * H), T, _f32(x_out, "x_out", T * H),
        _f32(xn_out, "xn_out", T * H), eps, _i32(ids_trace, "ids_trace", len(arr) * T * k),
        _u8(ws, "ws", ws_bytes), ws_bytes, _stream(stream)))


def moe_prefill_workspace_bytes(L: MoeLayer, T: int) -> int:
    return int(lib().moe_prefill_workspace_bytes(ctypes.byref(L), T))


def moe_prefill_q4(L: MoeLayer, x, T, out, ids_out, weights_out, sg_out, ws, ws_bytes,
                   stream=None) -> None:
    H, k = L.experts.hidden, L.top_k
    _check("moe_prefill_q4", lib().moe_prefill_q4(
        ctypes.byref(L), _f32(x, "x", T * H), T, _f32(out, "out", T * H),
        _i32(ids_out, "ids_out", T * k), _f32(weights_out, "weights_out", T * k),
        _f32(sg_out, "sg_out", T), _u8(ws, "ws", ws_bytes), ws_bytes, _stream(stream)))


def moe_pack_router(w_router, n_experts: int, hidden: int, dst, stream=None) -> None:
    n = n_experts * hidden
    _check("moe_pack_router", lib().moe_pack_router(
        _f32(w_router, "w_router", n), n_experts, hidden, _f32(dst, "dst", n), _stream(stream)))


def moe_qgemv(m: MoeQMatrix, x, y, stream=None) -> None:
    _check("moe_qgemv", lib().moe_qgemv(ctypes.byref(m), _f32(x, "x", m.cols),
                                        _f32(y, "y", m.rows), _stream(stream)))


def moe_rmsnorm(x, T: int, H: int, eps: float, out, stream=None) -> None:
    _check("moe_rmsnorm", lib().moe_rmsnorm(_f32(x, "x", T * H), T, H, eps,
                                            _f32(out, "out", T * H), _stream(stream)))


def moe_gdn_step(state, q, k, v, alpha, beta, n_heads: int, dk: int, dv: int, out,
                 stream=None) -> None:
    _check("moe_gdn_step", lib().moe_gdn_step(
        _f32(state, "state", n_heads * dv * dk), _f32(q, "q", n_heads * dk),
        _f32(k, "k", n_heads * dk), _f32(v, "v", n_heads * dv), _f32(alpha, "alpha", n_heads),
        _f32(beta, "beta", n_heads), n_heads, dk, dv, _f32(out, "out", n_heads * dv),
        _stream(stream)))


def moe_pack(canonical, n, slot0, dst: MoeExperts, stream=None) -> None:
    rec = _expert_bytes(dst.bits, dst.hidden, dst.inter, dst.group)
    _check("moe_pack", lib().moe_pack(_u8(canonical, "canonical", n * rec), n, slot0,
                                      ctypes.byref(dst), _stream(stream)))
