"""C-ABI checks that need no GPU: every symbol declared in include/*.h is exported by libmoe.so
and bound by the Python package under the same name, and host-side validation returns its
status code before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import group_quantized_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned stand-in address; never dereferenced on these paths


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("moe_router_topk", "moe_expert_ffn_q4", "moe_expert_ffn_q2", "moe_combine",
                     "moe_layer_decode", "moe_decode_stack", "moe_qgemv", "moe_rmsnorm",
                     "moe_gdn_step", "moe_pack"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name
        assert hasattr(moe, name) or name in ("moe_status_string", "moe_version"), name
    assert sorted(moe.EXPORTS) == _declared()


def test_status_strings():
    for st in range(7):
        assert moe.status_string(st)
    assert moe.status_string(0) == "ok"


def _experts(**kw):
    d = dict(base=FAKE, bits=4, hidden=4096, inter=1024, n_slots=513, slot_bytes=7077888)
    d.update(kw)
    return moe.experts(d["base"], d["bits"], d["hidden"], d["inter"], d["n_slots"],
                       d["slot_bytes"], group=d.get("group", 64))


@pytest.mark.parametrize("kw,status", [
    (dict(base=0), moe.MOE_E_NULL),
    (dict(bits=3), moe.MOE_E_BITS),
    (dict(group=32), moe.MOE_E_SHAPE),
    (dict(hidden=3000), moe.MOE_E_SHAPE),
    (dict(inter=1000), moe.MOE_E_SHAPE),
    (dict(slot_bytes=7077888 - 16), moe.MOE_E_SHAPE),
    (dict(slot_bytes=7077888 + 8), moe.MOE_E_ALIGN),
    (dict(base=FAKE + 4), moe.MOE_E_ALIGN),
])
def test_expert_ffn_validation(kw, status):
    w = _experts(**kw)
    st = moe.lib().moe_expert_ffn_q4(ctypes.byref(w), FAKE, FAKE, 5, FAKE, FAKE, None)
    assert st == status


def test_expert_ffn_bits_and_counts():
    L = moe.lib()
    w4 = _experts()
    assert L.moe_expert_ffn_q2(ctypes.byref(w4), FAKE, FAKE, 5, FAKE, FAKE, None) == moe.MOE_E_BITS
    assert L.moe_expert_ffn_q4(ctypes.byref(w4), FAKE, FAKE, 0, FAKE, FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_expert_ffn_q4(ctypes.byref(w4), FAKE, FAKE, 9, FAKE, FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_expert_ffn_q4(ctypes.byref(w4), None, FAKE, 5, FAKE, FAKE, None) == moe.MOE_E_NULL
    assert L.moe_expert_ffn_q4(ctypes.byref(w4), FAKE, FAKE, 5, FAKE, None, None) == moe.MOE_E_NULL


def test_router_validation():
    L = moe.lib()
    ws = moe.moe_router_workspace_bytes(1, 512)
    assert ws > 0
    ok = dict(x=FAKE, T=1, w=FAKE, wsg=FAKE, H=4096, E=512, k=4, ids=FAKE, ld=4, wts=FAKE,
              sg=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.moe_router_topk(a["x"], a["T"], a["w"], a["wsg"], a["H"], a["E"], a["k"],
                                 a["ids"], a["ld"], a["wts"], a["sg"], a["ws"], a["wsb"], None)
    assert call(x=None) == moe.MOE_E_NULL
    assert call(k=9) == moe.MOE_E_SHAPE
    assert call(k=5, ld=4) == moe.MOE_E_SHAPE
    assert call(E=2000) == moe.MOE_E_SHAPE
    assert call(H=100) == moe.MOE_E_SHAPE
    assert call(T=0) == moe.MOE_E_SHAPE
    assert call(x=FAKE + 8) == moe.MOE_E_ALIGN
    assert call(wsb=ws - 1) == moe.MOE_E_WORKSPACE
    assert call(ws=None) == moe.MOE_E_WORKSPACE


def test_layer_validation_and_workspace():
    L = moe.lib()
    lay = moe.layer(_experts(), FAKE, FAKE, 512, 4, 512)
    ws = moe.moe_layer_workspace_bytes(lay)
    assert ws > 0
    args = lambda lay_, x, out, wsb: L.moe_layer_decode(ctypes.byref(lay_), x, 0, 1e-6, out,
                                                          None, None, None, FAKE, wsb, None)
    assert args(lay, FAKE, FAKE + 4096 * 4, ws - 1) == moe.MOE_E_WORKSPACE
    assert args(lay, FAKE, FAKE, ws) == moe.MOE_E_SHAPE  # out aliases x
    assert args(lay, None, FAKE, ws) == moe.MOE_E_NULL
    bad_k = moe.layer(_experts(), FAKE, FAKE, 512, 9, 512)
    assert args(bad_k, FAKE, FAKE + 64, ws) == moe.MOE_E_SHAPE
    bad_shared = moe.layer(_experts(), FAKE, FAKE, 512, 4, 513)
    assert args(bad_shared, FAKE, FAKE + 64, ws) == moe.MOE_E_SHAPE
    too_many = moe.layer(_experts(n_slots=100), FAKE, FAKE, 512, 4, 99)
    assert args(too_many, FAKE, FAKE + 64, ws) == moe.MOE_E_SHAPE
    no_router = moe.layer(_experts(), None, FAKE, 512, 4, 512)
    assert args(no_router, FAKE, FAKE + 64, ws) == moe.MOE_E_NULL
    assert moe.moe_layer_workspace_bytes(bad_k) == 0


def test_stack_validation():
    L = moe.lib()
    lay = moe.layer(_experts(), FAKE, FAKE, 512, 4, 512)
    other = moe.layer(_experts(inter=512, slot_bytes=7077888), FAKE, FAKE, 512, 4, 512)
    arr = (moe.MoeLayer * 2)(lay, other)
    ws = moe.moe_stack_workspace_bytes([lay, lay])
    assert ws > moe.moe_layer_workspace_bytes(lay)
    assert L.moe_decode_stack(arr, 2, FAKE, FAKE + 64, None, 1e-6, None, 0, FAKE, ws,
                              None) == moe.MOE_E_SHAPE
    arr2 = (moe.MoeLayer * 2)(lay, lay)
    assert L.moe_decode_stack(arr2, 0, FAKE, FAKE + 64, None, 1e-6, None, 0, FAKE, ws,
                              None) == moe.MOE_E_SHAPE
    assert L.moe_decode_stack(arr2, 2, FAKE, FAKE, None, 1e-6, None, 0, FAKE, ws,
                              None) == moe.MOE_E_SHAPE
    assert L.moe_decode_stack(arr2, 2, FAKE, FAKE + 64, None, 1e-6, None, 0, FAKE, ws - 1,
                              None) == moe.MOE_E_WORKSPACE
    # the execution choice is a per-call argument: unknown modes and bits are refused
    for bad in (3, 4, 8, 32, moe.STACK_PLAIN_LAUNCH | 3, -1):
        assert L.moe_decode_stack(arr2, 2, FAKE, FAKE + 64, None, 1e-6, None, bad, FAKE, ws,
                                  None) == moe.MOE_E_SHAPE, bad


def test_binding_checks_tensor_arguments():
    """The binding refuses tensors the kernels would index out of bounds (wrong dtype, host
    memory, non-contiguous, too few elements) before any library call."""
    import pytest
    import torch
    x = torch.zeros(4096, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_rmsnorm(x, 1, 4096, 1e-6, x)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.experts(torch.zeros(16, dtype=torch.uint8), 4, 4096, 1024, 1, 7077888)

    class FakeCuda:  # the attributes the checks read, without a GPU
        is_cuda = True

        def __init__(self, dtype, n, contiguous=True):
            self.dtype, self.n, self.contig = dtype, n, contiguous

        def is_contiguous(self):
            return self.contig

        def numel(self):
            return self.n

        def data_ptr(self):
            return FAKE

    ok = FakeCuda(torch.float32, 64 * 128 * 128)
    small = FakeCuda(torch.float32, 64 * 128)
    for bad, msg in ((FakeCuda(torch.bfloat16, 64 * 128 * 128), "dtype"),
                     (FakeCuda(torch.float32, 64 * 128 * 128, contiguous=False), "contiguous"),
                     (FakeCuda(torch.float32, 64 * 128 * 128 - 1), "at least")):
        with pytest.raises(ValueError, match=msg):
            moe.moe_gdn_step(bad, small, small, small, small, small, 64, 128, 128, small)
    with pytest.raises(ValueError, match="at least"):
        moe.moe_gdn_step(ok, small, FakeCuda(torch.float32, 64 * 128 - 1), small, small, small,
                         64, 128, 128, small)
    with pytest.raises(ValueError, match="dtype"):
        moe.moe_expert_ffn_q4(_experts(), ok, FakeCuda(torch.int64, 8), 4, ok, ok)


def test_qgemv_and_pack_validation():
    L = moe.lib()
    m = moe.qmatrix(FAKE, 4, 1024, 4096)
    assert L.moe_qgemv(ctypes.byref(moe.qmatrix(FAKE, 3, 8, 256)), FAKE, FAKE, None) == moe.MOE_E_BITS
    assert L.moe_qgemv(ctypes.byref(moe.qmatrix(FAKE, 4, 8, 320)), FAKE, FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_qgemv(ctypes.byref(moe.qmatrix(FAKE, 4, 0, 256)), FAKE, FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_qgemv(ctypes.byref(m), FAKE + 4, FAKE, None) == moe.MOE_E_ALIGN
    assert L.moe_qgemv(ctypes.byref(m), None, FAKE, None) == moe.MOE_E_NULL
    assert L.moe_qgemv(ctypes.byref(moe.qmatrix(FAKE, 4, 8, 16384)), FAKE, FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_rmsnorm(None, 1, 4096, ctypes.c_float(1e-6), FAKE, None) == moe.MOE_E_NULL
    assert L.moe_rmsnorm(FAKE, 1, 4096, ctypes.c_float(1e-6), None, None) == moe.MOE_E_NULL
    assert L.moe_rmsnorm(FAKE, 0, 4096, ctypes.c_float(1e-6), FAKE, None) == moe.MOE_E_SHAPE
    assert L.moe_rmsnorm(FAKE, 1, 0, ctypes.c_float(1e-6), FAKE, None) == moe.MOE_E_SHAPE


def test_gdn_step_validation():
    L = moe.lib()
    F = FAKE
    assert L.moe_gdn_step(None, F, F, F, F, F, 64, 128, 128, F, None) == moe.MOE_E_NULL
    assert L.moe_gdn_step(F, F, F, F, F, None, 64, 128, 128, F, None) == moe.MOE_E_NULL
    assert L.moe_gdn_step(F, F, F, F, F, F, 64, 128, 128, None, None) == moe.MOE_E_NULL
    assert L.moe_gdn_step(F, F, F, F, F, F, 0, 128, 128, F, None) == moe.MOE_E_SHAPE
    assert L.moe_gdn_step(F, F, F, F, F, F, 64, 64, 128, F, None) == moe.MOE_E_SHAPE
    assert L.moe_gdn_step(F, F, F, F, F, F, 64, 128, 12, F, None) == moe.MOE_E_SHAPE
    assert L.moe_gdn_step(F, F, F, F, F, F, 64, 128, 4, F, None) == moe.MOE_E_SHAPE
    assert L.moe_gdn_step(F, F, F, F, F, F, 1 << 20, 128, 128, F, None) == moe.MOE_E_SHAPE
    assert L.moe_gdn_step(F + 4, F, F, F, F, F, 64, 128, 128, F, None) == moe.MOE_E_ALIGN
    assert L.moe_gdn_step(F, F, F + 8, F, F, F, 64, 128, 128, F, None) == moe.MOE_E_ALIGN
    dst = _experts(n_slots=4)
    assert L.moe_pack(FAKE, 5, 0, ctypes.byref(dst), None) == moe.MOE_E_SHAPE
    assert L.moe_pack(FAKE, 1, 4, ctypes.byref(dst), None) == moe.MOE_E_SHAPE
    assert L.moe_pack(None, 1, 0, ctypes.byref(dst), None) == moe.MOE_E_NULL
    assert L.moe_pack_router(FAKE, 512, 4096, None, None) == moe.MOE_E_NULL
    assert L.moe_pack_router(FAKE, 512, 4100, FAKE + 2 ** 24, None) == moe.MOE_E_SHAPE
    assert L.moe_pack_router(FAKE, 0, 4096, FAKE + 2 ** 24, None) == moe.MOE_E_SHAPE
    assert L.moe_pack_router(FAKE + 4, 512, 4096, FAKE + 2 ** 24, None) == moe.MOE_E_ALIGN
    # a misaligned blocked copy is refused like the other layer pointers
    lay = moe.layer(_experts(), FAKE, FAKE, 512, 4, 512, w_router_cb=FAKE + 8)
    assert moe.moe_layer_workspace_bytes(lay) == 0
