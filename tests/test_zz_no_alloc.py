"""The no-allocation stack decode (moe_decode_stack_static) against the workspace entry point
(marked gpu).  Both run the same kernels, so their results must be bitwise equal: for the
persistent kernel (full-size q4 layers) and for the three-kernel path (a 16-expert layer shape),
each on two calls in a row, the second with fewer layers, and with the device error word 0."""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, SEED_X, EPS = 31337, 2718, 1e-6


def _both(descs, x_np, flags):
    n = len(descs)
    wsb = moe.moe_stack_workspace_bytes(descs)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out = []
    for static in (False, True):
        x_in = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
        x_out = torch.full((gu.H,), 7.0, dtype=torch.float32, device="cuda")
        xn = torch.full((gu.H,), 7.0, dtype=torch.float32, device="cuda")
        trace = torch.full((n, gu.K), -7, dtype=torch.int32, device="cuda")
        if static:
            moe.moe_decode_stack_static(descs, x_in, x_out, xn, EPS, trace, flags=flags)
        else:
            moe.moe_decode_stack(descs, x_in, x_out, xn, EPS, trace, ws, wsb, flags=flags)
        torch.cuda.synchronize()
        out.append((x_out.cpu().numpy(), xn.cpu().numpy(), trace.cpu().numpy()))
    return out


@pytest.mark.parametrize("path", ["persistent", "kernels"])
def test_static_scratch_equals_workspace(gpu_available, path):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if path == "persistent":
        layers = [gu.Layer(SEED, L, 4, dev_err=err) for L in range(3)]
        flags = moe.STACK_PERSISTENT
    else:
        layers = [gu.Layer(SEED + 1, L, 4, n_experts=16, dev_err=err) for L in range(3)]
        flags = moe.STACK_KERNELS
    descs = [l.L for l in layers]
    for call, n in enumerate((3, 2)):  # the second call has the smaller input (fewer layers)
        x = synth.activations(SEED_X, call)
        (a, an, ta), (b, bn, tb) = _both(descs[:n], x, flags)
        assert int(err.item()) == 0
        assert np.array_equal(ta, tb), (path, call)
        assert np.array_equal(a, b) and np.array_equal(an, bn), (path, call)
        assert np.all(np.isfinite(b)) and np.all(tb >= 0)
    del layers
    torch.cuda.empty_cache()


def test_static_scratch_refuses_what_the_workspace_call_refuses(gpu_available):
    lay = gu.Layer(SEED + 2, 0, 4, n_experts=16)
    x = torch.zeros(gu.H, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_stack_static([lay.L], x, x, None, EPS, None)  # x_out aliases x_in
    assert e.value.status == moe.MOE_E_SHAPE
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_stack_static([lay.L], x, torch.empty_like(x), None, EPS, None, flags=3)
    assert e.value.status == moe.MOE_E_SHAPE
