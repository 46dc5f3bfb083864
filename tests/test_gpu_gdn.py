"""GPU parity of the GatedDeltaNet state update (moe_gdn_step) against the fp64 oracle.

Inputs follow the shape of a linear-attention decode step: 64 heads of 128 x 128 fp32 state at
full size, unit-norm keys and queries, values ~ N(0, 1), decay gates in (0, 1) and betas in
(0, 1), state entries ~ N(0, 0.1^2).  Acceptance: fp32 state and outputs within relative L2 1e-4
and max-abs 1e-3 * max|ref|; alpha = 1, beta = 0 leaves the state bit-identical.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs(seed, nh, dv, dk=128):
    rng = np.random.default_rng(seed)
    S = (0.1 * rng.standard_normal((nh, dv, dk))).astype(np.float32)
    q = rng.standard_normal((nh, dk))
    k = rng.standard_normal((nh, dk))
    q = (q / np.linalg.norm(q, axis=1, keepdims=True)).astype(np.float32)
    k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((nh, dv)).astype(np.float32)
    alpha = rng.uniform(0.05, 1.0, nh).astype(np.float32)
    beta = rng.uniform(0.05, 1.0, nh).astype(np.float32)
    return S, q, k, v, alpha, beta


def _run(S, q, k, v, alpha, beta):
    nh, dv, dk = S.shape
    d = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (S, q, k, v, alpha, beta)]
    out = torch.empty(nh, dv, dtype=torch.float32, device="cuda")
    moe.moe_gdn_step(*d, nh, dk, dv, out)
    torch.cuda.synchronize()
    return d[0].cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("nh,dv", [(64, 128), (1, 8), (3, 24), (5, 200), (2, 1024)])
def test_gdn_step_parity(gpu_available, nh, dv):
    S, q, k, v, alpha, beta = _inputs(nh * 1000 + dv, nh, dv)
    print(f"gdn_step nh={nh} dv={dv}", flush=True)
    got_S, got_o = _run(S, q, k, v, alpha, beta)
    ref_S, ref_o = oracle.gdn_step(S, q, k, v, alpha, beta)
    gu.assert_close(got_S, ref_S, f"gdn state {nh}x{dv}")
    gu.assert_close(got_o, ref_o, f"gdn out {nh}x{dv}")


def test_gdn_step_chain_of_tokens(gpu_available):
    """Eight consecutive tokens on the device state against the oracle's own chain."""
    nh, dv = 64, 128
    S, *_ = _inputs(7, nh, dv)
    d_S = torch.from_numpy(S).cuda()
    ref_S = S.astype(np.float64)
    out = torch.empty(nh, dv, dtype=torch.float32, device="cuda")
    for t in range(8):
        _, q, k, v, alpha, beta = _inputs(100 + t, nh, dv)
        d = [torch.from_numpy(a).cuda() for a in (q, k, v, alpha, beta)]
        moe.moe_gdn_step(d_S, *d, nh, 128, dv, out)
        ref_S, ref_o = oracle.gdn_step(ref_S, q, k, v, alpha, beta)
        torch.cuda.synchronize()
        gu.assert_close(out.cpu().numpy(), ref_o, f"gdn chain out {t}")
    gu.assert_close(d_S.cpu().numpy(), ref_S, "gdn chain state")


def test_gdn_step_identity_and_pure_decay(gpu_available):
    nh, dv = 4, 64
    S, q, k, v, _, _ = _inputs(11, nh, dv)
    got_S, got_o = _run(S, q, k, v, np.ones(nh, np.float32), np.zeros(nh, np.float32))
    assert np.array_equal(got_S, S)
    gu.assert_close(got_o, oracle.gdn_step(S, q, k, v, np.ones(nh), np.zeros(nh))[1], "identity out")
    half = np.full(nh, 0.5, np.float32)
    got_S, _ = _run(S, q, k, v, half, np.zeros(nh, np.float32))
    assert np.array_equal(got_S, S * np.float32(0.5))  # scaling by a power of two is exact
