"""GPU parity of the three-kernel layer decode at the other supported shapes (marked gpu).

The full-size tests use H 4096, I 1024.  The layer decode also takes H 1024 and 2048 and I from
256 to 2048, where the router/shared-expert kernel's input-split rows leave lanes idle and the
digit-plane records are fewer per token.  For q4 and q2, with and without the input norm, one
token and a 3-token batch (routed by its own launch) are checked against the fp64 oracle per
token (same expert sets on gap-enforced inputs, outputs within the relative L2 bar), and every
batch token bitwise against the single-token call.
"""
import numpy as np
import pytest
import torch

import group_quantized_expert_amd as moe
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SEED, E, K, EPS = 8642, 32, 4, 1e-6


def _decode(lay, xs, norm):
    T, H = len(xs), lay.H
    wsb = moe.moe_layer_batch_workspace_bytes(lay.L, T)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(np.ascontiguousarray(np.stack(xs), dtype=np.float32)).cuda()
    out = torch.empty(T * H, dtype=torch.float32, device="cuda")
    ids = torch.empty(T * (K + 1), dtype=torch.int32, device="cuda")
    w = torch.empty(T * K, dtype=torch.float32, device="cuda")
    sg = torch.empty(T, dtype=torch.float32, device="cuda")
    moe.moe_layer_decode_batch(lay.L, x, T, norm, EPS, out, ids, w, sg, ws, wsb)
    torch.cuda.synchronize()
    return (out.cpu().numpy().reshape(T, H), ids.cpu().numpy().reshape(T, K + 1),
            w.cpu().numpy().reshape(T, K), sg.cpu().numpy())


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("H,I", [(1024, 512), (2048, 256), (1024, 2048)])
@pytest.mark.parametrize("norm", [0, 1])
def test_layer_decode_shapes(gpu_available, bits, H, I, norm):
    lay = gu.Layer(SEED + H + I, 0, bits, n_experts=E, hidden=H, inter=I, top_k=K)
    xs, t = [], 0
    for _ in range(3):
        t, x = gu.gap_enforced_x(SEED + H, lay.wr, K, hidden=H, start=t, norm_input=bool(norm))
        xs.append(x)
        t += 1
    out3, ids3, w3, sg3 = _decode(lay, xs, norm)
    for i, x in enumerate(xs):
        ref = lay.oracle_layer(x, norm_input=bool(norm), eps=EPS)
        what = f"q{bits} H {H} I {I} norm {norm} token {i}"
        assert ids3[i, K] == E, what
        gu.assert_same_routing(ids3[i, :K].tolist(), w3[i], ref["ids"], ref["weights"])
        np.testing.assert_allclose(sg3[i], ref["sg"], rtol=1e-5)
        gu.assert_close(out3[i], ref["out"], what)
        out1, ids1, w1, sg1 = _decode(lay, [x], norm)
        assert np.array_equal(out1[0], out3[i]), what
        assert np.array_equal(ids1[0], ids3[i]) and np.array_equal(w1[0], w3[i]), what
        assert np.array_equal(sg1, sg3[i:i + 1]), what
