"""Shared helpers of the GPU parity tests: resident layers filled on the device from the seeded
generator, gap-enforced inputs chosen with the oracle, and the acceptance tolerance."""
from __future__ import annotations

import numpy as np
import torch

import group_quantized_expert_amd as moe
import oracle
import synth

H, I, G, E, K = synth.HIDDEN, synth.INTER, synth.GROUP, synth.N_EXPERTS, synth.TOP_K

# acceptance: relative L2 <= 1e-4 and max-abs <= 1e-3 * max|ref| on fp32 outputs
REL_L2 = 1e-4
MAX_ABS = 1e-3


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    e = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref)))
    assert e <= REL_L2, f"{what}: relative L2 {e:.3e} > {REL_L2}"
    assert m <= MAX_ABS * float(np.max(np.abs(ref))), f"{what}: max-abs {m:.3e}"


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


class Layer:
    """One resident MoE layer: n_slots expert records + router + shared-gate weights."""

    def __init__(self, seed: int, layer: int, bits: int, n_experts: int = E, hidden: int = H,
                 inter: int = I, top_k: int = K, shared: bool = True, dev_err=None):
        self.seed, self.layer, self.bits = seed, layer, bits
        self.E, self.H, self.I, self.k = n_experts, hidden, inter, top_k
        self.n_slots = n_experts + (1 if shared else 0)
        self.shared_slot = n_experts if shared else -1
        self.slot_bytes = synth.expert_bytes(bits, hidden, inter, G)
        dev = torch.device("cuda")
        self.buf = torch.empty(self.n_slots * self.slot_bytes, dtype=torch.uint8, device=dev)
        synth.gpu_fill_experts(self.buf.data_ptr(), self.slot_bytes, 0, self.n_slots, seed, layer,
                               bits, hidden, inter, G, stream_handle())
        self.wr = synth.router_weights(seed, layer, n_experts, hidden)
        self.wsg = synth.shared_gate_weights(seed, layer, hidden)
        self.d_wr = torch.from_numpy(self.wr).to(dev)
        self.d_wsg = torch.from_numpy(self.wsg).to(dev)
        self.dev_err = dev_err
        self.desc = moe.experts(self.buf, bits, hidden, inter, self.n_slots, self.slot_bytes,
                                dev_err=dev_err)
        # column-blocked router copy (read by the persistent stack decode); L carries it, as
        # the benchmark's layers do, L_plain does not
        self.d_wr_cb = torch.empty_like(self.d_wr)
        moe.moe_pack_router(self.d_wr, n_experts, hidden, self.d_wr_cb, stream_handle())
        self.L = moe.layer(self.desc, self.d_wr, self.d_wsg, n_experts, top_k, self.shared_slot,
                           w_router_cb=self.d_wr_cb)
        self.L_plain = moe.layer(self.desc, self.d_wr, self.d_wsg, n_experts, top_k,
                                 self.shared_slot)
        self._cache = {}

    def expert_cpu(self, slot: int) -> np.ndarray:
        if slot not in self._cache:
            self._cache[slot] = synth.expert(self.seed, self.layer, slot, self.bits, self.H,
                                             self.I, G)
        return self._cache[slot]

    def oracle_layer(self, x, norm_input=False, eps=1e-6):
        return oracle.layer(x, self.wr, self.wsg, self.expert_cpu, self.bits, self.k,
                            self.shared_slot if self.shared_slot >= 0 else None, self.H, self.I,
                            G, norm_input=norm_input, eps=eps)


def logit_gap(wr, x, k, norm_input=False, eps=1e-6) -> float:
    xin = oracle.rmsnorm(x, eps) if norm_input else np.asarray(x, dtype=np.float64)
    l = np.sort(oracle.router_logits(wr, xin))[::-1]
    return float(l[k - 1] - l[k])


def gap_enforced_x(seed: int, wr, k: int, hidden: int = H, start: int = 0, min_gap: float = 1e-3,
                   norm_input=False):
    """First token index t >= start whose N(0,1) input has oracle top-k / top-(k+1) logit gap
    >= min_gap; returns (t, x)."""
    t = start
    while True:
        x = synth.activations(seed, t, hidden)
        if logit_gap(wr, x, k, norm_input) >= min_gap:
            return t, x
        t += 1


def chained_routing(got, otrace, drift0, k, n_layers, what=""):
    """Routing of a chained GPU decode against the oracle's own chain.  Layer by layer the
    selected sets must match, except at a near-tie: where the oracle's k-th and (k+1)-th logits
    are closer, in units of the logits' standard deviation, than 10 x the chain's drift bound at
    that depth (drift0 grown by 4e4 over n_layers, the growth measured on the oracle alone), a set
    made of the oracle's k + 1 best minus one of that pair is also correct.  Returns the layer
    where the chains part (None if they never do); raises AssertionError otherwise."""
    for L, r in enumerate(otrace):
        g = sorted(int(v) for v in got[L])
        if g == sorted(int(v) for v in r["ids"]):
            continue
        lg = np.asarray(r["logits"], dtype=np.float64)
        order = np.argsort(-lg, kind="stable")
        gap = (lg[order[k - 1]] - lg[order[k]]) / np.std(lg)
        bound = 10.0 * drift0 * 4e4 ** (L / n_layers)
        assert gap <= bound, (what, L, g, r["ids"], gap, bound)
        assert set(g) | {int(order[k - 1]), int(order[k])} == set(int(v) for v in order[:k + 1]), \
            (what, L, g, r["ids"])
        return L
    return None


def assert_same_routing(got_ids, got_w, ref_ids, ref_w, what=""):
    """The selected expert set must match exactly; the order inside the top-k only reflects
    near-equal logits and carries no arithmetic, so weights are compared per expert id."""
    got_ids = [int(v) for v in got_ids]
    ref_ids = [int(v) for v in ref_ids]
    assert sorted(got_ids) == sorted(ref_ids), (what, got_ids, ref_ids)
    if got_w is not None:
        gw = dict(zip(got_ids, [float(v) for v in got_w]))
        for e, w in zip(ref_ids, ref_w):
            assert abs(gw[e] - float(w)) <= 1e-4 * abs(float(w)) + 1e-6, (what, e, gw[e], w)
