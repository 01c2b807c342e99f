"""The parity harness's reference for the sequential block's MoE path, on the CPU."""
from dataclasses import replace

import numpy as np

import synth
from oracle import oracle as O
from tests import parity


def test_sequential_router_reference_equals_the_oracle_on_the_oracle_inputs():
    """Fed the oracle's own x_l and Wo output, the reference is the oracle's router logits up to the
    fp32 sum the kernel forms (a bf16 flip of the MoE input aside, which this step does not have)."""
    s = replace(synth.TINY, block="sequential")
    W = O.Weights(s)
    kv = O.PagedKV(s, 2)
    ref = O.decode_step(W, kv, [17], np.arange(2, dtype=np.int32)[None], [0], trace=True)
    for l in range(s.n_layers):
        xp, xm = parity.seq_moe_input(W, ref.trace["x_in"][(l, 0)], ref.trace["attn"][(l, 0)], l)
        mo = O.moe_path(W, l, xm)
        assert np.max(np.abs(mo.r.astype(np.float64) - ref.router_logits[l, 0])) <= 2e-4
        # and the layer output from it is the oracle's, but for the fp32 sum x + Wo attn
        out = ref.trace["x_in"][(l + 1, 0)] if l + 1 < s.n_layers else ref.trace["x_final"][0]
        assert np.max(np.abs(xp + mo.moe - out)) <= 1e-5 * np.max(np.abs(out))


def test_sequential_router_reference_follows_the_kernel_wo_output():
    """A Wo output off by one bf16-sized step in one element moves the reference's logits by that
    element's weights, as it moves the kernel's."""
    s = replace(synth.TINY, block="sequential")
    W = O.Weights(s)
    kv = O.PagedKV(s, 2)
    ref = O.decode_step(W, kv, [17], np.arange(2, dtype=np.int32)[None], [0], trace=True)
    x, wo = ref.trace["x_in"][(0, 0)], ref.trace["attn"][(0, 0)].copy()
    r0 = O.moe_path(W, 0, parity.seq_moe_input(W, x, wo, 0)[1]).r.astype(np.float64)
    wo[3] += 0.25 * np.max(np.abs(x + wo))
    r1 = O.moe_path(W, 0, parity.seq_moe_input(W, x, wo, 0)[1]).r.astype(np.float64)
    assert np.max(np.abs(r1 - r0)) > 1e-3
