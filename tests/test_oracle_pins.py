"""Pins of the CPU oracle to things other than itself.

Each test ties one part of the oracle to a closed form, an invariant, a
library routine, a brute-force computation on tiny inputs, or the numbers the
pages print, chosen so that a plausible slip (a dropped gain, a wrong sign or
pairing in the rotation, an off-by-one position, a wrong GQA group, a
transposed operand, a wrong tie rule) fails at least one of them.
"""
import json
import math
import os

from dataclasses import replace

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import synth
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- bf16


def test_round_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        # exact ties between neighbouring bf16 values
                        (1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -8) * 2.0 ** rng.integers(-20, 20, 199)])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_rounds_the_exact_value_once():
    u = 2.0 ** -8
    cases = {
        1.0 + u: 1.0,                          # tie -> even
        1.0 + 3 * u: 1.0 + 4 * u,              # tie -> even (up)
        1.0 + u + 2.0 ** -40: 1.0 + 2 * u,     # above the tie: rounding via fp32 first would give 1.0
        -(1.0 + u + 2.0 ** -40): -(1.0 + 2 * u),
        0.0: 0.0,
        3.0: 3.0,
        2.0 ** -130 * 1.3: 2.0 ** -133 * round(1.3 * 8),   # subnormal quantum 2^-133
        3.5e38: math.inf,
    }
    for x, want in cases.items():
        assert O.round_bf16(np.array([x]))[0] == want, x


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    v = O.bf16_to_f64(bits[finite])
    assert np.array_equal(O.f64_to_bf16_bits(v), bits[finite])


# --------------------------------------------------------------------------- RMSNorm


def test_rmsnorm_closed_form_on_constant_vector():
    rng = np.random.default_rng(1)
    g = 1.0 + 0.02 * rng.standard_normal(64)
    for c, eps in ((3.0, 1e-6), (1e-3, 1e-6), (-2.0, 0.5)):
        got = O.rmsnorm(np.full(64, c), g, eps)
        assert np.allclose(got, c / math.sqrt(c * c + eps) * g, rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(256)
    g = np.ones(256)
    y = O.rmsnorm(x, g, 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    assert np.allclose(O.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-14)


# --------------------------------------------------------------------------- RoPE


def test_rope_position_zero_is_identity():
    v = np.random.default_rng(3).standard_normal((4, 64))
    assert np.array_equal(O.rope(v, 0, 1e4), v)


def test_rope_hand_computed_d4():
    # d = 4, theta = 1e4: inv_freq = [1, 1e-2]; pairs are (0, 2) and (1, 3)
    v = np.array([[1.0, 2.0, 3.0, 4.0]])
    p = 5
    a0, a1 = 5.0, 0.05
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            1 * math.sin(a0) + 3 * math.cos(a0), 2 * math.sin(a1) + 4 * math.cos(a1)]
    assert np.allclose(O.rope(v, p, 1e4)[0], want, rtol=1e-15, atol=1e-15)


def test_rope_equals_complex_rotation_and_is_relative():
    rng = np.random.default_rng(4)
    d, theta = 128, 1e4
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    m = 1234
    z = (q[: d // 2] + 1j * q[d // 2:]) * np.exp(1j * m * theta ** (-np.arange(0, d, 2) / d))
    r = O.rope(q[None], m, theta)[0]
    assert np.allclose(r[: d // 2], z.real, atol=1e-12) and np.allclose(r[d // 2:], z.imag, atol=1e-12)
    # norm preserved pair by pair
    assert np.allclose(r[: d // 2] ** 2 + r[d // 2:] ** 2, q[: d // 2] ** 2 + q[d // 2:] ** 2, rtol=1e-12)
    # <rope(q, m), rope(k, n)> depends only on m - n
    d1 = O.rope(q[None], 40, theta)[0] @ O.rope(k[None], 17, theta)[0]
    d2 = O.rope(q[None], 40 + 999, theta)[0] @ O.rope(k[None], 17 + 999, theta)[0]
    assert abs(d1 - d2) < 1e-10


# --------------------------------------------------------------------------- attention


def test_attention_single_position_returns_v():
    rng = np.random.default_rng(5)
    q, K, V = rng.standard_normal(64), rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    assert np.array_equal(O.attention_head(q, K, V), V[0])


def test_attention_equal_keys_give_mean_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(64)
    K = np.tile(rng.standard_normal(64), (37, 1))
    V = rng.standard_normal((37, 64))
    assert np.allclose(O.attention_head(q, K, V), V.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_matches_scipy_softmax_brute_force():
    rng = np.random.default_rng(7)
    for n in (2, 17, 300):
        q, K, V = rng.standard_normal(128), rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
        p = scipy.special.softmax(np.array([q @ K[t] for t in range(n)]) / math.sqrt(128))
        want = sum(p[t] * V[t] for t in range(n))
        assert np.allclose(O.attention_head(q, K, V), want, rtol=1e-12, atol=1e-14)
        assert abs(O.softmax(K @ q).sum() - 1.0) < 1e-14


# --------------------------------------------------------------------------- router


def test_topk_matches_stable_full_sort_with_ties():
    rng = np.random.default_rng(8)
    for _ in range(200):
        r = rng.integers(0, 6, 32).astype(np.float32)   # many exact ties
        k = int(rng.integers(1, 9))
        want = np.argsort(-r.astype(np.float64), kind="stable")[:k]
        assert np.array_equal(O.topk_desc(r, k), want)


def test_softmax_over_selected_equals_renormalised_full_softmax():
    rng = np.random.default_rng(9)
    r = rng.standard_normal(128)
    sel = O.topk_desc(r, 8)
    full = scipy.special.softmax(r)
    assert np.allclose(O.softmax(r[sel]), full[sel] / full[sel].sum(), rtol=1e-13)
    assert abs(O.softmax(r[sel]).sum() - 1.0) < 1e-15


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15


def test_gemv_matches_exact_sum():
    rng = np.random.default_rng(10)
    bits = synth.normal_bf16(0, 77, 0, 16 * 2048, 0.02).reshape(16, 2048)
    W = O.bf16_to_f64(bits)
    x = O.round_bf16(rng.standard_normal(2048))
    y = W @ x
    for i in range(16):
        exact = math.fsum(float(W[i, j]) * float(x[j]) for j in range(2048))
        assert abs(y[i] - exact) <= 1e-13 * max(1.0, abs(exact))


# --------------------------------------------------------------------------- whole step on the tiny model


def _tiny_setup(pages_shuffled: bool, source=None, n_prompt: int = 6):
    s = synth.TINY
    W = O.Weights(s, source=source)
    num_pages = 4
    pt = np.arange(num_pages, dtype=np.int32)
    if pages_shuffled:
        pt = np.array([2, 0, 3, 1], dtype=np.int32)
    kv = O.PagedKV(s, num_pages)
    return s, W, kv, pt


def test_paged_shuffled_equals_identity_bit_exact():
    toks = synth.uniform_u32(synth.SEED_PROMPT, synth.tid(synth.K_PROMPT, 0), 0, 20, synth.TINY.vocab)
    outs = []
    for shuffled in (False, True):
        s, W, kv, pt = _tiny_setup(shuffled)
        for t, tok in enumerate(toks):
            out = O.decode_step(W, kv, [int(tok)], pt[None], [t])
        outs.append(out.logits)
    assert np.array_equal(outs[0], outs[1])


def _full_recompute_logits(W, toks):
    """Non-cached causal forward over the whole sequence; logits of the last position.

    Each layer handles all positions at once: K/V of every position are
    computed in the same pass, and position t attends over rows 0..t.
    """
    s = W.shape
    n, d, nq, nkv = len(toks), s.head_dim, s.n_q_heads, s.n_kv_heads
    X = np.stack([W.get(synth.K_EMBED)[int(t)] for t in toks])
    for l in range(s.n_layers):
        XN = np.stack([O.round_bf16(O.rmsnorm(X[t], W.get(synth.K_ATTN_NORM, l), s.rms_eps)) for t in range(n)])
        QKV = np.stack([W.get(synth.K_WQKV, l) @ XN[t] for t in range(n)])
        Q = np.stack([O.round_bf16(O.rope(QKV[t, : nq * d].reshape(nq, d), t, s.rope_theta)) for t in range(n)])
        K = np.stack([O.round_bf16(O.rope(QKV[t, nq * d:(nq + nkv) * d].reshape(nkv, d), t, s.rope_theta)) for t in range(n)])
        V = np.stack([O.round_bf16(QKV[t, (nq + nkv) * d:].reshape(nkv, d)) for t in range(n)])
        Xn = np.empty_like(X)
        for t in range(n):
            o = np.stack([O.attention_head(Q[t, h], K[: t + 1, h // (nq // nkv)], V[: t + 1, h // (nq // nkv)])
                          for h in range(nq)])
            attn = W.get(synth.K_WO, l) @ O.round_bf16(o.reshape(-1))
            r = (W.get(synth.K_ROUTER, l) @ XN[t]).astype(np.float32)
            sel = np.argsort(-r.astype(np.float64), kind="stable")[: s.top_k]
            w = scipy.special.softmax(r[sel].astype(np.float64))
            moe = np.zeros(s.hidden)
            for j, e in enumerate(sel):
                h = O.round_bf16(O.silu(W.get(synth.K_W_GATE, l, int(e)) @ XN[t]) * (W.get(synth.K_W_UP, l, int(e)) @ XN[t]))
                moe = moe + w[j] * (W.get(synth.K_W_DOWN, l, int(e)) @ h)
            Xn[t] = (X[t] + attn) + moe
        X = Xn
    xf = O.round_bf16(O.rmsnorm(X[-1], W.get(synth.K_FINAL_NORM), s.rms_eps))
    return W.get(synth.K_LM_HEAD) @ xf


def test_cached_decode_equals_full_recompute():
    toks = synth.uniform_u32(synth.SEED_PROMPT, synth.tid(synth.K_PROMPT, 0), 0, 19, synth.TINY.vocab)
    s, W, kv, pt = _tiny_setup(True)
    for t, tok in enumerate(toks):
        out = O.decode_step(W, kv, [int(tok)], pt[None], [t])
    ref = _full_recompute_logits(W, toks)
    assert np.max(np.abs(out.logits[0] - ref)) <= 1e-9 * np.max(np.abs(ref))


def _modified_source(s, zero_kinds=(), identical_experts=False, zero_k_rows=False):
    def src(kind, layer, expert):
        if identical_experts and kind in (synth.K_W_GATE, synth.K_W_UP, synth.K_W_DOWN):
            a = synth.weight_bits(s, kind, layer, 0 if expert is not None else None)
            if expert is None:
                a = np.broadcast_to(a[0], a.shape).copy()
        else:
            a = synth.weight_bits(s, kind, layer, expert)
        if kind in zero_kinds:
            a = np.zeros_like(a)
        if zero_k_rows and kind == synth.K_WQKV:
            a = a.copy()
            nq, nkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
            a[nq * d:(nq + nkv) * d] = 0
        return a
    return src


def test_zero_attention_and_expert_outputs_leave_residual_as_embedding():
    s = synth.TINY
    W = O.Weights(s, source=_modified_source(s, zero_kinds=(synth.K_WO, synth.K_W_DOWN)))
    kv = O.PagedKV(s, 2)
    tok = 77
    out = O.decode_step(W, kv, [tok], np.arange(2, dtype=np.int32)[None], [0], trace=True)
    e = W.get(synth.K_EMBED)[tok]
    assert np.array_equal(out.trace["x_final"][0], e)
    want = W.get(synth.K_LM_HEAD) @ O.round_bf16(O.rmsnorm(e, W.get(synth.K_FINAL_NORM), s.rms_eps))
    assert np.array_equal(out.logits[0], want)


def _seq_source(s, zero_kinds=(), moe_gain_factor=None, wo_factor=None):
    """Sources for a sequential-block model: optionally zeroed kinds, the MoE norm gain as a multiple
    of the attention norm gain (exact for powers of two), Wo scaled (a power of two: exact)."""
    def src(kind, layer, expert):
        if kind == synth.K_MOE_NORM and moe_gain_factor is not None:
            g = O.bf16_to_f64(synth.weight_bits(s, synth.K_ATTN_NORM, layer)) * moe_gain_factor
            return O.f64_to_bf16_bits(g)
        a = synth.weight_bits(s, kind, layer, expert)
        if kind in zero_kinds:
            a = np.zeros_like(a)
        if kind == synth.K_WO and wo_factor is not None:
            a = O.f64_to_bf16_bits(O.bf16_to_f64(a) * wo_factor)
        return a
    return src


def _step_pair(zero_kinds=(), moe_gain_factor=None, toks=(77, 5, 301)):
    """The same three decode steps through the parallel and the sequential tiny model."""
    outs = []
    for block in ("parallel", "sequential"):
        s = replace(synth.TINY, block=block)
        W = O.Weights(s, source=_seq_source(s, zero_kinds, moe_gain_factor))
        kv = O.PagedKV(s, 2)
        pt = np.arange(2, dtype=np.int32)[None]
        outs.append([O.decode_step(W, kv, [t], pt, [i], trace=True) for i, t in enumerate(toks)])
    return outs


def test_sequential_block_without_expert_outputs_equals_parallel():
    """With every down matrix zero the MoE path adds nothing, so both blocks leave x + attn: a
    sequential block that added the attention output twice, or lost it, would differ."""
    par, seq = _step_pair(zero_kinds=(synth.K_W_DOWN,))
    for a, b in zip(par, seq):
        assert np.array_equal(a.logits, b.logits)
        for key in a.trace["x_in"]:
            assert np.array_equal(a.trace["x_in"][key], b.trace["x_in"][key])


def test_sequential_block_without_attention_output_equals_parallel():
    """With Wo zero and the MoE norm gain equal to the attention norm gain, x + attn = x and the MoE
    path sees the parallel block's normalized input: the steps agree bit for bit."""
    par, seq = _step_pair(zero_kinds=(synth.K_WO,), moe_gain_factor=1.0)
    for a, b in zip(par, seq):
        assert np.array_equal(a.logits, b.logits)
        assert np.array_equal(a.sel, b.sel)


def test_sequential_block_normalizes_with_the_moe_gain():
    """Wo zero and the MoE gain twice the attention gain: the MoE input is exactly twice the
    attention input (a power of two commutes with the bf16 rounding), so are the router logits."""
    s = replace(synth.TINY, block="sequential")
    W = O.Weights(s, source=_seq_source(s, zero_kinds=(synth.K_WO,), moe_gain_factor=2.0))
    kv = O.PagedKV(s, 2)
    out = O.decode_step(W, kv, [123], np.arange(2, dtype=np.int32)[None], [0], trace=True)
    for l in range(s.n_layers):
        xn, xm = out.trace["xn"][(l, 0)], out.trace["xm"][(l, 0)]
        assert np.array_equal(xm, 2.0 * xn)
        assert np.array_equal(out.router_logits[l, 0], (W.get(synth.K_ROUTER, l) @ (2.0 * xn)).astype(np.float32))


def test_sequential_block_moe_input_follows_the_attention_output():
    """Wo scaled by 2^20: in layer 0, x (an embedding row) + attn is attn to within ~2^-20
    relative, and rmsnorm ignores scale, so the MoE input is the normalized attention output (a
    block that fed the MoE path x alone, or the attention input, would not be).  Later layers'
    x carries the earlier layers' scaled attention outputs, so the check is layer 0's."""
    s = replace(synth.TINY, block="sequential")
    W = O.Weights(s, source=_seq_source(s, wo_factor=2.0 ** 20))
    kv = O.PagedKV(s, 2)
    for pos, tok in enumerate((9, 400, 33)):
        out = O.decode_step(W, kv, [tok], np.arange(2, dtype=np.int32)[None], [pos], trace=True)
        l = 0
        attn = out.trace["attn"][(l, 0)]
        want = O.round_bf16(O.rmsnorm(attn, W.get(synth.K_MOE_NORM, l), s.rms_eps))
        xm = out.trace["xm"][(l, 0)]
        # equal but for the rare element whose bf16 rounding the 2^-20 remainder tips
        assert np.mean(xm == want) > 0.97 and np.max(np.abs(xm - want)) <= 2.0 ** -7 * np.max(np.abs(want))
        assert np.mean(xm == out.trace["xn"][(l, 0)]) < 0.5


def test_identical_experts_reduce_to_one_dense_swiglu_ffn():
    s = synth.TINY
    W = O.Weights(s, source=_modified_source(s, identical_experts=True))
    kv = O.PagedKV(s, 2)
    out = O.decode_step(W, kv, [5], np.arange(2, dtype=np.int32)[None], [0], trace=True)
    for l in range(s.n_layers):
        xn = out.trace["xn"][(l, 0)]
        h = O.round_bf16(O.silu(W.get(synth.K_W_GATE, l, 0) @ xn) * (W.get(synth.K_W_UP, l, 0) @ xn))
        dense = W.get(synth.K_W_DOWN, l, 0) @ h
        assert np.allclose(out.trace["moe"][(l, 0)], dense, rtol=1e-13, atol=1e-16)


def test_gqa_groups_read_their_own_kv_head():
    """Zero keys give uniform attention: head h must average the V of kv head h // (nq/nkv)."""
    s = synth.TINY
    W = O.Weights(s, source=_modified_source(s, zero_k_rows=True))
    kv = O.PagedKV(s, 1)
    p = 5
    pt = np.zeros((1, 1), dtype=np.int32)
    consts = [0.5, -2.0]                       # V of kv head g is consts[g] at positions 0..p-1
    for g in range(s.n_kv_heads):
        kv.k[:, 0, g, :p, :] = 0
        kv.v[:, 0, g, :p, :] = O.f64_to_bf16_bits(np.array([consts[g]]))[0]
    out = O.decode_step(W, kv, [9], pt, [p], trace=True)
    group = s.n_q_heads // s.n_kv_heads
    for l in range(s.n_layers):
        v_new = out.trace["v16"][(l, 0)]
        a = out.trace["a16"][(l, 0)].reshape(s.n_q_heads, s.head_dim)
        for h in range(s.n_q_heads):
            g = h // group
            want = O.round_bf16((p * consts[g] + v_new[g]) / (p + 1))
            assert np.array_equal(a[h], want), (l, h)


def test_new_kv_written_at_position_slot_and_rotated_at_p():
    s, W, kv, pt = _tiny_setup(True)
    toks = [3, 900, 41]
    for t, tok in enumerate(toks):
        out = O.decode_step(W, kv, [tok], pt[None], [t], trace=True)
    p = len(toks) - 1
    for l in range(s.n_layers):
        xn = out.trace["xn"][(l, 0)]
        nq, nkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
        kk = (W.get(synth.K_WQKV, l) @ xn)[nq * d:(nq + nkv) * d].reshape(nkv, d)
        want = O.f64_to_bf16_bits(O.rope(kk, p, s.rope_theta))
        page, off = int(pt[p // s.page_size]), p % s.page_size
        assert np.array_equal(kv.k[l, page, :, off, :], want)
        # slots after p are still poison
        assert np.all(kv.k[l, page, :, off + 1:, :] == 0x7FC0)


def test_greedy_ties_go_to_lowest_id():
    logits = np.array([[0.0, 3.0, 1.0, 3.0]])
    assert int(np.argmax(logits, axis=1)[0]) == 1


# --------------------------------------------------------------------------- speed-of-light numbers the pages print


def test_sol_bound_reproduces_the_pages_numbers():
    with open(os.path.join(GOLDEN, "sol_bound_h100.json")) as f:
        g = json.load(f)
    bound = O.sol_tokens_per_s(g["hbm_bytes_per_s"], g["weight_bytes"] + g["kv_bytes"])
    assert abs(bound - g["bound_tok_s"]) / g["bound_tok_s"] < 0.01
    assert round(100 * g["megakernel_tok_s"] / g["bound_tok_s"]) == g["megakernel_pct"]
    assert round(100 * g["vllm_tok_s"] / g["bound_tok_s"]) == g["vllm_pct"]
    assert round(g["megakernel_tok_s"] / g["vllm_tok_s"], 2) == g["speedup"]


def test_step_bytes_30b_shape_8k():
    s = synth.MOE30B
    # 48 layers x 2 (K, V) x 4 kv heads x 128 x 2 bytes per token
    assert s.kv_bytes_per_token() == 98304
    b = O.step_bytes(s, [8192], s.top_k)
    w = s.active_weight_bytes(s.top_k)
    assert abs(w / 1e9 - 6.0835) < 5e-4
    assert abs((b - w - 2 * s.hidden) - 98304 * 8193) < 1


def test_non_square_shape_catches_transposed_operands():
    """Every matrix of this shape is non-square, so a transposed operand cannot broadcast."""
    s = synth.ModelShape(n_layers=2, hidden=96, n_q_heads=4, n_kv_heads=2, head_dim=16,
                         n_experts=6, top_k=2, inter=40, vocab=200)
    assert len({s.hidden, s.attn_dim, s.qkv_rows, s.inter, s.n_experts, s.vocab}) == 6
    W = O.Weights(s)
    kv = O.PagedKV(s, 2)
    out = None
    for t, tok in enumerate((1, 150, 7)):
        out = O.decode_step(W, kv, [tok], np.array([[1, 0]], dtype=np.int32), [t])
    assert out.logits.shape == (1, 200) and np.all(np.isfinite(out.logits))


def test_route_alternative_only_at_a_near_tie():
    """Equal router rows tie every logit: the alternative set swaps the k-th for the (k+1)-th."""
    s = synth.TINY

    def src(kind, layer, expert):
        a = synth.weight_bits(s, kind, layer, expert)
        if kind == synth.K_ROUTER:
            a = np.broadcast_to(a[0], a.shape).copy()
        return a
    W = O.Weights(s, source=src)
    out = O.decode_step(W, O.PagedKV(s, 1), [3], np.zeros((1, 1), dtype=np.int32), [0], route_alt={(1, 0)})
    assert list(out.sel[0, 0]) == [0, 1] and list(out.sel[1, 0]) == [0, 2]
    assert list(out.sel_alt[1, 0]) == [0, 2] and out.margin[1, 0] == 0.0
    with pytest.raises(ValueError):
        O.decode_step(O.Weights(s), O.PagedKV(s, 1), [3], np.zeros((1, 1), dtype=np.int32), [0], route_alt={(0, 0)})


def test_layer_subset_cache_gives_the_same_layer():
    """A cache holding only some layers serves those layers exactly as the full cache does."""
    w = synth.workload("tiny")
    s = w.shape
    W = O.Weights(s)
    pt = w.page_table()
    full = O.PagedKV(s, w.num_pages)
    part = O.PagedKV(s, w.num_pages, layers=[1])
    ctx = [40]
    full.fill_synthetic(pt, ctx)
    part.fill_synthetic(pt, ctx)
    x = O.bf16_to_f64(synth.normal_bf16(9, synth.tid(1, 0), 0, s.hidden, 0.5))
    a = O.layer_forward(W, full, 1, x, 40, pt[0])
    b = O.layer_forward(W, part, 1, x, 40, pt[0])
    assert np.array_equal(a.x, b.x) and np.array_equal(a.sel, b.sel) and np.array_equal(a.r, b.r)
    with pytest.raises(KeyError):
        part.gather(0, pt[0], 4, 0)


# --------------------------------------------------------------------------- synthetic KV fill and LM head


@pytest.mark.parametrize("name,context", [("tiny", [40, 0, 17, 16]), ("mid", [300, 33, 1])])
def test_fill_synthetic_places_every_position_at_its_page_slot(name, context):
    """Every logical position t of sequence b lands at (page_table[b][t // 16], t % 16) of every
    layer and kv head, K from the K stream and V from the V stream, bit for bit; every other
    slot, and every page no sequence owns, keeps the NaN poison.

    The expected values come straight from the generator, and the slot from the page-table
    rule, without going through the cache's own gather or slot lookup, so a swapped K/V, a
    wrong page index, a transposed [slot][head] block or an off-by-one position fails."""
    base = synth.workload(name)
    w = synth.Workload(name + "_pin", base.shape, batch=len(context), steps=2, context=context,
                       shuffle_pages=True, spare_pages=2)
    s, ps = w.shape, w.shape.page_size
    pt = w.page_table()
    assert not np.array_equal(pt[pt >= 0], np.sort(pt[pt >= 0])), "page order must be shuffled"
    kv = O.PagedKV(s, w.num_pages)
    kv.fill_synthetic(pt, context)
    written = np.zeros((w.num_pages, ps), dtype=bool)
    for b, n in enumerate(context):
        for t in range(n):
            written[pt[b, t // ps], t % ps] = True
    for l in range(s.n_layers):
        for b, n in enumerate(context):
            if n == 0:
                continue
            K = synth.kv_bits(s, l, "k", b, 0, n)     # [t][head][d]
            V = synth.kv_bits(s, l, "v", b, 0, n)
            pages = pt[b, np.arange(n) // ps]
            slots = np.arange(n) % ps
            for g in range(s.n_kv_heads):
                assert np.array_equal(kv.k[l, pages, g, slots, :], K[:, g, :]), (l, b, g)
                assert np.array_equal(kv.v[l, pages, g, slots, :], V[:, g, :]), (l, b, g)
        # everything else is untouched poison
        for arr in (kv.k[l], kv.v[l]):
            rest = arr.transpose(0, 2, 1, 3)[~written]   # [(page, slot)][head][d]
            assert np.all(rest == 0x7FC0)
    # K and V streams differ (a swap would go unnoticed otherwise)
    assert not np.array_equal(synth.kv_bits(s, 0, "k", 0, 0, 4), synth.kv_bits(s, 0, "v", 0, 0, 4))


def test_lm_logits_closed_form_through_the_final_gain():
    """x = (2, -2, 2, -2): mean(x^2) = 4, so rmsnorm(x) = (1, -1, 1, -1) * 2/sqrt(4 + eps); with the
    final gain (1.5, 0.75, 2, 1) the bf16-rounded input of the LM head is exactly
    (1.5, -0.75, 2, -1).  A 6 x 4 LM head of hand-picked rows then gives the logits by hand.
    A dropped gain, a skipped normalization, a transposed head or the embedding in place of the
    (untied) head all change them."""
    s = synth.ModelShape(n_layers=1, hidden=4, n_q_heads=1, n_kv_heads=1, head_dim=64,
                         n_experts=2, top_k=1, inter=4, vocab=6)
    head = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1], [1, 1, 1, 1], [2, -2, 0, 0]],
                    dtype=np.float64)
    gain = np.array([1.5, 0.75, 2.0, 1.0])

    def src(kind, layer, expert):
        if kind == synth.K_LM_HEAD:
            return O.f64_to_bf16_bits(head)
        if kind == synth.K_FINAL_NORM:
            return O.f64_to_bf16_bits(gain)
        if kind == synth.K_EMBED:
            return O.f64_to_bf16_bits(-head)     # untied: must not be read
        return synth.weight_bits(s, kind, layer, expert)

    W = O.Weights(s, source=src)
    got = O.lm_logits(W, np.array([2.0, -2.0, 2.0, -2.0]))
    assert np.array_equal(got, np.array([1.5, -0.75, 2.0, -1.0, 1.75, 4.5]))
    assert int(np.argmax(got)) == 5
    # the same input scaled by any positive factor normalizes to the same logits
    assert np.array_equal(O.lm_logits(W, np.array([0.5, -0.5, 0.5, -0.5])), got)


# ----------------------------------------------------------------------------
# sampling


def test_sampler_generator_is_splitmix64():
    """The sampler's generator reproduces SplitMix64's published reference outputs for seed 0
    (the sequence Vigna distributes with splitmix64.c), and output n depends on n alone."""
    got = [int(x) for x in O.splitmix64_at(0, np.arange(3))]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert int(O.splitmix64_at(0, np.array([2]))[0]) == got[2]


def test_gumbel_noise_moments():
    """Gumbel(0, 1): mean = Euler's constant, variance = pi^2 / 6.  Over 2^17 draws the sample
    moments lie within 5 standard errors.  A flipped sign (mean -0.577), log(u) for -log(-log(u))
    or a different scale all fail."""
    g = np.concatenate([O.gumbel_noise(11, pos, 0, 1, 4096) for pos in range(32)])
    n = g.size
    var = math.pi ** 2 / 6
    assert abs(g.mean() - np.euler_gamma) < 5 * math.sqrt(var / n)
    # variance of the sample variance: (mu4 - sigma^4) / n, mu4 = 27/5 sigma^4 for the Gumbel
    assert abs(g.var() - var) < 5 * math.sqrt((27 / 5 - 1) * var ** 2 / n)


def test_sampling_draws_softmax_over_temperature():
    """The Gumbel-max rule draws token i with probability softmax(z / T)_i: 40000 draws (one per
    position) of 5 tokens at T = 0.7 match those probabilities within 5 standard errors each, and
    a chi-square statistic stays under its 0.9999 quantile.  Dividing by T the wrong way (z * T),
    taking the argmin or a noise other than Gumbel each shift the frequencies far outside."""
    z = np.array([1.0, 0.2, -0.5, 1.4, 0.0])
    T = 0.7
    p = scipy.special.softmax(z / T)
    N = 40000
    counts = np.zeros(5)
    for pos in range(N):
        tok, _ = O.sample_token(z, T, 1234, pos, 0, 1)
        counts[tok] += 1
    f = counts / N
    assert np.all(np.abs(f - p) < 5 * np.sqrt(p * (1 - p) / N)), (f, p)
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    assert chi2 < scipy.stats.chi2.ppf(0.9999, df=4)


def test_sampling_special_cases():
    """T = 0 is the greedy argmax; a tiny T gives the argmax whenever the gap dwarfs T times the
    noise; the draw depends on the seed, the position and the batch slot, and repeats exactly."""
    rng = np.random.default_rng(5)
    z = rng.normal(size=1000)
    assert O.sample_token(z, 0.0, 7, 3, 0, 1)[0] == int(np.argmax(z))
    assert O.sample_token(z, 1e-9, 7, 3, 0, 1)[0] == int(np.argmax(z))
    a = O.sample_token(z, 1.0, 7, 3, 0, 2)
    assert a[0] == O.sample_token(z, 1.0, 7, 3, 0, 2)[0] and np.array_equal(a[1], O.sample_token(z, 1.0, 7, 3, 0, 2)[1])
    others = [O.sample_token(z, 1.0, s, p, b, 2)[1] for s, p, b in ((8, 3, 0), (7, 4, 0), (7, 3, 1))]
    for v in others:
        assert not np.array_equal(v, a[1])
    # slot b of max_batch 2 at position p is stream entry (2p + b) * V + i
    g = O.gumbel_noise(7, 3, 1, 2, 1000)
    n = np.arange(1000, dtype=np.uint64) + np.uint64((3 * 2 + 1) * 1000)
    u = ((O.splitmix64_at(7, n) >> np.uint64(11)).astype(np.float64) + 0.5) / 2.0 ** 53
    assert np.array_equal(g, -np.log(-np.log(u)))


# ----------------------------------------------------------------------------
# FP8 (E4M3) weights


def test_e4m3_decode_matches_torch_for_every_code():
    """The oracle's decoder, written from the format's definition, against torch's own
    float8_e4m3fn conversion (an independent implementation) on all 256 codes."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_lookup_is_the_decoder():
    codes = np.random.default_rng(3).integers(0, 256, size=(37, 129), dtype=np.uint8)
    a, b = O.e4m3_lookup(codes), O.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_e4m3_decode_spec_values():
    """Values fixed by the format: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest 448."""
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert O.e4m3_to_f64(np.uint8(c)) == v, hex(c)
    assert np.signbit(O.e4m3_to_f64(np.uint8(0x80))) and O.e4m3_to_f64(np.uint8(0x80)) == 0.0
    finite = O.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = finite[~np.isnan(finite)]
    assert not np.any(np.isinf(finite)) and finite.max() == 448.0
    # positive codes 0x00..0x7E are strictly increasing
    pos = O.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def _fp8(shape):
    from dataclasses import replace
    return replace(shape, weights="fp8")


def test_fp8_weights_are_codes_times_row_scales():
    """Weights.get of a quantized matrix = decode(code) * row scale, checked with torch's decoder in
    float64 (the product of a 4-significant-bit value and an fp32 scale is exact there)."""
    s = _fp8(synth.TINY)
    W = O.Weights(s)
    for kind, layer, expert in ((synth.K_WQKV, 1, None), (synth.K_W_DOWN, 0, 3), (synth.K_LM_HEAD, 0, None)):
        codes, scales = synth.weight_fp8(s, kind, layer, expert)
        dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64)
        ref = (dec * torch.from_numpy(scales).to(torch.float64)[..., None]).numpy()
        assert np.array_equal(W.get(kind, layer, expert), ref)
    # one expert's slice is that expert's rows of the whole tensor
    full = W.get(synth.K_W_GATE, 1)
    assert np.array_equal(full[5], O.Weights(s).get(synth.K_W_GATE, 1, 5))
    # router, gains and embedding stay bfloat16
    assert np.array_equal(W.get(synth.K_ROUTER, 0), O.bf16_to_f64(synth.weight_bits(s, synth.K_ROUTER, 0)))
    assert np.array_equal(W.get(synth.K_EMBED), O.bf16_to_f64(synth.weight_bits(s, synth.K_EMBED)))


def test_fp8_step_is_the_bf16_step_on_the_dequantized_weights():
    """The FP8 model changes nothing but the weight values: a step of it equals, bit for bit, a
    step of the bf16-format model whose quantized matrices are replaced by their dequantized values
    (computed here through torch's decoder)."""
    sq = _fp8(synth.TINY)
    Wq = O.Weights(sq)
    Wb = O.Weights(synth.TINY)
    for kind in synth.QUANT_KINDS:
        layers = range(sq.n_layers) if kind in synth.LAYER_KINDS else [0]
        for l in layers:
            codes, scales = synth.weight_fp8(sq, kind, l)
            dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64)
            sc = torch.from_numpy(scales).to(torch.float64).reshape(codes.shape[:-1] + (1,))
            Wb.cache[(kind, l, None)] = (dec * sc).numpy()
            if kind in (synth.K_W_GATE, synth.K_W_UP, synth.K_W_DOWN):
                for e in range(sq.n_experts):
                    Wb.cache[(kind, l, e)] = Wb.cache[(kind, l, None)][e]
    toks = [5, 77, 300]
    outs = []
    for W, s in ((Wq, sq), (Wb, synth.TINY)):
        kv = O.PagedKV(s, 4)
        pt = np.arange(4, dtype=np.int32)[None]
        for t, tok in enumerate(toks):
            out = O.decode_step(W, kv, [tok], pt, [t])
        outs.append(out.logits)
    assert np.array_equal(outs[0], outs[1])
    # and it differs from the bf16 model's own step (the weights did change)
    kv = O.PagedKV(synth.TINY, 4)
    W0 = O.Weights(synth.TINY)
    for t, tok in enumerate(toks):
        out0 = O.decode_step(W0, kv, [tok], np.arange(4, dtype=np.int32)[None], [t])
    assert not np.array_equal(out0.logits, outs[0])


def test_fp8_step_bytes_30b_shape():
    """Algorithmic bytes of the FP8 model: 1 byte per quantized weight plus 4 per quantized row."""
    s = _fp8(synth.MOE30B)
    H, I, E, V, L = s.hidden, s.inter, s.n_experts, s.vocab, s.n_layers
    qkv, ad = s.qkv_rows, s.attn_dim
    per_layer = (qkv * H + 4 * qkv) + (H * ad + 4 * H) + 2 * E * H + 8 * (2 * (I * H + 4 * I) + (H * I + 4 * H)) + 2 * H
    want = L * per_layer + (V * H + 4 * V) + 2 * H
    assert s.active_weight_bytes(8) == want
    assert abs(want / synth.MOE30B.active_weight_bytes(8) - 0.5) < 0.01


# ----------------------------------------------------------------------------
# FP4 (E2M1) weights


def test_e2m1_decode_table():
    """The OCP E2M1 values (the format's whole table: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = O.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == want and list(got[8:]) == [-v for v in want]
    assert np.signbit(got[8]) and got[8] == 0.0
    assert np.all(np.diff(got[:8]) > 0)


def test_fp4_unpack_nibble_order():
    """Byte j holds element 2j in its low nibble and 2j + 1 in its high nibble."""
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)   # elements: 1, 2, 7, 15
    assert O.fp4_unpack_f64(packed).tolist() == [[0.5, 1.0, 6.0, -6.0]]


def test_fp4_step_is_the_bf16_step_on_the_dequantized_weights():
    """As for FP8: a step of the FP4 model equals, bit for bit, the bf16-format step whose quantized
    matrices hold the dequantized values (decoded here from the table by hand)."""
    from dataclasses import replace
    sq = replace(synth.TINY, weights="fp4")
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    Wq, Wb = O.Weights(sq), O.Weights(synth.TINY)
    for kind in synth.QUANT_KINDS:
        for l in (range(sq.n_layers) if kind in synth.LAYER_KINDS else [0]):
            codes, scales = synth.weight_fp4(sq, kind, l)
            vals = np.stack([table[codes & 15], table[codes >> 4]], axis=-1).reshape(codes.shape[:-1] + (-1,))
            Wb.cache[(kind, l, None)] = vals * scales.astype(np.float64).reshape(codes.shape[:-1] + (1,))
            if kind in (synth.K_W_GATE, synth.K_W_UP, synth.K_W_DOWN):
                for e in range(sq.n_experts):
                    Wb.cache[(kind, l, e)] = Wb.cache[(kind, l, None)][e]
    outs = []
    for W, s in ((Wq, sq), (Wb, synth.TINY)):
        kv = O.PagedKV(s, 4)
        for t, tok in enumerate([5, 77, 300]):
            out = O.decode_step(W, kv, [tok], np.arange(4, dtype=np.int32)[None], [t])
        outs.append(out.logits)
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(Wq.get(synth.K_W_DOWN, 1, 3), Wq.get(synth.K_W_DOWN, 1)[3])


def test_fp4_step_bytes_30b_shape():
    from dataclasses import replace
    s = replace(synth.MOE30B, weights="fp4")
    H, I, E, V, L = s.hidden, s.inter, s.n_experts, s.vocab, s.n_layers
    qkv, ad = s.qkv_rows, s.attn_dim
    m = lambda r, c: r * c / 2 + 4 * r
    want = L * (m(qkv, H) + m(H, ad) + 2 * E * H + 8 * (2 * m(I, H) + m(H, I)) + 2 * H) + m(V, H) + 2 * H
    assert s.active_weight_bytes(8) == want


# --------------------------------------------------------------------------- top-p sampling

def _nucleus_brute(z_over_t: np.ndarray, p: float) -> set:
    """The nucleus by its definition, by trying every threshold: the largest value t among the
    scaled logits with mass(z >= t) >= p; the tokens at or above it."""
    q = np.exp(z_over_t - z_over_t.max())
    q = q / q.sum()
    best = None
    for t in sorted(set(z_over_t.tolist())):
        if q[z_over_t >= t].sum() >= p:
            best = t
    return set(np.flatnonzero(z_over_t >= best).tolist())


def test_top_p_nucleus_brute_force_on_small_vocabularies():
    rng = np.random.default_rng(21)
    for trial in range(300):
        V = int(rng.integers(1, 12))
        z = np.round(rng.standard_normal(V) * 2, 1)      # rounding makes ties common
        T = float(rng.choice([0.5, 1.0, 2.0]))
        p = float(rng.uniform(0.05, 0.999))
        got = set(np.flatnonzero(O.top_p_nucleus(z, T, p)).tolist())
        assert got == _nucleus_brute(z / T, p), (trial, z, T, p)


def test_top_p_closed_cases():
    z = np.array([3.0, 1.0, 1.0, -2.0])
    # p = 1: everything; p tiny: the top value only; mass of the top value exactly p: just it
    assert O.top_p_nucleus(z, 1.0, 1.0).all()
    assert O.top_p_nucleus(z, 1.0, 1e-9).tolist() == [True, False, False, False]
    q = np.exp(z - 3.0) / np.exp(z - 3.0).sum()
    assert O.top_p_nucleus(z, 1.0, q[0]).tolist() == [True, False, False, False]
    # just above the top mass: the tied pair comes in together
    assert O.top_p_nucleus(z, 1.0, q[0] + 1e-12).tolist() == [True, True, True, False]


def test_top_p_sampling_reduces_to_plain_and_greedy():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal(1000) * 3
    for pos in range(5):
        tok1, _ = O.sample_token_top_p(logits, 0.8, 1.0, 0x5EED, pos, 0, 1)
        tok0, _ = O.sample_token(logits, 0.8, 0x5EED, pos, 0, 1)
        assert tok1 == tok0
        tokg, nuc = O.sample_token_top_p(logits, 0.8, 1e-12, 0x5EED, pos, 0, 1)
        assert tokg == int(np.argmax(logits)) and nuc.sum() == 1


def test_top_p_draw_frequencies_follow_the_renormalized_distribution():
    """Many draws (different positions) from a small vocabulary: frequencies within 5 sigma of
    softmax(z / T) restricted to the nucleus and renormalized."""
    z = np.array([2.0, 1.5, 1.0, 0.0, -1.0, -3.0])
    T, p, n = 1.0, 0.8, 20000
    nuc = O.top_p_nucleus(z, T, p)
    q = np.where(nuc, np.exp(z / T), 0.0)
    q = q / q.sum()
    counts = np.zeros(z.size)
    for pos in range(n):
        counts[O.sample_token_top_p(z, T, p, 7, pos, 0, 1)[0]] += 1
    sigma = np.sqrt(n * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - n * q) <= 5 * sigma + 1e-9), (counts, n * q)
    assert np.all(counts[~nuc] == 0)
