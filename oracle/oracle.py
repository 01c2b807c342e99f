"""CPU oracle for one decode step of the parallel-block MoE decoder.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It shares no
code with the GPU path; both take their inputs from the ``synth`` generator.

What it computes is the decode forward pass the cited pages describe
(Cohere megakernel articles: the latestnews.news page, second paragraph, lists
the per-step weight and KV streaming; the ainews.surl.tw page, second
paragraph, says attention and MoE run concurrently from the same normalized
input; the aiweekly.co page, second paragraph, names the fused operation kinds:
QKV projection, attention, MoE routing, gather, GEMMs and normalization).  The
pages print no formulas, so each op below is its textbook definition, written
plainly, in float64, with bfloat16 rounding only at the points where the
method stores bfloat16 values:

* weights, KV cache entries, the normalized input ``xn``, q/k/v after the
  rotation, the attention output and the expert hidden vector ``h``;
* router logits are rounded to float32 before the top-k decision (the
  precision in which the GPU takes that integer decision); everything else,
  including the residual stream and the logits, stays float64.

Readings where the pages are silent (each also listed in the design notes):
parallel block ``x <- (x + attn) + moe`` with one RMSNorm per layer; rotate-half
RoPE with ``inv_freq_i = theta^(-2i/d)``; scale ``1/sqrt(d)``; q head ``h`` uses
kv head ``h // (n_q / n_kv)``; top-k by (value desc, index asc) and softmax over
the selected logits; SwiGLU experts ``Wd (silu(Wg xn) * (Wu xn))``; the new
token's K/V are written to slot ``seq_len`` before attention runs over
``0..seq_len`` inclusive; untied LM head after a final RMSNorm; greedy argmax
with ties to the lowest id; sampling at temperature T by the Gumbel-max rule
with SplitMix64 noise keyed by (seed, position, batch slot, token id).

FP8 weights (a model whose shape says ``weights="fp8"``): the pages list FP8
weight streaming as a next step (aiweekly.co page, sixth paragraph) and fix no
format.  The reading taken: the large streamed matrices (LM head, Wqkv, Wo,
expert gate/up/down) are OCP E4M3 codes times one fp32 scale per output row;
the weight value is decode(code) * scale, exactly, in float64, and every
product then runs as with bfloat16 weights.  Router, norm gains and embedding
stay bfloat16.  FP4 weights (``weights="fp4"``) are the same with OCP E2M1
codes, two a byte (the even element in the low nibble).

Top-p sampling (top_p_nucleus, sample_token_top_p): the pages call the
engine's sampling options incomplete (ainews.surl.tw page, fourth paragraph)
and define none.  The reading taken: at temperature T the nucleus is every
token whose scaled logit is at least the largest threshold keeping mass
>= top_p of softmax(logits / T), tokens tied at the threshold included, and
the draw is the Gumbel-max rule restricted to the nucleus.

Sequential block (a shape with ``block="sequential"``): the pages tailor the
engine to one model and ask whether it generalizes to other MoE models
(ainews.surl.tw page, fourth paragraph), naming none.  The reading taken: the
common pre-norm decoder layer of such models, attention then MoE, each behind
its own RMSNorm: x' = x + Wo attn(bf16(rmsnorm(x, g_attn))), then
x <- x' + moe(bf16(rmsnorm(x', g_moe))), with the same shapes, rounding points
and routing as the parallel block.

Parity unpinned: the composed multi-layer logits have no closed form; they
are pinned only through the pinned ops and the whole-step invariants in
``tests/test_oracle_pins.py``.  The ulp behaviour of exp/silu is covered only
by the comparison tolerance.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import synth

# ----------------------------------------------------------------------------
# bfloat16 representation


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP E4M3 codes (uint8) as float64: sign bit 7, exponent bits 6..3 with bias
    7, mantissa bits 2..0; exponent field 0 holds the subnormals m * 2^-9; 0x7F and 0xFF are NaN;
    there are no infinities."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 0xF) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP E2M1 codes (4-bit, in uint8) as float64: sign bit 3, exponent bits 2..1
    with bias 1, mantissa bit 0; exponent field 0 holds the subnormal m * 0.5; no NaN, no infinity."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2((e - 1).astype(np.float64)))
    return sign * mag


def fp4_unpack_f64(packed: np.ndarray) -> np.ndarray:
    """Values of packed E2M1 codes: byte j holds element 2j (low nibble) and 2j + 1 (high nibble);
    the last axis doubles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],))
    out[..., 0::2] = _E2M1_VALUES[p & 0xF]
    out[..., 1::2] = _E2M1_VALUES[p >> 4]
    return out


_E2M1_VALUES = e2m1_to_f64(np.arange(16, dtype=np.uint8))

# the 256 values of the definition above, for decoding whole weight tensors by lookup
_E4M3_VALUES = e4m3_to_f64(np.arange(256, dtype=np.uint8))


def e4m3_lookup(codes: np.ndarray) -> np.ndarray:
    """e4m3_to_f64 by a table of its 256 values (the same numbers, one gather per code)."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits: with x = m * 2^e, 0.5 <= |m| < 1, the
    representable neighbours are multiples of 2^(e-8) (2^-133 below the
    smallest normal 2^-126).  np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    return np.where(np.abs(q) > _BF16_MAX, np.copysign(np.inf, x), q)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of values that are already bfloat16-representable."""
    r = round_bf16(x)
    b = r.astype(np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# ops


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x_i / sqrt(mean(x^2) + eps) * g_i."""
    return x * (1.0 / np.sqrt(np.mean(x * x) + eps)) * g


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    return theta ** (-(2.0 * np.arange(d // 2, dtype=np.float64)) / d)


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of a [heads][d] array at position ``pos``.

    Pair (i, i + d/2) is rotated by the angle pos * theta^(-2i/d).
    """
    d = v.shape[-1]
    ang = pos * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def topk_desc(r: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values, ordered by (value desc, index asc)."""
    order = sorted(range(len(r)), key=lambda i: (-float(r[i]), i))
    return np.array(order[:k], dtype=np.int64)


def attention_head(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(K q / sqrt(d)) V for one query vector over rows of K, V."""
    s = (K @ q) / np.sqrt(q.shape[0])
    p = softmax(s)
    return p @ V


# ----------------------------------------------------------------------------
# weights and KV cache


class Weights:
    """Model weights as float64, generated from the synth recipe and cached.

    ``budget_bytes`` bounds the cache of float64 matrices; expert slices are
    regenerated on demand once the budget is used.
    """

    def __init__(self, shape: synth.ModelShape, budget_bytes: float = 6e9, source=None):
        self.shape = shape
        self.budget = budget_bytes
        self.used = 0
        self.cache: dict = {}
        self.source = source or (lambda kind, layer, expert: synth.weight_bits(shape, kind, layer, expert))
        self.source_fp8 = lambda kind, layer, expert: synth.weight_fp8(shape, kind, layer, expert)

    def get(self, kind: int, layer: int = 0, expert: int | None = None) -> np.ndarray:
        key = (kind, layer, expert)
        w = self.cache.get(key)
        if w is None:
            if self.shape.quantized(kind) and self.shape.weights == "fp4":
                # FP4 weights: each row's codes (two a byte) times the row's scale
                codes, scales = synth.weight_fp4(self.shape, kind, layer, expert)
                w = fp4_unpack_f64(codes) * scales.astype(np.float64).reshape(codes.shape[:-1] + (1,))
            elif self.shape.quantized(kind):
                # FP8 weights: each row's codes times the row's scale
                codes, scales = self.source_fp8(kind, layer, expert)
                w = e4m3_lookup(codes) * scales.astype(np.float64).reshape(codes.shape[:-1] + (1,))
            else:
                w = bf16_to_f64(self.source(kind, layer, expert))
            if self.used + w.nbytes <= self.budget:
                self.cache[key] = w
                self.used += w.nbytes
        return w


class PagedKV:
    """Paged K/V pools: per layer ``[num_pages][n_kv][page_size][d]`` bfloat16 bits.

    layers: the layers held (default all); the others cannot be written or read.
    """

    def __init__(self, shape: synth.ModelShape, num_pages: int, layers=None):
        s = shape
        self.shape = s
        self.layers = list(range(s.n_layers)) if layers is None else sorted(set(int(l) for l in layers))
        self._at = {l: i for i, l in enumerate(self.layers)}
        dims = (len(self.layers), num_pages, s.n_kv_heads, s.page_size, s.head_dim)
        self.k = np.full(dims, 0x7FC0, dtype=np.uint16)   # NaN: unwritten slots poison any stray read
        self.v = np.full(dims, 0x7FC0, dtype=np.uint16)

    def slots(self, page_table_row: np.ndarray, pos: np.ndarray):
        """(physical page, offset in page) of logical positions ``pos`` through one page-table row."""
        ps = self.shape.page_size
        pos = np.asarray(pos, dtype=np.int64)
        page = np.asarray(page_table_row, dtype=np.int64)[pos // ps]
        if np.any(page < 0) or np.any(page >= self.k.shape[1]):
            raise IndexError("page id out of range in page table")
        return page, pos % ps

    def write(self, layer: int, page_table_row: np.ndarray, pos: int, k_bits: np.ndarray, v_bits: np.ndarray):
        page, o = self.slots(page_table_row, [pos])
        i = self._at[layer]
        self.k[i, page[0], :, o[0], :] = k_bits
        self.v[i, page[0], :, o[0], :] = v_bits

    def gather(self, layer: int, page_table_row: np.ndarray, n: int, g: int):
        """K, V rows (float64 [n][d]) of kv head ``g`` for logical positions 0..n-1."""
        page, o = self.slots(page_table_row, np.arange(n))
        i = self._at[layer]
        return bf16_to_f64(self.k[i, page, g, o]), bf16_to_f64(self.v[i, page, g, o])

    def fill_synthetic(self, page_table: np.ndarray, context: list):
        """Fill positions 0..context[b]-1 of every sequence from the synth KV recipe."""
        s = self.shape
        ps = s.page_size
        for b, n in enumerate(context):
            for i, layer in enumerate(self.layers):
                K = synth.kv_bits(s, layer, "k", b, 0, n)
                V = synth.kv_bits(s, layer, "v", b, 0, n)
                for t0 in range(0, n, ps):
                    t1 = min(n, t0 + ps)
                    page = int(page_table[b, t0 // ps])
                    self.k[i, page, :, : t1 - t0, :] = K[t0:t1].transpose(1, 0, 2)
                    self.v[i, page, :, : t1 - t0, :] = V[t0:t1].transpose(1, 0, 2)


# ----------------------------------------------------------------------------
# one decode step


@dataclass
class StepOut:
    logits: np.ndarray                      # [B][V] float64
    router_logits: np.ndarray               # [L][B][E] float32 values
    sel: np.ndarray                         # [L][B][k] int64
    margin: np.ndarray                      # [L][B] float: r_(k) - r_(k+1) (inf when k == E)
    next_token: np.ndarray                  # [B] int64 greedy argmax
    top2_gap: np.ndarray                    # [B] logit gap between best and second best
    sel_alt: np.ndarray = None              # [L][B][k] the set with the k-th and (k+1)-th exchanged
    trace: dict = field(default_factory=dict)


ROUTE_TIE = 1e-3   # router margin below which either expert set is a correct result


@dataclass
class LayerOut:
    x: np.ndarray          # [H] float64: the residual leaving the layer
    r: np.ndarray          # [E] float32 values: router logits
    sel: np.ndarray        # [k] experts in slot order
    sel_alt: np.ndarray    # [k] the set with the k-th and (k+1)-th exchanged (or None when k == E)
    margin: float          # r_(k) - r_(k+1)
    parts: dict            # intermediates: xn, q16, k16, v16, a16, attn, moe, h16, w


@dataclass
class MoeOut:
    r: np.ndarray          # [E] float32 values: router logits
    sel: np.ndarray        # [k] experts in slot order
    sel_alt: np.ndarray    # [k] the set with the k-th and (k+1)-th exchanged (or None when k == E)
    margin: float          # r_(k) - r_(k+1)
    w: np.ndarray          # [k] softmax of the selected logits
    moe: np.ndarray        # [H] weighted sum of the experts' outputs
    h16: np.ndarray        # [k][I] the experts' bf16 hidden vectors


def moe_path(W: Weights, l: int, xm: np.ndarray, take_alt: bool = False) -> MoeOut:
    """Layer l's MoE path from its normalized input xm: router, top-k by (value desc, index asc),
    softmax over the selected logits, SwiGLU experts, weighted sum.  take_alt: take the other
    correct routing at a near-tie of the k-th and (k+1)-th router logits (checked)."""
    s = W.shape
    H, E, k = s.hidden, s.n_experts, s.top_k
    r = (W.get(synth.K_ROUTER, l) @ xm).astype(np.float32)
    sel = topk_desc(r, k)
    alt = None
    if k < E:
        ext = topk_desc(r, k + 1)
        alt = np.concatenate([ext[: k - 1], ext[k:]])
        if take_alt:
            if not float(r[ext[k - 1]]) - float(r[ext[k]]) <= ROUTE_TIE:
                raise ValueError(f"layer {l}: no routing near-tie to take the alternative of")
            sel = alt
    wsel = softmax(r[sel].astype(np.float64))
    moe = np.zeros(H)
    hs = []
    for j in range(k):
        e = int(sel[j])
        gate = W.get(synth.K_W_GATE, l, e) @ xm
        up = W.get(synth.K_W_UP, l, e) @ xm
        h16 = round_bf16(silu(gate) * up)
        hs.append(h16)
        moe = moe + wsel[j] * (W.get(synth.K_W_DOWN, l, e) @ h16)
    srt = np.sort(r.astype(np.float64))[::-1]
    margin = srt[k - 1] - srt[k] if k < E else np.inf
    return MoeOut(r, sel, alt, margin, wsel, moe, np.stack(hs))


def layer_forward(W: Weights, kv: PagedKV, l: int, x: np.ndarray, p: int, pt: np.ndarray,
                  take_alt: bool = False) -> LayerOut:
    """One decoder layer for one sequence whose new token sits at position p.

    Parallel block from one normalized input: attention (QKV, rotary, the new
    K/V written at p, attention over 0..p, O projection) and the MoE path
    (router, top-k, softmax over the selected logits, SwiGLU experts, weighted
    sum), then x <- (x + attn) + moe.  Sequential block (shape.block ==
    "sequential"): attention as above, then the MoE path from its own norm of
    the updated residual, x' = x + attn, xm = bf16(rmsnorm(x', g_moe)), and
    x <- x' + moe(xm).  take_alt: take the other correct routing at a
    near-tie of the k-th and (k+1)-th router logits (checked).
    """
    s = W.shape
    H, d, E, k = s.hidden, s.head_dim, s.n_experts, s.top_k
    nq, nkv = s.n_q_heads, s.n_kv_heads
    group = nq // nkv
    xn = round_bf16(rmsnorm(x, W.get(synth.K_ATTN_NORM, l), s.rms_eps))
    # attention path
    qkv = W.get(synth.K_WQKV, l) @ xn
    q = qkv[: nq * d].reshape(nq, d)
    kk = qkv[nq * d: (nq + nkv) * d].reshape(nkv, d)
    vv = qkv[(nq + nkv) * d:].reshape(nkv, d)
    q16 = round_bf16(rope(q, p, s.rope_theta))
    k16 = round_bf16(rope(kk, p, s.rope_theta))
    v16 = round_bf16(vv)
    kv.write(l, pt, p, f64_to_bf16_bits(k16), f64_to_bf16_bits(v16))
    o = np.zeros((nq, d))
    for g in range(nkv):
        K, V = kv.gather(l, pt, p + 1, g)
        for h in range(g * group, (g + 1) * group):
            o[h] = attention_head(q16[h], K, V)
    a16 = round_bf16(o.reshape(-1))
    attn = W.get(synth.K_WO, l) @ a16
    # MoE path: from the same normalized input (parallel block), or from the norm of x + attn
    # with the MoE path's own gain (sequential block)
    if s.sequential:
        xm = round_bf16(rmsnorm(x + attn, W.get(synth.K_MOE_NORM, l), s.rms_eps))
    else:
        xm = xn
    m = moe_path(W, l, xm, take_alt)
    parts = {"xn": xn, "xm": xm, "q16": q16, "k16": k16, "v16": v16, "a16": a16, "attn": attn, "moe": m.moe,
             "h16": m.h16, "w": m.w}
    return LayerOut((x + attn) + m.moe, m.r, m.sel, m.sel_alt, m.margin, parts)


def lm_logits(W: Weights, x: np.ndarray) -> np.ndarray:
    """Final RMSNorm, then the LM head."""
    xf = round_bf16(rmsnorm(x, W.get(synth.K_FINAL_NORM), W.shape.rms_eps))
    return W.get(synth.K_LM_HEAD) @ xf


def decode_step(W: Weights, kv: PagedKV, tokens, page_table, seq_lens, trace: bool = False,
                route_alt=None) -> StepOut:
    """One decode step for a ragged batch.

    tokens[b] is the new token of sequence b; seq_lens[b] tokens are already in
    the cache, so the new token sits at position p = seq_lens[b].  Its K/V are
    written to the cache, and attention runs over positions 0..p.

    route_alt: (layer, b) pairs at which the step takes the other correct
    routing: where the k-th and (k+1)-th router logits lie within ROUTE_TIE
    of each other, a decoder computing in a different precision may pick
    either, so the set with those two exchanged is also a correct result.
    Only valid at such near-ties (checked).
    """
    route_alt = route_alt or set()
    s = W.shape
    L, E, k = s.n_layers, s.n_experts, s.top_k
    B = len(tokens)
    logits = np.zeros((B, s.vocab))
    rl = np.zeros((L, B, E), dtype=np.float32)
    sel_all = np.zeros((L, B, k), dtype=np.int64)
    sel_alt = np.full((L, B, k), -1, dtype=np.int64)
    margin = np.zeros((L, B))
    tr: dict = {}
    for b in range(B):
        p = int(seq_lens[b])
        pt = np.asarray(page_table[b])
        x = W.get(synth.K_EMBED)[int(tokens[b])].copy()
        for l in range(L):
            out = layer_forward(W, kv, l, x, p, pt, take_alt=(l, b) in route_alt)
            rl[l, b] = out.r
            sel_all[l, b] = out.sel
            if out.sel_alt is not None:
                sel_alt[l, b] = out.sel_alt
            margin[l, b] = out.margin
            if trace:
                tr.setdefault("x_in", {})[(l, b)] = x
                for name, v in out.parts.items():
                    tr.setdefault(name, {})[(l, b)] = v
            x = out.x
        logits[b] = lm_logits(W, x)
        if trace:
            tr.setdefault("x_final", {})[b] = x
    nxt = np.argmax(logits, axis=1)
    srt = np.sort(logits, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    return StepOut(logits, rl, sel_all, margin, nxt, gap, sel_alt, tr)


def prefill_as_decode(W: Weights, kv: PagedKV, prompt, page_table_row) -> StepOut:
    """Feed prompt tokens one decode step at a time (positions 0..n-1) for one sequence."""
    out = None
    pt = np.asarray(page_table_row)[None, :]
    for t, tok in enumerate(prompt):
        out = decode_step(W, kv, [int(tok)], pt, [t])
    return out


# ----------------------------------------------------------------------------
# speed-of-light model


# ----------------------------------------------------------------------------
# sampling (the pages call the engine's sampling options incomplete: the
# ainews.surl.tw page, its paragraph on limitations; the reading here is
# temperature sampling, softmax(logits / T), drawn by the Gumbel-max rule)

_GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def splitmix64_at(seed: int, n: np.ndarray) -> np.ndarray:
    """Output n (0-based) of SplitMix64 seeded with `seed` (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", 2014): the state after n + 1 steps of adding the golden gamma
    0x9E3779B97F4A7C15, through the finalizer z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,
    z *= 0x94D049BB133111EB, z ^= z >> 31 (all arithmetic mod 2^64)."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _M64) + (n + np.uint64(1)) * np.uint64(_GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def gumbel_noise(seed: int, pos: int, b: int, max_batch: int, vocab: int) -> np.ndarray:
    """Gumbel(0, 1) noise for every vocabulary entry i of batch slot b whose step input token sits at
    position `pos`: u = (top 53 bits of output n + 1/2) / 2^53 with n = (pos * max_batch + b) * vocab + i,
    which lies in (0, 1), and g = -log(-log(u))."""
    n = (np.uint64(pos) * np.uint64(max_batch) + np.uint64(b)) * np.uint64(vocab) + np.arange(vocab, dtype=np.uint64)
    u = ((splitmix64_at(seed, n) >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    return -np.log(-np.log(u))


def sample_token(logits: np.ndarray, temperature: float, seed: int, pos: int, b: int, max_batch: int):
    """The sampled next token and the perturbed scores: argmax_i (logits_i / T + g_i) (ties to the
    lowest id), which draws i with probability softmax(logits / T)_i; T = 0 is the greedy argmax."""
    z = np.asarray(logits, dtype=np.float64)
    if temperature == 0:
        return int(np.argmax(z)), z
    v = z / temperature + gumbel_noise(seed, pos, b, max_batch, z.size)
    return int(np.argmax(v)), v


def top_p_nucleus(logits: np.ndarray, temperature: float, top_p: float) -> np.ndarray:
    """Boolean mask of the nucleus: with q = softmax(logits / T), every token whose scaled logit is
    at least the largest threshold tau (a scaled logit value) such that the tokens at or above tau
    hold mass >= top_p.  Tokens tied at tau are all in (the nucleus is a set of values, not of
    ids).  top_p >= 1: every token."""
    z = np.asarray(logits, dtype=np.float64) / temperature
    if top_p >= 1.0:
        return np.ones(z.size, dtype=bool)
    q = np.exp(z - np.max(z))
    q = q / q.sum()
    vals, inv = np.unique(-z, return_inverse=True)     # distinct scaled logits, largest first
    mass = np.bincount(inv, weights=q)                 # probability of each distinct value
    k = int(np.searchsorted(np.cumsum(mass), top_p))   # first value whose cumulative mass >= top_p
    k = min(k, vals.size - 1)
    return z >= -vals[k]


def sample_token_top_p(logits: np.ndarray, temperature: float, top_p: float, seed: int, pos: int, b: int,
                       max_batch: int):
    """Top-p sampling by the Gumbel-max rule restricted to the nucleus: argmax over the nucleus of
    logits_i / T + g_i (ties to the lowest id), which draws from softmax(logits / T) renormalized
    over the nucleus.  Returns (token, nucleus mask)."""
    nuc = top_p_nucleus(logits, temperature, top_p)
    v = np.asarray(logits, dtype=np.float64) / temperature + gumbel_noise(seed, pos, b, max_batch, len(logits))
    v = np.where(nuc, v, -np.inf)
    return int(np.argmax(v)), nuc


def sol_tokens_per_s(bandwidth_bytes_per_s: float, bytes_per_step: float, batch: int = 1) -> float:
    """Bandwidth bound on decode throughput: batch * bandwidth / bytes streamed per step."""
    return batch * bandwidth_bytes_per_s / bytes_per_step


def step_bytes(shape: synth.ModelShape, seq_lens, distinct_experts_per_layer: float) -> float:
    """Algorithmic HBM bytes read by one step: active weights, embedding rows and KV for 0..p."""
    w = shape.active_weight_bytes(distinct_experts_per_layer)
    w += 2.0 * shape.hidden * len(seq_lens)
    per_tok_kv = shape.kv_bytes_per_token()
    kv = sum(per_tok_kv * (int(p) + 1) for p in seq_lens)
    return w + kv
