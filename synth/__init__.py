"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Nothing here computes any part of the decode step.  The module turns
(seed, tensor id, element index) into weights, prompt tokens, KV contents,
page permutations and sequence lengths, so that the oracle and the GPU path
receive identical inputs without either one producing them for the other.

Two implementations of one generator spec (header of ``synth.c``):

* ``libsynth.so`` (plain C + OpenMP): the fast path used by everything;
* ``*_np`` functions here: a vectorised numpy mirror, used only to pin the C
  library bit for bit in the tests.

Tensor ids: ``kind << 20 | index`` with the kinds below.  Expert tensors are
generated whole (``[E][rows][cols]``) so one expert is a contiguous element
range; KV contents are indexed by logical position, never by physical page,
so paged and contiguous layouts see the same values.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

GOLDEN = 0x9E3779B97F4A7C15
TID_MUL = 0xD1B54A32D192ED03
_M64 = (1 << 64) - 1

# tensor kinds
K_EMBED, K_LM_HEAD, K_FINAL_NORM = 1, 2, 3
K_ATTN_NORM, K_WQKV, K_WO, K_ROUTER, K_W_GATE, K_W_UP, K_W_DOWN = 10, 11, 12, 13, 14, 15, 16
K_MOE_NORM = 17   # sequential block only: the gain of the norm in front of the MoE path
K_K_CACHE, K_V_CACHE = 20, 21
K_PROMPT, K_PAGE_PERM, K_SEQ_LENS = 30, 31, 32

# seeds (the recipe fixes these; any other value gives another workload)
SEED_WEIGHTS, SEED_PROMPT, SEED_PAGES, SEED_KV, SEED_LENS = 0, 1, 2, 3, 4
WEIGHT_SIGMA = 0.02
GAIN_SIGMA = 0.02
KV_SIGMA = 1.0


def tid(kind: int, index: int = 0) -> int:
    return (kind << 20) | index


# ----------------------------------------------------------------------------
# C library


def build_lib(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-std=c99",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_normal_scale.restype = ctypes.c_float
        L.synth_normal_scale.argtypes = [ctypes.c_double]
        for name in ("synth_normal_bf16", "synth_gain_bf16"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [u64, u64, u64, u64, ctypes.c_double, p]
        L.synth_fp8_codes.restype = None
        L.synth_fp8_codes.argtypes = [u64, u64, u64, u64, p]
        L.synth_fp8_scales.restype = None
        L.synth_fp8_scales.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, p]
        L.synth_e4m3_rne.restype = ctypes.c_uint8
        L.synth_e4m3_rne.argtypes = [ctypes.c_float]
        L.synth_fp4_codes.restype = None
        L.synth_fp4_codes.argtypes = [u64, u64, u64, u64, p]
        L.synth_fp4_scales.restype = None
        L.synth_fp4_scales.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, p]
        L.synth_e2m1_rne.restype = ctypes.c_uint8
        L.synth_e2m1_rne.argtypes = [ctypes.c_float]
        L.synth_uniform_u32.restype = None
        L.synth_uniform_u32.argtypes = [u64, u64, u64, u64, ctypes.c_uint32, p]
        L.synth_permutation.restype = None
        L.synth_permutation.argtypes = [u64, u64, ctypes.c_uint32, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_bf16(seed: int, t: int, start: int, count: int, sigma: float, out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits (uint16) of N(0, sigma^2) deviates ``start .. start+count-1`` of stream (seed, t)."""
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == count
    lib().synth_normal_bf16(seed, t, start, count, sigma, _ptr(out))
    return out


def normal_bf16_into_ptr(seed: int, t: int, start: int, count: int, sigma: float, ptr: int) -> None:
    """Same as :func:`normal_bf16`, written to raw host memory ``ptr`` (e.g. a pinned torch buffer)."""
    lib().synth_normal_bf16(seed, t, start, count, sigma, ptr)


def gain_bf16(seed: int, t: int, start: int, count: int, sigma: float) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    lib().synth_gain_bf16(seed, t, start, count, sigma, _ptr(out))
    return out


def uniform_u32(seed: int, t: int, start: int, count: int, n: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint32)
    lib().synth_uniform_u32(seed, t, start, count, n, _ptr(out))
    return out


def permutation(seed: int, t: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, t, n, _ptr(out))
    return out


# ----------------------------------------------------------------------------
# numpy mirror (pins the C library)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def key_int(seed: int, t: int) -> int:
    return _mix64_int(_mix64_int(seed + GOLDEN) ^ ((t * TID_MUL) & _M64))


def words_np(seed: int, t: int, start: int, count: int) -> np.ndarray:
    k = np.uint64(key_int(seed, t))
    i = np.arange(start, start + count, dtype=np.uint64) + np.uint64(1)
    with np.errstate(over="ignore"):
        return _mix64_np(k + i * np.uint64(GOLDEN))


def _irwin_hall_np(w: np.ndarray) -> np.ndarray:
    m = np.uint64(0xFFFF)
    s = (w & m).astype(np.int64) + ((w >> np.uint64(16)) & m).astype(np.int64) \
        + ((w >> np.uint64(32)) & m).astype(np.int64) + ((w >> np.uint64(48)) & m).astype(np.int64)
    return s - 131070


def _f32_to_bf16_np(f: np.ndarray) -> np.ndarray:
    u = f.astype(np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def normal_scale_np(sigma: float) -> np.float32:
    return np.float32(sigma / math.sqrt((65536.0 * 65536.0 - 1.0) / 3.0))


def normal_bf16_np(seed: int, t: int, start: int, count: int, sigma: float) -> np.ndarray:
    with np.errstate(over="ignore"):
        s = _irwin_hall_np(words_np(seed, t, start, count)).astype(np.float32)
    return _f32_to_bf16_np(s * normal_scale_np(sigma))


def gain_bf16_np(seed: int, t: int, start: int, count: int, sigma: float) -> np.ndarray:
    with np.errstate(over="ignore"):
        s = _irwin_hall_np(words_np(seed, t, start, count)).astype(np.float32)
    return _f32_to_bf16_np(np.float32(1.0) + s * normal_scale_np(sigma))


def e4m3_rne_np(f: np.ndarray) -> np.ndarray:
    """numpy mirror of the generator's E4M3 encoder (nearest code, ties to even, saturating)."""
    f = np.asarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    sign = ((u >> np.uint64(24)) & np.uint64(0x80)).astype(np.uint8)
    u = u & np.uint64(0x7FFFFFFF)
    a = u.astype(np.uint32).view(np.float32)
    sub = np.rint(a * np.float32(512.0)).astype(np.int64)
    r = u + np.uint64(0x7FFFF) + ((u >> np.uint64(20)) & np.uint64(1))
    e = (r >> np.uint64(23)).astype(np.int64) - 127
    nrm = np.minimum(((e + 7) << 3) | ((r >> np.uint64(20)) & np.uint64(7)).astype(np.int64), 0x7E)
    with np.errstate(invalid="ignore"):
        code = np.where(~(a < np.float32(464.0)), 0x7E, np.where(a < np.float32(0.015625), sub, nrm))
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def fp8_codes_np(seed: int, t: int, start: int, count: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        s = _irwin_hall_np(words_np(seed, t, start, count)).astype(np.float32)
    return e4m3_rne_np(s * normal_scale_np(32.0))


def fp8_scales_np(seed: int, t: int, start: int, count: int) -> np.ndarray:
    g = gain_bf16_np(seed, t, start, count, GAIN_SIGMA).astype(np.uint32) << np.uint32(16)
    return np.float32(WEIGHT_SIGMA / 32.0) * g.view(np.float32)


def e2m1_rne_np(f: np.ndarray) -> np.ndarray:
    """numpy mirror of the generator's E2M1 encoder (nearest code, ties to even, saturating at 6)."""
    f = np.asarray(f, dtype=np.float32)
    a = np.abs(f)
    m = np.select([a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0], [0, 1, 2, 3, 4, 5, 6], 7)
    sign = np.where(np.signbit(f), 8, 0)
    return (m | sign).astype(np.uint8)


def fp4_codes_np(seed: int, t: int, start: int, count: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        s = _irwin_hall_np(words_np(seed, t, start, count)).astype(np.float32)
    c = e2m1_rne_np(s * normal_scale_np(1.5))
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def fp4_scales_np(seed: int, t: int, start: int, count: int) -> np.ndarray:
    g = gain_bf16_np(seed, t, start, count, GAIN_SIGMA).astype(np.uint32) << np.uint32(16)
    return np.float32(WEIGHT_SIGMA / 1.5) * g.view(np.float32)


def uniform_u32_np(seed: int, t: int, start: int, count: int, n: int) -> np.ndarray:
    w = words_np(seed, t, start, count)
    hi = (w >> np.uint64(32))
    with np.errstate(over="ignore"):
        return ((hi * np.uint64(n)) >> np.uint64(32)).astype(np.uint32)


def permutation_np(seed: int, t: int, n: int) -> np.ndarray:
    a = list(range(n))
    k = key_int(seed, t)
    for i in range(n - 1, 0, -1):
        w = _mix64_int(k + (i + 1) * GOLDEN)
        j = ((w >> 32) * (i + 1)) >> 32
        a[i], a[j] = a[j], a[i]
    return np.array(a, dtype=np.int32)


# ----------------------------------------------------------------------------
# Model shapes and workloads


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    inter: int
    vocab: int
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-6
    page_size: int = 16
    weights: str = "bf16"   # "bf16"; "fp8" / "fp4": the QUANT_KINDS matrices as E4M3 / E2M1 codes + fp32 row scales
    block: str = "parallel"  # "parallel": attention and MoE from one normalized input; "sequential": the MoE
                             # path normalizes (x + attention) with its own gain (K_MOE_NORM)

    @property
    def sequential(self) -> bool:
        return self.block == "sequential"

    def layer_kinds(self) -> tuple:
        """Per-layer weight kinds: LAYER_KINDS, plus K_MOE_NORM in the sequential block."""
        return LAYER_KINDS + ((K_MOE_NORM,) if self.sequential else ())

    def bind_order(self) -> list:
        """(kind, layer) of every weight tensor in the order the library binds them: the global
        tensors, each layer's LAYER_KINDS, then (sequential block) every layer's K_MOE_NORM."""
        order = [(k, 0) for k in GLOBAL_KINDS] + [(k, l) for l in range(self.n_layers) for k in LAYER_KINDS]
        if self.sequential:
            order += [(K_MOE_NORM, l) for l in range(self.n_layers)]
        return order

    def quantized(self, kind: int) -> bool:
        return self.weights in ("fp8", "fp4") and kind in QUANT_KINDS

    def weight_nbytes(self, kind: int) -> int:
        """Bytes of one weight tensor as bound: bf16, or (quantized) codes then one fp32 scale per row."""
        shp = self.weight_shape(kind)
        n = int(np.prod(shp))
        if self.quantized(kind):
            return (n if self.weights == "fp8" else n // 2) + 4 * (n // shp[-1])
        return 2 * n

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def attn_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    def weight_shape(self, kind: int) -> tuple:
        H, E, I = self.hidden, self.n_experts, self.inter
        return {
            K_EMBED: (self.vocab, H), K_LM_HEAD: (self.vocab, H), K_FINAL_NORM: (H,),
            K_ATTN_NORM: (H,), K_MOE_NORM: (H,), K_WQKV: (self.qkv_rows, H), K_WO: (H, self.attn_dim),
            K_ROUTER: (E, H), K_W_GATE: (E, I, H), K_W_UP: (E, I, H), K_W_DOWN: (E, H, I),
        }[kind]

    def kv_bytes_per_token(self) -> int:
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim * 2

    def active_weight_bytes(self, distinct_experts_per_layer: float) -> float:
        """Algorithmic weight bytes read by one decode step (one embedding row per token aside):
        2 bytes per bf16 element; 1 per quantized element plus 4 per quantized row."""
        H, I = self.hidden, self.inter
        per_el = {"fp8": 1.0, "fp4": 0.5}.get(self.weights)

        def mat(rows: float, cols: int) -> float:
            return per_el * rows * cols + 4.0 * rows if per_el else 2.0 * rows * cols

        per_layer = (mat(self.qkv_rows, H) + mat(H, self.attn_dim) + 2.0 * H * self.n_experts
                     + distinct_experts_per_layer * (2 * mat(I, H) + mat(H, I)) + 2.0 * H * (2 if self.sequential else 1))
        return self.n_layers * per_layer + mat(self.vocab, H) + 2.0 * H


LAYER_KINDS = (K_ATTN_NORM, K_WQKV, K_WO, K_ROUTER, K_W_GATE, K_W_UP, K_W_DOWN)
PER_LAYER_KINDS = LAYER_KINDS + (K_MOE_NORM,)   # kinds with one tensor per layer (tensor id indexed by layer)
# matrices streamed as FP8 in an "fp8" model: every large weight stream; the router rows (which
# decide the routing), the norm gains and the embedding rows stay bf16
QUANT_KINDS = (K_LM_HEAD, K_WQKV, K_WO, K_W_GATE, K_W_UP, K_W_DOWN)
FP8_SCALE_KIND = 64   # scale stream of kind k: tensor id tid(FP8_SCALE_KIND + k, index)
GLOBAL_KINDS = (K_EMBED, K_LM_HEAD, K_FINAL_NORM)
GAIN_KINDS = (K_ATTN_NORM, K_FINAL_NORM, K_MOE_NORM)

TINY = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  n_experts=8, top_k=2, inter=128, vocab=1024)
MID = ModelShape(n_layers=8, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=128,
                 n_experts=32, top_k=4, inter=512, vocab=32000)
MOE30B = ModelShape(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
                    n_experts=128, top_k=8, inter=768, vocab=151936)


def weight_bits(shape: ModelShape, kind: int, layer: int = 0, expert: int | None = None) -> np.ndarray:
    """bf16 bits of one weight tensor (or one expert's slice of it), generated from the recipe."""
    full = shape.weight_shape(kind)
    t = tid(kind, layer if kind in PER_LAYER_KINDS else 0)
    if expert is not None:
        assert len(full) == 3
        per = full[1] * full[2]
        start, count, out_shape = expert * per, per, full[1:]
    else:
        start, count, out_shape = 0, int(np.prod(full)), full
    if kind in GAIN_KINDS:
        a = gain_bf16(SEED_WEIGHTS, t, start, count, GAIN_SIGMA)
    else:
        a = normal_bf16(SEED_WEIGHTS, t, start, count, WEIGHT_SIGMA)
    return a.reshape(out_shape)


def fp8_codes(seed: int, t: int, start: int, count: int, out: np.ndarray | None = None) -> np.ndarray:
    """E4M3 codes (uint8) of elements ``start .. start+count-1`` of stream (seed, t)."""
    if out is None:
        out = np.empty(count, dtype=np.uint8)
    lib().synth_fp8_codes(seed, t, start, count, _ptr(out))
    return out


def fp8_scales(seed: int, t: int, start: int, count: int) -> np.ndarray:
    """fp32 row scales ``start .. start+count-1`` of stream (seed, t)."""
    out = np.empty(count, dtype=np.float32)
    lib().synth_fp8_scales(seed, t, start, count, WEIGHT_SIGMA, GAIN_SIGMA, _ptr(out))
    return out


def fp4_codes(seed: int, t: int, start: int, count: int, out: np.ndarray | None = None) -> np.ndarray:
    """Packed E2M1 codes (uint8, two a byte, the even element in the low nibble) of elements
    ``start .. start+count-1`` of stream (seed, t); start and count even."""
    assert start % 2 == 0 and count % 2 == 0
    if out is None:
        out = np.empty(count // 2, dtype=np.uint8)
    lib().synth_fp4_codes(seed, t, start, count, _ptr(out))
    return out


def fp4_scales(seed: int, t: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    lib().synth_fp4_scales(seed, t, start, count, WEIGHT_SIGMA, GAIN_SIGMA, _ptr(out))
    return out


def weight_fp4(shape: ModelShape, kind: int, layer: int = 0, expert: int | None = None):
    """(packed codes uint8 [..][cols / 2], scales float32 [rows]) of one FP4 weight tensor (or one
    expert's slice of it), generated from the recipe."""
    assert shape.quantized(kind) and shape.weights == "fp4"
    full = shape.weight_shape(kind)
    index = layer if kind in PER_LAYER_KINDS else 0
    if expert is not None:
        per = full[1] * full[2]
        start, count, out_shape = expert * per, per, full[1:]
    else:
        start, count, out_shape = 0, int(np.prod(full)), full
    cols = full[-1]
    codes = fp4_codes(SEED_WEIGHTS, tid(kind, index), start, count).reshape(out_shape[:-1] + (cols // 2,))
    scales = fp4_scales(SEED_WEIGHTS, tid(FP8_SCALE_KIND + kind, index), start // cols, count // cols)
    return codes, scales


def weight_fp8(shape: ModelShape, kind: int, layer: int = 0, expert: int | None = None):
    """(codes uint8 [..][cols], scales float32 [rows]) of one quantized weight tensor (or one expert's
    slice of it), generated from the recipe."""
    assert shape.quantized(kind) and shape.weights == "fp8"
    full = shape.weight_shape(kind)
    index = layer if kind in PER_LAYER_KINDS else 0
    if expert is not None:
        assert len(full) == 3
        per = full[1] * full[2]
        start, count, out_shape = expert * per, per, full[1:]
    else:
        start, count, out_shape = 0, int(np.prod(full)), full
    cols = full[-1]
    codes = fp8_codes(SEED_WEIGHTS, tid(kind, index), start, count).reshape(out_shape)
    scales = fp8_scales(SEED_WEIGHTS, tid(FP8_SCALE_KIND + kind, index), start // cols, count // cols)
    return codes, scales


def kv_bits(shape: ModelShape, layer: int, which: str, seq: int, t0: int, t1: int) -> np.ndarray:
    """Synthetic K or V ([t1-t0][n_kv][d] bf16 bits) of sequence ``seq`` at logical positions t0..t1-1."""
    kind = K_K_CACHE if which == "k" else K_V_CACHE
    per_tok = shape.n_kv_heads * shape.head_dim
    t = tid(kind, (seq << 8) | layer)
    a = normal_bf16(SEED_KV, t, t0 * per_tok, (t1 - t0) * per_tok, KV_SIGMA)
    return a.reshape(t1 - t0, shape.n_kv_heads, shape.head_dim)


@dataclass
class Workload:
    """One decode workload: model shape, batch, per-sequence context, page layout, steps."""
    name: str
    shape: ModelShape
    batch: int
    steps: int
    context: list = field(default_factory=list)   # tokens already in the cache per sequence
    kv_mode: str = "synthetic"                    # "synthetic" or "prefill" (prompt run as decode steps)
    shuffle_pages: bool = True
    spare_pages: int = 0

    def pages_needed(self, b: int) -> int:
        ps = self.shape.page_size
        return (self.context[b] + self.steps + ps - 1) // ps

    @property
    def num_pages(self) -> int:
        return sum(self.pages_needed(b) for b in range(self.batch)) + self.spare_pages

    @property
    def max_pages_per_seq(self) -> int:
        return max(self.pages_needed(b) for b in range(self.batch))

    def page_table(self) -> np.ndarray:
        """[batch][max_pages_per_seq] int32, -1 past each sequence's pages."""
        P = self.num_pages
        perm = permutation(SEED_PAGES, tid(K_PAGE_PERM), P) if self.shuffle_pages else np.arange(P, dtype=np.int32)
        pt = np.full((self.batch, self.max_pages_per_seq), -1, dtype=np.int32)
        o = 0
        for b in range(self.batch):
            n = self.pages_needed(b)
            pt[b, :n] = perm[o:o + n]
            o += n
        return pt

    def prompt(self, b: int) -> np.ndarray:
        return uniform_u32(SEED_PROMPT, tid(K_PROMPT, b), 0, self.context[b] + 1, self.shape.vocab).astype(np.int32)


def ragged_lengths(batch: int, lo: int, hi: int) -> list:
    """Per-sequence context lengths uniform in [lo, hi] inclusive."""
    u = uniform_u32(SEED_LENS, tid(K_SEQ_LENS), 0, batch, hi - lo + 1)
    return [int(lo + v) for v in u]


def workload(name: str) -> Workload:
    """The five workloads: tiny, mid, moe30b_8k, moe30b_bs8_ragged, moe30b_256k; a name ending in
    ``_fp8`` (``_fp4``) is the same workload with the QUANT_KINDS matrices in FP8 (FP4), one ending
    in ``_seq`` the same with the sequential block (suffixes combine: ``mid_seq_fp8``)."""
    for fmt in ("fp8", "fp4"):
        if name.endswith("_" + fmt):
            w = workload(name[: -len(fmt) - 1])
            w.name = name
            w.shape = replace(w.shape, weights=fmt)
            return w
    if name.endswith("_seq"):
        w = workload(name[:-4])
        w.name = name
        w.shape = replace(w.shape, block="sequential")
        return w
    if name == "tiny":
        return Workload(name, TINY, batch=1, steps=16, context=[128], kv_mode="prefill", shuffle_pages=False)
    if name == "mid":
        return Workload(name, MID, batch=1, steps=64, context=[2048])
    if name == "moe30b_8k":
        return Workload(name, MOE30B, batch=1, steps=128, context=[8192])
    if name == "moe30b_bs8_ragged":
        return Workload(name, MOE30B, batch=8, steps=128, context=ragged_lengths(8, 1024, 32768))
    if name == "moe30b_256k":
        return Workload(name, MOE30B, batch=1, steps=32, context=[262144])
    raise KeyError(name)


WORKLOADS = ("tiny", "mid", "moe30b_8k", "moe30b_bs8_ragged", "moe30b_256k")
