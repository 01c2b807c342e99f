"""Device-side harness: PyTorch allocates, the C ABI computes.

``DeviceDecoder`` owns every device buffer of one workload (weights, paged KV
pools, page table, step buffers, the library's workspace), fills weights and
synthetic KV from the seeded ``synth`` generator through a pinned staging
buffer, binds them to an ``mk`` context and enqueues decode steps.  No part
of the decode step runs here.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from . import mk

POISON = 0x7FC0  # bfloat16 NaN: unwritten KV slots poison any stray read


class _Stager:
    """Double-buffered pinned host staging for host-generated data."""

    def __init__(self, nbytes: int = 1 << 26):
        self.nbytes = nbytes
        self.bufs = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.events = [None, None]
        self.k = 0

    def fill(self, dst_flat: torch.Tensor, gen, esize: int = 2) -> None:
        """dst_flat (uint8 view, on device) <- gen(start, count, host_ptr) in elements of esize bytes,
        chunk by chunk."""
        n = dst_flat.numel() // esize
        per = self.nbytes // esize
        for start in range(0, n, per):
            cnt = min(per, n - start)
            k = self.k
            if self.events[k] is not None:
                self.events[k].synchronize()
            buf = self.bufs[k]
            gen(start, cnt, buf.data_ptr())
            dst_flat[start * esize:(start + cnt) * esize].copy_(buf[:cnt * esize], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self.events[k] = ev
            self.k ^= 1

    def sync(self):
        for e in self.events:
            if e is not None:
                e.synchronize()


def _kind_gen(kind: int, layer: int):
    t = synth.tid(kind, layer if kind in synth.PER_LAYER_KINDS else 0)
    lib = synth.lib()
    if kind in synth.GAIN_KINDS:
        return lambda s, c, p: lib.synth_gain_bf16(synth.SEED_WEIGHTS, t, s, c, synth.GAIN_SIGMA, p)
    return lambda s, c, p: lib.synth_normal_bf16(synth.SEED_WEIGHTS, t, s, c, synth.WEIGHT_SIGMA, p)


def _fp8_gen(kind: int, layer: int):
    t = synth.tid(kind, layer if kind in synth.PER_LAYER_KINDS else 0)
    lib = synth.lib()
    return lambda s, c, p: lib.synth_fp8_codes(synth.SEED_WEIGHTS, t, s, c, p)


def _fp4_gen(kind: int, layer: int):
    """Packed E2M1 codes by byte: byte i holds elements 2i (low nibble) and 2i + 1."""
    t = synth.tid(kind, layer if kind in synth.PER_LAYER_KINDS else 0)
    lib = synth.lib()
    return lambda s, c, p: lib.synth_fp4_codes(synth.SEED_WEIGHTS, t, 2 * s, 2 * c, p)


class DeviceDecoder:
    """All device state of one workload, bound to one mk context."""

    def __init__(self, w: synth.Workload, device: str = "cuda:0", num_cus: int = 0, ctx_hint: int | None = None,
                 max_batch: int | None = None, static_workspace: bool = False, **sched):
        """static_workspace: bind with the library's static workspace (no workspace tensor);
        sched: further mk_schedule_params fields (attn_units, router_units, prefetch_bytes, pool_64ths)."""
        self.w = w
        self.shape = s = w.shape
        self.dev = torch.device(device)
        self.B = w.batch
        self.page_table_np = w.page_table()
        self.num_pages = w.num_pages
        self.max_pages = w.max_pages_per_seq
        cfg = mk.config_from_shape(s, max_batch or w.batch, self.max_pages, self.num_pages)
        self.ctx = mk.Context(cfg)
        hint = ctx_hint if ctx_hint is not None else int(np.mean(w.context)) + w.steps // 2
        self.ws_bytes = self.ctx.build_schedule(num_cus, hint, **sched)
        self.info = self.ctx.info()
        self.offsets = self.ctx.ws_offsets()
        stream = torch.cuda.current_stream(self.dev)
        self.stream = stream.cuda_stream
        with torch.cuda.device(self.dev):
            stager = _Stager()
            self.weights = []
            for kind, layer in s.bind_order():
                if s.quantized(kind):
                    # FP8 / FP4: the E4M3 / packed E2M1 codes, then one fp32 scale per row, in one buffer
                    shp = s.weight_shape(kind)
                    nel = int(np.prod(shp))
                    fp4 = s.weights == "fp4"
                    ncode = nel // 2 if fp4 else nel
                    t = torch.empty(s.weight_nbytes(kind), dtype=torch.uint8, device=self.dev)
                    stager.fill(t[:ncode], (_fp4_gen if fp4 else _fp8_gen)(kind, layer), esize=1)
                    idx = layer if kind in synth.PER_LAYER_KINDS else 0
                    scales = synth.fp4_scales if fp4 else synth.fp8_scales
                    sc = scales(synth.SEED_WEIGHTS, synth.tid(synth.FP8_SCALE_KIND + kind, idx), 0, nel // shp[-1])
                    t[ncode:].copy_(torch.from_numpy(sc.view(np.uint8)))
                else:
                    t = torch.empty(s.weight_shape(kind), dtype=torch.bfloat16, device=self.dev)
                    stager.fill(t.view(torch.uint8).view(-1), _kind_gen(kind, layer))
                self.weights.append(t)
            stager.sync()
            self.stager = stager
            # K pages are [slot][dim] per (layer, page, head); V pages are dims-major [dim][slot]
            k_shape = (s.n_layers, self.num_pages, s.n_kv_heads, s.page_size, s.head_dim)
            v_shape = (s.n_layers, self.num_pages, s.n_kv_heads, s.head_dim, s.page_size)
            self.k_pool = torch.full(k_shape, POISON, dtype=torch.int16, device=self.dev)
            self.v_pool = torch.full(v_shape, POISON, dtype=torch.int16, device=self.dev)
            if not static_workspace:
                self.ws = torch.zeros(self.ws_bytes + 256, dtype=torch.uint8, device=self.dev)
                self.ws_base = (self.ws.data_ptr() + 255) // 256 * 256
            self.page_table = torch.from_numpy(self.page_table_np).to(self.dev)
            self.tokens = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
            self.seq_lens = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
            self.logits = torch.zeros(self.B, s.vocab, dtype=torch.float32, device=self.dev)
            self.next_tok = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
            torch.cuda.synchronize(self.dev)
            ptrs = [t.data_ptr() for t in self.weights]
            if static_workspace:
                self.ctx.bind_scratch(ptrs, self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.stream)
            else:
                self.ctx.bind(ptrs, self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.ws_base, self.ws_bytes,
                              self.stream)

    # ------------------------------------------------------------------ KV

    def fill_synthetic_kv(self) -> None:
        """Positions 0..context[b]-1 of every sequence from the synth KV recipe."""
        s = self.shape
        ps = s.page_size
        for b, n in enumerate(self.w.context):
            if n == 0:
                continue
            npg = (n + ps - 1) // ps
            pages = torch.from_numpy(self.page_table_np[b, :npg].astype(np.int64)).to(self.dev)
            for layer in range(s.n_layers):
                for which, pool in (("k", self.k_pool), ("v", self.v_pool)):
                    a = synth.kv_bits(s, layer, which, b, 0, n)
                    buf = np.full((npg * ps, s.n_kv_heads, s.head_dim), POISON, dtype=np.uint16)
                    buf[:n] = a
                    blk = buf.reshape(npg, ps, s.n_kv_heads, s.head_dim)
                    # K pages [head][slot][dim]; V pages dims-major [head][dim][slot]
                    blk = blk.transpose(0, 2, 1, 3) if which == "k" else blk.transpose(0, 2, 3, 1)
                    src = torch.from_numpy(np.ascontiguousarray(blk).view(np.int16)).to(self.dev)
                    pool[layer].index_copy_(0, pages, src)
        torch.cuda.synchronize(self.dev)

    # ------------------------------------------------------------------ steps

    def step(self, tokens, seq_lens, n: int | None = None, next_out: torch.Tensor | None = None) -> None:
        """Enqueue one decode step; tokens/seq_lens are host sequences or device int32 tensors."""
        n = n or self.B
        tok = tokens if isinstance(tokens, torch.Tensor) else torch.tensor(list(tokens), dtype=torch.int32)
        sl = seq_lens if isinstance(seq_lens, torch.Tensor) else torch.tensor(list(seq_lens), dtype=torch.int32)
        if tok.device != self.dev:
            self.tokens[: len(tok)].copy_(tok)
            tok = self.tokens
        if sl.device != self.dev:
            self.seq_lens[: len(sl)].copy_(sl)
            sl = self.seq_lens
        nxt = self.next_tok if next_out is None else next_out
        self.ctx.decode_step(n, tok.data_ptr(), self.page_table.data_ptr(), sl.data_ptr(), self.logits.data_ptr(),
                             nxt.data_ptr(), self.stream)

    def close(self) -> None:
        """Ordered teardown: wait for the device, destroy the context, release every device buffer."""
        torch.cuda.synchronize(self.dev)
        if getattr(self, "ctx", None) is not None:
            self.ctx.close()
            self.ctx = None
        for name in ("weights", "k_pool", "v_pool", "ws", "page_table", "tokens", "seq_lens", "logits", "next_tok",
                     "stager"):
            if hasattr(self, name):
                delattr(self, name)
        torch.cuda.empty_cache()

    def check_error(self):
        code, cu, task = self.ctx.get_error(self.stream)
        if code != 0:
            raise mk.MkError(code, "device", f"raised by cu {cu}, task {task}")

    # ------------------------------------------------------------------ workspace views (debugging, parity)

    def _ws_view(self, off: int, count: int, dtype) -> torch.Tensor:
        if not hasattr(self, "ws"):
            raise RuntimeError("bound to the static workspace: no workspace tensor to view")
        esz = torch.tensor([], dtype=dtype).element_size()
        start = self.ws_base - self.ws.data_ptr() + off
        return self.ws[start:start + count * esz].view(dtype)

    def sel(self) -> np.ndarray:
        s = self.shape
        mb = self.ctx.cfg.max_batch
        v = self._ws_view(self.offsets.sel, s.n_layers * mb * s.top_k, torch.int32)
        return v.view(s.n_layers, mb, s.top_k).cpu().numpy()

    def router_logits(self) -> np.ndarray:
        s = self.shape
        mb = self.ctx.cfg.max_batch
        v = self._ws_view(self.offsets.router, s.n_layers * mb * s.n_experts, torch.float32)
        return v.view(s.n_layers, mb, s.n_experts).cpu().numpy()

    def residual(self) -> np.ndarray:
        s = self.shape
        mb = self.ctx.cfg.max_batch
        v = self._ws_view(self.offsets.x, (s.n_layers + 1) * mb * s.hidden, torch.float32)
        return v.view(s.n_layers + 1, mb, s.hidden).cpu().numpy()

    def residual_halves(self):
        """(moe_half [L+1][max_batch][H], attn_half [L][max_batch][H]): x_l + moe_l in slot l+1 and
        layer l's attention output times Wo; their sum is x_{l+1}."""
        s = self.shape
        mb = self.ctx.cfg.max_batch
        m = self._ws_view(self.offsets.moe_half, (s.n_layers + 1) * mb * s.hidden, torch.float32)
        a = self._ws_view(self.offsets.attn_half, s.n_layers * mb * s.hidden, torch.float32)
        return (m.view(s.n_layers + 1, mb, s.hidden).cpu().numpy(), a.view(s.n_layers, mb, s.hidden).cpu().numpy())

    def kv_at(self, layer: int, b: int, pos: int):
        """(K, V) bf16 bits [n_kv][d] stored for logical position pos of sequence b."""
        ps = self.shape.page_size
        page = int(self.page_table_np[b, pos // ps])
        k = self.k_pool[layer, page, :, pos % ps, :].cpu().numpy().view(np.uint16)
        v = self.v_pool[layer, page, :, :, pos % ps].cpu().numpy().view(np.uint16)
        return k, v
