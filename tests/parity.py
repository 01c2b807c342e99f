"""Step-by-step comparison of the GPU decode (through the C ABI) with the CPU oracle.

Protocol, per step:
  * logits: per sequence, max_i |gpu_i - oracle_i| / max_i |oracle_i| <= LOGIT_TOL;
  * expert choice: bit-exact wherever the oracle's k-th / (k+1)-th router margin
    exceeds MARGIN (1e-3); below it either set is a correct result and the
    flip is only counted;
  * greedy token: equal unless the oracle's top-1 / top-2 gap is within
    GAP_FACTOR times the step's largest absolute logit difference;
  * both sides are fed the oracle's greedy token (teacher forcing), each side
    keeps its own KV cache.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field

import numpy as np
import torch

import synth
from oracle import oracle as O

LOGIT_TOL = 2e-2
MARGIN = 1e-3
GAP_FACTOR = 4.0


@dataclass
class Report:
    steps: int = 0
    max_rel: float = 0.0
    route_checked: int = 0
    route_ties: int = 0
    greedy_checked: int = 0
    greedy_excused: int = 0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures


def compare_step(rep: Report, tag: str, dec, ref, n: int) -> None:
    torch.cuda.synchronize()
    dec.check_error()
    got = dec.logits[:n].cpu().numpy().astype(np.float64)
    rep.steps += 1
    for b in range(n):
        o = ref.logits[b]
        diff = np.abs(got[b] - o)
        rel = float(diff.max() / np.abs(o).max())
        rep.max_rel = max(rep.max_rel, rel)
        if not rel <= LOGIT_TOL:
            rep.failures.append(f"{tag} seq {b}: logit rel err {rel:.3e}")
        gtok = int(np.argmax(got[b]))
        rep.greedy_checked += 1
        if gtok != int(ref.next_token[b]):
            if ref.top2_gap[b] <= GAP_FACTOR * diff.max():
                rep.greedy_excused += 1
            else:
                rep.failures.append(f"{tag} seq {b}: greedy {gtok} vs {int(ref.next_token[b])} "
                                    f"(gap {ref.top2_gap[b]:.3e}, max diff {diff.max():.3e})")
    sel = dec.sel()
    L = ref.sel.shape[0]
    for l in range(L):
        for b in range(n):
            rep.route_checked += 1
            a = sorted(sel[l, b].tolist())
            e = sorted(ref.sel[l, b].tolist())
            if a != e:
                if ref.margin[l, b] <= MARGIN:
                    rep.route_ties += 1
                else:
                    rep.failures.append(f"{tag} layer {l} seq {b}: experts {a} vs {e} (margin {ref.margin[l, b]:.2e})")


def run(w: synth.Workload, steps: int | None = None, dec=None, W=None, log=print) -> Report:
    """Run `steps` decode steps of workload w on both sides; returns the report."""
    from persistent_moe_decode_amd.runtime import DeviceDecoder

    steps = w.steps if steps is None else steps
    t0 = time.time()
    dec = dec or DeviceDecoder(w)
    W = W or O.Weights(w.shape, budget_bytes=float(2 ** 36))
    pt = w.page_table()
    kv = O.PagedKV(w.shape, w.num_pages)
    rep = Report()
    n = w.batch
    if w.kv_mode == "synthetic":
        dec.fill_synthetic_kv()
        kv.fill_synthetic(pt, w.context)
        toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
    else:
        # prompt fed one decode step at a time on both sides
        assert n == 1
        prompt = w.prompt(0)[: w.context[0]]
        ref = None
        for t, tok in enumerate(prompt):
            dec.step([int(tok)], [t])
            ref = O.decode_step(W, kv, [int(tok)], pt, [t])
            compare_step(rep, f"prefill {t}", dec, ref, n)
        toks = [int(ref.next_token[0])]
    log(f"[parity {w.name}] setup+prefill {time.time() - t0:.1f}s")
    for step in range(steps):
        lens = [c + step for c in w.context]
        dec.step(toks, lens)
        ref = O.decode_step(W, kv, toks, pt, lens)
        compare_step(rep, f"step {step}", dec, ref, n)
        toks = [int(x) for x in ref.next_token]
        if step % 8 == 0:
            log(f"[parity {w.name}] step {step} max_rel {rep.max_rel:.3e} ties {rep.route_ties} "
                f"{time.time() - t0:.1f}s")
    return rep
