"""Step-by-step comparison of the GPU decode (through the C ABI) with the CPU oracle.

Why two modes.  The decoder rounds to bfloat16 at several points per layer
(xn, q/k/v, attention output, expert hidden).  Any change of accumulation
order (fp32 on the GPU, fp64 in the oracle) moves a pre-rounding value across
a rounding boundary now and then; the one-ulp flip shifts the residual by
~1e-5, which flips the rounding of ~2% of the next layer's xn, and the
difference grows ~20x per layer until it settles near 5e-3 relative.  So a
free-running comparison of many layers cannot keep router decisions
identical at 1e-3 margins; a layer-by-layer one can.

isolated (the strict check): each step, the oracle runs first and its
  residual entering every layer is handed to the GPU through the layer-input
  hook (oracle -> GPU only), so every layer of the GPU runs on the oracle's
  inputs.  Per layer: expert choice bit-exact wherever the oracle's k-th /
  (k+1)-th margin exceeds MARGIN (else the GPU's set must be one of the two
  correct ones); router logits within ROUTER_TOL; the layer's output
  residual within X_TOL; the new K/V entries within one bfloat16 ulp (plus
  KV_ABS of the head vector's largest entry, see below).
  Logits within LOGIT_TOL; greedy token equal unless the oracle's top-2 gap
  is within GAP_FACTOR times the step's largest logit difference.

free (end to end): each side keeps its own state.  Where the expert choice
  first differs at a margin above MARGIN, the GPU's set must still be a
  correct top-k for the oracle's logits perturbed by twice the measured
  router-logit difference at that layer (the drift described above), and
  the step's logits are not compared; all other steps meet LOGIT_TOL and
  the greedy rule.  At near-ties the oracle recomputes the step down the
  branch the GPU took (the oracle's own alternative, never GPU values).
  Both modes check every layer's GPU expert choice against the exact top-k
  of the GPU's own router logits (the kernel's integer logic, bit-exact).

Teacher forcing: by default both sides are fed the oracle's greedy token.  With
teacher=False each side feeds its own greedy token (the GPU its device argmax) and
the run reports the free-running agreement length: the steps until the first token
disagreement, which must fall where the oracle's top-2 gap is within the step's
measured logit error (after it the two sequences differ and comparison stops).

Every step also checks the device argmax (next_tok) bit for bit against the argmax of
the GPU's own logits, lowest id on ties.
"""
from __future__ import annotations

import json
import os
import time
from dataclasses import asdict, dataclass, field

import numpy as np
import torch

import synth
from oracle import oracle as O

LOGIT_TOL = 2e-2
MARGIN = 1e-3
GAP_FACTOR = 4.0
ROUTER_TOL = 5e-4    # isolated mode: |router logit| difference per layer
X_TOL = 2e-3         # isolated mode: max|dx| / max|x| of each layer's output residual
# isolated mode: new K/V slack beyond one ulp, relative to the head vector's max.  The
# injected residual is the oracle's rounded to fp32, so now and then one element of the
# normalized input lands on the other side of a bf16 rounding boundary; that moves every
# k/v entry by |w| * ulp(xn) ~ 1e-4, more than an ulp for entries near zero.  A wrong
# rotation, position or head gives differences of the order of the entries themselves.
KV_ABS = 5e-4


@dataclass
class Report:
    steps: int = 0
    max_rel: float = 0.0
    max_router: float = 0.0
    max_x: float = 0.0
    route_checked: int = 0
    route_ties: int = 0
    cascade_steps: int = 0
    kv_checked: int = 0
    greedy_checked: int = 0
    greedy_excused: int = 0
    next_tok_checked: int = 0
    kv_max_ulps: float = 0.0
    kv_over_1ulp: int = 0          # new K/V entries more than one bf16 ulp off (allowed only within KV_ABS of the head's max)
    agree_steps: int = -1          # free running without teacher forcing: steps before the first token disagreement
    disagree_cause: str = ""
    min_top2_gap: float = float("inf")
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        s = (f"steps {self.steps} logits max_rel {self.max_rel:.2e} router max {self.max_router:.2e} "
             f"x max_rel {self.max_x:.2e} routes {self.route_checked} ties {self.route_ties} "
             f"cascade-steps {self.cascade_steps} kv {self.kv_checked} kv-max-ulps {self.kv_max_ulps:.2f} "
             f"kv>1ulp {self.kv_over_1ulp} "
             f"greedy {self.greedy_checked} excused {self.greedy_excused} next-tok {self.next_tok_checked} "
             f"min-top2-gap {self.min_top2_gap:.2e}")
        if self.agree_steps >= 0:
            s += f" free-agree {self.agree_steps}"
        return s


def kernel_src_hash() -> str:
    """First 16 hex digits of the SHA-256 of the library's HIP/C++ sources (names the kernel a record is for)."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "persistent_moe_decode_amd", "csrc")
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_kernel_fp8.hip", "mk_kernel_fp4.hip", "mk_kernel_seq.hip", "mk_host.cpp", "mk_types.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def record(name: str, rep: Report, **extra) -> None:
    """Append the report's summary as one JSON line to $MK_PARITY_RECORDS/<name>.jsonl, when that is set."""
    d = os.environ.get("MK_PARITY_RECORDS")
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    rec = {k: v for k, v in asdict(rep).items() if k != "failures"}
    rec.update(name=name, ok=rep.ok(), n_failures=len(rep.failures), first_failures=rep.failures[:3],
               summary=rep.summary(), time=time.strftime("%Y-%m-%d %H:%M:%S"), kernel_src=kernel_src_hash(),
               **extra)
    rec = {k: (None if isinstance(v, float) and v == float("inf") else v) for k, v in rec.items()}
    with open(os.path.join(d, f"{name}.jsonl"), "a") as f:
        f.write(json.dumps(rec) + "\n")


def seq_moe_input(W, x_l: np.ndarray, wo_gpu: np.ndarray, l: int):
    """Sequential block, isolated mode: (x_l + Wo attn, bf16(rmsnorm(that, g_moe))) as the kernel
    forms them, in float64.  The MoE path reads the norm of x_l + Wo attn; the kernel's Wo attn
    (fp32, after its own bf16 rounding of the attention output) is a few ulps from the oracle's, and
    an element of the normalized input near a bf16 rounding midpoint may then round the other way,
    moving router logit e by |Wr[e][i]| times one bf16 ulp (and the experts' inputs with it).  So
    the reference takes the kernel's Wo rows (read back from the workspace) and the same x_l the
    kernel read (the injected fp32 input, or layer 0's embedding row), adds them in fp32 as the
    kernel does, and normalizes in float64 as the kernel does: the oracle's MoE path (moe_path) from
    that input leaves the router rows' and the experts' fp32 sums to compare."""
    s = W.shape
    xp = (x_l.astype(np.float32) + wo_gpu.astype(np.float32)).astype(np.float64)
    return xp, O.round_bf16(O.rmsnorm(xp, W.get(synth.K_MOE_NORM, l), s.rms_eps))


def _topk(r: np.ndarray, k: int) -> list:
    return sorted(np.argsort(-r.astype(np.float64), kind="stable")[:k].tolist())


def _admissible(r_or: np.ndarray, chosen: list, k: int, delta: float) -> bool:
    """True if `chosen` is a top-k of r_or perturbed by at most delta/2 per entry."""
    others = [i for i in range(len(r_or)) if i not in chosen]
    return min(float(r_or[i]) for i in chosen) >= max(float(r_or[j]) for j in others) - delta


def _check_logits(rep, tag, got, ref, b):
    o = ref.logits[b]
    diff = np.abs(got - o)
    rel = float(diff.max() / np.abs(o).max())
    rep.max_rel = max(rep.max_rel, rel)
    if not rel <= LOGIT_TOL:
        rep.failures.append(f"{tag} seq {b}: logit rel err {rel:.3e}")
    rep.greedy_checked += 1
    rep.min_top2_gap = min(rep.min_top2_gap, float(ref.top2_gap[b]))
    gtok = int(np.argmax(got))
    if gtok != int(ref.next_token[b]):
        if ref.top2_gap[b] <= GAP_FACTOR * diff.max():
            rep.greedy_excused += 1
        else:
            rep.failures.append(f"{tag} seq {b}: greedy {gtok} vs {int(ref.next_token[b])} "
                                f"(gap {ref.top2_gap[b]:.3e}, max diff {diff.max():.3e})")


def _check_next_tok(rep, tag, dec, got, n):
    """The device argmax must be the argmax of the GPU's own logits, lowest id on ties (integer, exact)."""
    dev = dec.next_tok[:n].cpu().numpy()
    for b in range(n):
        rep.next_tok_checked += 1
        want = int(np.argmax(got[b]))
        if int(dev[b]) != want:
            rep.failures.append(f"{tag} seq {b}: device next_tok {int(dev[b])} vs argmax of its logits {want}")
    return [int(t) for t in dev]


def _kv_ulps(rep, gv, o64):
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(o64), 1e-30))[1] - 8)
    r = np.abs(gv - o64) / ulp
    rep.kv_max_ulps = max(rep.kv_max_ulps, float(np.max(r)))
    rep.kv_over_1ulp += int(np.sum(r > 1.0000001))
    return ulp


def _self_consistent(rep, tag, sel, rl, n, k):
    for l in range(sel.shape[0]):
        for b in range(n):
            if sorted(sel[l, b].tolist()) != _topk(rl[l, b], k):
                rep.failures.append(f"{tag} layer {l} seq {b}: GPU experts {sorted(sel[l, b].tolist())} are not "
                                    f"the top-{k} of its own router logits")


def oracle_step(W, kv, toks, pt, lens, gpu_sel, n: int, trace=False):
    """Oracle step on the correct routing branch the GPU took at each near-tie."""
    alts = set()
    L = W.shape.n_layers
    while True:
        ref = O.decode_step(W, kv, toks, pt, lens, trace=trace, route_alt=alts)
        new = None
        for b in range(n):
            for l in range(L):
                if sorted(gpu_sel[l, b].tolist()) != sorted(ref.sel[l, b].tolist()):
                    if (ref.margin[l, b] <= MARGIN and (l, b) not in alts
                            and sorted(gpu_sel[l, b].tolist()) == sorted(ref.sel_alt[l, b].tolist())):
                        new = (l, b)
                    break  # later layers follow from this one
            if new:
                break
        if new is None or len(alts) >= 8:
            return ref, alts
        alts.add(new)


class Runner:
    """Both sides of one workload, stepped together."""

    def __init__(self, w: synth.Workload, dec=None, log=print, **sched):
        from persistent_moe_decode_amd.runtime import DeviceDecoder

        self.w, self.log = w, log
        t0 = time.time()
        self.dec = dec or DeviceDecoder(w, **sched)
        self.W = O.Weights(w.shape, budget_bytes=float(2 ** 36))
        self.pt = w.page_table()
        self.kv = O.PagedKV(w.shape, w.num_pages)
        self.rep = Report()
        self.n = w.batch
        s = w.shape
        self.x_inj = None
        if w.kv_mode == "synthetic":
            self.dec.fill_synthetic_kv()
            self.kv.fill_synthetic(self.pt, w.context)
        log(f"[parity {w.name}] setup {time.time() - t0:.1f}s")
        self.t0 = time.time()

    # -------------------------------------------------------------- free running

    def step_free(self, toks, lens, tag):
        rep, dec, n, k = self.rep, self.dec, self.n, self.w.shape.top_k
        dec.step(toks, lens)
        torch.cuda.synchronize()
        dec.check_error()
        sel, rl = dec.sel()[:, :n], dec.router_logits()[:, :n]
        ref, alts = oracle_step(self.W, self.kv, toks, self.pt, lens, sel, n)
        rep.steps += 1
        rep.route_ties += len(alts)
        _self_consistent(rep, tag, sel, rl, n, k)
        got = dec.logits[:n].cpu().numpy().astype(np.float64)
        self.dev_tok = _check_next_tok(rep, tag, dec, got, n)
        self.compared = [False] * n
        self.max_diff = [0.0] * n
        for b in range(n):
            diverged = False
            for l in range(self.w.shape.n_layers):
                rep.route_checked += 1
                a, e = sorted(sel[l, b].tolist()), sorted(ref.sel[l, b].tolist())
                if a == e:
                    continue
                drift = float(np.max(np.abs(rl[l, b] - ref.router_logits[l, b])))
                if not _admissible(ref.router_logits[l, b], a, k, max(2 * drift, MARGIN)):
                    rep.failures.append(f"{tag} layer {l} seq {b}: experts {a} vs {e} (margin "
                                        f"{ref.margin[l, b]:.2e}, router drift {drift:.2e})")
                diverged = True
                break
            if diverged:
                rep.cascade_steps += 1
            else:
                _check_logits(rep, tag, got[b], ref, b)
                self.compared[b] = True
                self.max_diff[b] = float(np.max(np.abs(got[b] - ref.logits[b])))
        return ref

    # -------------------------------------------------------------- isolated layers

    def step_isolated(self, toks, lens, tag):
        rep, dec, n, s = self.rep, self.dec, self.n, self.w.shape
        L, k = s.n_layers, s.top_k
        ref = O.decode_step(self.W, self.kv, toks, self.pt, lens, trace=True)
        mb = dec.ctx.cfg.max_batch
        if self.x_inj is None:
            self.x_inj = torch.zeros((L + 1, mb, s.hidden), dtype=torch.float32, device=dec.dev)
            dec.ctx.set_layer_inputs(self.x_inj.data_ptr())
        host = np.zeros((L + 1, mb, s.hidden), dtype=np.float32)
        for b in range(n):
            for l in range(1, L):
                host[l, b] = ref.trace["x_in"][(l, b)]
            host[L, b] = ref.trace["x_final"][b]
        self.x_inj.copy_(torch.from_numpy(host))
        dec.step(toks, lens)
        torch.cuda.synchronize()
        dec.check_error()
        rep.steps += 1
        sel, rl, xs = dec.sel()[:, :n], dec.router_logits()[:, :n], dec.residual()[:, :n]
        attn_half = dec.residual_halves()[1][:, :n] if s.sequential else None
        _self_consistent(rep, tag, sel, rl, n, k)
        got = dec.logits[:n].cpu().numpy().astype(np.float64)
        self.dev_tok = _check_next_tok(rep, tag, dec, got, n)
        self.compared = [True] * n
        self.max_diff = [float(np.max(np.abs(got[b] - ref.logits[b]))) for b in range(n)]
        for b in range(n):
            p = int(lens[b])
            for l in range(L):
                rep.route_checked += 1
                if s.sequential:
                    # the MoE path from the kernel's own MoE input (seq_moe_input); the layer's
                    # output is then x_l + Wo attn (the kernel's, fp32) plus that path's sum
                    x_l = ref.trace["x_in"][(l, b)] if l == 0 else host[l, b]
                    xp, xm_g = seq_moe_input(self.W, x_l, attn_half[l, b], l)
                    mo = O.moe_path(self.W, l, xm_g)
                    r_ref, r_sel, r_alt, r_margin = mo.r, mo.sel, mo.sel_alt, mo.margin
                else:
                    r_ref, r_sel, r_alt, r_margin = ref.router_logits[l, b], ref.sel[l, b], ref.sel_alt[l, b], ref.margin[l, b]
                dr = float(np.max(np.abs(rl[l, b].astype(np.float64) - r_ref)))
                rep.max_router = max(rep.max_router, dr)
                if not dr <= ROUTER_TOL:
                    rep.failures.append(f"{tag} layer {l} seq {b}: router logits differ by {dr:.2e}")
                a, e = sorted(sel[l, b].tolist()), sorted(r_sel.tolist())
                took_alt = False
                if a != e:
                    if r_margin <= MARGIN and a == sorted(r_alt.tolist()):
                        rep.route_ties += 1
                        took_alt = True
                    else:
                        rep.failures.append(f"{tag} layer {l} seq {b}: experts {a} vs {e} (margin {r_margin:.2e})")
                # the layer's output residual
                if s.sequential:
                    if took_alt:
                        mo = O.moe_path(self.W, l, xm_g, take_alt=True)
                    xo = xp + mo.moe
                    took_alt = False
                    # the kernel's Wo output, which that reference takes as given, against the
                    # oracle's, within the residual check's budget (the parallel block's residual
                    # check holds the same attention half to it)
                    rw = float(np.max(np.abs(attn_half[l, b] - ref.trace["attn"][(l, b)])) / np.max(np.abs(xo)))
                    rep.max_x = max(rep.max_x, rw)
                    if not rw <= X_TOL:
                        rep.failures.append(f"{tag} layer {l} seq {b}: Wo output rel err {rw:.2e}")
                else:
                    xo = ref.trace["x_in"][(l + 1, b)] if l + 1 < L else ref.trace["x_final"][b]
                if not took_alt:
                    rx = float(np.max(np.abs(xs[l + 1, b] - xo)) / np.max(np.abs(xo)))
                    rep.max_x = max(rep.max_x, rx)
                    if not rx <= X_TOL:
                        rep.failures.append(f"{tag} layer {l} seq {b}: output residual rel err {rx:.2e}")
                # the new K/V entries: within one bfloat16 ulp, plus the fp32 accumulation
                # error of the projection (KV_ABS of the head vector's scale) for entries
                # that cancel to almost nothing
                kg, vg = dec.kv_at(l, b, p)
                for name, g16, o64 in (("k", kg, ref.trace["k16"][(l, b)]), ("v", vg, ref.trace["v16"][(l, b)])):
                    gv = O.bf16_to_f64(g16)
                    ulp = _kv_ulps(rep, gv, o64)
                    scale = np.max(np.abs(o64), axis=-1, keepdims=True)
                    bad = np.abs(gv - o64) > ulp * 1.0000001 + KV_ABS * scale
                    rep.kv_checked += gv.size
                    if np.any(bad):
                        rep.failures.append(f"{tag} layer {l} seq {b}: new {name} off by more than one ulp "
                                            f"at {int(bad.sum())} entries")
            _check_logits(rep, tag, got[b], ref, b)
        return ref

    # -------------------------------------------------------------- driver

    def run(self, steps: int, mode: str, teacher: bool = True) -> Report:
        """Prefill (for prefill-as-decode workloads) then `steps` greedy steps.

        teacher=False: each side feeds its own greedy token; at the first disagreement the
        oracle's top-2 gap must be within GAP_FACTOR times that step's largest logit difference
        (a near-tie either token may win), rep.agree_steps records the steps before it, and the
        run stops there.  With no disagreement agree_steps = steps."""
        w, rep, n = self.w, self.rep, self.n
        assert teacher or n == 1
        step_fn = self.step_isolated if mode == "isolated" else self.step_free
        if w.kv_mode == "synthetic":
            toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
        else:
            assert n == 1
            ref = None
            for t, tok in enumerate(w.prompt(0)[: w.context[0]]):
                ref = step_fn([int(tok)], [t], f"prefill {t}")
            toks = [int(ref.next_token[0])]
            self.log(f"[parity {w.name}] prefill done {time.time() - self.t0:.1f}s")
        for step in range(steps):
            lens = [c + step for c in w.context]
            ref = step_fn(toks, lens, f"step {step}")
            if not teacher:
                mine, theirs = self.dev_tok[0], int(ref.next_token[0])
                if mine != theirs:
                    rep.agree_steps = step
                    gap = float(ref.top2_gap[0])
                    if not self.compared[0]:
                        # this step's routing already diverged at a margin within the measured
                        # router drift (step_free checked that): the two logit vectors are results
                        # of different, both admissible expert sets, and the tokens may differ
                        rep.disagree_cause = "routing divergence within the measured router drift"
                    elif gap <= GAP_FACTOR * self.max_diff[0]:
                        rep.disagree_cause = f"near-tie of the top-2 logits (gap {gap:.3e})"
                    else:
                        rep.failures.append(f"step {step}: free-running tokens {mine} vs {theirs} at a top-2 gap "
                                            f"{gap:.3e} (max logit diff {self.max_diff[0]:.3e})")
                    self.log(f"[parity {w.name} {mode} no-teacher] first disagreement at step {step}: "
                             f"{rep.summary()}")
                    return rep
                toks = [mine]
            else:
                toks = [int(x) for x in ref.next_token]
            if step % 8 == 0 or step == steps - 1:
                self.log(f"[parity {w.name} {mode}] step {step}: {rep.summary()} {time.time() - self.t0:.1f}s")
        if not teacher:
            rep.agree_steps = steps
        return rep


def run(w: synth.Workload, steps: int | None = None, mode: str = "isolated", log=print, teacher: bool = True,
        **sched) -> Report:
    """sched: mk_schedule_params fields passed to the device decoder (attn_units, prefetch_bytes, ...)."""
    return Runner(w, log=log, **sched).run(w.steps if steps is None else steps, mode, teacher)


# ------------------------------------------------------------------ sampled layers at full size

INPUT_SEED = 6       # seeded residuals injected into every layer (the shared input generator, its own seed)
INPUT_SIGMA = 0.5


def injected_inputs(shape: synth.ModelShape, max_batch: int, n: int) -> np.ndarray:
    """[L+1][max_batch][H] float32: the residual fed to layer l >= 1 and to the final norm (index L)."""
    L, H = shape.n_layers, shape.hidden
    x = np.zeros((L + 1, max_batch, H), dtype=np.float32)
    for l in range(1, L + 1):
        for b in range(n):
            bits = synth.normal_bf16(INPUT_SEED, synth.tid(l, b), 0, H, INPUT_SIGMA)
            x[l, b] = O.bf16_to_f64(bits).astype(np.float32)
    return x


def run_sampled(w: synth.Workload, layers, log=print) -> Report:
    """One step at full size with every layer fed a seeded residual; the oracle recomputes the
    sampled layers from the same inputs (layer 0 from the embedding) and the LM head from the
    final input, and each is compared in full: expert choice, router logits, output residual,
    new K/V entries, logits and the greedy token."""
    from persistent_moe_decode_amd.runtime import DeviceDecoder

    t0 = time.time()
    s = w.shape
    L, k, n = s.n_layers, s.top_k, w.batch
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    mb = dec.ctx.cfg.max_batch
    host = injected_inputs(s, mb, n)
    x_inj = torch.from_numpy(host).to(dec.dev)
    dec.ctx.set_layer_inputs(x_inj.data_ptr())
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
    lens = list(w.context)
    dec.step(toks, lens)
    torch.cuda.synchronize()
    dec.check_error()
    log(f"[sampled {w.name}] GPU step done {time.time() - t0:.1f}s")
    sel, rl, xs = dec.sel()[:, :n], dec.router_logits()[:, :n], dec.residual()[:, :n]
    got = dec.logits[:n].cpu().numpy().astype(np.float64)
    rep = Report(steps=1)
    _self_consistent(rep, "sampled", sel, rl, n, k)
    _check_next_tok(rep, "sampled", dec, got, n)
    W = O.Weights(s, budget_bytes=float(2 ** 34))
    pt = w.page_table()
    kv = O.PagedKV(s, w.num_pages, layers=layers)
    kv.fill_synthetic(pt, w.context)
    log(f"[sampled {w.name}] oracle cache for layers {list(layers)} filled {time.time() - t0:.1f}s")
    emb = W.get(synth.K_EMBED)
    for b in range(n):
        p = int(lens[b])
        for l in layers:
            tag = f"layer {l} seq {b}"
            x_in = emb[toks[b]].copy() if l == 0 else host[l, b].astype(np.float64)
            ref = O.layer_forward(W, kv, l, x_in, p, pt[b])
            a, e = sorted(sel[l, b].tolist()), sorted(ref.sel.tolist())
            if a != e:
                if ref.margin <= MARGIN and ref.sel_alt is not None and a == sorted(ref.sel_alt.tolist()):
                    rep.route_ties += 1
                    ref = O.layer_forward(W, kv, l, x_in, p, pt[b], take_alt=True)
                else:
                    rep.failures.append(f"{tag}: experts {a} vs {e} (margin {ref.margin:.2e})")
            rep.route_checked += 1
            dr = float(np.max(np.abs(rl[l, b] - ref.r)))
            rep.max_router = max(rep.max_router, dr)
            if not dr <= ROUTER_TOL:
                rep.failures.append(f"{tag}: router logits differ by {dr:.2e}")
            rx = float(np.max(np.abs(xs[l + 1, b] - ref.x)) / np.max(np.abs(ref.x)))
            rep.max_x = max(rep.max_x, rx)
            if not rx <= X_TOL:
                rep.failures.append(f"{tag}: output residual rel err {rx:.2e}")
            kg, vg = dec.kv_at(l, b, p)
            for name, g16, o64 in (("k", kg, ref.parts["k16"]), ("v", vg, ref.parts["v16"])):
                gv = O.bf16_to_f64(g16)
                ulp = _kv_ulps(rep, gv, o64)
                scale = np.max(np.abs(o64), axis=-1, keepdims=True)
                bad = np.abs(gv - o64) > ulp * 1.0000001 + KV_ABS * scale
                rep.kv_checked += gv.size
                if np.any(bad):
                    rep.failures.append(f"{tag}: new {name} off by more than one ulp at {int(bad.sum())} entries")
        lg = O.lm_logits(W, host[L, b].astype(np.float64))
        srt = np.sort(lg)
        ref_out = O.StepOut(lg[None, :], None, None, None, np.array([int(np.argmax(lg))]),
                            np.array([srt[-1] - srt[-2]]))
        _check_logits(rep, f"seq {b}", got[b], ref_out, 0)
        log(f"[sampled {w.name}] seq {b} checked {time.time() - t0:.1f}s: {rep.summary()}")
    return rep
