"""On-device sampling (mk_set_sampling) through the C ABI.

At temperature T the device draws the next token by the Gumbel-max rule with SplitMix64 noise keyed
by (seed, position, batch slot, token id).  Checked here:
  * the device token is the argmax of its own logits perturbed by that noise (recomputed on the
    host by the oracle's independent generator): exact, up to a near-tie within the rounding of
    the device's float scores;
  * the oracle, fed the same tokens and following the device's branch at router near-ties (as the
    free-running parity runs do), samples the same token from its float64 logits, except where its
    top-2 perturbed scores lie within GAP_FACTOR times the largest logit difference (over T);
    sequences whose routing diverged beyond a near-tie swap are not compared that step;
  * a multi-step launch samples exactly what single launches do;
  * temperature 0 is the greedy argmax.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

T, SEED = 0.8, 0x5EED


def _device_step(dec, toks, lens, n):
    dec.step(toks, lens)
    torch.cuda.synchronize()
    dec.check_error()
    return dec.logits[:n].cpu().numpy().copy(), [int(x) for x in dec.next_tok[:n].cpu().numpy()]


def _own_scores(O, logits_f32, pos, b, max_batch):
    """The device's score for every token, recomputed on the host: float(x * (1/T) + g)."""
    g = O.gumbel_noise(SEED, pos, b, max_batch, logits_f32.size)
    return (logits_f32.astype(np.float64) * (1.0 / T) + g).astype(np.float32)


def test_sampled_tokens_follow_the_rule_and_the_oracle():
    from oracle import oracle as O
    from tests.parity import GAP_FACTOR, LOGIT_TOL, oracle_step
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("mid_sample", synth.MID, batch=3, steps=5, context=[900, 17, 1500])
    n = w.batch
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    dec.ctx.set_sampling(T, SEED)
    W = O.Weights(w.shape)
    pt = w.page_table()
    kv = O.PagedKV(w.shape, w.num_pages)
    kv.fill_synthetic(pt, w.context)
    mb = dec.ctx.cfg.max_batch
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
    agree = excused = diverged = 0
    try:
        for step in range(w.steps):
            lens = [c + step for c in w.context]
            got, dev_tok = _device_step(dec, toks, lens, n)
            sel = dec.sel()[:, :n]
            ref, _ = oracle_step(W, kv, toks, pt, lens, sel, n)
            for b in range(n):
                # the device's own rule on its own logits
                sc = _own_scores(O, got[b], lens[b], b, mb)
                best = float(sc.max())
                assert sc[dev_tok[b]] >= best - 2.0 * np.spacing(np.float32(abs(best))), (step, b)
                if dev_tok[b] != int(np.argmax(sc)):
                    print(f"step {step} seq {b}: device score rounding near-tie", flush=True)
                # the oracle's draw from its own logits, where it took the device's routing
                if any(sorted(sel[l, b].tolist()) != sorted(ref.sel[l, b].tolist()) for l in range(w.shape.n_layers)):
                    diverged += 1
                    continue
                diff = float(np.max(np.abs(got[b] - ref.logits[b])))
                assert diff / np.max(np.abs(ref.logits[b])) <= LOGIT_TOL
                tok_o, v = O.sample_token(ref.logits[b], T, SEED, lens[b], b, mb)
                if dev_tok[b] == tok_o:
                    agree += 1
                else:
                    top2 = np.sort(v)[-2:]
                    assert top2[1] - top2[0] <= GAP_FACTOR * diff / T, (step, b, dev_tok[b], tok_o)
                    excused += 1
            print(f"step {step}: sampled {dev_tok}", flush=True)
            toks = dev_tok
    finally:
        dec.close()
    print(f"sampled tokens: {agree} equal to the oracle's draw, {excused} at a near-tie, "
          f"{diverged} not compared (routing diverged)", flush=True)
    assert agree >= n * w.steps // 2


def test_sampling_in_one_launch_equals_single_launches():
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    steps = 6
    w = synth.Workload("mid_sample_ms", synth.MID, batch=3, steps=steps + 1, context=[700, 33, 1200])
    n = w.batch
    dec = DeviceDecoder(w)
    dec.ctx.set_sampling(T, SEED)
    dev = dec.dev
    lens0 = torch.tensor(w.context, dtype=torch.int32, device=dev)
    tok0 = torch.tensor([int(w.prompt(b)[w.context[b]]) for b in range(n)], dtype=torch.int32, device=dev)
    try:
        dec.fill_synthetic_kv()
        toks = torch.zeros(steps + 1, n, dtype=torch.int32, device=dev)
        toks[0] = tok0
        lens = torch.stack([lens0 + s for s in range(steps)]).contiguous()
        for s in range(steps):
            dec.ctx.decode_step(n, toks[s].data_ptr(), dec.page_table.data_ptr(), lens[s].data_ptr(),
                                dec.logits.data_ptr(), toks[s + 1].data_ptr(), dec.stream)
        torch.cuda.synchronize()
        dec.check_error()
        single = (toks[1:].cpu().numpy(), dec.logits[:n].cpu().clone())
        dec.fill_synthetic_kv()
        out = torch.full((steps, n), -1, dtype=torch.int32, device=dev)
        dec.logits.zero_()
        dec.ctx.decode_steps(n, steps, tok0.data_ptr(), dec.page_table.data_ptr(), lens0.data_ptr(),
                             dec.logits.data_ptr(), out.data_ptr(), dec.stream)
        torch.cuda.synchronize()
        dec.check_error()
        print(f"sampled tokens per step: {out.cpu().numpy().tolist()}", flush=True)
        assert np.array_equal(out.cpu().numpy(), single[0])
        assert torch.equal(dec.logits[:n].cpu(), single[1])
        # the draws are not the greedy tokens throughout (the noise is in effect)
        dec.ctx.set_sampling(0.0)
        dec.fill_synthetic_kv()
        g = torch.full((steps, n), -1, dtype=torch.int32, device=dev)
        dec.ctx.decode_steps(n, steps, tok0.data_ptr(), dec.page_table.data_ptr(), lens0.data_ptr(),
                             dec.logits.data_ptr(), g.data_ptr(), dec.stream)
        torch.cuda.synchronize()
        dec.check_error()
        assert not np.array_equal(g.cpu().numpy(), single[0])
    finally:
        dec.close()


def test_zero_temperature_is_the_greedy_argmax():
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("tiny_t0", synth.TINY, batch=2, steps=1, context=[37, 5])
    dec = DeviceDecoder(w)
    try:
        dec.fill_synthetic_kv()
        dec.ctx.set_sampling(0.5, 3)
        dec.ctx.set_sampling(0.0, 3)
        got, tok = _device_step(dec, [int(w.prompt(b)[w.context[b]]) for b in range(2)], w.context, 2)
        assert tok == [int(np.argmax(got[b])) for b in range(2)]
    finally:
        dec.close()


@pytest.mark.parametrize("top_p", [0.9, 0.5])
def test_top_p_draw_follows_the_nucleus_of_the_device_logits(top_p):
    """mk_set_top_p: each step's device token is the Gumbel-max argmax within the nucleus that the
    oracle's definition gives for the device's own logits; only where the mass at the threshold is
    within the fixed-point rounding of top_p may the device take the neighbouring nucleus."""
    from oracle import oracle as O
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("mid_top_p", synth.MID, batch=3, steps=6, context=[900, 17, 1500])
    n = w.batch
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    dec.ctx.set_sampling(T, SEED)
    dec.ctx.set_top_p(top_p)
    mb = dec.ctx.cfg.max_batch
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
    exact = near = 0
    try:
        for step in range(w.steps):
            lens = [c + step for c in w.context]
            got, dev_tok = _device_step(dec, toks, lens, n)
            for b in range(n):
                lg = got[b].astype(np.float32).astype(np.float64)
                want, nuc = O.sample_token_top_p(lg, T, top_p, SEED, lens[b], b, mb)
                if dev_tok[b] == want:
                    exact += 1
                    continue
                # the neighbouring nuclei: the threshold one distinct value lower or higher
                lo, _ = O.sample_token_top_p(lg, T, min(1.0, top_p * (1 + 1e-6)), SEED, lens[b], b, mb)
                hi, _ = O.sample_token_top_p(lg, T, top_p * (1 - 1e-6), SEED, lens[b], b, mb)
                assert dev_tok[b] in (lo, hi), (step, b, dev_tok[b], want, int(nuc.sum()))
                near += 1
            toks = dev_tok
    finally:
        dec.close()
    print(f"top-p {top_p}: {exact} draws equal, {near} at a threshold near-tie", flush=True)
    assert exact >= 3 * w.steps - 1
