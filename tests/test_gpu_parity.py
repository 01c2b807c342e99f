"""GPU decode through the C ABI against the CPU oracle, element by element.

"isolated" runs every layer on the oracle's inputs (strict per-layer checks);
"free" runs both sides end to end (see tests/parity.py for the protocol).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check(rep):
    _log(rep.summary())
    assert rep.ok(), "\n".join(rep.failures[:20])


def test_tiny_prefill_then_greedy_free():
    """Tiny MoE: 128-token prompt run as decode steps on both sides, then 16 teacher-forced steps."""
    from tests import parity
    rep = parity.run(synth.workload("tiny"), mode="free", log=_log)
    assert rep.steps == 128 + 16
    _check(rep)


def test_tiny_prefill_then_greedy_isolated():
    from tests import parity
    rep = parity.run(synth.workload("tiny"), mode="isolated", log=_log)
    assert rep.steps == 128 + 16
    _check(rep)


def test_tiny_ragged_batch_edges():
    """Batch of 8 with empty, sub-page, page-boundary and multi-page contexts, shuffled pages."""
    from tests import parity
    w = synth.Workload("tiny_ragged", synth.TINY, batch=8, steps=4, context=[0, 1, 15, 16, 17, 31, 32, 100],
                       spare_pages=3)
    _check(parity.run(w, mode="isolated", log=_log))


def test_mid_isolated_64_steps():
    """Mid MoE, 2048-token synthetic context, shuffled page order, 64 greedy steps, every layer on oracle inputs."""
    from tests import parity
    rep = parity.run(synth.workload("mid"), mode="isolated", log=_log)
    assert rep.steps == 64
    _check(rep)


def test_mid_free_running_64_steps():
    from tests import parity
    rep = parity.run(synth.workload("mid"), mode="free", log=_log)
    assert rep.steps == 64
    # most steps keep the same routing end to end and are compared in full
    assert rep.cascade_steps <= 24, rep.summary()
    _check(rep)


def test_mid_batch8_ragged():
    from tests import parity
    w = synth.Workload("mid_bs8", synth.MID, batch=8, steps=3,
                       context=[1, 700, 2048, 33, 1500, 16, 4000, 257])
    _check(parity.run(w, mode="isolated", log=_log))


def test_repeat_step_is_bit_identical():
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("rep", synth.MID, batch=2, steps=1, context=[300, 17])
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(2)]
    outs = []
    for _ in range(3):
        dec.step(toks, w.context)   # same position each time: rewrites the same KV slot
        torch.cuda.synchronize()
        dec.check_error()
        outs.append(dec.logits.cpu().clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert int(dec.next_tok[0]) == int(torch.argmax(outs[0][0]))
    assert int(dec.next_tok[1]) == int(torch.argmax(outs[0][1]))


@pytest.mark.parametrize("pf_bytes", [0, 8192])
def test_mid_small_prefetch_region(pf_bytes, monkeypatch):
    """LDS prefetch region capped: weight tiles and K/V pages partly or not at all in LDS, attention merge from registers."""
    from tests import parity
    monkeypatch.setenv("MK_PREFETCH_BYTES", str(pf_bytes))
    w = synth.Workload(f"mid_pf{pf_bytes}", synth.MID, batch=3, steps=3, context=[2048, 40, 1000])
    _check(parity.run(w, mode="isolated", log=_log))


@pytest.mark.parametrize("attn_cus", [13, 40])
def test_mid_attention_unit_counts(attn_cus, monkeypatch):
    """Attention units forced to leads + 1 (one unit takes every Wo row and every chunk past a
    segment's first) and to 40 (larger chunks): same parity bar."""
    from tests import parity
    monkeypatch.setenv("MK_ATTN_CUS", str(attn_cus))
    w = synth.Workload(f"mid_attn{attn_cus}", synth.MID, batch=3, steps=2, context=[1500, 17, 600])
    _check(parity.run(w, mode="isolated", log=_log))
