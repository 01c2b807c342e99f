"""The sequential block (attention, then the MoE path behind its own norm) through the C ABI against
the CPU oracle's sequential model.

Same checks and tolerances as the parallel block: every logit, the device argmax, and in isolated
mode every layer's expert choice, router logits (here computed from the norm of x + this layer's
Wo rows), residual and new K/V entries.  Covers the embedding-plus-Wo input of layer 0's MoE path
(tiny, prefill-as-decode), batch 1 and 8 at mid, free running, and the 30B shape at 8K.
"""
import gc

import pytest

import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check(name, rep):
    from tests import parity
    _log(rep.summary())
    parity.record(name, rep)
    assert rep.ok(), "\n".join(rep.failures[:20])


def _seq(w: synth.Workload) -> synth.Workload:
    from dataclasses import replace
    w.shape = replace(w.shape, block="sequential")
    w.name = w.name + "_seq"
    return w


def test_seq_tiny_prefill_then_greedy_isolated():
    from tests import parity
    rep = parity.run(synth.workload("tiny_seq"), mode="isolated", log=_log)
    assert rep.steps == 128 + 16
    _check("tiny_seq_isolated", rep)


def test_seq_tiny_free_running():
    from tests import parity
    _check("tiny_seq_free", parity.run(synth.workload("tiny_seq"), mode="free", log=_log))


def test_seq_mid_isolated_16_steps():
    from tests import parity
    _check("mid_seq_isolated_16", parity.run(synth.workload("mid_seq"), steps=16, mode="isolated", log=_log))


def test_seq_mid_free_running_16_steps():
    from tests import parity
    _check("mid_seq_free_16", parity.run(synth.workload("mid_seq"), steps=16, mode="free", log=_log))


def test_seq_mid_batch8_ragged():
    from tests import parity
    w = _seq(synth.Workload("mid_bs8", synth.MID, batch=8, steps=2, context=[1, 700, 2048, 33, 1500, 16, 4000, 257]))
    _check("mid_bs8_seq", parity.run(w, mode="isolated", log=_log))


def test_seq_30b_bs1_8k_isolated_2_steps():
    import torch
    from tests import parity
    gc.collect()
    torch.cuda.empty_cache()
    rep = parity.run(synth.workload("moe30b_8k_seq"), steps=2, mode="isolated", log=_log)
    _check("moe30b_8k_seq_isolated_2", rep)


def test_seq_30b_bs8_ragged_isolated_1_step():
    """Batch 8 at the 30B shape: the schedule where every unit takes part in every phase."""
    import torch
    from tests import parity
    gc.collect()
    torch.cuda.empty_cache()
    rep = parity.run(synth.workload("moe30b_bs8_ragged_seq"), steps=1, mode="isolated", log=_log)
    assert rep.route_checked == 8 * 48
    _check("moe30b_bs8_ragged_seq_isolated_1", rep)


def test_seq_mid_free_running_no_teacher_forcing():
    """Up to 64 steps, each side feeding its own greedy token until they first disagree: the
    agreement length is recorded, and the disagreement must be admissible (a near-tie of the top-2
    logits, or a routing divergence within the measured router drift)."""
    from tests import parity
    rep = parity.run(synth.workload("mid_seq"), mode="free", log=_log, teacher=False)
    assert rep.agree_steps == 64 or rep.disagree_cause, rep.summary()
    _check("mid_seq_free_no_teacher", rep)
    _log(f"free-running agreement: {rep.agree_steps} of 64 steps ({rep.disagree_cause or 'no disagreement'})")
