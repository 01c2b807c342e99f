"""The 30B-total / 3.3B-active shape at full size against the CPU oracle.

Every check compares every logit, the device argmax and, in isolated mode, every layer's
expert choice, router logits, output residual and new K/V entries.  The oracle's cost
bounds the number of steps: the first 8 steps at batch 1 and 8K end to end (the GPU's own
residual hand-off across 48 layers and 256 compute units), 2 steps with every layer on the
oracle's inputs; batch 8 with ragged contexts and batch 1 at 262144 cached tokens over all
48 layers on the oracle's own residuals.
"""
import gc

import pytest

import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _fresh():
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _check(name, rep, **extra):
    from tests import parity
    _log(rep.summary())
    parity.record(name, rep, **extra)
    assert rep.ok(), "\n".join(rep.failures[:20])


def test_30b_bs1_8k_free_running_8_steps():
    """No layer-input hook: the megakernel's own residual hand-off through all 48 layers, 8 steps."""
    from tests import parity
    _fresh()
    rep = parity.run(synth.workload("moe30b_8k"), steps=8, mode="free", log=_log)
    assert rep.steps == 8
    _check("moe30b_8k_free_8", rep)


def test_30b_bs1_8k_isolated_first_steps():
    from tests import parity
    _fresh()
    rep = parity.run(synth.workload("moe30b_8k"), steps=2, mode="isolated", log=_log)
    _check("moe30b_8k_isolated_2", rep)


def test_30b_bs8_ragged_isolated_all_layers():
    """Batch 8, contexts U[1024, 32768]: one step, every one of the 48 layers on the oracle's residuals."""
    from tests import parity
    _fresh()
    rep = parity.run(synth.workload("moe30b_bs8_ragged"), steps=1, mode="isolated", log=_log)
    assert rep.route_checked == 8 * 48
    _check("moe30b_bs8_ragged_isolated_1", rep)


def test_30b_256k_isolated_2_steps():
    """Batch 1 at 262144 cached tokens: 2 steps, every layer on the oracle's residuals."""
    from tests import parity
    _fresh()
    rep = parity.run(synth.workload("moe30b_256k"), steps=2, mode="isolated", log=_log)
    assert rep.route_checked == 2 * 48
    _check("moe30b_256k_isolated_2", rep)
