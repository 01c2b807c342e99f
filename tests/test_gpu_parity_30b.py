"""The 30B-total / 3.3B-active shape at full size against the CPU oracle.

The first decode steps are compared in full (every logit; every layer's
expert choice, router logits, output residual and new K/V entries); the
oracle's cost bounds how many.
"""
import pytest

import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def test_30b_bs1_8k_isolated_first_steps():
    from tests import parity
    rep = parity.run(synth.workload("moe30b_8k"), steps=2, mode="isolated", log=_log)
    _log(rep.summary())
    assert rep.ok(), "\n".join(rep.failures[:20])


def _fresh():
    import gc

    import torch
    gc.collect()
    torch.cuda.empty_cache()


def test_30b_bs8_ragged_sampled_layers():
    """Batch 8, contexts U[1024, 32768], full size: layers 0, 24, 47 and the LM head from seeded layer inputs."""
    from tests import parity
    _fresh()
    rep = parity.run_sampled(synth.workload("moe30b_bs8_ragged"), layers=(0, 24, 47), log=_log)
    _log(rep.summary())
    assert rep.ok(), "\n".join(rep.failures[:20])


def test_30b_256k_sampled_layers():
    """Batch 1, 262144 cached tokens, full size: layers 0, 24, 47 and the LM head from seeded layer inputs."""
    from tests import parity
    _fresh()
    rep = parity.run_sampled(synth.workload("moe30b_256k"), layers=(0, 24, 47), log=_log)
    _log(rep.summary())
    assert rep.ok(), "\n".join(rep.failures[:20])
