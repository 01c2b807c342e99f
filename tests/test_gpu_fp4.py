"""FP4 (E2M1) weights: the FP4 kernel through the C ABI against the CPU oracle's FP4 model.

The oracle unpacks the same packed codes (element 2j in the low nibble of byte j) and scales
(each weight is code value * row scale, exactly) and runs the same step; the kernel converts
codes to bf16 in registers and multiplies each row's fp32 sum by its scale.  Every check is the
bf16 path's: every logit, the device argmax, and in isolated mode every layer's expert choice,
router logits, residual and new K/V entries.  Shapes cover each FP4 row path: 128- and
256-element rows (tiny: 4 and 8 lanes a row), 512 and 1024 (mid), 768 (24 chunks: 8 lanes of
3), 2048 and 4096 (30B), at batch 1 (register rows, LDS tiles) and batch 8 (matrix-core tiles
for rows of a multiple of 1024 elements, register rows otherwise).
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


def _fp4(w: synth.Workload) -> synth.Workload:
    from dataclasses import replace
    w.shape = replace(w.shape, weights="fp4")
    w.name = w.name + "_fp4"
    return w


def test_fp4_tiny_prefill_then_greedy_isolated():
    from tests import parity
    rep = parity.run(synth.workload("tiny_fp4"), mode="isolated", log=_log)
    assert rep.steps == 128 + 16
    _check("tiny_fp4_isolated", rep)


def test_fp4_tiny_ragged_batch_edges():
    from tests import parity
    w = _fp4(synth.Workload("tiny_ragged", synth.TINY, batch=8, steps=3, context=[0, 1, 15, 16, 17, 31, 32, 100],
                            spare_pages=3))
    _check("tiny_ragged_fp4", parity.run(w, mode="isolated", log=_log))


def test_fp4_mid_isolated_16_steps():
    from tests import parity
    rep = parity.run(synth.workload("mid_fp4"), steps=16, mode="isolated", log=_log)
    _check("mid_fp4_isolated_16", rep)


def test_fp4_mid_free_running_16_steps():
    from tests import parity
    rep = parity.run(synth.workload("mid_fp4"), steps=16, mode="free", log=_log)
    _check("mid_fp4_free_16", rep)


def test_fp4_mid_batch8_ragged():
    from tests import parity
    w = _fp4(synth.Workload("mid_bs8", synth.MID, batch=8, steps=2, context=[1, 700, 2048, 33, 1500, 16, 4000, 257]))
    _check("mid_bs8_fp4", parity.run(w, mode="isolated", log=_log))


def test_fp4_30b_bs1_8k_isolated_2_steps():
    import torch
    from tests import parity
    gc.collect()
    torch.cuda.empty_cache()
    rep = parity.run(synth.workload("moe30b_8k_fp4"), steps=2, mode="isolated", log=_log)
    _check("moe30b_8k_fp4_isolated_2", rep)


def test_fp4_30b_bs8_ragged_isolated_1_step():
    import torch
    from tests import parity
    gc.collect()
    torch.cuda.empty_cache()
    rep = parity.run(synth.workload("moe30b_bs8_ragged_fp4"), steps=1, mode="isolated", log=_log)
    assert rep.route_checked == 8 * 48
    _check("moe30b_bs8_ragged_fp4_isolated_1", rep)
