"""The device greedy argmax (next_tok) on exact logit ties: the lowest id wins.

Two identical LM-head rows give bit-identical logits (each row's dot product runs the same
instruction sequence on the same input), so copying the winning row onto a lower-numbered row
makes an exact tie at the top: the device must then return the lower id.  Copying it onto a
higher-numbered row must leave the winner unchanged.  The rows are chosen in different LM-head
tasks, so the tie is broken by the cross-task merge, and in the same task, so it is broken
inside one task.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _step(dec, tok, p):
    dec.step([tok], [p])
    torch.cuda.synchronize()
    dec.check_error()
    return dec.logits[0].cpu().numpy(), int(dec.next_tok[0])


def test_device_argmax_ties_go_to_the_lowest_id():
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("mid_tie", synth.MID, batch=1, steps=1, context=[300])
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    tok, p = int(w.prompt(0)[300]), 300
    lm = dec.weights[1]                      # [vocab][hidden] bf16, the LM head
    logits, nxt = _step(dec, tok, p)
    win = int(np.argmax(logits))
    assert nxt == win
    V = w.shape.vocab
    tasks, _ = dec.ctx.schedule()
    lm_tasks = tasks[tasks[:, 0] == 5]
    r0, r1 = lm_tasks[:, 7], lm_tasks[:, 8]
    mine = int(np.nonzero((r0 <= win) & (win < r1))[0][0])
    cases = []
    if mine > 0:                             # a lower row in an earlier task
        cases.append((int(r0[mine - 1]), "lower, other task"))
    if win > r0[mine]:                       # a lower row in the same task
        cases.append((int(r0[mine]), "lower, same task"))
    cases.append((int(min(win + 1 + (V - win - 1) // 2, V - 1)), "higher"))
    for j, what in cases:
        if j == win:
            continue
        saved = lm[j].clone()
        lm[j].copy_(lm[win])
        logits, nxt = _step(dec, tok, p)
        print(f"tie {what}: rows {win} and {j}, logits {logits[win]!r} {logits[j]!r}, next {nxt}", flush=True)
        assert logits[j] == logits[win]
        assert nxt == min(j, win), what
        lm[j].copy_(saved)
    _, nxt = _step(dec, tok, p)
    assert nxt == win
