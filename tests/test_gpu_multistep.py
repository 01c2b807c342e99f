"""Several decode steps in one persistent launch (mk_decode_steps) against the same steps run as
separate launches that feed back the device's greedy token.  The launch must be bit-identical:
every step's greedy token, the last step's logits and every K/V slot the steps wrote.  (The
single-step path is checked against the oracle by the parity tests.)"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _kv_slots(dec, n, lens, steps):
    out = []
    for b in range(n):
        for s in range(steps):
            for l in range(dec.shape.n_layers):
                k, v = dec.kv_at(l, b, lens[b] + s)
                out.append(np.concatenate([k.reshape(-1), v.reshape(-1)]))
    return np.stack(out)


@pytest.mark.parametrize("batch,context,pool,top_p", [(1, [2048], 0, None), (3, [900, 17, 1500], 0, None),
                                                     (3, [900, 17, 1500], 16, None), (3, [900, 17, 1500], 0, 0.9)])
def test_steps_in_one_launch_equal_single_launches(batch, context, pool, top_p):
    """pool: 64ths of the gate/up rows in the shared pool (its claim counters run across the steps);
    top_p: nucleus sampling at temperature 0.8 (each step's draw feeds the next step on the device)."""
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    steps = 8
    w = synth.Workload(f"mid_ms{batch}", synth.MID, batch=batch, steps=steps + 1, context=context)
    print(f"workload {w.name}: batch {batch}, {steps} steps, pool {pool}", flush=True)
    dec = DeviceDecoder(w, pool_64ths=pool)
    if top_p is not None:
        dec.ctx.set_sampling(0.8, 0x5EED)
        dec.ctx.set_top_p(top_p)
    dev, n = dec.dev, batch
    lens0 = torch.tensor(context, dtype=torch.int32, device=dev)
    tok0 = torch.tensor([int(w.prompt(b)[context[b]]) for b in range(n)], dtype=torch.int32, device=dev)
    # separate launches: the device argmax of one step is the next step's token
    dec.fill_synthetic_kv()
    toks = torch.zeros(steps + 1, n, dtype=torch.int32, device=dev)
    toks[0] = tok0
    lens = torch.stack([lens0 + s for s in range(steps)]).contiguous()
    for s in range(steps):
        dec.ctx.decode_step(n, toks[s].data_ptr(), dec.page_table.data_ptr(), lens[s].data_ptr(),
                            dec.logits.data_ptr(), toks[s + 1].data_ptr(), dec.stream)
    torch.cuda.synchronize()
    dec.check_error()
    single_toks = toks[1:].cpu().numpy()
    single_logits = dec.logits[:n].cpu().clone()
    single_kv = _kv_slots(dec, n, context, steps)
    # one launch of all steps, from a freshly filled cache
    dec.fill_synthetic_kv()
    out = torch.full((steps, n), -1, dtype=torch.int32, device=dev)
    dec.logits.zero_()
    dec.ctx.decode_steps(n, steps, tok0.data_ptr(), dec.page_table.data_ptr(), lens0.data_ptr(),
                         dec.logits.data_ptr(), out.data_ptr(), dec.stream)
    torch.cuda.synchronize()
    dec.check_error()
    multi_toks = out.cpu().numpy()
    print(f"tokens per step: {multi_toks.tolist()}", flush=True)
    assert np.array_equal(multi_toks, single_toks)
    assert torch.equal(dec.logits[:n].cpu(), single_logits)
    assert np.array_equal(_kv_slots(dec, n, context, steps), single_kv)


def test_steps_argument_checks():
    from persistent_moe_decode_amd import mk
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("tiny_ms", synth.TINY, batch=1, steps=4, context=[20])
    dec = DeviceDecoder(w)
    t = torch.zeros(4, dtype=torch.int32, device=dec.dev)
    for steps, nxt in ((0, t), (2, None)):
        with pytest.raises(mk.MkError) as e:
            dec.ctx.decode_steps(1, steps, t.data_ptr(), dec.page_table.data_ptr(), t.data_ptr(),
                                 dec.logits.data_ptr(), nxt.data_ptr() if nxt is not None else None, dec.stream)
        assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"]
