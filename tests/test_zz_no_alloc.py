"""mk_bind_scratch, the binding that allocates nothing (its workspace is the library's static
per-GPU array), against mk_bind with a caller-allocated workspace: on the same weights, cache
and inputs the steps must be bit-identical (greedy tokens of every step, the last step's logits,
every K/V slot written).  Two bindings of the static array in a row, the second with a smaller
model and batch, so the second runs over what the first left there; the first context must then
refuse to run."""
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


def _run(dec, w, steps):
    """`steps` greedy steps in one launch from a freshly filled cache: (tokens, logits, K/V slots)."""
    n, dev = w.batch, dec.dev
    dec.fill_synthetic_kv()
    lens0 = torch.tensor(w.context, dtype=torch.int32, device=dev)
    tok0 = torch.tensor([int(w.prompt(b)[w.context[b]]) for b in range(n)], dtype=torch.int32, device=dev)
    out = torch.full((steps, n), -1, dtype=torch.int32, device=dev)
    dec.logits.zero_()
    dec.ctx.decode_steps(n, steps, tok0.data_ptr(), dec.page_table.data_ptr(), lens0.data_ptr(),
                         dec.logits.data_ptr(), out.data_ptr(), dec.stream)
    torch.cuda.synchronize()
    dec.check_error()
    return out.cpu().numpy(), dec.logits[:n].cpu().clone(), _kv_slots(dec, n, w.context, steps)


def _same(ref, got):
    assert np.array_equal(got[0], ref[0]), (got[0].tolist(), ref[0].tolist())
    assert torch.equal(got[1], ref[1])
    assert np.array_equal(got[2], ref[2])


def test_static_workspace_matches_caller_workspace_twice_in_a_row():
    from persistent_moe_decode_amd import mk
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    cap = mk.scratch_capacity()
    first = synth.Workload("mid_na", synth.MID, batch=3, steps=5, context=[700, 13, 1900])
    second = synth.Workload("tiny_na", synth.TINY, batch=1, steps=4, context=[45])
    decs = []
    try:
        print(f"first binding: {first.name}, batch {first.batch}, 4 steps", flush=True)
        ref1 = DeviceDecoder(first)
        st1 = DeviceDecoder(first, static_workspace=True)
        decs += [ref1, st1]
        assert ref1.ws_bytes <= cap
        r1 = _run(ref1, first, 4)
        _same(r1, _run(st1, first, 4))
        print(f"second binding: {second.name}, batch {second.batch}, 3 steps", flush=True)
        ref2 = DeviceDecoder(second)
        st2 = DeviceDecoder(second, static_workspace=True)
        decs += [ref2, st2]
        assert st2.ws_bytes < st1.ws_bytes
        r2 = _run(ref2, second, 3)
        _same(r2, _run(st2, second, 3))
        # the first context lost the array to the second
        t = torch.zeros(4, dtype=torch.int32, device=st1.dev)
        with pytest.raises(mk.MkError) as e:
            st1.ctx.decode_step(1, t.data_ptr(), st1.page_table.data_ptr(), t.data_ptr(), st1.logits.data_ptr(),
                                None, st1.stream)
        assert e.value.code == mk.CODES["MK_ERR_STATE"]
        with pytest.raises(mk.MkError) as e:
            st1.ctx.get_error(st1.stream)
        assert e.value.code == mk.CODES["MK_ERR_STATE"]
        # the second one still runs, and again matches
        _same(r2, _run(st2, second, 3))
    finally:
        for d in decs:
            d.close()
