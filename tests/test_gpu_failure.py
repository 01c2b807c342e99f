"""Failure detection through the C ABI, forced from the host so that every kernel still exits normally.

Each case makes the kernel raise a device error on purpose: a spin limit so small that the
kernel's own bounded dependency waits give up, an out-of-range token id, an out-of-range page
id and an out-of-range sequence length.  The bad ids are clamped before they index memory
(the token to row 0, the page to no load and no write, the length into the table's range);
the error word reports the first error and the grid drains.  Then mk_get_error must report
the code, the next step must be refused until mk_reset, and after mk_reset the same step must
match the oracle again.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _setup(context=40):
    from oracle import oracle as O
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    w = synth.Workload("tiny_fail", synth.TINY, batch=1, steps=2, context=[context], shuffle_pages=True)
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    W = O.Weights(w.shape)
    pt = w.page_table()
    kv = O.PagedKV(w.shape, w.num_pages)
    kv.fill_synthetic(pt, w.context)
    tok = int(w.prompt(0)[context])
    ref = O.decode_step(W, kv, [tok], pt, [context])
    return w, dec, ref, tok


def _expect_error(dec, code_name):
    from persistent_moe_decode_amd import mk
    code, cu, task = dec.ctx.get_error(dec.stream)
    print(f"device error {mk.ERRORS.get(code, code)} from cu {cu} task {task}", flush=True)
    assert code == mk.CODES[code_name]
    # the context refuses to step until it is reset
    with pytest.raises(mk.MkError) as e:
        dec.step([0], [0])
    assert e.value.code == mk.CODES["MK_ERR_STATE"]
    dec.ctx.reset(dec.stream)


def _recovered(dec, ref, tok, context):
    dec.step([tok], [context])
    torch.cuda.synchronize()
    dec.check_error()
    got = dec.logits[0].cpu().numpy().astype(np.float64)
    err = np.max(np.abs(got - ref.logits[0])) / np.max(np.abs(ref.logits[0]))
    print(f"after reset: max relative logit error {err:.3e}", flush=True)
    assert err <= 2e-2
    assert int(dec.next_tok[0]) == int(np.argmax(got))


def test_spin_limit_timeout_drains_and_recovers():
    w, dec, ref, tok = _setup()
    dec.ctx.set_spin_limit_us(1)          # every dependency wait gives up after ~1 us
    dec.step([tok], [40])
    torch.cuda.synchronize()
    _expect_error(dec, "MK_ERR_DEVICE_TIMEOUT")
    dec.ctx.set_spin_limit_us(2_000_000)
    _recovered(dec, ref, tok, 40)


def test_bad_token_id_is_reported():
    w, dec, ref, tok = _setup()
    dec.step([w.shape.vocab + 5], [40])
    torch.cuda.synchronize()
    _expect_error(dec, "MK_ERR_DEVICE_TOKEN")
    _recovered(dec, ref, tok, 40)


def test_bad_page_id_is_reported():
    w, dec, ref, tok = _setup()
    good = dec.page_table.clone()
    dec.page_table[0, 40 // 16] = w.num_pages + 7   # the page that receives the new token
    dec.step([tok], [40])
    torch.cuda.synchronize()
    _expect_error(dec, "MK_ERR_DEVICE_PAGE")
    dec.page_table.copy_(good)
    _recovered(dec, ref, tok, 40)


def test_bad_seq_len_is_reported():
    w, dec, ref, tok = _setup()
    cap = w.max_pages_per_seq * w.shape.page_size
    dec.step([tok], [cap])                  # the new token would sit past the page-table row
    torch.cuda.synchronize()
    _expect_error(dec, "MK_ERR_DEVICE_SEQ")
    _recovered(dec, ref, tok, 40)
