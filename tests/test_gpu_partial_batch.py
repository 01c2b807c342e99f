"""A schedule built for 8 sequences, stepped with fewer: idle segment leads, the
matrix-core rows with tokens past the batch masked off (3 sequences), and the
batch-1 vector path on the same table (1 sequence); logits against the oracle."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [3, 1])
def test_fewer_sequences_than_the_schedule(n):
    from oracle import oracle as O
    from persistent_moe_decode_amd.runtime import DeviceDecoder

    w = synth.Workload(f"mid_part{n}", synth.MID, batch=8, steps=2,
                       context=[900, 31, 2048, 16, 5, 400, 77, 1200], shuffle_pages=True)
    print(f"workload {w.name}: n={n} of max_batch 8", flush=True)
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    W = O.Weights(w.shape)
    pt = w.page_table()
    kv = O.PagedKV(w.shape, w.num_pages)
    kv.fill_synthetic(pt, w.context)
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(n)]
    for step in range(w.steps):
        lens = [w.context[b] + step for b in range(n)]
        dec.step(toks, lens, n=n)
        torch.cuda.synchronize()
        dec.check_error()
        got = dec.logits[:n].cpu().numpy().astype(np.float64)
        ref = O.decode_step(W, kv, toks, pt[:n], lens)
        for b in range(n):
            err = np.max(np.abs(got[b] - ref.logits[b])) / np.max(np.abs(ref.logits[b]))
            assert err <= 2e-2, f"step {step} seq {b}: max relative logit error {err:.3e}"
        nxt = dec.next_tok[:n].cpu().numpy()
        for b in range(n):
            top2 = np.sort(ref.logits[b])[-2:]
            if top2[1] - top2[0] > 1e-2:  # a clear winner: the device argmax must pick it
                assert int(nxt[b]) == int(np.argmax(ref.logits[b])), f"step {step} seq {b}: greedy token"
        toks = [int(t) for t in ref.next_token]
