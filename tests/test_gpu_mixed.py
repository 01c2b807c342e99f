"""Chunked prefill mixed with decode (mk_mixed_step) through the C ABI against the CPU oracle.

A mixed step's entries may belong to one sequence (same page-table row, distinct positions):
its result must equal running the entries one at a time in position order as decode steps,
which is what the oracle's decode_step does with the same entries in that order.  Both sides run
free (each on its own residual stream); logits are compared by the max-normalized relative error
(2e-2) and every new K/V entry likewise; a layer whose GPU expert set differs from the oracle's is
admitted only at a router near-tie (margin below ROUTE_TIE), and that entry's logits are then not
compared.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _log(msg):
    print(msg, flush=True)


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _routes_agree(gpu_sel, ref: O.StepOut, entries, gpu_rows, tag):
    """True when every layer's expert set agrees for these oracle entries (GPU rows gpu_rows);
    a disagreement must sit at a router near-tie."""
    ok = True
    for l in range(gpu_sel.shape[0]):
        for e, r in zip(entries, gpu_rows):
            if sorted(gpu_sel[l, r].tolist()) != sorted(ref.sel[l, e].tolist()):
                assert ref.margin[l, e] <= O.ROUTE_TIE, (tag, l, e, ref.margin[l, e])
                ok = False
    return ok


def _kv_rel(dec, kv: O.PagedKV, layer, row_b, pt_row, pos):
    k, v = dec.kv_at(layer, row_b, pos)
    page, o = kv.slots(pt_row, [pos])
    i = kv._at[layer]
    kr, vr = O.bf16_to_f64(kv.k[i, page[0], :, o[0], :]), O.bf16_to_f64(kv.v[i, page[0], :, o[0], :])
    return max(_rel(O.bf16_to_f64(k), kr), _rel(O.bf16_to_f64(v), vr))


def test_chunked_prefill_equals_token_at_a_time():
    """The tiny model's 128-token prompt as 16 mixed steps of 8 entries of one sequence, against the
    oracle's prefill-as-decode: every K/V slot of every layer, the logits after the last prompt token."""
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    s = synth.TINY
    prompt = synth.workload("tiny").prompt(0)
    T, C = 128, 8
    w = synth.Workload("tiny_chunked", s, batch=C, steps=T, context=[0] * C, shuffle_pages=True)
    _log(f"workload {w.name}: prompt {T} tokens in chunks of {C}")
    dec = DeviceDecoder(w)
    dev = dec.dev
    row = dec.page_table_np[0]
    pt = torch.from_numpy(np.ascontiguousarray(np.tile(row, (C, 1)))).to(dev)
    tok = torch.zeros(C, dtype=torch.int32, device=dev)
    lens = torch.zeros(C, dtype=torch.int32, device=dev)
    nxt = torch.zeros(C, dtype=torch.int32, device=dev)
    sels = []
    for c in range(T // C):
        tok.copy_(torch.from_numpy(prompt[c * C:(c + 1) * C].astype(np.int32)))
        lens.copy_(torch.arange(c * C, (c + 1) * C, dtype=torch.int32))
        dec.ctx.mixed_step(C, tok.data_ptr(), pt.data_ptr(), lens.data_ptr(), dec.logits.data_ptr(),
                           nxt.data_ptr(), dec.stream)
        torch.cuda.synchronize()
        dec.check_error()
        sels.append(dec.sel()[:, :C, :])
    g_logits = dec.logits[C - 1].cpu().numpy().astype(np.float64)
    g_next = int(nxt[C - 1].item())
    # the oracle, one token at a time
    W = O.Weights(s)
    kv = O.PagedKV(s, w.num_pages)
    all_agree = True
    for t in range(T):
        ref = O.decode_step(W, kv, [int(prompt[t])], row[None], [t])
        all_agree &= _routes_agree(sels[t // C], ref, [0], [t % C], f"token {t}")
    worst = max(_kv_rel(dec, kv, l, 0, row, p) for l in range(s.n_layers) for p in range(T))
    _log(f"chunked prefill: K/V max rel {worst:.2e}; routes agree {all_agree}")
    assert worst < TOL
    if all_agree:
        r = _rel(g_logits, ref.logits[0])
        _log(f"last-token logits rel {r:.2e}; next token gpu {g_next} oracle {int(ref.next_token[0])} "
             f"(top-2 gap {ref.top2_gap[0]:.2e})")
        assert r < TOL
        if ref.top2_gap[0] > 2 * np.max(np.abs(g_logits - ref.logits[0])):
            assert g_next == int(ref.next_token[0])


@pytest.mark.parametrize("shape_name", ["mid", "mid_fp8", "mid_fp4", "mid_seq"])
def test_decode_and_prefill_chunk_in_one_step(shape_name):
    """One step: sequence A decodes at position 300 while sequence B's first 7 prompt tokens run as
    entries 1..7 (B's row, positions 0..6).  Against the oracle's step over the same entries in order."""
    from dataclasses import replace
    from persistent_moe_decode_amd.runtime import DeviceDecoder
    suffix = shape_name.split("_")[1] if "_" in shape_name else ""
    s = replace(synth.MID, block="sequential") if suffix == "seq" else replace(synth.MID, weights=suffix or "bf16")
    w = synth.Workload("mixed_" + shape_name, s, batch=8, steps=2, context=[300] + [0] * 7)
    _log(f"workload {w.name}: A at 300, B positions 0..6")
    dec = DeviceDecoder(w)
    dec.fill_synthetic_kv()
    dev = dec.dev
    pt_np = dec.page_table_np.copy()
    pt_np[2:] = pt_np[1]
    b_prompt = synth.uniform_u32(synth.SEED_PROMPT, synth.tid(synth.K_PROMPT, 1), 0, 7, s.vocab).astype(np.int32)
    toks = np.concatenate([[int(w.prompt(0)[300])], b_prompt]).astype(np.int32)
    lens_np = np.array([300, 0, 1, 2, 3, 4, 5, 6], dtype=np.int32)
    pt = torch.from_numpy(np.ascontiguousarray(pt_np)).to(dev)
    tok = torch.from_numpy(toks).to(dev)
    lens = torch.from_numpy(lens_np).to(dev)
    nxt = torch.zeros(8, dtype=torch.int32, device=dev)
    dec.ctx.mixed_step(8, tok.data_ptr(), pt.data_ptr(), lens.data_ptr(), dec.logits.data_ptr(), nxt.data_ptr(),
                       dec.stream)
    torch.cuda.synchronize()
    dec.check_error()
    g_logits = dec.logits[:8].cpu().numpy().astype(np.float64)
    g_sel = dec.sel()[:, :8, :]
    W = O.Weights(s)
    kv = O.PagedKV(s, w.num_pages)
    kv.fill_synthetic(w.page_table(), w.context)
    ref = O.decode_step(W, kv, toks.tolist(), pt_np, lens_np.tolist())
    compared = 0
    for b in range(8):
        worst_kv = max(_kv_rel(dec, kv, l, b if b < 2 else 1, pt_np[b], int(lens_np[b])) for l in range(s.n_layers))
        assert worst_kv < TOL, (b, worst_kv)
        if _routes_agree(g_sel, ref, [b], [b], f"entry {b}"):
            r = _rel(g_logits[b], ref.logits[b])
            _log(f"entry {b} (pos {lens_np[b]}): logits rel {r:.2e}, K/V rel {worst_kv:.2e}, next gpu "
                 f"{int(nxt[b].item())} oracle {int(ref.next_token[b])}")
            assert r < TOL, (b, r)
            compared += 1
    assert compared >= 6
