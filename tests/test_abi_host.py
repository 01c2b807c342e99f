"""Host-only checks of the C ABI library: exports, config checks, schedule, simulator, attention split.

None of these make a GPU call.
"""
import ctypes

import numpy as np
import pytest

import synth
from persistent_moe_decode_amd import mk

OP_PRE, OP_ATTN, OP_GATEUP, OP_OUT, OP_LMHEAD, OP_WO = 1, 2, 3, 4, 5, 6
F_OP, F_LAYER, F_WAIT0, F_WAIT1, F_FAN0, F_FAN1, F_SIGNAL, F_R0, F_R1, F_IDX, F_COUNT, F_LATE, F_LATE_FAN, F_SLOT = range(14)


def test_library_exports_every_declared_symbol():
    L = mk.lib()
    names = mk.header_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n


def _ctx(shape, max_batch=1, max_pages=16, num_pages=16):
    return mk.Context(mk.config_from_shape(shape, max_batch, max_pages, num_pages))


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 200, "MK_ERR_UNSUPPORTED"), ("head_dim", 96, "MK_ERR_UNSUPPORTED"),
    ("page_size", 32, "MK_ERR_UNSUPPORTED"), ("max_batch", 9, "MK_ERR_UNSUPPORTED"),
    ("n_kv_heads", 3, "MK_ERR_UNSUPPORTED"), ("top_k", 9, "MK_ERR_UNSUPPORTED"),
    ("n_layers", 0, "MK_ERR_INVALID_ARG"), ("num_pages", 0, "MK_ERR_INVALID_ARG"),
])
def test_create_rejects_bad_configs(field, value, code):
    cfg = mk.config_from_shape(synth.TINY, 1, 8, 8)
    setattr(cfg, field, value)
    with pytest.raises(mk.MkError) as e:
        mk.Context(cfg)
    assert e.value.code == mk.CODES[code]


def test_calls_out_of_order_fail_cleanly():
    c = _ctx(synth.TINY)
    with pytest.raises(mk.MkError) as e:
        c.info()
    assert e.value.code == mk.CODES["MK_ERR_STATE"]
    c.build_schedule(64, 100)
    with pytest.raises(mk.MkError) as e:
        c.decode_step(1, 0, 0, 0, 0, None, 0)
    assert e.value.code == mk.CODES["MK_ERR_STATE"]


@pytest.mark.parametrize("name", synth.WORKLOADS)
@pytest.mark.parametrize("ncu", [256, 80, 7])
def test_schedule_builds_and_simulates(name, ncu):
    w = synth.workload(name)
    c = _ctx(w.shape, w.batch, w.max_pages_per_seq, w.num_pages)
    if ncu < w.batch * w.shape.n_kv_heads + 3:
        with pytest.raises(mk.MkError):
            c.build_schedule(ncu, int(np.mean(w.context)))
        return
    ws = c.build_schedule(ncu, int(np.mean(w.context)))
    info = c.info()
    assert info.num_cus == ncu and info.workspace_bytes == ws and info.lds_bytes <= 160 * 1024
    assert c.validate() == info.n_tasks
    tasks, qoff = c.schedule()
    L = w.shape.n_layers
    ops = tasks[:, F_OP]
    assert np.sum(ops == OP_ATTN) == L * info.n_attn
    assert np.sum(ops == OP_GATEUP) == L * info.n_gateup
    assert info.n_attn + info.n_gateup == ncu
    assert w.batch * w.shape.n_kv_heads < info.n_attn <= ncu - 2
    # attention units run their chunk and Wo rows, no stage-1 or output rows; every other
    # unit one stage-1, one gate/up and one output task
    for q in range(ncu):
        mine = tasks[qoff[q]:qoff[q + 1]]
        l0 = mine[:, F_LAYER] == 0
        n = tuple(int(np.sum((mine[:, F_OP] == op) & l0)) for op in (OP_PRE, OP_ATTN, OP_GATEUP, OP_OUT, OP_WO))
        if q < info.n_attn:
            assert n[:4] == (0, 1, 0, 0) and n[4] <= 1, q
        else:
            assert n[:3] == (1, 0, 1) and n[4] == 0, q
    # PRE rows cover [Wqkv; router] exactly once per layer; OUT rows cover hidden; LM rows cover vocab
    for l in range(L):
        pre = tasks[(ops == OP_PRE) & (tasks[:, F_LAYER] == l)]
        cover = np.zeros(w.shape.qkv_rows + w.shape.n_experts, dtype=int)
        for t in pre:
            cover[t[F_R0]:t[F_R1]] += 1
            assert t[F_R1] <= w.shape.qkv_rows or t[F_R0] >= w.shape.qkv_rows
        assert np.all(cover == 1)
        for op in (OP_OUT, OP_WO):
            out = tasks[(ops == op) & (tasks[:, F_LAYER] == l)]
            cover = np.zeros(w.shape.hidden, dtype=int)
            for t in out:
                cover[t[F_R0]:t[F_R1]] += 1
            assert np.all(cover == 1)
    lm = tasks[ops == OP_LMHEAD]
    cover = np.zeros(w.shape.vocab, dtype=int)
    for t in lm:
        cover[t[F_R0]:t[F_R1]] += 1
    assert np.all(cover == 1)
    # every queue runs layers in order
    for q in range(ncu):
        layers = tasks[qoff[q]:qoff[q + 1], F_LAYER]
        assert np.all(np.diff(layers) >= 0)


def test_schedule_is_deterministic():
    w = synth.workload("moe30b_8k")
    a = _ctx(w.shape, 1, w.max_pages_per_seq, w.num_pages)
    b = _ctx(w.shape, 1, w.max_pages_per_seq, w.num_pages)
    assert a.build_schedule(256, 8192) == b.build_schedule(256, 8192)
    ta, qa = a.schedule()
    tb, qb = b.schedule()
    assert np.array_equal(ta, tb) and np.array_equal(qa, qb)


def _tiny_table():
    w = synth.workload("tiny")
    c = _ctx(w.shape, 1, w.max_pages_per_seq, w.num_pages)
    c.build_schedule(16, 128)
    tasks, qoff = c.schedule()
    return tasks, qoff, c.info().n_counters


def test_simulator_accepts_the_built_table():
    tasks, qoff, nctr = _tiny_table()
    code, done = mk.simulate_table(tasks, qoff, nctr)
    assert code == 0 and done == len(tasks)


def test_simulator_catches_a_dropped_signal():
    tasks, qoff, nctr = _tiny_table()
    t = tasks.copy()
    i = int(np.nonzero(t[:, F_OP] == OP_PRE)[0][0])
    t[i, F_SIGNAL] = -1
    code, _ = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"]


def test_simulator_catches_consumer_before_producer():
    tasks, qoff, nctr = _tiny_table()
    t = tasks.copy()
    # on the last queue (a unit with stage-1 rows), put the OUT task of layer 0 before its own PRE task
    k = len(qoff) - 2
    q = t[qoff[k]:qoff[k + 1]]
    i_pre = int(np.nonzero((q[:, F_OP] == OP_PRE) & (q[:, F_LAYER] == 0))[0][0])
    i_out = int(np.nonzero((q[:, F_OP] == OP_OUT) & (q[:, F_LAYER] == 0))[0][0])
    q[[i_pre, i_out]] = q[[i_out, i_pre]]
    t[qoff[k]:qoff[k + 1]] = q
    code, done = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"] and done < len(t)


def test_simulator_catches_wrong_fanin():
    tasks, qoff, nctr = _tiny_table()
    t = tasks.copy()
    i = int(np.nonzero(t[:, F_OP] == OP_OUT)[0][0])
    t[i, F_FAN0] -= 1
    code, _ = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"]


def test_every_counter_has_one_flag_word_per_signalling_task():
    tasks, qoff, nctr = _tiny_table()
    sig = tasks[:, F_SIGNAL]
    for c in np.unique(sig[sig >= 0]):
        slots = np.sort(tasks[sig == c, F_SLOT])
        assert np.array_equal(slots, np.arange(len(slots)))


def test_simulator_catches_a_shared_flag_word():
    tasks, qoff, nctr = _tiny_table()
    t = tasks.copy()
    outs = np.nonzero((t[:, F_OP] == OP_OUT) & (t[:, F_LAYER] == 0))[0]
    t[outs[1], F_SLOT] = t[outs[0], F_SLOT]      # two tasks would set the same word
    code, _ = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"]
    t = tasks.copy()
    t[outs[0], F_SLOT] = len(outs)                # a word past the counter's signallers
    code, _ = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"]


def test_simulator_counts_the_in_body_wait():
    tasks, qoff, nctr = _tiny_table()
    outs = np.nonzero(tasks[:, F_OP] == OP_OUT)[0]
    assert np.all(tasks[outs, F_LATE] < 0)            # the built table has no in-body counter wait
    # an output task that waited inside its body for its layer's Wo rows: still deadlock free
    wo = tasks[(tasks[:, F_OP] == OP_WO) & (tasks[:, F_LAYER] == tasks[outs[0], F_LAYER])]
    t = tasks.copy()
    t[outs[0], F_LATE] = wo[0, F_SIGNAL]
    t[outs[0], F_LATE_FAN] = len(wo)
    code, done = mk.simulate_table(t, qoff, nctr)
    assert code == 0 and done == len(t)
    # the wrong fan-in on it is caught
    t[outs[0], F_LATE_FAN] += 1
    code, _ = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"]
    # an in-body wait on a counter that only a later task of the same queue signals deadlocks
    t = tasks.copy()
    k = len(qoff) - 2
    q0 = t[qoff[k]:qoff[k + 1]]
    i_out = int(np.nonzero((q0[:, F_OP] == OP_OUT) & (q0[:, F_LAYER] == 0))[0][0])
    nxt_pre = int(np.nonzero((q0[:, F_OP] == OP_PRE) & (q0[:, F_LAYER] == 1))[0][0])
    q0[i_out, F_LATE] = q0[nxt_pre, F_SIGNAL]
    q0[i_out, F_LATE_FAN] = int(np.sum(t[:, F_SIGNAL] == q0[nxt_pre, F_SIGNAL]))
    t[qoff[k]:qoff[k + 1]] = q0
    code, done = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"] and done < len(t)


def test_router_rows_have_their_own_units():
    w = synth.workload("moe30b_8k")
    c = _ctx(w.shape, 1, w.max_pages_per_seq, w.num_pages)
    c.build_schedule(256, 8192)
    tasks, qoff = c.schedule()
    routers = tasks[(tasks[:, F_OP] == OP_PRE) & (tasks[:, F_R0] >= w.shape.qkv_rows) & (tasks[:, F_LAYER] == 0)]
    assert 1 <= len(routers) <= 8
    assert np.all((routers[:, F_R1] <= w.shape.qkv_rows) | (routers[:, F_R0] >= w.shape.qkv_rows))
    # gate/up tasks wait for the router rows only, not for the QKV rows
    gu = tasks[(tasks[:, F_OP] == OP_GATEUP) & (tasks[:, F_LAYER] == 0)]
    assert np.all(gu[:, F_WAIT0] == routers[0, F_SIGNAL]) and np.all(gu[:, F_FAN0] == len(routers))


@pytest.mark.parametrize("lens,nkv,ntasks,nlead", [
    ([0], 4, 64, 4), ([8192], 4, 64, 4), ([8192], 4, 86, 4), ([8192], 4, 86, 32), ([15], 2, 64, 2), ([16], 2, 64, 16),
    ([17], 2, 3, 2), ([262144], 4, 256, 4), ([1024, 32768, 7, 0, 16, 15, 17, 5000], 4, 40, 32), ([3, 3, 3], 1, 3, 3),
])
def test_attention_split_partitions_every_segment(lens, nkv, ntasks, nlead):
    C, plan = mk.attn_plan(lens, nkv, ntasks, nlead)
    assert C % 16 == 0 and C >= 16
    seen = {}
    for i, (b, g, t0, t1) in enumerate(plan):
        if b < 0:
            continue
        assert t0 % 16 == 0 and 0 <= t0 < t1 <= lens[b] + 1 and t1 - t0 <= C
        seen.setdefault((b, g), []).append((t0, t1, i))
    assert len(seen) == len(lens) * nkv
    for (b, g), chunks in seen.items():
        chunks.sort()
        # the lead of segment m = b * nkv + g holds its first chunk; the others follow in
        # consecutive task numbers past the leads
        assert chunks[0][0] == 0 and chunks[0][2] == b * nkv + g and chunks[-1][1] == lens[b] + 1
        for (a0, a1, ia), (b0, b1, ib) in zip(chunks, chunks[1:]):
            assert a1 == b0 and ib >= nlead
        assert [c[2] for c in chunks[1:]] == list(range(chunks[1][2], chunks[1][2] + len(chunks) - 1)) if len(chunks) > 1 else True
    # lead tasks beyond the segments are idle
    assert all(plan[i][0] < 0 for i in range(len(lens) * nkv, nlead))
    # C is the smallest page multiple that fits: one page less would need more than the tasks there are
    cap = ntasks - nlead + len(lens) * nkv
    need = lambda c: sum(nkv * -(-(l + 1) // c) for l in lens)
    assert need(C) <= cap
    if C > 16:
        assert need(C - 16) > cap


def test_attention_split_rejects_too_few_tasks():
    with pytest.raises(mk.MkError):
        mk.attn_plan([10, 10], 4, 7)
    with pytest.raises(mk.MkError):
        mk.attn_plan([10, 10], 4, 9, 7)  # fewer leads than segments


def test_attention_split_random_shapes():
    """Seeded sweep: every segment's positions covered once, in page-aligned chunks, first chunk on its lead."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        nkv = int(rng.integers(1, 5))
        nseg = n * nkv
        nlead = int(rng.integers(nseg, 8 * nkv + 1)) if nseg < 8 * nkv else nseg
        ntasks = nlead + int(rng.integers(0, 120))
        lens = [int(x) for x in rng.integers(0, 5000, size=n)]
        if rng.random() < 0.2:
            lens[int(rng.integers(0, n))] = 0
        C, plan = mk.attn_plan(lens, nkv, ntasks, nlead)
        assert C % 16 == 0 and C >= 16
        covered = {}
        for i, (b, g, t0, t1) in enumerate(plan):
            if b < 0:
                continue
            assert 0 <= t0 < t1 <= lens[b] + 1 and t0 % 16 == 0 and t1 - t0 <= C
            if t0 == 0:
                assert i == b * nkv + g          # the lead holds the first chunk
            else:
                assert i >= nlead
            covered.setdefault((b, g), []).append((t0, t1))
        assert len(covered) == nseg
        for (b, g), ch in covered.items():
            ch.sort()
            assert ch[0][0] == 0 and ch[-1][1] == lens[b] + 1
            assert all(a1 == b0 for (_, a1), (b0, _) in zip(ch, ch[1:]))


# --------------------------------------------------------------------------- schedule parameters


def _mid_ctx(max_batch=3):
    w = synth.Workload("mid_p", synth.MID, batch=max_batch, steps=3, context=[2048, 40, 1000][:max_batch])
    return w, _ctx(w.shape, max_batch, w.max_pages_per_seq, w.num_pages)


def test_schedule_params_null_means_defaults():
    """NULL params = all-zero params: both query the current device (no GPU here: MK_ERR_HIP, no crash)."""
    import torch
    w, a = _mid_ctx()
    _, b = _mid_ctx()
    ws_a, ws_b = ctypes.c_size_t(), ctypes.c_size_t()
    ra = mk.lib().mk_build_schedule(a.h, None, ctypes.byref(ws_a))
    zero = mk.ScheduleParams()
    rb = mk.lib().mk_build_schedule(b.h, ctypes.byref(zero), ctypes.byref(ws_b))
    assert ra == rb
    if torch.cuda.is_available():
        assert ra == 0 and ws_a.value == ws_b.value
        assert np.array_equal(a.schedule()[0], b.schedule()[0])
    else:
        assert ra == mk.CODES["MK_ERR_HIP"]
    p = mk.ScheduleParams()
    mk.lib().mk_schedule_params_default(ctypes.byref(p))
    assert (p.num_cus, p.attn_units, p.router_units, p.prefetch_bytes, p.ctx_hint) == (0, 0, 0, 0, 0)


def test_schedule_params_attn_units_and_clamping():
    w, c = _mid_ctx()
    n_lead = 3 * w.shape.n_kv_heads
    for want, got in ((40, 40), (13, 13), (1, n_lead + 1), (10_000, 256 - 2)):
        c.build_schedule(256, 1000, attn_units=want)
        assert c.info().n_attn == got, want
        assert c.validate() == c.info().n_tasks


def test_default_split_follows_both_bounds():
    """The default attention/stage-1 split on the 30B shape (256 units): at 8K and at batch 8 it sits where
    the expert bytes meet the K/V bytes (gate/up + down at 2.25x the per-unit rate of K/V); at 256K it is
    capped where the QKV-then-attention chain is shortest, n / (256 - n) = sqrt(2.25 K/V / QKV bytes).
    Both bounds are written out here so a change of either formula shows."""
    s = synth.MOE30B
    qkv = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim * s.hidden * 2.0
    got = {}
    for batch, hint in ((1, 8256), (8, 12780), (1, 262160)):
        kv = 2.25 * hint * batch * s.n_kv_heads * s.head_dim * 4.0
        ex = min(s.n_experts, batch * s.top_k) * 3.0 * s.inter * s.hidden * 2.0
        balance = 256 * kv / (kv + ex)
        r = np.sqrt(kv / qkv)
        chain = 256 * r / (1 + r)
        c = _ctx(s, batch, 4, 8)
        c.build_schedule(256, hint)
        got[(batch, hint)] = (c.info().n_attn, balance, chain)
        assert c.info().n_attn == round(min(balance, chain))
        assert c.validate() == c.info().n_tasks
    assert got[(1, 8256)][0] == 86 and got[(1, 8256)][1] < got[(1, 8256)][2]
    assert got[(8, 12780)][0] == 112 and got[(8, 12780)][1] < got[(8, 12780)][2]
    assert got[(1, 262160)][0] == 226 and got[(1, 262160)][2] < got[(1, 262160)][1]
    # FP8 weights at batch 1: streamed-matrix rows count 1.5 bytes per element (measured cost), so
    # more units go to attention at 8K; at batch 8 the bf16 split
    from dataclasses import replace
    sq = replace(s, weights="fp8")
    for batch, hint, want in ((1, 8256, 103), (8, 12780, 112), (1, 262160, 230)):
        c = _ctx(sq, batch, 4, 8)
        c.build_schedule(256, hint)
        assert c.info().n_attn == want, (batch, hint, c.info().n_attn)
    # FP4 weights take the FP8 split (measured best at 8K, batch 1)
    s4 = replace(s, weights="fp4")
    for batch, hint, want in ((1, 8256, 103), (8, 12780, 112), (1, 262160, 230)):
        c = _ctx(s4, batch, 4, 8)
        c.build_schedule(256, hint)
        assert c.info().n_attn == want, (batch, hint, c.info().n_attn)


def test_schedule_params_router_units():
    w, c = _mid_ctx()
    for nr in (1, 2, 7):
        c.build_schedule(256, 1000, router_units=nr)
        tasks, qoff = c.schedule()
        pre0 = tasks[(tasks[:, F_OP] == OP_PRE) & (tasks[:, F_LAYER] == 0)]
        router = pre0[pre0[:, F_R0] >= w.shape.qkv_rows]
        assert len(router) == nr
        assert c.validate() == c.info().n_tasks


def test_schedule_params_prefetch_cap():
    w, c = _mid_ctx()
    c.build_schedule(256, 1000)
    full = c.info().lds_bytes
    c.build_schedule(256, 1000, prefetch_bytes=8192)
    capped = c.info().lds_bytes
    c.build_schedule(256, 1000, prefetch_bytes=-1)
    none = c.info().lds_bytes
    assert none + 8192 == capped and capped < full <= 160 * 1024


def test_schedule_params_negative_counts_rejected():
    w, c = _mid_ctx()
    for kw in ({"attn_units": -1}, {"router_units": -2}, {"ctx_hint": -5}, {"num_cus": -1}):
        with pytest.raises(mk.MkError) as e:
            c.build_schedule(**{"num_cus": 256, **kw})
        assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"], kw


def test_bind_scratch_rejects_a_workspace_beyond_the_static_one():
    """A schedule whose workspace exceeds the static array is refused before any device call."""
    import dataclasses
    shape = dataclasses.replace(synth.workload("moe30b_bs8_ragged").shape, n_layers=96)
    c = _ctx(shape, 8, 64, 512)
    ws = c.build_schedule(256, 4096)
    cap = mk.scratch_capacity()
    assert cap == 64 << 20 and ws > cap
    fake = [16 * (i + 1) for i in range(3 + 7 * shape.n_layers)]
    with pytest.raises(mk.MkError) as e:
        c.bind_scratch(fake, 1 << 20, 2 << 20, 0)
    assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"]
    assert "exceeds the static workspace" in str(e.value)
    with pytest.raises(mk.MkError) as e:  # nothing was bound
        c.decode_step(1, 0, 0, 0, 0, None, 0)
    assert e.value.code == mk.CODES["MK_ERR_STATE"]


def test_sampling_arguments():
    c = _ctx(synth.TINY)
    for bad in (-1.0, float("nan"), float("inf"), 1e-320):
        with pytest.raises(mk.MkError) as e:
            c.set_sampling(bad, 1)
        assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"], bad
    c.set_sampling(0.0)
    c.set_sampling(0.7, 2 ** 64 - 1)


def test_simulator_models_the_leads_ticket_wait():
    """Every segment lead waits inside its body for the other chunks of its layer (modelled as a
    superset, the split being decided at run time); a table where a non-lead chunk sits behind a
    task that needs the leads' merge must deadlock in the simulation."""
    F_REPORT = 18
    w = synth.workload("mid")
    c = _ctx(w.shape, 1, w.max_pages_per_seq, w.num_pages)
    c.build_schedule(64, 2048)
    tasks, qoff = c.schedule()
    nctr = c.info().n_counters
    attn0 = tasks[(tasks[:, F_OP] == OP_ATTN) & (tasks[:, F_LAYER] == 0)]
    leads = attn0[attn0[:, F_SIGNAL] >= 0]
    others = attn0[attn0[:, F_SIGNAL] < 0]
    assert len(leads) >= 1 and len(others) >= 1
    assert np.all(leads[:, F_LATE] >= 0) and np.all(leads[:, F_LATE_FAN] == len(others))
    assert np.all(others[:, F_REPORT] == leads[0, F_LATE])
    assert mk.simulate_table(tasks, qoff, nctr) == (0, len(tasks))
    # on a unit with Wo rows, put its layer-0 Wo task in front of its layer-0 chunk
    t = tasks.copy()
    for q in range(len(qoff) - 1):
        qt = t[qoff[q]:qoff[q + 1]]
        ia = np.nonzero((qt[:, F_OP] == OP_ATTN) & (qt[:, F_LAYER] == 0) & (qt[:, F_SIGNAL] < 0))[0]
        iw = np.nonzero((qt[:, F_OP] == OP_WO) & (qt[:, F_LAYER] == 0))[0]
        if len(ia) and len(iw):
            a, b = int(ia[0]), int(iw[0])
            qt[[a, b]] = qt[[b, a]]
            t[qoff[q]:qoff[q + 1]] = qt
            break
    else:
        pytest.fail("no unit with both a chunk and Wo rows")
    code, done = mk.simulate_table(t, qoff, nctr)
    assert code == mk.CODES["MK_ERR_SCHEDULE"] and done < len(t)


# --------------------------------------------------------------------------- sequential block

def test_create_rejects_an_unknown_block_style():
    cfg = mk.config_from_shape(synth.TINY, 1, 8, 8)
    cfg.block_style = 2
    with pytest.raises(mk.MkError) as e:
        mk.Context(cfg)
    assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"]


def test_sequential_block_schedule():
    """Sequential block: every router task (a PRE task with router rows) waits for its own layer's Wo
    rows; the Wqkv tasks keep the parallel block's waits; the table simulates to completion."""
    from dataclasses import replace
    s = replace(synth.MID, block="sequential")
    c = _ctx(s, 2, 16, 64)
    c.build_schedule(256, 2000)
    tasks, qoff = c.schedule()
    assert c.validate() == c.info().n_tasks
    op, layer, w0, w1 = tasks[:, 0], tasks[:, 1], tasks[:, 2], tasks[:, 3]
    r0 = tasks[:, 7]
    pre = op == 1
    router = pre & (r0 >= s.qkv_rows)
    assert router.any() and (pre & ~router).any()
    n_ctr_layer, c_wo = 9, 6
    assert np.array_equal(w1[router], layer[router] * n_ctr_layer + c_wo)
    # the parallel block's router tasks wait on the previous layer's Wo rows instead
    p = _ctx(synth.MID, 2, 16, 64)
    p.build_schedule(256, 2000)
    pt, _ = p.schedule()
    prouter = (pt[:, 0] == 1) & (pt[:, 7] >= s.qkv_rows) & (pt[:, 1] > 0)
    assert np.array_equal(pt[prouter, 3], (pt[prouter, 1] - 1) * n_ctr_layer + c_wo)
    # dedicated QKV units and the shared pool are not offered with the sequential block
    for kw in ({"qkv_units": 20}, {"pool_64ths": 8}):
        with pytest.raises(mk.MkError) as e:
            c.build_schedule(256, 2000, **kw)
        assert e.value.code == mk.CODES["MK_ERR_UNSUPPORTED"]


def test_sequential_block_schedule_puts_every_unit_in_every_phase():
    """From batch 2, every unit, per layer: its Wqkv rows (if any), its attention chunk, its Wo rows
    (non-leads), its router rows (if any: after its Wo rows), its gate/up rows, its output rows;
    attn_units still limits the attention to the first units.  At batch 1 the parallel split."""
    from dataclasses import replace
    s = replace(synth.MID, block="sequential")
    c1 = _ctx(s, 1, 16, 64)
    c1.build_schedule(256, 2000)
    assert c1.info().n_attn < 200 and c1.validate() == c1.info().n_tasks
    c = _ctx(s, 2, 16, 64)
    c.build_schedule(256, 2000)
    assert c.info().n_attn == 256 and c.validate() == c.info().n_tasks
    tasks, qoff = c.schedule()
    PRE, ATTN, GATEUP, OUT, WO, KVW = 1, 2, 3, 4, 6, 8
    for q in range(256):
        t = tasks[qoff[q]:qoff[q + 1]]
        lay0 = t[t[:, 1] == 0]
        ops = [int(o) for o in lay0[:, 0]]
        plain = [o for o in ops if o != KVW]
        assert ATTN in plain and GATEUP in plain and OUT in plain, (q, ops)
        assert plain.index(ATTN) < plain.index(GATEUP) < plain.index(OUT)
        pres = lay0[lay0[:, 0] == PRE]
        for r in pres:
            i = plain.index(PRE) if r[7] < s.qkv_rows else len(plain) - 1 - plain[::-1].index(PRE)
            if r[7] < s.qkv_rows:
                assert i < plain.index(ATTN)
            else:
                assert WO in plain[:i] and i < plain.index(GATEUP), (q, plain)
    c.build_schedule(256, 2000, attn_units=100)
    assert c.info().n_attn == 100 and c.validate() == c.info().n_tasks


def test_sequential_block_binds_eight_tensors_per_layer():
    """3 + 8 * n_layers weight pointers (the MoE norm gains after every layer's seven); the count is
    checked before any device call, so fake aligned pointers suffice to see it refused."""
    from dataclasses import replace
    s = replace(synth.TINY, block="sequential")
    c = _ctx(s, 1, 8, 8)
    c.build_schedule(256, 100)
    fake = [0x1000 * (i + 1) for i in range(3 + 7 * s.n_layers)]
    with pytest.raises(mk.MkError) as e:
        c.bind(fake, 0x100000, 0x200000, 0, 0, 0)
    assert e.value.code == mk.CODES["MK_ERR_INVALID_ARG"] and "3 + 7*n_layers" in str(e.value)
    fake = [0x1000 * (i + 1) for i in range(3 + 8 * s.n_layers)]
    with pytest.raises(mk.MkError) as e:   # now the count passes and the missing workspace is refused
        c.bind(fake, 0x100000, 0x200000, 0, 0, 0)
    assert "n_layers" not in str(e.value)
    assert len(s.bind_order()) == 3 + 8 * s.n_layers
    assert s.bind_order()[3 + 7 * s.n_layers:] == [(synth.K_MOE_NORM, l) for l in range(s.n_layers)]


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_sequential_block_is_built_for_bf16_weights_only(fmt):
    from dataclasses import replace
    s = replace(synth.TINY, block="sequential", weights=fmt)
    with pytest.raises(mk.MkError) as e:
        _ctx(s, 1, 8, 8)
    assert e.value.code == mk.CODES["MK_ERR_UNSUPPORTED"]
