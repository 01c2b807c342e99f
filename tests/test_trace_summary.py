"""The per-task timeline's summary from hand-made records (no GPU): waits, busy times, phases, layer spans,
and a task whose ready word was never written."""
import numpy as np

from persistent_moe_decode_amd import mk, trace

OP = {v: k for k, v in mk.OPS.items()}


def _rec(fetch, ready, marks, done):
    r = np.zeros(trace.WORDS, dtype=np.uint64)
    r[0], r[1], r[6] = fetch, ready, done
    for k, m in enumerate(marks):
        r[2 + k] = m
    return r


def test_summary_of_two_layers():
    # ticks of 10 ns; clock origin 1000
    tasks = np.array([[OP["PRE"], 0], [OP["GATEUP"], 0], [OP["PRE"], 1], [OP["KVW"], 1]], dtype=np.int32)
    rec = np.stack([
        _rec(1000, 1100, [1200, 1300], 1500),   # PRE L0: wait 1 us, busy 4 us, phases 1, 1, 2 us
        _rec(1000, 1300, [1400], 2000),         # GATEUP L0: wait 3 us, busy 7 us
        _rec(2000, 2100, [], 2600),             # PRE L1: wait 1 us, busy 5 us
        _rec(2000, 0, [], 2050),                # KVW L1 whose ready word was never written
    ])
    out = trace.summarize(tasks, np.array([0, 4]), rec)
    assert out["span_us"] == 16.0
    pre = out["ops"]["PRE"]
    assert pre["tasks"] == 2 and pre["wait_us_mean"] == 1.0 and pre["busy_us_mean"] == 4.5 and pre["busy_us_max"] == 5.0
    assert pre["phase_us_mean"][:2] == [1.0, 1.0]
    gu = out["ops"]["GATEUP"]
    assert gu["wait_us_mean"] == 3.0 and gu["busy_us_mean"] == 7.0 and gu["phase_us_mean"] == [1.0, 6.0]
    kvw = out["ops"]["KVW"]
    assert kvw["wait_us_mean"] == 0.0 and kvw["busy_us_mean"] == 0.5
    # layer 0: ready 1 us .. end 10 us; layer 1: ready 10 (the KVW's fetch) .. 16 us
    assert out["layer_span_us_mean"] == 7.5
    assert out["stage_end_us_first_layers"]["PRE"] == [5.0, 16.0]
    ev = trace.perfetto(tasks, np.array([0, 4]), rec)["traceEvents"]
    assert all(e["dur"] >= 0 for e in ev)
