"""Per-task timeline of one decode step: summary statistics and Perfetto JSON.

The megakernel writes, per task, eight words when tracing is on
(mk_set_trace): readings of the constant 100 MHz clock when the task was
fetched, when its dependencies were met, up to four phase marks inside the
body, and when it had signalled.  This module joins them with the task table.

Phase marks per op: PRE [inputs loaded, norm done, rows done]; ATTN [q
rotated and new K/V written, copied pages landed, positions done, partial
stored]; GATEUP [top-k selected (wave 0), routing tables built, norm done, own rows done];
GUTAIL [top-k selected (wave 0), norm done, pool items done];
OUT [h loaded, wave 0's down rows done, all down rows done, residual rows stored]; WO [attention output loaded, rows done];
LMHEAD [norm done, rows done, local argmax done]; KVW none.  Tasks that wait
inside their body (ATTN, GATEUP, OUT, WO, KVW) record as "ready" the moment
their inputs were there (for GATEUP: the epoch tags of the router logits
matched); a KVW task in a plain decode step waits for nothing.  A task that gave
up on its wait (abort or time-out) leaves its ready word zero.
"""
from __future__ import annotations

import json

import numpy as np

from . import mk

TICK_US = 0.01  # s_memrealtime runs at 100 MHz
WORDS = 8


def _ready_filled(rec: np.ndarray) -> np.ndarray:
    """Records as int64 [tasks][WORDS], a ready word never written (a task that gave up on its wait)
    taken as its fetch time."""
    rec = rec.astype(np.int64).reshape(-1, WORDS).copy()
    unset = rec[:, 1] == 0
    rec[unset, 1] = rec[unset, 0]
    return rec


def summarize(tasks: np.ndarray, qoff: np.ndarray, rec: np.ndarray) -> dict:
    """Per op kind: mean wait, busy time and phase durations (us); per layer span; overall span."""
    rec = _ready_filled(rec)
    t0 = rec[:, 0].min()
    start, ready, end = (rec[:, 0] - t0) * TICK_US, (rec[:, 1] - t0) * TICK_US, (rec[:, 6] - t0) * TICK_US
    ops = tasks[:, 0]
    out = {"span_us": round(float(end.max()), 2), "ops": {}}
    for code, name in mk.OPS.items():
        m = ops == code
        if not m.any():
            continue
        d = {
            "tasks": int(m.sum()),
            "wait_us_mean": round(float((ready[m] - start[m]).mean()), 2),
            "busy_us_mean": round(float((end[m] - ready[m]).mean()), 2),
            "busy_us_max": round(float((end[m] - ready[m]).max()), 2),
        }
        # phase durations: consecutive marks that were written
        prev = rec[m, 1]
        phases = []
        for k in range(4):
            mk_ = rec[m, 2 + k]
            ok = mk_ > 0
            if not ok.any():
                break
            phases.append(round(float(((mk_[ok] - prev[ok]) * TICK_US).mean()), 2))
            prev = np.where(ok, mk_, prev)
        phases.append(round(float(((rec[m, 6] - prev) * TICK_US).mean()), 2))
        d["phase_us_mean"] = phases
        out["ops"][name] = d
    layers = tasks[:, 1]
    spans = [float(end[layers == l].max() - ready[layers == l].min()) for l in np.unique(layers)]
    out["layer_span_us_mean"] = round(float(np.mean(spans)), 2)
    stage_end = {}
    for code, name in mk.OPS.items():
        for l in np.unique(layers):
            sel = (ops == code) & (layers == l)
            if sel.any():
                stage_end.setdefault(name, []).append(round(float(end[sel].max()), 2))
    out["stage_end_us_first_layers"] = {k: v[:3] for k, v in stage_end.items()}
    return out


def perfetto(tasks: np.ndarray, qoff: np.ndarray, rec: np.ndarray) -> dict:
    """Chrome/Perfetto trace events: one track per compute unit, wait and busy slices."""
    rec = _ready_filled(rec)
    t0 = rec[:, 0].min()
    ev = []
    for cu in range(len(qoff) - 1):
        for q in range(qoff[cu], qoff[cu + 1]):
            op = mk.OPS.get(int(tasks[q, 0]), "?")
            a, b, c = ((rec[q, [0, 1, 6]] - t0) * TICK_US).tolist()
            name = f"{op} L{int(tasks[q, 1])}"
            if b > a:
                ev.append({"name": "wait " + name, "ph": "X", "ts": a, "dur": b - a, "pid": 0, "tid": cu})
            marks = [float((m - t0) * TICK_US) for m in rec[q, 2:6] if m > 0]
            ev.append({"name": name, "ph": "X", "ts": b, "dur": max(c - b, 0.001), "pid": 0, "tid": cu,
                       "args": {"phase_ends_us": [round(m, 3) for m in marks], "task": int(q)}})
    return {"traceEvents": ev, "displayTimeUnit": "ns"}


def dump(path: str, tasks, qoff, rec) -> None:
    with open(path, "w") as f:
        json.dump(perfetto(tasks, qoff, rec), f)
