"""ctypes binding of libmk.so (include/mk.h): argument marshalling only.

Every step of the decode runs in the HIP library; this module converts Python
integers and torch device pointers into the C ABI's plain pointers and
sizes, and turns negative return codes into exceptions.  Importing it fails
loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
# MK_LIBRARY names another build of the same library (for side-by-side timing of build variants)
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(_HERE, "libmk.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mk.h")

MK_OK = 0
ERRORS = {
    -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_UNSUPPORTED", -3: "MK_ERR_STATE", -4: "MK_ERR_SCHEDULE",
    -5: "MK_ERR_HIP", -10: "MK_ERR_DEVICE_PAGE", -11: "MK_ERR_DEVICE_SEQ", -12: "MK_ERR_DEVICE_TOKEN",
    -13: "MK_ERR_DEVICE_TIMEOUT",
}
CODES = {v: k for k, v in ERRORS.items()}
TASK_INT32S = 32
OPS = {1: "PRE", 2: "ATTN", 3: "GATEUP", 4: "OUT", 5: "LMHEAD", 6: "WO", 7: "GUTAIL", 8: "KVW"}


class MkError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {ERRORS.get(code, code)}: {msg}")
        self.code = code


class MkConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double),
        ("weight_format", ctypes.c_int32), ("block_style", ctypes.c_int32),
    ]


class ScheduleParams(ctypes.Structure):
    """mk_schedule_params: how the schedule is cut (all zero = defaults)."""
    _fields_ = [("num_cus", ctypes.c_int32), ("attn_units", ctypes.c_int32), ("router_units", ctypes.c_int32),
                ("prefetch_bytes", ctypes.c_int32), ("pool_64ths", ctypes.c_int32), ("qkv_units", ctypes.c_int32),
                ("ctx_hint", ctypes.c_int64)]


class ScheduleInfo(ctypes.Structure):
    _fields_ = [
        ("num_cus", ctypes.c_int32), ("n_tasks", ctypes.c_int32), ("n_counters", ctypes.c_int32),
        ("n_attn", ctypes.c_int32), ("n_gateup", ctypes.c_int32), ("n_out", ctypes.c_int32),
        ("n_lmhead", ctypes.c_int32), ("task_int32s", ctypes.c_int32), ("lds_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
    ]


class WsOffsets(ctypes.Structure):
    _fields_ = [("x", ctypes.c_int64), ("qkv", ctypes.c_int64), ("router", ctypes.c_int64),
                ("attn_out", ctypes.c_int64), ("h", ctypes.c_int64), ("sel", ctypes.c_int64),
                ("moe_half", ctypes.c_int64), ("attn_half", ctypes.c_int64)]


_lib = None


def lib():
    """Load libmk.so; raises if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "mk_create": [ctypes.POINTER(MkConfig), ctypes.POINTER(P)],
        "mk_build_schedule": [P, ctypes.POINTER(ScheduleParams), ctypes.POINTER(SZ)],
        "mk_bind": [P, ctypes.POINTER(P), I32, P, P, P, SZ, P],
        "mk_bind_scratch": [P, ctypes.POINTER(P), I32, P, P, P],
        "mk_decode_step": [P, I32, P, P, P, P, P, P],
        "mk_decode_steps": [P, I32, I32, P, P, P, P, P, P],
        "mk_mixed_step": [P, I32, P, P, P, P, P, P],
        "mk_get_error": [P, pi32, pi32, pi32, P],
        "mk_reset": [P, P],
        "mk_set_spin_limit_us": [P, I64],
        "mk_set_layer_inputs": [P, P],
        "mk_set_trace": [P, P, I64],
        "mk_set_sampling": [P, ctypes.c_double, ctypes.c_uint64],
        "mk_set_top_p": [P, ctypes.c_float],
        "mk_get_schedule_info": [P, ctypes.POINTER(ScheduleInfo)],
        "mk_copy_schedule": [P, pi32, I64, pi32, I64],
        "mk_validate_schedule": [P, pi32],
        "mk_simulate_table": [pi32, I32, pi32, I32, I32, pi32],
        "mk_attn_plan": [pi32, I32, I32, I32, I32, I32, pi32, pi32],
        "mk_get_ws_offsets": [P, ctypes.POINTER(WsOffsets)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.mk_last_error_message.argtypes = []
    L.mk_last_error_message.restype = ctypes.c_char_p
    L.mk_destroy.argtypes = [P]
    L.mk_destroy.restype = None
    L.mk_schedule_params_default.argtypes = [ctypes.POINTER(ScheduleParams)]
    L.mk_schedule_params_default.restype = None
    L.mk_scratch_capacity.argtypes = []
    L.mk_scratch_capacity.restype = SZ
    _lib = L
    return L


def unload() -> None:
    """dlclose libmk.so: its HIP module destructor (code-object unregistration) runs now, while the
    HIP runtime is fully alive, instead of among the process's exit handlers.  Every context must be
    destroyed and the device idle first; lib() loads it again if needed."""
    global _lib
    if _lib is None:
        return
    import _ctypes
    handle = _lib._handle
    _lib = None
    _ctypes.dlclose(handle)


def header_symbols() -> list:
    """Function names declared in include/mk.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", text)))


def check(code: int, where: str) -> None:
    if code != MK_OK:
        raise MkError(code, where, lib().mk_last_error_message().decode())


def _i32p(arr):
    """ctypes int32* of a contiguous numpy int32 array."""
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


WEIGHT_FORMATS = {"bf16": 0, "fp8": 1, "fp4": 2}   # MK_WEIGHTS_BF16, _FP8_E4M3, _FP4_E2M1
BLOCK_STYLES = {"parallel": 0, "sequential": 1}     # MK_BLOCK_PARALLEL, MK_BLOCK_SEQUENTIAL


def config_from_shape(shape, max_batch: int, max_pages_per_seq: int, num_pages: int) -> MkConfig:
    return MkConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                    shape.n_experts, shape.top_k, shape.inter, shape.vocab, shape.page_size, max_batch,
                    max_pages_per_seq, num_pages, shape.rms_eps, shape.rope_theta,
                    WEIGHT_FORMATS[getattr(shape, "weights", "bf16")], BLOCK_STYLES[getattr(shape, "block", "parallel")])


class Context:
    """One mk_ctx: a model shape with its schedule and bound buffers."""

    def __init__(self, cfg: MkConfig):
        self.cfg = cfg
        h = ctypes.c_void_p()
        check(lib().mk_create(ctypes.byref(cfg), ctypes.byref(h)), "mk_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().mk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def build_schedule(self, num_cus: int = 0, ctx_hint: int = 0, attn_units: int = 0, router_units: int = 0,
                       prefetch_bytes: int = 0, pool_64ths: int = 0, qkv_units: int = 0) -> int:
        """mk_build_schedule; returns the workspace size in bytes."""
        p = ScheduleParams()
        lib().mk_schedule_params_default(ctypes.byref(p))
        p.num_cus, p.ctx_hint, p.attn_units, p.router_units, p.prefetch_bytes, p.pool_64ths, p.qkv_units = (
            num_cus, ctx_hint, attn_units, router_units, prefetch_bytes, pool_64ths, qkv_units)
        ws = ctypes.c_size_t()
        check(lib().mk_build_schedule(self.h, ctypes.byref(p), ctypes.byref(ws)), "mk_build_schedule")
        return ws.value

    def info(self) -> ScheduleInfo:
        i = ScheduleInfo()
        check(lib().mk_get_schedule_info(self.h, ctypes.byref(i)), "mk_get_schedule_info")
        return i

    def schedule(self):
        import numpy as np
        i = self.info()
        tasks = np.zeros((i.n_tasks, TASK_INT32S), dtype=np.int32)
        qoff = np.zeros(i.num_cus + 1, dtype=np.int32)
        check(lib().mk_copy_schedule(self.h, _i32p(tasks), tasks.size, _i32p(qoff), qoff.size), "mk_copy_schedule")
        return tasks, qoff

    def validate(self) -> int:
        done = ctypes.c_int32()
        check(lib().mk_validate_schedule(self.h, ctypes.byref(done)), "mk_validate_schedule")
        return done.value

    def ws_offsets(self) -> WsOffsets:
        o = WsOffsets()
        check(lib().mk_get_ws_offsets(self.h, ctypes.byref(o)), "mk_get_ws_offsets")
        return o

    def bind(self, weight_ptrs, k_pool_ptr: int, v_pool_ptr: int, ws_ptr: int, ws_bytes: int, stream: int):
        arr = (ctypes.c_void_p * len(weight_ptrs))(*weight_ptrs)
        check(lib().mk_bind(self.h, arr, len(weight_ptrs), k_pool_ptr, v_pool_ptr, ws_ptr, ws_bytes, stream), "mk_bind")

    def bind_scratch(self, weight_ptrs, k_pool_ptr: int, v_pool_ptr: int, stream: int):
        """Bind with the library's static workspace instead of a caller-provided one."""
        arr = (ctypes.c_void_p * len(weight_ptrs))(*weight_ptrs)
        check(lib().mk_bind_scratch(self.h, arr, len(weight_ptrs), k_pool_ptr, v_pool_ptr, stream), "mk_bind_scratch")

    def decode_step(self, n: int, tokens_ptr: int, page_table_ptr: int, seq_lens_ptr: int, logits_ptr: int,
                    next_ptr: int | None, stream: int):
        check(lib().mk_decode_step(self.h, n, tokens_ptr, page_table_ptr, seq_lens_ptr, logits_ptr,
                                   next_ptr or None, stream), "mk_decode_step")

    def mixed_step(self, n: int, tokens_ptr: int, page_table_ptr: int, seq_lens_ptr: int, logits_ptr: int,
                   next_ptr: int | None, stream: int):
        check(lib().mk_mixed_step(self.h, n, tokens_ptr, page_table_ptr, seq_lens_ptr, logits_ptr,
                                  next_ptr or None, stream), "mk_mixed_step")

    def decode_steps(self, n: int, steps: int, tokens_ptr: int, page_table_ptr: int, seq_lens_ptr: int,
                     logits_ptr: int, next_ptr: int | None, stream: int):
        check(lib().mk_decode_steps(self.h, n, steps, tokens_ptr, page_table_ptr, seq_lens_ptr, logits_ptr,
                                    next_ptr or None, stream), "mk_decode_steps")

    def get_error(self, stream: int):
        code, cu, task = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(lib().mk_get_error(self.h, ctypes.byref(code), ctypes.byref(cu), ctypes.byref(task), stream),
              "mk_get_error")
        return code.value, cu.value, task.value

    def reset(self, stream: int):
        check(lib().mk_reset(self.h, stream), "mk_reset")

    def set_layer_inputs(self, ptr: int | None):
        check(lib().mk_set_layer_inputs(self.h, ptr or None), "mk_set_layer_inputs")

    def set_trace(self, ptr: int | None, capacity: int = 0):
        check(lib().mk_set_trace(self.h, ptr or None, capacity), "mk_set_trace")

    def set_sampling(self, temperature: float, seed: int = 0):
        """Temperature 0 (the default) is the greedy argmax; > 0 samples softmax(logits / T)."""
        check(lib().mk_set_sampling(self.h, float(temperature), int(seed) & ((1 << 64) - 1)), "mk_set_sampling")

    def set_top_p(self, top_p: float):
        """Nucleus mass for sampling at temperature > 0 (1, the default: every token)."""
        check(lib().mk_set_top_p(self.h, float(top_p)), "mk_set_top_p")

    def set_spin_limit_us(self, us: int):
        check(lib().mk_set_spin_limit_us(self.h, us), "mk_set_spin_limit_us")


def scratch_capacity() -> int:
    """Bytes of the static workspace that Context.bind_scratch uses."""
    return int(lib().mk_scratch_capacity())


def simulate_table(tasks, qoff, n_counters: int):
    """Run the host simulator on an arbitrary table; returns (code, completed)."""
    import numpy as np
    tasks = np.ascontiguousarray(tasks, dtype=np.int32)
    qoff = np.ascontiguousarray(qoff, dtype=np.int32)
    done = ctypes.c_int32()
    code = lib().mk_simulate_table(_i32p(tasks), tasks.shape[0], _i32p(qoff), qoff.size - 1, n_counters,
                                   ctypes.byref(done))
    return code, done.value


def attn_plan(seq_lens, n_kv: int, n_tasks: int, n_lead: int = -1, page_size: int = 16):
    """Host mirror of the kernel's runtime attention split: (chunk, plan[n_tasks][4]).

    n_lead: split tasks that lead a (sequence, kv head) segment (default: one per segment)."""
    import numpy as np
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    plan = np.zeros((n_tasks, 4), dtype=np.int32)
    chunk = ctypes.c_int32()
    if n_lead < 0:
        n_lead = sl.size * n_kv
    check(lib().mk_attn_plan(_i32p(sl), sl.size, n_kv, n_tasks, n_lead, page_size, ctypes.byref(chunk),
                             _i32p(plan)), "mk_attn_plan")
    return chunk.value, plan
