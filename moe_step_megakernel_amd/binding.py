"""Python binding of the C ABI in ``include/moe_step.h`` (ctypes).

Argument marshalling only: every step of the update runs in the HIP library.
PyTorch supplies device memory and the stream.  The library must be built
(``__graft_entry__.build()``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_STEP_LIB") or os.path.join(_HERE, "_lib", "libmoe_step.so")

MOE_STEP_ABI_VERSION = 1
MOE_OK, MOE_ERR_ARG, MOE_ERR_SHAPE, MOE_ERR_HIP, MOE_ERR_NOMEM, MOE_ERR_DEVICE, MOE_ERR_STATE = 0, -1, -2, -3, -4, -5, -6
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_RUN_ZERO_GRAD, MOE_RUN_APPLY, MOE_RUN_REFRESH_SHADOW, MOE_RUN_TRACE = 0x1, 0x2, 0x4, 0x8
MOE_RUN_SKIP_GATHER, MOE_RUN_SKIP_ROWSUM = 0x100000, 0x200000
MOE_RUN_SKIP_MASK = 0xFF00 | MOE_RUN_SKIP_GATHER | MOE_RUN_SKIP_ROWSUM
MOE_RUN_ZERO_GRAD_ROUTER, MOE_RUN_ZERO_GRAD_EXPERTS = 0x10, 0x20
MOE_RUN_APPLY_ROUTER, MOE_RUN_APPLY_EXPERTS = 0x40, 0x80
MOE_RUN_READY_GEMM12 = 0x10000
MOE_RUN_COOPERATIVE = 0x20000
MOE_RUN_TEST_TIMEOUT = 0x40000
MOE_RUN_BARRIER_PER_WORKGROUP = 0x80000


def MOE_RUN_SKIP_PHASE(i: int) -> int:
    return 0x100 << i

MOE_DEVICE_BARRIER_TIMEOUT, MOE_DEVICE_NONFINITE_LOGIT, MOE_DEVICE_BAD_ROUTE = 0x1, 0x2, 0x4
MOE_STEP_STATIC_SCRATCH_BYTES = 32 << 20
MOE_MEM_RECOMPUTE = 0x1
MOE_MEM_GUARDS = 0x2
N_PHASES = 8

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_HIP", -4: "MOE_ERR_NOMEM",
                -5: "MOE_ERR_DEVICE", -6: "MOE_ERR_STATE"}


class moe_step_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("abi_version", ctypes.c_uint32),
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
        ("adam_eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("clip_norm", ctypes.c_double),
        ("device", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32), ("memory_rules", ctypes.c_uint32),
        ("max_microbatches", ctypes.c_int32),
    ]


class moe_step_io(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "x", "target", "router_bias", "params", "grads", "exp_avg", "exp_avg_sq", "dx", "stats",
        "router_logits", "topk_idx", "topk_gate", "expert_counts", "route_perm", "trace")]


class MoeStepError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func} -> {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.moe_step_param_count.argtypes = [P(moe_step_config)]
    lib.moe_step_param_count.restype = ctypes.c_size_t
    lib.moe_step_check_config.argtypes = [P(moe_step_config)]
    lib.moe_step_check_config.restype = ctypes.c_int
    lib.moe_step_create.argtypes = [P(moe_step_config), P(ctypes.c_void_p)]
    lib.moe_step_create.restype = ctypes.c_int
    lib.moe_step_run.argtypes = [ctypes.c_void_p, P(moe_step_io), ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_uint32, ctypes.c_void_p]
    lib.moe_step_run.restype = ctypes.c_int
    lib.moe_step_run_groups.argtypes = [ctypes.c_void_p, P(moe_step_io), ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.moe_step_run_groups.restype = ctypes.c_int
    lib.moe_step_run_static.argtypes = [P(moe_step_config), P(moe_step_io), ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.moe_step_run_static.restype = ctypes.c_int
    lib.moe_step_status.argtypes = [ctypes.c_void_p]
    lib.moe_step_status.restype = ctypes.c_int
    lib.moe_step_check_guards.argtypes = [ctypes.c_void_p, P(ctypes.c_int32)]
    lib.moe_step_check_guards.restype = ctypes.c_int
    lib.moe_step_trace_words.argtypes = [ctypes.c_void_p]
    lib.moe_step_trace_words.restype = ctypes.c_size_t
    lib.moe_step_grid_size.argtypes = [ctypes.c_void_p]
    lib.moe_step_grid_size.restype = ctypes.c_int
    lib.moe_step_arena_bytes.argtypes = [ctypes.c_void_p]
    lib.moe_step_arena_bytes.restype = ctypes.c_size_t
    lib.moe_step_last_error.argtypes = [ctypes.c_void_p]
    lib.moe_step_last_error.restype = ctypes.c_char_p
    lib.moe_step_destroy.argtypes = [ctypes.c_void_p]
    lib.moe_step_destroy.restype = None
    _lib = lib
    return lib


def make_config(d_model, d_ff, n_experts, top_k, max_tokens, dtype="bf16", lr=1e-3, beta1=0.9, beta2=0.999,
                adam_eps=1e-8, weight_decay=0.01, clip_norm=1.0, device=0, wg_per_cu=0,
                memory_rules=0, max_microbatches=0) -> moe_step_config:
    return moe_step_config(
        ctypes.sizeof(moe_step_config), MOE_STEP_ABI_VERSION, d_model, d_ff, n_experts, top_k, max_tokens,
        MOE_DTYPE_BF16 if dtype == "bf16" else MOE_DTYPE_F32, lr, beta1, beta2, adam_eps, weight_decay,
        clip_norm, device, wg_per_cu, memory_rules, max_microbatches)


# --- the C entry points, same names -------------------------------------------------------------
def moe_step_param_count(cfg: moe_step_config) -> int:
    return int(load_library().moe_step_param_count(ctypes.byref(cfg)))


def moe_step_check_config(cfg: moe_step_config) -> int:
    return int(load_library().moe_step_check_config(ctypes.byref(cfg)))


def moe_step_last_error(handle) -> str:
    return load_library().moe_step_last_error(handle).decode()


def moe_step_create(cfg: moe_step_config):
    lib = load_library()
    h = ctypes.c_void_p()
    rc = lib.moe_step_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != MOE_OK:
        raise MoeStepError("moe_step_create", rc, moe_step_last_error(None))
    return h


def moe_step_run(handle, io: moe_step_io, n_tokens: int, tokens_in_update: int, step: int, run_flags: int,
                 stream=None) -> None:
    rc = load_library().moe_step_run(handle, ctypes.byref(io), n_tokens, tokens_in_update, step, run_flags,
                                     stream)
    if rc != MOE_OK:
        raise MoeStepError("moe_step_run", rc, moe_step_last_error(handle))


def moe_step_run_groups(handle, io: moe_step_io, n_tokens: int, tokens_in_update: int, step_router: int,
                        step_experts: int, run_flags: int, stream=None) -> None:
    rc = load_library().moe_step_run_groups(handle, ctypes.byref(io), n_tokens, tokens_in_update, step_router,
                                            step_experts, run_flags, stream)
    if rc != MOE_OK:
        raise MoeStepError("moe_step_run_groups", rc, moe_step_last_error(handle))


def moe_step_run_static(cfg: moe_step_config, io: moe_step_io, n_tokens: int, tokens_in_update: int, step: int,
                        run_flags: int, stream=None) -> None:
    rc = load_library().moe_step_run_static(ctypes.byref(cfg), ctypes.byref(io), n_tokens, tokens_in_update, step,
                                            run_flags, stream)
    if rc != MOE_OK:
        raise MoeStepError("moe_step_run_static", rc, moe_step_last_error(None))


def moe_step_status(handle) -> None:
    rc = load_library().moe_step_status(handle)
    if rc != MOE_OK:
        raise MoeStepError("moe_step_status", rc, moe_step_last_error(handle))


def moe_step_check_guards(handle) -> None:
    damaged = ctypes.c_int32(0)
    rc = load_library().moe_step_check_guards(handle, ctypes.byref(damaged))
    if rc != MOE_OK:
        raise MoeStepError("moe_step_check_guards", rc, moe_step_last_error(handle))


def moe_step_trace_words(handle) -> int:
    return int(load_library().moe_step_trace_words(handle))


def moe_step_grid_size(handle) -> int:
    return int(load_library().moe_step_grid_size(handle))


def moe_step_arena_bytes(handle) -> int:
    return int(load_library().moe_step_arena_bytes(handle))


def moe_step_destroy(handle) -> None:
    if handle:
        load_library().moe_step_destroy(handle)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def make_io(x=None, target=None, router_bias=None, params=None, grads=None, exp_avg=None, exp_avg_sq=None,
            dx=None, stats=None, router_logits=None, topk_idx=None, topk_gate=None, expert_counts=None,
            route_perm=None, trace=None) -> moe_step_io:
    """Builds a moe_step_io from torch tensors (or None)."""
    return moe_step_io(*(_ptr(t) for t in (x, target, router_bias, params, grads, exp_avg, exp_avg_sq, dx, stats,
                                            router_logits, topk_idx, topk_gate, expert_counts, route_perm,
                                            trace)))
