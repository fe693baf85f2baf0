"""ctypes loader for libkda.so (the C ABI declared in include/kda.h).

The library must have been built in-tree (``python -m
gated_delta_rule_92_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# KDA_HOST_CHECK_LIB names a host-check build of the C ABI (argument
# validation and dispatch compiled with sanitizers, kernel launches replaced by
# stubs that do nothing): used only by the CPU sanitizer test, it computes
# nothing.
LIB_PATH = os.environ.get("KDA_HOST_CHECK_LIB") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_SUCCESS = 0
KDA_ERROR_INVALID_VALUE = 1
KDA_ERROR_NOT_SUPPORTED = 2
KDA_ERROR_INSUFFICIENT_WORKSPACE = 3
KDA_ERROR_LAUNCH_FAILURE = 4

KDA_FLOAT32 = 0
KDA_BFLOAT16 = 1

KDA_GATE_LOGDECAY = 0
KDA_GATE_CUMSUM = 1
KDA_GATE_LOGITS = 2
KDA_GATE_SOFTPLUS = 3

# Every symbol include/kda.h declares.
EXPORTED = ("kda_status_string", "kda_version", "kda_gate", "kda_chunk_fwd_workspace_size",
            "kda_chunk_fwd", "kda_chunk_fwd_split_workspace_size", "kda_chunk_fwd_split",
            "kda_chunk_fwd_gated", "kda_gated_rmsnorm", "kda_chunk_transition",
            "kda_compose_states", "kda_recurrent_step", "kda_chunk_bwd_workspace_size",
            "kda_chunk_bwd", "kda_gate_bwd", "kda_device_status", "kda_chunk_fwd_noalloc",
            "kda_debug_set_spin_limit", "kda_chunk_fwd_train", "kda_chunk_bwd_saved")

KDA_DEVICE_WAIT_TIMEOUT = 0x1
KDA_DEVICE_DECAY_OUT_OF_RANGE = 0x2

_lib = None


class KdaError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load and bind libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise KdaError(f"{path} not found: build it with `python -m gated_delta_rule_92_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32, f32, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i32
    lib.kda_gate.argtypes = [fp, fp, f32, ip, i32, i32, i32, i32, i32, i32, fp, vp]
    lib.kda_gate.restype = i32
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                                 ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_workspace_size.restype = i32
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                  i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk
                                  f32, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                          i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk
                                          f32, vp, fp, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                        i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk
                                        f32, vp, fp, f32, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd_gated.restype = i32
    lib.kda_gated_rmsnorm.argtypes = [vp, vp, i32, fp, f32, ctypes.c_long, i32, vp, vp]
    lib.kda_gated_rmsnorm.restype = i32
    lib.kda_chunk_fwd_split_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                       ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_split_workspace_size.restype = i32
    lib.kda_chunk_fwd_split.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                        i32, i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk segs
                                        f32, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd_split.restype = i32
    lib.kda_chunk_transition.argtypes = [vp, i32, fp, i32, fp, f32, fp, ip,
                                         i32, i32, i32, i32, i32, i32,  # N B T H Dk chunk
                                         fp, vp, sz, vp]
    lib.kda_chunk_transition.restype = i32
    lib.kda_compose_states.argtypes = [fp, fp, fp, i32, i32, i32, i32, i32, fp, vp]
    lib.kda_compose_states.restype = i32
    lib.kda_recurrent_step.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, i32, i32, i32,
                                       i32, f32, vp, vp]
    lib.kda_recurrent_step.restype = i32
    lib.kda_chunk_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                                 ctypes.POINTER(sz)]
    lib.kda_chunk_bwd_workspace_size.restype = i32
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                  i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk
                                  f32, vp, fp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_chunk_bwd_saved.argtypes = lib.kda_chunk_bwd.argtypes
    lib.kda_chunk_bwd_saved.restype = i32
    lib.kda_chunk_fwd_train.argtypes = [vp, vp, vp, i32, fp, i32, fp, f32, fp, fp, ip,
                                        i32, i32, i32, i32, i32, i32, i32,  # N B T H Dk Dv chunk
                                        f32, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd_train.restype = i32
    lib.kda_gate_bwd.argtypes = [fp, fp, f32, fp, ctypes.c_long, i32, i32, fp, fp, vp]
    lib.kda_gate_bwd.restype = i32
    lib.kda_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32, vp]
    lib.kda_device_status.restype = i32
    lib.kda_debug_set_spin_limit.argtypes = [i32]
    lib.kda_debug_set_spin_limit.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().kda_status_string(code).decode()


def check(code: int, what: str):
    if code == KDA_SUCCESS:
        return
    msg = f"{what}: {status_string(code)}"
    if code == KDA_ERROR_INVALID_VALUE:
        raise ValueError(msg)
    if code == KDA_ERROR_NOT_SUPPORTED:
        raise NotImplementedError(msg)
    raise KdaError(msg)
