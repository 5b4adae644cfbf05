"""ctypes view of libgdn.so, the C ABI declared in include/gdn.h.

The library is built in-tree by ``linear_attention_recurrence_step_amd.build``.
There is no fallback: if it is missing or fails to load, importing this module
raises.  torch is imported first so that libgdn.so binds to the HIP runtime
already loaded by torch (same soname) and shares its streams.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libgdn.so links against)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

# include/gdn.h
GDN_F32, GDN_F16, GDN_BF16 = 0, 1, 2
GDN_GQA_BLOCK, GDN_GQA_TILED = 0, 1
STATUS = {
    0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_ZERO_DIM", -3: "GDN_ERR_GQA_RATIO",
    -4: "GDN_ERR_UNSUPPORTED_SHAPE", -5: "GDN_ERR_OVERFLOW", -6: "GDN_ERR_ALIAS",
    -7: "GDN_ERR_BAD_ENUM", -8: "GDN_ERR_LAUNCH", -9: "GDN_ERR_MISALIGNED",
    -10: "GDN_ERR_WORKSPACE",
}
GDN_FOLD_AUTO, GDN_FOLD_VALU, GDN_FOLD_MATRIX = 0, 1, 2
EXPORTS = ("gdn_record", "gdn_replay", "gqa_expand", "gdn_prefill", "gdn_prefill_workspace_size",
           "rms_norm_bf16", "gdn_record_debug", "gdn_replay_debug", "gdn_prefill_noalloc",
           "gdn_strerror", "gdn_last_error", "gdn_abi_version")
PREFILL_SCRATCH_BYTES = 68157440     # GDN_PREFILL_SCRATCH_BYTES
ABI_VERSION = 6


class LaunchChoice(ctypes.Structure):
    """gdn_launch_choice of include/gdn.h."""
    _fields_ = [("rows_per_thread", ctypes.c_uint32), ("threads", ctypes.c_uint32),
                ("replay_fold", ctypes.c_int32), ("matrix_waves", ctypes.c_uint32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libgdn.so is not built (%s); run `python -m linear_attention_recurrence_step_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
    lib.gdn_record.argtypes = [vp] * 12 + [u32] * 6 + [i32, i32, vp]
    lib.gdn_record.restype = i32
    lib.gdn_replay.argtypes = [vp] * 6 + [u32] * 6 + [i32, vp]
    lib.gdn_replay.restype = i32
    lc = ctypes.POINTER(LaunchChoice)
    lib.gdn_record_debug.argtypes = [lc] + lib.gdn_record.argtypes
    lib.gdn_record_debug.restype = i32
    lib.gdn_replay_debug.argtypes = [lc] + lib.gdn_replay.argtypes
    lib.gdn_replay_debug.restype = i32
    lib.gqa_expand.argtypes = [vp, vp] + [u32] * 4 + [i32, i32, vp]
    lib.gqa_expand.restype = i32
    lib.gdn_prefill.argtypes = [vp] * 13 + [ctypes.c_uint64] + [u32] * 6 + [i32, i32, vp]
    lib.gdn_prefill.restype = i32
    lib.gdn_prefill_noalloc.argtypes = [vp] * 12 + [u32] * 6 + [i32, i32, vp]
    lib.gdn_prefill_noalloc.restype = i32
    lib.gdn_prefill_workspace_size.argtypes = [u32] * 3
    lib.gdn_prefill_workspace_size.restype = ctypes.c_uint64
    lib.rms_norm_bf16.argtypes = [vp, vp, vp, u32, u32, ctypes.c_float, vp]
    lib.rms_norm_bf16.restype = i32
    lib.gdn_strerror.argtypes = [i32]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = i32
    if lib.gdn_abi_version() != ABI_VERSION:
        raise ImportError("libgdn.so ABI version %d, binding expects %d"
                          % (lib.gdn_abi_version(), ABI_VERSION))
    return lib


lib = _load()


class GdnError(RuntimeError):
    """A libgdn call returned a negative gdn_status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        detail = lib.gdn_last_error().decode(errors="replace")
        super().__init__("%s failed with %s: %s" % (fn, self.status_name, detail))


def check(fn: str, status: int) -> None:
    if status != 0:
        raise GdnError(fn, status)
