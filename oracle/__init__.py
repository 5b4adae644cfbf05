"""CPU oracle for the Gated DeltaNet record / replay / GQA-expand path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library and its
Python binding never do.  It shares no code with the HIP path.

The arithmetic lives in ``gdn_oracle.c`` (plain double-precision loops, built
with ``gcc -O2 -ffp-contract=off``).  This module only builds and loads that
library and marshals numpy arrays: inputs are widened to float64 (exact for
fp32, fp16 and bf16), outputs come back as float64.

Sources: metaltile-std 0.1.0 ``src/ffai/gated_delta_replay.rs`` (record kernel
``gated_delta_record!``, replay kernel ``state_replay!``, "Tape layout") and
mlx-native 0.6.5 ``mlx_native/ops/repeat_tiled.rs`` ("Mapping").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GQA_BLOCK = 0
GQA_TILED = 1
_MAPS = {"block": GQA_BLOCK, "tiled": GQA_TILED, GQA_BLOCK: GQA_BLOCK, GQA_TILED: GQA_TILED}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` with gcc; returns the path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("GDN_ORACLE_LIB")   # a planted-mistake build, in the mutation tests
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        up = ctypes.POINTER(ctypes.c_uint32)
        u32 = ctypes.c_uint32
        lib.oracle_gdn_record.argtypes = [dp, dp, dp, dp, dp, dp, up, dp, dp, dp,
                                          u32, u32, u32, u32, u32, u32, ctypes.c_int]
        lib.oracle_gdn_record.restype = ctypes.c_int
        lib.oracle_gdn_replay.argtypes = [dp, dp, dp, dp, up, dp,
                                          u32, u32, u32, u32, u32, u32]
        lib.oracle_gdn_replay.restype = ctypes.c_int
        lib.oracle_gqa_expand.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                          u32, u32, u32, u32, u32, ctypes.c_int]
        lib.oracle_gqa_expand.restype = ctypes.c_int
        lib.oracle_rms_norm_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, dp, u32, u32,
                                             ctypes.c_double]
        lib.oracle_rms_norm_bf16.restype = ctypes.c_int
        _lib = lib
        return lib


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous float64 array (torch tensors included)."""
    if hasattr(x, "detach"):
        import torch  # only reached when the caller already holds torch tensors
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _u32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    a = np.asarray(x)
    if a.dtype.kind not in "iub":
        raise TypeError("mask must be an integer array")
    if a.dtype.kind == "i" and a.size and a.min() < 0:
        raise ValueError("mask entries are unsigned")
    return np.ascontiguousarray(a, dtype=np.uint32)


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _up(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def gdn_record(q, k, v, g, beta, state_in, mask=None, gqa_map="block",
               y_init=None, delta_init=None, want_delta=True):
    """Gated delta-rule forward step with tape capture, in float64.

    Shapes: q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g, beta [B,T,Hv];
    state_in [B,Hv,Dv,Dk]; mask [B,T] or None (every step active).
    Returns (y, state_out, delta_log) as float64 arrays.  Positions of inactive
    steps in y / delta_log keep ``y_init`` / ``delta_init`` (NaN by default),
    because the method writes nothing there.  With ``want_delta=False`` no tape
    is written and the third result is None.
    """
    q, k, v, g, beta, s0 = (_f64(a) for a in (q, k, v, g, beta, state_in))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape != (B, T, Hv, Dv) or g.shape != (B, T, Hv) \
            or beta.shape != (B, T, Hv) or s0.shape != (B, Hv, Dv, Dk):
        raise ValueError("inconsistent shapes")
    m = _u32(mask)
    if m is not None and m.shape != (B, T):
        raise ValueError("mask must be [B, T]")
    y = np.full(v.shape, np.nan) if y_init is None else _f64(y_init).copy()
    d = None
    if want_delta:
        d = np.full(v.shape, np.nan) if delta_init is None else _f64(delta_init).copy()
    s1 = np.empty_like(s0)
    rc = _load().oracle_gdn_record(_dp(q), _dp(k), _dp(v), _dp(g), _dp(beta), _dp(s0),
                                   _up(m), _dp(y), _dp(s1),
                                   _dp(d) if d is not None else None,
                                   B, T, Hk, Hv, Dk, Dv, _MAPS[gqa_map])
    if rc != 0:
        raise ValueError("oracle_gdn_record rejected its arguments")
    return y, s1, d


def gdn_replay(delta_log, k_log, g_log, state_in, mask=None, accepted=None):
    """Re-fold the accepted prefix of a tape onto a snapshot, in float64.

    Shapes: delta_log [B,T,Hv,Dv]; k_log [B,T,Hv,Dk]; g_log [B,T,Hv];
    state_in [B,Hv,Dv,Dk]; mask [B,T] or None.  ``accepted`` defaults to T.
    Returns state_out (float64).
    """
    d, kl, gl, s0 = (_f64(a) for a in (delta_log, k_log, g_log, state_in))
    B, T, Hv, Dv = d.shape
    Dk = kl.shape[3]
    if kl.shape != (B, T, Hv, Dk) or gl.shape != (B, T, Hv) or s0.shape != (B, Hv, Dv, Dk):
        raise ValueError("inconsistent shapes")
    m = _u32(mask)
    if m is not None and m.shape != (B, T):
        raise ValueError("mask must be [B, T]")
    if accepted is None:
        accepted = T
    s1 = np.empty_like(s0)
    rc = _load().oracle_gdn_replay(_dp(d), _dp(kl), _dp(gl), _dp(s0), _up(m), _dp(s1),
                                   B, T, Hv, Dk, Dv, int(accepted))
    if rc != 0:
        raise ValueError("oracle_gdn_replay rejected its arguments")
    return s1


def gqa_expand(src: np.ndarray, h: int, gqa_map="tiled") -> np.ndarray:
    """Byte-exact head broadcast [seq, hg, k] -> [seq, h, k] of any element type."""
    a = np.ascontiguousarray(src)
    if a.ndim != 3:
        raise ValueError("src must be [seq, hg, k]")
    seq, hg, kk = a.shape
    out = np.empty((seq, h, kk), dtype=a.dtype)
    rc = _load().oracle_gqa_expand(a.ctypes.data, out.ctypes.data, seq, hg, h, kk,
                                   a.dtype.itemsize, _MAPS[gqa_map])
    if rc != 0:
        raise ValueError("oracle_gqa_expand rejected its arguments")
    return out


def rms_norm_bf16(x, weight, eps: float) -> np.ndarray:
    """RMSNorm with bf16 weights ([P2] "GPU RMSNorm"), in float64.

    x: float32 [n, dim] (numpy or a torch tensor); weight: the bf16 weight [dim],
    given as a torch bfloat16 tensor or as its raw uint16 bits.  Returns
    out [n, dim] float64: out[t, i] = x[t, i] / sqrt(mean_i x[t]^2 + eps) * w[i].
    """
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    xa = np.ascontiguousarray(x, dtype=np.float32)
    if hasattr(weight, "detach"):
        import torch  # only reached when the caller already holds torch tensors
        weight = weight.detach().cpu().contiguous().view(torch.int16).numpy()
    wa = np.asarray(weight)
    if wa.dtype.itemsize != 2 or wa.dtype.kind not in "iu":
        raise TypeError("weight must be a bfloat16 tensor or its raw 16-bit pattern")
    wa = np.ascontiguousarray(wa.view(np.uint16))
    if xa.ndim != 2 or wa.shape != (xa.shape[1],):
        raise ValueError("x must be [n, dim] and weight [dim]")
    n, dim = xa.shape
    out = np.empty((n, dim), dtype=np.float64)
    if _load().oracle_rms_norm_bf16(xa.ctypes.data, wa.ctypes.data, _dp(out), n, dim, float(eps)) != 0:
        raise ValueError("oracle_rms_norm_bf16 rejected its arguments")
    return out


# ------------------------------------------------------------ prepared calls
#
# For timing the oracle itself (the CPU-baseline leg of the benchmark): the
# inputs are widened to float64 and the outputs allocated once, and the
# returned callable makes only the C call (ctypes releases the GIL around
# it, so threads run the oracle in parallel).  Same functions as above.

def prepare_record(q, k, v, g, beta, state_in, mask=None, gqa_map="block"):
    """A callable running oracle_gdn_record on fixed inputs; returns it and
    the output arrays (y, state_out, delta_log) it writes."""
    q, k, v, g, beta, s0 = (_f64(a) for a in (q, k, v, g, beta, state_in))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    m = _u32(mask)
    y = np.full(v.shape, np.nan)
    d = np.full(v.shape, np.nan)
    s1 = np.empty_like(s0)
    lib = _load()
    args = (_dp(q), _dp(k), _dp(v), _dp(g), _dp(beta), _dp(s0), _up(m), _dp(y), _dp(s1), _dp(d),
            B, T, Hk, Hv, Dk, Dv, _MAPS[gqa_map])
    keep = (q, k, v, g, beta, s0, m, y, d, s1)    # every array the pointers in args refer to

    def run():
        if lib.oracle_gdn_record(*args) != 0:
            raise ValueError("oracle_gdn_record rejected its arguments")
        return keep is not None
    return run, (y, s1, d)


def prepare_replay(delta_log, k_log, g_log, state_in, mask=None, accepted=None):
    """A callable running oracle_gdn_replay on fixed inputs; returns it and
    the state_out array it writes."""
    d, kl, gl, s0 = (_f64(a) for a in (delta_log, k_log, g_log, state_in))
    B, T, Hv, Dv = d.shape
    Dk = kl.shape[3]
    m = _u32(mask)
    s1 = np.empty_like(s0)
    lib = _load()
    args = (_dp(d), _dp(kl), _dp(gl), _dp(s0), _up(m), _dp(s1), B, T, Hv, Dk, Dv,
            T if accepted is None else int(accepted))
    keep = (d, kl, gl, s0, m, s1)

    def run():
        if lib.oracle_gdn_replay(*args) != 0:
            raise ValueError("oracle_gdn_replay rejected its arguments")
        return keep is not None
    return run, s1


def prepare_expand(src: np.ndarray, h: int, gqa_map="tiled"):
    """A callable running oracle_gqa_expand on a fixed [seq, hg, k] source;
    returns it and the destination array."""
    a = np.ascontiguousarray(src)
    seq, hg, kk = a.shape
    out = np.empty((seq, h, kk), dtype=a.dtype)
    lib = _load()
    args = (a.ctypes.data, out.ctypes.data, seq, hg, h, kk, a.dtype.itemsize, _MAPS[gqa_map])
    keep = (a, out)

    def run():
        if lib.oracle_gqa_expand(*args) != 0:
            raise ValueError("oracle_gqa_expand rejected its arguments")
        return keep is not None
    return run, out


def prepare_rms_norm_bf16(x, weight, eps: float):
    """A callable running oracle_rms_norm_bf16 on fixed inputs; returns it and
    the output array."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    xa = np.ascontiguousarray(x, dtype=np.float32)
    if hasattr(weight, "detach"):
        import torch  # only reached when the caller already holds torch tensors
        weight = weight.detach().cpu().contiguous().view(torch.int16).numpy()
    wa = np.ascontiguousarray(np.asarray(weight).view(np.uint16))
    n, dim = xa.shape
    out = np.empty((n, dim), dtype=np.float64)
    lib = _load()
    args = (xa.ctypes.data, wa.ctypes.data, _dp(out), n, dim, float(eps))
    keep = (xa, wa, out)

    def run():
        if lib.oracle_rms_norm_bf16(*args) != 0:
            raise ValueError("oracle_rms_norm_bf16 rejected its arguments")
        return keep is not None
    return run, out
