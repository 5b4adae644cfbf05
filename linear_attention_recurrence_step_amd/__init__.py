"""Gated DeltaNet record / replay / GQA-expand for AMD Instinct MI355X (gfx950).

Python binding of libgdn (include/gdn.h).  Each function has the name of its
C entry point, checks that the torch tensors it is given have the layouts the
C ABI expects, allocates missing outputs with torch, and calls the library on
the current torch stream.  Every step of the computation runs in the HIP
kernels; there is no CPU fallback, and importing this package fails if the
library has not been built.

Layouts (dense, contiguous):
    q, k [B,T,Hk,Dk]; v, y, delta_log [B,T,Hv,Dv]; g, beta [B,T,Hv];
    state [B,Hv,Dv,Dk] float32; mask [B,T] int32/uint32 (active iff > 0);
    k_log [B,T,Hv,Dk]; g_log [B,T,Hv].
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _native
from ._native import GdnError, lib

__all__ = ["gdn_record", "gdn_replay", "gqa_expand", "gdn_prefill", "gdn_prefill_workspace_size",
           "rms_norm_bf16", "gdn_record_debug", "gdn_replay_debug", "gdn_prefill_noalloc", "GdnError",
           "IO_DTYPES", "PREFILL_SCRATCH_BYTES"]

PREFILL_SCRATCH_BYTES = _native.PREFILL_SCRATCH_BYTES

IO_DTYPES = {torch.float32: _native.GDN_F32, torch.float16: _native.GDN_F16,
             torch.bfloat16: _native.GDN_BF16}
_MAPS = {"block": _native.GDN_GQA_BLOCK, "tiled": _native.GDN_GQA_TILED}
_FOLDS = {"auto": _native.GDN_FOLD_AUTO, "valu": _native.GDN_FOLD_VALU,
          "matrix": _native.GDN_FOLD_MATRIX}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> torch.cuda.Stream:
    """The torch stream a call's kernels are enqueued on: the current stream
    when none is given, a torch stream as given, or a raw hipStream_t handle
    (an int) wrapped as an external stream.  Outputs and workspaces the
    binding allocates are allocated on this stream, so the caching allocator
    never hands their memory to other work before these kernels are done."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _choice(launch: Optional[dict]):
    """gdn_launch_choice from {"tiling": (rows_per_thread, threads),
    "fold": "auto"|"valu"|"matrix", "matrix_waves": 0|2|4} (None: all automatic)."""
    if launch is None:
        return None
    unknown = set(launch) - {"tiling", "fold", "matrix_waves"}
    if unknown:
        raise ValueError("unknown launch choice keys: %s" % sorted(unknown))
    rpt, nt = launch.get("tiling", (0, 0))
    fold = launch.get("fold", "auto")
    if fold not in _FOLDS:
        raise ValueError("fold must be one of %s" % sorted(_FOLDS))
    return _native.LaunchChoice(int(rpt), int(nt), _FOLDS[fold], int(launch.get("matrix_waves", 0)))


def _want(name: str, t: torch.Tensor, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if isinstance(dtype, tuple):
        if t.dtype not in dtype:
            raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtype))
    elif t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _device_of(t: torch.Tensor) -> torch.device:
    """The GPU all tensors of a call must live on; host tensors are refused
    here, before any pointer reaches the library."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device, got %s" % t.device)
    return t.device


def _io_code(t: torch.Tensor) -> int:
    if t.dtype not in IO_DTYPES:
        raise TypeError("I/O tensors must be float32, float16 or bfloat16, got %s" % t.dtype)
    return IO_DTYPES[t.dtype]


_MASK_DTYPES = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _record(choice, q, k, v, g, beta, state_in, mask, gqa_map, y, state_out, delta_log, write_tape,
            k_log, g_log, stream):
    if gqa_map not in _MAPS:
        raise ValueError("gqa_map must be 'block' or 'tiled'")
    dev = _device_of(q)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    io = q.dtype
    _io_code(q)
    _want("q", q, (B, T, Hk, Dk), io, dev)
    _want("k", k, (B, T, Hk, Dk), io, dev)
    _want("v", v, (B, T, Hv, Dv), io, dev)
    _want("g", g, (B, T, Hv), io, dev)
    _want("beta", beta, (B, T, Hv), io, dev)
    _want("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if mask is not None:
        _want("mask", mask, (B, T), _MASK_DTYPES, dev)
    st = _stream(stream, dev)
    with torch.cuda.stream(st):
        if y is None:
            y = torch.empty((B, T, Hv, Dv), dtype=io, device=dev)
        if state_out is None:
            state_out = torch.empty_like(state_in)
        if delta_log is None and write_tape:
            delta_log = torch.empty((B, T, Hv, Dv), dtype=io, device=dev)
    _want("y", y, (B, T, Hv, Dv), io, dev)
    _want("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    if delta_log is not None:
        _want("delta_log", delta_log, (B, T, Hv, Dv), io, dev)
    if k_log is not None:
        _want("k_log", k_log, (B, T, Hv, Dk), io, dev)
    if g_log is not None:
        _want("g_log", g_log, (B, T, Hv), io, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(mask), _ptr(y),
            _ptr(state_out), _ptr(delta_log), _ptr(k_log), _ptr(g_log), B, T, Hk, Hv, Dk, Dv,
            _io_code(q), _MAPS[gqa_map], st.cuda_stream)
    if choice is None:
        _native.check("gdn_record", lib.gdn_record(*args))
    else:
        _native.check("gdn_record_debug", lib.gdn_record_debug(choice, *args))
    return y, state_out, delta_log


def gdn_record(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
               beta: torch.Tensor, state_in: torch.Tensor, mask: Optional[torch.Tensor] = None,
               *, gqa_map: str = "block", y: Optional[torch.Tensor] = None,
               state_out: Optional[torch.Tensor] = None,
               delta_log: Optional[torch.Tensor] = None, write_tape: bool = True,
               k_log: Optional[torch.Tensor] = None, g_log: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Gated delta-rule step with tape capture; returns (y, state_out, delta_log).

    Outputs that are not given are allocated (uninitialised: the positions of
    inactive steps in y and delta_log are not written).  ``state_out`` may be
    ``state_in`` itself.  With ``write_tape=False`` and no ``delta_log`` the
    plain forward step runs and the third result is None.  ``k_log``
    [B,T,Hv,Dk] and ``g_log`` [B,T,Hv], if given, receive the rest of the tape
    (keys expanded to value heads, and gates) at active steps.  ``stream`` is a
    torch stream or a raw hipStream_t (default: the current stream).
    """
    return _record(None, q, k, v, g, beta, state_in, mask, gqa_map, y, state_out, delta_log,
                   write_tape, k_log, g_log, stream)


def gdn_record_debug(launch: Optional[dict], q, k, v, g, beta, state_in, mask=None, *,
                     gqa_map: str = "block", y=None, state_out=None, delta_log=None,
                     write_tape: bool = True, k_log=None, g_log=None, stream=None):
    """gdn_record with its launch shape forced (tests and launch-shape sweeps):
    ``launch`` = {"tiling": (rows_per_thread, threads)}; None or {} is gdn_record."""
    return _record(_choice(launch), q, k, v, g, beta, state_in, mask, gqa_map, y, state_out,
                   delta_log, write_tape, k_log, g_log, stream)


def gdn_prefill_workspace_size(B: int, T: int, Hv: int) -> int:
    """Bytes of device workspace gdn_prefill needs for these sizes."""
    return int(lib.gdn_prefill_workspace_size(B, T, Hv))


def _prefill(noalloc, q, k, v, g, beta, state_in, mask, gqa_map, y, state_out, delta_log,
             write_tape, k_log, g_log, workspace, stream):
    if gqa_map not in _MAPS:
        raise ValueError("gqa_map must be 'block' or 'tiled'")
    dev = _device_of(q)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    io = q.dtype
    _io_code(q)
    _want("q", q, (B, T, Hk, Dk), io, dev)
    _want("k", k, (B, T, Hk, Dk), io, dev)
    _want("v", v, (B, T, Hv, Dv), io, dev)
    _want("g", g, (B, T, Hv), io, dev)
    _want("beta", beta, (B, T, Hv), io, dev)
    _want("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if mask is not None:
        _want("mask", mask, (B, T), _MASK_DTYPES, dev)
    st = _stream(stream, dev)
    need = gdn_prefill_workspace_size(B, T, Hv)
    with torch.cuda.stream(st):
        if y is None:
            y = torch.empty((B, T, Hv, Dv), dtype=io, device=dev)
        if state_out is None:
            state_out = torch.empty_like(state_in)
        if delta_log is None and write_tape:
            delta_log = torch.empty((B, T, Hv, Dv), dtype=io, device=dev)
        if workspace is None and not noalloc:
            # freed when this call returns: allocated on the kernels' stream, so
            # its memory is not reused before they have finished with it
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _want("y", y, (B, T, Hv, Dv), io, dev)
    _want("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    if delta_log is not None:
        _want("delta_log", delta_log, (B, T, Hv, Dv), io, dev)
    if k_log is not None:
        _want("k_log", k_log, (B, T, Hv, Dk), io, dev)
    if g_log is not None:
        _want("g_log", g_log, (B, T, Hv), io, dev)
    outs = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(mask), _ptr(y),
            _ptr(state_out), _ptr(delta_log), _ptr(k_log), _ptr(g_log))
    if noalloc:
        rc = lib.gdn_prefill_noalloc(*outs, B, T, Hk, Hv, Dk, Dv, _io_code(q), _MAPS[gqa_map],
                                     st.cuda_stream)
        _native.check("gdn_prefill_noalloc", rc)
        return y, state_out, delta_log
    _want("workspace", workspace, (workspace.numel(),), torch.uint8, dev)
    rc = lib.gdn_prefill(*outs, _ptr(workspace), workspace.numel(), B, T, Hk, Hv, Dk, Dv,
                         _io_code(q), _MAPS[gqa_map], st.cuda_stream)
    _native.check("gdn_prefill", rc)
    return y, state_out, delta_log


def gdn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state_in: torch.Tensor, mask: Optional[torch.Tensor] = None,
                *, gqa_map: str = "block", y: Optional[torch.Tensor] = None,
                state_out: Optional[torch.Tensor] = None,
                delta_log: Optional[torch.Tensor] = None, write_tape: bool = True,
                k_log: Optional[torch.Tensor] = None, g_log: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """The record step over a long sequence, 64 steps at a time on the matrix
    cores; returns (y, state_out, delta_log) as gdn_record does.

    bf16 or fp16 I/O, Dk = 128 or 192, Dv a multiple of 16.  ``k_log`` and ``g_log``, if given,
    receive the rest of the tape as in gdn_record.  ``workspace`` (a uint8
    device tensor of at least gdn_prefill_workspace_size(B, T, Hv) bytes) is
    allocated when not given; pass one to reuse it across calls on one stream.
    """
    return _prefill(False, q, k, v, g, beta, state_in, mask, gqa_map, y, state_out, delta_log,
                    write_tape, k_log, g_log, workspace, stream)


def gdn_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, state_in: torch.Tensor,
                        mask: Optional[torch.Tensor] = None, *, gqa_map: str = "block",
                        y: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                        delta_log: Optional[torch.Tensor] = None, write_tape: bool = True,
                        k_log: Optional[torch.Tensor] = None, g_log: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """gdn_prefill with its workspace in the library's own scratch area
    (PREFILL_SCRATCH_BYTES per GPU, shared by every such call on that GPU):
    the library call allocates nothing.  Pass y, state_out and delta_log (or
    write_tape=False) so that this binding allocates nothing either.  Calls
    whose kernels overlap in time on one GPU race; calls on one stream are
    ordered."""
    return _prefill(True, q, k, v, g, beta, state_in, mask, gqa_map, y, state_out, delta_log,
                    write_tape, k_log, g_log, None, stream)


def _replay(choice, delta_log, k_log, g_log, state_in, mask, accepted, state_out, stream):
    dev = _device_of(delta_log)
    B, T, Hv, Dv = delta_log.shape
    Dk = k_log.shape[3]
    io = delta_log.dtype
    _io_code(delta_log)
    _want("delta_log", delta_log, (B, T, Hv, Dv), io, dev)
    _want("k_log", k_log, (B, T, Hv, Dk), io, dev)
    _want("g_log", g_log, (B, T, Hv), io, dev)
    _want("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if mask is not None:
        _want("mask", mask, (B, T), _MASK_DTYPES, dev)
    if accepted is None:
        accepted = T
    if not 0 <= int(accepted) < 2 ** 32:
        raise ValueError("accepted must fit in uint32")
    st = _stream(stream, dev)
    if state_out is None:
        with torch.cuda.stream(st):
            state_out = torch.empty_like(state_in)
    _want("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    args = (_ptr(delta_log), _ptr(k_log), _ptr(g_log), _ptr(state_in), _ptr(mask), _ptr(state_out),
            B, T, Hv, Dk, Dv, int(accepted), _io_code(delta_log), st.cuda_stream)
    if choice is None:
        _native.check("gdn_replay", lib.gdn_replay(*args))
    else:
        _native.check("gdn_replay_debug", lib.gdn_replay_debug(choice, *args))
    return state_out


def gdn_replay(delta_log: torch.Tensor, k_log: torch.Tensor, g_log: torch.Tensor,
               state_in: torch.Tensor, mask: Optional[torch.Tensor] = None,
               accepted: Optional[int] = None, *, state_out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Speculative-decode rollback: apply tape positions [0, accepted) to the
    snapshot; returns state_out.

    ``accepted`` defaults to the tape length; values past it act as the tape
    length.  ``state_out`` may be ``state_in`` itself.
    """
    return _replay(None, delta_log, k_log, g_log, state_in, mask, accepted, state_out, stream)


def gdn_replay_debug(launch: Optional[dict], delta_log, k_log, g_log, state_in, mask=None,
                     accepted=None, *, state_out=None, stream=None):
    """gdn_replay with its kernel forced (tests and launch-shape sweeps):
    ``launch`` = {"fold": "valu"|"matrix"|"auto", "tiling": (rows_per_thread,
    threads), "matrix_waves": 2|4}; None or {} is gdn_replay."""
    return _replay(_choice(launch), delta_log, k_log, g_log, state_in, mask, accepted, state_out,
                   stream)


def gqa_expand(src: torch.Tensor, h: int, gqa_map: str = "tiled", *,
               dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Head broadcast [..., hg, k] -> [..., h, k] (all leading dims flattened to seq)."""
    if gqa_map not in _MAPS:
        raise ValueError("gqa_map must be 'block' or 'tiled'")
    if src.dim() < 2:
        raise ValueError("src must be [..., hg, k]")
    dev = _device_of(src)
    hg, kk = src.shape[-2], src.shape[-1]
    seq = 1
    for d in src.shape[:-2]:
        seq *= d
    code = _io_code(src)
    out_shape = tuple(src.shape[:-2]) + (h, kk)
    _want("src", src, tuple(src.shape), src.dtype, dev)
    st = _stream(stream, dev)
    if dst is None:
        with torch.cuda.stream(st):
            dst = torch.empty(out_shape, dtype=src.dtype, device=dev)
    _want("dst", dst, out_shape, src.dtype, dev)
    rc = lib.gqa_expand(_ptr(src), _ptr(dst), seq, hg, h, kk, code, _MAPS[gqa_map], st.cuda_stream)
    _native.check("gqa_expand", rc)
    return dst


def rms_norm_bf16(x: torch.Tensor, weight: torch.Tensor, eps: float, *,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """RMSNorm with a bf16 weight: out[t] = x[t] / sqrt(mean(x[t]^2) + eps) * weight.

    x: float32 [..., dim] (leading dims flattened to tokens); weight: bfloat16
    [dim].  ``out`` may be ``x`` itself.
    """
    if x.dim() < 1:
        raise ValueError("x must be [..., dim]")
    dev = _device_of(x)
    dim = x.shape[-1]
    n = x.numel() // dim if dim else 0
    _want("x", x, tuple(x.shape), torch.float32, dev)
    _want("weight", weight, (dim,), torch.bfloat16, dev)
    st = _stream(stream, dev)
    if out is None:
        with torch.cuda.stream(st):
            out = torch.empty_like(x)
    _want("out", out, tuple(x.shape), torch.float32, dev)
    rc = lib.rms_norm_bf16(_ptr(x), _ptr(weight), _ptr(out), n, dim, float(eps), st.cuda_stream)
    _native.check("rms_norm_bf16", rc)
    return out
