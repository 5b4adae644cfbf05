"""Seeded synthetic inputs for the Gated DeltaNet record / replay / GQA-expand path.

Shared by the tests, the smoke check and the benchmark; used to feed both the
HIP library and the CPU oracle.  It holds none of the method's arithmetic:
it only draws random numbers, shapes them like the workloads below and casts
them to the I/O dtype.

Recipe (every draw from ``numpy.random.Generator(PCG64(seed))`` in float64,
then cast to float32, then to the I/O dtype by torch on the CPU, which rounds
to nearest even):

* q, k ~ N(0, 1), each Dk-vector divided by its L2 norm (in float32) before the
  cast -- the record kernel applies no normalisation of its own, so callers
  normalise;
* v ~ N(0, 1);
* g = exp(-softplus(x)) = sigmoid(-x), x ~ N(0, 1), so 0 < g < 1;
* beta = sigmoid(x), x ~ N(0, 1);
* state ~ N(0, 0.1^2) in float32 (the recurrent state is always float32);
* masks: all ones, per-row trailing zeros (z_b ~ U{0,1,2} inactive trailing
  steps per batch row), or Bernoulli(p) per (b, t);
* replay tapes: delta ~ N(0, 0.5^2), k_log and g_log drawn like k and g.

Workload table: the five shapes the path is measured and tested on.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

IO_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    io: str                       # "f32" | "f16" | "bf16"
    gqa_map: str                  # "block" | "tiled"
    mask: str                     # "none" | "ones" | "trailing" | "bernoulli"
    accepted: Tuple[int, ...] = ()
    expand_io: Optional[str] = None   # dtype of the standalone GQA expansion, if any
    mask_p: float = 0.7
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=4, Hk=2, Hv=4, Dk=32, Dv=32, io="f32",
                     gqa_map="block", mask="ones", accepted=(3,),
                     note="small parity case"),
    "spec_decode": Workload("spec_decode", B=8, T=4, Hk=16, Hv=32, Dk=128, Dv=128,
                            io="bf16", gqa_map="block", mask="trailing",
                            accepted=(0, 1, 2, 3, 4),
                            note="speculative-decode step, record then rollback"),
    "large_batch_decode": Workload("large_batch_decode", B=256, T=1, Hk=16, Hv=32,
                                   Dk=128, Dv=128, io="bf16", gqa_map="block",
                                   mask="ones", accepted=(1,),
                                   note="decode step at batch 256; 512 MiB of fp32 state"),
    "chunk_prefill": Workload("chunk_prefill", B=1, T=4096, Hk=16, Hv=32, Dk=128,
                              Dv=128, io="bf16", gqa_map="tiled", mask="none",
                              expand_io="f32",
                              note="4096-step recurrence after a tiled fp32 q/k expansion"),
    "long_tape_replay": Workload("long_tape_replay", B=32, T=64, Hk=48, Hv=48, Dk=128,
                                 Dv=128, io="f16", gqa_map="block", mask="bernoulli",
                                 accepted=(0, 1, 16, 63, 64), mask_p=0.7,
                                 note="replay of a 64-step fp16 tape, keys pre-expanded"),
    # The two head-shape cells the record/replay page instantiates besides the
    # main one, as decode steps with a state of a few hundred MiB (the page
    # gives no batch size for them).
    "cell_d192_128": Workload("cell_d192_128", B=1024, T=1, Hk=4, Hv=4, Dk=192, Dv=128,
                              io="bf16", gqa_map="block", mask="ones", accepted=(1,),
                              note="Dk=192, Dv=128, Hk=Hv=4 decode step; 384 MiB of fp32 state"),
    "cell_d64_32": Workload("cell_d64_32", B=16384, T=1, Hk=2, Hv=2, Dk=64, Dv=32,
                            io="bf16", gqa_map="block", mask="ones", accepted=(1,),
                            note="Dk=64, Dv=32, Hk=Hv=2 decode step; 256 MiB of fp32 state"),
    # The main cell's record over a 4096-step sequence (the prefill length of
    # chunk_prefill), keys already one per value head.
    "prefill_d192_128": Workload("prefill_d192_128", B=1, T=4096, Hk=4, Hv=4, Dk=192, Dv=128,
                                 io="bf16", gqa_map="block", mask="none",
                                 note="4096-step record at the Dk=192, Dv=128, Hk=Hv=4 cell"),
}

# Workloads whose step is one long record (a prefill), not a decode step.
PREFILL_WORKLOADS = ("chunk_prefill", "prefill_d192_128")


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_io(a: np.ndarray, io: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(IO_DTYPES[io]).contiguous()


def _unit_rows(r: np.random.Generator, shape) -> np.ndarray:
    x = r.standard_normal(shape).astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return x / np.maximum(n, np.float32(1e-30))


def _gate(r: np.random.Generator, shape) -> np.ndarray:
    x = r.standard_normal(shape)
    return (1.0 / (1.0 + np.exp(x))).astype(np.float32)        # exp(-softplus(x))


def _sigmoid(r: np.random.Generator, shape) -> np.ndarray:
    x = r.standard_normal(shape)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def make_mask(r: np.random.Generator, B: int, T: int, kind: str, p: float = 0.7):
    """uint32-valued int32 tensor [B, T] (or None for kind == "none")."""
    if kind == "none":
        return None
    if kind == "ones":
        m = np.ones((B, T), dtype=np.int32)
    elif kind == "zeros":
        m = np.zeros((B, T), dtype=np.int32)
    elif kind == "trailing":
        z = r.integers(0, 3, size=B)                     # 0, 1 or 2 trailing inactive steps
        m = (np.arange(T)[None, :] < (T - z)[:, None]).astype(np.int32)
    elif kind == "bernoulli":
        m = (r.random((B, T)) < p).astype(np.int32)
    else:
        raise ValueError(kind)
    return torch.from_numpy(m)


def record_inputs(B, T, Hk, Hv, Dk, Dv, io="bf16", seed=0, mask="ones", mask_p=0.7):
    """Inputs of one record call as torch CPU tensors (state in float32)."""
    r = rng(seed)
    q = _to_io(_unit_rows(r, (B, T, Hk, Dk)), io)
    k = _to_io(_unit_rows(r, (B, T, Hk, Dk)), io)
    v = _to_io(r.standard_normal((B, T, Hv, Dv)), io)
    g = _to_io(_gate(r, (B, T, Hv)), io)
    beta = _to_io(_sigmoid(r, (B, T, Hv)), io)
    state = torch.from_numpy((0.1 * r.standard_normal((B, Hv, Dv, Dk))).astype(np.float32))
    m = make_mask(r, B, T, mask, mask_p)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state, mask=m)


def tape_inputs(B, T, Hv, Dk, Dv, io="f16", seed=0, mask="bernoulli", mask_p=0.7):
    """A synthetic innovation tape (delta_log, k_log, g_log), snapshot and mask."""
    r = rng(seed)
    delta = _to_io(0.5 * r.standard_normal((B, T, Hv, Dv)), io)
    k_log = _to_io(_unit_rows(r, (B, T, Hv, Dk)), io)
    g_log = _to_io(_gate(r, (B, T, Hv)), io)
    state = torch.from_numpy((0.1 * r.standard_normal((B, Hv, Dv, Dk))).astype(np.float32))
    m = make_mask(r, B, T, mask, mask_p)
    return dict(delta_log=delta, k_log=k_log, g_log=g_log, state_in=state, mask=m)


def poison_untaken(tape: dict, accepted: int, value: float = float("nan")) -> dict:
    """Copy of a tape whose slots the replay must not take (masked, or at
    t >= accepted) are overwritten with ``value`` (NaN by default)."""
    out = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in tape.items()}
    B, T = out["delta_log"].shape[:2]
    taken = torch.arange(T)[None, :] < accepted
    if out.get("mask") is not None:
        taken = taken & (out["mask"] > 0)
    untaken = ~taken.expand(B, T)
    for name in ("delta_log", "k_log", "g_log"):
        out[name][untaken] = value
    return out


def expand_source(seq, hg, k, io="f32", seed=0):
    """Source tensor [seq, hg, k] for a standalone GQA expansion."""
    r = rng(seed)
    return _to_io(r.standard_normal((seq, hg, k)), io)


def workload_inputs(name: str, seed: int = 0, B: Optional[int] = None):
    """Record inputs for a named workload (optionally with a smaller batch)."""
    w = WORKLOADS[name]
    return record_inputs(B or w.B, w.T, w.Hk, w.Hv, w.Dk, w.Dv, w.io, seed, w.mask, w.mask_p)


# RMSNorm workload: the pre-norm of the layer over a prefill's tokens.  The
# page gives no hidden size; 2048 is taken, with the prefill length above.
NORM_WORKLOADS = {
    "rms_norm_prefill": dict(n_tokens=4096, dim=2048, eps=1e-6,
                             note="RMSNorm of 4096 fp32 hidden states of width 2048, bf16 weight"),
}


def norm_inputs(n_tokens, dim, seed=0):
    """Hidden states x ~ N(0, 1) in float32 [n, dim] and a bf16 weight near 1,
    1 + N(0, 0.1), [dim] (torch CPU tensors)."""
    r = rng(seed)
    x = torch.from_numpy(r.standard_normal((n_tokens, dim)).astype(np.float32))
    w = torch.from_numpy((1.0 + 0.1 * r.standard_normal(dim)).astype(np.float32)).to(torch.bfloat16)
    return x, w


def norm_inputs_on_device(n_tokens, dim, device, seed=0):
    """norm_inputs' distributions for sizes too large to draw on the host: x
    ~ N(0, 1) float32 [n, dim] drawn on `device` by torch's seeded generator,
    and the bf16 weight [dim] as a CPU tensor (from the host generator)."""
    x = torch.empty((n_tokens, dim), dtype=torch.float32, device=device)
    x.normal_(generator=torch.Generator(device=device).manual_seed(seed))
    r = rng(seed)
    w = torch.from_numpy((1.0 + 0.1 * r.standard_normal(dim)).astype(np.float32)).to(torch.bfloat16)
    return x, w
