"""gdn_prefill_noalloc: the chunked prefill with its workspace in the library's
own scratch area (no allocation in the call), through the C ABI, against
gdn_prefill with a caller-owned workspace (the same kernels: the outputs must
agree bit for bit) and against the oracle's per-step record (2e-2, bf16 I/O).

Two calls in a row, the second on a smaller input, show that a call does not
depend on what the previous one left in the shared scratch area; the largest
size the area holds (a 4096-step prefill over 32 value heads) runs too, and
one block more is refused before any launch.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
import linear_attention_recurrence_step_amd as gdn
from gpu_util import assert_close, dev, f64, note, step_mask, to_dev

pytestmark = pytest.mark.gpu

Y_SENTINEL = -7.5
D_SENTINEL = 3.25


def _outputs(d):
    io = d["q"].dtype
    return dict(y=torch.full(d["v"].shape, Y_SENTINEL, dtype=io, device=dev()),
                delta_log=torch.full(d["v"].shape, D_SENTINEL, dtype=io, device=dev()),
                state_out=torch.empty_like(d["state_in"]))


def _bits(t):
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def _both(inp, gqa_map):
    """(noalloc outputs, workspace outputs) for the same inputs."""
    d = to_dev(inp)
    o1, o2 = _outputs(d), _outputs(d)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"])
    gdn.gdn_prefill_noalloc(*args, gqa_map=gqa_map, **o1)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(*d["v"].shape[:3]), dtype=torch.uint8, device=dev())
    gdn.gdn_prefill(*args, gqa_map=gqa_map, workspace=ws, **o2)
    torch.cuda.synchronize()
    return o1, o2


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_prefill_equals_workspace_prefill_on_consecutive_calls(order):
    cases = [(2, 300, 2, 4, 128, "bernoulli", "tiled", 11), (1, 70, 1, 2, 64, "trailing", "block", 12)]
    for B, T, Hk, Hv, Dv, mask, gqa_map, seed in cases:
        inp = gi.record_inputs(B, T, Hk, Hv, 128, Dv, "bf16", seed=seed, mask=mask)
        note("gdn_prefill_noalloc B=%d T=%d Hk=%d Hv=%d Dv=%d %s %s" % (B, T, Hk, Hv, Dv, mask, gqa_map))
        o1, o2 = _both(inp, gqa_map)
        for name in ("y", "delta_log", "state_out"):
            assert torch.equal(_bits(o1[name]), _bits(o2[name])), name
        ry, rs, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                       inp["state_in"], inp["mask"], gqa_map=gqa_map)
        act = np.broadcast_to(step_mask(inp["mask"], B, T)[:, :, None, None], ry.shape)
        assert_close(o1["y"], ry, torch.bfloat16, "noalloc y", where=act)
        assert_close(o1["delta_log"], rd, torch.bfloat16, "noalloc delta", where=act)
        assert_close(o1["state_out"], rs, torch.bfloat16, "noalloc state")
        assert np.all(f64(o1["y"])[~act] == Y_SENTINEL)
        assert np.all(f64(o1["delta_log"])[~act] == D_SENTINEL)


def test_noalloc_prefill_at_the_scratch_capacity():
    """B * Hv * ceil(T / 64) = 2048 blocks: the whole scratch area."""
    w = gi.WORKLOADS["chunk_prefill"]
    inp = gi.workload_inputs("chunk_prefill", 4)
    assert gdn.gdn_prefill_workspace_size(w.B, w.T, w.Hv) == gdn.PREFILL_SCRATCH_BYTES
    note("gdn_prefill_noalloc at the scratch capacity (4096 steps, 32 heads)")
    o1, o2 = _both(inp, w.gqa_map)
    for name in ("y", "delta_log", "state_out"):
        assert torch.equal(_bits(o1[name]), _bits(o2[name])), name
    for hv in (5, 30):
        hk = hv % w.Hk                                              # tiled map
        ry, rs, rd = oracle.gdn_record(inp["q"][:, :, hk:hk + 1], inp["k"][:, :, hk:hk + 1],
                                       inp["v"][:, :, hv:hv + 1], inp["g"][:, :, hv:hv + 1],
                                       inp["beta"][:, :, hv:hv + 1], inp["state_in"][:, hv:hv + 1], None)
        assert_close(o1["y"][:, :, hv:hv + 1], ry, torch.bfloat16, "noalloc y head %d" % hv)
        assert_close(o1["state_out"][:, hv:hv + 1], rs, torch.bfloat16, "noalloc state head %d" % hv)


def test_noalloc_prefill_refuses_more_than_the_scratch():
    inp = gi.record_inputs(1, 4097, 1, 32, 128, 16, "bf16", seed=13, mask="none")   # 65 chunks x 32 heads
    d = to_dev(inp)
    o = _outputs(d)
    note("gdn_prefill_noalloc past the scratch capacity (refused on the host)")
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], None, **o)
    assert err.value.status_name == "GDN_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(o["y"] == Y_SENTINEL)                          # nothing ran


def test_prefill_noalloc_captures_like_prefill():
    inp = gi.record_inputs(2, 90, 2, 4, 128, 32, io="bf16", seed=77, mask="bernoulli")
    note("prefill_noalloc with capture")
    d = to_dev(inp)
    logs = []
    for fn in (gdn.gdn_prefill, gdn.gdn_prefill_noalloc):
        kl = torch.full((2, 90, 4, 128), 5.5, dtype=torch.bfloat16, device=dev())
        gl = torch.full((2, 90, 4), -0.625, dtype=torch.bfloat16, device=dev())
        fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"], gqa_map="tiled",
           k_log=kl, g_log=gl)
        torch.cuda.synchronize()
        logs.append((kl, gl))
    assert torch.equal(logs[0][0], logs[1][0]) and torch.equal(logs[0][1], logs[1][1])
