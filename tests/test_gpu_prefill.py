"""GPU parity of gdn_prefill (the record step computed 64 steps at a time on the
matrix cores) against the CPU oracle's record, through the C ABI.

gdn_prefill computes the record kernel's outputs with the arithmetic reordered
into chunk products, so the oracle's plain per-step record is the reference:
y and delta_log at active steps and the final state must be within 2e-2
(bf16 I/O) of it, scaled as |gpu - oracle| <= tol * (1 + |oracle|), and
positions of inactive steps must keep the caller's sentinel.
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


def _prefill_gpu(inp, gqa_map, write_tape=True, workspace=None, in_place=False):
    d = to_dev(inp)
    io = d["q"].dtype
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=io, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=io, device=dev()) if write_tape else None
    s_out = d["state_in"] if in_place else None
    y, s, dl = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                               gqa_map=gqa_map, y=y, delta_log=dl, write_tape=write_tape,
                               state_out=s_out, workspace=workspace)
    torch.cuda.synchronize()
    return y, s, dl


def _check(inp, gqa_map, what):
    note("prefill %s map=%s" % (what, gqa_map))
    y, s, dl = _prefill_gpu(inp, gqa_map)
    ry, rs, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["state_in"], inp["mask"], gqa_map=gqa_map)
    io = inp["q"].dtype
    B, T = inp["q"].shape[:2]
    act = np.broadcast_to(step_mask(inp["mask"], B, T)[:, :, None, None], ry.shape)
    assert_close(y, ry, io, what + " y", where=act)
    assert_close(dl, rd, io, what + " delta", where=act)
    assert_close(s, rs, io, what + " state")
    assert np.all(f64(y)[~act] == Y_SENTINEL), what + ": y written at an inactive step"
    assert np.all(f64(dl)[~act] == D_SENTINEL), what + ": delta written at an inactive step"
    return y, s, dl


# (B, T, Hk, Hv, Dv, mask, map): one step, exactly one chunk, ragged chunk
# tails, several chunks, masks, both GQA maps, several row blocks per head.
CASES = [
    (1, 1, 1, 1, 16, "ones", "block"),
    (1, 64, 2, 4, 32, "ones", "block"),
    (1, 65, 1, 1, 16, "ones", "tiled"),
    (2, 200, 2, 4, 128, "bernoulli", "tiled"),
    (1, 130, 1, 2, 48, "trailing", "block"),
    (3, 127, 4, 4, 16, "bernoulli", "block"),
    (2, 256, 2, 6, 64, "none", "tiled"),
    (1, 100, 1, 1, 1024, "bernoulli", "block"),     # the widest head the ABI takes
    (16, 33, 4, 8, 32, "trailing", "tiled"),        # many heads, one ragged chunk each
    # more value heads per key head than one prep workgroup takes (four):
    # a full and a partial set of value heads, and two full sets
    (1, 70, 1, 5, 32, "bernoulli", "block"),
    (2, 65, 2, 16, 16, "trailing", "tiled"),
    (1, 100, 2, 8, 32, "bernoulli", "tiled"),       # exactly one full set of four
]


@pytest.mark.parametrize("case", CASES, ids=["B%d_T%d_Hk%d_Hv%d_Dv%d_%s_%s" % c for c in CASES])
def test_prefill_matches_oracle(case):
    B, T, Hk, Hv, Dv, mask, gmap = case
    inp = gi.record_inputs(B, T, Hk, Hv, 128, Dv, io="bf16", seed=11 + T, mask=mask)
    _check(inp, gmap, "B%d T%d Dv%d %s" % (B, T, Dv, mask))


def test_prefill_workload_sampled_heads():
    """The 4096-step prefill at full size; the oracle re-runs four sampled
    value heads one by one (each head is an independent recurrence)."""
    w = gi.WORKLOADS["chunk_prefill"]
    inp = gi.workload_inputs("chunk_prefill", 0)
    note("prefill chunk_prefill full size")
    y, s, dl = _prefill_gpu(inp, w.gqa_map)
    io = inp["q"].dtype
    for hv in (0, 5, 16, 31):
        hk = hv % w.Hk                                              # tiled map
        sub = dict(q=inp["q"][:, :, hk:hk + 1], k=inp["k"][:, :, hk:hk + 1],
                   v=inp["v"][:, :, hv:hv + 1], g=inp["g"][:, :, hv:hv + 1],
                   beta=inp["beta"][:, :, hv:hv + 1], state_in=inp["state_in"][:, hv:hv + 1])
        ry, rs, rd = oracle.gdn_record(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                       sub["state_in"], None)
        assert_close(y[:, :, hv:hv + 1], ry, io, "prefill y head %d" % hv)
        assert_close(dl[:, :, hv:hv + 1], rd, io, "prefill delta head %d" % hv)
        assert_close(s[:, hv:hv + 1], rs, io, "prefill state head %d" % hv)


def test_prefill_workload_all_heads_near_sequential_record():
    """Every head of the 4096-step workload: the chunked and the sequential
    GPU records agree to the bf16 tolerance (the sequential record is itself
    pinned to the oracle by the record parity tests)."""
    w = gi.WORKLOADS["chunk_prefill"]
    inp = gi.workload_inputs("chunk_prefill", 1)
    note("prefill vs sequential record, chunk_prefill full size")
    y, s, dl = _prefill_gpu(inp, w.gqa_map)
    d = to_dev(inp)
    y2, s2, dl2 = gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], None,
                                 gqa_map=w.gqa_map)
    torch.cuda.synchronize()
    io = inp["q"].dtype
    assert_close(y, f64(y2), io, "y vs sequential record")
    assert_close(dl, f64(dl2), io, "delta vs sequential record")
    assert_close(s, f64(s2), io, "state vs sequential record")


def test_prefill_in_place_reused_workspace_and_no_tape():
    """state_out == state_in, a workspace holding an earlier call's contents,
    and delta_log = NULL all give the same bits as a fresh out-of-place call."""
    inp = gi.record_inputs(2, 150, 2, 4, 128, 64, io="bf16", seed=5, mask="bernoulli")
    note("prefill in place / reused workspace / no tape")
    ws = torch.empty(gdn.gdn_prefill_workspace_size(2, 150, 4), dtype=torch.uint8, device=dev())
    y0, s0, d0 = _prefill_gpu(inp, "block", workspace=ws)
    other = gi.record_inputs(2, 150, 2, 4, 128, 64, io="bf16", seed=6, mask="ones")
    _prefill_gpu(other, "tiled", workspace=ws)                       # leave other contents behind
    y1, s1, d1 = _prefill_gpu(inp, "block", workspace=ws, in_place=True)
    y2, s2, _ = _prefill_gpu(inp, "block", write_tape=False)
    assert torch.equal(y0, y1) and torch.equal(s0, s1) and torch.equal(d0, d1)
    assert torch.equal(y0, y2) and torch.equal(s0, s2)


def test_prefill_zero_and_unit_gates():
    """Gates of exactly 0 (the state is reset) and identity steps (g = 1,
    beta = 0) inside chunks: the gate products are formed without division."""
    inp = gi.record_inputs(1, 192, 1, 2, 128, 32, io="bf16", seed=9, mask="ones")
    g = inp["g"].clone()
    beta = inp["beta"].clone()
    g[0, [3, 64, 100, 101, 191], :] = 0.0
    g[0, 10:30, 1] = 1.0
    beta[0, 10:30, 1] = 0.0
    inp = dict(inp, g=g, beta=beta)
    _check(inp, "block", "zero and unit gates")


@pytest.mark.parametrize("io,Dk", [("bf16", 128), ("f16", 192)])
def test_prefill_nan_at_inactive_steps_never_reaches_an_output(io, Dk):
    """Inactive steps are skipped by selection, not by a product with zero:
    NaN in their q, k, v, g and beta cannot reach y, delta or the state."""
    inp = gi.record_inputs(2, 100, 2, 4, Dk, 32, io=io, seed=4, mask="bernoulli")
    m = inp["mask"].numpy() > 0
    poisoned = {}
    for name in ("q", "k", "v", "g", "beta"):
        t = inp[name].clone()
        t[torch.from_numpy(~m)] = float("nan")
        poisoned[name] = t
    inp = dict(inp, **poisoned)
    y, s, dl = _check(inp, "tiled", "NaN at inactive steps")
    assert not torch.isnan(s).any()


def _sweep_cases(n=24, seed=4242):
    """A fixed, seeded list of mixed configurations for the chunked prefill:
    lengths from one step to several chunks with ragged last chunks, batch
    rows, GQA ratios 1-3, value widths 16-256, both maps and every mask kind
    (an all-zero mask included)."""
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Dv = int(r.choice([16, 32, 48, 64, 96, 128, 256]))
        Hk = int(r.integers(1, 4))
        Hv = Hk * int(r.integers(1, 4))
        B = int(r.integers(1, 4))
        T = int(r.choice([1, 3, 17, 63, 64, 65, 100, 128, 129, 191, 256, 300]))
        while B * Hv * Dv * 128 * T > 12_000_000 and T > 1:   # keep the oracle to about a second
            T //= 2
        gmap = str(r.choice(["block", "tiled"]))
        mask = str(r.choice(["none", "ones", "trailing", "bernoulli", "zeros"]))
        cases.append((B, T, Hk, Hv, Dv, gmap, mask, seed + i))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dv%d_%s_%s_s%d" % c)
def test_prefill_seeded_sweep(case):
    B, T, Hk, Hv, Dv, gmap, mask, seed = case
    inp = gi.record_inputs(B, T, Hk, Hv, 128, Dv, io="bf16", seed=seed, mask=mask)
    _check(inp, gmap, "sweep %s" % (case,))


K_SENTINEL = 5.5
G_SENTINEL = -0.625


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy()


CAPTURE = [
    # B, T, Hk, Hv, Dk, Dv, io, map, mask: one step, ragged chunks, several
    # chunks, both maps, both key widths and both dtypes
    (1, 1, 1, 2, 128, 16, "bf16", "block", "ones"),
    (2, 70, 2, 4, 128, 64, "bf16", "tiled", "bernoulli"),
    (1, 129, 1, 3, 128, 32, "bf16", "block", "trailing"),
    (3, 64, 2, 2, 128, 16, "bf16", "tiled", "zeros"),
    (1, 100, 2, 4, 192, 32, "f16", "tiled", "bernoulli"),
    (2, 65, 4, 4, 192, 128, "bf16", "block", "trailing"),
    (1, 70, 1, 6, 128, 16, "bf16", "tiled", "bernoulli"),     # two sets of value heads per key head
    (1, 64, 2, 12, 128, 16, "f16", "block", "ones"),
]


@pytest.mark.parametrize("case", CAPTURE, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s" % c)
def test_prefill_captures_expanded_keys_and_gates(case):
    """k_log holds the keys expanded to value heads and g_log the gates, bit
    for bit, at active steps only; capturing changes no other output, and the
    captured tape replays exactly like one expanded by a separate pass."""
    B, T, Hk, Hv, Dk, Dv, io, gmap, mask = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io=io, seed=31 + T, mask=mask)
    note("prefill with capture %s" % (case,))
    d = to_dev(inp)
    dt = d["q"].dtype
    kl = torch.full((B, T, Hv, Dk), K_SENTINEL, dtype=dt, device=dev())
    gl = torch.full((B, T, Hv), G_SENTINEL, dtype=dt, device=dev())
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=dt, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=dt, device=dev())
    y, s, dl = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                               gqa_map=gmap, y=y, delta_log=dl, k_log=kl, g_log=gl)
    torch.cuda.synchronize()
    y0, s0, dl0 = _prefill_gpu(inp, gmap)
    assert torch.equal(y, y0) and torch.equal(s, s0) and torch.equal(dl, dl0)
    act = step_mask(inp["mask"], B, T).reshape(B * T)
    ref_k = oracle.gqa_expand(_bits(inp["k"]).reshape(B * T, Hk, Dk), Hv, gmap)
    got_k = _bits(kl).reshape(B * T, Hv, Dk)
    assert np.array_equal(got_k[act], ref_k[act]), "k_log differs from the expanded keys"
    assert np.all(f64(kl).reshape(B * T, Hv, Dk)[~act] == K_SENTINEL), "k_log written at an inactive step"
    got_g, ref_g = _bits(gl).reshape(B * T, Hv), _bits(inp["g"]).reshape(B * T, Hv)
    assert np.array_equal(got_g[act], ref_g[act]), "g_log differs from g"
    assert np.all(f64(gl).reshape(B * T, Hv)[~act] == G_SENTINEL), "g_log written at an inactive step"
    k_exp = gdn.gqa_expand(d["k"], Hv, gmap)
    for acc in sorted({0, 1, min(T, 6)}):
        note("replay of a prefill-captured tape, accepted=%d" % acc)
        r1 = gdn.gdn_replay(dl, kl, gl, d["state_in"], d["mask"], acc)
        r2 = gdn.gdn_replay(dl, k_exp, d["g"], d["state_in"], d["mask"], acc)
        torch.cuda.synchronize()
        assert torch.equal(r1, r2), acc


# Key width 192 (the record page's shape-cell heads) and fp16 I/O: one step,
# ragged chunks, several chunks, masks, both maps, Hk < Hv.
WIDE = [
    # B, T, Hk, Hv, Dk, Dv, io, mask, map
    (1, 1, 4, 4, 192, 128, "bf16", "ones", "block"),
    (1, 200, 4, 4, 192, 128, "bf16", "bernoulli", "block"),
    (2, 130, 1, 2, 192, 32, "bf16", "trailing", "tiled"),
    (1, 65, 2, 4, 128, 64, "f16", "ones", "tiled"),
    (2, 150, 2, 4, 128, 128, "f16", "bernoulli", "block"),
    (1, 129, 4, 4, 192, 128, "f16", "trailing", "block"),
    (3, 64, 1, 3, 192, 16, "f16", "none", "tiled"),
    (1, 100, 1, 1, 192, 1024, "f16", "bernoulli", "block"),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s" % c)
def test_prefill_wide_keys_and_f16(case):
    B, T, Hk, Hv, Dk, Dv, io, mask, gmap = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io=io, seed=57 + T, mask=mask)
    _check(inp, gmap, "B%d T%d Dk%d Dv%d %s %s" % (B, T, Dk, Dv, io, mask))


def test_prefill_d192_workload_all_heads():
    """The 4096-step prefill at the Dk=192, Dv=128, Hk=Hv=4 cell at full size,
    every head against the oracle."""
    w = gi.WORKLOADS["prefill_d192_128"]
    inp = gi.workload_inputs("prefill_d192_128", 0)
    _check(inp, w.gqa_map, "prefill_d192_128 full size")


def test_prefill_f16_zero_and_unit_gates():
    inp = gi.record_inputs(1, 150, 2, 2, 192, 32, io="f16", seed=19, mask="ones")
    g = inp["g"].clone()
    beta = inp["beta"].clone()
    g[0, [0, 63, 64, 120], :] = 0.0
    g[0, 70:90, 0] = 1.0
    beta[0, 70:90, 0] = 0.0
    inp = dict(inp, g=g, beta=beta)
    _check(inp, "tiled", "fp16 zero and unit gates")


def _wide_sweep(n=12, seed=777):
    """Seeded mixed configurations over both key widths and both dtypes."""
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Dk = int(r.choice([128, 192]))
        io = str(r.choice(["bf16", "f16"]))
        Dv = int(r.choice([16, 32, 64, 128]))
        Hk = int(r.integers(1, 4))
        Hv = Hk * int(r.integers(1, 3))
        B = int(r.integers(1, 3))
        T = int(r.choice([1, 17, 64, 65, 129, 200]))
        while B * Hv * Dv * Dk * T > 12_000_000 and T > 1:
            T //= 2
        cases.append((B, T, Hk, Hv, Dk, Dv, io, str(r.choice(["block", "tiled"])),
                      str(r.choice(["none", "ones", "trailing", "bernoulli"])), seed + i))
    return cases


@pytest.mark.parametrize("case", _wide_sweep(), ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s_s%d" % c)
def test_prefill_wide_seeded_sweep(case):
    B, T, Hk, Hv, Dk, Dv, io, gmap, mask, seed = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io=io, seed=seed, mask=mask)
    _check(inp, gmap, "wide sweep %s" % (case,))


def test_prefill_on_a_side_stream_with_its_own_workspace():
    """On a stream that is not the current one, with the workspace allocated
    by the binding: the workspace belongs to that stream, so memory the
    current stream allocates and writes while the kernels run cannot be it."""
    inp = gi.record_inputs(2, 300, 2, 4, 128, 64, io="bf16", seed=21, mask="bernoulli")
    note("prefill on a side stream, binding-allocated workspace")
    d = to_dev(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=torch.bfloat16, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=torch.bfloat16, device=dev())
    y, s, dl = gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                               gqa_map="tiled", y=y, delta_log=dl, stream=side)
    junk = [torch.full((gdn.gdn_prefill_workspace_size(2, 300, 4) // 4,), float("nan"), device=dev())
            for _ in range(4)]                      # the current stream's pool, written at once
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    ry, rs, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["state_in"], inp["mask"], gqa_map="tiled")
    act = np.broadcast_to(step_mask(inp["mask"], 2, 300)[:, :, None, None], ry.shape)
    assert_close(y, ry, torch.bfloat16, "side-stream y", where=act)
    assert_close(dl, rd, torch.bfloat16, "side-stream delta", where=act)
    assert_close(s, rs, torch.bfloat16, "side-stream state")
