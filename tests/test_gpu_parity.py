"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input comes from the seeded generators in gdn_inputs; every expected
value comes from the oracle (or, for the cross-kernel identities, from another
call of the HIP path, compared bit for bit).  Floating-point outputs must be
within 1e-3 (float32 I/O) or 2e-2 (float16 / bfloat16 I/O) of the oracle,
scaled as |gpu - oracle| <= tol * (1 + |oracle|); GQA expansion must match
byte for byte.  Positions of inactive steps must keep the caller's sentinel.
"""
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
import linear_attention_recurrence_step_amd as gdn
from gpu_util import TOL, assert_close, dev, f64, note, step_mask, to_dev

pytestmark = pytest.mark.gpu

Y_SENTINEL = -7.5       # exact in every I/O dtype
D_SENTINEL = 3.25


def _record_gpu(inp, gqa_map, write_tape=True):
    d = to_dev(inp)
    io = d["q"].dtype
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=io, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=io, device=dev()) if write_tape else None
    y, s, dl = gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                              gqa_map=gqa_map, y=y, delta_log=dl, write_tape=write_tape)
    torch.cuda.synchronize()
    return y, s, dl


def _check_record(inp, gqa_map, what):
    note("record %s map=%s" % (what, gqa_map))
    y, s, dl = _record_gpu(inp, gqa_map)
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


def _check_replay(tape, accepted, what):
    note("replay %s accepted=%d" % (what, accepted))
    d = to_dev(tape)
    s = gdn.gdn_replay(d["delta_log"], d["k_log"], d["g_log"], d["state_in"], d["mask"], accepted)
    torch.cuda.synchronize()
    rs = oracle.gdn_replay(tape["delta_log"], tape["k_log"], tape["g_log"], tape["state_in"],
                           tape["mask"], accepted)
    assert_close(s, rs, tape["delta_log"].dtype, what + " state")
    return s


# ------------------------------------------------------------------ record

@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("spec_decode", 0),
                                       ("spec_decode", 1), ("large_batch_decode", 0)])
def test_record_workloads(name, seed):
    w = gi.WORKLOADS[name]
    _check_record(gi.workload_inputs(name, seed), w.gqa_map, "%s/seed%d" % (name, seed))


def test_record_chunk_prefill_sampled_heads():
    """Full 4096-step prefill on the GPU; the oracle re-runs four sampled value
    heads one by one (each head is an independent recurrence)."""
    w = gi.WORKLOADS["chunk_prefill"]
    inp = gi.workload_inputs("chunk_prefill", 0)
    note("record chunk_prefill full size")
    y, s, dl = _record_gpu(inp, w.gqa_map)
    io = inp["q"].dtype
    for hv in (0, 7, 16, 31):
        hk = hv % w.Hk                                              # tiled map
        sub = dict(q=inp["q"][:, :, hk:hk + 1], k=inp["k"][:, :, hk:hk + 1],
                   v=inp["v"][:, :, hv:hv + 1], g=inp["g"][:, :, hv:hv + 1],
                   beta=inp["beta"][:, :, hv:hv + 1], state_in=inp["state_in"][:, hv:hv + 1])
        ry, rs, rd = oracle.gdn_record(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                       sub["state_in"], None)
        assert_close(y[:, :, hv:hv + 1], ry, io, "prefill y head %d" % hv)
        assert_close(dl[:, :, hv:hv + 1], rd, io, "prefill delta head %d" % hv)
        assert_close(s[:, hv:hv + 1], rs, io, "prefill state head %d" % hv)


# The page's two other head-shape cells: decode at the workload size (sampled
# batch rows re-run by the oracle), and short tapes with masks at small B.
@pytest.mark.parametrize("name", ["cell_d192_128", "cell_d64_32"])
def test_shape_cell_decode_workloads(name):
    w = gi.WORKLOADS[name]
    inp = gi.workload_inputs(name, 3)
    note("record %s at full size" % name)
    y, s, dl = _record_gpu(inp, w.gqa_map)
    rows = np.random.Generator(np.random.PCG64(5)).choice(w.B, size=8, replace=False)
    sub = {k2: (v[rows] if isinstance(v, torch.Tensor) else v) for k2, v in inp.items()}
    ry, rs, rd = oracle.gdn_record(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                   sub["state_in"], sub["mask"], gqa_map=w.gqa_map)
    io = inp["q"].dtype
    assert_close(y[rows], ry, io, name + " y")
    assert_close(dl[rows], rd, io, name + " delta")
    assert_close(s[rows], rs, io, name + " state")
    d = to_dev(inp)
    k_log = gdn.gqa_expand(d["k"], w.Hv, w.gqa_map)
    s_rep = gdn.gdn_replay(dl, k_log, d["g"], d["state_in"], d["mask"], 1)
    torch.cuda.synchronize()
    if io == torch.float32:
        assert torch.equal(s_rep, s)
    else:
        assert_close(s_rep[rows], rs, io, name + " replay")


@pytest.mark.parametrize("cell", [(192, 128, 4, 4), (64, 32, 2, 2)])
@pytest.mark.parametrize("T,mask", [(4, "trailing"), (3, "bernoulli"), (37, "none")])
def test_shape_cell_short_tapes(cell, T, mask):
    Dk, Dv, Hk, Hv = cell
    for io in ("bf16", "f32"):
        inp = gi.record_inputs(3, T, Hk, Hv, Dk, Dv, io, seed=7 + T, mask=mask)
        _check_record(inp, "block", "cell %s T=%d %s %s" % (cell, T, mask, io))
        tape = gi.tape_inputs(2, T, Hv, Dk, Dv, io, seed=9 + T, mask="bernoulli")
        for a in sorted({1, T // 2, T}):
            _check_replay(gi.poison_untaken(tape, a), a, "cell %s T=%d %s" % (cell, T, io))


RAGGED = [
    # B, T, Hk, Hv, Dk, Dv, io, map, mask
    (3, 5, 1, 3, 32, 16, "f32", "block", "bernoulli"),
    (2, 3, 2, 6, 64, 48, "bf16", "tiled", "trailing"),
    (1, 7, 4, 4, 192, 128, "f16", "block", "bernoulli"),     # Dk=192, Dv=128, Hk=Hv=4 cell
    (2, 2, 2, 2, 64, 32, "f32", "block", "ones"),            # Dk=64, Dv=32, Hk=Hv=2 cell
    (1, 3, 3, 3, 256, 64, "bf16", "tiled", "none"),
    (5, 1, 2, 8, 128, 80, "bf16", "block", "ones"),
    (4, 9, 2, 4, 128, 128, "f16", "tiled", "bernoulli"),
    (1, 33, 1, 2, 32, 32, "f32", "tiled", "none"),
    # chunk lengths: 16 (up to 16 steps), 32 (a grid of more workgroups than
    # CUs), 64 (long tapes over few heads), each with a ragged last chunk
    (2, 14, 2, 4, 64, 64, "f32", "block", "none"),
    (4, 37, 8, 16, 128, 128, "bf16", "block", "bernoulli"),
    (1, 150, 2, 4, 128, 128, "bf16", "tiled", "bernoulli"),
    (1, 131, 1, 2, 64, 32, "f16", "block", "none"),
    # the largest head the library takes: Dk = 256, Dv = 1024 (1 MiB of state per head)
    (2, 1, 1, 2, 256, 1024, "bf16", "block", "ones"),
    (1, 5, 1, 1, 256, 1024, "f32", "block", "bernoulli"),
    (1, 40, 1, 1, 256, 1024, "bf16", "block", "none"),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s" % c)
def test_record_ragged_shapes(case):
    B, T, Hk, Hv, Dk, Dv, io, m, mk = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io, seed=B * 100 + T, mask=mk)
    if mk == "bernoulli":
        inp["mask"][0, 0] = 0          # make sure some step is inactive
        inp["mask"][:, -1] *= 5        # and that mask values > 1 count as active
    _check_record(inp, m, "ragged")


def _hand_inputs(name, io):
    """A golden hand case with Dk = Dv = 2, zero-padded into a 32 x 32 state."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        c = json.load(f)
    T = c.get("T", 1)
    pad = lambda a, shape: torch.nn.functional.pad(torch.tensor(a, dtype=torch.float64).reshape(shape),
                                                   (0, 30))
    q = pad(c["q"], (1, T, 1, 2))
    k = pad(c["k"], (1, T, 1, 2))
    v = pad(c["v"], (1, T, 1, 2))
    s0 = torch.zeros(1, 1, 32, 32, dtype=torch.float64)
    s0[0, 0, :2, :2] = torch.tensor(c["S0"], dtype=torch.float64)
    g = torch.tensor(c["g"], dtype=torch.float64).reshape(1, T, 1)
    beta = torch.tensor(c["beta"], dtype=torch.float64).reshape(1, T, 1)
    mask = torch.tensor(c.get("mask", [1] * T), dtype=torch.int32).reshape(1, T)
    dt = gi.IO_DTYPES[io]
    inp = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.to(dt), beta=beta.to(dt),
               state_in=s0.to(torch.float32), mask=mask)
    return c, inp


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
def test_record_and_replay_hand_cases_exact(io):
    """The golden hand cases use short dyadic numbers: every intermediate is
    exact in float32 and every output exact in the I/O dtype."""
    c, inp = _hand_inputs("hand_t1.json", io)
    y, s, dl = _record_gpu(inp, "block")
    assert f64(y)[0, 0, 0, :2].tolist() == c["expect"]["y"]
    assert f64(dl)[0, 0, 0, :2].tolist() == c["expect"]["delta"]
    assert f64(s)[0, 0, :2, :2].tolist() == c["expect"]["S1"]
    assert np.all(f64(s)[0, 0, 2:] == 0) and np.all(f64(s)[0, 0, :, 2:] == 0)

    c, inp = _hand_inputs("hand_t3_mask.json", io)
    y, s, dl = _record_gpu(inp, "block")
    e = c["expect"]
    for t in range(3):
        if e["y"][t] is None:
            assert np.all(f64(y)[0, t] == Y_SENTINEL) and np.all(f64(dl)[0, t] == D_SENTINEL)
        else:
            assert f64(y)[0, t, 0, :2].tolist() == e["y"][t]
            assert f64(dl)[0, t, 0, :2].tolist() == e["delta"][t]
    assert f64(s)[0, 0, :2, :2].tolist() == e["S_final"]
    d = to_dev(inp)
    for a, want in e["replay"].items():
        note("hand replay accepted=%s io=%s" % (a, io))
        rs = gdn.gdn_replay(dl, d["k"], d["g"], d["state_in"], d["mask"], int(a))
        torch.cuda.synchronize()
        assert f64(rs)[0, 0, :2, :2].tolist() == want, a


# ------------------------------------------------------------------ replay

@pytest.mark.parametrize("accepted", [0, 1, 2, 3, 4, 9])
def test_replay_spec_decode(accepted):
    w = gi.WORKLOADS["spec_decode"]
    tape = gi.tape_inputs(w.B, w.T, w.Hv, w.Dk, w.Dv, w.io, seed=accepted, mask="trailing")
    _check_replay(gi.poison_untaken(tape, accepted), accepted, "spec_decode")


def test_replay_large_batch_decode():
    w = gi.WORKLOADS["large_batch_decode"]
    tape = gi.tape_inputs(w.B, w.T, w.Hv, w.Dk, w.Dv, w.io, seed=3, mask="ones")
    _check_replay(tape, 1, "large_batch_decode")


@pytest.mark.parametrize("accepted", [0, 1, 16, 63, 64])
def test_replay_long_tape_nan_poisoned(accepted):
    """Untaken slots (masked, or at or past `accepted`) hold NaN: none may leak."""
    w = gi.WORKLOADS["long_tape_replay"]
    tape = gi.tape_inputs(w.B, w.T, w.Hv, w.Dk, w.Dv, w.io, seed=11, mask="bernoulli", mask_p=w.mask_p)
    s = _check_replay(gi.poison_untaken(tape, accepted), accepted, "long_tape")
    assert torch.isfinite(s).all()


@pytest.mark.parametrize("io", ["f32", "f16"])
def test_replay_long_fold_with_extreme_gates(io):
    """Long folds carry the state with a running scale; gates of 0, 1e-20, 1e-6
    and runs of 1.9 (the scale leaves its range both ways) must still match."""
    B, T, Hv, Dk, Dv = 2, 48, 2, 64, 32
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=71, mask="bernoulli", mask_p=0.9)
    g = torch.full((B, T, Hv), 0.8)
    g[:, 3] = 0.0
    g[:, 7, 0] = 1e-20 if io == "f32" else 1e-7
    g[:, 11:45, 1] = 1.9
    g[:, 20] = 1e-6 if io == "f32" else 1e-4
    tape["g_log"] = g.to(gi.IO_DTYPES[io])
    for a in (T, 30):
        _check_replay(tape, a, "extreme gates")


MFMA_REPLAY = [
    # B, T_log, Hv, Dk, Dv, io, mask, accepted values (Dv a multiple of 64 takes the
    # matrix cores; the Dv = 48 case checks that other shapes keep the VALU fold)
    (2, 40, 3, 128, 128, "f16", "bernoulli", (16, 17, 33, 40)),
    (3, 20, 2, 64, 64, "bf16", "none", (16, 20)),
    (1, 35, 2, 32, 64, "f16", "trailing", (35,)),
    (2, 18, 2, 192, 64, "bf16", "bernoulli", (18,)),
    (1, 24, 1, 256, 128, "f16", "none", (24,)),
    (2, 64, 4, 128, 192, "bf16", "bernoulli", (64,)),
    (2, 20, 2, 64, 48, "f16", "bernoulli", (20,)),
]


def _replay_fold(tape, accepted, fold, state_out=None, waves=0):
    """gdn_replay_debug with the fold forced ("valu" or "matrix")."""
    d = to_dev(tape)
    so = None
    if state_out == "in_place":
        so = d["state_in"]
    s = gdn.gdn_replay_debug({"fold": fold, "matrix_waves": waves}, d["delta_log"], d["k_log"],
                             d["g_log"], d["state_in"], d["mask"], accepted, state_out=so)
    torch.cuda.synchronize()
    return s


@pytest.mark.parametrize("case", MFMA_REPLAY, ids=lambda c: "B%d_T%d_Hv%d_Dk%d_Dv%d_%s_%s" % c[:7])
def test_replay_long_fold_on_matrix_cores(case):
    """Folds of 16+ positions of a 16-bit tape run as MFMA products over
    chunks of positions; against the oracle at the I/O tolerance, untaken
    slots NaN-poisoned, and against the VALU fold of the same tape."""
    B, T, Hv, Dk, Dv, io, mask, accepted = case
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=111 + Dk + T, mask=mask)
    for a in accepted:
        pt = gi.poison_untaken(tape, a)
        s_auto = _check_replay(pt, a, "matrix-core fold %s" % (case[:7],))
        note("VALU fold of the same tape, accepted=%d" % a)
        s_valu = _replay_fold(pt, a, "valu")
        assert_close(s_auto, f64(s_valu), torch.float32, "matrix-core vs VALU fold")
        if Dv % 64 == 0:
            note("forced matrix-core fold, accepted=%d" % a)
            s_mat = _replay_fold(pt, a, "matrix")
            assert torch.equal(_bit_view(s_auto), _bit_view(s_mat)), "automatic fold is not the matrix one"


def _gate_case(B, T, Hv, Dk, Dv, io, seed, gates):
    """A NaN-poisoned Bernoulli tape whose taken gates are overwritten at
    given (t0, t1, value) ranges (all heads)."""
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=seed, mask="bernoulli", mask_p=0.8)
    g = tape["g_log"].float().clone()
    for t0, t1, val in gates:
        g[:, t0:t1] = val
    tape["g_log"] = g.to(gi.IO_DTYPES[io])
    return tape


# Chunks of 32 positions whose taken gates leave [0, 1] (or are NaN or
# infinite) run the matrix-core fold's per-position path on the state itself;
# the neighbouring chunks keep the one-pass contraction.
GATE_CASES = [
    # name, Dv, io, T, gate ranges (t0, t1, value)
    ("above_one_then_whole", 64, "f16", 48, [(5, 6, 1.5), (9, 10, 1.9), (20, 21, -0.5)]),
    ("whole_then_above_one", 128, "bf16", 70, [(40, 41, 1.5), (50, 51, 1.9), (60, 61, -0.5)]),
    ("negative_gates", 128, "f16", 40, [(0, 3, -0.5), (33, 34, -1.0)]),
    ("run_of_four_64", 64, "f16", 64, [(0, 64, 4.0)]),
    ("run_of_four_bf16", 128, "bf16", 64, [(0, 64, 4.0)]),
    ("large_then_tiny", 64, "bf16", 96, [(0, 30, 3.0), (64, 96, 1e-3)]),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_matrix_core_fold_with_gates_outside_unit_interval(case):
    """Taken gates of 1.5, 1.9, -0.5, runs of 3 and 4 (the state grows by 2^128
    over 64 positions without overflowing) in some chunks but not others:
    the matrix-core fold against the oracle and against the VALU fold."""
    name, Dv, io, T, gates = case
    B, Hv, Dk = 2, 2, 128
    tape = _gate_case(B, T, Hv, Dk, Dv, io, seed=131 + T, gates=gates)
    if name.startswith("run_of_four"):
        tape["mask"] = None                         # every one of the 64 gates is taken
    for a in sorted({T, T - 7, 40}):
        pt = gi.poison_untaken(tape, a)
        note("matrix-core fold with gates outside [0, 1]: %s accepted=%d" % (name, a))
        s_mat = _replay_fold(pt, a, "matrix")
        rs = oracle.gdn_replay(pt["delta_log"], pt["k_log"], pt["g_log"], pt["state_in"], pt["mask"], a)
        assert np.isfinite(rs).all()
        assert_close(s_mat, rs, tape["delta_log"].dtype, "%s matrix fold a=%d" % (name, a))
        s_valu = _replay_fold(pt, a, "valu")
        assert_close(s_mat, f64(s_valu), tape["delta_log"].dtype, "%s matrix vs VALU a=%d" % (name, a))


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("bad", ["nan", "inf", "-inf"])
def test_matrix_core_fold_with_non_finite_gates(io, bad):
    """A NaN or infinite gate at one taken position: the oracle's state holds
    NaN or infinities there on, and the matrix-core fold must put NaN exactly
    where the oracle does (other values within tolerance)."""
    B, T, Hv, Dk, Dv = 2, 48, 2, 64, 64
    val = {"nan": float("nan"), "inf": float("inf"), "-inf": float("-inf")}[bad]
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=141, mask="none")
    g = tape["g_log"].float().clone()
    g[0, 37, 1] = val                               # second chunk, batch row 0, head 1 only
    tape["g_log"] = g.to(gi.IO_DTYPES[io])
    for a in (T, 30):
        note("matrix-core fold with a %s gate, %s, accepted=%d" % (bad, io, a))
        s_mat = _replay_fold(tape, a, "matrix")
        rs = oracle.gdn_replay(tape["delta_log"], tape["k_log"], tape["g_log"], tape["state_in"],
                               None, a)
        got = f64(s_mat)
        assert np.array_equal(np.isnan(got), np.isnan(rs)), "NaN positions differ"
        assert np.array_equal(np.isinf(got), np.isinf(rs)), "infinite positions differ"
        fin = np.isfinite(rs)
        assert_close(got[fin], rs[fin], tape["delta_log"].dtype, "%s gate, finite part" % bad)
        if a == 30:                                 # the bad gate lies past `accepted`
            assert np.isfinite(got).all()


@pytest.mark.parametrize("gates", ["unit", "outside"])
@pytest.mark.parametrize("waves", [2, 4])
def test_matrix_core_fold_in_place(gates, waves):
    """state_out == state_in on the matrix-core fold (both workgroup shapes),
    with whole-chunk contractions and with the per-position path, equals the
    out-of-place result bit for bit."""
    B, T, Hv, Dk, Dv = 3, 45, 2, 128, 128
    if gates == "unit":
        tape = gi.tape_inputs(B, T, Hv, Dk, Dv, "bf16", seed=151, mask="bernoulli")
    else:
        tape = _gate_case(B, T, Hv, Dk, Dv, "bf16", 152, [(3, 4, 1.7), (35, 36, -0.25)])
    note("matrix-core fold out of place, %s gates, %d waves" % (gates, waves))
    ref = _replay_fold(tape, T, "matrix", waves=waves)
    d = to_dev(tape)
    st = d["state_in"].clone()
    note("matrix-core fold in place, %s gates, %d waves" % (gates, waves))
    gdn.gdn_replay_debug({"fold": "matrix", "matrix_waves": waves}, d["delta_log"], d["k_log"],
                         d["g_log"], st, d["mask"], T, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(_bit_view(st), _bit_view(ref))
    rs = oracle.gdn_replay(tape["delta_log"], tape["k_log"], tape["g_log"], tape["state_in"],
                           tape["mask"], T)
    assert_close(st, rs, torch.bfloat16, "in-place matrix fold")


@pytest.mark.parametrize("case", [(3, 5, 2, 32, 16, "f32"), (2, 6, 3, 64, 48, "bf16"),
                                  (1, 20, 1, 256, 1024, "f16"), (2, 3, 1, 256, 1024, "f32"),
                                  (1, 4, 4, 192, 128, "f16"), (2, 3, 2, 256, 32, "bf16")],
                         ids=lambda c: "B%d_T%d_Hv%d_Dk%d_Dv%d_%s" % c)
def test_replay_ragged_shapes(case):
    B, T, Hv, Dk, Dv, io = case
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=B + T, mask="bernoulli", mask_p=0.6)
    for a in (0, 1, T - 1, T, T + 3):
        _check_replay(gi.poison_untaken(tape, a), a, "ragged")


# ------------------------------------------------------- cross-kernel identities

def _tape_from_record(inp, gqa_map):
    y, s, dl = _record_gpu(inp, gqa_map)
    d = to_dev(inp)
    Hv = inp["v"].shape[2]
    k_log = gdn.gqa_expand(d["k"], Hv, gqa_map)
    return s, dl, k_log, d


@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
def test_full_replay_reproduces_record_fp32_bitwise(gqa_map):
    inp = gi.record_inputs(4, 6, 2, 4, 128, 128, "f32", seed=21, mask="bernoulli")
    s_rec, dl, k_log, d = _tape_from_record(inp, gqa_map)
    note("replay of a recorded fp32 tape, map=%s" % gqa_map)
    s_rep = gdn.gdn_replay(dl, k_log, d["g"], d["state_in"], d["mask"], 6)
    torch.cuda.synchronize()
    assert torch.equal(s_rep, s_rec)


def test_full_replay_reproduces_record_bf16_within_tolerance():
    """With bf16 I/O the tape holds delta rounded to bf16 while the record
    kernel updated its state with the unrounded value."""
    w = gi.WORKLOADS["spec_decode"]
    inp = gi.workload_inputs("spec_decode", 5)
    s_rec, dl, k_log, d = _tape_from_record(inp, w.gqa_map)
    for a in range(w.T + 1):
        note("replay of a recorded bf16 tape, accepted=%d" % a)
        s_rep = gdn.gdn_replay(dl, k_log, d["g"], d["state_in"], d["mask"], a)
        torch.cuda.synchronize()
        if a == w.T:
            assert_close(s_rep, f64(s_rec), torch.bfloat16, "replay vs record")
        # and the prefix replay equals recording only the prefix
        sub = {k2: (v[:, :a] if k2 in ("q", "k", "v", "g", "beta", "mask") else v) for k2, v in inp.items()}
        if a > 0:
            _, s_pre, _ = _record_gpu(sub, w.gqa_map)
            assert_close(s_rep, f64(s_pre), torch.bfloat16, "prefix replay vs prefix record")


@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
def test_head_map_equals_pre_expanded_keys_bitwise(gqa_map):
    inp = gi.record_inputs(2, 4, 4, 8, 64, 64, "bf16", seed=31, mask="trailing")
    y1, s1, d1 = _record_gpu(inp, gqa_map)
    d = to_dev(inp)
    exp = dict(inp)
    exp["q"] = gdn.gqa_expand(d["q"], 8, gqa_map).cpu()
    exp["k"] = gdn.gqa_expand(d["k"], 8, gqa_map).cpu()
    y2, s2, d2 = _record_gpu(exp, "block")
    assert torch.equal(y1, y2) and torch.equal(s1, s2) and torch.equal(d1, d2)


def test_chained_single_steps_equal_one_call_bitwise():
    inp = gi.record_inputs(3, 5, 2, 4, 128, 64, "bf16", seed=41, mask="bernoulli")
    y, s, dl = _record_gpu(inp, "block")
    st = inp["state_in"]
    for t in range(5):
        sub = {k2: (v[:, t:t + 1] if k2 in ("q", "k", "v", "g", "beta", "mask") else v)
               for k2, v in inp.items()}
        sub["state_in"] = st
        yt, st, dt = _record_gpu(sub, "block")
        assert torch.equal(yt, y[:, t:t + 1]) and torch.equal(dt, dl[:, t:t + 1])
        st = st.cpu()
    assert torch.equal(st.to(dev()), s)


def _bit_view(t):
    """The raw bit patterns of a device tensor (so that -0 differs from +0)."""
    return t.view({4: torch.int32, 2: torch.int16}[t.element_size()])


# P-h on the HIP path: accepting a positions equals taking the whole tape with
# the mask cleared from position a on.  Both calls run the same path (the VALU
# fold below 16 positions and for float32 tapes, the matrix-core fold from 16
# positions of a 16-bit tape), so the bits agree.
@pytest.mark.parametrize("case", [(3, 6, 4, 128, 64, "f32", (0, 1, 4, 6)),
                                  (4, 12, 4, 128, 128, "bf16", (0, 3, 11)),
                                  (4, 64, 4, 128, 128, "f16", (16, 20, 40, 63))],
                         ids=lambda c: "T%d_%s" % (c[1], c[5]))
def test_accepted_equals_masking_the_tail_bitwise(case):
    B, T, Hv, Dk, Dv, io, accepted = case
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=61 + T, mask="bernoulli")
    d = to_dev(tape)
    for a in accepted:
        note("replay accepted=%d vs tail-masked full tape, T=%d %s" % (a, T, io))
        m2 = d["mask"].clone()
        m2[:, a:] = 0
        s1 = gdn.gdn_replay(d["delta_log"], d["k_log"], d["g_log"], d["state_in"], d["mask"], a)
        s2 = gdn.gdn_replay(d["delta_log"], d["k_log"], d["g_log"], d["state_in"], m2, T)
        torch.cuda.synchronize()
        assert torch.equal(_bit_view(s1), _bit_view(s2)), a


# P-l on the HIP path: batch rows are independent, so permuting them permutes
# every output bit for bit (record with its tape, then the replay of that tape).
def test_batch_permutation_permutes_outputs_bitwise():
    inp = gi.record_inputs(6, 4, 2, 4, 128, 128, "bf16", seed=71, mask="trailing")
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    pinp = {k2: (v[perm] if v is not None else None) for k2, v in inp.items()}
    note("record of permuted batch rows")
    s_a, dl_a, kl_a, d_a = _tape_from_record(inp, "block")
    s_b, dl_b, kl_b, d_b = _tape_from_record(pinp, "block")
    y_a, _, _ = _record_gpu(inp, "block")
    y_b, _, _ = _record_gpu(pinp, "block")
    pd = perm.to(dev())
    assert torch.equal(_bit_view(y_a[pd]), _bit_view(y_b))
    assert torch.equal(_bit_view(dl_a[pd]), _bit_view(dl_b))
    assert torch.equal(_bit_view(s_a[pd]), _bit_view(s_b))
    note("replay of permuted batch rows")
    r_a = gdn.gdn_replay(dl_a, kl_a, d_a["g"], d_a["state_in"], d_a["mask"], 3)
    r_b = gdn.gdn_replay(dl_b, kl_b, d_b["g"], d_b["state_in"], d_b["mask"], 3)
    torch.cuda.synchronize()
    assert torch.equal(_bit_view(r_a[pd]), _bit_view(r_b))


TILINGS = [(8, 256), (4, 256), (2, 256), (1, 256), (1, 64)]


def _record_tiled(inp, gqa_map, tiling):
    d = to_dev(inp)
    io = d["q"].dtype
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=io, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=io, device=dev())
    out = gdn.gdn_record_debug({"tiling": tiling}, d["q"], d["k"], d["v"], d["g"], d["beta"],
                               d["state_in"], d["mask"], gqa_map=gqa_map, y=y, delta_log=dl)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [1, 3, 12, 40])
def test_every_tiling_gives_identical_bits(T):
    """Row tilings (and with them the staged kernel's chunk lengths: one row
    per thread over few heads takes 64-step chunks, more rows per thread 32)
    change no bit of any output; the first tiling's outputs also match the
    oracle."""
    inp = gi.record_inputs(2, T, 2, 4, 128, 128, "bf16", seed=51, mask="bernoulli")
    tape = gi.tape_inputs(2, 3, 4, 128, 128, "bf16", seed=52)
    d = to_dev(tape)
    ref = None
    for til in TILINGS:
        if T > 1 and til[0] * til[1] // 16 > 64:       # the staged record takes at most 64 rows
            continue
        note("tiling %s T=%d" % (til, T))
        out = _record_tiled(inp, "tiled", til)
        rs = gdn.gdn_replay_debug({"tiling": til, "fold": "valu"}, d["delta_log"], d["k_log"],
                                  d["g_log"], d["state_in"], d["mask"], 2)
        torch.cuda.synchronize()
        cur = [t.cpu() for t in out] + [rs.cpu()]
        if ref is None:
            ref = cur
            ry, rs_, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                            inp["state_in"], inp["mask"], gqa_map="tiled")
            assert_close(cur[1], rs_, torch.bfloat16, "tiling %s state" % (til,))
        else:
            assert all(torch.equal(a, b) for a, b in zip(ref, cur)), til


# Records of 2..4 steps of bf16 I/O with Dv a multiple of 64 run their dense
# products on the matrix cores; a forced tiling runs the VALU kernels.
MFMA_RECORD = [
    # B, T, Hk, Hv, Dk, Dv, map, mask
    (8, 4, 16, 32, 128, 128, "block", "trailing"),     # the speculative-decode shape
    (3, 2, 2, 4, 64, 64, "tiled", "bernoulli"),
    (2, 3, 1, 3, 192, 128, "block", "none"),
    (4, 4, 2, 2, 32, 256, "tiled", "ones"),
    (2, 4, 2, 4, 128, 64, "block", "zeros"),
    (1, 2, 4, 8, 64, 192, "tiled", "bernoulli"),
    (5, 3, 3, 6, 128, 128, "tiled", "trailing"),
]


@pytest.mark.parametrize("case", MFMA_RECORD, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s" % c)
def test_short_record_on_matrix_cores(case):
    """Against the oracle (sentinels at inactive steps) and against the VALU
    kernels (a forced tiling) at the bf16 tolerance."""
    B, T, Hk, Hv, Dk, Dv, gqa_map, mask = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, "bf16", seed=171 + T + Dk, mask=mask)
    _check_record(inp, gqa_map, "matrix-core record %s" % (case,))
    note("matrix-core record against the VALU kernels %s" % (case,))
    y0, s0, d0 = _record_gpu(inp, gqa_map)
    y1, s1, d1 = _record_tiled(inp, gqa_map, (1, 64))
    act = np.broadcast_to(step_mask(inp["mask"], B, T)[:, :, None, None], y0.shape)
    assert_close(y0, f64(y1), torch.bfloat16, "y, matrix cores vs VALU", where=act)
    assert_close(d0, f64(d1), torch.bfloat16, "delta, matrix cores vs VALU", where=act)
    assert_close(s0, f64(s1), torch.bfloat16, "state, matrix cores vs VALU")


@pytest.mark.parametrize("T", [2, 4])
def test_short_record_on_matrix_cores_with_extreme_gates_and_betas(T):
    """Gates of exactly 0, 1, 1e-6 and 1.25 and beta of exactly 0 and 1."""
    B, Hk, Hv, Dk, Dv = 3, 2, 4, 128, 64
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, "bf16", seed=181 + T, mask="bernoulli")
    g = inp["g"].float().clone()
    beta = inp["beta"].float().clone()
    g[:, 0, 0] = 0.0
    g[:, 1, 1] = 1.0
    g[:, T - 1, 2] = 1e-6
    g[:, 1:, 3] = 1.25
    beta[:, 0, 1] = 0.0
    beta[:, T - 1, 0] = 1.0
    inp["g"] = g.to(torch.bfloat16)
    inp["beta"] = beta.to(torch.bfloat16)
    _check_record(inp, "block", "matrix-core record, extreme gates T=%d" % T)


def test_launch_choice_none_is_the_plain_call():
    """gdn_record_debug / gdn_replay_debug with nothing forced give the plain
    calls' bits."""
    inp = gi.record_inputs(2, 5, 2, 4, 128, 128, "bf16", seed=53, mask="bernoulli")
    tape = gi.tape_inputs(2, 20, 4, 128, 128, "f16", seed=54)
    d, t = to_dev(inp), to_dev(tape)
    note("launch choice {} against the plain calls")
    # masked positions of y and delta_log are never written: start both from sentinels
    outs = [dict(y=torch.full(d["v"].shape, Y_SENTINEL, dtype=d["v"].dtype, device=dev()),
                 delta_log=torch.full(d["v"].shape, D_SENTINEL, dtype=d["v"].dtype, device=dev()))
            for _ in range(2)]
    a = gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"], **outs[0])
    b = gdn.gdn_record_debug({}, d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                             **outs[1])
    r1 = gdn.gdn_replay(t["delta_log"], t["k_log"], t["g_log"], t["state_in"], t["mask"], 18)
    r2 = gdn.gdn_replay_debug(None, t["delta_log"], t["k_log"], t["g_log"], t["state_in"], t["mask"], 18)
    torch.cuda.synchronize()
    assert all(torch.equal(_bit_view(x), _bit_view(z)) for x, z in zip(a, b))
    assert torch.equal(_bit_view(r1), _bit_view(r2))


def test_in_place_state_and_tapeless_step():
    inp = gi.record_inputs(2, 4, 2, 4, 128, 128, "bf16", seed=61, mask="trailing")
    y, s, dl = _record_gpu(inp, "block")
    d = to_dev(inp)
    st = d["state_in"].clone()
    note("record in place, no tape")
    y2, s2, dl2 = gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["mask"],
                                 state_out=st, y=torch.full_like(y, Y_SENTINEL), write_tape=False)
    torch.cuda.synchronize()
    assert dl2 is None and s2.data_ptr() == st.data_ptr()
    assert torch.equal(s2, s) and torch.equal(y2, y)
    tape = to_dev(gi.tape_inputs(2, 4, 4, 128, 128, "bf16", seed=62))
    ref = gdn.gdn_replay(tape["delta_log"], tape["k_log"], tape["g_log"], tape["state_in"], tape["mask"], 3)
    st = tape["state_in"].clone()
    gdn.gdn_replay(tape["delta_log"], tape["k_log"], tape["g_log"], st, tape["mask"], 3, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(st, ref)


def test_repeated_runs_are_bitwise_identical():
    inp = gi.workload_inputs("spec_decode", 7)
    a = _record_gpu(inp, "block")
    b = _record_gpu(inp, "block")
    assert all(torch.equal(x, z) for x, z in zip(a, b))


# ---------------------------------------------------------------- tape capture

K_SENTINEL = 5.5        # exact in every I/O dtype
G_SENTINEL = -0.625


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a tensor as a numpy integer array."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16).numpy()


def _record_capture(inp, gqa_map, want_k=True, want_g=True, tiling=None):
    d = to_dev(inp)
    B, T, Hk, Dk = d["k"].shape
    Hv = d["v"].shape[2]
    io = d["q"].dtype
    y = torch.full(d["v"].shape, Y_SENTINEL, dtype=io, device=dev())
    dl = torch.full(d["v"].shape, D_SENTINEL, dtype=io, device=dev())
    kl = torch.full((B, T, Hv, Dk), K_SENTINEL, dtype=io, device=dev()) if want_k else None
    gl = torch.full((B, T, Hv), G_SENTINEL, dtype=io, device=dev()) if want_g else None
    y, s, dl = gdn.gdn_record_debug({"tiling": tiling} if tiling else None, d["q"], d["k"], d["v"],
                                    d["g"], d["beta"], d["state_in"], d["mask"], gqa_map=gqa_map,
                                    y=y, delta_log=dl, k_log=kl, g_log=gl)
    torch.cuda.synchronize()
    return y, s, dl, kl, gl


CAPTURE = [
    # B, T, Hk, Hv, Dk, Dv, io, map, mask
    (4, 1, 2, 4, 128, 128, "bf16", "block", "bernoulli"),     # single step
    (3, 1, 3, 6, 64, 48, "f32", "tiled", "none"),
    (2, 3, 2, 4, 128, 128, "bf16", "tiled", "bernoulli"),     # short tape
    (2, 5, 1, 3, 256, 64, "f16", "block", "none"),
    (2, 37, 2, 4, 128, 64, "bf16", "block", "trailing"),      # several chunks, ragged last one
    (1, 20, 3, 3, 192, 32, "f32", "tiled", "bernoulli"),
    (2, 9, 4, 8, 32, 16, "bf16", "tiled", "none"),
    (2, 4, 2, 4, 64, 64, "bf16", "block", "zeros"),
]


@pytest.mark.parametrize("case", CAPTURE, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s" % c)
def test_record_captures_expanded_keys_and_gates(case):
    B, T, Hk, Hv, Dk, Dv, io, gqa_map, mask = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io, seed=81 + T, mask=mask)
    note("record with capture %s" % (case,))
    y, s, dl, kl, gl = _record_capture(inp, gqa_map)
    # capturing changes none of the other outputs
    y0, s0, dl0 = _record_gpu(inp, gqa_map)
    assert torch.equal(y, y0) and torch.equal(s, s0) and torch.equal(dl, dl0)
    act = step_mask(inp["mask"], B, T)
    ref_k = oracle.gqa_expand(_bits(inp["k"]).reshape(B * T, Hk, Dk), Hv, gqa_map)
    got_k = _bits(kl).reshape(B * T, Hv, Dk)
    a = act.reshape(B * T)
    assert np.array_equal(got_k[a], ref_k[a]), "k_log differs from the expanded keys"
    assert np.all(f64(kl).reshape(B * T, Hv, Dk)[~a] == K_SENTINEL), "k_log written at an inactive step"
    got_g, ref_g = _bits(gl), _bits(inp["g"])
    assert np.array_equal(got_g[act], ref_g[act]), "g_log differs from g"
    assert np.all(f64(gl)[~act] == G_SENTINEL), "g_log written at an inactive step"
    # the captured tape replays exactly like one expanded by a separate pass
    d = to_dev(inp)
    k_exp = gdn.gqa_expand(d["k"], Hv, gqa_map)
    for acc in sorted({0, 1, T}):
        note("replay of a captured tape, accepted=%d" % acc)
        r1 = gdn.gdn_replay(dl, kl, gl, d["state_in"], d["mask"], acc)
        r2 = gdn.gdn_replay(dl, k_exp, d["g"], d["state_in"], d["mask"], acc)
        torch.cuda.synchronize()
        assert torch.equal(r1, r2), acc
    if io == "f32" and T < 16:   # longer folds keep a running scale: equal within rounding only
        assert torch.equal(r1, s), "fp32 replay of the whole captured tape differs from the record"


@pytest.mark.parametrize("want_k,want_g", [(True, False), (False, True)])
def test_record_captures_one_log_alone(want_k, want_g):
    inp = gi.record_inputs(2, 6, 2, 4, 128, 64, "bf16", seed=91, mask="bernoulli")
    note("record capturing k_log=%s g_log=%s" % (want_k, want_g))
    y, s, dl, kl, gl = _record_capture(inp, "tiled", want_k, want_g)
    ref = _record_capture(inp, "tiled")
    assert torch.equal(y, ref[0]) and torch.equal(s, ref[1]) and torch.equal(dl, ref[2])
    if want_k:
        assert gl is None and torch.equal(kl, ref[3])
    else:
        assert kl is None and torch.equal(gl, ref[4])


@pytest.mark.parametrize("T", [1, 11])
def test_capture_identical_under_every_tiling(T):
    inp = gi.record_inputs(2, T, 2, 4, 128, 128, "bf16", seed=93, mask="bernoulli")
    ref = None
    for til in TILINGS:
        if T > 1 and til[0] * til[1] // 16 > 64:
            continue
        note("capture under tiling %s T=%d" % (til, T))
        cur = [t.cpu() for t in _record_capture(inp, "block", tiling=til)]
        if ref is None:
            ref = cur
        else:
            assert all(torch.equal(a, b) for a, b in zip(ref, cur)), til


# ---------------------------------------------------------------- gqa_expand

EXPAND = [
    # seq, hg, h, k, dtype, map
    (1, 1, 1, 1, "f32", "tiled"),
    (5, 2, 4, 33, "f16", "block"),
    (7, 3, 12, 64, "bf16", "tiled"),
    (9, 4, 8, 7, "f32", "block"),
    (32, 16, 32, 128, "bf16", "block"),
    (4096, 16, 32, 128, "f32", "tiled"),      # chunk-prefill q/k expansion
    # divisors that are not powers of two in both index decompositions
    (37, 5, 15, 200, "f32", "tiled"),         # 50 vectors per row, hg = 5
    (101, 7, 21, 96, "bf16", "block"),        # 12 vectors per row, hg = 7
    (33, 12, 48, 40, "f16", "tiled"),         # 5 vectors per row, hg = 12
    (3, 48, 96, 24, "bf16", "block"),         # 3 vectors per row, hg = 48
]


@pytest.mark.parametrize("case", EXPAND, ids=lambda c: "%d_%d_%d_%d_%s_%s" % c)
def test_gqa_expand_bit_exact(case):
    seq, hg, h, kk, io, m = case
    src = gi.expand_source(seq, hg, kk, io, seed=seq + kk)
    raw = src.view(torch.int16 if src.element_size() == 2 else torch.int32)
    raw.view(-1)[:: 97] = -1                 # plant NaN bit patterns: the copy must keep them
    note("gqa_expand %s" % (case,))
    out = gdn.gqa_expand(src.to(dev()), h, m)
    torch.cuda.synchronize()
    want = oracle.gqa_expand(raw.numpy(), h, m)
    got = out.cpu().view(raw.dtype).numpy()
    assert got.tobytes() == want.tobytes()


def test_gqa_expand_unaligned_views_and_batch_dims():
    src = gi.expand_source(3 * 5 + 1, 2, 24, "bf16", seed=5)
    d = src.to(dev())
    view = d[1:].view(3, 5, 2, 24)                 # base 96 bytes in: still fine, 2-byte vectors or wider
    odd = torch.empty(3 * 5 * 6 * 24 + 1, dtype=torch.bfloat16, device=dev())[1:].view(3, 5, 6, 24)
    note("gqa_expand unaligned")
    out = gdn.gqa_expand(view, 6, "block", dst=odd)
    torch.cuda.synchronize()
    want = oracle.gqa_expand(src[1:].view(torch.int16).numpy().reshape(15, 2, 24), 6, "block")
    assert out.cpu().view(torch.int16).numpy().reshape(15, 6, 24).tobytes() == want.tobytes()


def test_gqa_expand_past_32_bit_indices():
    """More than 2^32 source vectors (2-byte elements at a 2-byte offset, so
    one element per vector) take the kernel's 64-bit index path: 8.8 GB
    expanded into 17.6 GB on the device, with rows sampled around the 2^32
    vector boundary, at both ends and at random checked against the oracle's
    expansion of the same rows."""
    seq, hg, h, kk = 22_000_000, 2, 4, 100                   # 4.4e9 source elements
    assert seq * hg * kk > 2 ** 32
    note("gqa_expand with 64-bit indices: %d x %d x %d bf16 -> %d heads" % (seq, hg, kk, h))
    raw = torch.empty(seq * hg * kk + 1, dtype=torch.int16, device=dev())
    raw.random_(-32768, 32767, generator=torch.Generator(device=dev()).manual_seed(7))
    src = raw[1:].view(torch.bfloat16).view(seq, hg, kk)      # 2-byte offset: 2-byte vectors
    out = gdn.gqa_expand(src, h, "block")
    torch.cuda.synchronize()
    boundary = (2 ** 32) // (hg * kk)                         # the seq row holding vector 2^32
    rows = sorted({0, 1, seq - 1, boundary - 1, boundary, boundary + 1} |
                  set(np.random.Generator(np.random.PCG64(3)).integers(0, seq, size=12).tolist()))
    assert max(rows) < seq
    idx = torch.tensor(rows, device=dev())
    got = out.index_select(0, idx).view(torch.int16).cpu().numpy()
    want = oracle.gqa_expand(src.index_select(0, idx).view(torch.int16).cpu().numpy(), h, "block")
    assert got.tobytes() == want.tobytes()
    del out, raw, src
    torch.cuda.empty_cache()


def test_tolerances_are_the_stated_ones():
    assert TOL[torch.float32] == 1e-3 and TOL[torch.bfloat16] == 2e-2 and TOL[torch.float16] == 2e-2


# ------------------------------------------------------------------ HIP graphs

def test_graph_captured_step_replays_match_eager_bitwise():
    """record (with tape capture) + replay + RMSNorm captured once in a HIP
    graph and replayed with fresh inputs copied into the captured buffers, with
    eager work and synchronisations between replays: every replay equals the
    eager calls bit for bit."""
    w = gi.WORKLOADS["spec_decode"]
    d = to_dev(gi.workload_inputs("spec_decode", 0))
    io = d["q"].dtype
    B, T, Hk, Dk = d["k"].shape
    Hv, Dv = w.Hv, w.Dv
    y = torch.empty(d["v"].shape, dtype=io, device=dev())
    dl = torch.empty_like(y)
    kl = torch.empty((B, T, Hv, Dk), dtype=io, device=dev())
    gl = torch.empty((B, T, Hv), dtype=io, device=dev())
    s1 = torch.empty_like(d["state_in"])
    s2 = torch.empty_like(d["state_in"])
    xn, wn = (t.to(dev()) for t in gi.norm_inputs(64, 2048, seed=1))
    on = torch.empty_like(xn)

    def step():
        gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"], d["mask"],
                       gqa_map=w.gqa_map, y=y, state_out=s1, delta_log=dl, k_log=kl, g_log=gl)
        gdn.gdn_replay(dl, kl, gl, d["state_in"], d["mask"], 3, state_out=s2)
        gdn.rms_norm_bf16(xn, wn, 1e-6, out=on)

    note("graph capture of record + replay + rms_norm")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                                # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = to_dev(gi.workload_inputs("spec_decode", 10 + rep))
        for name in ("q", "k", "v", "g", "beta", "state_in", "mask"):
            d[name].copy_(fresh[name])
        xn.copy_(gi.norm_inputs(64, 2048, seed=20 + rep)[0].to(dev()))
        note("graph replay %d" % rep)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y, dl, kl, gl, s1, s2, on)]
        step()                                                # eager, same buffers
        torch.cuda.synchronize()
        # inactive positions are written by neither run, so whole tensors compare,
        # as bit patterns (never-written memory may hold NaNs)
        for i, (a, b) in enumerate(zip(got, (y, dl, kl, gl, s1, s2, on))):
            bits = torch.int32 if a.element_size() == 4 else torch.int16
            assert torch.equal(a.view(bits), b.view(bits)), (rep, i)


# ------------------------------------------------------- seeded shape sweep

def _sweep_cases(n=48, seed=2026):
    """A fixed, seeded list of mixed configurations: every supported Dk, value
    widths that are and are not multiples of the row blocks, GQA ratios,
    tapes that are short, medium and long (every staged chunk length, ragged
    last chunks), all I/O dtypes, maps and mask kinds, and replays on either
    fold (VALU, or matrix cores for 16+ positions of a 16-bit tape)."""
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Dk = int(r.choice([32, 64, 128, 192, 256]))
        Dv = int(r.choice([16, 32, 48, 64, 80, 128, 192, 256]))
        Hk = int(r.integers(1, 4))
        Hv = Hk * int(r.integers(1, 4))
        B = int(r.integers(1, 5))
        T = int(r.choice([1, 2, 5, 8, 9, 13, 16, 17, 31, 40, 65, 70]))
        while B * Hv * Dv * Dk * T > 6_000_000 and T > 1:   # keep the oracle to about a second
            T //= 2
        io = str(r.choice(["f32", "f16", "bf16"]))
        gmap = str(r.choice(["block", "tiled"]))
        mask = str(r.choice(["none", "ones", "trailing", "bernoulli", "zeros"]))
        acc = int(r.integers(0, T + 3))
        cases.append((B, T, Hk, Hv, Dk, Dv, io, gmap, mask, acc, seed + i))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(),
                         ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s_a%d_s%d" % c)
def test_seeded_shape_sweep(case):
    B, T, Hk, Hv, Dk, Dv, io, gmap, mask, acc, seed = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io, seed=seed, mask=mask)
    _check_record(inp, gmap, "sweep %s" % (case,))
    tape = gi.tape_inputs(B, T, Hv, Dk, Dv, io, seed=seed + 1,
                          mask=mask if mask != "none" else "bernoulli")
    _check_replay(gi.poison_untaken(tape, acc), acc, "sweep %s" % (case,))


# ------------------------------------------------------- record edge values

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 12, 40, 70])
def test_record_with_extreme_gates_and_betas(io, T):
    """Gates of exactly 0 (the state resets to the step's rank-1 write), 1
    (no decay), tiny and above 1, and beta of exactly 0 and 1, on every path
    (direct, short, 16-, 32- and 64-step chunks), against the oracle."""
    B, Hk, Hv, Dk, Dv = 2, 2, 4, 64, 32
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io, seed=81 + T, mask="bernoulli")
    g = inp["g"].float().clone()
    beta = inp["beta"].float().clone()
    g[:, 0::7] = 0.0
    g[:, 1::5, 0] = 1.0
    g[:, 2::9, 1] = 1e-6
    g[:, 3::4, 2] = 1.25
    beta[:, 1::3] = 0.0
    beta[:, 2::6] = 1.0
    inp["g"] = g.to(inp["g"].dtype)
    inp["beta"] = beta.to(inp["beta"].dtype)
    _check_record(inp, "tiled", "extreme gates/betas T=%d %s" % (T, io))


@pytest.mark.parametrize("T", [3, 12, 40])
def test_record_ignores_nan_inputs_at_inactive_steps(T):
    """q, k, v, g and beta are NaN at every inactive step: those steps are
    skipped, so nothing non-finite reaches y, delta or the state."""
    inp = gi.record_inputs(3, T, 2, 4, 128, 64, "bf16", seed=91 + T, mask="bernoulli")
    off = ~(inp["mask"] > 0)
    for name in ("q", "k", "v", "g", "beta"):
        t = inp[name].clone()
        t[off] = float("nan")
        inp[name] = t
    _check_record(inp, "block", "NaN at inactive steps T=%d" % T)
    _, s, _ = _record_gpu(inp, "block")
    assert torch.isfinite(s).all()
