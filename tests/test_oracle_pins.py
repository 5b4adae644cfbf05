"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes part of what the record / replay / expand operations compute,
from hand-worked cases (tests/golden/, each with its source), closed forms of
the recurrence, an independent formulation (the transition-matrix form of the
gated delta rule), library routines (numpy repeat / tile) and identities
between record and replay.  tests/test_oracle_mutants.py checks that planted
mistakes in the oracle's C source make at least one of these fail.

Source of the method: metaltile-std 0.1.0, src/ffai/gated_delta_replay.rs
(record kernel ``gated_delta_record!``, replay kernel ``state_replay!``) and
mlx-native 0.6.5, mlx_native/ops/repeat_tiled.rs ("Mapping").
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_case(seed, B=2, T=5, Hk=2, Hv=4, Dk=3, Dv=2, masked=True, unit_k=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, Hk, Dk))
    k = r.standard_normal((B, T, Hk, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, Hv, Dv))
    g = r.uniform(0.05, 0.95, (B, T, Hv))
    beta = r.uniform(0.05, 0.95, (B, T, Hv))
    s0 = 0.5 * r.standard_normal((B, Hv, Dv, Dk))
    mask = (r.random((B, T)) < 0.7).astype(np.uint32) if masked else None
    if mask is not None:
        mask[:, 0] = 1
        mask[0, -1] = 0
        mask = mask * r.integers(1, 5, size=mask.shape).astype(np.uint32)  # any value > 0 passes
    return q, k, v, g, beta, s0, mask


def _head_table(Hk, Hv, gqa_map):
    """Key head per value head, from library routines: np.repeat is the block
    layout (consecutive value heads share a key head), np.tile the tiled one."""
    if gqa_map == "block":
        return np.repeat(np.arange(Hk), Hv // Hk)
    return np.tile(np.arange(Hk), Hv // Hk)


def _transition_form(q, k, v, g, beta, s0, mask, gqa_map):
    """Gated delta rule in transition-matrix form:
    S_t = S_{t-1} @ (g_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T,
    delta_t = beta_t (v_t - g_t S_{t-1} k_t), y_t = S_t q_t."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2:]
    table = _head_table(Hk, Hv, gqa_map)
    y = np.full(v.shape, np.nan)
    d = np.full(v.shape, np.nan)
    S = s0.copy()
    eye = np.eye(Dk)
    for b in range(B):
        for h in range(Hv):
            hk = table[h]
            for t in range(T):
                if mask is not None and mask[b, t] == 0:
                    continue
                kt = k[b, t, hk][:, None]
                A = g[b, t, h] * (eye - beta[b, t, h] * (kt @ kt.T))
                d[b, t, h] = beta[b, t, h] * (v[b, t, h] - g[b, t, h] * (S[b, h] @ kt)[:, 0])
                S[b, h] = S[b, h] @ A + beta[b, t, h] * np.outer(v[b, t, h], kt[:, 0])
                y[b, t, h] = S[b, h] @ q[b, t, hk]
    return y, S, d


def _replay_closed_form(d, kl, gl, s0, mask, accepted):
    """S_a = (prod of taken g) S0 + sum over taken t of (prod of taken g after t) delta_t k_t^T."""
    B, T, Hv, Dv = d.shape
    out = np.empty_like(s0)
    for b in range(B):
        taken = [t for t in range(min(accepted, T)) if mask is None or mask[b, t] > 0]
        for h in range(Hv):
            gs = np.array([gl[b, t, h] for t in taken])
            acc = np.prod(gs) * s0[b, h] if len(gs) else s0[b, h].copy()
            for i, t in enumerate(taken):
                acc = acc + np.prod(gs[i + 1:]) * np.outer(d[b, t, h], kl[b, t, h])
            out[b, h] = acc
    return out


def _expand_heads(x, Hv, gqa_map):
    """[B,T,Hk,D] -> [B,T,Hv,D] with numpy's repeat / tile."""
    Hk = x.shape[2]
    if gqa_map == "block":
        return np.repeat(x, Hv // Hk, axis=2)
    return np.tile(x, (1, 1, Hv // Hk, 1))


# ---------------------------------------------------------------- hand cases

def test_hand_single_step():
    c = _gold("hand_t1.json")
    s0 = np.array(c["S0"]).reshape(1, 1, 2, 2)
    q = np.array(c["q"]).reshape(1, 1, 1, 2)
    k = np.array(c["k"]).reshape(1, 1, 1, 2)
    v = np.array(c["v"]).reshape(1, 1, 1, 2)
    g = np.full((1, 1, 1), c["g"])
    beta = np.full((1, 1, 1), c["beta"])
    y, s1, d = oracle.gdn_record(q, k, v, g, beta, s0)
    assert np.array_equal(d.ravel(), c["expect"]["delta"])
    assert np.array_equal(s1[0, 0], np.array(c["expect"]["S1"]))
    assert np.array_equal(y.ravel(), c["expect"]["y"])
    s_rep = oracle.gdn_replay(d, k, g, s0, accepted=1)
    assert np.array_equal(s_rep, s1)


def test_hand_masked_three_steps():
    c = _gold("hand_t3_mask.json")
    T = c["T"]
    s0 = np.array(c["S0"]).reshape(1, 1, 2, 2)
    q = np.array(c["q"]).reshape(1, T, 1, 2)
    k = np.array(c["k"]).reshape(1, T, 1, 2)
    v = np.array(c["v"]).reshape(1, T, 1, 2)
    g = np.array(c["g"]).reshape(1, T, 1)
    beta = np.array(c["beta"]).reshape(1, T, 1)
    mask = np.array(c["mask"], dtype=np.uint32).reshape(1, T)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask)
    e = c["expect"]
    for t in range(T):
        if e["y"][t] is None:
            assert np.isnan(y[0, t]).all() and np.isnan(d[0, t]).all()
        else:
            assert np.array_equal(y[0, t, 0], e["y"][t])
            assert np.array_equal(d[0, t, 0], e["delta"][t])
    assert np.array_equal(s[0, 0], np.array(e["S_final"]))
    for a, want in e["replay"].items():
        got = oracle.gdn_replay(d, k, g, s0, mask, accepted=int(a))
        assert np.array_equal(got[0, 0], np.array(want)), a


def test_hand_gqa_maps_in_record():
    c = _gold("gqa_heads.json")
    rc = c["record_case"]
    Hk, Hv = c["Hk"], c["Hv"]
    q = np.array(rc["q"]).reshape(1, 1, Hk, 1)
    k = np.ones((1, 1, Hk, 1))
    v = np.ones((1, 1, Hv, 1))
    g = np.ones((1, 1, Hv))
    beta = np.ones((1, 1, Hv))
    s0 = np.ones((1, Hv, 1, 1))
    for m in ("block", "tiled"):
        y, s1, d = oracle.gdn_record(q, k, v, g, beta, s0, gqa_map=m)
        assert np.array_equal(y.ravel(), rc["y_" + m])
        assert np.array_equal(s1, s0)
        assert np.array_equal(d.ravel(), np.zeros(Hv))


# ------------------------------------------------------------ GQA expansion

def test_gqa_expand_brute_force_tiny():
    c = _gold("gqa_heads.json")
    Hk, Hv = c["Hk"], c["Hv"]
    src = np.arange(Hk, dtype=np.float32).reshape(1, Hk, 1)
    for m in ("block", "tiled"):
        out = oracle.gqa_expand(src, Hv, m)
        assert out.ravel().tolist() == c[m]


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.float64, np.uint8])
@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (3, 2, 4, 5), (7, 4, 12, 33), (2, 16, 32, 128)])
def test_gqa_expand_matches_numpy(dtype, gqa_map, shape):
    seq, hg, h, kk = shape
    r = np.random.default_rng(seq * 1000 + hg)
    raw = r.integers(0, 256, size=seq * hg * kk * np.dtype(dtype).itemsize, dtype=np.uint8)
    src = raw.view(dtype).reshape(seq, hg, kk)       # arbitrary bit patterns, NaNs included
    out = oracle.gqa_expand(src, h, gqa_map)
    want = np.repeat(src, h // hg, axis=1) if gqa_map == "block" else np.tile(src, (1, h // hg, 1))
    assert out.tobytes() == want.tobytes()


def test_gqa_expand_rejects_bad_ratio():
    with pytest.raises(ValueError):
        oracle.gqa_expand(np.zeros((1, 3, 4), np.float32), 4, "tiled")


# ------------------------------------------------- independent formulation

@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_record_matches_transition_form(gqa_map, seed):
    case = _rand_case(seed)
    y, s, d = oracle.gdn_record(*case, gqa_map=gqa_map)
    y2, s2, d2 = _transition_form(*case, gqa_map)
    np.testing.assert_array_equal(np.isnan(y), np.isnan(y2))
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d, d2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, s2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_replay_matches_closed_form(seed):
    r = np.random.default_rng(100 + seed)
    B, T, Hv, Dk, Dv = 3, 6, 2, 4, 3
    d = r.standard_normal((B, T, Hv, Dv))
    kl = r.standard_normal((B, T, Hv, Dk))
    gl = r.uniform(0.1, 0.9, (B, T, Hv))
    s0 = r.standard_normal((B, Hv, Dv, Dk))
    mask = (r.random((B, T)) < 0.6).astype(np.uint32)
    for a in (0, 1, 3, T, T + 5):
        got = oracle.gdn_replay(d, kl, gl, s0, mask, accepted=a)
        want = _replay_closed_form(d, kl, gl, s0, mask, a)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- closed forms

def test_identity_gate_zero_beta_keeps_state():
    q, k, v, g, beta, s0, mask = _rand_case(3, masked=False)
    g[:] = 1.0
    beta[:] = 0.0
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0)
    assert np.array_equal(s, s0)
    assert np.all(d == 0.0)
    table = _head_table(q.shape[2], v.shape[2], "block")
    want = np.einsum("bhvk,bthk->bthv", s0, q[:, :, table])
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)


def test_zero_beta_is_pure_decay():
    q, k, v, g, beta, s0, mask = _rand_case(4)
    beta[:] = 0.0
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask)
    B, T = mask.shape
    table = _head_table(q.shape[2], v.shape[2], "block")
    for b in range(B):
        for h in range(v.shape[2]):
            scale = 1.0
            for t in range(T):
                if mask[b, t] == 0:
                    continue
                scale *= g[b, t, h]
                np.testing.assert_allclose(y[b, t, h], scale * s0[b, h] @ q[b, t, table[h]],
                                           rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(s[b, h], scale * s0[b, h], rtol=1e-12, atol=1e-14)


def test_unit_beta_unit_key_writes_value():
    q, k, v, g, beta, s0, _ = _rand_case(5, T=1, Dk=6, Dv=4, masked=False, unit_k=True)
    beta[:] = 1.0
    q = k.copy()                                  # read back with the written key
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0)
    table = _head_table(q.shape[2], v.shape[2], "block")
    for b in range(v.shape[0]):
        for h in range(v.shape[2]):
            np.testing.assert_allclose(s[b, h] @ k[b, 0, table[h]], v[b, 0, h], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, v, rtol=1e-12, atol=1e-12)


def test_one_hot_keys_overwrite_columns():
    B, T, Hk, Hv, Dk, Dv = 1, 4, 1, 1, 6, 3
    r = np.random.default_rng(6)
    cols = [4, 1, 5, 0]
    k = np.zeros((B, T, Hk, Dk))
    for t, c in enumerate(cols):
        k[0, t, 0, c] = 1.0
    q = r.standard_normal((B, T, Hk, Dk))
    v = r.standard_normal((B, T, Hv, Dv))
    g = np.ones((B, T, Hv))
    beta = np.ones((B, T, Hv))
    s0 = np.zeros((B, Hv, Dv, Dk))
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0)
    want = np.zeros((Dv, Dk))
    for t, c in enumerate(cols):
        want[:, c] = v[0, t, 0]
    assert np.array_equal(s[0, 0], want)


def test_accepted_zero_and_all_masked_are_no_ops():
    q, k, v, g, beta, s0, mask = _rand_case(7)
    zero = np.zeros_like(mask)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, zero, y_init=np.full(v.shape, 7.0),
                                delta_init=np.full(v.shape, -3.0))
    assert np.array_equal(s, s0)
    assert np.all(y == 7.0) and np.all(d == -3.0)
    kl = _expand_heads(k, v.shape[2], "block")
    dd = np.random.default_rng(8).standard_normal(v.shape)
    assert np.array_equal(oracle.gdn_replay(dd, kl, g, s0, mask, accepted=0), s0)
    assert np.array_equal(oracle.gdn_replay(dd, kl, g, s0, zero, accepted=5), s0)


# ------------------------------------------------------------------- identities

@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
@pytest.mark.parametrize("masked", [False, True])
def test_full_replay_reproduces_record(gqa_map, masked):
    q, k, v, g, beta, s0, mask = _rand_case(9, masked=masked)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask, gqa_map=gqa_map)
    B, T, Hk, Dk = k.shape
    k_log = oracle.gqa_expand(k.reshape(B * T, Hk, Dk), v.shape[2], gqa_map).reshape(B, T, -1, Dk)
    rep = oracle.gdn_replay(d, k_log, g, s0, mask, accepted=T)   # masked slots hold NaN
    assert np.array_equal(rep, s)       # same products and sums in the same order


def test_accepted_equals_masking_the_tail():
    r = np.random.default_rng(10)
    B, T, Hv, Dk, Dv = 2, 7, 3, 4, 5
    d = r.standard_normal((B, T, Hv, Dv))
    kl = r.standard_normal((B, T, Hv, Dk))
    gl = r.uniform(0.1, 0.9, (B, T, Hv))
    s0 = r.standard_normal((B, Hv, Dv, Dk))
    mask = (r.random((B, T)) < 0.6).astype(np.uint32)
    for a in range(T + 2):
        tail = mask * (np.arange(T)[None, :] < a)
        assert np.array_equal(oracle.gdn_replay(d, kl, gl, s0, mask, accepted=a),
                              oracle.gdn_replay(d, kl, gl, s0, tail.astype(np.uint32), accepted=T))


def test_chained_single_steps_equal_one_call():
    q, k, v, g, beta, s0, mask = _rand_case(11)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask)
    st = s0
    T = q.shape[1]
    for t in range(T):
        sl = slice(t, t + 1)
        yt, st, dt = oracle.gdn_record(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], st,
                                       mask[:, sl])
        np.testing.assert_array_equal(yt, y[:, sl])
        np.testing.assert_array_equal(dt, d[:, sl])
    assert np.array_equal(st, s)


@pytest.mark.parametrize("gqa_map", ["block", "tiled"])
def test_head_map_equals_pre_expanded_keys(gqa_map):
    q, k, v, g, beta, s0, mask = _rand_case(12, Hk=2, Hv=6)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask, gqa_map=gqa_map)
    Hv = v.shape[2]
    y2, s2, d2 = oracle.gdn_record(_expand_heads(q, Hv, gqa_map), _expand_heads(k, Hv, gqa_map),
                                   v, g, beta, s0, mask, gqa_map="block")
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(d, d2)
    assert np.array_equal(s, s2)


def test_batch_rows_are_independent():
    q, k, v, g, beta, s0, mask = _rand_case(13, B=4)
    perm = np.array([2, 0, 3, 1])
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask)
    y2, s2, d2 = oracle.gdn_record(q[perm], k[perm], v[perm], g[perm], beta[perm], s0[perm], mask[perm])
    np.testing.assert_array_equal(y[perm], y2)
    np.testing.assert_array_equal(d[perm], d2)
    assert np.array_equal(s[perm], s2)


def test_tapeless_step_matches_taped_step():
    q, k, v, g, beta, s0, mask = _rand_case(14)
    y, s, d = oracle.gdn_record(q, k, v, g, beta, s0, mask, want_delta=False)
    assert d is None
    y2, s2, _ = oracle.gdn_record(q, k, v, g, beta, s0, mask)
    np.testing.assert_array_equal(y, y2)
    assert np.array_equal(s, s2)


# --------------------------------------------------------------- RMSNorm (bf16 weight)

def _bf16_bits(a):
    """bf16 bit patterns of float values that bf16 holds exactly."""
    import torch
    t = torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(np.asarray(a, dtype=np.float32))), "not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def test_rms_norm_hand_case():
    g = json.load(open(os.path.join(GOLD, "rms_norm_hand.json")))
    out = oracle.rms_norm_bf16(np.array(g["x"], dtype=np.float32), _bf16_bits(g["weight"]), g["eps"])
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=1e-15, atol=0)


def test_rms_norm_constant_row_closed_form():
    r = np.random.Generator(np.random.PCG64(301))
    dim = 96
    w = np.round(r.normal(1.0, 0.25, dim) * 64) / 64          # exact in bf16
    for c, eps in ((0.75, 1e-6), (-3.0, 0.5), (1e-3, 1e-5)):
        x = np.full((2, dim), c, dtype=np.float32)
        out = oracle.rms_norm_bf16(x, _bf16_bits(w), eps)
        cx = float(np.float32(c))
        ref = cx / np.sqrt(cx * cx + eps) * w
        np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=0)
        np.testing.assert_array_equal(out[0], out[1])


def test_rms_norm_one_hot_and_unit_rms():
    dim = 40
    w = np.ones(dim)
    x = np.zeros((1, dim), dtype=np.float32)
    x[0, 7] = -2.5
    out = oracle.rms_norm_bf16(x, _bf16_bits(w), 0.0)
    ref = np.zeros(dim)
    ref[7] = -np.sqrt(dim)
    np.testing.assert_allclose(out[0], ref, rtol=1e-14, atol=0)
    r = np.random.Generator(np.random.PCG64(302))
    x = r.standard_normal((5, dim)).astype(np.float32)
    out = oracle.rms_norm_bf16(x, _bf16_bits(w), 0.0)
    np.testing.assert_allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-13)


def test_rms_norm_scale_invariance_and_weight_per_column():
    r = np.random.Generator(np.random.PCG64(303))
    dim = 64
    w = np.round(r.normal(1.0, 0.5, dim) * 32) / 32
    wb = _bf16_bits(w)
    x = r.standard_normal((3, dim)).astype(np.float32)
    base = oracle.rms_norm_bf16(x, wb, 0.0)
    np.testing.assert_allclose(oracle.rms_norm_bf16(x * np.float32(4.0), wb, 0.0), base, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm_bf16(-x, wb, 0.0), -base, rtol=1e-13)
    # out / (x * w) is the same 1/rms for every column of a row, and equals it
    ratio = base / (x.astype(np.float64) * w)
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1, keepdims=True))
    np.testing.assert_allclose(ratio, np.broadcast_to(1.0 / rms, ratio.shape), rtol=1e-12)


def test_rms_norm_rows_are_independent():
    r = np.random.Generator(np.random.PCG64(304))
    x = r.standard_normal((6, 33)).astype(np.float32)
    wb = _bf16_bits(np.round(r.normal(1.0, 0.2, 33) * 16) / 16)
    out = oracle.rms_norm_bf16(x, wb, 1e-6)
    perm = r.permutation(6)
    np.testing.assert_array_equal(oracle.rms_norm_bf16(x[perm], wb, 1e-6), out[perm])
