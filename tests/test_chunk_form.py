"""The chunk form of the record step, checked on the CPU against the oracle.

gdn_prefill (64 steps per chunk) and the matrix-core record of short tapes
(the whole tape of 2-4 steps as one chunk) compute the record kernel's outputs
from an unrolled form of its recurrence, derived from the record kernel
(``gated_delta_record!``) of the metaltile-std 0.1.0 page
``src/ffai/gated_delta_replay.rs`` alone.  Over a chunk of C steps that
starts from state S0, with inactive steps taken as identity steps (g = 1,
beta = 0, k = q = v = 0) and

    gamma_t = g_0 ... g_t,  M[t,s] = g_{s+1} ... g_t (s <= t, else 0),
    G = K K^T,  H = Q K^T,  A[t,s] = beta_t M[t,s] G[t,s] (s < t),

the innovations are Delta = (I + A)^-1 diag(beta) (V - gamma o (K S0^T)), then
Y = gamma o (Q S0^T) + (M o H) Delta and S_C = gamma_{C-1} S0 + (rho o Delta)^T K
with rho_s = M[C-1,s].  Here those equations are written out in float64 numpy
(no code shared with the kernels) and compared with the oracle's per-step record
at 1e-9: the derivation itself is pinned, independently of the GPU.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle


def chunk_form(q, k, v, g, beta, S0, mask, gqa_map, C):
    q, k, v, g, beta, S0 = (np.asarray(x.double().numpy(), np.float64) for x in (q, k, v, g, beta, S0))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    act_bt = np.ones((B, T), bool) if mask is None else mask.numpy() > 0
    y = np.full((B, T, Hv, Dv), np.nan)
    dl = np.full((B, T, Hv, Dv), np.nan)
    s_out = np.empty_like(S0)
    for b in range(B):
        for hv in range(Hv):
            hk = hv % Hk if gqa_map == "tiled" else hv // (Hv // Hk)
            S = S0[b, hv].copy()
            for t0 in range(0, T, C):
                steps = np.arange(t0, t0 + C)
                act = np.array([t < T and act_bt[b, t] for t in steps])
                K = np.zeros((C, Dk)); Q = np.zeros((C, Dk)); V = np.zeros((C, Dv))
                gt = np.ones(C); bt = np.zeros(C)
                for i, t in enumerate(steps):
                    if act[i]:
                        K[i], Q[i], V[i] = k[b, t, hk], q[b, t, hk], v[b, t, hv]
                        gt[i], bt[i] = g[b, t, hv], beta[b, t, hv]
                M = np.zeros((C, C))
                for t in range(C):                          # running products, no division
                    p = 1.0
                    for s in range(t, -1, -1):
                        M[t, s] = p
                        p *= gt[s]
                gamma = np.cumprod(gt)
                A = np.tril(bt[:, None] * M * (K @ K.T), -1)
                R = V - gamma[:, None] * (K @ S.T)
                Delta = np.linalg.solve(np.eye(C) + A, bt[:, None] * R)
                Y = gamma[:, None] * (Q @ S.T) + np.tril(M * (Q @ K.T)) @ Delta
                S = gamma[-1] * S + (M[-1][:, None] * Delta).T @ K
                for i, t in enumerate(steps):
                    if act[i]:
                        y[b, t, hv], dl[b, t, hv] = Y[i], Delta[i]
            s_out[b, hv] = S
    return y, s_out, dl


CASES = [
    # B, T, Hk, Hv, Dk, Dv, io, mask, map, C
    (1, 130, 2, 4, 32, 16, "f32", "ones", "block", 64),     # several chunks, ragged last one
    (2, 70, 1, 2, 64, 16, "bf16", "bernoulli", "tiled", 64),
    (1, 64, 2, 2, 32, 32, "f16", "trailing", "block", 64),  # exactly one chunk
    (3, 4, 2, 4, 32, 16, "bf16", "trailing", "block", 4),   # a short tape as one chunk
    (2, 3, 1, 3, 64, 16, "f32", "bernoulli", "tiled", 3),
    (1, 40, 1, 1, 32, 16, "f32", "none", "block", 16),      # another chunk length
    (2, 9, 2, 2, 32, 16, "bf16", "zeros", "tiled", 4),      # nothing active
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_T%d_Hk%d_Hv%d_Dk%d_Dv%d_%s_%s_%s_C%d" % c)
def test_chunk_form_equals_the_per_step_record(case):
    B, T, Hk, Hv, Dk, Dv, io, mask, gmap, C = case
    inp = gi.record_inputs(B, T, Hk, Hv, Dk, Dv, io=io, seed=7 + T, mask=mask)
    y, s, dl = chunk_form(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state_in"],
                          inp["mask"], gmap, C)
    ry, rs, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["state_in"], inp["mask"], gqa_map=gmap)
    act = np.ones((B, T), bool) if inp["mask"] is None else inp["mask"].numpy() > 0
    a4 = np.broadcast_to(act[:, :, None, None], ry.shape)
    scale = lambda r: 1.0 + np.abs(r)
    assert np.all(np.abs(y - ry)[a4] <= 1e-9 * scale(ry)[a4]), "y"
    assert np.all(np.abs(dl - rd)[a4] <= 1e-9 * scale(rd)[a4]), "delta"
    assert np.all(np.abs(s - rs) <= 1e-9 * scale(rs)), "state"


def test_chunk_form_with_zero_and_unit_gates():
    """A gate of exactly 0 resets the state inside a chunk; g = 1 with beta = 0
    is the identity step.  Running products of the gates keep both exact."""
    inp = gi.record_inputs(1, 100, 1, 2, 32, 16, io="f32", seed=3, mask="ones")
    g, beta = inp["g"].clone(), inp["beta"].clone()
    g[0, [0, 17, 63, 64, 99], :] = 0.0
    g[0, 30:40, 1] = 1.0
    beta[0, 30:40, 1] = 0.0
    y, s, dl = chunk_form(inp["q"], inp["k"], inp["v"], g, beta, inp["state_in"], None, "block", 64)
    ry, rs, rd = oracle.gdn_record(inp["q"], inp["k"], inp["v"], g, beta, inp["state_in"], None)
    assert np.allclose(y, ry, rtol=1e-9, atol=1e-9)
    assert np.allclose(dl, rd, rtol=1e-9, atol=1e-9)
    assert np.allclose(s, rs, rtol=1e-9, atol=1e-9)


def test_a_planted_mistake_in_the_chunk_form_is_caught():
    """The comparison has teeth: y read from the state before the chunk's own
    innovations (P Delta dropped) is far off."""
    inp = gi.record_inputs(1, 20, 1, 1, 32, 16, io="f32", seed=5, mask="ones")
    y, _, _ = chunk_form(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state_in"],
                         None, "block", 64)
    ry, _, _ = oracle.gdn_record(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                 inp["state_in"], None)
    q, k, S0 = (np.asarray(x.double().numpy()) for x in (inp["q"], inp["k"], inp["state_in"]))
    g = np.asarray(inp["g"].double().numpy())[0, :, 0]
    wrong = np.cumprod(g)[:, None] * (q[0, :, 0] @ S0[0, 0].T)
    assert np.allclose(y[0, :, 0], ry[0, :, 0], rtol=1e-9, atol=1e-9)
    assert not np.allclose(wrong, ry[0, :, 0], rtol=1e-3, atol=1e-3)
