"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU only.  Each pin checks the oracle against a
*different* statement of the method (a special case with a closed form, the
matrix form printed on another page, an invariant, brute force, exact rational
arithmetic), so that a dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of them.

Page names used in citations:
  [notes]   "Kimi K3 notes 1: KDA" (jaimeyzzz.com)
  [deriv]   "KDA derivation summary" (hn.213312.xyz article 49085909)
  [linsp]   "Linear/sparse attention tutorial" (mathieu0905.github.io ai-knowledge)
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def softplus(x):
    return np.logaddexp(0.0, x)


def rand_inputs(rng, B, T, H, dk, dv, unit_keys=True, g_mu=-3.0, g_sigma=1.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.0, 1.0, size=(B, T, H))
    log_alpha = -softplus(rng.normal(g_mu, g_sigma, size=(B, T, H, dk)))
    return q, k, v, log_alpha, beta


def rel_err(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


# --- P1: alpha = 1, additive write, beta = 1  =>  o = (Q K^T (.) M_incl) V ------------
# [notes] sect. 1 (S_t = S_{t-1} + k_t v_t^T, o_t = S_t^T q_t) and [linsp] sect. 2.2
# (parallel form (phi(Q) phi(K)^T (.) M) V with the inclusive causal mask).
def test_pin_linear_attention_equals_masked_quadratic_form():
    rng = np.random.default_rng(101)
    B, T, H, dk, dv = 2, 37, 3, 8, 5
    q, k, v, _, _ = rand_inputs(rng, B, T, H, dk, dv, unit_keys=False)
    la = np.zeros((B, T, H, dk))
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0, write="add")
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = Q @ S0[b, h].T + np.tril(Q @ K.T) @ V
            assert rel_err(out[b, :, h], ref) < 1e-12
            assert rel_err(S[b, h], S0[b, h] + V.T @ K) < 1e-12


# --- P2: unit keys, beta = 1  =>  S_t k_t = v_t for ANY per-channel decay ----------------
# [deriv] sect. 3 (the write replaces the value stored along k_t) and [linsp] sect. 5.1
# (with ||k|| = 1 the projection (I - k k^T) clears the k_t direction before the write).
# Reading q_t := k_t gives o_t = S_t k_t, which must equal v_t at every step; this
# also pins that the readout uses the post-write state.
def test_pin_replacement_property_every_step():
    rng = np.random.default_rng(102)
    B, T, H, dk, dv = 2, 50, 2, 16, 7
    _, k, v, la, _ = rand_inputs(rng, B, T, H, dk, dv, g_mu=-1.0, g_sigma=2.0)
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(k, k, v, la, beta, S0=S0)
    assert rel_err(out, v) < 1e-12
    for b in range(B):
        for h in range(H):
            assert rel_err(S[b, h] @ k[b, -1, h], v[b, -1, h]) < 1e-12


# --- P3: scalar decay broadcast  =>  Gated DeltaNet in matrix form -------------------------
# [linsp] sect. 5.2: S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
def test_pin_scalar_decay_is_gated_deltanet_matrix_form():
    rng = np.random.default_rng(103)
    B, T, H, dk, dv = 1, 40, 3, 8, 6
    q, k, v, _, beta = rand_inputs(rng, B, T, H, dk, dv)
    la_scalar = -softplus(rng.normal(-2.0, 1.0, size=(B, T, H)))
    la = np.repeat(la_scalar[..., None], dk, axis=-1)
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    I = np.eye(dk)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            kt, vt, bt = k[0, t, h], v[0, t, h], beta[0, t, h]
            St = np.exp(la_scalar[0, t, h]) * St @ (I - bt * np.outer(kt, kt)) + bt * np.outer(vt, kt)
            assert rel_err(out[0, t, h], St @ q[0, t, h]) < 1e-11
        assert rel_err(S[0, h], St) < 1e-11


# --- P3b: general KDA step vs the transposed matrix form of [notes] sect. 4 ---------------
# S^kv_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S^kv_{t-1} + beta_t k_t v_t^T with the state
# stored d_k x d_v and o_t = (S^kv_t)^T q_t ([notes] sect. 1).  Per-channel decay, beta in
# (0, 1) and keys that are NOT unit norm: the identity does not need ||k|| = 1.
def test_pin_general_kda_vs_transposed_matrix_form():
    rng = np.random.default_rng(104)
    B, T, H, dk, dv = 2, 33, 2, 9, 4
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv, unit_keys=False, g_mu=-1.5, g_sigma=1.5)
    k *= 0.4
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            Skv = S0[b, h].T.copy()
            for t in range(T):
                kt, vt, bt = k[b, t, h], v[b, t, h], beta[b, t, h]
                Skv = (I - bt * np.outer(kt, kt)) @ np.diag(np.exp(la[b, t, h])) @ Skv + bt * np.outer(kt, vt)
                assert rel_err(out[b, t, h], Skv.T @ q[b, t, h]) < 1e-11
            assert rel_err(S[b, h], Skv.T) < 1e-11


# --- P4: chunked schedule (direct and WY) = token-by-token, every chunk size ---------------
# [deriv] sect. 6: the recurrent and chunk modes are one recurrence with two schedules.
# [linsp] appendix A items 1-2: equality for C = 1, non-divisors and C = T.
@pytest.mark.parametrize("C", [1, 4, 7, 16, 37])
@pytest.mark.parametrize("variant", ["direct", "wy"])
def test_pin_chunked_schedule_equals_recurrence(C, variant):
    rng = np.random.default_rng(105)
    B, T, H, dk, dv = 1, 37, 2, 8, 6
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv, g_mu=-1.0, g_sigma=2.0)
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    out_c, S_c = chunked.chunk_forward(q, k, v, la, beta, S0=S0, C=C, variant=variant)
    assert rel_err(out_c, out) < 1e-12
    assert rel_err(S_c, S) < 1e-12


def test_pin_chunked_schedule_with_extreme_decay():
    """Per-token log-decays down to about -40 (cumulative decays far below the
    float range inside one chunk) still agree: nothing in either schedule
    forms exp of a positive cumulative decay."""
    rng = np.random.default_rng(106)
    B, T, H, dk, dv = 1, 45, 1, 8, 8
    q, k, v, _, beta = rand_inputs(rng, B, T, H, dk, dv)
    la = -rng.uniform(0.0, 40.0, size=(B, T, H, dk)) * (rng.uniform(size=(B, T, H, dk)) < 0.3)
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    out_c, S_c = chunked.chunk_forward(q, k, v, la, beta, S0=S0, C=16)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(S))
    assert rel_err(out_c, out) < 1e-12
    assert rel_err(S_c, S) < 1e-12


# --- P5: orthonormal keys, beta = 1, alpha = 1  =>  delta write = additive write ---------
# [linsp] sect. 5.1 (keys orthogonal to the history: nothing to erase) and appendix A [e].
def test_pin_orthonormal_keys_make_delta_equal_additive():
    rng = np.random.default_rng(107)
    T, dk, dv = 8, 8, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:T][None, :, None, :]                   # T orthonormal rows
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    la = np.zeros((1, T, 1, dk))
    beta = np.ones((1, T, 1))
    o_d, S_d = oracle.forward(q, k, v, la, beta, write="delta")
    o_a, S_a = oracle.forward(q, k, v, la, beta, write="add")
    printed = json.load(open(os.path.join(GOLDEN, "linsparse_sanity_printed.json")))
    bound = printed["delta_vs_additive_final_state_frobenius"]["orthonormal_keys"]
    assert np.linalg.norm(S_d - S_a) <= bound          # page: 3.58e-07 in float32
    assert np.linalg.norm(S_d - S_a) < 1e-12            # float64
    assert rel_err(o_d, o_a) < 1e-12
    # Non-orthogonal unit keys: the rewrite term is active and the two differ by O(1)
    # (the page prints 8.315 for its own random draw at L = 12, d = 8).
    k2 = rng.standard_normal((1, 12, 1, 8))
    k2 /= np.linalg.norm(k2, axis=-1, keepdims=True)
    v2 = rng.standard_normal((1, 12, 1, 8))
    z = np.zeros((1, 12, 1, 8))
    one = np.ones((1, 12, 1))
    _, S_d2 = oracle.forward(z, k2, v2, z, one, write="delta")
    _, S_a2 = oracle.forward(z, k2, v2, z, one, write="add")
    assert np.linalg.norm(S_d2 - S_a2) > 0.5


# --- P6: additive write with per-channel decay  =>  brute-force GLA ------------------------
# [linsp] sect. 2.4 (S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T) and sect. 6.2 (cumulative decay
# folded into the state and the intra-chunk mask): o_t = S0 Diag(e^{G_t}) q_t +
# sum_{j<=t} beta_j v_j sum_c q_tc k_jc e^{G_tc - G_jc}.
def test_pin_additive_per_channel_decay_equals_bruteforce_gla():
    rng = np.random.default_rng(108)
    B, T, H, dk, dv = 1, 30, 2, 6, 5
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv, unit_keys=False, g_mu=-1.0, g_sigma=1.0)
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0, write="add")
    for h in range(H):
        G = np.cumsum(la[0, :, h], axis=0)
        for t in range(T):
            ref = S0[0, h] @ (np.exp(G[t]) * q[0, t, h])
            for j in range(t + 1):
                w = np.sum(q[0, t, h] * k[0, j, h] * np.exp(G[t] - G[j]))
                ref = ref + beta[0, j, h] * v[0, j, h] * w
            assert rel_err(out[0, t, h], ref) < 1e-12
        S_ref = S0[0, h] * np.exp(G[-1])[None, :]
        for j in range(T):
            S_ref = S_ref + beta[0, j, h] * np.outer(v[0, j, h], k[0, j, h] * np.exp(G[-1] - G[j]))
        assert rel_err(S[0, h], S_ref) < 1e-12


# --- P7: state hand-off: run(T1) then run(T2, S0 = S_final) = run(T1 + T2) ----------------
# [linsp] sect. 6.2 (the state entering a chunk carries all earlier history) and sect. 8.1
# (decode touches only the fixed-size state).
def test_pin_resume_from_final_state_is_exact():
    rng = np.random.default_rng(109)
    B, T, H, dk, dv = 2, 41, 2, 8, 8
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dv, dk)) * 0.1
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    T1 = 17
    o1, S1 = oracle.forward(q[:, :T1], k[:, :T1], v[:, :T1], la[:, :T1], beta[:, :T1], S0=S0)
    o2, S2 = oracle.forward(q[:, T1:], k[:, T1:], v[:, T1:], la[:, T1:], beta[:, T1:], S0=S1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(S2, S)
    # token-by-token steps (the decode schedule) give the same result
    St = S0
    for t in range(T):
        sl = slice(t, t + 1)
        ot, St = oracle.forward(q[:, sl], k[:, sl], v[:, sl], la[:, sl], beta[:, sl], S0=St)
        assert np.array_equal(ot[:, 0], out[:, t])
    assert np.array_equal(St, S)


# --- P8: identity tokens and pure decay -----------------------------------------------------
# Derived from the recurrence: k = 0, beta = 0, log alpha = 0 leaves S unchanged (this is
# the padding of a partial last chunk, [linsp] sect. 6.3); beta = 0 leaves only the decay.
def test_pin_identity_tokens_leave_state_unchanged():
    rng = np.random.default_rng(110)
    B, T, H, dk, dv = 1, 24, 2, 8, 4
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dv, dk))
    pad = np.array([3, 4, 11, 23])
    k[:, pad] = 0.0
    beta[:, pad] = 0.0
    la[:, pad] = 0.0
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    keep = np.setdiff1d(np.arange(T), pad)
    out_k, S_k = oracle.forward(q[:, keep], k[:, keep], v[:, keep], la[:, keep], beta[:, keep], S0=S0)
    assert np.array_equal(S, S_k)
    assert np.array_equal(out[:, keep], out_k)
    # an identity token reads the unchanged state
    _, S_before = oracle.forward(q[:, :11], k[:, :11], v[:, :11], la[:, :11], beta[:, :11], S0=S0)
    for h in range(H):
        assert rel_err(out[0, 11, h], S_before[0, h] @ q[0, 11, h]) < 1e-13


def test_pin_zero_beta_is_pure_decay():
    rng = np.random.default_rng(111)
    B, T, H, dk, dv = 1, 20, 1, 8, 3
    q, k, v, la, _ = rand_inputs(rng, B, T, H, dk, dv)
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    G = np.cumsum(la[0, :, 0], axis=0)
    for t in range(T):
        St = S0[0, 0] * np.exp(G[t])[None, :]
        assert rel_err(out[0, t, 0], St @ q[0, t, 0]) < 1e-13
    assert rel_err(S[0, 0], S0[0, 0] * np.exp(G[-1])[None, :]) < 1e-13


# --- P9: exact rational arithmetic on tiny inputs --------------------------------------------
# Brute force with Python fractions: decays given as rationals p/q, log alpha passed to the
# oracle as log(p/q).  Everything else is exact; the float64 oracle must agree to ~1e-14.
def _exact_recurrence(q, k, v, alpha, beta, S0):
    T = len(q)
    dv, dk = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        S = [[S[i][c] * alpha[t][c] for c in range(dk)] for i in range(dv)]
        vhat = [sum(S[i][c] * k[t][c] for c in range(dk)) for i in range(dv)]
        e = [beta[t] * (v[t][i] - vhat[i]) for i in range(dv)]
        S = [[S[i][c] + e[i] * k[t][c] for c in range(dk)] for i in range(dv)]
        outs.append([sum(S[i][c] * q[t][c] for c in range(dk)) for i in range(dv)])
    return outs, S


@pytest.mark.parametrize("T,dk,dv", [(1, 1, 1), (3, 2, 3), (6, 3, 2), (5, 3, 3)])
def test_pin_exact_rational(T, dk, dv):
    rng = np.random.default_rng(112 + T * 10 + dk)

    def frac(x):
        return Fraction(int(round(x * 8)), 8)

    q = [[frac(rng.normal()) for _ in range(dk)] for _ in range(T)]
    k = [[frac(rng.normal() * 0.5) for _ in range(dk)] for _ in range(T)]
    v = [[frac(rng.normal()) for _ in range(dv)] for _ in range(T)]
    alpha = [[Fraction(int(rng.integers(1, 16)), 16) for _ in range(dk)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S0 = [[frac(rng.normal()) for _ in range(dk)] for _ in range(dv)]
    outs, S = _exact_recurrence(q, k, v, alpha, beta, S0)

    f = lambda m: np.array([[float(x) for x in row] for row in m])
    qa, ka, va = f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None]
    la = np.log(f(alpha))[None, :, None]
    ba = np.array([float(b) for b in beta])[None, :, None]
    out, Sf = oracle.forward(qa, ka, va, la, ba, S0=f(S0)[None, None])
    assert rel_err(out[0, :, 0], f(outs)) < 1e-13
    assert rel_err(Sf[0, 0], f(S)) < 1e-13


# --- P10: stability: with unit keys, beta in [0,1], alpha in (0,1] the transition is a
# contraction, so ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||  ([linsp] sect. 5.1 and 10).
def test_pin_state_norm_bound():
    rng = np.random.default_rng(113)
    B, T, H, dk, dv = 1, 300, 1, 16, 16
    q, k, v, la, beta = rand_inputs(rng, B, T, H, dk, dv)
    S = rng.standard_normal((B, H, dv, dk))
    for t in range(T):
        sl = slice(t, t + 1)
        n0 = np.linalg.norm(S)
        _, S = oracle.forward(q[:, sl], k[:, sl], v[:, sl], la[:, sl], beta[:, sl], S0=S)
        assert np.linalg.norm(S) <= n0 + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12


# --- appendix-A printed results of the tutorial page, used as bounds -------------------------
def test_pin_page_printed_linear_attention_chunk_equivalence():
    printed = json.load(open(os.path.join(GOLDEN, "linsparse_sanity_printed.json")))
    a = printed["chunkwise_vs_recurrent_linear_attention"]
    rng = np.random.default_rng(114)
    L, d = a["L"], a["d"]
    q = rng.standard_normal((1, L, 1, d))
    k = rng.standard_normal((1, L, 1, d))
    v = rng.standard_normal((1, L, 1, d))
    z = np.zeros((1, L, 1, d))
    one = np.ones((1, L, 1))
    o_rec, _ = oracle.forward(q, k, v, z, one, write="add")
    worst = 0.0
    for C in a["chunk_sizes"]:
        o_c, _ = chunked.chunk_forward(q, k, v, z, one, C=C, write="add")
        worst = max(worst, float(np.max(np.abs(o_c - o_rec))))
    assert worst <= a["max_abs_diff"] <= a["atol"]
    # item [d]: additive write with beta = 1 is S += v k^T
    dd = printed["delta_without_rewrite_beta1_vs_additive"]
    _, S = oracle.forward(q, k, v, z, one, write="add")
    assert np.max(np.abs(S[0, 0] - v[0, :, 0].T @ k[0, :, 0])) <= dd["abs_diff"] + 1e-12


# --- edge cases -------------------------------------------------------------------------------
def test_oracle_empty_sequence_and_varlen():
    rng = np.random.default_rng(115)
    H, dk, dv = 2, 8, 4
    q, k, v, la, beta = rand_inputs(rng, 1, 0, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    out, S = oracle.forward(q, k, v, la, beta, S0=S0)
    assert out.shape == (1, 0, H, dv) and np.array_equal(S, S0)
    # varlen = independent dense runs, including a zero-length sequence
    lens = [5, 0, 13, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    q, k, v, la, beta = rand_inputs(rng, 1, Tt, H, dk, dv)
    S0 = rng.standard_normal((len(lens), H, dv, dk))
    out, S = oracle.forward_varlen(q, k, v, la, beta, cu, S0=S0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        o_n, S_n = oracle.forward(q[:, sl], k[:, sl], v[:, sl], la[:, sl], beta[:, sl], S0=S0[n:n + 1])
        assert np.array_equal(out[:, sl], o_n)
        assert np.array_equal(S[n:n + 1], S_n)


# ---------------------------------------------------------------- input preparation
def test_prepare_normalises_and_applies_the_gate():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 7, 3, 16)) * 3.0
    k = rng.standard_normal((2, 7, 3, 16)) * 0.2
    k[0, 2, 1] = 0.0                                   # a zero key stays zero
    g = rng.standard_normal((2, 7, 3, 16)) * 4.0
    qn, kn, la = oracle.prepare(q, k, g)
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-14)
    norms = np.linalg.norm(kn, axis=-1)
    assert np.all(kn[0, 2, 1] == 0.0)
    assert np.allclose(np.delete(norms.reshape(-1), np.ravel_multi_index((0, 2, 1), norms.shape)), 1.0,
                       atol=1e-14)
    # direction kept, scale removed
    assert np.allclose(qn * np.linalg.norm(q, axis=-1, keepdims=True), q, atol=1e-12)
    # log alpha = log(sigmoid(-g)) written another way, and its limits
    assert np.allclose(la, np.log(1.0 / (1.0 + np.exp(g))), atol=1e-12)
    assert np.all(la < 0.0)
    _, _, l0 = oracle.prepare(q[:1, :1, :1, :1], q[:1, :1, :1, :1], np.zeros((1, 1, 1, 1)))
    assert abs(l0[0, 0, 0, 0] + np.log(2.0)) < 1e-15
    _, _, lbig = oracle.prepare(q[:1, :1, :1, :1], q[:1, :1, :1, :1], np.full((1, 1, 1, 1), 800.0))
    assert lbig[0, 0, 0, 0] == -800.0                  # no overflow for large pre-activations


def test_prepare_scalar_gate_and_scale_invariance():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 5, 2, 8))
    k = rng.standard_normal((1, 5, 2, 8))
    gs = rng.standard_normal((1, 5, 2))
    _, _, la = oracle.prepare(q, k, gs, gate="scalar")
    assert la.shape == (1, 5, 2, 8) and np.all(la == la[..., :1])
    _, _, la0 = oracle.prepare(q, k, None, gate="none")
    assert np.all(la0 == 0.0)
    a1 = oracle.prepare(q, k, gs, gate="scalar")
    a2 = oracle.prepare(q * 7.5, k * 0.01, gs, gate="scalar")
    assert all(np.allclose(x, y, atol=1e-14) for x, y in zip(a1, a2))
