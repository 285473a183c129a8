"""Pins for the fp64 oracle: values the pages print, closed forms, special
cases that reduce to simpler recurrences, and identities between independent
formulations.  CPU only.

Each test names the passage it pins.  Page tags:
  [LA-KDA]  "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制", blog-3d3.pages.dev/posts/150
  [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构",
            forceinjection.github.io/.../kimi_k3_attention.html
  [K3-NOTES] "Kimi K3", llm.rainlin.net/llm-inference/kimi-k3
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

BIG = 1.0e4   # a logit this large saturates the logistic exactly in float64


def _rand_case(rng, T, H, dk, dv, unit_k=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    z = rng.standard_normal((T, H, dk))
    b = rng.standard_normal((T, H))
    A = rng.uniform(-1, 1, H)
    h0 = 0.3 * rng.standard_normal((H, dk, dv))
    return q, k, v, z, b, A, h0


# ---------------------------------------------------------------- printed values

def test_linear_attention_worked_example(golden_dir):
    """[LA-KDA §3]: (k,v) = (2,5), (3,7), q3 = 4 -> S2 = 31, o3 = 124.
    Erasure off, alpha = 1 (z = -BIG), beta = 1 (b = +BIG).  The third token
    carries k3 = 0 so that o3 reads the state built by the first two."""
    g = json.load(open(os.path.join(golden_dir, "linear_attention_1d.json")))
    k = np.array([g["k"][0], g["k"][1], 0.0]).reshape(3, 1, 1)
    v = np.array([g["v"][0], g["v"][1], 0.0]).reshape(3, 1, 1)
    q = np.array([1.0, 1.0, g["q3"]]).reshape(3, 1, 1)
    z = np.full((3, 1, 1), -BIG)
    b = np.full((3, 1), BIG)
    o, S = oracle.recurrence(q, k, v, z, b, np.zeros(1), erase=False)
    assert o[1, 0, 0] == g["S2"]          # q2 = 1 reads S2 directly
    assert o[2, 0, 0] == g["o3"]
    assert S[0, 0, 0] == g["S2"]


def test_delta_rule_hand_check(golden_dir):
    """[LA-KDA §7.4]: k = (1,1), v = (5,7), beta = (0.5, 0.4), S0 = 0 ->
    S1 = 2.5, S2 = 4.3 token by token; u = (2.5, 1.8) from the triangular solve.
    alpha = 1 via z = -BIG.  beta comes through the logistic of its logit."""
    g = json.load(open(os.path.join(golden_dir, "delta_rule_chunk_c2.json")))
    beta = np.array(g["beta"])
    blog = np.log(beta / (1 - beta)).reshape(2, 1)
    k = np.array(g["k"]).reshape(2, 1, 1)
    v = np.array(g["v"]).reshape(2, 1, 1)
    q = np.ones((2, 1, 1))
    z = np.full((2, 1, 1), -BIG)
    o, S = oracle.recurrence(q, k, v, z, blog, np.zeros(1))
    assert o[0, 0, 0] == pytest.approx(g["S1"], abs=1e-14)
    assert o[1, 0, 0] == pytest.approx(g["S2"], abs=1e-14)
    oc, Sc, inter = oracle.chunkwise(q, k, v, z, blog, np.zeros(1), chunk=2, keep=True)
    u = inter[0][0]["Vt"][:, 0]                 # S0 = 0, so V~ = U
    assert u == pytest.approx(g["u"], abs=1e-14)
    assert Sc[0, 0, 0] == pytest.approx(g["S2"], abs=1e-14)


# ------------------------------------------------------------------ the gate

def test_gate_closed_forms():
    """[LA-KDA §5.4]: g = -5 sigmoid(e^A z) lies in (-5, 0); z = 0 gives -2.5;
    the limits are alpha -> 1 and alpha -> e^-5; A enters only as e^A * z."""
    A = np.array([0.0, math.log(2.0), -1.0])
    z = np.zeros((1, 3, 4))
    assert np.all(oracle.gate_log_decay(z, A) == -2.5)
    rng = np.random.default_rng(1)
    z = rng.standard_normal((50, 3, 8)) * 4
    g = oracle.gate_log_decay(z, A)
    assert np.all(g < 0) and np.all(g > -5)
    # e^A z: A = ln 2 must equal doubling z with A = 0
    assert np.allclose(oracle.gate_log_decay(z[:, 1:2], A[1:2]),
                       oracle.gate_log_decay(2 * z[:, 1:2], np.zeros(1)), rtol=0, atol=1e-15)
    lim = oracle.gate_log_decay(np.array([[[-BIG, BIG]]]), np.zeros(1))
    assert np.exp(lim[0, 0, 0]) == 1.0
    assert np.exp(lim[0, 0, 1]) == pytest.approx(math.exp(-5.0), rel=1e-15)
    # monotone decreasing in z
    zz = np.linspace(-20, 20, 401).reshape(-1, 1, 1)
    gg = oracle.gate_log_decay(zz, np.zeros(1)).ravel()
    assert np.all(np.diff(gg) < 0)


def test_beta_saturation():
    """beta = sigmoid(b) in (0,1) ([LA-KDA §5.1]) or [0,1] ([K3-ATTN §2.1]);
    saturated logits give exactly 0 and 1 in float64."""
    bb = oracle.beta_of(np.array([-BIG, 0.0, BIG]))
    assert bb[0] == 0.0 and bb[1] == 0.5 and bb[2] == 1.0


# ---------------------------------------------------- family special cases

def test_linear_attention_limit():
    """[LA-KDA §3]: erasure off and alpha = 1 leave S_t = S_0 + sum beta_i k_i v_i^T,
    so o_t = S_0^T q_t + sum_{i<=t} beta_i (q_t . k_i) v_i."""
    rng = np.random.default_rng(2)
    q, k, v, z, b, A, h0 = _rand_case(rng, 23, 2, 5, 3)
    z = np.full_like(z, -BIG)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0, erase=False)
    beta = 1 / (1 + np.exp(-b))
    for t in range(23):
        for h in range(2):
            ref = h0[h].T @ q[t, h]
            for i in range(t + 1):
                ref = ref + beta[i, h] * (q[t, h] @ k[i, h]) * v[i, h]
            assert np.allclose(o[t, h], ref, atol=1e-12)


def test_gated_linear_attention_limit():
    """[LA-KDA §4] (GLA row) and the expansion of [LA-KDA §7.2]: without erasure,
    S_t = Diag(gamma_t) S_0 + sum_{i<=t} Diag(gamma_t / gamma_i) beta_i k_i v_i^T
    with gamma_t = alpha_1 * ... * alpha_t."""
    rng = np.random.default_rng(3)
    q, k, v, z, b, A, h0 = _rand_case(rng, 19, 2, 4, 3)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0, erase=False)
    alpha = np.exp(-5 / (1 + np.exp(-np.exp(A)[None, :, None] * z)))
    beta = 1 / (1 + np.exp(-b))
    for h in range(2):
        for t in range(19):
            gam_t = np.prod(alpha[: t + 1, h], axis=0)
            St = gam_t[:, None] * h0[h]
            for i in range(t + 1):
                ratio = np.prod(alpha[i + 1: t + 1, h], axis=0)
                St = St + beta[i, h] * np.outer(ratio * k[i, h], v[i, h])
            assert np.allclose(o[t, h], St.T @ q[t, h], atol=1e-12)


def test_deltanet_limit_matches_printed_chunk_equations():
    """[LA-KDA §7.3] for alpha = 1, one chunk spanning the sequence:
    (I + B L) U = B (V - K S_0), L = StrictLowerTri(K K^T);
    O = Q S_0 + Tril(Q K^T) U;  S_C = S_0 + K^T U."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 11, 1, 6, 4
    q, k, v, z, b, A, h0 = _rand_case(rng, T, H, dk, dv)
    z = np.full_like(z, -BIG)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0)
    Q, K, V, S0 = q[:, 0], k[:, 0], v[:, 0], h0[0]
    Bm = np.diag(1 / (1 + np.exp(-b[:, 0])))
    L = np.tril(K @ K.T, -1)
    U = np.linalg.solve(np.eye(T) + Bm @ L, Bm @ (V - K @ S0))
    assert np.allclose(o[:, 0], Q @ S0 + np.tril(Q @ K.T) @ U, atol=1e-12)
    assert np.allclose(S[0], S0 + K.T @ U, atol=1e-12)


def test_exact_recall_after_full_write():
    """[K3-ATTN §2.1] calls (I - beta k k^T) a generalised Householder map that
    removes the old component along k.  With beta = 1 and |k| = 1 the new state
    returns v exactly at key k, whatever alpha and S_{t-1}: S_t^T k_t = v_t."""
    rng = np.random.default_rng(5)
    T, H, dk, dv = 9, 3, 7, 5
    q, k, v, z, b, A, h0 = _rand_case(rng, T, H, dk, dv)
    b = np.full_like(b, BIG)
    o, _ = oracle.recurrence(k, k, v, z, b, A, h0)   # read with q_t = k_t
    assert np.allclose(o, v, atol=1e-12)


def test_pure_decay_when_beta_is_zero():
    """beta = 0 writes nothing: S_t = Diag(prod alpha) S_0 ([LA-KDA §5.2] with
    the delta and write terms scaled by beta)."""
    rng = np.random.default_rng(6)
    q, k, v, z, b, A, h0 = _rand_case(rng, 13, 2, 4, 3)
    b = np.full_like(b, -BIG)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0)
    alpha = np.exp(-5 / (1 + np.exp(-np.exp(A)[None, :, None] * z)))
    for t in range(13):
        gam = np.prod(alpha[: t + 1], axis=0)
        St = gam[:, :, None] * h0
        assert np.allclose(o[t], np.einsum("hkv,hk->hv", St, q[t]), atol=1e-14)


# ------------------------------------------------------------------ identities

@pytest.mark.parametrize("seed", [7, 8])
def test_three_step_dplr_equals_matrix_form(seed):
    """The three-step DPLR update of [K3-ATTN §2.2], the delta form of
    [K3-NOTES] and the explicit d_k x d_k transition of [LA-KDA §5.2] agree."""
    rng = np.random.default_rng(seed)
    args = _rand_case(rng, 17, 2, 6, 5)
    o1, S1 = oracle.recurrence(*args)
    o2, S2 = oracle.recurrence_dplr(*args)
    o3, S3 = oracle.recurrence_matrix(*args)
    for o, S in ((o2, S2), (o3, S3)):
        assert np.allclose(o, o1, atol=1e-13) and np.allclose(S, S1, atol=1e-13)


@pytest.mark.parametrize("T,chunk", [(70, 16), (64, 16), (5, 16), (37, 8), (130, 64)])
def test_chunkwise_equals_recurrence(T, chunk):
    """[LA-KDA §7]: the chunked form reaches the token recurrence's result,
    with a ragged last chunk, with and without an initial state."""
    rng = np.random.default_rng(T + chunk)
    q, k, v, z, b, A, h0 = _rand_case(rng, T, 2, 8, 6)
    for init in (None, h0):
        o1, S1 = oracle.recurrence(q, k, v, z, b, A, init)
        o2, S2 = oracle.chunkwise(q, k, v, z, b, A, init, chunk=chunk)
        assert np.abs(o1 - o2).max() < 1e-12
        assert np.abs(S1 - S2).max() < 1e-12


def test_chunkwise_slow_decay_long_memory():
    """Near-1 decay (very negative z) keeps the initial state alive across many
    chunks; the chunked form must still agree."""
    rng = np.random.default_rng(9)
    q, k, v, z, b, A, h0 = _rand_case(rng, 96, 1, 8, 8)
    z = z - 6.0
    o1, S1 = oracle.recurrence(q, k, v, z, b, A, h0)
    o2, S2 = oracle.chunkwise(q, k, v, z, b, A, h0, chunk=16)
    assert np.abs(S1).max() > 1e-2
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(S1 - S2).max() < 1e-12


def test_linear_in_values_and_initial_state():
    """For fixed q, k, z, b, A the outputs and final state are linear in (V, S_0):
    every operation on the pages is linear in the state and in v."""
    rng = np.random.default_rng(10)
    q, k, v, z, b, A, h0 = _rand_case(rng, 21, 2, 5, 4)
    v2 = rng.standard_normal(v.shape)
    h2 = rng.standard_normal(h0.shape)
    a1, a2 = 0.7, -1.3
    o1, S1 = oracle.recurrence(q, k, v, z, b, A, h0)
    o2, S2 = oracle.recurrence(q, k, v2, z, b, A, h2)
    o3, S3 = oracle.recurrence(q, k, a1 * v + a2 * v2, z, b, A, a1 * h0 + a2 * h2)
    assert np.allclose(o3, a1 * o1 + a2 * o2, atol=1e-12)
    assert np.allclose(S3, a1 * S1 + a2 * S2, atol=1e-12)


def test_value_columns_are_independent():
    """Permuting the d_v columns of v and S_0 permutes those of o and S."""
    rng = np.random.default_rng(11)
    q, k, v, z, b, A, h0 = _rand_case(rng, 15, 2, 4, 6)
    perm = rng.permutation(6)
    o1, S1 = oracle.recurrence(q, k, v, z, b, A, h0)
    o2, S2 = oracle.recurrence(q, k, v[..., perm], z, b, A, h0[..., perm])
    assert np.allclose(o2, o1[..., perm], atol=1e-14)
    assert np.allclose(S2, S1[..., perm], atol=1e-14)


def test_resume_from_returned_state():
    """Running T1 tokens then T2 tokens from the returned state equals one run
    over T1 + T2 ([K3-NOTES]: the state is stored and handed back)."""
    rng = np.random.default_rng(12)
    q, k, v, z, b, A, h0 = _rand_case(rng, 40, 2, 5, 4)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0)
    oa, Sa = oracle.recurrence(q[:25], k[:25], v[:25], z[:25], b[:25], A, h0)
    ob, Sb = oracle.recurrence(q[25:], k[25:], v[25:], z[25:], b[25:], A, Sa)
    assert np.allclose(np.concatenate([oa, ob]), o, atol=1e-13)
    assert np.allclose(Sb, S, atol=1e-13)


def test_segment_maps_compose_to_the_recurrence():
    """A segment acts on its incoming state affinely, S_end = M S_start + R
    (for fixed inputs the update is affine in the state): R is the run from a
    zero state and, with d_v = d_k, the run from the identity is M + R.
    Composing the segments' maps in order, S_start(j+1) = M_j S_start(j) +
    R_j ([LA-KDA §7.5], the chunk-level recursion that the segmented chain
    computes), gives the state of one uninterrupted run at every segment
    boundary, for segments of 17, 23, 1 and 49 tokens."""
    rng = np.random.default_rng(21)
    T, H, d = 90, 2, 6
    q, k, v, z, b, A, h0 = _rand_case(rng, T, H, d, d)
    z = z - 3.0          # slow decay: the maps carry the state across segments
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    S = h0
    cuts = [0, 17, 40, 41, 90]
    for a, e in zip(cuts[:-1], cuts[1:]):
        seg = (q[a:e], k[a:e], v[a:e], z[a:e], b[a:e], A)
        _, R = oracle.recurrence(*seg, None)
        _, MR = oracle.recurrence(*seg, eye)
        M = MR - R
        S = M @ S + R
        _, S_run = oracle.recurrence(q[:e], k[:e], v[:e], z[:e], b[:e], A, h0)
        assert np.allclose(S, S_run, atol=1e-12)
        assert not np.allclose(S_run, R, atol=1e-3)   # the incoming state matters


def test_packed_equals_separate_and_empty_sequence():
    """A packed batch restarts at every offset; an empty sequence returns its
    initial state unchanged."""
    rng = np.random.default_rng(13)
    lens = [5, 0, 17, 1]
    T = sum(lens)
    q, k, v, z, b, A, _ = _rand_case(rng, T, 2, 4, 3)
    h0 = rng.standard_normal((len(lens), 2, 4, 3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = oracle.packed(q[None], k[None], v[None], z[None], b[None], A, h0, cu)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        if e == a:
            assert np.array_equal(S[s], h0[s])
            continue
        o_s, S_s = oracle.recurrence(q[a:e], k[a:e], v[a:e], z[a:e], b[a:e], A, h0[s])
        assert np.array_equal(o[a:e], o_s) and np.array_equal(S[s], S_s)


def test_decode_step_equals_one_token_of_prefill():
    """[K3-NOTES]: the recurrent call and the chunked call share state semantics;
    one decode step equals one token of the recurrence."""
    rng = np.random.default_rng(14)
    N, H, dk, dv = 3, 2, 4, 5
    q, k, v, z, b, A, _ = _rand_case(rng, N, H, dk, dv)
    st = rng.standard_normal((N, H, dk, dv))
    o, S = oracle.decode_step(q, k, v, z, b, A, st)
    for n in range(N):
        o1, S1 = oracle.recurrence(q[n:n + 1], k[n:n + 1], v[n:n + 1], z[n:n + 1],
                                   b[n:n + 1], A, st[n])
        assert np.allclose(o[n], o1[0], atol=1e-15) and np.allclose(S[n], S1, atol=1e-15)


def test_chunkwise_records_the_incoming_state():
    """The recorded per-chunk S_0 is the state entering that chunk, i.e. the
    recurrence's state after the preceding tokens."""
    rng = np.random.default_rng(15)
    q, k, v, z, b, A, h0 = _rand_case(rng, 40, 1, 4, 4)
    _, _, inter = oracle.chunkwise(q, k, v, z, b, A, h0, chunk=16, keep=True)
    assert np.array_equal(inter[0][0]["S0"], h0[0])
    _, S16 = oracle.recurrence(q[:16], k[:16], v[:16], z[:16], b[:16], A, h0)
    assert np.allclose(inter[1][0]["S0"], S16[0], atol=1e-13)


# ---------------------------------------------------------------- replay fold

def _window(rng, N, W, H, dk, dv):
    k = rng.standard_normal((N, W, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, W, H, dv))
    z = rng.standard_normal((N, W, H, dk))
    b = rng.standard_normal((N, W, H))
    A = rng.uniform(-1, 1, H)
    state = 0.3 * rng.standard_normal((N, H, dk, dv))
    return k, v, z, b, A, state


def test_replay_fold_counts_zero_and_clamped():
    """[K3-ATTN §6.2]: only the accepted prefix is replayed.  A count of zero
    (or below) leaves the checkpoint as it is; a count above the window length
    replays the whole window."""
    rng = np.random.default_rng(11)
    k, v, z, b, A, state = _window(rng, 4, 5, 2, 6, 5)
    out = oracle.replay_fold(k, v, z, b, A, state, [0, -3, 5, 9])
    assert np.array_equal(out[0], state[0]) and np.array_equal(out[1], state[1])
    full = oracle.replay_fold(k, v, z, b, A, state, [5, 5, 5, 5])
    assert np.array_equal(out[3], full[3]) and np.array_equal(out[2], full[2])


def test_replay_fold_pure_decay_closed_form():
    """[K3-ATTN §6.2] with beta = 0 (b = -1e4): no write happens, so replaying
    n tokens multiplies each state row by the product of the n decays
    alpha = exp(-5 sigma(e^{A_h} z)) of [LA-KDA §5.4]."""
    rng = np.random.default_rng(12)
    N, W, H, dk, dv = 3, 6, 2, 5, 4
    k, v, z, b, A, state = _window(rng, N, W, H, dk, dv)
    b = np.full_like(b, -BIG)
    n_acc = [2, 6, 4]
    out = oracle.replay_fold(k, v, z, b, A, state, n_acc)
    for s, n in enumerate(n_acc):
        for h in range(H):
            logit = np.exp(A[h]) * z[s, :n, h]                     # [n, dk]
            alpha = np.exp(-5.0 / (1.0 + np.exp(-logit)))
            expect = np.prod(alpha, axis=0)[:, None] * state[s, h]
            assert np.allclose(out[s, h], expect, rtol=1e-12, atol=0)


def test_replay_fold_exact_recall_of_last_token():
    """With beta = 1 and a unit key, the state after a token recalls that
    token's value exactly at its key, S^T k = v ([K3-ATTN §2.2]); this holds
    for the state the fold leaves after the last accepted token."""
    rng = np.random.default_rng(13)
    N, W, H, dk, dv = 3, 4, 2, 6, 3
    k, v, z, b, A, state = _window(rng, N, W, H, dk, dv)
    b = np.full_like(b, BIG)
    n_acc = [1, 3, 4]
    out = oracle.replay_fold(k, v, z, b, A, state, n_acc)
    for s, n in enumerate(n_acc):
        for h in range(H):
            kk = k[s, n - 1, h]
            assert np.allclose(out[s, h].T @ kk, v[s, n - 1, h], rtol=0, atol=1e-12)


def test_replay_fold_equals_chunked_final_state():
    """The fold's state equals the final state of the chunked formulation
    ([LA-KDA §7.3] with the decay) run over the accepted tokens from the same
    checkpoint: two independent routes to the same state."""
    rng = np.random.default_rng(14)
    N, W, H, dk, dv = 3, 7, 2, 8, 6
    k, v, z, b, A, state = _window(rng, N, W, H, dk, dv)
    n_acc = [7, 5, 3]
    out = oracle.replay_fold(k, v, z, b, A, state, n_acc)
    for s, n in enumerate(n_acc):
        q = rng.standard_normal((n, H, dk))
        _, S = oracle.chunkwise(q, k[s, :n], v[s, :n], z[s, :n], b[s, :n], A, state[s], chunk=4)
        assert np.allclose(out[s], S, rtol=1e-12, atol=1e-13)


def test_replay_window_token_is_about_one_kilobyte():
    """[K3-ATTN §6.2] keeps about 1 KB of inputs per draft token instead of a
    64 KB state snapshot: at d_k = d_v = 128 the fold's per-token inputs are
    k and v in bf16 plus the fp32 gate logits and beta logit."""
    dk = dv = 128
    per_token = 2 * dk + 2 * dv + 4 * dk + 4
    assert 1000 <= per_token <= 1100
    assert dk * dv * 4 == 64 * 1024


# ---------------------------------------------------------------- around the core

def test_short_conv_worked_example():
    """[K3-ATTN §2.3] kernel-size-4 causal convolution on one channel: with taps
    (1, 10, 100, 1000) oldest first each output spells its last four inputs as
    decimal digits, x = 1..5 -> 1000, 2100, 3210, 4321, 5432; a carried history
    (7, 8, 9) gives 9 * 100 + 8 * 10 + 7 + 1000 = 1987 first."""
    x = np.arange(1.0, 6.0).reshape(5, 1, 1)
    w = np.array([1.0, 10.0, 100.0, 1000.0]).reshape(1, 1, 4)
    y, st = oracle.short_conv(x, w)
    assert y[:, 0, 0].tolist() == [1000.0, 2100.0, 3210.0, 4321.0, 5432.0]
    assert st[:, 0, 0].tolist() == [3.0, 4.0, 5.0]
    y2, _ = oracle.short_conv(x[:1], w, np.array([7.0, 8.0, 9.0]).reshape(3, 1, 1))
    assert y2[0, 0, 0] == 1987.0


def test_short_conv_is_causal_and_resumable():
    """Depthwise and causal ([K3-ATTN §2.3]): an output never sees later inputs
    or other channels, and running a sequence in two pieces with the carried
    state equals one pass."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((11, 2, 5))
    w = rng.standard_normal((2, 5, 4))
    y, st = oracle.short_conv(x, w)
    x2 = x.copy()
    x2[7:] += 3.0                       # change the future
    x2[:, 1, 2] += 1.0                  # and one other channel
    y2, _ = oracle.short_conv(x2, w)
    assert np.array_equal(y[:7, 0], y2[:7, 0]) and np.array_equal(y[:7, 1, :2], y2[:7, 1, :2])
    ya, sa = oracle.short_conv(x[:4], w)
    yb, sb = oracle.short_conv(x[4:], w, sa)
    assert np.allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-14)
    assert np.array_equal(sb, st)


def test_swish_l2norm_rmsnorm_closed_forms():
    """Swish(0) = 0 and Swish(ln 3) = 3/4 ln 3 (sigma(ln 3) = 3/4); L2Norm
    returns unit rows whatever the scale; Sigmoid(g) RMSNorm(c 1) =
    sigma(g) c / sqrt(c^2 + eps) per channel ([LA-KDA §5.5])."""
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(float(oracle.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert math.isclose(float(oracle.silu(40.0)), 40.0, rel_tol=1e-15)
    rng = np.random.default_rng(32)
    x = rng.standard_normal((4, 3, 16))
    n = oracle.l2norm(x, 0.0)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=1e-14)
    assert np.allclose(oracle.l2norm(1e3 * x, 0.0), n, rtol=1e-13)
    assert np.array_equal(oracle.l2norm(np.zeros(8), 1e-6), np.zeros(8))
    c, eps = -2.5, 1e-5
    o = np.full((1, 1, 8), c)
    y0 = oracle.rmsnorm_gated(o, np.zeros((1, 1, 8)), np.ones(8), eps)
    assert np.allclose(y0, 0.5 * c / math.sqrt(c * c + eps), rtol=1e-15)
    y1 = oracle.rmsnorm_gated(o, np.full((1, 1, 8), BIG), 2 * np.ones(8), eps)
    assert np.allclose(y1, 2 * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_fused_layer_resumes_with_both_states():
    """[K3-NOTES]: KDA carries a short-convolution state for q, k, v beside the
    recurrent state; a sequence cut in two and resumed from both states gives
    the same outputs and final states as one pass."""
    rng = np.random.default_rng(33)
    T, H, d = 13, 2, 8
    q_in, k_in, v_in, gate = (rng.standard_normal((T, H, d)) for _ in range(4))
    z = rng.standard_normal((T, H, d))
    b = rng.standard_normal((T, H))
    A = rng.uniform(-1, 1, H)
    cw = rng.standard_normal((3, H, d, 4))
    nw = rng.uniform(0.5, 1.5, d)
    y, S, cs = oracle.fused_forward(q_in, k_in, v_in, cw, z, b, A, gate, nw)
    a = 5
    y1, S1, cs1 = oracle.fused_forward(q_in[:a], k_in[:a], v_in[:a], cw, z[:a], b[:a], A, gate[:a], nw)
    y2, S2, cs2 = oracle.fused_forward(q_in[a:], k_in[a:], v_in[a:], cw, z[a:], b[a:], A, gate[a:], nw,
                                       h0=S1, conv_state=cs1)
    assert np.allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-12)
    assert np.allclose(S2, S, rtol=1e-12, atol=1e-13)
    assert np.array_equal(cs2, cs)


def test_fused_layer_identity_taps_reduce_to_the_core():
    """With the taps (0, 0, 0, 1) the convolution passes its input through, so
    the layer is the recurrence on L2Norm(Swish(.)) inputs followed by the
    output gate; with Swish inputs already unit rows the L2Norm is exact."""
    rng = np.random.default_rng(34)
    T, H, d = 9, 2, 6
    q_in, k_in, v_in, gate = (rng.standard_normal((T, H, d)) for _ in range(4))
    z = rng.standard_normal((T, H, d))
    b = rng.standard_normal((T, H))
    A = rng.uniform(-1, 1, H)
    cw = np.zeros((3, H, d, 4))
    cw[..., 3] = 1.0
    nw = np.ones(d)
    y, S, _ = oracle.fused_forward(q_in, k_in, v_in, cw, z, b, A, gate, nw, l2_eps=0.0, rms_eps=0.0)
    sq = q_in / (1 + np.exp(-q_in)) * 1.0
    sk = k_in / (1 + np.exp(-k_in))
    q = sq / np.linalg.norm(sq, axis=-1, keepdims=True)
    k = sk / np.linalg.norm(sk, axis=-1, keepdims=True)
    o, S_ref = oracle.recurrence(q, k, v_in / (1 + np.exp(-v_in)), z, b, A)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    assert np.allclose(S, S_ref, rtol=1e-13, atol=1e-14)
    assert np.allclose(y, o / rms / (1 + np.exp(-gate)), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ family modes
# The rows of the family table in [LA-KDA §4] as switches of the oracle:
# decay=False is DeltaNet (alpha = 1), erase=False gated linear attention.

def test_decay_off_is_the_printed_delta_rule(golden_dir):
    """[LA-KDA §7.4] printed values with decay=False: the gate logits are not
    read (random z and A give the same S1 = 2.5, S2 = 4.3)."""
    g = json.load(open(os.path.join(golden_dir, "delta_rule_chunk_c2.json")))
    beta = np.array(g["beta"])
    blog = np.log(beta / (1 - beta)).reshape(2, 1)
    k = np.array(g["k"]).reshape(2, 1, 1)
    v = np.array(g["v"]).reshape(2, 1, 1)
    q = np.ones((2, 1, 1))
    rng = np.random.default_rng(40)
    o, S = oracle.recurrence(q, k, v, rng.standard_normal((2, 1, 1)), blog,
                             rng.standard_normal(1), decay=False)
    assert o[0, 0, 0] == pytest.approx(g["S1"], abs=1e-14)
    assert o[1, 0, 0] == pytest.approx(g["S2"], abs=1e-14)
    o2, _ = oracle.recurrence(q, k, v, None, blog, None, decay=False)
    assert np.array_equal(o, o2)


def test_decay_and_erase_off_is_linear_attention(golden_dir):
    """[LA-KDA §3] printed o3 = 124 with both switches off and beta = 1."""
    g = json.load(open(os.path.join(golden_dir, "linear_attention_1d.json")))
    k = np.array([g["k"][0], g["k"][1], 0.0]).reshape(3, 1, 1)
    v = np.array([g["v"][0], g["v"][1], 0.0]).reshape(3, 1, 1)
    q = np.array([1.0, 1.0, g["q3"]]).reshape(3, 1, 1)
    b = np.full((3, 1), BIG)
    o, _ = oracle.recurrence(q, k, v, None, b, None, erase=False, decay=False)
    assert o[2, 0, 0] == g["o3"]


def test_decay_off_matches_the_deltanet_matrix_recurrence():
    """[LA-KDA §4] DeltaNet row written as explicit matrices:
    S_t = (I - beta k k^T) S_{t-1} + beta k v^T, o_t = S_t^T q_t."""
    rng = np.random.default_rng(41)
    q, k, v, z, b, A, h0 = _rand_case(rng, 15, 2, 5, 4)
    o, S = oracle.recurrence(q, k, v, z, b, A, h0, decay=False)
    beta = 1 / (1 + np.exp(-b))
    for h in range(2):
        St = h0[h].copy()
        for t in range(15):
            St = (np.eye(5) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ St \
                + beta[t, h] * np.outer(k[t, h], v[t, h])
            assert np.allclose(o[t, h], St.T @ q[t, h], atol=1e-13)
        assert np.allclose(S[h], St, atol=1e-13)


# ------------------------------------------------- general DPLR (a != b)

def _dplr_case(rng, T, H, dk, dv):
    q, k, v, z, b, A, h0 = _rand_case(rng, T, H, dk, dv)
    ah = rng.standard_normal((T, H, dk))
    ah /= np.linalg.norm(ah, axis=-1, keepdims=True)
    bv = ah + 0.5 * rng.standard_normal((T, H, dk)) / np.sqrt(dk)
    bv /= np.linalg.norm(bv, axis=-1, keepdims=True)
    a = -(1 / (1 + np.exp(-b)))[..., None] * ah
    return q, k, v, a, bv, z, A, h0


@pytest.mark.parametrize("seed", [42, 43])
def test_dplr_general_reduces_to_kda(seed):
    """[K3-ATTN §2.2]: binding both low-rank vectors and the write key to k
    (a = -beta k, b = k, write key beta k) gives KDA; checked against the
    delta form of [K3-NOTES] (`recurrence`, pinned above)."""
    rng = np.random.default_rng(seed)
    q, k, v, z, b, A, h0 = _rand_case(rng, 21, 2, 6, 4)
    beta = 1 / (1 + np.exp(-b))
    o1, S1 = oracle.recurrence(q, k, v, z, b, A, h0)
    o2, S2 = oracle.recurrence_dplr_general(q, beta[..., None] * k, v, -beta[..., None] * k, k,
                                            z, A, h0)
    assert np.allclose(o2, o1, atol=1e-13) and np.allclose(S2, S1, atol=1e-13)


def test_dplr_general_equals_explicit_matrices():
    """The general update as explicit d_k x d_k matrices:
    S_t = (I + a b^T) Diag(alpha) S_{t-1} + k v^T."""
    rng = np.random.default_rng(44)
    q, k, v, a, bv, z, A, h0 = _dplr_case(rng, 14, 2, 6, 3)
    o, S = oracle.recurrence_dplr_general(q, k, v, a, bv, z, A, h0)
    alpha = np.exp(-5 / (1 + np.exp(-np.exp(A)[None, :, None] * z)))
    for h in range(2):
        St = h0[h].copy()
        for t in range(14):
            M = (np.eye(6) + np.outer(a[t, h], bv[t, h])) @ np.diag(alpha[t, h])
            St = M @ St + np.outer(k[t, h], v[t, h])
            assert np.allclose(o[t, h], St.T @ q[t, h], atol=1e-13)
        assert np.allclose(S[h], St, atol=1e-13)


def test_dplr_general_without_low_rank_is_gla():
    """a = 0 leaves Diag(alpha) S + k v^T: the GLA row of [LA-KDA §4] with
    beta = 1, in the closed form of its expansion ([LA-KDA §7.2])."""
    rng = np.random.default_rng(45)
    q, k, v, a, bv, z, A, h0 = _dplr_case(rng, 12, 2, 4, 3)
    o, _ = oracle.recurrence_dplr_general(q, k, v, np.zeros_like(a), bv, z, A, h0)
    alpha = np.exp(-5 / (1 + np.exp(-np.exp(A)[None, :, None] * z)))
    for h in range(2):
        for t in range(12):
            St = np.prod(alpha[: t + 1, h], axis=0)[:, None] * h0[h]
            for i in range(t + 1):
                St = St + np.outer(np.prod(alpha[i + 1: t + 1, h], axis=0) * k[i, h], v[i, h])
            assert np.allclose(o[t, h], St.T @ q[t, h], atol=1e-13)


def test_dplr_general_projection_recalls_exactly():
    """With a = -b, |b| = 1 and write key b, (I - b b^T) removes the component
    along b before the write ([K3-ATTN §2.1], Householder view), so the new
    state returns v exactly at b: S_t^T b_t = v_t."""
    rng = np.random.default_rng(46)
    q, k, v, a, bv, z, A, h0 = _dplr_case(rng, 10, 2, 5, 4)
    o, _ = oracle.recurrence_dplr_general(bv, bv, v, -bv, bv, z, A, h0)
    assert np.allclose(o, v, atol=1e-12)


@pytest.mark.parametrize("T,chunk", [(37, 16), (40, 8), (5, 16)])
def test_chunkwise_dplr_equals_recurrence(T, chunk):
    """The four-matrix chunked form (derivation in `chunkwise_dplr`) against the
    token recurrence, with a partial last chunk."""
    rng = np.random.default_rng(47 + T)
    args = _dplr_case(rng, T, 2, 6, 5)
    o1, S1 = oracle.recurrence_dplr_general(*args)
    o2, S2 = oracle.chunkwise_dplr(*args, chunk=chunk)
    assert np.allclose(o2, o1, atol=1e-12) and np.allclose(S2, S1, atol=1e-12)


def test_chunkwise_dplr_collapses_to_two_matrices_for_kda():
    """For KDA inputs (a = -beta k, b = k, write key beta k) the four chunk
    matrices are two up to scales ([K3-ATTN §2.2]): A_ba = -A_bk and
    A_qa = -A_qk, and the chunked result is the KDA one."""
    rng = np.random.default_rng(48)
    q, k, v, z, b, A, h0 = _rand_case(rng, 16, 1, 6, 4)
    beta = (1 / (1 + np.exp(-b)))[..., None]
    o, S, inter = oracle.chunkwise_dplr(q, beta * k, v, -beta * k, k, z, A, h0, chunk=16, keep=True)
    r = inter[0][0]
    assert np.allclose(r["Aba"], -r["Abk"], atol=1e-14) and np.allclose(r["Aqa"], -r["Aqk"], atol=1e-14)
    o1, S1 = oracle.recurrence(q, k, v, z, b, A, h0)
    assert np.allclose(o, o1, atol=1e-12) and np.allclose(S, S1, atol=1e-12)


def test_dplr_decode_step_is_one_token_of_the_recurrence():
    rng = np.random.default_rng(49)
    q, k, v, a, bv, z, A, h0 = _dplr_case(rng, 3, 2, 4, 3)
    st = np.stack([h0, 0.5 * h0])
    o, S = oracle.decode_step_dplr(q[:2], k[:2], v[:2], a[:2], bv[:2], z[:2], A, st)
    for n in range(2):
        r = lambda x: x[n:n + 1]
        o1, S1 = oracle.recurrence_dplr_general(r(q), r(k), r(v), r(a), r(bv), r(z), A, st[n])
        assert np.allclose(o[n], o1[0], atol=1e-14) and np.allclose(S[n], S1, atol=1e-14)


def test_verify_window_matches_explicit_matrices_and_leaves_state():
    """[K3-ATTN §6.2] verify pass: every draft token's output from the
    checkpoint, checked against the explicit-matrix recurrence of
    [LA-KDA §5.2]; the checkpoint passed in is not modified."""
    rng = np.random.default_rng(60)
    N, W, H, dk, dv = 3, 5, 2, 6, 4
    q, k, v, z, b, A, _ = _rand_case(rng, N * W, H, dk, dv)
    sh = lambda x: x.reshape(N, W, *x.shape[1:])   # noqa: E731
    st = 0.3 * rng.standard_normal((N, H, dk, dv))
    st0 = st.copy()
    o = oracle.verify_window(sh(q), sh(k), sh(v), sh(z), sh(b), A, st)
    assert np.array_equal(st, st0)
    for n in range(N):
        on, _ = oracle.recurrence_matrix(sh(q)[n], sh(k)[n], sh(v)[n], sh(z)[n], sh(b)[n], A, st[n])
        assert np.allclose(o[n], on, atol=1e-13)
