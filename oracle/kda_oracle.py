"""Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) core.

TEST INFRASTRUCTURE.  Only the tests, `__graft_entry__.smoke()` and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or constants) and imports
nothing from it; the product path never calls it.

Sources (web pages; citations are "[tag §section]"):
  [LA-KDA]   "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制",
             blog-3d3.pages.dev/posts/150
  [K3-ATTN]  "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构",
             forceinjection.github.io/09_inference_system/vllm/module_analysis/kimi_k3_attention.html
  [K3-NOTES] "Kimi K3", llm.rainlin.net/llm-inference/kimi-k3 (section "Kimi Delta Attention")

What the core computes, per (sequence, head), token by token:
  alpha_t = exp(g_min * sigmoid(exp(A_h) * z_t)), g_min = -5, per channel   [LA-KDA §5.4]
  beta_t  = sigmoid(b_t)                                                     [LA-KDA §5.3]
  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T      [LA-KDA §5.2], [K3-ATTN §2.1]
  o_t = S_t^T q_t   (read after the update)                                  [LA-KDA §5.5], [K3-ATTN §2.1]
with S in R^{d_k x d_v}.  The order of one step is decay -> erase -> write ->
read ([LA-KDA §5.2] four-step reading; [K3-NOTES] update equations).

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * no query scale: o_t = S_t^T q_t exactly; a caller wanting 1/sqrt(d_k)
    pre-scales q (no formula on any page carries a scale);
  * A_h is one scalar per head used as exp(A_h) * z inside the sigmoid; the
    per-head bias that [LA-KDA §5.3] mentions is folded into z upstream;
  * the recurrent (decode) call applies the same gate to the same raw logits
    as the chunked call ([K3-NOTES]: both paths share state semantics);
  * a packed batch restarts the state at every sequence from that
    sequence's initial state; an empty sequence returns its initial state.

Functions:
  gate_log_decay, beta_of           -- the two activations
  recurrence                        -- the oracle proper (delta form of [K3-NOTES])
  recurrence_dplr                   -- the three-step DPLR form of [K3-ATTN §2.2]
  recurrence_matrix                 -- the explicit d_k x d_k transition of [LA-KDA §5.2]
  chunkwise                         -- the chunked reformulation of [LA-KDA §7]
                                       extended with the decay (derivation in the
                                       design notes); exposes its intermediates
  packed                            -- loops `recurrence` over a cu_seqlens batch
  decode_step, replay_fold,
  verify_window                     -- the recurrent call, and the replay and verify
                                       passes over a draft window
  recurrence_dplr_general           -- the diagonal-plus-low-rank update with its own
                                       low-rank pair (a, b) and write key
  chunkwise_dplr, decode_step_dplr  -- its chunked form with four C x C matrices, and
                                       its single-token step
  short_conv, silu, l2norm,
  rmsnorm_gated, fused_forward      -- the layer around the core ([LA-KDA §5.3, §5.5]):
                                       causal short convolution, Swish, L2Norm before,
                                       Sigmoid(gate) * RMSNorm after
All arithmetic is float64.  Inputs are converted to float64 exactly as given
(bf16 tensors are first widened, so the oracle sees the same rounded values
the GPU sees); nothing is rounded internally.
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0  # lower bound of log(alpha) [LA-KDA §5.4]


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):            # torch tensor -> float64 numpy, exact widening
        x = x.detach().to("cpu")
        if x.dtype.is_floating_point:
            x = x.double()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def logistic(x):
    """sigma(x) = 1 / (1 + e^{-x}), evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def gate_log_decay(z, A_h):
    """g = log(alpha) = g_min * sigmoid(exp(A_h) * z), per channel.

    [LA-KDA §5.4]: the decay map is a scaled sigmoid bounded below by g_min=-5,
    so alpha lies in (e^-5, 1).  `A_h` broadcasts against the head axis of z
    (z [..., H, d_k], A_h [H]).
    """
    z = _f64(z)
    a = np.exp(_f64(A_h))[..., :, None]
    return G_MIN * logistic(a * z)


def beta_of(b):
    """beta = sigmoid(b), the write strength [LA-KDA §5.3], [K3-ATTN §2.3]."""
    return logistic(_f64(b))


def recurrence(q, k, v, z, b, A, h0=None, erase=True, decay=True):
    """Token-by-token KDA over one sequence, all heads at once.

    q, k: [T, H, d_k]; v: [T, H, d_v]; z: [T, H, d_k]; b: [T, H]; A: [H];
    h0: [H, d_k, d_v] or None (zeros).  Returns (o [T, H, d_v], S [H, d_k, d_v]).

    Each step follows the update of [K3-NOTES]: the decayed state
    S~ = Diag(alpha_t) S_{t-1}; the prediction v^ = S~^T k_t; the correction
    delta = beta_t (v_t - v^); S_t = S~ + k_t delta^T; o_t = S_t^T q_t.
    The two switches give the other rows of the family table in [LA-KDA §4]:
    erase=False replaces the correction by plain accumulation,
    S_t = S~ + beta_t k_t v_t^T (gated linear attention, here with the write
    strength beta; the table's row is beta = 1), and decay=False sets
    alpha = 1 (DeltaNet); with both off it is linear attention.  z and A are
    not read when decay=False.
    """
    q, k, v, b = map(_f64, (q, k, v, b))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    if decay:
        alpha = np.exp(gate_log_decay(_f64(z), _f64(A)))   # [T, H, d_k]
    else:
        alpha = np.ones((T, H, dk))
    beta = beta_of(b)                             # [T, H]
    for t in range(T):
        S = alpha[t][:, :, None] * S                          # decay
        if erase:
            v_hat = np.einsum("hkv,hk->hv", S, k[t])          # read at key k_t
            delta = beta[t][:, None] * (v[t] - v_hat)         # error, scaled
            S = S + k[t][:, :, None] * delta[:, None, :]      # erase + write
        else:
            S = S + beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, q[t])               # read with q_t
    return o, S


def recurrence_dplr(q, k, v, z, b, A, h0=None):
    """The same recurrence written as the three DPLR steps of [K3-ATTN §2.2]:
    S' = Diag(alpha) S; S'' = S' - beta k (k^T S'); S = S'' + beta k v^T."""
    q, k, v, z, b, A = map(_f64, (q, k, v, z, b, A))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    alpha = np.exp(gate_log_decay(z, A))
    beta = beta_of(b)
    for t in range(T):
        S1 = alpha[t][:, :, None] * S
        kS = np.einsum("hk,hkv->hv", k[t], S1)
        S2 = S1 - beta[t][:, None, None] * k[t][:, :, None] * kS[:, None, :]
        S = S2 + beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, q[t])
    return o, S


def recurrence_matrix(q, k, v, z, b, A, h0=None):
    """The recurrence with the transition formed explicitly as a d_k x d_k matrix,
    S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T  [LA-KDA §5.2].
    Cost O(d_k^2 d_v) per token; meant for tiny d_k."""
    q, k, v, z, b, A = map(_f64, (q, k, v, z, b, A))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    alpha = np.exp(gate_log_decay(z, A))
    beta = beta_of(b)
    eye = np.eye(dk)
    for t in range(T):
        for h in range(H):
            kk = np.outer(k[t, h], k[t, h])
            M = (eye - beta[t, h] * kk) @ np.diag(alpha[t, h])
            S[h] = M @ S[h] + beta[t, h] * np.outer(k[t, h], v[t, h])
            o[t, h] = S[h].T @ q[t, h]
    return o, S


def chunkwise(q, k, v, z, b, A, h0=None, chunk=16, keep=False):
    """The chunked form of the recurrence, one sequence, all heads.

    [LA-KDA §7.1-§7.3] rewrites the recurrence chunk by chunk: inside a chunk
    the corrected values U solve a unit-lower-triangular system (the "UT
    transform"), everything else is matrix products, and only the state is
    carried from chunk to chunk.  The page defers the version with the decay
    to the paper; with G_i the in-chunk cumulative log-decay (inclusive of
    token i) and Gamma_i = exp(G_i), substituting the ansatz
    S_i = Diag(Gamma_i) S_0 + sum_{j<=i} Diag(Gamma_i / Gamma_j) k_j u_j^T into
    the recurrence gives, per chunk:
        A_kk[i,j] = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (j < i)
        A_qk[i,j] =        sum_c q_ic k_jc e^{G_ic - G_jc}   (j <= i)
        T  = (I + A_kk)^{-1} Diag(beta);  W = T (K . Gamma);  U = T V
        V~ = U - W S_0
        O  = (Q . Gamma) S_0 + A_qk V~
        S_C = Diag(Gamma_C) S_0 + (K . e^{G_C - G})^T V~
    With alpha = 1 these are exactly the equations printed in [LA-KDA §7.3].
    A partial last chunk is just a shorter chunk.  The triangular system is
    solved with numpy's dense solver.  With keep=True the per-chunk
    intermediates are returned in a list of dicts (for stage-level checks).
    """
    q, k, v, z, b, A = map(_f64, (q, k, v, z, b, A))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    g_all = gate_log_decay(z, A)                  # [T, H, d_k]
    beta_all = beta_of(b)                         # [T, H]
    inter = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        n = c1 - c0
        rec = {}
        for h in range(H):
            Q, K, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
            beta = beta_all[c0:c1, h]
            G = np.cumsum(g_all[c0:c1, h], axis=0)            # [n, d_k]
            # decay factor e^{G_ic - G_jc}, needed only for j <= i
            D = np.zeros((n, n, dk))
            for i in range(n):
                D[i, : i + 1] = np.exp(G[i][None, :] - G[: i + 1])
            Akk = np.einsum("ic,jc,ijc->ij", K, K, D) * beta[:, None]
            Akk = np.tril(Akk, -1)
            Aqk = np.tril(np.einsum("ic,jc,ijc->ij", Q, K, D))
            Tm = np.linalg.solve(np.eye(n) + Akk, np.diag(beta))
            Gam = np.exp(G)
            W = Tm @ (K * Gam)
            U = Tm @ V
            S0 = S[h].copy()
            Vt = U - W @ S0
            o[c0:c1, h] = (Q * Gam) @ S0 + Aqk @ Vt
            Kbar = K * np.exp(G[-1][None, :] - G)
            S[h] = np.exp(G[-1])[:, None] * S0 + Kbar.T @ Vt
            if keep:
                rec[h] = dict(G=G, beta=beta, Akk=Akk, Aqk=Aqk, T=Tm, W=W, U=U,
                              S0=S0, Vt=Vt, Kbar=Kbar, gammaC=np.exp(G[-1]))
        if keep:
            inter.append(rec)
    if keep:
        return o, S, inter
    return o, S


def recurrence_dplr_general(q, k, v, a, bv, z, A, h0=None):
    """Diagonal-plus-low-rank update with its own low-rank pair, one sequence,
    all heads: the three steps of [K3-ATTN §2.2] with the rank-1 correction
    and the write no longer tied to one key,
        S'  = Diag(alpha_t) S_{t-1}
        S'' = S' + a_t (b_t^T S')
        S_t = S'' + k_t v_t^T,          o_t = S_t^T q_t.
    KDA is the case a = -beta k, b = k with write key beta k ([K3-ATTN §2.2]
    binds the diagonal and low-rank terms to the same k).  alpha is the KDA
    gate of z and A ([LA-KDA §5.4]).
    q, k, a, bv, z: [T, H, d_k]; v: [T, H, d_v]; A: [H]; h0: [H, d_k, d_v] or None.
    Returns (o [T, H, d_v], S [H, d_k, d_v])."""
    q, k, v, a, bv, z, A = map(_f64, (q, k, v, a, bv, z, A))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    alpha = np.exp(gate_log_decay(z, A))
    for t in range(T):
        S1 = alpha[t][:, :, None] * S
        w = np.einsum("hk,hkv->hv", bv[t], S1)                   # b^T S'
        S = S1 + a[t][:, :, None] * w[:, None, :] + k[t][:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, q[t])
    return o, S


def chunkwise_dplr(q, k, v, a, bv, z, A, h0=None, chunk=16, keep=False):
    """The chunked form of `recurrence_dplr_general`, one sequence, all heads.

    With the unknowns x_i = S'_i^T b_i (the low-rank read of each token) the
    ansatz S_i = Diag(Gamma_i) S_0 + sum_{j<=i} Diag(Gamma_i / Gamma_j)
    (a_j x_j^T + k_j v_j^T) solves the recurrence, where G is the in-chunk
    inclusive cumulative log-decay and Gamma = e^G.  Per chunk, with
    e_ij = e^{G_i - G_j} per channel:
        A_ba[i,j] = sum_c b_ic a_jc e_ijc  (j < i)    A_bk[i,j] = sum_c b_ic k_jc e_ijc  (j < i)
        A_qa[i,j] = sum_c q_ic a_jc e_ijc  (j <= i)   A_qk[i,j] = sum_c q_ic k_jc e_ijc  (j <= i)
        T = (I - A_ba)^{-1};  Wb = T (B . Gamma);  Ub = T A_bk V
        X = Wb S_0 + Ub
        O = (Q . Gamma) S_0 + A_qa X + A_qk V
        S_C = Diag(Gamma_C) S_0 + (A . e^{G_C - G})^T X + (K . e^{G_C - G})^T V
    These are the four chunk matrices of the general form; when a and the
    write key are both multiples of b (KDA) the pairs coincide up to row
    and column scales and two remain ([K3-ATTN §2.2]).  The derivation is the
    one of `chunkwise` with a second low-rank vector.  keep=True also
    returns the per-chunk intermediates."""
    q, k, v, a, bv, z, A = map(_f64, (q, k, v, a, bv, z, A))
    T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0).copy()
    o = np.zeros((T, H, dv))
    g_all = gate_log_decay(z, A)
    inter = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        n = c1 - c0
        rec = {}
        for h in range(H):
            Q, K, V, Av, Bv = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], a[c0:c1, h], bv[c0:c1, h]
            G = np.cumsum(g_all[c0:c1, h], axis=0)
            D = np.zeros((n, n, dk))
            for i in range(n):
                D[i, : i + 1] = np.exp(G[i][None, :] - G[: i + 1])
            Aba = np.tril(np.einsum("ic,jc,ijc->ij", Bv, Av, D), -1)
            Abk = np.tril(np.einsum("ic,jc,ijc->ij", Bv, K, D), -1)
            Aqa = np.tril(np.einsum("ic,jc,ijc->ij", Q, Av, D))
            Aqk = np.tril(np.einsum("ic,jc,ijc->ij", Q, K, D))
            Tm = np.linalg.inv(np.eye(n) - Aba)
            Gam = np.exp(G)
            Wb = Tm @ (Bv * Gam)
            Ub = Tm @ (Abk @ V)
            S0 = S[h].copy()
            X = Wb @ S0 + Ub
            o[c0:c1, h] = (Q * Gam) @ S0 + Aqa @ X + Aqk @ V
            dec = np.exp(G[-1][None, :] - G)
            S[h] = np.exp(G[-1])[:, None] * S0 + (Av * dec).T @ X + (K * dec).T @ V
            if keep:
                rec[h] = dict(G=G, Aba=Aba, Abk=Abk, Aqa=Aqa, Aqk=Aqk, T=Tm, Wb=Wb, Ub=Ub,
                              S0=S0, X=X, gammaC=np.exp(G[-1]))
        if keep:
            inter.append(rec)
    if keep:
        return o, S, inter
    return o, S


def decode_step_dplr(q, k, v, a, bv, z, A, state):
    """One token of `recurrence_dplr_general` for a batch of sequences:
    q, k, a, bv, z [N, H, d_k]; v [N, H, d_v]; state [N, H, d_k, d_v].
    Returns (o [N, H, d_v], new state)."""
    q, k, v, a, bv, z, A, state = map(_f64, (q, k, v, a, bv, z, A, state))
    N, H, dk = q.shape
    dv = v.shape[2]
    r = lambda x: x.reshape(1, N * H, x.shape[-1])
    o, S = recurrence_dplr_general(r(q), r(k), r(v), r(a), r(bv), r(z), np.tile(A, N),
                                   state.reshape(N * H, dk, dv))
    return o.reshape(N, H, dv), S.reshape(N, H, dk, dv)


def _drop_batch(x, nd):
    x = _f64(x)
    return x[0] if x.ndim == nd + 1 else x


def packed(q, k, v, z, b, A, h0, cu_seqlens, fn=recurrence, **kw):
    """Run `fn` over every sequence of a packed batch.

    q, k, v, z: [1, T, H, d] (or [T, H, d]); b: [1, T, H]; cu_seqlens: N+1
    offsets; h0: [N, H, d_k, d_v] or None.  Returns (o [T, H, d_v],
    S [N, H, d_k, d_v]).  Each sequence starts from its own initial state.
    """
    q, k, v, z = (_drop_batch(x, 3) for x in (q, k, v, z))
    b = _drop_batch(b, 2)
    cu = [int(x) for x in _f64(cu_seqlens)]
    N = len(cu) - 1
    H, dk, dv = k.shape[1], k.shape[2], v.shape[2]
    o = np.zeros((k.shape[0], H, dv))
    S = np.zeros((N, H, dk, dv))
    h0 = None if h0 is None else _f64(h0)
    for s in range(N):
        a, e = cu[s], cu[s + 1]
        init = None if h0 is None else h0[s]
        if e == a:
            S[s] = 0.0 if init is None else init
            continue
        o_s, S_s = fn(q[a:e], k[a:e], v[a:e], z[a:e], b[a:e], A, init, **kw)
        o[a:e] = o_s
        S[s] = S_s
    return o, S


def decode_step(q, k, v, z, b, A, state, **kw):
    """One single-token step for a batch of sequences (the recurrent call of
    [K3-NOTES]): q, k [N, H, d_k]; v [N, H, d_v]; z [N, H, d_k]; b [N, H];
    state [N, H, d_k, d_v].  Returns (o [N, H, d_v], new state); the input
    state is not modified.  Keyword switches go to `recurrence`."""
    q, k, v, b, state = map(_f64, (q, k, v, b, state))
    N, H, dk = q.shape
    dv = v.shape[2]
    zz = None if z is None else _f64(z).reshape(1, N * H, dk)
    AA = None if A is None else np.tile(_f64(A), N)
    # every (sequence, head) pair is an independent one-token recurrence
    o, S = recurrence(q.reshape(1, N * H, dk), k.reshape(1, N * H, dk),
                      v.reshape(1, N * H, dv), zz, b.reshape(1, N * H), AA,
                      state.reshape(N * H, dk, dv), **kw)
    return o.reshape(N, H, dv), S.reshape(N, H, dk, dv)


def replay_fold(k, v, z, b, A, state, n_accept):
    """The replay of [K3-ATTN §6.2] (ReplaySSM): from a checkpoint state,
    advance sequence s by the first n_accept[s] tokens of its stored window
    (k, z [N, W, H, d_k]; v [N, W, H, d_v]; b [N, W, H]); counts outside
    [0, W] are clamped.  The state after a token does not depend on q, so the
    window carries none.  Returns the new state [N, H, d_k, d_v]; the input is
    not modified."""
    k, v, z, b, A, state = map(_f64, (k, v, z, b, A, state))
    N, W, H, dk = k.shape
    out = state.copy()
    for s in range(N):
        n = min(max(int(n_accept[s]), 0), W)
        if n == 0:
            continue
        # the accepted prefix is a short sequence of its own, started from the checkpoint
        _, out[s] = recurrence(np.zeros_like(k[s, :n]), k[s, :n], v[s, :n], z[s, :n], b[s, :n], A,
                               state[s])
    return out


def verify_window(q, k, v, z, b, A, state):
    """The verify pass of [K3-ATTN §6.2] (ReplaySSM): from each sequence's
    checkpoint state, the outputs of every token of its draft window
    (q, k, z [N, W, H, d_k]; v [N, W, H, d_v]; b [N, W, H]), the state itself
    left as it is (the accepted prefix is committed later by `replay_fold`).
    Returns o [N, W, H, d_v]."""
    q, k, v, z, b, A, state = map(_f64, (q, k, v, z, b, A, state))
    N, W, H, dk = k.shape
    o = np.zeros((N, W, H, v.shape[-1]))
    for s in range(N):
        o[s], _ = recurrence(q[s], k[s], v[s], z[s], b[s], A, state[s])
    return o


# ------------------------------------------------------------ around the core
# The steps either side of the recurrence that act on one token-head row:
# [LA-KDA §5.3] q, k = L2Norm(Swish(ShortConv(W x))), v = Swish(ShortConv(W x));
# [LA-KDA §5.5] y = W_o [Sigmoid(W_g x) * RMSNorm(o)], the RMSNorm per head
# ([K3-ATTN §2.3]).  The projections W are outside: these functions take their
# outputs.  Readings where the pages are silent: the convolution has no bias,
# its four taps are ordered oldest first; Swish has unit slope; L2Norm and
# RMSNorm take an additive epsilon under the square root; RMSNorm has one
# weight per channel shared by the heads.

CONV_TAPS = 4   # depthwise causal convolution, kernel size 4 [K3-ATTN §2.3]


def short_conv(x, w, state=None):
    """Depthwise causal convolution over time: y_t = sum_j w[..., j] x_{t-3+j}
    (j = 0..3, taps oldest first, no bias).  x [T, H, d]; w [H, d, 4]; state
    [3, H, d] holds the three inputs before x[0] (None: zeros, a sequence
    start).  Returns (y [T, H, d], the state after x: its last three inputs)."""
    x, w = _f64(x), _f64(w)
    T, H, d = x.shape
    hist = np.zeros((CONV_TAPS - 1, H, d)) if state is None else _f64(state)
    xs = np.concatenate([hist, x], axis=0)
    y = np.zeros((T, H, d))
    for t in range(T):
        for j in range(CONV_TAPS):
            y[t] += w[..., j] * xs[t + j]
    return y, xs[len(xs) - (CONV_TAPS - 1):].copy()


def silu(x):
    """Swish with unit slope: x * sigma(x)."""
    x = _f64(x)
    return x * logistic(x)


def l2norm(x, eps):
    """x / sqrt(sum_c x_c^2 + eps) over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def rmsnorm_gated(o, g, w, eps):
    """sigma(g) * RMSNorm(o): RMSNorm over one head's d_v channels,
    o / sqrt(mean_c o_c^2 + eps) * w, then the output gate sigma(g)."""
    o, g, w = _f64(o), _f64(g), _f64(w)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return logistic(g) * r * w


def fused_forward(q_in, k_in, v_in, conv_w, z, b, A, gate, norm_w, h0=None, conv_state=None,
                  l2_eps=1e-6, rms_eps=1e-5, with_o=False):
    """One sequence through the whole KDA layer between its projections:
    q, k = L2Norm(Swish(ShortConv(.))), v = Swish(ShortConv(.)), the
    recurrence, then Sigmoid(gate) * RMSNorm(o).
    q_in, k_in, v_in, gate [T, H, d]; conv_w [3, H, d, 4] (q, k, v taps);
    conv_state [3, 3, H, d] or None (q, k, v histories); norm_w [d].
    Returns (y [T, H, d], S [H, d, d], conv_state_out [3, 3, H, d]), and with
    with_o also the core's output o [T, H, d] before the gate."""
    conv_w = _f64(conv_w)
    cs = [None] * 3 if conv_state is None else [_f64(conv_state)[i] for i in range(3)]
    qc, sq = short_conv(q_in, conv_w[0], cs[0])
    kc, sk = short_conv(k_in, conv_w[1], cs[1])
    vc, sv = short_conv(v_in, conv_w[2], cs[2])
    q = l2norm(silu(qc), l2_eps)
    k = l2norm(silu(kc), l2_eps)
    v = silu(vc)
    o, S = recurrence(q, k, v, z, b, A, h0)
    y = rmsnorm_gated(o, gate, norm_w, rms_eps)
    cs_out = np.stack([sq, sk, sv])
    return (y, S, cs_out, o) if with_o else (y, S, cs_out)
