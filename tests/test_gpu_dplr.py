"""GPU parity of the general DPLR entry points against the oracle's
`recurrence_dplr_general` (pinned on the CPU: it reduces to KDA, matches the
explicit-matrix form, the GLA closed form without its low-rank term, and
the four-matrix chunked form).

The update generalises the three steps of [K3-ATTN §2.2] with its own
low-rank pair (a, b) and write key k: S' = Diag(alpha) S,
S'' = S' + a (b^T S'), S = S'' + k v^T, o = S^T q.
Page tags: [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构".
"""
import pytest
import torch

import kda_inputs as KI
import oracle
from kda_testutil import report, TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_77_amd as m
    m.lib()
    return m


def _report(tag, **errs):
    report("dplr", tag, **errs)


def _dev(d):
    keys = ("q", "k", "v", "la", "lb", "z", "A", "h0", "cu_seqlens")
    return {x: (d[x].cuda().contiguous() if d.get(x) is not None else None) for x in keys}


def _gpu(kda, g, chunk):
    return kda.kda_dplr_chunk_fwd(g["q"], g["k"], g["v"], g["la"], g["lb"], g["z"], g["A"],
                                  initial_state=g["h0"], cu_seqlens=g["cu_seqlens"],
                                  chunk_size=chunk)


def _oracle(d, bi, sl, h0, heads=None):
    hs = slice(None) if heads is None else list(heads)
    pick = lambda x: x[bi, sl][:, hs].cpu()   # noqa: E731
    return oracle.recurrence_dplr_general(pick(d["q"]), pick(d["k"]), pick(d["v"]),
                                          pick(d["la"]), pick(d["lb"]), pick(d["z"]),
                                          d["A"].cpu()[hs], None if h0 is None else h0.cpu()[hs])


@pytest.mark.parametrize("dtype,dk,chunk,B,T,H", [("fp32", 16, 16, 2, 100, 2),
                                                   ("fp32", 64, 64, 1, 150, 2),
                                                   ("bf16", 16, 16, 1, 90, 3),
                                                   ("bf16", 128, 64, 2, 300, 3)])
def test_dplr_prefill_vs_oracle(kda, dtype, dk, chunk, B, T, H):
    case = KI.PrefillCase("dplr", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=B, T=T,
                          zero_h0=False)
    d = KI.make_dplr(case, seed=51)
    o, hT = _gpu(kda, _dev(d), chunk)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    for bi in range(B):
        ro, rS = _oracle(d, bi, slice(0, T), d["h0"][bi])
        eo, eS = rel_err(o[bi], ro), rel_err(hT[bi], rS)
        _report(f"{dtype} d={dk} C={chunk} B={B} T={T} seq {bi}", o=eo, hT=eS)
        assert eo <= tol and eS <= tol


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_dplr_packed_vs_oracle(kda, dtype, dk, chunk):
    """Packed batch with an empty sequence, a one-token sequence and ragged
    tails.  The metric is the per-tensor one of every parity test: the
    packed o (and hT) is one tensor, so each sequence's error is taken
    relative to the largest reference value of the whole tensor (a one-token
    output is the small product (q . k) v, whose own maximum would measure
    the bf16 rounding of q and k rather than the path; see kda_testutil)."""
    case = KI.PrefillCase("dplrvar", H=2, dk=dk, dv=dk, chunk=chunk, dtype=dtype, n_seqs=4,
                          len_lo=1, len_hi=200, zero_h0=False)
    lens = [130, 0, 1, 77]
    d = KI.make_dplr(case, seed=52, lengths=lens)
    o, hT = _gpu(kda, _dev(d), chunk)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    cu = [int(x) for x in d["cu_seqlens"].tolist()]
    refs = {s: _oracle(d, 0, slice(cu[s], cu[s + 1]), d["h0"][s]) for s, n in enumerate(lens) if n}
    o_scale = max(float(abs(r[0]).max()) for r in refs.values())
    s_scale = max(float(abs(r[1]).max()) for r in refs.values())
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s].cpu(), d["h0"][s])
            continue
        ro, rS = refs[s]
        eo = rel_err(o[0, cu[s]:cu[s + 1]], ro, scale=o_scale)
        eS = rel_err(hT[s], rS, scale=s_scale)
        _report(f"packed {dtype} seq {s} (len {n}), per tensor", o=eo, hT=eS,
                o_own_max=rel_err(o[0, cu[s]:cu[s + 1]], ro))
        assert eo <= tol and eS <= tol


def test_dplr_without_initial_state_and_split_resume(kda):
    """No h0 (zeros), and a run split at a chunk-unaligned point resumes from
    the returned state to the same result."""
    case = KI.PrefillCase("dplrres", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=250,
                          zero_h0=True)
    d = KI.make_dplr(case, seed=53)
    g = _dev(d)
    o, hT = _gpu(kda, g, 64)
    cut = 101
    part = lambda x, sl: x[:, sl].contiguous()   # noqa: E731
    g1 = {x: (part(g[x], slice(0, cut)) if x in ("q", "k", "v", "la", "lb", "z") else g[x])
          for x in g}
    g2 = {x: (part(g[x], slice(cut, None)) if x in ("q", "k", "v", "la", "lb", "z") else g[x])
          for x in g}
    o1, h1 = _gpu(kda, g1, 64)
    g2["h0"] = h1
    o2, h2 = _gpu(kda, g2, 64)
    torch.cuda.synchronize()
    ro, rS = _oracle(d, 0, slice(0, 250), None)
    e = dict(o=rel_err(o[0], ro), hT=rel_err(hT[0], rS),
             o_split=rel_err(torch.cat([o1, o2], 1)[0], ro), hT_split=rel_err(h2[0], rS))
    _report("no h0 / split at 101", **e)
    assert all(x <= TOL_BF16 for x in e.values())


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 32)])
def test_dplr_decode_vs_oracle_and_prefill(kda, dtype, dk):
    """Each decode step against the oracle's step, and the steps together
    against a prefill over the same tokens."""
    N, H, steps = 5, 3, 9
    case = KI.PrefillCase("dplrdec", H=H, dk=dk, dv=dk, chunk=16 if dk < 128 else 64,
                          dtype=dtype, B=N, T=steps, zero_h0=False)
    d = KI.make_dplr(case, seed=54)
    g = _dev(d)
    st = g["h0"].clone()
    S = d["h0"]
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    outs = []
    for t in range(steps):
        tk = lambda x: g[x][:, t].contiguous()   # noqa: E731
        outs.append(kda.kda_dplr_recurrent_step(tk("q"), tk("k"), tk("v"), tk("la"), tk("lb"),
                                                tk("z"), g["A"], st))
        hk = lambda x: d[x][:, t]                # noqa: E731
        ro, S = oracle.decode_step_dplr(hk("q"), hk("k"), hk("v"), hk("la"), hk("lb"), hk("z"),
                                        d["A"], S)
        torch.cuda.synchronize()
        assert rel_err(outs[-1], ro) <= tol
    assert rel_err(st, S) <= tol
    op, hp = _gpu(kda, g, case.chunk)
    torch.cuda.synchronize()
    e1, e2 = rel_err(torch.stack(outs, 1), op), rel_err(st, hp)
    _report(f"decode {dtype} d={dk} vs prefill", o=e1, state=e2)
    assert e1 <= tol and e2 <= tol


@pytest.mark.parametrize("B,T,H,heads", [(1, 8192, 1, [0]), (3, 1500, 5, [0, 4]),
                                         (1, 4096, 40, [7, 39])])
def test_dplr_segment_layouts_vs_oracle(kda, B, T, H, heads):
    """bf16, d = 128, C = 64 runs the MFMA path: the sequence is cut into about
    256 / H segments of at least 16 chunks, whose transitions (with the folded
    constant Cs) are composed in fp32; one head over 9 segments, several short
    sequences, and 40 heads, each against the oracle."""
    case = KI.PrefillCase("dplrseg", H=H, dk=128, dv=128, chunk=64, dtype="bf16", B=B, T=T,
                          zero_h0=False)
    d = KI.make_dplr(case, seed=55)
    o, hT = _gpu(kda, _dev(d), 64)
    torch.cuda.synchronize()
    for bi in range(B):
        ro, rS = _oracle(d, bi, slice(0, T), d["h0"][bi], heads=heads)
        eo, eS = rel_err(o[bi][:, heads], ro), rel_err(hT[bi][heads], rS)
        _report(f"segments B={B} T={T} H={H} seq {bi} heads {heads}", o=eo, hT=eS)
        assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.parametrize("case_id", range(6))
def test_dplr_random_packed_layouts(kda, case_id):
    """Seeded random packed batches of the general update: length mixes with
    empty, one-token and multi-chunk sequences, several head counts, on the
    MFMA path and the fp32 path; the first and last head of every sequence
    against the oracle (per-tensor metric)."""
    import random
    rng = random.Random(9000 + case_id)
    dk, chunk, dtype = ((128, 64, "bf16") if case_id % 3 != 2
                        else (rng.choice([16, 32]), rng.choice([16, 64]), rng.choice(["fp32", "bf16"])))
    H = rng.choice([1, 2, 5, 12, 33])
    lens = [rng.choice([0, 1, rng.randint(1, 200), rng.randint(1, 2000)])
            for _ in range(rng.randint(1, 6))]
    budget = 5000 if dk == 128 else 2000
    if sum(lens) > budget:
        lens = [n * budget // sum(lens) for n in lens]
    if sum(lens) == 0:
        lens[-1] = 1
    case = KI.PrefillCase("dplrrand", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype, zero_h0=False)
    d = KI.make_dplr(case, seed=9100 + case_id, lengths=lens)
    o, hT = _gpu(kda, _dev(d), chunk)
    torch.cuda.synchronize()
    heads = sorted({0, H - 1})
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    cu = [int(x) for x in d["cu_seqlens"].tolist()]
    refs = {s: _oracle(d, 0, slice(cu[s], cu[s + 1]), d["h0"][s], heads=heads)
            for s, n in enumerate(lens) if n}
    o_scale = max(float(abs(r[0]).max()) for r in refs.values())
    s_scale = max(float(abs(r[1]).max()) for r in refs.values())
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s].cpu(), d["h0"][s])
            continue
        ro, rS = refs[s]
        eo = rel_err(o[0, cu[s]:cu[s + 1]][:, heads], ro, scale=o_scale)
        eS = rel_err(hT[s][heads], rS, scale=s_scale)
        assert eo <= tol and eS <= tol, (case_id, dk, chunk, dtype, H, lens, s, eo, eS)
    _report(f"random layout {case_id}: d={dk} C={chunk} {dtype} H={H} lens={lens}", ok=0.0)


def test_dplr_long_1m_column_permutation_and_scaling(kda):
    """Every output and final state of the general DPLR update on the
    1M-token shapes, through two properties that hold at any size: value
    columns evolve independently (permuting the d_v columns of v and h0
    permutes those of o and the final state), and (o, hT) is linear in
    (v, h0) (doubling both doubles both, exactly in floating point).  Bar:
    1e-6 of the largest value (only flushed denormals may differ)."""
    case = KI.CONFIGS["long_1m"]
    d = KI.make_dplr(case, device="cuda", seed=0)
    d["cu_seqlens"] = None
    o, hT = _gpu(kda, d, 64)
    perm = torch.randperm(case.dv, generator=torch.Generator().manual_seed(6)).cuda()
    dp = dict(d, v=d["v"][..., perm].contiguous(), h0=d["h0"][..., perm].contiguous())
    op, hp = _gpu(kda, dp, 64)
    torch.cuda.synchronize()
    omax, smax = o.float().abs().max(), hT.abs().max()
    e_o = float((op.float() - o[..., perm].float()).abs().max() / omax)
    e_s = float((hp - hT[..., perm]).abs().max() / smax)
    del dp, op, hp
    d2 = dict(d, v=d["v"] * 2, h0=d["h0"] * 2)
    o2, h2 = _gpu(kda, d2, 64)
    torch.cuda.synchronize()
    e2_o = float((o2.float() - 2 * o.float()).abs().max() / omax)
    e2_s = float((h2 - 2 * hT).abs().max() / smax)
    _report("long_1m permuted columns", o=e_o, hT=e_s)
    _report("long_1m doubled v, h0", o=e2_o, hT=e2_s)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    assert max(e_o, e_s, e2_o, e2_s) <= 1e-6
