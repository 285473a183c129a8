"""GPU parity of the family modes of the prefill and decode entry points
(the rows of the family table in [LA-KDA §4]): gated linear attention, where
the erase step is off, and DeltaNet, where alpha = 1.  Both are checked
against the oracle's switches (`recurrence(erase=False)` and
`recurrence(decay=False)`, pinned on the CPU), on the fp32 path and on the
MFMA path, with ragged tails and a packed batch, and decode against prefill
in each mode.

Page tags: [LA-KDA] "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制",
blog-3d3.pages.dev/posts/150.
"""
import pytest
import torch

import kda_inputs as KI
import oracle
from kda_testutil import report, TOL_BF16, TOL_F32, rel_err, to_dev

pytestmark = pytest.mark.gpu

SWITCH = {"gla": dict(erase=False), "deltanet": dict(decay=False)}


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_77_amd as m
    m.lib()
    return m


def _report(tag, **errs):
    report("modes", tag, **errs)


def _gpu(kda, d, mode, chunk):
    # DeltaNet reads no gate logits: pass none, so the NULL path is the one tested
    g, A = (None, None) if mode == "deltanet" else (d["z"], d["A"])
    return kda.kda_chunk_fwd_mode(d["q"], d["k"], d["v"], g, d["b"], A, mode,
                                  initial_state=d.get("h0"), cu_seqlens=d.get("cu_seqlens"),
                                  chunk_size=chunk)


def _oracle_seq(inp, mode, bi, sl, heads=None):
    hs = slice(None) if heads is None else list(heads)
    pick = lambda x: x[bi, sl][:, hs].cpu()   # noqa: E731
    h0 = inp.get("h0")
    return oracle.recurrence(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["z"]),
                             inp["b"][bi, sl][:, hs].cpu(), inp["A"].cpu()[hs],
                             None if h0 is None else h0[bi].cpu()[hs], **SWITCH[mode])


@pytest.mark.parametrize("mode", ["gla", "deltanet"])
@pytest.mark.parametrize("dtype,dk,chunk,B,T,H", [("fp32", 16, 16, 2, 100, 2),
                                                   ("fp32", 64, 64, 1, 150, 2),
                                                   ("bf16", 128, 64, 2, 300, 3)])
def test_prefill_mode_vs_oracle(kda, mode, dtype, dk, chunk, B, T, H):
    case = KI.PrefillCase("mode", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=B, T=T,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=31)
    o, hT = _gpu(kda, to_dev(inp), mode, chunk)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    for bi in range(B):
        ro, rS = _oracle_seq(inp, mode, bi, slice(0, T))
        eo, eS = rel_err(o[bi], ro), rel_err(hT[bi], rS)
        _report(f"{mode} {dtype} d={dk} C={chunk} B={B} T={T} seq {bi}", o=eo, hT=eS)
        assert eo <= tol and eS <= tol


@pytest.mark.parametrize("mode", ["gla", "deltanet"])
@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_packed_mode_vs_oracle(kda, mode, dtype, dk, chunk):
    """A packed batch with an empty sequence, a one-token sequence and ragged
    chunk tails; errors per sequence relative to the packed tensor's largest
    reference value (the per-tensor metric, see kda_testutil)."""
    case = KI.PrefillCase("modevar", H=2, dk=dk, dv=dk, chunk=chunk, dtype=dtype, n_seqs=4,
                          len_lo=1, len_hi=200, zero_h0=False)
    lens = [130, 0, 1, 77]
    inp = KI.make_prefill(case, seed=32, lengths=lens)
    o, hT = _gpu(kda, to_dev(inp), mode, chunk)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    cu = [int(x) for x in inp["cu_seqlens"].tolist()]
    refs = {}
    for s, n in enumerate(lens):
        if n:
            pick = lambda x: x[0, cu[s]:cu[s + 1]].cpu()   # noqa: E731
            refs[s] = oracle.recurrence(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                        pick(inp["z"]), inp["b"][0, cu[s]:cu[s + 1]], inp["A"],
                                        inp["h0"][s], **SWITCH[mode])
    o_scale = max(float(abs(r[0]).max()) for r in refs.values())
    s_scale = max(float(abs(r[1]).max()) for r in refs.values())
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s].cpu(), inp["h0"][s])
            continue
        ro, rS = refs[s]
        eo = rel_err(o[0, cu[s]:cu[s + 1]], ro, scale=o_scale)
        eS = rel_err(hT[s], rS, scale=s_scale)
        _report(f"{mode} packed {dtype} seq {s} (len {n}), per tensor", o=eo, hT=eS,
                o_own_max=rel_err(o[0, cu[s]:cu[s + 1]], ro))
        assert eo <= tol and eS <= tol


def test_mode_kda_equals_plain_entry_point(kda):
    """KDA_MODE_KDA is exactly kda_chunk_fwd (same kernels, same bits)."""
    case = KI.PrefillCase("modekda", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=200,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=33))
    o1, h1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                               initial_state=d["h0"])
    o2, h2 = kda.kda_chunk_fwd_mode(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"], "kda",
                                    initial_state=d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("mode", ["gla", "deltanet"])
@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 32)])
def test_decode_mode_vs_oracle_and_prefill(kda, mode, dtype, dk):
    """Each decode step against the oracle's step; the steps together against
    a prefill over the same tokens in the same mode."""
    case = KI.DecodeCase("dmode", N=6, H=3, dk=dk, dv=dk, steps=9, dtype=dtype)
    run = KI.make_decode(case, seed=34)
    A = run["A"].cuda()
    st = run["state"].cuda().contiguous()
    st0 = st.clone()
    S = run["state"]
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    outs = []
    for s in run["steps"]:
        sd = to_dev(s)
        g, AA = (None, None) if mode == "deltanet" else (sd["z"], A)
        outs.append(kda.kda_recurrent_step_mode(sd["q"], sd["k"], sd["v"], g, sd["b"], AA, st,
                                                mode))
        ro, S = oracle.decode_step(s["q"], s["k"], s["v"], s["z"], s["b"], run["A"], S,
                                   **SWITCH[mode])
        torch.cuda.synchronize()
        assert rel_err(outs[-1], ro) <= tol
    assert rel_err(st, S) <= tol
    cat = lambda key: torch.stack([s[key] for s in run["steps"]], 1).cuda().contiguous()  # noqa: E731
    g, AA = (None, None) if mode == "deltanet" else (cat("z"), A)
    op, hp = kda.kda_chunk_fwd_mode(cat("q"), cat("k"), cat("v"), g, cat("b"), AA, mode,
                                    initial_state=st0, chunk_size=16 if dk < 128 else 64)
    torch.cuda.synchronize()
    e1, e2 = rel_err(torch.stack(outs, 1), op), rel_err(st, hp)
    _report(f"{mode} decode {dtype} d={dk} vs prefill", o=e1, state=e2)
    assert e1 <= tol and e2 <= tol


@pytest.mark.parametrize("mode", ["gla", "deltanet"])
def test_mode_long_1m_column_permutation_and_scaling(kda, mode):
    """Every output and final state of a family mode on the 1M-token
    workload, through two properties that hold at any size: permuting the d_v
    columns of v and h0 permutes those of o and the final state, and doubling
    (v, h0) doubles (o, hT), exactly in floating point.  Bar: 1e-6 of the
    largest value (only flushed denormals may differ)."""
    d = KI.make_prefill(KI.CONFIGS["long_1m"], device="cuda", seed=0)
    o, hT = _gpu(kda, d, mode, 64)
    perm = torch.randperm(d["dv"], generator=torch.Generator().manual_seed(7)).cuda()
    dp = dict(d, v=d["v"][..., perm].contiguous(), h0=d["h0"][..., perm].contiguous())
    op, hp = _gpu(kda, dp, mode, 64)
    torch.cuda.synchronize()
    omax, smax = o.float().abs().max(), hT.abs().max()
    e_o = float((op.float() - o[..., perm].float()).abs().max() / omax)
    e_s = float((hp - hT[..., perm]).abs().max() / smax)
    del dp, op, hp
    o2, h2 = _gpu(kda, dict(d, v=d["v"] * 2, h0=d["h0"] * 2), mode, 64)
    torch.cuda.synchronize()
    e2_o = float((o2.float() - 2 * o.float()).abs().max() / omax)
    e2_s = float((h2 - 2 * hT).abs().max() / smax)
    _report(f"{mode} long_1m permuted columns", o=e_o, hT=e_s)
    _report(f"{mode} long_1m doubled v, h0", o=e2_o, hT=e2_s)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    assert max(e_o, e_s, e2_o, e2_s) <= 1e-6
