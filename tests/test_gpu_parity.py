"""GPU parity of libkda against the fp64 oracle, through the C ABI binding.

Sizes: small cases span several 64-token chunks and 16-token sub-tiles with a
ragged tail; the named workloads run at full size and are checked on outputs
the oracle computes one (sequence, head) at a time, or through properties that
hold at any size (decode == prefill, packed == separate, determinism).
"""
import numpy as np
import pytest
import torch

import kda_inputs as KI
import oracle
from kda_testutil import report, TOL_BF16, TOL_F32, gpu_prefill, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu

BIG = 1.0e4


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_77_amd as m
    m.lib()   # raises if libkda.so is missing: no silent fallback
    return m


def _case(name, **over):
    import dataclasses
    return dataclasses.replace(KI.CONFIGS[name], **over)


def _report(tag, **errs):
    report("parity", tag, **errs)


# --------------------------------------------------------------- named configs

def test_tiny_fp32_config(kda):
    """B=1, H=2, T=64, d=16, C=16, fp32, A=0, zero state (the fp32 config)."""
    inp = KI.make_prefill(KI.CONFIGS["tiny_fp32"], seed=0)
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp)
    eo, eS = rel_err(o[0], ro), rel_err(hT[0], rS)
    _report("tiny_fp32", o=eo, hT=eS)
    assert eo <= TOL_F32 and eS <= TOL_F32


def test_prefill_4k_config(kda):
    """B=1, H=16, T=4096, d=128, C=64, bf16 (all heads, all tokens)."""
    inp = KI.make_prefill(KI.CONFIGS["prefill_4k"], seed=0)
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp)
    eo, eS = rel_err(o[0], ro), rel_err(hT[0], rS)
    _report("prefill_4k", o=eo, hT=eS)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def test_varlen_config_sampled(kda):
    """8 packed sequences (lengths U[512, 16384]), H=12, per-sequence states:
    three sampled (sequence, head) pairs against the oracle in full, and the
    packed call against separate per-sequence calls (bitwise)."""
    inp = KI.make_prefill(KI.CONFIGS["varlen_8"], seed=0)
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    rng = np.random.default_rng(0)
    for s, h in [(0, 0), (int(rng.integers(1, 8)), int(rng.integers(0, 12))), (7, 11)]:
        ro, rS = oracle_prefill(inp, heads=[h], seq=s)
        eo = rel_err(o[0, cu[s]:cu[s + 1], h], ro[:, 0])
        eS = rel_err(hT[s, h], rS[0])
        _report(f"varlen_8 seq {s} head {h}", o=eo, hT=eS)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    for s in (0, 5):
        a, e = cu[s], cu[s + 1]
        sub = {k: d[k] for k in ("A",)}
        sub.update(q=d["q"][:, a:e].contiguous(), k=d["k"][:, a:e].contiguous(),
                   v=d["v"][:, a:e].contiguous(), z=d["z"][:, a:e].contiguous(),
                   b=d["b"][:, a:e].contiguous(), h0=d["h0"][s:s + 1].contiguous(), chunk=64)
        o1, h1 = gpu_prefill(kda, sub)
        assert torch.equal(o1[0], o[0, a:e]) and torch.equal(h1[0], hT[s])


def test_long_1m_config_sampled(kda):
    """B=1, H=12, T=2^20 (inputs drawn on the device).  The first 32768
    outputs of two heads against the oracle, and the final state of a separate
    65536-token run against the oracle state there."""
    case = KI.CONFIGS["long_1m"]
    d = KI.make_prefill(case, device="cuda", seed=0)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    prefix = {k: (d[k][:, :32768].cpu() if k in ("q", "k", "v", "z", "b") else d[k])
              for k in ("q", "k", "v", "z", "b")}
    prefix.update(A=d["A"].cpu(), h0=d["h0"].cpu())
    heads = [0, 7]
    ro, _ = oracle_prefill(prefix, heads=heads)
    eo = rel_err(o[0, :32768][:, heads], ro)
    _report("long_1m o[:32768]", o=eo)
    assert eo <= TOL_BF16
    sub = {k: d[k][:, :65536].contiguous() for k in ("q", "k", "v", "z", "b")}
    sub.update(A=d["A"], h0=d["h0"], chunk=64)
    _, h64 = gpu_prefill(kda, sub)
    torch.cuda.synchronize()
    p64 = {k: sub[k].cpu() for k in ("q", "k", "v", "z", "b")}
    p64.update(A=d["A"].cpu(), h0=d["h0"].cpu())
    _, rS = oracle_prefill(p64, heads=heads)
    eS = rel_err(h64[0][heads], rS)
    _report("long_1m hT@65536", hT=eS)
    assert eS <= TOL_BF16


@pytest.mark.parametrize("name", ["long_1m", "varlen_8"])
def test_column_permutation_and_scaling(kda, name):
    """Properties that hold at any size, checked on every output of the
    1M-token and packed workloads: value columns evolve independently (permuting the d_v
    columns of v and h0 permutes those of o and of the final state), and
    (o, hT) is linear in (v, h0) (doubling both doubles both; a factor of two
    is exact in floating point).  Both hold to rounding-free precision on this
    path: the bar is 1e-6 of the largest value (denormals flushed to zero are
    the only allowed difference)."""
    case = KI.CONFIGS[name]
    d = KI.make_prefill(case, device="cuda", seed=0)
    o, hT = gpu_prefill(kda, d)
    perm = torch.randperm(case.dv, generator=torch.Generator().manual_seed(5)).cuda()
    dp = dict(d, v=d["v"][..., perm].contiguous(), h0=d["h0"][..., perm].contiguous())
    op, hp = gpu_prefill(kda, dp)
    torch.cuda.synchronize()
    omax, smax = o.float().abs().max(), hT.abs().max()
    e_o = float((op.float() - o[..., perm].float()).abs().max() / omax)
    e_s = float((hp - hT[..., perm]).abs().max() / smax)
    del dp, op, hp
    d2 = dict(d, v=d["v"] * 2, h0=d["h0"] * 2)
    o2, h2 = gpu_prefill(kda, d2)
    torch.cuda.synchronize()
    e2_o = float((o2.float() - 2 * o.float()).abs().max() / omax)
    e2_s = float((h2 - 2 * hT).abs().max() / smax)
    _report(f"{name} permuted columns", o=e_o, hT=e_s)
    _report(f"{name} doubled v, h0", o=e2_o, hT=e2_s)
    assert max(e_o, e_s, e2_o, e2_s) <= 1e-6


def test_decode_config(kda):
    """N=256, H=12, 16 steps, state updated in place: equals a 16-token chunked
    prefill from the same state (all sequences and heads), and four sampled
    (sequence, head) pairs equal the oracle."""
    case = KI.CONFIGS["decode_256"]
    run = KI.make_decode(case, seed=0)
    A = run["A"].cuda()
    st = run["state"].cuda().contiguous()
    st0 = st.clone()
    outs = []
    for s in run["steps"]:
        sd = to_dev(s)
        outs.append(kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, st))
    torch.cuda.synchronize()
    O = torch.stack(outs, 1)   # [N, 16, H, dv]
    # the same tokens as one prefill per sequence
    cat = lambda key: torch.stack([s[key] for s in run["steps"]], 1).cuda().contiguous()  # noqa: E731
    op, hp = kda.kda_chunk_fwd(cat("q"), cat("k"), cat("v"), cat("z"), cat("b"), A,
                               initial_state=st0, chunk_size=64)
    torch.cuda.synchronize()
    e1, e2 = rel_err(O, op), rel_err(st, hp)
    _report("decode_256 vs prefill", o=e1, state=e2)
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16
    for n, h in [(0, 0), (17, 3), (128, 11), (255, 6)]:
        S = run["state"][n, h].double().numpy()
        for t, s in enumerate(run["steps"]):
            o_ref, S_ref = oracle.decode_step(s["q"][n:n + 1, h:h + 1], s["k"][n:n + 1, h:h + 1],
                                              s["v"][n:n + 1, h:h + 1], s["z"][n:n + 1, h:h + 1],
                                              s["b"][n:n + 1, h:h + 1], run["A"][h:h + 1],
                                              S[None, None])
            S = S_ref[0, 0]
            assert rel_err(O[n, t, h], o_ref[0, 0]) <= TOL_BF16
        assert rel_err(st[n, h], S) <= TOL_BF16


def test_decode_large_batch_sampled(kda):
    """One decode step on 32,768 sequences x 12 heads: a 24 GiB fp32 state of
    6.4e9 elements, so state offsets pass 32 bits.  Sampled (sequence, head)
    pairs, the first and the last included, against the oracle's step from
    the same drawn state; every output and the whole new state finite."""
    N, H = 32768, 12
    case = KI.DecodeCase("decode_big", N=N, H=H, dk=128, dv=128, steps=1)
    run = KI.make_decode(case, device="cuda", seed=3)
    picks = [(0, 0), (N - 1, H - 1), (N // 2, 5), (21845, 7), (N - 2, 0)]
    before = {p: run["state"][p].double().cpu().numpy() for p in picks}
    s = run["steps"][0]
    o = kda.kda_recurrent_step(s["q"], s["k"], s["v"], s["z"], s["b"], run["A"], run["state"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(run["state"]).all()
    worst = 0.0
    for n, h in picks:
        one = lambda x: x[n:n + 1, h:h + 1].cpu()   # noqa: E731
        o_ref, S_ref = oracle.decode_step(one(s["q"]), one(s["k"]), one(s["v"]), one(s["z"]),
                                          one(s["b"]), run["A"][h:h + 1].cpu(), before[(n, h)][None, None])
        eo, eS = rel_err(o[n, h].cpu(), o_ref[0, 0]), rel_err(run["state"][n, h].cpu(), S_ref[0, 0])
        worst = max(worst, eo, eS)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    _report("decode 32768 x 12 sampled", worst=worst)
    del run, s, o
    torch.cuda.empty_cache()            # the 24 GiB state, released for the tests after this one


# ------------------------------------------------------------- smaller cases

@pytest.mark.parametrize("dtype,dk,chunk,T,H", [
    ("bf16", 128, 64, 200, 2),     # MFMA path: 3 full chunks + 8-token tail
    ("bf16", 128, 64, 64, 1),      # exactly one chunk
    ("bf16", 128, 64, 17, 3),      # one partial chunk
    ("fp32", 128, 64, 150, 1),     # fp32 path at d = 128
    ("fp32", 16, 16, 70, 2),       # fp32 path, ragged
    ("bf16", 16, 16, 45, 2),       # bf16 inputs on the fp32 path
    ("fp32", 64, 16, 40, 2),
    ("fp32", 32, 64, 90, 2),
])
def test_prefill_small_vs_oracle(kda, dtype, dk, chunk, T, H):
    case = KI.PrefillCase("small", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=1, T=T,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=T + dk)
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp)
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    eo, eS = rel_err(o[0], ro), rel_err(hT[0], rS)
    _report(f"small {dtype} d={dk} C={chunk} T={T}", o=eo, hT=eS)
    assert eo <= tol and eS <= tol


def test_slow_decay_long_memory(kda):
    """Near-1 decay (z shifted to very negative values) keeps the initial state
    and early tokens alive across many chunks: stresses the chunk-to-chunk chain."""
    case = KI.PrefillCase("slow", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=700,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=3)
    inp["z"] = inp["z"] - 6.0
    inp["h0"] = inp["h0"] * 50
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp)
    eo, eS = rel_err(o[0], ro), rel_err(hT[0], rS)
    _report("slow decay", o=eo, hT=eS)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_extreme_gates(kda, dtype, dk, chunk):
    """Saturated gates: on every other channel alpha = e^-5 (the lower bound,
    g = -5 exactly) and on the rest alpha = 1, so decay exponents inside a
    chunk span the whole range the 16-token sub-tiles are built for (a
    reciprocal of up to e^80 on the diagonal tiles) next to channels that
    never decay; a sequence with a ragged tail, from an initial state."""
    case = KI.PrefillCase("extreme", H=2, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=1, T=300,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=21)
    sign = torch.tensor([1.0 if c % 2 == 0 else -1.0 for c in range(dk)])
    inp["z"] = (BIG * sign).expand_as(inp["z"]).contiguous()
    inp["A"] = torch.zeros_like(inp["A"])
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(inp)
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    eo, eS = rel_err(o[0], ro), rel_err(hT[0], rS)
    _report(f"extreme gates {dtype}", o=eo, hT=eS)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    assert eo <= tol and eS <= tol


def test_extreme_gates_decode(kda):
    """The decode step with the saturated gates above: alpha = e^-5 and 1 on
    alternate channels, five steps against the oracle's step."""
    case = KI.DecodeCase("extremedec", N=4, H=2, dk=128, dv=128, steps=5, dtype="bf16")
    run = KI.make_decode(case, seed=22)
    sign = torch.tensor([1.0 if c % 2 == 0 else -1.0 for c in range(128)])
    A = torch.zeros_like(run["A"])
    st = run["state"].cuda().contiguous()
    S = run["state"]
    for s in run["steps"]:
        z = (BIG * sign).expand_as(s["z"]).contiguous()
        o = kda.kda_recurrent_step(s["q"].cuda(), s["k"].cuda(), s["v"].cuda(), z.cuda(),
                                   s["b"].cuda(), A.cuda(), st)
        ro, S = oracle.decode_step(s["q"], s["k"], s["v"], z, s["b"], A, S)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and rel_err(o, ro) <= TOL_BF16
    assert rel_err(st, S) <= TOL_BF16


def test_stage_intermediates_match_chunked_oracle(kda):
    """Per-chunk G, A_kk, A_qk, T and the state entering each chunk match the
    oracle's chunked form (MFMA path, 3 chunks + tail, with h0)."""
    case = KI.PrefillCase("stage", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=200,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=11)
    d = to_dev(inp)
    o, hT, it = kda.kda_chunk_fwd_debug(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                                        initial_state=d["h0"], chunk_size=64)
    torch.cuda.synchronize()
    q, k, v, z, b = (inp[x][0] for x in ("q", "k", "v", "z", "b"))
    _, _, inter = oracle.chunkwise(q, k, v, z, b, inp["A"], inp["h0"][0], chunk=64, keep=True)
    for c, rec in enumerate(inter):
        n = rec[0]["G"].shape[0]
        for h in range(2):
            r = rec[h]
            eG = np.abs(it["G"][c, h, :n].double().cpu().numpy() - r["G"]).max()
            e = dict(Akk=rel_err(it["Akk"][c, h, :n, :n], r["Akk"]),
                     Aqk=rel_err(it["Aqk"][c, h, :n, :n], r["Aqk"]),
                     T=rel_err(it["T"][c, h, :n, :n], r["T"]),
                     S0=rel_err(it["S0"][c, h], r["S0"]))
            _report(f"stage chunk {c} head {h}", G_abs=eG, **e)
            assert eG <= 1e-3
            assert all(x <= 2e-2 for x in e.values())


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_varlen_edge_lengths(kda, dtype, dk, chunk):
    """Empty, single-token, exactly-one-chunk, chunk +- 1 and multi-chunk
    sequences in one packed batch, each from its own initial state."""
    lens = [0, 1, chunk - 1, chunk, chunk + 1, 2 * chunk + 3, 0, 7]
    case = KI.PrefillCase("edge", H=3, dk=dk, dv=dk, chunk=chunk, dtype=dtype, zero_h0=False)
    inp = KI.make_prefill(case, seed=5, lengths=lens)
    d = to_dev(inp)
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    ro, rS = oracle.packed(inp["q"], inp["k"], inp["v"], inp["z"], inp["b"], inp["A"],
                           inp["h0"], inp["cu_seqlens"])
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    eo, eS = rel_err(o[0], ro), rel_err(hT, rS)
    _report(f"varlen edges {dtype}", o=eo, hT=eS)
    assert eo <= tol and eS <= tol
    # empty sequences return their initial state exactly
    assert torch.equal(hT[0], d["h0"][0]) and torch.equal(hT[6], d["h0"][6])


def test_zero_tokens_copies_state(kda):
    case = KI.PrefillCase("empty", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=2, T=0,
                          zero_h0=False)
    inp = to_dev(KI.make_prefill(case, seed=1))
    o, hT = gpu_prefill(kda, inp)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hT, inp["h0"])


def test_malformed_offsets_are_clamped(kda):
    """cu_seqlens that break 0 = cu[0] <= ... <= cu[N] = T are clamped into
    [0, T] on the device (the header's contract).  With T = 200 and cu = [0,
    120, 60, 500, 10] the sequences are [0, 120), empty, [60, 200) and empty:
    the final states are defined (each sequence reads only its own tokens) and
    held to the oracle, the empty ones return h0 exactly, and the output rows
    that only sequence 0 covers match it (rows two sequences cover are
    unspecified, but finite).  With cu = [0, 200, 0, 200, 0, 200] three
    sequences cover every token, 12 chunks against a capacity of 9: the chunks
    past the capacity are dropped, and the call stays in its buffers."""
    case = KI.PrefillCase("badcu", H=2, dk=128, dv=128, chunk=64, dtype="bf16", zero_h0=False)
    inp = KI.make_prefill(case, seed=3, lengths=[50, 50, 50, 50])
    d = to_dev(inp)
    d["cu_seqlens"] = torch.tensor([0, 120, 60, 500, 10], dtype=torch.int32, device="cuda")
    o, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(hT).all()
    q, k, v, z, b = (inp[x][0] for x in ("q", "k", "v", "z", "b"))
    ro0, rS0 = oracle.recurrence(q[:120], k[:120], v[:120], z[:120], b[:120], inp["A"], inp["h0"][0])
    _, rS2 = oracle.recurrence(q[60:], k[60:], v[60:], z[60:], b[60:], inp["A"], inp["h0"][2])
    e0, eo, e2 = rel_err(hT[0], rS0), rel_err(o[0, :60], ro0[:60]), rel_err(hT[2], rS2)
    _report("malformed cu_seqlens", hT0=e0, o0=eo, hT2=e2)
    assert e0 <= TOL_BF16 and eo <= TOL_BF16 and e2 <= TOL_BF16
    assert torch.equal(hT[1], d["h0"][1]) and torch.equal(hT[3], d["h0"][3])
    inp5 = KI.make_prefill(case, seed=4, lengths=[40] * 5)
    d5 = to_dev(inp5)
    d5["cu_seqlens"] = torch.tensor([0, 200, 0, 200, 0, 200], dtype=torch.int32, device="cuda")
    o, hT = gpu_prefill(kda, d5)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(hT).all()
    assert torch.equal(hT[1], d5["h0"][1]) and torch.equal(hT[3], d5["h0"][3])
    _, rS0 = oracle.recurrence(*(inp5[x][0] for x in ("q", "k", "v", "z", "b")), inp5["A"],
                               inp5["h0"][0])
    assert rel_err(hT[0], rS0) <= TOL_BF16


def test_misaligned_tensor_is_refused(kda):
    """A contiguous view that starts 4 bytes into its storage is refused by
    the library's 16-byte alignment check (no kernel is launched), and the
    aligned call on the same values runs."""
    case = KI.PrefillCase("align", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=64,
                          zero_h0=False)
    inp = to_dev(KI.make_prefill(case, seed=2))
    n = inp["q"].numel()
    buf = torch.empty(n + 8, dtype=inp["q"].dtype, device=inp["q"].device)
    buf[2:2 + n].copy_(inp["q"].reshape(-1))
    q_mis = buf[2:2 + n].view(inp["q"].shape)
    assert q_mis.is_contiguous() and q_mis.data_ptr() % 16 == 4
    with pytest.raises(kda.KdaError, match="misaligned"):
        kda.kda_chunk_fwd(q_mis, inp["k"], inp["v"], inp["z"], inp["b"], inp["A"],
                          initial_state=inp["h0"])
    o, hT = kda.kda_chunk_fwd(q_mis.clone(), inp["k"], inp["v"], inp["z"], inp["b"], inp["A"],
                              initial_state=inp["h0"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_batch_of_fixed_length_sequences(kda):
    """B > 1 without cu_seqlens equals separate calls per sequence."""
    case = KI.PrefillCase("batch", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=3, T=100,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=9))
    o, hT = gpu_prefill(kda, d)
    for bi in range(3):
        sub = {k: d[k][bi:bi + 1].contiguous() for k in ("q", "k", "v", "z", "b", "h0")}
        sub.update(A=d["A"], chunk=64)
        o1, h1 = gpu_prefill(kda, sub)
        assert torch.equal(o1[0], o[bi]) and torch.equal(h1[0], hT[bi])


def _table_regions(B, T, H, N, C=64):
    """Byte ranges of the workspace's bookkeeping: the header (3 int32), the
    chunk table (cap int4), the sequence and sequence-segment tables (N int2
    each) and the segment table (seg_cap int4), each region 256-byte aligned
    after the 256-byte header (the workspace layout the library documents)."""
    al = lambda x: (x + 255) // 256 * 256   # noqa: E731
    cap = B * ((T + C - 1) // C) + N
    nseg = 1 if H >= 256 else 256 // H
    per = max((cap + nseg - 1) // nseg, 8)
    per = min(per, cap) if cap > 0 else 1
    seg_cap = (cap + per - 1) // per + max(N, 1)
    off_seqs = al(256 + cap * 16)
    off_seqsegs = al(off_seqs + max(N, 1) * 8)
    off_segs = al(off_seqsegs + max(N, 1) * 8)
    return [(0, 12), (256, 256 + cap * 16), (off_seqs, off_seqs + N * 8),
            (off_seqsegs, off_seqsegs + N * 8), (off_segs, off_segs + seg_cap * 16)]


@pytest.mark.parametrize("B,T,H", [(3, 640, 2), (2, 4096, 16), (5, 128, 1), (1, 2560, 12),
                                   (80, 64, 1), (4, 0, 2), (7, 320, 40), (2, 192, 300)])
def test_fixed_batch_tables_equal_packed(kda, B, T, H):
    """B equal-length sequences without cu_seqlens (the chunk and segment
    tables planned on the host and written by the intra launch) against the
    same tokens packed with cu_seqlens = 0, T, 2T, ... (the tables written by
    the bookkeeping launch).  With T a multiple of the chunk both calls use
    one workspace layout: the header and the chunk, sequence and segment
    tables agree byte for byte, the outputs and final states bit for bit."""
    case = KI.PrefillCase("fixedplan", H=H, dk=128, dv=128, chunk=64, dtype="bf16", B=B, T=T,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=33))
    nbytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, 128, 128, B, 64, torch.bfloat16)
    assert nbytes == kda.kda_chunk_fwd_workspace_bytes(1, B * T, H, 128, 128, B, 64, torch.bfloat16)
    ws_f = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    ws_p = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    o_f, h_f = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                                 initial_state=d["h0"], chunk_size=64, workspace=ws_f)
    flat = lambda x: x.reshape(1, B * T, *x.shape[2:]).contiguous()   # noqa: E731
    cu = (torch.arange(B + 1, dtype=torch.int32, device="cuda") * T).contiguous()
    o_p, h_p = kda.kda_chunk_fwd(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["z"]), flat(d["b"]),
                                 d["A"], initial_state=d["h0"], cu_seqlens=cu, chunk_size=64,
                                 workspace=ws_p)
    torch.cuda.synchronize()
    for a, e in _table_regions(B, T, H, B):
        assert torch.equal(ws_f[a:e], ws_p[a:e]), f"bookkeeping bytes [{a}, {e}) differ"
    assert torch.equal(o_f.reshape(1, B * T, H, 128), o_p) and torch.equal(h_f, h_p)


def test_split_prefill_equals_single_pass(kda):
    """prefill(T1) then prefill(T2) from the returned state == prefill(T1 + T2)."""
    case = KI.PrefillCase("split", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=300,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=21))
    o, hT = gpu_prefill(kda, d)
    part = lambda a, e: {**{k: d[k][:, a:e].contiguous() for k in ("q", "k", "v", "z", "b")},  # noqa: E731
                         "A": d["A"], "chunk": 64}
    p1 = part(0, 100)
    p1["h0"] = d["h0"]
    o1, h1 = gpu_prefill(kda, p1)
    p2 = part(100, 300)
    p2["h0"] = h1
    o2, h2 = gpu_prefill(kda, p2)
    torch.cuda.synchronize()
    e1, e2 = rel_err(torch.cat([o1, o2], 1), o), rel_err(h2, hT)
    _report("split 100+200", o=e1, hT=e2)
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16)])
def test_prefill_then_decode_equals_longer_prefill(kda, dtype, dk):
    """Chunked prefill of T1 tokens followed by recurrent decode of the next
    tokens equals one chunked pass over all of them."""
    chunk = 64 if dk == 128 else 16
    T1, steps = 130, 6
    case = KI.PrefillCase("pd", H=2, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=1, T=T1 + steps,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=31))
    o_all, h_all = gpu_prefill(kda, d)
    p1 = {k: d[k][:, :T1].contiguous() for k in ("q", "k", "v", "z", "b")}
    p1.update(A=d["A"], h0=d["h0"], chunk=chunk)
    o1, st = gpu_prefill(kda, p1)
    outs = []
    for t in range(T1, T1 + steps):
        outs.append(kda.kda_recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                           d["v"][:, t].contiguous(), d["z"][:, t].contiguous(),
                                           d["b"][:, t].contiguous(), d["A"], st))
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    e1 = rel_err(torch.stack(outs, 1), o_all[:, T1:])
    e2 = rel_err(st, h_all)
    _report(f"prefill+decode {dtype}", o=e1, state=e2)
    assert e1 <= tol and e2 <= tol


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16), ("bf16", 64)])
def test_decode_small_vs_oracle(kda, dtype, dk):
    case = KI.DecodeCase("dec", N=5, H=3, dk=dk, dv=dk, steps=4, dtype=dtype)
    run = KI.make_decode(case, seed=2)
    A = run["A"].cuda()
    st = run["state"].cuda().contiguous()
    S = run["state"]
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    for s in run["steps"]:
        sd = to_dev(s)
        o = kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, st)
        ro, S = oracle.decode_step(s["q"], s["k"], s["v"], s["z"], s["b"], run["A"], S)
        torch.cuda.synchronize()
        assert rel_err(o, ro) <= tol
    assert rel_err(st, S) <= tol


# --------------------------------------------------------------------- pins

@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_delta_rule_hand_check_on_gpu(kda, dtype, dk, chunk):
    """[LA-KDA §7.4] embedded along one channel: k1 = k2 = q = e_0, v = (5, 7) e_0,
    beta = (0.5, 0.4), alpha = 1 (z = -1e4) -> o1[0] = 2.5, o2[0] = 4.3, all
    other entries 0.  Decode gives the same numbers."""
    dt = KI.dtype_of(dtype)
    T, H = 2, 1
    e0 = torch.zeros(dk)
    e0[0] = 1
    q = e0.expand(1, T, H, dk).to(dt).contiguous().cuda()
    v = torch.zeros(1, T, H, dk)
    v[0, 0, 0, 0], v[0, 1, 0, 0] = 5.0, 7.0
    v = v.to(dt).cuda()
    z = torch.full((1, T, H, dk), -BIG).cuda()
    b = torch.tensor([[[0.0], [float(np.log(0.4 / 0.6))]]]).float().cuda()
    A = torch.zeros(H).cuda()
    o, hT = kda.kda_chunk_fwd(q, q, v, z, b, A, chunk_size=chunk)
    torch.cuda.synchronize()
    o = o.float().cpu()
    tol = 1e-5 if dtype == "fp32" else 5e-3
    assert abs(o[0, 0, 0, 0].item() - 2.5) <= tol * 2.5
    assert abs(o[0, 1, 0, 0].item() - 4.3) <= tol * 4.3
    assert o[0, :, 0, 1:].abs().max().item() == 0.0
    st = torch.zeros(1, H, dk, dk).cuda()
    for t in range(T):
        od = kda.kda_recurrent_step(q[:, t].contiguous(), q[:, t].contiguous(), v[:, t].contiguous(),
                                    z[:, t].contiguous(), b[:, t].contiguous(), A, st)
        assert abs(od[0, 0, 0].float().item() - [2.5, 4.3][t]) <= tol * 4.3
    assert abs(st[0, 0, 0, 0].item() - 4.3) <= 1e-5


def test_exact_recall_on_gpu(kda):
    """[K3-ATTN §2.1] Householder erase: beta = 1 (b = +1e4) and a unit k make
    S_t^T k_t = v_t for any decay and history; read with q_t = k_t."""
    H, dk, T = 2, 128, 96
    g = torch.Generator().manual_seed(4)
    idx = torch.randint(0, dk, (T, H), generator=g)
    k = torch.nn.functional.one_hot(idx, dk).float().unsqueeze(0)
    v = torch.randn(1, T, H, dk, generator=g)
    z = torch.randn(1, T, H, dk, generator=g)
    b = torch.full((1, T, H), BIG)
    A = torch.zeros(H)
    h0 = torch.randn(1, H, dk, dk, generator=g)
    for dtype, chunk, tol in (("bf16", 64, TOL_BF16), ("fp32", 16, TOL_F32)):
        dt = KI.dtype_of(dtype)
        kk = k.to(dt).cuda()
        vv = v.to(dt).cuda()
        o, _ = kda.kda_chunk_fwd(kk, kk, vv, z.cuda(), b.cuda(), A.cuda(), initial_state=h0.cuda(),
                                 chunk_size=chunk)
        torch.cuda.synchronize()
        assert rel_err(o, vv.float()) <= tol, dtype


def test_pure_decay_on_gpu(kda):
    """beta = 0 (b = -1e4) writes nothing: S_T = Diag(prod alpha) S_0."""
    case = KI.PrefillCase("decay", H=2, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=80,
                          zero_h0=False)
    inp = KI.make_prefill(case, seed=8)
    inp["b"] = torch.full_like(inp["b"], -BIG)
    inp["z"] = inp["z"] - 3.0
    d = to_dev(inp)
    _, hT = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    g = oracle.gate_log_decay(inp["z"][0], inp["A"])       # [T, H, dk]
    ref = np.exp(g.sum(0))[:, :, None] * inp["h0"][0].double().numpy()
    assert rel_err(hT[0], ref) <= 1e-4


def test_deterministic(kda):
    """Two runs are bitwise identical (no atomics on the path)."""
    case = KI.PrefillCase("det", H=4, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=333,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=12))
    o1, h1 = gpu_prefill(kda, d)
    o2, h2 = gpu_prefill(kda, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("dtype,dk,chunk", [
    ("bf16", 128, 64),     # MFMA path
    ("fp32", 128, 64),     # fp32 path: eight 16-column slices per (sequence, head)
    ("fp32", 64, 16),      # fp32 path: four slices, 16-token chunks
])
def test_in_place_final_state(kda, dtype, dk, chunk):
    """hT may alias h0: the in-place call equals the out-of-place one bit for bit."""
    T, H = 130, 2
    case = KI.PrefillCase("alias", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype, B=1, T=T,
                          zero_h0=False)
    d = to_dev(KI.make_prefill(case, seed=13))
    o1, h1 = gpu_prefill(kda, d)
    st = d["h0"].clone()
    L = kda.lib()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(1, T, H, dk, dk, 1, chunk, tdt),
                     dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    rc = L.kda_chunk_fwd(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["z"].data_ptr(),
                         d["b"].data_ptr(), d["A"].data_ptr(), st.data_ptr(), None, 1, T, H, dk,
                         dk, 1, chunk, 1 if dtype == "bf16" else 0, o2.data_ptr(), st.data_ptr(),
                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o1, o2) and torch.equal(h1, st)
    ro, rS = oracle_prefill(KI.make_prefill(case, seed=13))
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    assert rel_err(o2[0], ro) <= tol and rel_err(st[0], rS) <= tol


# ---------------------------------------------------------------- replay fold

def _fold_window(dtype, dk, N, H, W, seed):
    """A speculative window of W draft tokens per sequence from the seeded
    decode generator, stacked to [N, W, H, .], plus the checkpoint state."""
    case = KI.DecodeCase("fold", N=N, H=H, dk=dk, dv=dk, steps=W, dtype=dtype)
    run = KI.make_decode(case, seed=seed)
    st = run["steps"]
    win = {key: torch.stack([s[key] for s in st], dim=1) for key in ("q", "k", "v", "z", "b")}
    return run, st, win


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16), ("bf16", 64)])
def test_fold_bit_identical_to_recurrent_steps(kda, dtype, dk):
    """[K3-ATTN §6.2]: the fold replays the accepted prefix with results
    bit-identical to the token-by-token recurrent calls.  Counts cover none,
    part, all, and out-of-range values (clamped)."""
    N, H, W = 7, 3, 7
    run, steps, win = _fold_window(dtype, dk, N, H, W, seed=21)
    n_acc = torch.tensor([0, 1, 3, 7, 5, 9, -2], dtype=torch.int32)
    A = run["A"].cuda()
    st0 = run["state"].cuda().contiguous()
    folded = st0.clone()
    kda.kda_recurrent_fold(win["k"].cuda().contiguous(), win["v"].cuda().contiguous(),
                           win["z"].cuda().contiguous(), win["b"].cuda().contiguous(), A,
                           n_acc.cuda(), folded)
    # reference: the recurrent call token by token, state snapshotted at each
    # sequence's count
    ref = st0.clone()
    cur = st0.clone()
    cnt = n_acc.clamp(0, W)
    for t, s in enumerate(steps):
        sd = to_dev(s)
        kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, cur)
        for n in range(N):
            if int(cnt[n]) == t + 1:
                ref[n] = cur[n]
    torch.cuda.synchronize()
    print(f"[parity] fold {dtype} d={dk}: max|fold - steps| = "
          f"{float((folded - ref).abs().max()):.3e}", flush=True)
    assert torch.equal(folded, ref)


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16)])
def test_fold_vs_oracle(kda, dtype, dk):
    """The folded states against the oracle's replay on the same (rounded)
    inputs; the arithmetic is fp32 in both dtypes."""
    N, H, W = 6, 4, 7
    run, _, win = _fold_window(dtype, dk, N, H, W, seed=22)
    n_acc = [7, 2, 0, 4, 7, 1]
    st = run["state"].cuda().contiguous()
    kda.kda_recurrent_fold(win["k"].cuda().contiguous(), win["v"].cuda().contiguous(),
                           win["z"].cuda().contiguous(), win["b"].cuda().contiguous(),
                           run["A"].cuda(), torch.tensor(n_acc, dtype=torch.int32).cuda(), st)
    ref = oracle.replay_fold(win["k"], win["v"], win["z"], win["b"], run["A"], run["state"], n_acc)
    torch.cuda.synchronize()
    err = rel_err(st, ref)
    _report(f"fold vs oracle {dtype} d={dk}", state=err)
    assert err <= TOL_F32


def test_fold_decode_workload_window(kda):
    """The decode workload's shape (256 sequences, 12 heads, d = 128, bf16)
    with a window of 7 draft tokens (the page's num_speculative_tokens) and
    mixed acceptance: equal bits to the recurrent steps, and the oracle on
    sampled sequences."""
    N, H, W = 256, 12, 7
    run, steps, win = _fold_window("bf16", 128, N, H, W, seed=23)
    g = torch.Generator().manual_seed(5)
    n_acc = torch.randint(0, W + 1, (N,), generator=g, dtype=torch.int32)
    A = run["A"].cuda()
    st0 = run["state"].cuda().contiguous()
    folded = st0.clone()
    kda.kda_recurrent_fold(win["k"].cuda().contiguous(), win["v"].cuda().contiguous(),
                           win["z"].cuda().contiguous(), win["b"].cuda().contiguous(), A,
                           n_acc.cuda(), folded)
    cur = st0.clone()
    ref = st0.clone()
    for t, s in enumerate(steps):
        sd = to_dev(s)
        kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, cur)
        sel = (n_acc == t + 1).nonzero().flatten().cuda()
        ref[sel] = cur[sel]
    torch.cuda.synchronize()
    assert torch.equal(folded, ref)
    for n in (0, 97, 255):
        r = oracle.replay_fold(win["k"][n:n + 1], win["v"][n:n + 1], win["z"][n:n + 1],
                               win["b"][n:n + 1], run["A"], run["state"][n:n + 1], [int(n_acc[n])])
        assert rel_err(folded[n], r[0]) <= TOL_F32


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16), ("bf16", 64)])
def test_verify_then_fold_bit_identical_to_recurrent_steps(kda, dtype, dk):
    """[K3-ATTN §6.2] verify pass: every window token's output from the
    checkpoint, bit-identical to the recurrent calls, with the checkpoint left
    untouched; then the fold commits each sequence's accepted prefix, again
    bit-identical.  Against the oracle's verify pass on the same inputs."""
    N, H, W = 6, 3, 7
    run, steps, win = _fold_window(dtype, dk, N, H, W, seed=24)
    A = run["A"].cuda()
    st0 = run["state"].cuda().contiguous()
    ck = st0.clone()
    dev = {key: win[key].cuda().contiguous() for key in win}
    o = kda.kda_recurrent_verify(dev["q"], dev["k"], dev["v"], dev["z"], dev["b"], A, ck)
    cur = st0.clone()
    outs = []
    for s in steps:
        sd = to_dev(s)
        outs.append(kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, cur))
    ref = torch.stack(outs, 1)
    n_acc = torch.tensor([7, 0, 3, 1, 6, 7], dtype=torch.int32)
    kda.kda_recurrent_fold(dev["k"], dev["v"], dev["z"], dev["b"], A, n_acc.cuda(), ck)
    torch.cuda.synchronize()
    assert torch.equal(o, ref), float((o.float() - ref.float()).abs().max())
    expect = st0.clone()
    for n in range(N):
        if int(n_acc[n]) == W:
            expect[n] = cur[n]
    full = [n for n in range(N) if int(n_acc[n]) == W]
    none = [n for n in range(N) if int(n_acc[n]) == 0]
    assert torch.equal(ck[full], expect[full]) and torch.equal(ck[none], st0[none])
    ro = oracle.verify_window(win["q"], win["k"], win["v"], win["z"], win["b"], run["A"],
                              run["state"])
    e = rel_err(o, ro)
    _report(f"verify vs oracle {dtype} d={dk}", o=e)
    assert e <= (TOL_F32 if dtype == "fp32" else TOL_BF16)


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 16)])
def test_verify_single_token_window(kda, dtype, dk):
    """A one-token window (no next token to load during the step): the
    verify output equals one recurrent step's output bit for bit, and the
    checkpoint is untouched."""
    N, H, W = 5, 2, 1
    run, steps, win = _fold_window(dtype, dk, N, H, W, seed=26)
    A = run["A"].cuda()
    st0 = run["state"].cuda().contiguous()
    ck = st0.clone()
    dev = {key: win[key].cuda().contiguous() for key in win}
    o = kda.kda_recurrent_verify(dev["q"], dev["k"], dev["v"], dev["z"], dev["b"], A, ck)
    sd = to_dev(steps[0])
    cur = st0.clone()
    ref = kda.kda_recurrent_step(sd["q"], sd["k"], sd["v"], sd["z"], sd["b"], A, cur)
    torch.cuda.synchronize()
    assert torch.equal(o[:, 0], ref) and torch.equal(ck, st0)


def test_verify_reads_state_only(kda):
    """The checkpoint state is bit-for-bit unchanged by the verify pass, and
    W = 0 is a no-op."""
    run, _, win = _fold_window("bf16", 128, 4, 2, 5, seed=25)
    st = run["state"].cuda().contiguous()
    st0 = st.clone()
    dev = {key: win[key].cuda().contiguous() for key in win}
    kda.kda_recurrent_verify(dev["q"], dev["k"], dev["v"], dev["z"], dev["b"], run["A"].cuda(), st)
    kda.kda_recurrent_verify(dev["q"][:, :0].contiguous(), dev["k"][:, :0].contiguous(),
                             dev["v"][:, :0].contiguous(), dev["z"][:, :0].contiguous(),
                             dev["b"][:, :0].contiguous(), run["A"].cuda(), st)
    torch.cuda.synchronize()
    assert torch.equal(st, st0)


# ------------------------------------------------------ segment layouts

@pytest.mark.parametrize("B,T,H,heads", [(1, 8192, 1, [0]), (3, 1500, 5, [0, 4]),
                                         (1, 4096, 40, [7, 39])])
def test_segment_layouts_vs_oracle(kda, B, T, H, heads):
    """The MFMA path cuts the sequences into about 256 / H segments in all, of
    at least 8 chunks: one head with many segments, several sequences with
    three segments each, and many heads with few.  Sampled heads of every
    sequence against the oracle."""
    case = KI.PrefillCase("seg", H=H, dk=128, dv=128, chunk=64, dtype="bf16", B=B, T=T,
                          zero_h0=False)
    d = KI.make_prefill(case, seed=17)
    o, hT = gpu_prefill(kda, to_dev(d))
    torch.cuda.synchronize()
    for bi in range(B):
        sub = {k: d[k][bi:bi + 1] for k in ("q", "k", "v", "z", "b", "h0")}
        sub["A"] = d["A"]
        ro, rS = oracle_prefill(sub, heads=heads)
        e_o = rel_err(o[bi][:, heads], ro)
        e_s = rel_err(hT[bi][heads], rS)
        _report(f"segments B={B} T={T} H={H} seq {bi}", o=e_o, hT=e_s)
        assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_packed_segment_lengths_vs_oracle(kda):
    """Sequences of 11, 21, 32 and 6 chunks (and an empty and a one-chunk one)
    at H = 32: the smallest segment length the capacity allows (10 chunks)
    would give 11 segments per head where one round holds 8, so the device
    lengthens the segments (11 chunks: 8 segments).  Sampled heads of every
    sequence against the oracle."""
    lens = [700, 1300, 2000, 333, 0, 64]
    heads = [0, 31]
    case = KI.PrefillCase("segpack", H=32, dk=128, dv=128, chunk=64, dtype="bf16", zero_h0=False)
    d = KI.make_prefill(case, seed=19, lengths=lens)
    o, hT = gpu_prefill(kda, to_dev(d))
    torch.cuda.synchronize()
    cu = [int(x) for x in d["cu_seqlens"].tolist()]
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s].cpu(), d["h0"][s])
            continue
        ro, rS = oracle_prefill(d, heads=heads, seq=s)
        e_o = rel_err(o[0, cu[s]:cu[s + 1]][:, heads], ro)
        e_s = rel_err(hT[s][heads], rS)
        _report(f"packed segments seq {s} (len {n})", o=e_o, hT=e_s)
        assert e_o <= TOL_BF16 and e_s <= TOL_BF16


@pytest.mark.parametrize("case_id", range(12))
def test_random_packed_layouts(kda, case_id):
    """Seeded random packed batches: 1-9 sequences whose lengths mix empty,
    one-token, short and multi-chunk ones, 1-40 heads, on the MFMA path and
    on the fp32 path; the first and last head of every sequence against the
    oracle (per-tensor metric), empty sequences return h0 exactly."""
    import random
    rng = random.Random(7000 + case_id)
    mfma = case_id % 3 != 2
    if mfma:
        dk, chunk, dtype = 128, 64, "bf16"
    else:
        dk, chunk, dtype = rng.choice([16, 32, 64]), rng.choice([16, 64]), rng.choice(["fp32", "bf16"])
    H = rng.choice([1, 2, 3, 5, 12, 16, 33, 40])
    lens = [rng.choice([0, 1, rng.randint(1, 200), rng.randint(1, 2500)])
            for _ in range(rng.randint(1, 9))]
    budget = 8000 if dk == 128 else 3000
    if sum(lens) > budget:
        lens = [n * budget // sum(lens) for n in lens]
    if sum(lens) == 0:
        lens[-1] = 1
    case = KI.PrefillCase("randlayout", H=H, dk=dk, dv=dk, chunk=chunk, dtype=dtype,
                          zero_h0=False)
    d = KI.make_prefill(case, seed=7100 + case_id, lengths=lens)
    o, hT = gpu_prefill(kda, to_dev(d))
    torch.cuda.synchronize()
    heads = sorted({0, H - 1})
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    cu = [int(x) for x in d["cu_seqlens"].tolist()]
    refs = {s: oracle_prefill(d, heads=heads, seq=s) for s, n in enumerate(lens) if n}
    o_scale = max(float(abs(r[0]).max()) for r in refs.values())
    s_scale = max(float(abs(r[1]).max()) for r in refs.values())
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s].cpu(), d["h0"][s])
            continue
        ro, rS = refs[s]
        e_o = rel_err(o[0, cu[s]:cu[s + 1]][:, heads], ro, scale=o_scale)
        e_s = rel_err(hT[s][heads], rS, scale=s_scale)
        assert e_o <= tol and e_s <= tol, (case_id, dk, chunk, dtype, H, lens, s, e_o, e_s)
    _report(f"random layout {case_id}: d={dk} C={chunk} {dtype} H={H} lens={lens}", ok=0.0)


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("fp32", 16, 16)])
def test_packed_batch_beyond_64_sequences(kda, dtype, dk, chunk):
    """A packed batch of 100 sequences (empty, one-token, ragged and
    multi-chunk lengths): the chunk bookkeeping's block-wide path (more than
    64 sequences) instead of its single-wave one.  Seven sequences against
    the oracle on both heads (per-tensor metric over the checked ones), every
    empty sequence's state equal to its h0, and the packed call equal bit for
    bit to separate calls of the same sequences."""
    import random
    rng = random.Random(9100 + dk)
    lens = [rng.choice([0, 1, rng.randint(2, 63), rng.randint(64, 300)]) for _ in range(100)]
    lens[0], lens[50], lens[99] = 0, 1, 257
    case = KI.PrefillCase("packed100", H=2, dk=dk, dv=dk, chunk=chunk, dtype=dtype, zero_h0=False)
    d = KI.make_prefill(case, seed=9200 + dk, lengths=lens)
    g = to_dev(d)
    o, hT = gpu_prefill(kda, g)
    torch.cuda.synchronize()
    cu = [int(x) for x in d["cu_seqlens"].tolist()]
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    checked = [s for s in (1, 13, 49, 50, 64, 65, 99) if lens[s] > 0]
    refs = {s: oracle_prefill(d, seq=s) for s in checked}
    o_scale = max(float(np.abs(r[0]).max()) for r in refs.values())
    s_scale = max(float(np.abs(r[1]).max()) for r in refs.values())
    for s in checked:
        ro, rS = refs[s]
        eo = rel_err(o[0, cu[s]:cu[s + 1]], ro, scale=o_scale)
        eS = rel_err(hT[s], rS, scale=s_scale)
        _report(f"packed 100 {dtype} seq {s} (len {lens[s]})", o=eo, hT=eS)
        assert eo <= tol and eS <= tol
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s], g["h0"][s])
    for s in (13, 64, 99):
        a, e = cu[s], cu[s + 1]
        sub = {k: g[k][:, a:e].contiguous() for k in ("q", "k", "v", "z", "b")}
        sub.update(A=g["A"], h0=g["h0"][s:s + 1].contiguous(), chunk=chunk)
        o1, h1 = gpu_prefill(kda, sub)
        assert torch.equal(o1[0], o[0, a:e]) and torch.equal(h1[0], hT[s])
