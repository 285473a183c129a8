"""The entry points under HIP graph capture and on concurrent streams.
libkda allocates nothing, synchronises nothing, clears no memory with memset
and keeps no mutable global state: every call is a sequence of kernel
launches on the caller's stream, so a caller can capture it once and replay
it, or run independent calls side by side.  The graph tests replay a
captured call several times, with eager work and synchronisations between
the replays, and check every replay bit for bit against the same call run
eagerly (same kernels, same inputs).
"""
import pytest
import torch

import kda_inputs as KI
from kda_testutil import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_77_amd as m
    m.lib()
    return m


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns the
    graph and the tensors the captured call returned (its static outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


@pytest.mark.parametrize("lengths", [None, [700, 0, 1, 1300]])
def test_prefill_graph_replays_match_eager(kda, lengths):
    """kda_chunk_fwd (MFMA path) captured with its workspace; a fixed-length
    batch and a packed one with an empty and a one-token sequence."""
    if lengths is None:
        case = KI.PrefillCase("graph", H=4, dk=128, dv=128, chunk=64, dtype="bf16", B=2, T=777,
                              zero_h0=False)
        d = to_dev(KI.make_prefill(case, seed=41))
    else:
        case = KI.PrefillCase("graphvar", H=4, dk=128, dv=128, chunk=64, dtype="bf16",
                              zero_h0=False)
        d = to_dev(KI.make_prefill(case, seed=42, lengths=lengths))
    B, T, H = d["q"].shape[0], d["q"].shape[1], d["q"].shape[2]
    N = d["h0"].shape[0]
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, 128, 128, N, 64, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def call():
        return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                                 initial_state=d["h0"], cu_seqlens=d.get("cu_seqlens"),
                                 workspace=ws)
    o_ref, h_ref = call()
    torch.cuda.synchronize()
    o_ref, h_ref = o_ref.clone(), h_ref.clone()
    g, (o_g, h_g) = _capture(call)
    for r in range(3):
        o_g.fill_(float("nan"))              # stale outputs would show
        h_g.zero_()
        call()                               # eager work on the same workspace in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(h_g, h_ref), f"replay {r}"


def test_decode_graph_replays_match_eager(kda):
    """kda_recurrent_step captured on a static state: each replay advances the
    state in place exactly as one eager step does."""
    case = KI.DecodeCase("graphdec", N=8, H=4, dk=128, dv=128, steps=1, dtype="bf16")
    run = KI.make_decode(case, seed=43)
    st0 = run["state"].cuda()
    A = run["A"].cuda()
    tok = {k: run["steps"][0][k].cuda().contiguous() for k in ("q", "k", "v", "z", "b")}

    def step(st):
        return kda.kda_recurrent_step(tok["q"], tok["k"], tok["v"], tok["z"], tok["b"], A, st)
    # eager: one and two steps from st0
    s1 = st0.clone()
    o1 = step(s1).clone()
    s2 = s1.clone()
    o2 = step(s2).clone()
    torch.cuda.synchronize()
    st = st0.clone()
    g, o_g = _capture(lambda: step(st))
    for r in range(3):
        st.copy_(st0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o1) and torch.equal(st, s1), f"replay {r}"
        g.replay()                           # a second step from the replayed state
        torch.cuda.synchronize()
        assert torch.equal(o_g, o2) and torch.equal(st, s2), f"replay {r}, second step"


def test_concurrent_streams_match_sequential(kda):
    """The library holds no mutable global state: two prefill calls and two
    decode calls on two streams at once, each with its own buffers, give the
    bits of the same calls run one after the other."""
    case = KI.PrefillCase("streams", H=3, dk=128, dv=128, chunk=64, dtype="bf16", B=1, T=900,
                          zero_h0=False)
    d1 = to_dev(KI.make_prefill(case, seed=44))
    d2 = to_dev(KI.make_prefill(case, seed=45))
    dec = KI.make_decode(KI.DecodeCase("streamsdec", N=16, H=3, dk=128, dv=128, steps=1,
                                       dtype="bf16"), seed=46)
    A = dec["A"].cuda()
    tok = {k: dec["steps"][0][k].cuda().contiguous() for k in ("q", "k", "v", "z", "b")}

    def prefill(d):
        return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                                 initial_state=d["h0"])
    ref1, ref2 = prefill(d1), prefill(d2)
    s_ref = [dec["state"].cuda().clone() for _ in range(2)]
    o_ref = [kda.kda_recurrent_step(tok["q"], tok["k"], tok["v"], tok["z"], tok["b"], A, s)
             for s in s_ref]
    st = [dec["state"].cuda().clone() for _ in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    out = [None, None]
    for i, (s, d) in enumerate(zip(streams, (d1, d2))):
        with torch.cuda.stream(s):
            out[i] = (prefill(d),
                      kda.kda_recurrent_step(tok["q"], tok["k"], tok["v"], tok["z"], tok["b"], A,
                                             st[i]))
    torch.cuda.synchronize()
    for i, ref in enumerate((ref1, ref2)):
        (o, hT), od = out[i]
        assert torch.equal(o, ref[0]) and torch.equal(hT, ref[1])
        assert torch.equal(od, o_ref[i]) and torch.equal(st[i], s_ref[i])
