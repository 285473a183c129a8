"""The entry points under HIP graph capture.  libkda allocates nothing,
synchronises nothing and clears no memory with memset: every call is a
sequence of kernel launches on the caller's stream, so a caller can capture
it once and replay it.  Each test replays a captured call several times, with
eager work and synchronisations between the replays, and checks every replay
bit for bit against the same call run eagerly (same kernels, same inputs).
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
