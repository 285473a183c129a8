"""Helpers shared by the GPU tests: moving seeded inputs to the device,
running the oracle on the same (already rounded) values, and the error metric.

Tolerance metric, per tensor: max|gpu - ref| / max|ref|.  Bars: 1e-4 for the
fp32 path, 1e-2 for bf16 inputs on the MFMA path (oracle on the same
bf16-rounded inputs).  A packed batch's output is one tensor: its sequences
are checked one at a time against the largest reference value of the whole
tensor (`scale`).  Dividing by a sequence's own maximum would be stricter than
the metric and, for a one-token sequence, measure something else: its output
is dominated by (q . k) v with |q . k| ~ 1/sqrt(d_k) for the unit-norm random
q, k of the input recipe, and the MFMA operands round q and k (scaled by
their decay factors) to bf16, which alone moves that small dot product by
about 1% of itself (reproduced by a CPU emulation of the rounding points).
"""
import json
import os

import numpy as np
import torch

import oracle

TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def report(suite: str, tag: str, **errs) -> None:
    """Print a case's measured errors; with KDA_PARITY_LOG set, also append
    them as one JSON line to that file, so that a GPU run keeps the margin of
    every case against its bar (tests/parity_margins.py summarises the
    log)."""
    print(f"[{suite}] {tag}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    path = os.environ.get("KDA_PARITY_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps({"suite": suite, "test": test, "case": tag,
                                "errors": {k: float(v) for k, v in errs.items()}}) + "\n")


def rel_err(got, ref, scale=None) -> float:
    got = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = ref.detach().double().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref)
    if scale is None:
        scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def to_dev(inp: dict, device="cuda") -> dict:
    out = dict(inp)
    for key in ("q", "k", "v", "z", "b", "A", "h0", "cu_seqlens"):
        if inp.get(key) is not None:
            out[key] = inp[key].to(device).contiguous()
    return out


def gpu_prefill(kda, d: dict, chunk=None, **kw):
    return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["b"], d["A"],
                             initial_state=d.get("h0"), cu_seqlens=d.get("cu_seqlens"),
                             chunk_size=chunk or d["chunk"], **kw)


def oracle_prefill(inp: dict, heads=None, T=None, seq=None):
    """Oracle outputs for a fixed-length batch with B == 1 (or one sequence of
    a packed batch when `seq` is given).  `heads` restricts to a subset of
    heads, `T` to a prefix of the tokens.  Returns (o [T, h, dv], S [h, dk, dv])."""
    q, k, v, z, b, A, h0 = (inp[x] for x in ("q", "k", "v", "z", "b", "A", "h0"))
    if seq is not None:
        cu = [int(x) for x in inp["cu_seqlens"].cpu().tolist()]
        a, e = cu[seq], cu[seq + 1]
        sl = slice(a, e if T is None else min(e, a + T))
        h0s = None if h0 is None else h0[seq]
    else:
        assert q.shape[0] == 1
        sl = slice(0, q.shape[1] if T is None else T)
        h0s = None if h0 is None else h0[0]
    hs = slice(None) if heads is None else list(heads)
    pick = lambda x: x[0, sl][:, hs].cpu()   # noqa: E731
    o, S = oracle.recurrence(pick(q), pick(k), pick(v), pick(z), b[0, sl][:, hs].cpu(),
                             A.cpu()[hs], None if h0s is None else h0s.cpu()[hs])
    return o, S
