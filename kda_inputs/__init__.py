"""Seeded synthetic inputs for the Kimi Delta Attention (KDA) core.

This module is shared by the tests, the benchmark and the oracle's callers.  It
draws random tensors and nothing else: it holds none of the method's arithmetic
(no gate, no recurrence, no chunking).  The one transformation it applies is
the upstream L2 normalisation of q and k, which the pages place before the core
("q, k = L2Norm(Swish(ShortConv(W x)))", [LA-KDA §5.3]); the core itself never
normalises.

Sources:
  [LA-KDA]  "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制",
            blog-3d3.pages.dev/posts/150
  [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构",
            forceinjection.github.io/09_inference_system/vllm/module_analysis/kimi_k3_attention.html

Recipe (one torch.Generator per call, seeded; the draw order is fixed):
  [lengths] -> q -> k -> v -> z -> A -> b -> h0
  q, k : N(0,1) fp32, L2-normalised over d_k per (token, head), then cast to
         the config dtype (bf16 = round-to-nearest-even)
  v    : N(0,1) fp32 cast to the config dtype
  z    : N(0,1) fp32 per channel (raw gate logits)
  A    : U(-1,1) fp32 per head (zeros where the config says A_h = 0)
  b    : N(0,1) fp32 per (token, head) (raw beta logits)
  h0   : 0.02 * N(0,1) fp32 per (sequence, head), or None for a zero state
Decode draws A and h0 first, then (q, k, v, z, b) for every step in turn.

Layer inputs (the projections before the short convolution, make_layer): the
prefill draw above, then q_in, k_in, v_in ~ N(0,1) and gate ~ N(0,1) cast to
the config dtype, conv_w ~ 0.5 N(0,1) fp32 [3, H, d, 4], norm_w ~ U(0.5, 1.5)
fp32 [d], and conv_state0 ~ N(0,1) cast to the config dtype [N, 3, 3, H, d]
(or None).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = [
    "PrefillCase", "DecodeCase", "CONFIGS", "make_prefill", "make_decode", "make_layer",
    "varlen_lengths", "dtype_of",
]


@dataclasses.dataclass(frozen=True)
class PrefillCase:
    name: str
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str                 # "fp32" | "bf16"
    B: int = 1
    T: int = 0                 # tokens per sequence (fixed-length layout)
    n_seqs: int = 0            # > 0 selects the packed variable-length layout
    len_lo: int = 0            # inclusive bounds of the per-sequence length draw
    len_hi: int = 0
    zero_A: bool = False
    zero_h0: bool = True


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str = "bf16"


CONFIGS = {
    # tiny fp32 forward: B=1, H=2, T=64, d=16, C=16, A_h=0, zero state
    "tiny_fp32": PrefillCase("tiny_fp32", H=2, dk=16, dv=16, chunk=16, dtype="fp32",
                             B=1, T=64, zero_A=True, zero_h0=True),
    # single-sequence prefill: B=1, H=16, T=4096, d=128, C=64, bf16, zero state
    "prefill_4k": PrefillCase("prefill_4k", H=16, dk=128, dv=128, chunk=64, dtype="bf16",
                              B=1, T=4096, zero_h0=True),
    # packed batch: 8 sequences, lengths U[512, 16384], H=12, nonzero states
    "varlen_8": PrefillCase("varlen_8", H=12, dk=128, dv=128, chunk=64, dtype="bf16",
                            n_seqs=8, len_lo=512, len_hi=16384, zero_h0=False),
    # long context: B=1, H=12, T=2^20, nonzero state
    "long_1m": PrefillCase("long_1m", H=12, dk=128, dv=128, chunk=64, dtype="bf16",
                           B=1, T=1 << 20, zero_h0=False),
    # recurrent decode: 256 sequences x 12 heads, 16 single-token steps
    "decode_256": DecodeCase("decode_256", N=256, H=12, dk=128, dv=128, steps=16),
}


def dtype_of(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # upstream L2 normalisation over the last (d_k) axis
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-12)


def varlen_lengths(n: int, lo: int, hi: int, gen: torch.Generator) -> list:
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen,
                                          device=gen.device).tolist()]


def make_prefill(case: PrefillCase, device="cpu", seed: int = 0,
                 T: Optional[int] = None, lengths: Optional[list] = None) -> dict:
    """Draw one prefill batch.

    Returns a dict with q, k, v [B, T, H, d] (config dtype), z [B, T, H, dk] fp32,
    b [B, T, H] fp32, A [H] fp32, h0 [N, H, dk, dv] fp32 or None, cu_seqlens
    (int32 [N+1] or None) and the sizes.  `T` overrides the per-sequence length
    of a fixed-length case; `lengths` overrides the drawn lengths of a packed one.
    """
    dev = torch.device(device)
    gen = _gen(dev, seed)
    dt = dtype_of(case.dtype)
    cu = None
    if case.n_seqs > 0 or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(case.n_seqs, case.len_lo, case.len_hi, gen)
        lengths = [int(x) for x in lengths]
        B, Ttot, N = 1, sum(lengths), len(lengths)
        offs = [0]
        for n in lengths:
            offs.append(offs[-1] + n)
        cu = torch.tensor(offs, dtype=torch.int32, device=dev)
    else:
        B, Ttot = case.B, (case.T if T is None else int(T))
        N = B
    H, dk, dv = case.H, case.dk, case.dv
    f32 = torch.float32
    q = _unit_rows(torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32)).to(dt)
    k = _unit_rows(torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32)).to(dt)
    v = torch.randn(B, Ttot, H, dv, generator=gen, device=dev, dtype=f32).to(dt)
    z = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32)
    A = torch.rand(H, generator=gen, device=dev, dtype=f32) * 2.0 - 1.0
    if case.zero_A:
        A = torch.zeros_like(A)
    b = torch.randn(B, Ttot, H, generator=gen, device=dev, dtype=f32)
    h0 = None
    if not case.zero_h0:
        h0 = 0.02 * torch.randn(N, H, dk, dv, generator=gen, device=dev, dtype=f32)
    return dict(q=q, k=k, v=v, z=z, b=b, A=A, h0=h0, cu_seqlens=cu, lengths=lengths,
                B=B, T=Ttot, H=H, dk=dk, dv=dv, N=N, chunk=case.chunk, dtype=case.dtype)


def make_decode(case: DecodeCase, device="cpu", seed: int = 0,
                N: Optional[int] = None, steps: Optional[int] = None) -> dict:
    """Draw a decode run: A [H], state [N, H, dk, dv] fp32 and a list of per-step
    dicts with q, k [N, H, dk], v [N, H, dv] (config dtype), z [N, H, dk] fp32
    and b [N, H] fp32."""
    dev = torch.device(device)
    gen = _gen(dev, seed)
    dt = dtype_of(case.dtype)
    n = case.N if N is None else int(N)
    s = case.steps if steps is None else int(steps)
    H, dk, dv = case.H, case.dk, case.dv
    f32 = torch.float32
    A = torch.rand(H, generator=gen, device=dev, dtype=f32) * 2.0 - 1.0
    state = 0.02 * torch.randn(n, H, dk, dv, generator=gen, device=dev, dtype=f32)
    per_step = []
    for _ in range(s):
        q = _unit_rows(torch.randn(n, H, dk, generator=gen, device=dev, dtype=f32)).to(dt)
        k = _unit_rows(torch.randn(n, H, dk, generator=gen, device=dev, dtype=f32)).to(dt)
        v = torch.randn(n, H, dv, generator=gen, device=dev, dtype=f32).to(dt)
        z = torch.randn(n, H, dk, generator=gen, device=dev, dtype=f32)
        b = torch.randn(n, H, generator=gen, device=dev, dtype=f32)
        per_step.append(dict(q=q, k=k, v=v, z=z, b=b))
    return dict(A=A, state=state, steps=per_step, N=n, H=H, dk=dk, dv=dv, dtype=case.dtype)


def make_dplr(case: PrefillCase, device="cpu", seed: int = 0, T: Optional[int] = None,
              lengths: Optional[list] = None) -> dict:
    """A prefill draw (make_prefill) extended with the low-rank pair of the
    general DPLR update: la = -s * a_hat and lb = unit(a_hat + 0.5 n / sqrt(dk)),
    with a_hat a unit direction, s ~ U(0, 1) per token and head, and n
    standard normal, so that b leans on a (a strong erase) without being tied
    to it or to the write key k.  Both [B, T, H, dk] in the config dtype."""
    d = make_prefill(case, device=device, seed=seed, T=T, lengths=lengths)
    dev = torch.device(device)
    gen = _gen(dev, seed + 104729)
    dt = dtype_of(case.dtype)
    f32 = torch.float32
    B, Ttot, H, dk = d["B"], d["T"], d["H"], d["dk"]
    ah = _unit_rows(torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32))
    nz = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32)
    sc = torch.rand(B, Ttot, H, 1, generator=gen, device=dev, dtype=f32)
    d["lb"] = _unit_rows(ah + 0.5 * nz / dk ** 0.5).to(dt)
    d["la"] = (-sc * ah).to(dt)
    return d


def make_layer(case: PrefillCase, device="cpu", seed: int = 0, T: Optional[int] = None,
               lengths: Optional[list] = None, conv_state: bool = True) -> dict:
    """A prefill draw (make_prefill) extended with the layer's inputs:
    q_in, k_in, v_in, gate [B, T, H, d] (config dtype), conv_w [3, H, d, 4],
    norm_w [d] (fp32) and conv_state0 [N, 3, 3, H, d] (config dtype) or None.
    The core's q, k, v of the prefill draw are kept but unused by the layer."""
    d = make_prefill(case, device=device, seed=seed, T=T, lengths=lengths)
    dev = torch.device(device)
    gen = _gen(dev, seed + 7919)
    dt = dtype_of(case.dtype)
    f32 = torch.float32
    B, Ttot, H, dk, N = d["B"], d["T"], d["H"], d["dk"], d["N"]
    d["q_in"] = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32).to(dt)
    d["k_in"] = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32).to(dt)
    d["v_in"] = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32).to(dt)
    d["gate"] = torch.randn(B, Ttot, H, dk, generator=gen, device=dev, dtype=f32).to(dt)
    d["conv_w"] = 0.5 * torch.randn(3, H, dk, 4, generator=gen, device=dev, dtype=f32)
    d["norm_w"] = torch.rand(dk, generator=gen, device=dev, dtype=f32) + 0.5
    d["conv_state0"] = (torch.randn(N, 3, 3, H, dk, generator=gen, device=dev, dtype=f32).to(dt)
                        if conv_state else None)
    return d
