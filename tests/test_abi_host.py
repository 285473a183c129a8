"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/kda.h declares, and rejects bad arguments before
anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import gated_delta_rule_77_amd as kda
    if not os.path.exists(kda.lib_path):
        from gated_delta_rule_77_amd import build
        build.build()
    return kda.lib()


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]*?\b(kda_\w+)\s*\(", src)))


def test_header_declares_the_binding_symbols():
    import gated_delta_rule_77_amd as kda
    assert _declared_symbols() == sorted(kda.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared_symbols():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, word in [(0, "KDA_OK"), (1, "INVALID"), (2, "UNSUPPORTED"), (3, "WORKSPACE"), (4, "HIP"),
                       (5, "SCRATCH")]:
        assert word in L.kda_status_string(code).decode()
    assert L.kda_status_string(99)


def test_supported_sets(L):
    assert L.kda_chunk_fwd_supported(128, 128, 64, 1) == 1
    assert L.kda_chunk_fwd_supported(16, 16, 16, 0) == 1
    assert L.kda_chunk_fwd_supported(128, 64, 64, 1) == 0
    assert L.kda_chunk_fwd_supported(96, 96, 64, 1) == 0
    assert L.kda_chunk_fwd_supported(128, 128, 32, 1) == 0
    assert L.kda_chunk_fwd_supported(128, 128, 64, 7) == 0
    assert L.kda_recurrent_step_supported(128, 128, 1) == 1
    assert L.kda_recurrent_step_supported(128, 128, 0) == 1
    assert L.kda_recurrent_step_supported(256, 256, 1) == 0


def test_workspace_bytes(L):
    # the workspace holds per-(chunk, head) records (tens of KiB each on the MFMA
    # path) for a capacity of B * ceil(T / C) + N chunks, plus per-segment states
    n = L.kda_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 1, 64, 1)
    assert n >= (64 + 1) * 16 * 65536
    assert n < (64 + 1) * 16 * 256 * 1024
    n2 = L.kda_chunk_fwd_workspace_bytes(1, 8192, 16, 128, 128, 1, 64, 1)
    assert n2 > n
    assert L.kda_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 64, 1, 64, 1) == 0
    assert L.kda_chunk_fwd_workspace_bytes(-1, 4096, 16, 128, 128, 1, 64, 1) == 0
    assert L.kda_chunk_fwd_workspace_bytes(1, 64, 2, 16, 16, 1, 16, 0) > 0


def _chunk(L, **kw):
    a = dict(q=None, k=None, v=None, z=None, b=None, A=None, h0=None, cu=None, B=1, T=64, H=2,
             dk=16, dv=16, N=1, chunk=16, dtype=0, o=None, hT=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    fn = L.kda_chunk_fwd
    fn.restype = ctypes.c_int
    vp = ctypes.c_void_p
    i = ctypes.c_int
    fn.argtypes = [vp] * 8 + [i] * 8 + [vp, vp, vp, ctypes.c_size_t, vp]
    return fn(a["q"], a["k"], a["v"], a["z"], a["b"], a["A"], a["h0"], a["cu"], a["B"], a["T"],
              a["H"], a["dk"], a["dv"], a["N"], a["chunk"], a["dtype"], a["o"], a["hT"], a["ws"],
              a["wsb"], a["stream"])


FAKE = 1 << 20   # never dereferenced: validation fails before any launch


def test_noalloc_rejects_before_any_device_call(L):
    """kda_chunk_fwd_noalloc checks the call's workspace need against its
    scratch array (and the arguments) on the host: a call beyond the array
    returns KDA_ERR_SCRATCH and an invalid one KDA_ERR_INVALID_ARG, both
    before any HIP call (so this runs without a GPU)."""
    import gated_delta_rule_77_amd as kda
    fn = L.kda_chunk_fwd_noalloc
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn.restype = i
    fn.argtypes = [vp] * 8 + [i] * 8 + [vp, vp, vp]
    big = L.kda_chunk_fwd_workspace_bytes(1, 8192, 12, 128, 128, 1, 64, 1)
    assert big > kda.NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 6 + [None, None]
    assert fn(*args, 1, 8192, 12, 128, 128, 1, 64, 1, FAKE, FAKE, None) == 5
    assert fn(*args, 1, 64, 0, 16, 16, 1, 16, 0, FAKE, FAKE, None) == 1      # H = 0
    assert fn(*args, 1, 64, 2, 96, 96, 1, 64, 1, FAKE, FAKE, None) == 2      # unsupported shape
    assert fn(*args, 1, 64, 2, 16, 16, 0, 16, 0, FAKE, FAKE, None) == 1      # N != B


def test_chunk_fwd_rejects_bad_arguments(L):
    full = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, b=FAKE, A=FAKE, o=FAKE)
    assert _chunk(L, **full, T=-1) == 1
    assert _chunk(L, **full, H=0) == 1
    assert _chunk(L, **full, dtype=5) == 1
    assert _chunk(L, **full, N=2) == 1                 # N must equal B without cu_seqlens
    assert _chunk(L, **full, cu=FAKE, B=2, N=2) == 1   # cu_seqlens needs B == 1
    assert _chunk(L, **full, dk=96, dv=96) == 2
    assert _chunk(L, **full, chunk=32) == 2
    assert _chunk(L, **dict(full, q=None)) == 1
    assert _chunk(L, **dict(full, A=None)) == 1
    assert _chunk(L, **full, ws=None) == 3
    assert _chunk(L, **full, ws=FAKE, wsb=16) == 3
    assert _chunk(L, **full, ws=FAKE + 8, wsb=1 << 40) == 3    # misaligned workspace
    assert _chunk(L, N=0, B=0) == 1                    # B must be >= 1
    assert _chunk(L, B=1, N=1, T=8, q=None, k=None, v=None, z=None, b=None, o=None,
                  A=None) == 1


def test_recurrent_step_rejects_bad_arguments(L):
    fn = L.kda_recurrent_step
    fn.restype = ctypes.c_int
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn.argtypes = [vp] * 8 + [i] * 5 + [vp]
    ok = [FAKE] * 8
    assert fn(*ok, 4, 2, 96, 96, 1, None) == 2
    assert fn(*ok, 4, 2, 128, 64, 1, None) == 2
    assert fn(*ok, -1, 2, 128, 128, 1, None) == 1
    assert fn(*ok, 4, 0, 128, 128, 1, None) == 1
    assert fn(*ok, 4, 2, 128, 128, 3, None) == 1
    assert fn(*([None] + ok[1:]), 4, 2, 128, 128, 1, None) == 1
    assert fn(*([None] * 8), 0, 2, 128, 128, 1, None) == 0   # N = 0 is a no-op


def test_binding_refuses_cpu_tensors():
    import torch
    import gated_delta_rule_77_amd as kda
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1), torch.zeros(1))
    with pytest.raises(ValueError):
        kda.kda_recurrent_step(x[0], x[0], x[0], x[0], torch.zeros(4, 1), torch.zeros(1),
                               torch.zeros(4, 1, 16, 16))


def test_binding_refuses_a_host_workspace():
    """A caller's workspace must be device memory: a host tensor raises before
    its pointer could reach a kernel."""
    import torch
    import gated_delta_rule_77_amd as kda
    with pytest.raises(ValueError):
        kda._workspace(torch.zeros(1024, dtype=torch.uint8), 512, torch.device("cuda", 0))


def test_binding_raises_on_a_short_or_misaligned_workspace(monkeypatch):
    """A caller who passes a workspace gets no allocation: one that is too
    small or not 256-byte aligned raises KdaError, and nothing is allocated in
    its place (the device checks of _req are bypassed so that a host tensor
    can stand in on a machine without a GPU)."""
    import torch
    import gated_delta_rule_77_amd as kda
    monkeypatch.setattr(kda, "_req", lambda t, *a, **k: t)

    def no_alloc(*a, **k):
        raise AssertionError("the binding allocated a workspace")

    buf = torch.zeros(4096 + 256, dtype=torch.uint8)
    off = (-buf.data_ptr()) % 256
    aligned = buf[off:off + 4096]
    monkeypatch.setattr(torch, "empty", no_alloc)
    dev = torch.device("cuda", 0)
    with pytest.raises(kda.KdaError, match="needs 8192"):
        kda._workspace(aligned, 8192, dev)
    with pytest.raises(kda.KdaError, match="aligned"):
        kda._workspace(buf[off + 16:off + 16 + 1024], 512, dev)
    assert kda._workspace(aligned, 4096, dev) is aligned


def test_recurrent_fold_rejects_bad_arguments(L):
    fn = L.kda_recurrent_fold
    fn.restype = ctypes.c_int
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn.argtypes = [vp] * 7 + [i] * 6 + [vp]
    ok = [FAKE] * 7
    assert fn(*ok, 4, 7, 2, 96, 96, 1, None) == 2
    assert fn(*ok, 4, 7, 2, 128, 64, 1, None) == 2
    assert fn(*ok, -1, 7, 2, 128, 128, 1, None) == 1
    assert fn(*ok, 4, -1, 2, 128, 128, 1, None) == 1
    assert fn(*ok, 4, 7, 0, 128, 128, 1, None) == 1
    assert fn(*ok, 4, 7, 2, 128, 128, 3, None) == 1
    assert fn(*([FAKE] * 5 + [None, FAKE]), 4, 7, 2, 128, 128, 1, None) == 1   # n_accept missing
    assert fn(*([None] * 7), 0, 7, 2, 128, 128, 1, None) == 0    # N = 0 is a no-op
    assert fn(*([None] * 7), 4, 0, 2, 128, 128, 1, None) == 0    # an empty window is a no-op


def test_layer_entry_points_reject_bad_arguments(L):
    fl = ctypes.c_float
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fwd = L.kda_layer_fwd
    fwd.restype = i
    fwd.argtypes = [vp] * 13 + [fl, fl] + [i] * 7 + [vp, vp, vp, sz, vp]

    def call(**kw):
        a = dict(ptrs=[FAKE] * 13, l2=1e-6, rms=1e-5, B=1, T=64, H=2, d=16, N=1, chunk=16,
                 dtype=0, y=FAKE, hT=None, ws=FAKE, wsb=1 << 40, stream=None)
        a.update(kw)
        p = list(a["ptrs"])
        for idx, val in a.get("set", {}).items():
            p[idx] = val
        return fwd(*p, a["l2"], a["rms"], a["B"], a["T"], a["H"], a["d"], a["N"], a["chunk"],
                   a["dtype"], a["y"], a["hT"], a["ws"], a["wsb"], a["stream"])

    assert call(l2=-1.0) == 1
    assert call(rms=float("nan")) == 1
    assert call(d=96) == 2
    assert call(chunk=32) == 2
    assert call(set={3: None}) == 1                     # conv_w missing
    assert call(set={12: None}) == 1                    # norm_w missing
    assert call(set={11: None}) == 1                    # gate missing
    assert call(ws=None) == 3
    assert call(wsb=16) == 3
    L.kda_layer_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    assert L.kda_layer_fwd_workspace_bytes(1, 64, 2, 16, 1, 16, 0) > \
        L.kda_chunk_fwd_workspace_bytes(1, 64, 2, 16, 16, 1, 16, 0)
    step = L.kda_layer_step
    step.restype = i
    step.argtypes = [vp] * 11 + [fl, fl, vp] + [i] * 4 + [vp]
    ok = [FAKE] * 11
    assert step(*ok, 1e-6, 1e-5, FAKE, 4, 2, 96, 1, None) == 2
    assert step(*ok, -1.0, 1e-5, FAKE, 4, 2, 128, 1, None) == 1
    assert step(*([FAKE] * 4 + [None] + [FAKE] * 6), 1e-6, 1e-5, FAKE, 4, 2, 128, 1, None) == 1
    assert step(*([None] * 11), 1e-6, 1e-5, None, 0, 2, 128, 1, None) == 0


def test_mode_entry_points_validate_the_mode(L):
    fn = L.kda_chunk_fwd_mode
    fn.restype = ctypes.c_int
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn.argtypes = [vp] * 8 + [i] * 9 + [vp, vp, vp, ctypes.c_size_t, vp]

    def call(mode, z=FAKE, A=FAKE, ws=None):
        return fn(FAKE, FAKE, FAKE, z, FAKE, A, None, None, 1, 64, 2, 16, 16, 1, 16, 0, mode,
                  FAKE, None, ws, 0, None)

    assert call(3) == 1 and call(-1) == 1
    assert call(0, A=None) == 1 and call(1, z=None) == 1   # KDA and GLA read the gate logits
    assert call(2, z=None, A=None) == 3                    # DeltaNet does not: on to the workspace check
    step = L.kda_recurrent_step_mode
    step.restype = i
    step.argtypes = [vp] * 8 + [i] * 6 + [vp]
    assert step(*[FAKE] * 8, 4, 2, 128, 128, 1, 3, None) == 1
    assert step(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 4, 2, 128, 128, 1, 0, None) == 1
    assert step(None, None, None, None, None, None, None, None, 0, 2, 128, 128, 1, 2, None) == 0


def test_dplr_entry_points_reject_bad_arguments(L):
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fn = L.kda_dplr_chunk_fwd
    fn.restype = i
    fn.argtypes = [vp] * 9 + [i] * 8 + [vp, vp, vp, sz, vp]

    def call(ptrs=None, **kw):
        a = dict(B=1, T=64, H=2, dk=16, dv=16, N=1, chunk=16, dtype=0, ws=None, wsb=0)
        a.update(kw)
        p = [FAKE] * 7 + [None, None] if ptrs is None else ptrs
        return fn(*p, a["B"], a["T"], a["H"], a["dk"], a["dv"], a["N"], a["chunk"], a["dtype"],
                  FAKE, None, a["ws"], a["wsb"], None)

    assert call(dk=96, dv=96) == 2
    assert call(dtype=4) == 1
    assert call([FAKE] * 3 + [None] + [FAKE] * 3 + [None, None]) == 1    # a missing
    assert call([FAKE] * 4 + [None] + [FAKE] * 2 + [None, None]) == 1    # b missing
    assert call() == 3                                                   # no workspace
    L.kda_dplr_chunk_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    assert L.kda_dplr_chunk_fwd_workspace_bytes(1, 64, 2, 16, 16, 1, 16, 0) > 0
    assert L.kda_dplr_chunk_fwd_workspace_bytes(1, 64, 2, 96, 96, 1, 16, 0) == 0
    st = L.kda_dplr_recurrent_step
    st.restype = i
    st.argtypes = [vp] * 9 + [i] * 5 + [vp]
    assert st(*[FAKE] * 9, 4, 2, 96, 96, 1, None) == 2
    assert st(*([FAKE] * 3 + [None] + [FAKE] * 5), 4, 2, 128, 128, 1, None) == 1
    assert st(*[None] * 9, 0, 2, 128, 128, 1, None) == 0


def test_recurrent_verify_rejects_bad_arguments(L):
    fn = L.kda_recurrent_verify
    fn.restype = ctypes.c_int
    vp, i = ctypes.c_void_p, ctypes.c_int
    fn.argtypes = [vp] * 8 + [i] * 6 + [vp]
    ok = [FAKE] * 8
    assert fn(*ok, 4, 7, 2, 96, 96, 1, None) == 2
    assert fn(*ok, -1, 7, 2, 128, 128, 1, None) == 1
    assert fn(*ok, 4, -1, 2, 128, 128, 1, None) == 1
    assert fn(*ok, 4, 7, 2, 128, 128, 5, None) == 1
    assert fn(*([FAKE] * 6 + [None, FAKE]), 4, 7, 2, 128, 128, 1, None) == 1   # state missing
    assert fn(*([None] * 8), 0, 7, 2, 128, 128, 1, None) == 0
    assert fn(*([None] * 8), 4, 0, 2, 128, 128, 1, None) == 0


def test_grid_limits_are_validated(L):
    """One workgroup per (chunk, head): chunk capacity x heads must stay within
    int32, checked on the host (no launch with a wrapped grid)."""
    L.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    # B * T fits int32, but ceil(T / 16) * H does not
    assert L.kda_chunk_fwd_workspace_bytes(1, 2000000000, 1024, 16, 16, 1, 16, 0) == 0
    assert _chunk(L, q=FAKE, k=FAKE, v=FAKE, z=FAKE, b=FAKE, A=FAKE, o=FAKE, T=2000000000, H=1024) == 1


def test_work_item_and_offset_limits_are_validated(L):
    """Each dispatch counts work-items in 32 bits and the intra-chunk kernels
    address a chunk's rows with 32-bit offsets: shapes past either limit are
    refused on the host, before any launch; shapes just inside are accepted."""
    ws = L.kda_chunk_fwd_workspace_bytes
    ws.restype = ctypes.c_size_t
    full = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, b=FAKE, A=FAKE, o=FAKE)
    # H * 128 * 64 >= 2^32: one chunk of 600,000 heads on the MFMA path
    assert ws(1, 64, 600000, 128, 128, 1, 64, 1) == 0
    assert _chunk(L, **full, T=64, H=600000, dk=128, dv=128, chunk=64, dtype=1) == 1
    # just inside: H * 128 * 64 = 2^32 - 65,536
    assert ws(1, 64, 524287, 128, 128, 1, 64, 1) > 0
    # N * H * 2048 >= 2^32: 300,000 packed sequences of 12 heads
    assert ws(1, 3000000, 12, 16, 16, 300000, 16, 0) == 0
    assert _chunk(L, **full, cu=FAKE, T=3000000, H=12, N=300000) == 1
    # recurrent calls: N * H * 256 >= 2^32
    fn = L.kda_recurrent_step
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    assert fn(*([FAKE] * 8), 1 << 20, 16, 128, 128, 1, None) == 1
    # the fp32 layer path's per-row passes: B * T * H * 64 >= 2^32
    lw = L.kda_layer_fwd_workspace_bytes
    lw.restype = ctypes.c_size_t
    assert lw(1, 100000000, 1, 16, 1, 16, 0) == 0
    assert lw(1, 1000000, 1, 16, 1, 16, 0) > 0


def test_misaligned_row_tensors_are_refused(L):
    """The header requires 16-byte aligned tensor pointers; the entry points
    refuse a misaligned row tensor before anything is enqueued (an aligned
    call with too small a workspace gets as far as the workspace check)."""
    vp, i, sz, fl = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    full = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, b=FAKE, A=FAKE, o=FAKE, ws=FAKE, wsb=16)
    assert _chunk(L, **full) == 3
    assert _chunk(L, **dict(full, q=FAKE + 8)) == 1
    assert _chunk(L, **dict(full, o=FAKE + 4)) == 1
    assert _chunk(L, **dict(full, z=FAKE + 4)) == 1
    assert _chunk(L, **dict(full, h0=FAKE + 8)) == 1
    assert _chunk(L, **dict(full, hT=FAKE + 12)) == 1
    assert _chunk(L, **dict(full, b=FAKE + 4)) == 3       # beta logits: 4-byte reads only

    step = L.kda_recurrent_step
    step.restype = i
    step.argtypes = [vp] * 8 + [i] * 5 + [vp]
    ok = [FAKE] * 8
    assert step(*(ok[:6] + [FAKE + 4, FAKE]), 4, 2, 128, 128, 1, None) == 1      # state
    assert step(*([FAKE + 2] + ok[1:]), 4, 2, 128, 128, 1, None) == 1            # q

    fold = L.kda_recurrent_fold
    fold.restype = i
    fold.argtypes = [vp] * 7 + [i] * 6 + [vp]
    assert fold(*([FAKE] * 6 + [FAKE + 4]), 4, 7, 2, 128, 128, 1, None) == 1

    ver = L.kda_recurrent_verify
    ver.restype = i
    ver.argtypes = [vp] * 8 + [i] * 6 + [vp]
    assert ver(*([FAKE] * 7 + [FAKE + 8]), 4, 7, 2, 128, 128, 1, None) == 1        # o

    lstep = L.kda_layer_step
    lstep.restype = i
    lstep.argtypes = [vp] * 11 + [fl, fl, vp] + [i] * 4 + [vp]
    assert lstep(*([FAKE] * 4 + [FAKE + 8] + [FAKE] * 6), 1e-6, 1e-5, FAKE, 4, 2, 128, 1, None) == 1

    lfwd = L.kda_layer_fwd
    lfwd.restype = i
    lfwd.argtypes = [vp] * 13 + [fl, fl] + [i] * 7 + [vp, vp, vp, sz, vp]
    lp = [FAKE] * 10 + [None, FAKE, FAKE]
    assert lfwd(*lp, 1e-6, 1e-5, 1, 64, 2, 16, 1, 16, 0, FAKE, None, FAKE, 16, None) == 3
    assert lfwd(*([FAKE + 8] + lp[1:]), 1e-6, 1e-5, 1, 64, 2, 16, 1, 16, 0, FAKE, None, FAKE, 16,
                None) == 1
    assert lfwd(*(lp[:3] + [FAKE + 4] + lp[4:]), 1e-6, 1e-5, 1, 64, 2, 16, 1, 16, 0, FAKE, None,
                FAKE, 16, None) == 1                                             # taps

    dch = L.kda_dplr_chunk_fwd
    dch.restype = i
    dch.argtypes = [vp] * 9 + [i] * 8 + [vp, vp, vp, sz, vp]
    dp = [FAKE] * 7 + [None, None]
    assert dch(*dp, 1, 64, 2, 16, 16, 1, 16, 0, FAKE, None, FAKE, 16, None) == 3
    assert dch(*(dp[:3] + [FAKE + 8] + dp[4:]), 1, 64, 2, 16, 16, 1, 16, 0, FAKE, None, FAKE, 16,
               None) == 1
    dst = L.kda_dplr_recurrent_step
    dst.restype = i
    dst.argtypes = [vp] * 9 + [i] * 5 + [vp]
    assert dst(*([FAKE] * 7 + [FAKE + 4, FAKE]), 4, 2, 128, 128, 1, None) == 1
