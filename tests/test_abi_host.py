"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

- libkda.so loads and exports every function include/kda.h declares;
- status strings and the workspace query;
- argument validation returns its error before anything reaches the device
  (every call here is built to fail validation; the pointers are never
  dereferenced);
- the input generator's recipe (ranges, determinism, varlen lengths).
"""
import ctypes
import functools
import os
import re
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gated_delta_rule_25_amd", "libkda.so")
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, PRECONDITION, SCRATCH = range(7)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from gated_delta_rule_25_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [i32]
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, vp]
    L.kda_chunk_fwd.restype = i32
    L.kda_chunk_fwd.argtypes = [vp] * 7 + [i32, i64, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.kda_chunk_fwd_noalloc.restype = i32
    L.kda_chunk_fwd_noalloc.argtypes = [vp] * 7 + [i32, i64, i32, i32, i32, i32, vp, vp, vp, vp]
    L.kda_chunk_bwd_workspace_bytes.restype = sz
    L.kda_chunk_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    L.kda_chunk_bwd.restype = i32
    L.kda_chunk_bwd.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32] + [vp] * 7 + [sz, vp]
    L.kda_chunk_bwd_saved.restype = i32
    L.kda_chunk_bwd_saved.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32] + [vp] * 7 + [sz, vp]
    L.kda_chunk_fwd_save.restype = i32
    L.kda_chunk_fwd_save.argtypes = [vp] * 7 + [i32, i64, i32, i32, i32, i32] + [vp] * 3 + [sz, vp]
    L.kda_decode_step.restype = i32
    L.kda_decode_step.argtypes = [vp] * 6 + [i32, i32, i32, i32, i32, vp, vp]
    L.kda_decode_replay.restype = i32
    L.kda_decode_replay.argtypes = [vp] * 8 + [i32] * 6 + [vp] * 5
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == {"kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_workspace_bytes", "kda_chunk_bwd",
                          "kda_chunk_bwd_workspace_bytes", "kda_chunk_fwd_save", "kda_chunk_bwd_saved",
                          "kda_decode_step",
                          "kda_decode_replay", "kda_last_precondition_flags", "kda_status_string"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(kda_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code in range(7):
        s = lib.kda_status_string(code).decode()
        assert s and s != "unknown kda_status"
    assert lib.kda_status_string(99).decode() == "unknown kda_status"


def test_workspace_bytes(lib):
    # the two-kernel schedule keeps a factor store in the workspace: it grows
    # with the number of (chunk, head) blocks and is capped at 16 GiB (long
    # inputs run in windows), so a one-layer 1M-token input needs about that
    w8k = lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, None)
    w16k = lib.kda_chunk_fwd_workspace_bytes(1, 16384, 96, 128, 128, BF16, None)
    assert w8k > 0 and w16k > w8k
    assert w8k % 256 == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 1 << 20, 96, 128, 128, BF16, None) < 17 << 30
    assert lib.kda_chunk_fwd_workspace_bytes(64, 10 ** 6, 96, 128, 128, BF16, None) < 17 << 30
    # fp32 chunks are half as long, so more blocks
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, 0, None) > w8k
    # at most 65535 heads: a chunk's rows of a [T, H, 128] tensor are
    # addressed with 32-bit byte offsets
    assert lib.kda_chunk_fwd_workspace_bytes(1, 64, 65535, 128, 128, 0, None) > 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 64, 65536, 128, 128, BF16, None) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(1, 64, 65536, 128, 128, BF16) == 0
    assert chunk(lib, T=0, H=65536) == INVALID
    assert lib.kda_chunk_fwd_workspace_bytes(2, 10, 2, 64, 128, BF16, None) == 0  # invalid sizes
    assert lib.kda_chunk_fwd_workspace_bytes(0, 10, 2, 128, 128, BF16, None) == 0


def test_workspace_factor_budget_field(lib, monkeypatch):
    # kda_fused_opts.factor_budget_mib caps one window's factor store:
    # 129 chunk slots x 96 heads x 70.5 KiB fit one window; a 64 MiB cap needs
    # 14 windows of 129 // 14 + 2 = 11 slots; 0 and anything above 16384 keep
    # the default; a negative cap is refused.  No environment variable changes it.
    one = lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, None)
    assert one == two_kernel_ws(1, 8192, 96)
    capped = lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, opts_p(Opts(factor_budget_mib=64)))
    assert capped == 768 + 96 * 128 * 128 * 4 + 11 * 96 * FB_BF16  # + the state carried between windows
    for mib in (0, 4096, 16384, 1 << 20):
        assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16,
                                                 opts_p(Opts(factor_budget_mib=mib))) == one
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, opts_p(Opts(factor_budget_mib=-1))) == 0
    monkeypatch.setenv("KDA_FACTOR_BUDGET_MIB", "64")
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, None) == one


# Fake, never-dereferenced device addresses for validation-only calls.
BASE = 0x7F0000000000
MB = 1 << 20


def p(i):
    return ctypes.c_void_p(BASE + i * 64 * MB)


def chunk(lib, **kw):
    a = dict(q=p(0), k=p(1), v=p(2), la=p(3), b=p(4), s0=None, cu=None, N=1, T=10, H=2, dk=128, dv=128,
             dt=BF16, opts=None, o=p(5), fs=p(6), ws=p(8), wsb=32 * MB)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["la"], a["b"], a["s0"], a["cu"], a["N"], a["T"], a["H"],
                             a["dk"], a["dv"], a["dt"], a["opts"], a["o"], a["fs"], a["ws"], a["wsb"], None)


def test_chunk_validation(lib):
    assert chunk(lib, dk=64) == UNSUPPORTED
    assert chunk(lib, dv=256) == UNSUPPORTED
    assert chunk(lib, dt=7) == UNSUPPORTED
    assert chunk(lib, N=0) == INVALID
    assert chunk(lib, H=0) == INVALID
    assert chunk(lib, T=-1) == INVALID
    assert chunk(lib, q=None) == INVALID
    assert chunk(lib, o=None) == INVALID
    assert chunk(lib, N=2) == INVALID                          # several sequences need cu_seqlens
    assert chunk(lib, N=2, cu=p(7), ws=None, wsb=0) == WORKSPACE  # ... and a workspace
    assert chunk(lib, N=2, cu=p(7), ws=p(8), wsb=16) == WORKSPACE
    assert chunk(lib, o=p(0)) == INVALID                       # output aliases q
    assert chunk(lib, fs=p(3)) == INVALID                      # final state aliases log_alpha
    assert chunk(lib, s0=p(6), fs=ctypes.c_void_p(BASE + 6 * 64 * MB + 4)) == INVALID  # partial overlap
    # in-place continuation exempts initial_state only: q spanning exactly the
    # bytes of initial_state == final_state (T=256, H=2, bf16: 128 KiB each)
    # is still an input that the final state would overwrite
    assert chunk(lib, T=256, s0=p(0), fs=p(0)) == INVALID
    assert chunk(lib, T=128, dt=0, s0=p(3), fs=p(3)) == INVALID  # ... and so is log_alpha (fp32, 128 KiB)
    need2 = lib.kda_chunk_fwd_workspace_bytes(2, 10, 2, 128, 128, BF16, None)
    assert chunk(lib, N=2, cu=p(7), ws=p(0), wsb=need2) == INVALID  # workspace aliases q
    need1 = lib.kda_chunk_fwd_workspace_bytes(1, 10, 2, 128, 128, BF16, None)
    assert chunk(lib, ws=None, wsb=0) == WORKSPACE             # the factor store is always needed
    assert chunk(lib, ws=p(8), wsb=need1 - 1) == WORKSPACE
    assert chunk(lib, q=ctypes.c_void_p(BASE + 8)) == INVALID  # not 16-byte aligned
    assert chunk(lib, fs=ctypes.c_void_p(BASE + 6 * 64 * MB + 4)) == INVALID
    assert chunk(lib, b=ctypes.c_void_p(BASE + 4 * 64 * MB + 2)) == INVALID  # beta not 4-byte aligned
    assert chunk(lib, N=2, cu=p(7), ws=ctypes.c_void_p(BASE + 8 * 64 * MB + 4), wsb=need2) == INVALID  # workspace


class Opts(ctypes.Structure):
    _fields_ = [("conv_q_w", ctypes.c_void_p), ("conv_k_w", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("segment_tokens", ctypes.c_int), ("unbounded_decay", ctypes.c_int),
                ("factor_budget_mib", ctypes.c_int)]


def opts_p(o):
    return ctypes.cast(ctypes.pointer(o), ctypes.c_void_p)


FB_BF16 = 72192  # factor block of one (64-token chunk, head), bf16 I/O


def a256(x):
    return (x + 255) // 256 * 256


def two_kernel_ws(N, T, H, seg_tokens=0, C=64, fb=FB_BF16):
    """Workspace of one factor-store window (the layout kda_api.hip documents):
    longest-first order (N > 1), window table, [segment table and affine
    pairs], factor store of `slots` chunks."""
    slots = T // C + N + N + 1
    b = (a256(4 * N) if N > 1 else 0) + a256(4 * (N + 1)) + 2 * a256(4 * N)
    if seg_tokens:
        cap = slots // (seg_tokens // C) + N + 1
        b += a256(4 * (N + 1)) + 256 + a256(8 * cap) + cap * H * 2 * 65536
    return b + slots * H * fb


def test_workspace_bytes_segmented(lib):
    # forced segments of 64 tokens, N=1, T=1000, H=2: 18 factor slots, at most 20 segments
    o = Opts(None, None, None, None, 1e-6, 1e-6, 64)
    assert two_kernel_ws(1, 1000, 2, 64) == 768 + 768 + 20 * 2 * 2 * 65536 + 18 * 2 * FB_BF16
    assert lib.kda_chunk_fwd_workspace_bytes(1, 1000, 2, 128, 128, BF16, opts_p(o)) == two_kernel_ws(1, 1000, 2, 64)
    o.segment_tokens = 100                                     # not a multiple of 64
    assert lib.kda_chunk_fwd_workspace_bytes(1, 1000, 2, 128, 128, BF16, opts_p(o)) == 0
    o.segment_tokens = -1                                      # sequential schedule forced
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 8, 128, 128, BF16, opts_p(o)) == two_kernel_ws(1, 8192, 8)
    # automatic choice (256 compute units when no device is visible): H=8 leaves
    # 16 of 256 workgroups busy, so 16 segments of 512 tokens
    o.segment_tokens = 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 8, 128, 128, BF16, opts_p(o)) == two_kernel_ws(1, 8192, 8, 512)
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 8, 128, 128, BF16, None) == two_kernel_ws(1, 8192, 8, 512)
    # H=96 fills the GPU: the two-kernel schedule, the same plan as when forced
    o.segment_tokens = -1
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, None) == \
        lib.kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, BF16, opts_p(o))
    # short sequences are not split
    assert lib.kda_chunk_fwd_workspace_bytes(1, 512, 8, 128, 128, BF16, None) == \
        lib.kda_chunk_fwd_workspace_bytes(1, 512, 8, 128, 128, BF16, opts_p(o))


def test_chunk_validation_segmented(lib):
    o = Opts(None, None, None, None, 1e-6, 1e-6, 100)
    assert chunk(lib, opts=opts_p(o)) == INVALID                # segment length not a multiple of 64
    o.segment_tokens = 64
    assert chunk(lib, opts=opts_p(o), ws=None, wsb=0) == WORKSPACE  # the segmented form needs a workspace
    need = lib.kda_chunk_fwd_workspace_bytes(1, 10, 2, 128, 128, BF16, opts_p(o))
    assert chunk(lib, opts=opts_p(o), ws=p(8), wsb=need - 1) == WORKSPACE
    assert chunk(lib, opts=opts_p(o), ws=ctypes.c_void_p(BASE + 8 * 64 * MB + 4), wsb=need) == INVALID  # alignment
    assert chunk(lib, opts=opts_p(o), ws=p(5), wsb=need) == INVALID  # workspace aliases the output


def test_chunk_validation_fused(lib):
    o = Opts(None, None, p(5).value, None, 1e-6, 1e-6, 0)     # gate aliases the output
    assert chunk(lib, opts=ctypes.cast(ctypes.pointer(o), ctypes.c_void_p)) == INVALID
    o2 = Opts(None, None, None, None, -1.0, 1e-6, 0)          # negative epsilon
    assert chunk(lib, opts=ctypes.cast(ctypes.pointer(o2), ctypes.c_void_p)) == INVALID


def test_noalloc_limits(lib):
    """kda_chunk_fwd_noalloc: its scratch size in the binding matches the
    header, and sizes whose smallest windows exceed the array are refused on
    the host (64 sequences x 96 heads need ~65 x 96 factor blocks of 70.5 KiB
    plus the carried states, far past 128 MiB), as are bad sizes."""
    import gated_delta_rule_25_amd as kda
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert kda.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))

    def na(**kw):
        a = dict(q=p(0), k=p(1), v=p(2), la=p(3), b=p(4), s0=None, cu=p(7), N=64, T=256, H=96, dk=128, dv=128,
                 dt=BF16, opts=None, o=p(5), fs=None)
        a.update(kw)
        return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["la"], a["b"], a["s0"], a["cu"], a["N"], a["T"],
                                         a["H"], a["dk"], a["dv"], a["dt"], a["opts"], a["o"], a["fs"], None)
    assert na() == SCRATCH
    assert na(N=1, cu=None, H=2000) == SCRATCH
    assert na(dk=64) == UNSUPPORTED
    assert na(N=0) == INVALID
    assert na(T=-1) == INVALID
    assert na(opts=opts_p(Opts(factor_budget_mib=-5))) == INVALID
    assert na(N=1, cu=None, H=2, opts=opts_p(Opts(segment_tokens=100))) == INVALID


def bwd_ws(N, T, H, C=64, fb=FB_BF16, db=82944, es=2):
    """Workspace of kda_chunk_bwd (the layout kda_api.hip documents): order
    (N > 1), chunk table, then per (slot, head) the forward factor block, the
    reverse-carry block, two 128 x 128 states and two C x 128 blocks in the
    I/O dtype (es bytes per element)."""
    slots = T // C + N + 1
    b = (a256(4 * N) if N > 1 else 0) + a256(4 * (N + 1)) + 2 * a256(4 * N)
    return b + slots * H * (fb + db + 2 * 128 * 128 * es + 2 * C * 128 * es)


def test_bwd_workspace_bytes(lib):
    # reverse-carry block (bf16, 64-token chunks): Kb 16 KiB + -W^T 16 KiB + gamma
    # 1 KiB + P^T dO 16 KiB + Qt^T dO 32 KiB = 82944 bytes
    assert lib.kda_chunk_bwd_workspace_bytes(1, 8192, 96, 128, 128, BF16) == bwd_ws(1, 8192, 96)
    assert lib.kda_chunk_bwd_workspace_bytes(3, 1000, 2, 128, 128, BF16) == bwd_ws(3, 1000, 2)
    assert lib.kda_chunk_bwd_workspace_bytes(1, 0, 2, 128, 128, BF16) == bwd_ws(1, 0, 2)
    assert lib.kda_chunk_bwd_workspace_bytes(1, 100, 2, 64, 128, BF16) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(0, 100, 2, 128, 128, BF16) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(1, 100, 2, 128, 128, 9) == 0


def bwd(lib, fn="kda_chunk_bwd", **kw):
    a = dict(q=p(0), k=p(1), v=p(2), la=p(3), b=p(4), s0=None, cu=None, do=p(5), dsT=None, N=1, T=10, H=2,
             dk_=128, dv_=128, dt=BF16, gq=p(6), gk=p(7), gv=p(8), gla=p(9), gb=p(10), gs0=None, ws=p(11),
             wsb=64 * MB)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["la"], a["b"], a["s0"], a["cu"], a["do"], a["dsT"], a["N"],
                            a["T"], a["H"], a["dk_"], a["dv_"], a["dt"], a["gq"], a["gk"], a["gv"], a["gla"], a["gb"],
                            a["gs0"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("fn", ["kda_chunk_bwd", "kda_chunk_bwd_saved"])
def test_bwd_validation(lib, fn):
    bwd = functools.partial(globals()["bwd"], fn=fn)
    assert bwd(lib, dk_=64) == UNSUPPORTED
    assert bwd(lib, dt=3) == UNSUPPORTED
    assert bwd(lib, N=0) == INVALID
    assert bwd(lib, N=2) == INVALID                            # several sequences need cu_seqlens
    assert bwd(lib, do=None) == INVALID
    assert bwd(lib, gla=None) == INVALID
    assert bwd(lib, ws=None, wsb=0) == WORKSPACE
    need = lib.kda_chunk_bwd_workspace_bytes(1, 10, 2, 128, 128, BF16)
    assert bwd(lib, wsb=need - 1) == WORKSPACE
    assert bwd(lib, gq=p(0)) == INVALID                        # dq aliases q
    assert bwd(lib, gk=p(6)) == INVALID                        # two gradients share memory
    assert bwd(lib, gb=p(5)) == INVALID                        # dbeta aliases d_o
    assert bwd(lib, ws=p(9)) == INVALID                        # workspace aliases dlog_alpha
    assert bwd(lib, gs0=p(12), s0=p(12)) == INVALID            # d_initial_state aliases initial_state
    assert bwd(lib, gv=ctypes.c_void_p(BASE + 8 * 64 * MB + 8)) == INVALID  # not 16-byte aligned
    assert bwd(lib, gb=ctypes.c_void_p(BASE + 10 * 64 * MB + 2)) == INVALID  # dbeta not 4-byte aligned


def fwd_save(lib, **kw):
    a = dict(q=p(0), k=p(1), v=p(2), la=p(3), b=p(4), s0=None, cu=None, N=1, T=10, H=2, dk_=128, dv_=128, dt=BF16,
             o=p(6), fs=None, ws=p(11), wsb=64 * MB)
    a.update(kw)
    return lib.kda_chunk_fwd_save(a["q"], a["k"], a["v"], a["la"], a["b"], a["s0"], a["cu"], a["N"], a["T"], a["H"],
                                  a["dk_"], a["dv_"], a["dt"], a["o"], a["fs"], a["ws"], a["wsb"], None)


def test_fwd_save_validation(lib):
    assert fwd_save(lib, dk_=64) == UNSUPPORTED
    assert fwd_save(lib, dt=3) == UNSUPPORTED
    assert fwd_save(lib, N=0) == INVALID
    assert fwd_save(lib, N=2) == INVALID                       # several sequences need cu_seqlens
    assert fwd_save(lib, o=None) == INVALID
    assert fwd_save(lib, ws=None, wsb=0) == WORKSPACE
    need = lib.kda_chunk_bwd_workspace_bytes(1, 10, 2, 128, 128, BF16)
    assert fwd_save(lib, wsb=need - 1) == WORKSPACE
    assert fwd_save(lib, o=p(1)) == INVALID                    # o aliases k
    assert fwd_save(lib, ws=p(3)) == INVALID                   # workspace aliases log_alpha
    assert fwd_save(lib, fs=p(6)) == INVALID                   # final state aliases o
    assert fwd_save(lib, s0=p(12), fs=ctypes.c_void_p(BASE + 12 * 64 * MB + 4096)) == INVALID  # partial overlap
    assert fwd_save(lib, o=ctypes.c_void_p(BASE + 6 * 64 * MB + 8)) == INVALID  # not 16-byte aligned
    assert fwd_save(lib, H=65536) == INVALID


def decode(lib, **kw):
    a = dict(s=p(0), q=p(1), k=p(2), v=p(3), la=p(4), b=p(5), N=2, H=2, dk=128, dv=128, dt=BF16, o=p(6))
    a.update(kw)
    return lib.kda_decode_step(a["s"], a["q"], a["k"], a["v"], a["la"], a["b"], a["N"], a["H"], a["dk"], a["dv"],
                               a["dt"], a["o"], None)


def test_decode_validation(lib):
    assert decode(lib, dk=64) == UNSUPPORTED
    assert decode(lib, dt=5) == UNSUPPORTED
    assert decode(lib, N=0) == INVALID
    assert decode(lib, s=None) == INVALID
    assert decode(lib, o=p(1)) == INVALID      # output aliases q
    assert decode(lib, s=p(2)) == INVALID      # state aliases k
    assert decode(lib, s=ctypes.c_void_p(BASE + 8)) == INVALID  # state not 16-byte aligned
    assert decode(lib, q=ctypes.c_void_p(BASE + 64 * MB + 1)) == INVALID  # not element aligned


def replay(lib, **kw):
    a = dict(s0=p(0), s1=p(0), q=p(1), k=p(2), v=p(3), la=p(4), b=p(5), nt=p(7), N=2, L=4, H=2, dk=128, dv=128,
             dt=BF16, opts=None, hq=None, hk=None, o=p(6))
    a.update(kw)
    return lib.kda_decode_replay(a["s0"], a["s1"], a["q"], a["k"], a["v"], a["la"], a["b"], a["nt"], a["N"],
                                 a["L"], a["H"], a["dk"], a["dv"], a["dt"], a["opts"], a["hq"], a["hk"], a["o"],
                                 None)


def test_replay_validation(lib):
    assert replay(lib, L=17) == UNSUPPORTED                  # more cached tokens than supported
    assert replay(lib, dk=64) == UNSUPPORTED
    assert replay(lib, L=0) == INVALID
    assert replay(lib, N=0) == INVALID
    assert replay(lib, q=None) == INVALID
    assert replay(lib, o=p(3)) == INVALID                    # output aliases v
    assert replay(lib, s1=p(1)) == INVALID                   # state output aliases q
    assert replay(lib, s1=ctypes.c_void_p(BASE + 4096)) == INVALID  # partial overlap with state_in
    assert replay(lib, s0=p(1), s1=p(1)) == INVALID          # in place, but the state is also q
    assert replay(lib, s1=p(6)) == INVALID                   # state output aliases o
    assert replay(lib, s0=ctypes.c_void_p(BASE + 8), s1=None) == INVALID  # not 16-byte aligned
    assert replay(lib, nt=ctypes.c_void_p(BASE + 7 * 64 * MB + 2)) == INVALID  # counts not 4-byte aligned
    wq = Opts(p(8).value, None, None, None, 1e-6, 1e-6, 0)
    assert replay(lib, opts=opts_p(wq)) == INVALID           # convolution without its history
    assert replay(lib, opts=opts_p(wq), hq=p(6)) == INVALID  # history aliases o
    assert replay(lib, opts=opts_p(wq), hq=p(8)) == INVALID  # history aliases the weights
    assert replay(lib, opts=opts_p(wq), hq=ctypes.c_void_p(BASE + 9 * 64 * MB + 8)) == INVALID  # alignment
    g = Opts(None, None, p(6).value, None, 1e-6, 1e-6, 0)
    assert replay(lib, opts=opts_p(g)) == INVALID            # gate aliases o
    neg = Opts(None, None, None, None, 1e-6, -1.0, 0)
    assert replay(lib, opts=opts_p(neg)) == INVALID          # negative epsilon
    unb = Opts(None, None, None, None, 1e-6, 1e-6, 0, 1)
    assert replay(lib, opts=opts_p(unb), L=17) == UNSUPPORTED  # the flag is accepted; sizes still checked
    assert replay(lib, opts=opts_p(unb), o=p(3)) == INVALID
    # nothing to produce: accepted without launching anything
    assert replay(lib, s1=None, o=None) == OK


def test_precondition_flags_start_clear(lib):
    L = ctypes.CDLL(LIB)
    L.kda_last_precondition_flags.restype = ctypes.c_uint32
    assert L.kda_last_precondition_flags() == 0
    assert "KDA_DEBUG_CHECKS" in lib.kda_status_string(5).decode()


def test_binding_fails_loudly_without_gpu_tensors():
    import gated_delta_rule_25_amd as kda
    x = torch.zeros(4, 2, 128)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(4, 2))


# ---------------------------------------------------------------------------
# Input generator recipe
# ---------------------------------------------------------------------------

def test_generator_recipe_and_determinism():
    import kda_inputs
    a = kda_inputs.make_prefill(3, [40, 0, 25], "bf16", 0.02, False, "cpu", seed=1)
    b = kda_inputs.make_prefill(3, [40, 0, 25], "bf16", 0.02, False, "cpu", seed=1)
    for key in ("q", "k", "v", "log_alpha", "beta", "initial_state"):
        assert torch.equal(a[key], b[key]), key
    la = a["log_alpha"]
    assert (la < 0).all() and (la > -5).all()
    assert (a["beta"] > 0).all() and (a["beta"] < 1).all()
    nq = a["q"].float().norm(dim=-1)
    assert torch.allclose(nq, torch.ones_like(nq), atol=1e-2)
    assert a["cu_host"].tolist() == [0, 40, 40, 65]
    # 16-token tiles of the drawn decay stay inside the pages' (-80, 0] range
    tiles = la[:32].reshape(2, 16, 3, 128).sum(1)
    assert (tiles > -80).all() and (tiles <= 0).all()


def test_varlen_lengths_loguniform():
    import kda_inputs
    L = kda_inputs.workload_lengths(4)
    assert len(L) == 64 and min(L) >= 1024 and max(L) <= 65536
    assert L == kda_inputs.workload_lengths(4)
    s = sum(L)
    assert 0.5e6 < s < 1.6e6


def test_c_consumer_compiles_as_c99(lib, tmp_path):
    """include/kda.h is valid C99: the plain C test program that calls every
    compute entry point compiles with gcc -std=c99 -Wall -Wextra -Werror and
    links against libkda.so and the HIP runtime (it is not run here)."""
    import sys
    sys.path.insert(0, os.path.join(ROOT, "tests", "c_abi"))
    import build_abi_check
    out = str(tmp_path / "abi_check")
    try:
        build_abi_check.build(out)
    except subprocess.CalledProcessError as e:
        pytest.fail("gcc failed:\n" + e.stderr)
    dyn = subprocess.run(["readelf", "-d", out], check=True, capture_output=True, text=True).stdout
    assert "libkda.so" in dyn and "libamdhip64" in dyn


def test_fused_opts_layout_matches_header():
    """The ctypes mirrors of kda_fused_opts (the binding's and this file's)
    list the header's fields in order with matching C types, so a field added
    to the header cannot be read past the end of a Python-built struct."""
    import gated_delta_rule_25_amd as kda
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} kda_fused_opts;", text, re.S).group(1)
    fields = re.findall(r"^\s*(const \w+\*|\w+)\s+(\w+);", body, re.M)
    kinds = {"const float*": ctypes.c_void_p, "const void*": ctypes.c_void_p, "float": ctypes.c_float,
             "int": ctypes.c_int}
    want = [(name, kinds[t]) for t, name in fields]
    assert [n for n, _ in want] == ["conv_q_w", "conv_k_w", "gate", "norm_w", "l2_eps", "rms_eps",
                                    "segment_tokens", "unbounded_decay", "factor_budget_mib"]
    for mirror in (kda._FusedOpts, Opts):
        assert [(n, t) for n, t in mirror._fields_] == want, mirror
        assert ctypes.sizeof(mirror) == 56
