"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the KDA recurrence.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library's compute path
(``gated_delta_rule_25_amd``) never imports it, and it never imports that
package: the two share no code.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, one token at a
time); this module only builds it with gcc, loads it with ctypes and
marshals numpy arrays.  See that file's header for what is computed and the
passages of the pages it follows.

Pins (tests/test_oracle_pins.py, tests/test_oracle_replay_pins.py,
tests/test_oracle_bwd_pins.py) tie it to the pages' worked examples, closed
forms, brute-force products, for the multi-token decode to the prefill run
over the same tokens, and for the backward pass to central finite
differences of the forward, closed forms and exact homogeneity identities.  The prologue/epilogue epsilon values
and the convolution tap order are fixed only by our own reading of the pages
(they print no numbers for them): parity unpinned for those constants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c into libkda_oracle.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_chunk_fwd.restype = ctypes.c_int
        lib.kda_oracle_chunk_fwd.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int64),
                                             ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, dp, dp, dp, dp, ctypes.c_double,
                                             ctypes.c_double, dp, dp, ctypes.c_int]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, dp, ctypes.c_int]
        lib.kda_oracle_decode_multi.restype = ctypes.c_int
        lib.kda_oracle_decode_multi.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int64),
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                                ctypes.c_double, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_chunk_bwd.restype = ctypes.c_int
        lib.kda_oracle_chunk_bwd.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                             dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def chunk_fwd(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None, *, conv_q_w=None,
              conv_k_w=None, gate=None, norm_w=None, l2_eps=1e-6, rms_eps=1e-6, threads=0):
    """Per-token fp64 recurrence over a packed batch.

    q, k, log_alpha: [T, H, dk]; v (and gate): [T, H, dv]; beta: [T, H];
    initial_state: [N, H, dk, dv] or None (zeros); cu_seqlens: [N+1] or None
    (one sequence).  Returns (o [T, H, dv], final_state [N, H, dk, dv]).
    """
    lib = _load()
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and la.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert b.shape == (T, H)
    if cu_seqlens is None:
        N, cu = 1, None
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0 = _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    cq, ck, g, nw = _f64(conv_q_w), _f64(conv_k_w), _f64(gate), _f64(norm_w)
    if cq is not None:
        assert cq.shape == (H * dk, 4)
    if ck is not None:
        assert ck.shape == (H * dk, 4)
    if g is not None:
        assert g.shape == (T, H, dv)
    if nw is not None:
        assert nw.shape == (dv,)
    o = np.zeros((T, H, dv), dtype=np.float64)
    fs = np.zeros((N, H, dk, dv), dtype=np.float64)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.kda_oracle_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(s0), cu_p, N, T,
                                  H, dk, dv, _ptr(cq), _ptr(ck), _ptr(g), _ptr(nw), float(l2_eps),
                                  float(rms_eps), _ptr(o), _ptr(fs), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_chunk_fwd failed with code %d" % rc)
    return o, fs


def chunk_bwd(q, k, v, log_alpha, beta, d_o, initial_state=None, cu_seqlens=None, d_final_state=None,
              threads=0):
    """Gradients of L = sum_t <d_o_t, o_t> + <d_final_state, S_T> through the
    per-token recurrence (no prologue or epilogue).

    Shapes as chunk_fwd; d_o [T, H, dv]; d_final_state [N, H, dk, dv] or None
    (zero).  Returns (dq, dk, dv, dlog_alpha, dbeta, d_initial_state) with the
    shapes of q, k, v, log_alpha, beta and [N, H, dk, dv].
    """
    lib = _load()
    q, k, v, la, b, do = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta), _f64(d_o)
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and la.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert b.shape == (T, H) and do.shape == (T, H, dv)
    if cu_seqlens is None:
        N, cu = 1, None
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0, dsT = _f64(initial_state), _f64(d_final_state)
    for x in (s0, dsT):
        if x is not None:
            assert x.shape == (N, H, dk, dv)
    gq, gk, gla = (np.zeros((T, H, dk)) for _ in range(3))
    gv = np.zeros((T, H, dv))
    gb = np.zeros((T, H))
    gs0 = np.zeros((N, H, dk, dv))
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.kda_oracle_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(s0), cu_p, N, T, H, dk, dv,
                                  _ptr(do), _ptr(dsT), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gla), _ptr(gb),
                                  _ptr(gs0), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_chunk_bwd failed with code %d" % rc)
    return gq, gk, gv, gla, gb, gs0


def decode_step(state, q, k, v, log_alpha, beta, threads=0):
    """One token per (n, h).  ``state`` [N, H, dk, dv] float64 C-contiguous is
    updated in place; q, k, log_alpha [N, H, dk]; v [N, H, dv]; beta [N, H].
    Returns o [N, H, dv]."""
    lib = _load()
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous):
        raise TypeError("state must be a C-contiguous float64 numpy array (updated in place)")
    N, H, dk, dv = state.shape
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    assert q.shape == (N, H, dk) and k.shape == (N, H, dk) and la.shape == (N, H, dk)
    assert v.shape == (N, H, dv) and b.shape == (N, H)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.kda_oracle_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), N, H, dk,
                                    dv, _ptr(o), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_step failed with code %d" % rc)
    return o


def decode_multi(state, q, k, v, log_alpha, beta, num_tokens=None, *, conv_q_w=None, conv_k_w=None,
                 conv_q_hist=None, conv_k_hist=None, gate=None, norm_w=None, l2_eps=1e-6, rms_eps=1e-6,
                 threads=0):
    """Multi-token decode (speculative-decoding replay) from cached inputs.

    state: [N, H, dk, dv] or None (zeros); q, k, log_alpha: [N, L, H, dk];
    v (and gate): [N, L, H, dv]; beta: [N, L, H]; num_tokens: [N] tokens to
    run per sequence (clamped to [0, L]) or None (all L); conv_*_hist:
    [N, 3, H, dk] raw rows before token 0, oldest first, or None (zeros).
    Returns (o [N, L, H, dv] with zero rows past each sequence's count,
    state after the tokens [N, H, dk, dv], q history and k history after
    them [N, 3, H, dk]).
    """
    lib = _load()
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    N, L, H, dk = q.shape
    dv = v.shape[3]
    assert k.shape == (N, L, H, dk) and la.shape == (N, L, H, dk) and v.shape == (N, L, H, dv)
    assert b.shape == (N, L, H)
    s0 = _f64(state)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    nt = None
    if num_tokens is not None:
        nt = np.ascontiguousarray(np.asarray(num_tokens, dtype=np.int64))
        assert nt.shape == (N,)
    cq, ck, hq, hk = _f64(conv_q_w), _f64(conv_k_w), _f64(conv_q_hist), _f64(conv_k_hist)
    g, nw = _f64(gate), _f64(norm_w)
    for w_ in (cq, ck):
        if w_ is not None:
            assert w_.shape == (H * dk, 4)
    for h_ in (hq, hk):
        if h_ is not None:
            assert h_.shape == (N, 3, H, dk)
    if g is not None:
        assert g.shape == (N, L, H, dv)
    if nw is not None:
        assert nw.shape == (dv,)
    o = np.zeros((N, L, H, dv), dtype=np.float64)
    s1 = np.zeros((N, H, dk, dv), dtype=np.float64)
    oq = np.zeros((N, 3, H, dk), dtype=np.float64)
    ok = np.zeros((N, 3, H, dk), dtype=np.float64)
    nt_p = None if nt is None else nt.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.kda_oracle_decode_multi(_ptr(s0), _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), nt_p, N, L, H,
                                     dk, dv, _ptr(cq), _ptr(ck), _ptr(hq), _ptr(hk), _ptr(g), _ptr(nw),
                                     float(l2_eps), float(rms_eps), _ptr(o), _ptr(s1), _ptr(oq), _ptr(ok),
                                     int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_multi failed with code %d" % rc)
    return o, s1, oq, ok
