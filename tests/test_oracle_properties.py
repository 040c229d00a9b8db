"""Randomised invariants of the fp64 oracle (hypothesis; CPU only).

The fixed-case pins in test_oracle_pins.py and test_oracle_replay_pins.py
check each invariant on a few chosen inputs; these draw shapes and values at
random (tiny d, short sequences, empty sequences, extreme beta and decay) so
that an index or boundary slip that only some shapes expose still fails:
- the explicit dense unrolling of the recurrence (brute force);
- the affine structure of a segment ("Kimi K3 架构…" section 7.1, KCP);
- varlen packing = separate runs; token-by-token decode = prefill;
- replaying cached tokens = the tail of one prefill ("Kimi K3 架构…" 7.4).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def draw_problem(seed, T, H, dk, dv, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -5.0 * rng.random((T, H, dk))
    b = rng.random((T, H))
    b[rng.random((T, H)) < 0.2] = 1.0  # exact projections
    b[rng.random((T, H)) < 0.1] = 0.0  # pure decayed reads
    return q, k, v, la, b, rng


@SETTINGS
@given(seed=st.integers(0, 2**31), T=st.integers(1, 6), dk=st.sampled_from([1, 2, 3, 4]),
       dv=st.sampled_from([1, 2, 5]))
def test_dense_unroll(seed, T, dk, dv):
    q, k, v, la, b, rng = draw_problem(seed, T, 1, dk, dv)
    s0 = rng.standard_normal((1, 1, dk, dv))
    o, fs = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0)
    S = s0[0, 0].copy()
    for t in range(T):
        kt, qt = k[t, 0], q[t, 0]
        A = (np.eye(dk) - b[t, 0] * np.outer(kt, kt)) @ np.diag(np.exp(la[t, 0]))
        S = A @ S + b[t, 0] * np.outer(kt, v[t, 0])
        np.testing.assert_allclose(o[t, 0], S.T @ qt, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fs[0, 0], S, rtol=1e-10, atol=1e-12)


@SETTINGS
@given(seed=st.integers(0, 2**31), T=st.integers(2, 40), H=st.integers(1, 3), d=st.sampled_from([2, 4, 8]),
       cut=st.floats(0.0, 1.0))
def test_affine_segment(seed, T, H, d, cut):
    q, k, v, la, b, rng = draw_problem(seed, T, H, d, d)
    s0 = rng.standard_normal((1, H, d, d))
    t = int(round(cut * T))
    o, fs = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0)
    o1, fs1 = oracle.chunk_fwd(q[:t], k[:t], v[:t], la[:t], b[:t], initial_state=s0)
    o2, fs2 = oracle.chunk_fwd(q[t:], k[t:], v[t:], la[t:], b[t:], initial_state=fs1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fs2, fs, rtol=1e-11, atol=1e-12)
    _, B = oracle.chunk_fwd(q, k, v, la, b)
    eye = np.broadcast_to(np.eye(d), (1, H, d, d)).copy()
    _, M = oracle.chunk_fwd(q, k, np.zeros_like(v), la, b, initial_state=eye)
    np.testing.assert_allclose(M[0] @ s0[0] + B[0], fs[0], rtol=1e-10, atol=1e-11)


@SETTINGS
@given(seed=st.integers(0, 2**31), lens=st.lists(st.integers(0, 12), min_size=1, max_size=6), H=st.integers(1, 3))
def test_varlen_and_decode(seed, lens, H):
    d = 4
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    if T == 0:
        return
    q, k, v, la, b, rng = draw_problem(seed, T, H, d, d)
    s0 = rng.standard_normal((len(lens), H, d, d))
    o, fs = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        state = s0[n:n + 1].copy()
        for t in range(a, e):
            ot = oracle.decode_step(state, q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], b[t:t + 1])
            np.testing.assert_allclose(ot[0], o[t], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(state[0], fs[n], rtol=1e-12, atol=1e-13)


@SETTINGS
@given(seed=st.integers(0, 2**31), P=st.integers(0, 7), L=st.integers(1, 9), H=st.integers(1, 2),
       conv=st.booleans(), gate=st.booleans())
def test_replay_is_prefill_tail(seed, P, L, H, conv, gate):
    d = 4
    T = P + L
    q, k, v, la, b, rng = draw_problem(seed, T, H, d, d, unit=not conv)
    s0 = rng.standard_normal((1, H, d, d))
    wq = rng.standard_normal((H * d, 4)) if conv else None
    wk = rng.standard_normal((H * d, 4)) if conv else None
    g = rng.standard_normal((T, H, d)) if gate else None
    kw = dict(conv_q_w=wq, conv_k_w=wk)
    o_full, fs_full = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, gate=g, **kw)
    _, fs_p = oracle.chunk_fwd(q[:P], k[:P], v[:P], la[:P], b[:P], initial_state=s0,
                               gate=None if g is None else g[:P], **kw)
    hist = lambda x: np.stack([x[P - 3 + r] if P - 3 + r >= 0 else np.zeros((H, d)) for r in range(3)])[None]
    o, s1, hq, hk = oracle.decode_multi(fs_p, q[None, P:], k[None, P:], v[None, P:], la[None, P:], b[None, P:],
                                        conv_q_hist=hist(q) if conv else None, conv_k_hist=hist(k) if conv else None,
                                        gate=None if g is None else g[None, P:], **kw)
    np.testing.assert_allclose(o[0], o_full[P:], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s1, fs_full, rtol=1e-10, atol=1e-12)
    if conv:
        np.testing.assert_array_equal(hq[0], np.stack([q[T - 3 + r] if T - 3 + r >= 0 else np.zeros((H, d))
                                                       for r in range(3)]))
