"""Pins of the oracle's multi-token decode (speculative-decoding replay).

"Kimi K3 架构、训练与系统全景解析", section 7.4 (KDA state replay under
speculative decoding): the per-token inputs of the draft tokens are kept,
the accepted prefix is replayed from the verified state inside one fused
kernel (short convolution, norms, gate, recurrence), and only the final
state is written back.  What the replay computes is therefore fixed by the
recurrence itself: replaying tokens from a state equals running them as the
tail of one longer sequence.  The tests below check that against the
prefill path (itself pinned in test_oracle_pins.py), plus closed forms that
fix the convolution history's orientation and the truncation rule.  CPU only.
"""
import numpy as np

import oracle

RNG = np.random.default_rng(20261203)


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def silu(x):
    return x / (1.0 + np.exp(-x))


def l2(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def tokens(N, L, H, dk, dv, rng=RNG):
    """Raw per-token inputs [N, L, H, ...] shaped like the pages' decode workload."""
    q = rng.standard_normal((N, L, H, dk))
    k = rng.standard_normal((N, L, H, dk))
    v = rng.standard_normal((N, L, H, dv))
    la = -5.0 / (1.0 + np.exp(-rng.standard_normal((N, L, H, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, L, H))))
    return q, k, v, la, b


def test_replay_is_the_tail_of_a_prefill():
    """Replaying L tokens from the state after a prefix P, with the prefix's
    last three raw rows as the convolution history, gives the prefill's
    outputs for those L tokens, its final state, and the last three raw rows
    as the new history.  Prefix lengths 0, 1, 2 and 5 cover a history that
    is all zeros, partly zeros and full."""
    H, dk, dv, L = 2, 8, 6, 5
    wq = RNG.standard_normal((H * dk, 4)) * 0.5
    wk = RNG.standard_normal((H * dk, 4)) * 0.5
    for P in (0, 1, 2, 5):
        T = P + L
        q, k, v, la, b = (x[0] for x in tokens(1, T, H, dk, dv))
        g = RNG.standard_normal((T, H, dv))
        nw = RNG.standard_normal(dv)
        s0 = RNG.standard_normal((1, H, dk, dv))
        o_full, fs_full = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, conv_q_w=wq, conv_k_w=wk,
                                           gate=g, norm_w=nw)
        _, fs_p = oracle.chunk_fwd(q[:P], k[:P], v[:P], la[:P], b[:P], initial_state=s0, conv_q_w=wq,
                                   conv_k_w=wk, gate=g[:P], norm_w=nw)
        hist_q = np.zeros((1, 3, H, dk))
        hist_k = np.zeros((1, 3, H, dk))
        for r in range(3):
            if P - 3 + r >= 0:
                hist_q[0, r] = q[P - 3 + r]
                hist_k[0, r] = k[P - 3 + r]
        o, s1, hq, hk = oracle.decode_multi(fs_p, q[None, P:], k[None, P:], v[None, P:], la[None, P:],
                                            b[None, P:], conv_q_w=wq, conv_k_w=wk, conv_q_hist=hist_q,
                                            conv_k_hist=hist_k, gate=g[None, P:], norm_w=nw)
        np.testing.assert_allclose(o[0], o_full[P:], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s1, fs_full, rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(hq[0], q[T - 3:T])
        np.testing.assert_array_equal(hk[0], k[T - 3:T])


def test_history_orientation_closed_form():
    """With beta = 0 and log_alpha = 0 the state never changes, so
    o_t = S0^T q'_t.  With one-hot taps on the oldest row, q'_t =
    L2(SiLU(x_{t-3})): token 0 reads history row 0 (the oldest), token 2
    reads history row 2, token 3 reads cached token 0."""
    N, L, H, d = 2, 6, 3, 8
    q, k, v, la, b = tokens(N, L, H, d, d)
    la[:] = 0.0
    b[:] = 0.0
    s0 = RNG.standard_normal((N, H, d, d))
    hist = RNG.standard_normal((N, 3, H, d))
    w_old = np.tile([1.0, 0.0, 0.0, 0.0], (H * d, 1))
    o, s1, hq, _ = oracle.decode_multi(s0, q, k, v, la, b, conv_q_w=w_old, conv_q_hist=hist)
    rows = np.concatenate([hist, q], axis=1)  # positions -3 .. L-1
    for t in range(L):
        qp = l2(silu(rows[:, t]))  # x_{t-3}
        np.testing.assert_allclose(o[:, t], np.einsum("nhij,nhi->nhj", s0, qp), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_array_equal(hq, q[:, L - 3:])


def test_unit_key_projection_after_prologue():
    """The prologue's L2 makes k'_t a unit vector, so with beta = 1 on a
    sequence's last token the state after it satisfies S^T k' = v exactly
    (derived from the update: (I - k k^T) k = 0).  Identity taps make
    k' = L2(SiLU(k)) in closed form."""
    N, L, H, d = 3, 4, 2, 8
    q, k, v, la, b = tokens(N, L, H, d, d)
    b[:, L - 1] = 1.0
    s0 = RNG.standard_normal((N, H, d, d))
    w_id = np.tile([0.0, 0.0, 0.0, 1.0], (H * d, 1))
    _, s1, _, _ = oracle.decode_multi(s0, q, k, v, la, b, conv_k_w=w_id, conv_k_hist=np.zeros((N, 3, H, d)),
                                      l2_eps=0.0)
    kp = l2(silu(k[:, L - 1]), eps=0.0)
    np.testing.assert_allclose(np.einsum("nhij,nhi->nhj", s1, kp), v[:, L - 1], rtol=1e-11, atol=1e-12)


def test_truncation_to_accepted_count():
    """num_tokens[n] = a runs exactly the first a cached tokens: the same as a
    call holding only those a tokens.  Rows past a are not written, and the
    new history is the three raw rows before token a (reaching back into the
    old history when a < 3).  a = 0 leaves state and history as they were."""
    N, L, H, d = 5, 6, 2, 8
    q, k, v, la, b = tokens(N, L, H, d, d)
    g = RNG.standard_normal((N, L, H, d))
    s0 = RNG.standard_normal((N, H, d, d))
    hq0 = RNG.standard_normal((N, 3, H, d))
    hk0 = RNG.standard_normal((N, 3, H, d))
    w = RNG.standard_normal((H * d, 4))
    acc = np.array([0, 1, 2, 4, 6])
    kw = dict(conv_q_w=w, conv_k_w=w[::-1].copy(), conv_q_hist=hq0, conv_k_hist=hk0, gate=g)
    o, s1, hq, hk = oracle.decode_multi(s0, q, k, v, la, b, acc, **kw)
    for n, a in enumerate(acc):
        np.testing.assert_array_equal(o[n, a:], 0.0)
        rows_q = np.concatenate([hq0[n], q[n]])
        rows_k = np.concatenate([hk0[n], k[n]])
        np.testing.assert_array_equal(hq[n], rows_q[a:a + 3])
        np.testing.assert_array_equal(hk[n], rows_k[a:a + 3])
        if a == 0:
            np.testing.assert_array_equal(s1[n], s0[n])
            continue
        sl = slice(n, n + 1)
        kw_n = dict(conv_q_w=w, conv_k_w=w[::-1].copy(), conv_q_hist=hq0[sl], conv_k_hist=hk0[sl],
                    gate=g[sl, :a])
        on, sn, _, _ = oracle.decode_multi(s0[sl], q[sl, :a], k[sl, :a], v[sl, :a], la[sl, :a], b[sl, :a],
                                           **kw_n)
        np.testing.assert_allclose(o[n, :a], on[0], rtol=1e-14, atol=0)
        np.testing.assert_allclose(s1[n], sn[0], rtol=1e-14, atol=0)
    # counts outside [0, L] are clamped
    o_c, s_c, _, _ = oracle.decode_multi(s0, q, k, v, la, b, np.array([-3, 9, 2, 4, 6]), **kw)
    np.testing.assert_array_equal(s_c[0], s0[0])
    o_all, s_all, _, _ = oracle.decode_multi(s0, q, k, v, la, b, **kw)
    np.testing.assert_array_equal(s_c[1], s_all[1])
    np.testing.assert_array_equal(o_c[1], o_all[1])


def test_single_token_without_prologue_is_one_decode_step():
    """L = 1 with no prologue or epilogue is one in-place decode step."""
    N, H, d = 3, 2, 8
    q, k, v, la, b = tokens(N, 1, H, d, d)
    q, k = unit_rows(q), unit_rows(k)
    s0 = RNG.standard_normal((N, H, d, d))
    o, s1, _, _ = oracle.decode_multi(s0, q, k, v, la, b)
    state = s0.copy()
    o_ref = oracle.decode_step(state, q[:, 0], k[:, 0], v[:, 0], la[:, 0], b[:, 0])
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=1e-14, atol=0)
    np.testing.assert_allclose(s1, state, rtol=1e-14, atol=0)
