"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names the passage (page title + section) or the mathematical fact
it checks.  They are chosen so that a plausible slip in the oracle — a
dropped term, the decay on the wrong axis, the read before the write, the
correction read from the undecayed state, a transposed state — fails one of
them.  CPU only.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(20261202)


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def one_head(q, k, v, la, b):
    """Add the head axis (H=1) to per-token arrays."""
    return q[:, None, :], k[:, None, :], v[:, None, :], la[:, None, :], b[:, None]


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------

def test_write_then_query_2d(golden):
    """AI-Workshop #15, section 7.2: two one-hot keys written with their values
    read back exactly by one-hot queries; the state equals [v1^T; v2^T]."""
    ex = golden["write_then_query_2d"]
    v_place = np.array([0.3, -1.2, 2.0])
    v_job = np.array([-0.7, 0.4, 1.1])
    k1, k2 = np.array(ex["k_place"]), np.array(ex["k_job"])
    # tokens: write place, write job, then two pure reads (beta = 0, no decay)
    k = np.stack([k1, k2, k1, k2])
    v = np.stack([v_place, v_job, np.zeros(3), np.zeros(3)])
    q = np.stack([k1, k2, np.array(ex["q_place"]), np.array(ex["q_job"])])
    b = np.array([1.0, 1.0, 0.0, 0.0])
    la = np.zeros((4, 2))
    o, fs = oracle.chunk_fwd(*one_head(q, k, v, la, b))
    np.testing.assert_allclose(o[2, 0], v_place, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[3, 0], v_job, rtol=0, atol=1e-15)
    np.testing.assert_allclose(fs[0, 0], np.stack([v_place, v_job]), rtol=0, atol=1e-15)


def test_orthonormal_retrieval_d128():
    """The same write-then-query fact at d = 128 with a random orthonormal key
    basis: beta = 1, alpha = 1, S0 = 0 retrieves every stored value exactly."""
    d, m = 128, 128
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    keys = Qm.T[:m]
    vals = RNG.standard_normal((m, d))
    # m writes followed by m reads (beta = 0) with q = k_j
    k = np.concatenate([keys, keys])
    q = np.concatenate([keys, keys])
    v = np.concatenate([vals, np.zeros_like(vals)])
    b = np.concatenate([np.ones(m), np.zeros(m)])
    la = np.zeros((2 * m, d))
    o, _ = oracle.chunk_fwd(*one_head(q, k, v, la, b))
    np.testing.assert_allclose(o[m:, 0], vals, rtol=0, atol=1e-12)
    # during the write phase, reading with the key just written returns its value
    np.testing.assert_allclose(o[:m, 0], vals, rtol=0, atol=1e-12)


def test_delta_scalar_example(golden):
    """AI-Workshop #15, section 7.2 'Delta' paragraph: old read-out 0.7, new
    value 0.9, beta 0.5 -> 0.7 + 0.5 * 0.2 = 0.8."""
    ex = golden["delta_scalar"]
    s0 = np.array([[[[ex["vhat_old"]]]]])
    one = np.ones((1, 1, 1))
    o, fs = oracle.chunk_fwd(one, one, np.full((1, 1, 1), ex["v_new"]), np.zeros((1, 1, 1)),
                             np.full((1, 1), ex["beta"]), initial_state=s0)
    assert abs(o[0, 0, 0] - ex["expect"]) < 1e-15
    assert abs(fs[0, 0, 0, 0] - ex["expect"]) < 1e-15


def test_overwrite_same_key():
    """AI-Workshop #15, section 7.2 (the moving-house story) and the delta-rule
    erase of "Kimi K3 架构…" section 4.2.2: writing (k, v_new) with beta = 1
    after (k, v_old) leaves S^T k = v_new and keeps an orthogonal key's value."""
    d = 16
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    ka, kb = Qm[:, 0], Qm[:, 1]
    v_old, v_new, v_b = RNG.standard_normal((3, d))
    k = np.stack([ka, kb, ka, ka, kb])
    v = np.stack([v_old, v_b, v_new, np.zeros(d), np.zeros(d)])
    q = np.stack([ka, kb, ka, ka, kb])
    b = np.array([1.0, 1.0, 1.0, 0.0, 0.0])
    o, _ = oracle.chunk_fwd(*one_head(q, k, v, np.zeros((5, d)), b))
    np.testing.assert_allclose(o[3, 0], v_new, atol=1e-13)
    np.testing.assert_allclose(o[4, 0], v_b, atol=1e-13)


# ---------------------------------------------------------------------------
# Closed forms and special cases
# ---------------------------------------------------------------------------

def test_beta_zero_is_pure_decay_read():
    """beta = 0: nothing is written, so o_t = S0^T (exp(g_t) * q_t) with g_t the
    inclusive cumulative log-decay; with alpha = 1 this is o_t = S0^T q_t."""
    T, dk, dv = 9, 8, 5
    q = RNG.standard_normal((T, dk))
    k = unit_rows(RNG.standard_normal((T, dk)))
    v = RNG.standard_normal((T, dv))
    la = -5.0 / (1.0 + np.exp(-RNG.standard_normal((T, dk))))
    s0 = RNG.standard_normal((1, 1, dk, dv))
    b = np.zeros(T)
    o, fs = oracle.chunk_fwd(*one_head(q, k, v, la, b), initial_state=s0)
    g = np.cumsum(la, axis=0)
    expect = (np.exp(g) * q) @ s0[0, 0]
    np.testing.assert_allclose(o[:, 0], expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fs[0, 0], np.exp(g[-1])[:, None] * s0[0, 0], rtol=1e-13)
    o1, _ = oracle.chunk_fwd(*one_head(q, k, v, np.zeros_like(la), b), initial_state=s0)
    np.testing.assert_allclose(o1[:, 0], q @ s0[0, 0], rtol=1e-13, atol=1e-14)


def test_beta_one_unit_key_projects_exactly():
    """beta = 1 and ||k|| = 1: (I - k k^T) k = 0, so after every token
    S_t^T k_t = v_t whatever the decay and the earlier state."""
    T, d = 12, 16
    k = unit_rows(RNG.standard_normal((T, d)))
    v = RNG.standard_normal((T, d))
    la = -5.0 / (1.0 + np.exp(-RNG.standard_normal((T, d))))
    s0 = RNG.standard_normal((1, 1, d, d))
    o, _ = oracle.chunk_fwd(*one_head(k, k, v, la, np.ones(T)), initial_state=s0)
    np.testing.assert_allclose(o[:, 0], v, atol=1e-12)


def test_scalar_closed_form():
    """d = 1: s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t and
    o_t = s_t q_t, the scalar case of the update equation."""
    T = 20
    q, k, v = RNG.standard_normal((3, T))
    la = -5.0 / (1.0 + np.exp(-RNG.standard_normal(T)))
    b = 1.0 / (1.0 + np.exp(-RNG.standard_normal(T)))
    s = 0.37
    expect = []
    for t in range(T):
        s = np.exp(la[t]) * (1 - b[t] * k[t] ** 2) * s + b[t] * k[t] * v[t]
        expect.append(s * q[t])
    o, fs = oracle.chunk_fwd(q[:, None, None], k[:, None, None], v[:, None, None], la[:, None, None],
                             b[:, None], initial_state=np.full((1, 1, 1, 1), 0.37))
    np.testing.assert_allclose(o[:, 0, 0], expect, rtol=1e-13)
    assert abs(fs[0, 0, 0, 0] - s) < 1e-13


@pytest.mark.parametrize("d", [1, 2, 4, 8])
def test_brute_force_dense_unroll(d):
    """Explicit product form of the update equation on tiny T:
    A_t = (I - b_t k_t k_t^T) Diag(alpha_t),
    S_t = A_t...A_1 S0 + sum_i A_t...A_{i+1} b_i k_i v_i^T,  o_t = S_t^T q_t."""
    T, dv = 6, d + 1
    q = RNG.standard_normal((T, d))
    k = unit_rows(RNG.standard_normal((T, d)))
    v = RNG.standard_normal((T, dv))
    la = -5.0 / (1.0 + np.exp(-RNG.standard_normal((T, d))))
    b = 1.0 / (1.0 + np.exp(-RNG.standard_normal(T)))
    s0 = RNG.standard_normal((d, dv))
    A = [(np.eye(d) - b[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(la[t])) for t in range(T)]

    def prod(hi, lo):  # A_hi ... A_{lo+1}  (1-based token indices)
        M = np.eye(d)
        for t in range(lo + 1, hi + 1):
            M = A[t - 1] @ M
        return M

    o_ref = []
    for t in range(1, T + 1):
        S = prod(t, 0) @ s0 + sum(prod(t, i) @ (b[i - 1] * np.outer(k[i - 1], v[i - 1]))
                                  for i in range(1, t + 1))
        o_ref.append(S.T @ q[t - 1])
    o, fs = oracle.chunk_fwd(*one_head(q, k, v, la, b), initial_state=s0[None, None])
    np.testing.assert_allclose(o[:, 0], np.array(o_ref), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fs[0, 0], S, rtol=1e-12, atol=1e-13)


def test_decay_acts_on_key_rows():
    """"Kimi K3 架构…" section 4.2.2: each KEY channel keeps its own share of the
    old state, i.e. Diag(alpha) multiplies the rows (d_k index) of S.  With
    beta = 0 and a decay on key channel 3 only, only row 3 shrinks."""
    T, d = 7, 8
    la = np.zeros((T, d))
    la[:, 3] = -0.5
    s0 = RNG.standard_normal((1, 1, d, d))
    z = np.zeros((T, d))
    _, fs = oracle.chunk_fwd(*one_head(z, z, z, la, np.zeros(T)), initial_state=s0)
    expect = s0[0, 0].copy()
    expect[3, :] *= np.exp(-0.5 * T)
    np.testing.assert_allclose(fs[0, 0], expect, rtol=1e-14)


def test_read_after_write():
    """Study notes section 3-2 item 2): the output reads S_t, the state AFTER the
    token's own write.  From S0 = 0, one token with k = q = e1, beta = 1
    returns v (a read before the write would return 0)."""
    d = 4
    e1 = np.eye(d)[0]
    v = np.array([1.5, -2.0, 0.25, 3.0])
    o, _ = oracle.chunk_fwd(e1[None, None], e1[None, None], v[None, None], np.zeros((1, 1, d)),
                            np.ones((1, 1)))
    np.testing.assert_allclose(o[0, 0], v, atol=1e-15)


def test_decay_before_erase():
    """Study notes section 3-2 item 2) applies (I - b k k^T) to Diag(alpha) S:
    the correction reads the DECAYED state.  With row 1 of S0 = w, alpha = 0.5,
    k = e1, beta = 1, v = 0 the row is erased to exactly 0 and the other rows are
    halved.  (The talk's simplified teaching formula, which reads the undecayed
    state, would leave -0.5 w in that row.)"""
    d = 4
    s0 = RNG.standard_normal((1, 1, d, d))
    e1 = np.eye(d)[0]
    la = np.full((1, 1, d), np.log(0.5))
    o, fs = oracle.chunk_fwd(e1[None, None], e1[None, None], np.zeros((1, 1, d)), la, np.ones((1, 1)),
                             initial_state=s0)
    expect = 0.5 * s0[0, 0]
    expect[0, :] = 0.0
    np.testing.assert_allclose(fs[0, 0], expect, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], np.zeros(d), atol=1e-15)


# ---------------------------------------------------------------------------
# Structural invariants
# ---------------------------------------------------------------------------

def random_problem(T, H, dk, dv, rng=RNG):
    q = unit_rows(rng.standard_normal((T, H, dk)))
    k = unit_rows(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    la = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, la, b


def test_affine_composition_and_resume():
    """"Kimi K3 架构…" section 7.1 (KCP): a segment acts on its incoming state as
    an affine map S -> M S + B.  So (i) running [0, T) equals running [t, T)
    from the state after [0, t); (ii) S_T = M S0 + B, with B the run from
    S0 = 0 and M the run with V = 0 started from S0 = I."""
    T, H, d = 37, 2, 6
    q, k, v, la, b = random_problem(T, H, d, d)
    s0 = RNG.standard_normal((1, H, d, d))
    o_full, fs_full = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0)
    t = 15
    o1, fs1 = oracle.chunk_fwd(q[:t], k[:t], v[:t], la[:t], b[:t], initial_state=s0)
    o2, fs2 = oracle.chunk_fwd(q[t:], k[t:], v[t:], la[t:], b[t:], initial_state=fs1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fs2, fs_full, rtol=1e-12, atol=1e-13)
    _, B = oracle.chunk_fwd(q, k, v, la, b)
    eye = np.broadcast_to(np.eye(d), (1, H, d, d)).copy()
    _, M = oracle.chunk_fwd(q, k, np.zeros_like(v), la, b, initial_state=eye)
    np.testing.assert_allclose(np.einsum("hij,hjk->hik", M[0], s0[0]) + B[0], fs_full[0],
                               rtol=1e-12, atol=1e-13)


def test_varlen_equals_separate_runs():
    """Packed sequences are independent: a packed run with cu_seqlens equals
    separate runs, including empty and one-token sequences."""
    H, d = 3, 5
    lens = [7, 0, 1, 12, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, la, b = random_problem(T, H, d, d)
    s0 = RNG.standard_normal((len(lens), H, d, d))
    o, fs = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        on, fsn = oracle.chunk_fwd(q[a:e], k[a:e], v[a:e], la[a:e], b[a:e],
                                   initial_state=s0[n:n + 1])
        np.testing.assert_allclose(o[a:e], on, rtol=1e-14, atol=0)
        np.testing.assert_allclose(fs[n], fsn[0], rtol=1e-14, atol=0)
    np.testing.assert_allclose(fs[1], s0[1], rtol=0, atol=0)  # empty sequence keeps its state


def test_decode_steps_equal_prefill():
    """Decoding token by token in place ("Kimi K3 架构…" section 4.2.7) gives the
    same outputs and final state as one prefill over the same tokens."""
    T, N, H, d = 16, 2, 3, 8
    q, k, v, la, b = random_problem(T * N, H, d, d)
    s0 = RNG.standard_normal((N, H, d, d))
    cu = np.arange(N + 1) * T
    o_pf, fs_pf = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, cu_seqlens=cu)
    state = s0.copy()
    for t in range(T):
        idx = [n * T + t for n in range(N)]
        o_t = oracle.decode_step(state, q[idx], k[idx], v[idx], la[idx], b[idx])
        np.testing.assert_allclose(o_t, o_pf[idx], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(state, fs_pf, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# Prologue and epilogue pieces (definitions; the constants are our reading)
# ---------------------------------------------------------------------------

def silu(x):
    return x / (1.0 + np.exp(-x))


def l2(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def test_prologue_identity_and_tap_order():
    """"Kimi K3 架构…" section 4.2.3: ShortConv(4) -> Swish -> L2Norm on q and k.
    With taps (0,0,0,1) the conv is the identity; with (1,0,0,0) it reads the
    token three steps back (zero before the sequence start)."""
    T, H, d = 10, 2, 8
    lens = [6, 4]
    cu = np.array([0, 6, 10])
    q, k, v, la, b = random_problem(T, H, d, d)
    qr, kr = RNG.standard_normal((2, T, H, d))
    w_id = np.tile([0.0, 0.0, 0.0, 1.0], (H * d, 1))
    o, fs = oracle.chunk_fwd(qr, kr, v, la, b, cu_seqlens=cu, conv_q_w=w_id, conv_k_w=w_id)
    o_ref, fs_ref = oracle.chunk_fwd(l2(silu(qr)), l2(silu(kr)), v, la, b, cu_seqlens=cu)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fs, fs_ref, rtol=1e-12, atol=1e-14)
    w_back = np.tile([1.0, 0.0, 0.0, 0.0], (H * d, 1))
    shifted_q = np.zeros_like(qr)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        shifted_q[a + 3:e] = qr[a:e - 3]
    o2, _ = oracle.chunk_fwd(qr, k, v, la, b, cu_seqlens=cu, conv_q_w=w_back)
    o2_ref, _ = oracle.chunk_fwd(l2(silu(shifted_q)), k, v, la, b, cu_seqlens=cu)
    np.testing.assert_allclose(o2, o2_ref, rtol=1e-12, atol=1e-14)
    # per-channel weights: channel c of head h uses row h*d + c
    w_rand = RNG.standard_normal((H * d, 4))
    o3, _ = oracle.chunk_fwd(qr, k, v, la, b, cu_seqlens=cu, conv_q_w=w_rand)
    conv = np.zeros_like(qr)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        for t in range(a, e):
            for m in range(4):
                s = t - 3 + m
                if s >= a:
                    conv[t] += w_rand[:, m].reshape(H, d) * qr[s]
    o3_ref, _ = oracle.chunk_fwd(l2(silu(conv)), k, v, la, b, cu_seqlens=cu)
    np.testing.assert_allclose(o3, o3_ref, rtol=1e-12, atol=1e-14)


def test_epilogue_rmsnorm_and_gate():
    """"Kimi K3 架构…" section 4.2.6: head-wise RMSNorm of the output, then a
    channel-wise sigmoid gate.  Gate logit 0 halves; the result has RMS 0.5
    (up to eps) and follows norm_w per channel."""
    T, H, d = 9, 2, 8
    q, k, v, la, b = random_problem(T, H, d, d)
    o, _ = oracle.chunk_fwd(q, k, v, la, b)
    y, _ = oracle.chunk_fwd(q, k, v, la, b, gate=np.zeros((T, H, d)), rms_eps=1e-6)
    ms = (o * o).mean(-1, keepdims=True)
    np.testing.assert_allclose(y, 0.5 * o / np.sqrt(ms + 1e-6), rtol=1e-13)
    rms_y = np.sqrt((y * y).mean(-1))
    np.testing.assert_allclose(rms_y, 0.5 * np.sqrt(ms[..., 0] / (ms[..., 0] + 1e-6)), rtol=1e-12)
    g = RNG.standard_normal((T, H, d))
    w = RNG.standard_normal(d)
    y2, _ = oracle.chunk_fwd(q, k, v, la, b, gate=g, norm_w=w)
    np.testing.assert_allclose(y2, o / np.sqrt(ms + 1e-6) * w / (1 + np.exp(-g)), rtol=1e-12)


def test_tile_decay_bound(golden):
    """"Kimi K3 架构…" section 4.2.5: with log-decay bounded below by -5, the
    cumulative log-decay over a 16-token tile lies in [-80, 0]; the worst case
    -5 per token reaches exactly -80."""
    ex = golden["tile_decay_bound"]
    la = np.full(ex["tile_tokens"], ex["log_decay_lower_bound"])
    assert np.cumsum(la)[-1] == ex["cumulative_range"][0]


def test_unbounded_decay_reset_and_deep_decay():
    """Unbounded decay ("Kimi K3 架构…" section 4.2.5, Kimi Linear's
    negative-softplus gate): log_alpha = -inf on every channel is alpha = 0,
    so the token first erases the whole state and S_t = beta_t k_t v_t^T
    exactly, after which the run continues as one started from a zero state;
    on a single channel it zeroes that key row only.  A finite decay far past
    the bound, -700 per token, still follows the closed form of the beta = 0
    read (o = S0^T (exp(g) * q)) without overflow."""
    T, d = 7, 6
    q = unit_rows(RNG.standard_normal((T, d)))
    k = unit_rows(RNG.standard_normal((T, d)))
    v = RNG.standard_normal((T, d))
    la = -3.0 * RNG.random((T, d))
    b = RNG.random(T)
    s0 = RNG.standard_normal((1, 1, d, d))
    la_r = la.copy()
    la_r[3] = -np.inf
    o, fs = oracle.chunk_fwd(*one_head(q, k, v, la_r, b), initial_state=s0)
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    o_tail, fs_tail = oracle.chunk_fwd(*one_head(q[3:], k[3:], v[3:], la_r[3:], b[3:]))
    np.testing.assert_allclose(o[3:, 0], o_tail[:, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fs, fs_tail, rtol=1e-13, atol=1e-14)
    # one channel reset: row 2 of the state before token 0's erase is gone
    la_c = np.zeros((1, d))
    la_c[0, 2] = -np.inf
    _, fs1 = oracle.chunk_fwd(*one_head(q[:1], k[:1], v[:1], la_c, np.zeros(1)), initial_state=s0)
    expect = s0[0, 0].copy()
    expect[2] = 0.0
    np.testing.assert_array_equal(fs1[0, 0], expect)
    # deep finite decay with beta = 0
    la_d = -700.0 * RNG.random((T, d))
    o2, _ = oracle.chunk_fwd(*one_head(q, k, v, la_d, np.zeros(T)), initial_state=s0)
    g = np.cumsum(la_d, axis=0)
    np.testing.assert_allclose(o2[:, 0], (np.exp(g) * q) @ s0[0, 0], rtol=1e-13, atol=1e-300)
