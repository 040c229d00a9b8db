"""Pins of the oracle's backward pass (oracle.chunk_bwd), CPU only.

The gradients are those of L = sum_t <d_o_t, o_t> + <d_final_state, S_T>
through the per-token recurrence.  They are tied to facts outside the
backward code itself:
  - central finite differences of the forward oracle, for every element of
    every input, on tiny shapes (d in {1, 2, 4}, several sequences);
  - a closed form at beta = 0, where the recurrence is a pure decayed read of
    S_0 and every gradient has an explicit sum;
  - a closed form at d = 1, written out as its own scalar adjoint recursion;
  - exact identities at d = 128: L is jointly linear in (S_0, V), so
    <dS_0, S_0> + <dV, V> = L, and o_t is linear in q_t, so <dq, q> = sum <d_o, o>;
  - composition: the backward of a run split in two, the first half fed the
    second half's d_initial_state as its d_final_state, equals the backward of
    the whole run; varlen packing equals separate runs.
"""
import numpy as np
import pytest

import oracle


def rand_inputs(rng, T, H, d, N_lengths=None, s0=True):
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d)) / np.sqrt(d)
    v = rng.standard_normal((T, H, d))
    la = -rng.random((T, H, d))
    b = rng.random((T, H))
    N = 1 if N_lengths is None else len(N_lengths)
    S0 = rng.standard_normal((N, H, d, d)) * 0.3 if s0 else None
    do = rng.standard_normal((T, H, d))
    dsT = rng.standard_normal((N, H, d, d))
    cu = None if N_lengths is None else np.concatenate([[0], np.cumsum(N_lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, initial_state=S0, cu_seqlens=cu, d_o=do, d_final_state=dsT)


def loss(x):
    o, fs = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], initial_state=x["initial_state"],
                             cu_seqlens=x["cu_seqlens"])
    val = float(np.sum(o * x["d_o"]))
    if x["d_final_state"] is not None:
        val += float(np.sum(fs * x["d_final_state"]))
    return val


def grads(x):
    return oracle.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["d_o"],
                            initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"],
                            d_final_state=x["d_final_state"])


NAMES = ["q", "k", "v", "log_alpha", "beta", "initial_state"]


@pytest.mark.parametrize("d,lengths", [(1, [5]), (2, [3, 0, 4]), (4, [7]), (4, [1, 6])])
def test_central_finite_differences(d, lengths):
    rng = np.random.default_rng(100 + d + len(lengths))
    T = sum(lengths)
    x = rand_inputs(rng, T, 2, d, lengths if len(lengths) > 1 else None)
    g = dict(zip(NAMES, grads(x)))
    h = 1e-5
    worst = 0.0
    for name in NAMES:
        arr = x[name]
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + h
            lp = loss(x)
            arr[idx] = keep - h
            lm = loss(x)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.abs(fd).max()))
        err = float(np.abs(g[name] - fd).max()) / scale
        worst = max(worst, err)
        assert err < 1e-7, (name, err)
    assert worst < 1e-7


def test_beta_zero_closed_form():
    """beta = 0: S_t = Diag(e^{g_t}) S_0, o_t = S_0^T (e^{g_t} . q_t) with g_t the
    inclusive cumulative log-decay.  Then dk = dv = 0 and
      dq_t          = Diag(e^{g_t}) S_0 do_t
      dS_0          = sum_t (e^{g_t} . q_t) do_t^T + Diag(e^{g_T}) dS_T
      dlog_alpha_t  = sum_{s>=t} e^{g_s} . q_s . (S_0 do_s) + e^{g_T} . rowdot(S_0, dS_T)
      dbeta_t       = k_t^T G_t (v_t - S_0^T (e^{g_t} . k_t)),
                      G_t = sum_{s>=t} (e^{g_s - g_t} . q_s) do_s^T + Diag(e^{g_T - g_t}) dS_T."""
    rng = np.random.default_rng(7)
    T, d = 10, 8
    x = rand_inputs(rng, T, 1, d)
    x["beta"][:] = 0.0
    dq, dk, dv, dla, db, ds0 = grads(x)
    q, k, v, la = x["q"][:, 0], x["k"][:, 0], x["v"][:, 0], x["log_alpha"][:, 0]
    S0, do, dsT = x["initial_state"][0, 0], x["d_o"][:, 0], x["d_final_state"][0, 0]
    g = np.cumsum(la, axis=0)
    gT = g[-1]
    assert np.abs(dk).max() == 0.0 and np.abs(dv).max() == 0.0
    for t in range(T):
        assert np.allclose(dq[t, 0], np.exp(g[t]) * (S0 @ do[t]), rtol=1e-12, atol=1e-12)
    ref_s0 = sum(np.outer(np.exp(g[t]) * q[t], do[t]) for t in range(T)) + np.exp(gT)[:, None] * dsT
    assert np.allclose(ds0[0, 0], ref_s0, rtol=1e-12, atol=1e-12)
    for t in range(T):
        ref = sum(np.exp(g[s]) * q[s] * (S0 @ do[s]) for s in range(t, T)) + np.exp(gT) * np.sum(S0 * dsT, axis=1)
        assert np.allclose(dla[t, 0], ref, rtol=1e-11, atol=1e-12), t
        G = sum(np.outer(np.exp(g[s] - g[t]) * q[s], do[s]) for s in range(t, T)) + np.exp(gT - g[t])[:, None] * dsT
        ref_b = k[t] @ G @ (v[t] - S0.T @ (np.exp(g[t]) * k[t]))
        assert abs(db[t, 0] - ref_b) <= 1e-11 * max(1.0, abs(ref_b)), t


def test_d1_scalar_adjoint():
    """d = 1: s_t = m_t s_{t-1} + beta_t k_t v_t with m_t = a_t (1 - beta_t k_t^2),
    o_t = s_t q_t.  The adjoint lam_t = dL/ds_t obeys lam_t = q_t do_t + m_{t+1} lam_{t+1}
    (lam_T adds dS_T), and
      dq_t = s_t do_t,  dv_t = lam_t beta_t k_t,
      dbeta_t = lam_t (k_t v_t - a_t k_t^2 s_{t-1}),
      dk_t = lam_t (beta_t v_t - 2 a_t beta_t k_t s_{t-1}),
      dlog_alpha_t = lam_t m_t s_{t-1},   dS_0 = m_1 lam_1."""
    rng = np.random.default_rng(11)
    T = 9
    x = rand_inputs(rng, T, 1, 1)
    dq, dk, dv, dla, db, ds0 = grads(x)
    q, k, v = x["q"][:, 0, 0], x["k"][:, 0, 0], x["v"][:, 0, 0]
    a, b = np.exp(x["log_alpha"][:, 0, 0]), x["beta"][:, 0]
    do, dsT, s0 = x["d_o"][:, 0, 0], x["d_final_state"][0, 0, 0, 0], x["initial_state"][0, 0, 0, 0]
    m = a * (1 - b * k * k)
    s = np.zeros(T + 1)
    s[0] = s0
    for t in range(T):
        s[t + 1] = m[t] * s[t] + b[t] * k[t] * v[t]
    lam = np.zeros(T)
    nxt = dsT
    for t in range(T - 1, -1, -1):
        lam[t] = q[t] * do[t] + nxt
        nxt = m[t] * lam[t]
    close = lambda a_, b_: np.allclose(a_, b_, rtol=1e-12, atol=1e-13)
    assert close(dq[:, 0, 0], s[1:] * do)
    assert close(dv[:, 0, 0], lam * b * k)
    assert close(db[:, 0], lam * (k * v - a * k * k * s[:-1]))
    assert close(dk[:, 0, 0], lam * (b * v - 2 * a * b * k * s[:-1]))
    assert close(dla[:, 0, 0], lam * m * s[:-1])
    assert close(ds0[0, 0, 0, 0], m[0] * lam[0])


def test_linearity_identities_d128():
    rng = np.random.default_rng(5)
    lengths = [130, 70]
    x = rand_inputs(rng, sum(lengths), 2, 128, lengths)
    x["q"] /= np.linalg.norm(x["q"], axis=-1, keepdims=True)
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)
    x["log_alpha"] *= 0.05  # slow decay: the initial state matters to the end
    dq, dk, dv, dla, db, ds0 = grads(x)
    o, fs = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], initial_state=x["initial_state"],
                             cu_seqlens=x["cu_seqlens"])
    L = float(np.sum(o * x["d_o"]) + np.sum(fs * x["d_final_state"]))
    euler = float(np.sum(ds0 * x["initial_state"]) + np.sum(dv * x["v"]))
    assert abs(euler - L) <= 1e-10 * max(1.0, abs(L)), (euler, L)
    assert abs(float(np.sum(dq * x["q"])) - float(np.sum(o * x["d_o"]))) <= 1e-10 * max(1.0, abs(L))
    assert np.abs(ds0).max() > 1e-3  # the check is not vacuous


def test_split_run_composes():
    rng = np.random.default_rng(9)
    T, t, H, d = 90, 37, 2, 16
    x = rand_inputs(rng, T, H, d)
    whole = grads(x)
    _, s_mid = oracle.chunk_fwd(x["q"][:t], x["k"][:t], x["v"][:t], x["log_alpha"][:t], x["beta"][:t],
                                initial_state=x["initial_state"])
    sl2 = slice(t, T)
    second = oracle.chunk_bwd(x["q"][sl2], x["k"][sl2], x["v"][sl2], x["log_alpha"][sl2], x["beta"][sl2],
                              x["d_o"][sl2], initial_state=s_mid, d_final_state=x["d_final_state"])
    sl1 = slice(0, t)
    first = oracle.chunk_bwd(x["q"][sl1], x["k"][sl1], x["v"][sl1], x["log_alpha"][sl1], x["beta"][sl1],
                             x["d_o"][sl1], initial_state=x["initial_state"], d_final_state=second[5])
    for i in range(5):
        assert np.allclose(whole[i][:t], first[i], rtol=1e-11, atol=1e-12), NAMES[i]
        assert np.allclose(whole[i][t:], second[i], rtol=1e-11, atol=1e-12), NAMES[i]
    assert np.allclose(whole[5], first[5], rtol=1e-11, atol=1e-12)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(13)
    lengths = [20, 0, 33, 1]
    H, d = 2, 8
    x = rand_inputs(rng, sum(lengths), H, d, lengths)
    packed = grads(x)
    cu = x["cu_seqlens"]
    for n in range(len(lengths)):
        a, e = int(cu[n]), int(cu[n + 1])
        sl = slice(a, e)
        one = oracle.chunk_bwd(x["q"][sl], x["k"][sl], x["v"][sl], x["log_alpha"][sl], x["beta"][sl], x["d_o"][sl],
                               initial_state=x["initial_state"][n:n + 1],
                               d_final_state=x["d_final_state"][n:n + 1])
        for i in range(5):
            assert np.array_equal(packed[i][a:e], one[i]), (n, NAMES[i])
        assert np.array_equal(packed[5][n], one[5][0])
        if e == a:  # an empty sequence passes its final-state gradient straight through
            assert np.array_equal(packed[5][n], x["d_final_state"][n])
