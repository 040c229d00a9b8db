"""GPU parity of the multi-token decode (kda_decode_replay) against the oracle.

The replay runs the cached inputs of up to 16 tokens per sequence from a
state, with the fused convolution (rolling three-row history) and output
gate, and writes the state and history only when committing
("Kimi K3 架构…" section 7.4).  Each case runs the HIP path through the C
ABI, reads back the exact input bytes and compares with
oracle.decode_multi slice by slice (per (sequence, head), normwise; bars
2e-2 for bf16, 1e-4 for fp32).  Histories are byte copies and must match
exactly; rows and buffers the call must not write are checked untouched.
"""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
from kda_testlib import TOL, to64, slice_err, sync
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def clone(t):
    return None if t is None else t.clone()


def run_lib(inp, num_tokens, commit, in_place=False):
    """One library call; returns (o, state after, the state tensor given as
    input, q history, k history) with histories and state cloned first."""
    N, L, H = inp["N"], inp["L"], inp["H"]
    dt = inp["q"].dtype
    s_in = clone(inp["state"])
    hq, hk = clone(inp.get("conv_q_state")), clone(inp.get("conv_k_state"))
    o = torch.full((N, L, H, D), float("nan"), dtype=dt, device=DEV)
    state_out = None
    if commit:
        state_out = s_in if (in_place and s_in is not None) else "new"
    o, s_out = kda.decode_replay(s_in, inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], num_tokens,
                                 state_out=state_out, conv_q_w=inp.get("conv_q_w"),
                                 conv_k_w=inp.get("conv_k_w"), conv_q_state=hq, conv_k_state=hk,
                                 gate=inp.get("gate"), norm_w=inp.get("norm_w"), out=o,
                                 unbounded_decay=inp.get("decay") == "softplus")
    sync()
    return o, s_out, s_in, hq, hk


def run_oracle(inp, counts, seqs=None):
    sel = slice(None) if seqs is None else list(seqs)
    g = lambda name: None if inp.get(name) is None else to64(inp[name][sel])
    return oracle.decode_multi(g("state"), g("q"), g("k"), g("v"), g("log_alpha"), g("beta"),
                               None if counts is None else np.asarray(counts)[sel],
                               conv_q_w=to64(inp.get("conv_q_w")), conv_k_w=to64(inp.get("conv_k_w")),
                               conv_q_hist=g("conv_q_state"), conv_k_hist=g("conv_k_state"), gate=g("gate"),
                               norm_w=to64(inp.get("norm_w")))


def clamp_counts(counts, N, L):
    if counts is None:
        return [L] * N
    return [min(max(int(c), 0), L) for c in counts]


def compare(inp, counts, res, ref, commit, dtype, seqs=None):
    o, s_out, s_in, hq, hk = res
    o_ref, s_ref, hq_ref, hk_ref = ref
    N, L, H = inp["N"], inp["L"], inp["H"]
    nts = clamp_counts(counts, N, L)
    seqs = list(range(N)) if seqs is None else list(seqs)
    y = to64(o[seqs])
    worst_o = worst_s = 0.0
    for i, n in enumerate(seqs):
        nt = nts[n]
        assert np.isnan(y[i, nt:]).all(), "rows past the token count were written (seq %d)" % n
        for h in range(H):
            if nt:
                worst_o = max(worst_o, slice_err(y[i, :nt, h], o_ref[i, :nt, h]))
    if commit:
        st = to64(s_out[seqs])
        for i in range(len(seqs)):
            for h in range(H):
                worst_s = max(worst_s, slice_err(st[i, h], s_ref[i, h]))
        if hq is not None:
            np.testing.assert_array_equal(to64(hq[seqs]), hq_ref)
        if hk is not None:
            np.testing.assert_array_equal(to64(hk[seqs]), hk_ref)
    else:
        assert s_out is None
        if inp["state"] is not None:
            assert torch.equal(s_in, inp["state"]), "verification pass changed the state"
        for name, h_ in (("conv_q_state", hq), ("conv_k_state", hk)):
            if h_ is not None:
                assert torch.equal(h_, inp[name]), "verification pass changed %s" % name
    say("  worst o %.3e state %.3e" % (worst_o, worst_s))
    assert worst_o <= TOL[dtype] and worst_s <= TOL[dtype]


CASES = [
    # (name, dtype, fused, L, N, H, counts, s0_std)
    ("f32_L1_plain", "f32", False, 1, 3, 2, None, 0.5),
    ("f32_L5_fused_ragged", "f32", True, 5, 4, 3, [0, 1, 3, 5], 0.5),
    ("bf16_L8_fused_ragged", "bf16", True, 8, 5, 4, [8, 1, 2, 0, 6], 0.02),
    ("bf16_L16_plain_max", "bf16", False, 16, 3, 2, [16, 7, 13], 0.02),
    ("f32_L16_fused_all", "f32", True, 16, 2, 2, None, 0.5),
    ("bf16_L3_fused_clamped", "bf16", True, 3, 3, 2, [-2, 9, 2], 0.02),
    ("bf16_L4_zero_state", "bf16", True, 4, 2, 3, [4, 3], 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", ["verify", "commit", "commit_in_place"])
def test_replay_parity(case, mode):
    name, dtype, fused, L, N, H, counts, s0 = case
    say("case replay %s %s" % (name, mode))
    inp = kda_inputs.make_replay(N, H, L, dtype, s0, fused, DEV, seed=31 + len(name))
    nt = None if counts is None else torch.tensor(counts, dtype=torch.int32, device=DEV)
    commit = mode != "verify"
    res = run_lib(inp, nt, commit, in_place=(mode == "commit_in_place"))
    ref = run_oracle(inp, counts)
    compare(inp, counts, res, ref, commit, dtype)


def test_replay_single_token_is_decode_step():
    """One cached token without the fused options is one decode step."""
    say("case replay L=1 vs decode_step")
    N, H = 4, 3
    dec = kda_inputs.make_decode(N, H, 1, "f32", 0.5, DEV, seed=41)
    state = dec["state"].clone()
    o_dec = kda.decode_step(state, dec["q"][0], dec["k"][0], dec["v"][0], dec["log_alpha"][0], dec["beta"][0])
    o_rep, s_rep = kda.decode_replay(dec["state"], dec["q"][0][:, None], dec["k"][0][:, None],
                                     dec["v"][0][:, None], dec["log_alpha"][0][:, None], dec["beta"][0][:, None],
                                     state_out="new")
    sync()
    eo = max(slice_err(to64(o_rep)[n, 0, h], to64(o_dec)[n, h]) for n in range(N) for h in range(H))
    es = max(slice_err(to64(s_rep)[n, h], to64(state)[n, h]) for n in range(N) for h in range(H))
    say("  err o %.3e state %.3e" % (eo, es))
    assert eo <= 1e-6 and es <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_speculative_rounds_equal_one_prefill(dtype):
    """Three rounds of verify (all 8 drafts, nothing written) + commit
    (accepted prefix, in place) with fresh drafts each round give the state,
    history and outputs of one fused prefill over the accepted tokens, from
    a zero history at the sequence start."""
    say("case speculative rounds %s" % dtype)
    N, H, L, rounds = 3, 2, 8, 3
    first = kda_inputs.make_replay(N, H, L, dtype, 0.3, True, DEV, seed=50)
    state = first["state"].clone()
    hq = torch.zeros_like(first["conv_q_state"])
    hk = torch.zeros_like(first["conv_k_state"])
    accepted_rows = [[] for _ in range(N)]  # per sequence: (round, token) of every committed token
    outs = []
    drafts = []
    rng = np.random.Generator(np.random.Philox(51))
    for r in range(rounds):
        inp = kda_inputs.make_replay(N, H, L, dtype, 0.3, True, DEV, seed=60 + r)
        for key in ("conv_q_w", "conv_k_w"):
            inp[key] = first[key]
        drafts.append(inp)
        kw = dict(conv_q_w=inp["conv_q_w"], conv_k_w=inp["conv_k_w"], gate=inp["gate"])
        o_ver, none = kda.decode_replay(state, inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                        conv_q_state=hq, conv_k_state=hk, **kw)
        assert none is None
        counts = [int(c) for c in rng.integers(1, L + 1, size=N)]
        nt = torch.tensor(counts, dtype=torch.int32, device=DEV)
        o_com, _ = kda.decode_replay(state, inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], nt,
                                     state_out=state, conv_q_state=hq, conv_k_state=hk, **kw)
        sync()
        for n in range(N):
            # the committed tokens' outputs are those of the verification pass
            assert torch.equal(o_com[n, :counts[n]], o_ver[n, :counts[n]])
            accepted_rows[n] += [(r, t) for t in range(counts[n])]
            outs.append((n, o_com[n, :counts[n]].clone()))
    # the same tokens as one packed fused prefill per sequence
    lens = [len(a) for a in accepted_rows]
    pick = lambda key: np.concatenate([np.stack([to64(drafts[r][key][n, t]) for r, t in accepted_rows[n]])
                                       for n in range(N)])
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_ref, s_ref = oracle.chunk_fwd(pick("q"), pick("k"), pick("v"), pick("log_alpha"), pick("beta"),
                                    initial_state=to64(first["state"]), cu_seqlens=cu,
                                    conv_q_w=to64(first["conv_q_w"]), conv_k_w=to64(first["conv_k_w"]),
                                    gate=pick("gate"))
    worst_s = max(slice_err(to64(state)[n, h], s_ref[n, h]) for n in range(N) for h in range(H))
    # outputs, in commit order per sequence
    pos = [int(cu[n]) for n in range(N)]
    worst_o = 0.0
    for n, o_n in outs:
        c = o_n.shape[0]
        for h in range(H):
            worst_o = max(worst_o, slice_err(to64(o_n)[:, h], o_ref[pos[n]:pos[n] + c, h]))
        pos[n] += c
    # history = the last three raw rows committed
    for n in range(N):
        last = accepted_rows[n][-3:]
        for key, hist in (("q", hq), ("k", hk)):
            want = np.stack([to64(drafts[r][key][n, t]) for r, t in last])
            np.testing.assert_array_equal(to64(hist[n]), want)
    say("  lens %s worst o %.3e state %.3e" % (lens, worst_o, worst_s))
    assert worst_o <= TOL[dtype] and worst_s <= TOL[dtype]


def test_replay_fullsize_sampled():
    """The benchmark's launches at full size (256 sequences x 96 heads x 8
    cached tokens, bf16, fused): the verification pass and the in-place
    commit with the drawn token counts, compared on sampled sequences."""
    say("case replay full size N=256 H=96 L=8")
    inp = kda_inputs.make_workload(6, device=DEV)
    N, L, H = inp["N"], inp["L"], inp["H"]
    seqs = [0, 97, 255]
    counts = inp["num_tokens_host"]
    kw = dict(conv_q_w=inp["conv_q_w"], conv_k_w=inp["conv_k_w"], gate=inp["gate"])
    state = inp["state"].clone()
    hq, hk = inp["conv_q_state"].clone(), inp["conv_k_state"].clone()
    o_ver, _ = kda.decode_replay(state, inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                 conv_q_state=hq, conv_k_state=hk, **kw)
    o_com, _ = kda.decode_replay(state, inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                 inp["num_tokens"], state_out=state, conv_q_state=hq, conv_k_state=hk,
                                 out=False, **kw)
    sync()
    assert o_com is None
    o_ref_all, _, _, _ = run_oracle(inp, None, seqs)
    _, s_ref, hq_ref, hk_ref = run_oracle(inp, counts, seqs)
    y = to64(o_ver[seqs])
    st = to64(state[seqs])
    worst_o = max(slice_err(y[i, :, h], o_ref_all[i, :, h]) for i in range(len(seqs)) for h in range(H))
    worst_s = max(slice_err(st[i, h], s_ref[i, h]) for i in range(len(seqs)) for h in range(H))
    np.testing.assert_array_equal(to64(hq[seqs]), hq_ref)
    np.testing.assert_array_equal(to64(hk[seqs]), hk_ref)
    say("  counts %s worst o %.3e state %.3e" % ([counts[n] for n in seqs], worst_o, worst_s))
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]
    assert torch.isfinite(state).all()


def test_replay_errors():
    inp = kda_inputs.make_replay(2, 2, 4, "bf16", 0.02, True, DEV, seed=70)
    with pytest.raises(kda.KDAError):  # convolution without its history
        kda.decode_replay(inp["state"], inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                          conv_q_w=inp["conv_q_w"])
    with pytest.raises(kda.KDAError):  # output aliases v
        kda.decode_replay(inp["state"], inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], out=inp["v"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_decay_at_the_bound(dtype):
    """log_alpha = -5 on every channel of 16 tokens: the block's decay factors
    reach e^{+-80}, the range the lower-bounded decay guarantees ("Kimi K3
    架构…" section 4.2.5).  The result stays finite and within tolerance."""
    say("case replay worst decay L=16 %s" % dtype)
    r = kda_inputs.make_replay(2, 2, 16, dtype, 0.5, True, DEV, seed=101)
    r["log_alpha"].fill_(-5.0)
    res = run_lib(r, None, True)
    assert torch.isfinite(res[1]).all() and torch.isfinite(res[0]).all()
    compare(r, None, res, run_oracle(r, None), True, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_no_decay_and_beta_extremes(dtype):
    """No decay (log_alpha = 0) with beta alternating between 0 and 1."""
    say("case replay no decay, beta 0/1 %s" % dtype)
    r = kda_inputs.make_replay(3, 2, 8, dtype, 0.5, False, DEV, seed=102)
    r["log_alpha"].zero_()
    r["beta"].copy_((torch.arange(8, device=DEV) % 2).float().view(1, 8, 1).expand(3, 8, 2))
    counts = [8, 5, 1]
    nt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    res = run_lib(r, nt, True)
    compare(r, counts, res, run_oracle(r, counts), True, dtype)


UNB_CASES = [
    # (name, dtype, fused, L, N, H, counts, s0_std)
    ("f32_L8_fused_ragged", "f32", True, 8, 4, 3, [8, 3, 0, 5], 0.5),
    ("bf16_L8_fused_ragged", "bf16", True, 8, 5, 4, [8, 1, 2, 0, 6], 0.02),
    ("bf16_L16_plain", "bf16", False, 16, 3, 2, [16, 7, 13], 0.3),
    ("f32_L16_plain_all", "f32", False, 16, 2, 2, None, 0.5),
]


@pytest.mark.parametrize("case", UNB_CASES, ids=[c[0] for c in UNB_CASES])
@pytest.mark.parametrize("mode", ["verify", "commit_in_place"])
def test_replay_unbounded_decay(case, mode):
    """Kimi Linear's unbounded negative-softplus decay ("Kimi K3 架构…"
    section 4.2.5): log_alpha = -a_h softplus(z) with per-head rates up to 16,
    far past the bounded block's range; the pairwise decay products keep every
    factor <= 1."""
    name, dtype, fused, L, N, H, counts, s0 = case
    say("case replay unbounded %s %s" % (name, mode))
    inp = kda_inputs.make_replay(N, H, L, dtype, s0, fused, DEV, seed=131 + len(name), decay="softplus")
    say("  log_alpha min %.1f, 16-token sum min %.1f" % (float(inp["log_alpha"].min()),
                                                        float(inp["log_alpha"].sum(dim=1).min())))
    nt = None if counts is None else torch.tensor(counts, dtype=torch.int32, device=DEV)
    commit = mode != "verify"
    res = run_lib(inp, nt, commit, in_place=(mode == "commit_in_place"))
    assert torch.isfinite(res[0].float()[~torch.isnan(res[0].float())]).all()
    ref = run_oracle(inp, counts)
    compare(inp, counts, res, ref, commit, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_unbounded_extremes(dtype):
    """Unbounded decay with log_alpha = -20 on every channel (the bounded
    block's 1/D would be e^320), then single channels at -1e4 and -inf (the
    channel forgets everything) beside tokens with no decay at all."""
    say("case replay unbounded extremes %s" % dtype)
    r = kda_inputs.make_replay(3, 2, 16, dtype, 0.5, True, DEV, seed=141, decay="softplus")
    r["log_alpha"].fill_(-20.0)
    r["log_alpha"][1, 3:6] = 0.0
    r["log_alpha"][1, 4, :, 7] = -1e4
    r["log_alpha"][2, 2, :, 0:5] = float("-inf")
    r["log_alpha"][2, 9:12] = 0.0
    counts = [16, 12, 16]
    nt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    res = run_lib(r, nt, True)
    assert torch.isfinite(res[1]).all()
    compare(r, counts, res, run_oracle(r, counts), True, dtype)
