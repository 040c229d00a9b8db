"""Precondition checks of the C ABI (environment variable KDA_DEBUG_CHECKS).

With the checks on, every compute entry point tests the documented
preconditions on the device before launching anything: log_alpha in [-5, 0]
(the lower-bounded decay, "Kimi K3 架构…" sections 2.1 and 4.2.5), beta in
[0, 1], unit-norm q and k when no prologue normalises them, cu_seqlens
non-decreasing from 0 to total_tokens.  A failed check returns
KDA_ERR_PRECONDITION with the failed bits, and the outputs stay untouched.
"""
import sys

import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
from kda_testlib import sync

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture
def checks_on(monkeypatch):
    monkeypatch.setenv("KDA_DEBUG_CHECKS", "1")


def prefill_inputs():
    return kda_inputs.make_prefill(3, [100, 37], "bf16", 0.02, False, DEV, seed=81)


def run_prefill(inp, **kw):
    out = torch.full((inp["T"], inp["H"], 128), 7.0, dtype=torch.bfloat16, device=DEV)
    args = dict(initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], out=out)
    args.update(kw)
    res = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **args)
    sync()
    return res, out


def expect_flags(fn, bits, out):
    with pytest.raises(kda.KDAError) as ei:
        fn()
    sync()
    assert ei.value.code == kda.KDA_ERR_PRECONDITION
    assert kda.last_precondition_flags() == bits, kda.last_precondition_flags()
    assert bool((out == 7.0).all()), "a refused call wrote its output"


def test_valid_inputs_pass(checks_on):
    say("case debug checks: valid prefill, decode, replay")
    inp = prefill_inputs()
    run_prefill(inp)
    assert kda.last_precondition_flags() == 0
    d = kda_inputs.make_decode(2, 3, 1, "bf16", 0.02, DEV, seed=82)
    kda.decode_step(d["state"], d["q"][0], d["k"][0], d["v"][0], d["log_alpha"][0], d["beta"][0])
    sync()
    assert kda.last_precondition_flags() == 0
    r = kda_inputs.make_replay(2, 3, 4, "bf16", 0.02, True, DEV, seed=83)
    kda.decode_replay(r["state"], r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], r["num_tokens"],
                      conv_q_w=r["conv_q_w"], conv_k_w=r["conv_k_w"], conv_q_state=r["conv_q_state"],
                      conv_k_state=r["conv_k_state"], gate=r["gate"])
    sync()
    assert kda.last_precondition_flags() == 0


def test_prefill_checks(checks_on):
    say("case debug checks: prefill")
    inp = prefill_inputs()
    la = inp["log_alpha"].clone()
    la[57, 1, 3] = -6.0
    out = torch.full((inp["T"], inp["H"], 128), 7.0, dtype=torch.bfloat16, device=DEV)
    call = lambda **kw: kda.chunk_fwd(kw.get("q", inp["q"]), kw.get("k", inp["k"]), inp["v"],
                                      kw.get("la", inp["log_alpha"]), kw.get("beta", inp["beta"]),
                                      initial_state=inp["initial_state"],
                                      cu_seqlens=kw.get("cu", inp["cu_seqlens"]), out=out)
    expect_flags(lambda: call(la=la), kda.CHECK_LOG_ALPHA, out)
    b = inp["beta"].clone()
    b[3, 2] = 1.5
    expect_flags(lambda: call(beta=b), kda.CHECK_BETA, out)
    q = inp["q"].clone()
    q[10, 0] *= 1.5
    expect_flags(lambda: call(q=q), kda.CHECK_Q_NORM, out)
    k = inp["k"].clone()
    k[136, 2] *= 0.5
    expect_flags(lambda: call(k=k, la=la), kda.CHECK_K_NORM | kda.CHECK_LOG_ALPHA, out)
    # cu_seqlens: decreasing, and not ending at total_tokens
    expect_flags(lambda: call(cu=torch.tensor([0, 120, 100], dtype=torch.int32, device=DEV)), kda.CHECK_CU_SEQLENS,
                 out)
    expect_flags(lambda: call(cu=torch.tensor([0, 100, 130], dtype=torch.int32, device=DEV)), kda.CHECK_CU_SEQLENS,
                 out)
    # with the prologue, raw q and k need not be unit vectors
    f = kda_inputs.make_prefill(2, [70], "bf16", 0.0, True, DEV, seed=84)
    kda.chunk_fwd(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], conv_q_w=f["conv_q_w"], conv_k_w=f["conv_k_w"],
                  gate=f["gate"])
    sync()
    assert kda.last_precondition_flags() == 0


def test_decode_and_replay_checks(checks_on):
    say("case debug checks: decode, replay")
    d = kda_inputs.make_decode(2, 3, 1, "bf16", 0.02, DEV, seed=85)
    out = torch.full((2, 3, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    b = d["beta"][0].clone()
    b[1, 2] = -0.25
    st = d["state"].clone()
    expect_flags(lambda: kda.decode_step(st, d["q"][0], d["k"][0], d["v"][0], d["log_alpha"][0], b, out=out),
                 kda.CHECK_BETA, out)
    assert torch.equal(st, d["state"]), "a refused decode step changed the state"
    r = kda_inputs.make_replay(3, 2, 4, "bf16", 0.02, False, DEV, seed=86)
    counts = torch.tensor([4, 2, 0], dtype=torch.int32, device=DEV)
    la = r["log_alpha"].clone()
    la[1, 3, 0, 5] = -9.0  # a token the call does not run: not checked
    la[2, 0, 1, 5] = -9.0
    o = torch.full((3, 4, 2, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    kda.decode_replay(r["state"], r["q"], r["k"], r["v"], la, r["beta"], counts, out=o)
    sync()
    assert kda.last_precondition_flags() == 0
    la[0, 1, 1, 7] = 0.5  # a token it runs
    o.fill_(7.0)
    expect_flags(lambda: kda.decode_replay(r["state"], r["q"], r["k"], r["v"], la, r["beta"], counts, out=o),
                 kda.CHECK_LOG_ALPHA, o)


def test_checks_off_by_default(monkeypatch):
    monkeypatch.delenv("KDA_DEBUG_CHECKS", raising=False)
    say("case debug checks off")
    inp = prefill_inputs()
    b = inp["beta"].clone()
    b[3, 2] = 1.5  # outside the preconditions, but only arithmetic depends on it
    kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], b, initial_state=inp["initial_state"],
                  cu_seqlens=inp["cu_seqlens"])
    sync()


def test_unbounded_decay_range(checks_on):
    """With unbounded_decay the prefill accepts any log_alpha <= 0 (-inf
    included) and still flags NaN and positive values; without it a value
    below -5 is flagged.  A decode step takes any log_alpha <= 0."""
    say("case debug checks: unbounded decay range")
    inp = prefill_inputs()
    inp["log_alpha"][5, 1, 3] = -40.0
    inp["log_alpha"][7, 0, 0] = float("-inf")
    out = torch.full((inp["T"], inp["H"], 128), 7.0, dtype=torch.bfloat16, device=DEV)
    expect_flags(lambda: run_prefill(inp, out=out), kda.CHECK_LOG_ALPHA, out)
    run_prefill(inp, unbounded_decay=True)
    assert kda.last_precondition_flags() == 0
    inp["log_alpha"][9, 2, 1] = float("nan")
    out.fill_(7.0)
    expect_flags(lambda: run_prefill(inp, out=out, unbounded_decay=True), kda.CHECK_LOG_ALPHA, out)
    inp["log_alpha"][9, 2, 1] = 0.25
    out.fill_(7.0)
    expect_flags(lambda: run_prefill(inp, out=out, unbounded_decay=True), kda.CHECK_LOG_ALPHA, out)
    d = kda_inputs.make_decode(2, 3, 1, "bf16", 0.02, DEV, seed=87)
    la = d["log_alpha"][0].clone()
    la[0, 1, :8] = -60.0
    la[1, 2, 4] = float("-inf")
    kda.decode_step(d["state"].clone(), d["q"][0], d["k"][0], d["v"][0], la, d["beta"][0])
    sync()
    assert kda.last_precondition_flags() == 0
