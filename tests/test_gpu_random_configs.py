"""Seeded random configurations of kda_chunk_fwd, kda_chunk_bwd and
kda_decode_replay against the fp64 oracle (run with -m gpu on an MI355X).

Each case draws its configuration from its own seed: the I/O type, 1..4
heads, 1..6 sequences of 0..300 tokens, the initial-state scale, which fused
options are given (ShortConv on q, on k, the output gate with or without a
norm weight), the decay (bounded, or negative-softplus with unbounded_decay
set), the schedule (automatic, sequential, or forced segments of 64..256
tokens) and the factor-store budget (one window, or 1 MiB, which splits most
of these inputs into several windows).  The fixed cases pair these options a
few at a time; here they meet in combinations nobody chose, which is where a
dispatch or indexing mistake would hide.  Same metric and bars as the other
parity tests (normwise per (sequence, head) slice; 2e-2 bf16, 1e-4 fp32).
The backward and replay sweeps draw the options those calls take in the same
way and reuse the comparisons of tests/test_gpu_bwd.py and
tests/test_gpu_replay.py.
"""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
from kda_testlib import TOL, compare_prefill, library_inputs, sync
from test_gpu_bwd import NAMES, compare_bwd, run_bwd
from test_gpu_replay import compare, run_lib, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = 64


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def unit_rows(x):
    y = x.float()
    return (y / y.norm(dim=-1, keepdim=True).clamp_min(1e-30)).to(x.dtype)


def draw(case):
    rng = np.random.Generator(np.random.Philox(0x7A3D0000 + case))
    n = int(rng.integers(1, 7))
    lengths = [int(x) for x in rng.integers(0, 301, size=n)]
    if rng.random() < 0.3:
        lengths[int(rng.integers(0, n))] = 0
    if sum(lengths) == 0:
        lengths[0] = 1
    fused = bool(rng.random() < 0.5)
    return dict(
        dtype="f32" if rng.random() < 0.35 else "bf16",
        H=int(rng.integers(1, 5)),
        lengths=lengths,
        s0=float(rng.choice([0.0, 0.02, 0.3])),
        fused=fused,
        conv_q=fused and bool(rng.random() < 0.7),
        conv_k=fused and bool(rng.random() < 0.7),
        gate=fused and bool(rng.random() < 0.7),
        norm_w=bool(rng.random() < 0.5),
        unbounded=bool(rng.random() < 0.35),
        seg=int(rng.choice([0, -1, 64, 128, 256])),
        budget=int(rng.choice([0, 1])),
    )


@pytest.mark.parametrize("case", range(CASES))
def test_random_config(case):
    c = draw(case)
    say("case random %d: %s" % (case, c))
    inp = kda_inputs.make_prefill(c["H"], c["lengths"], c["dtype"], c["s0"], c["fused"], DEV, seed=5000 + case,
                                  decay="softplus" if c["unbounded"] else "bounded")
    if c["fused"]:
        if not c["conv_q"]:
            inp["conv_q_w"] = None
        if not c["conv_k"]:
            inp["conv_k_w"] = None
        if not c["gate"]:
            inp["gate"] = None
        elif c["norm_w"]:
            inp["norm_w"] = 1.0 + 0.1 * torch.randn(128, device=DEV)
        # a tensor with no prologue must arrive unit-norm, as the plain path requires
        for key, conv in (("q", c["conv_q"]), ("k", c["conv_k"])):
            if not conv:
                inp[key] = unit_rows(inp[key])
    kw = library_inputs(inp)
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], segment_tokens=c["seg"],
                          unbounded_decay=c["unbounded"], factor_budget_mib=c["budget"], **kw)
    sync()
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[c["dtype"]] and es <= TOL[c["dtype"]], (eo, es)


@pytest.mark.parametrize("case", range(24))
def test_random_backward(case):
    rng = np.random.Generator(np.random.Philox(0x7A3E0000 + case))
    n = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 201, size=n)]
    if sum(lengths) == 0:
        lengths[0] = 1
    dtype = "f32" if rng.random() < 0.35 else "bf16"
    H = int(rng.integers(1, 4))
    s0 = float(rng.choice([0.0, 0.02, 0.3]))
    ds = float(rng.choice([0.0, 1.0]))
    scale = float(rng.choice([1.0, 0.002]))
    say("case random backward %d: %s H=%d lengths=%s S0 %g dS_T %g decay x%g" % (case, dtype, H, lengths, s0, ds,
                                                                               scale))
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, False, DEV, seed=6000 + case)
    inp["log_alpha"].mul_(scale)
    d_o, dsT = kda_inputs.make_grad_seeds(H, n, sum(lengths), dtype, ds, DEV, seed=6500 + case)
    got = run_bwd(inp, d_o, dsT)
    worst, _ = compare_bwd(inp, d_o, dsT, got)
    say("  " + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
    for k in NAMES:
        assert worst[k] <= TOL[dtype], (k, worst[k])


@pytest.mark.parametrize("case", range(32))
def test_random_replay(case):
    rng = np.random.Generator(np.random.Philox(0x7A3F0000 + case))
    dtype = "f32" if rng.random() < 0.35 else "bf16"
    N, H, L = int(rng.integers(1, 7)), int(rng.integers(1, 5)), int(rng.integers(1, 17))
    fused = bool(rng.random() < 0.6)
    conv_q, conv_k = fused and bool(rng.random() < 0.75), fused and bool(rng.random() < 0.75)
    gate, norm_w = fused and bool(rng.random() < 0.7), bool(rng.random() < 0.5)
    unbounded = bool(rng.random() < 0.35)
    s0 = float(rng.choice([0.0, 0.02, 0.5]))
    counts = None if rng.random() < 0.25 else [int(x) for x in rng.integers(-1, L + 3, size=N)]
    mode = str(rng.choice(["verify", "commit", "commit_in_place"]))
    say("case random replay %d: %s N=%d H=%d L=%d conv q %s k %s gate %s norm %s unbounded %s S0 %g counts %s %s"
        % (case, dtype, N, H, L, conv_q, conv_k, gate, norm_w, unbounded, s0, counts, mode))
    inp = kda_inputs.make_replay(N, H, L, dtype, s0, fused, DEV, seed=7000 + case,
                                 decay="softplus" if unbounded else "bounded")
    if fused:
        for key, conv in (("q", conv_q), ("k", conv_k)):
            if not conv:  # no prologue for this tensor: no history, and it must arrive unit-norm
                inp["conv_%s_w" % key] = None
                inp["conv_%s_state" % key] = None
                inp[key] = unit_rows(inp[key])
        if not gate:
            inp["gate"] = None
        elif norm_w:
            inp["norm_w"] = 1.0 + 0.1 * torch.randn(128, device=DEV)
    nt = None if counts is None else torch.tensor(counts, dtype=torch.int32, device=DEV)
    commit = mode != "verify"
    res = run_lib(inp, nt, commit, in_place=(mode == "commit_in_place"))
    ref = run_oracle(inp, counts)
    compare(inp, counts, res, ref, commit, dtype)


@pytest.mark.parametrize("case", range(24))
def test_random_training_pair(case):
    """kda_chunk_fwd_save + kda_chunk_bwd_saved against kda_chunk_fwd (sequential
    schedule) + kda_chunk_bwd, bit for bit, over random sizes, empty
    sequences, a single sequence without cu_seqlens, with and without an
    initial state, a final state or an in-place continuation."""
    rng = np.random.Generator(np.random.Philox(0x7A400000 + case))
    n = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 181, size=n)]
    if rng.random() < 0.15:
        lengths = [0] * n
    dtype = "f32" if rng.random() < 0.35 else "bf16"
    H = int(rng.integers(1, 4))
    s0 = float(rng.choice([0.0, 0.3]))
    keep_fs = bool(rng.random() < 0.8)
    in_place = keep_fs and s0 > 0 and bool(rng.random() < 0.4)
    say("case random training pair %d: %s H=%d lengths=%s S0 %g final state %s in place %s"
        % (case, dtype, H, lengths, s0, keep_fs, in_place))
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, False, DEV, seed=8000 + case)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    s0_orig = None if inp["initial_state"] is None else inp["initial_state"].clone()
    o_ref, fs_ref = kda.chunk_fwd(*args, s0_orig, inp["cu_seqlens"], segment_tokens=-1)
    if in_place:
        st = s0_orig.clone()
        o, fs, ws = kda.chunk_fwd_save(*args, st, inp["cu_seqlens"], final_state=st)
    else:
        o, fs, ws = kda.chunk_fwd_save(*args, inp["initial_state"], inp["cu_seqlens"], output_final_state=keep_fs)
    d_o, dsT = kda_inputs.make_grad_seeds(H, n, sum(lengths), dtype, 1.0, DEV, seed=8500 + case)
    ref = kda.chunk_bwd(*args, d_o, s0_orig, inp["cu_seqlens"], dsT)
    got = kda.chunk_bwd(*args, d_o, fs if in_place else inp["initial_state"], inp["cu_seqlens"], dsT, saved=ws)
    sync()
    assert torch.equal(o, o_ref)
    assert (fs is None) == (not keep_fs)
    if keep_fs:
        assert torch.equal(fs, fs_ref)
    for g, r in zip(got, ref):
        assert (g is None and r is None) or torch.equal(g, r)
