"""Parity at the full workload sizes (run with -m gpu on an MI355X).

The library runs the whole workload exactly as bench.py launches it; the fp64
oracle then recomputes (sequence, head) slices from the same device bytes,
16 heads per oracle call, and every output of those slices is compared
(metric and bars as in tests/kda_testlib.py; the secondary elementwise
figure is printed beside it).  Sizes:
  - one K3 layer, H=96, T=8192, bf16, S0 ~ 0.02 N(0,1)     (every head)
  - the same with log_alpha scaled into (-0.01, 0)          (every head)
  - long context, H=96, T=131072                            (every head)
  - decode, N=256 x H=96, 64 in-place steps                 (every (n,h): all
                                                            64 outputs and the final state)
  - varlen 64 sequences (log-uniform 1K..64K), fused prologue/epilogue
                                                            (every head of the longest,
                                                            the shortest and the first sequence)
  - few heads, H=8, T=131072 (segmented schedule)           (every head, and every
                                                            head vs the sequential schedule),
    with the workload's decay and with a ~5000x slower one
plus the small fp32 workload H=2, T=256 compared in full.
"""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
import oracle
from kda_testlib import TOL, compare_all_heads, compare_prefill, library_inputs, slice_err, sync, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_workload(wid):
    inp = kda_inputs.make_workload(wid, device=DEV)
    sync()
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **library_inputs(inp))
    sync()
    return inp, o, fs


def test_fp32_small_workload_full():
    say("workload 0: fp32 H=2 T=256, all outputs")
    inp, o, fs = run_workload(0)
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def check_all(inp, o, fs, seqs=None):
    w = compare_all_heads(inp, o, fs, seqs=seqs, say=say)
    say("  all heads: err_o %.3e err_state %.3e (elementwise %.3e / %.3e)"
        % (w["err_o"], w["err_state"], w["elem_o"], w["elem_state"]))
    assert w["err_o"] <= TOL["bf16"] and w["err_state"] <= TOL["bf16"], w


@pytest.mark.timeout(600)
def test_one_layer_T8192_all_heads():
    say("workload 1: bf16 H=96 T=8192, every head")
    inp, o, fs = run_workload(1)
    assert torch.isfinite(o.float()).all() and torch.isfinite(fs).all()
    check_all(inp, o, fs)
    del inp, o, fs
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_one_layer_T8192_slow_decay_all_heads():
    """The layer's shape with log_alpha scaled into (-0.01, 0): the carried
    state spans all 128 chunks (with the workloads' decay a chunk forgets it)."""
    say("workload 1 with slow decay: bf16 H=96 T=8192, every head")
    inp = kda_inputs.make_workload(1, device=DEV)
    inp["log_alpha"].mul_(0.002)
    sync()
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **library_inputs(inp))
    sync()
    check_all(inp, o, fs)
    del inp, o, fs
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_long_context_T131072_all_heads():
    say("workload 2: bf16 H=96 T=131072, every head")
    inp, o, fs = run_workload(2)
    check_all(inp, o, fs)
    del inp, o, fs
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_few_heads_T131072_segmented_all_heads():
    """H=8, T=131072: the library picks the segmented schedule (16 segments
    per head); every head against the oracle and against the same call
    forced onto the sequential schedule.  With this decay (log_alpha =
    -5 sigmoid(N(0,1))) a segment's transition M_j underflows to zero, so the
    two schedules agree to the bit; the slow-decay test below covers M_j != 0."""
    say("workload 5: bf16 H=8 T=131072 (segmented), every head; all heads vs sequential")
    inp = kda_inputs.make_workload(5, device=DEV)
    sync()
    kw = library_inputs(inp)
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **kw)
    o_seq, fs_seq = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], segment_tokens=-1,
                                  **kw)
    sync()
    w = compare_all_heads(inp, o, fs, group=8)
    eo, es = w["err_o"], w["err_state"]
    worst = 0.0
    for h in range(inp["H"]):
        worst = max(worst, slice_err(to64(o[:, h]), to64(o_seq[:, h])), slice_err(to64(fs[0, h]), to64(fs_seq[0, h])))
    say("  err_o %.3e err_state %.3e (elementwise %.3e / %.3e) | segmented vs sequential worst %.3e"
        % (eo, es, w["elem_o"], w["elem_state"], worst))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and worst <= TOL["bf16"]
    del inp, o, fs, o_seq, fs_seq
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_few_heads_T131072_segmented_slow_decay():
    """As above with log_alpha scaled into (-0.001, 0): a segment of 8192
    tokens then decays by about e^-4 instead of underflowing, so every
    segment's incoming state comes from the scan over the pairs (M_j, B_j).
    (With the workload's own decay M_j is exactly zero in fp32 and both
    schedules give the same bits.)"""
    say("workload 5 with slow decay: bf16 H=8 T=131072 (segmented), every head; all heads vs sequential")
    inp = kda_inputs.make_workload(5, device=DEV)
    inp["log_alpha"].mul_(0.0002)
    sync()
    kw = library_inputs(inp)
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **kw)
    o_seq, fs_seq = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], segment_tokens=-1,
                                  **kw)
    sync()
    w = compare_all_heads(inp, o, fs, group=8)
    eo, es = w["err_o"], w["err_state"]
    worst = 0.0
    for h in range(inp["H"]):
        worst = max(worst, slice_err(to64(o[:, h]), to64(o_seq[:, h])), slice_err(to64(fs[0, h]), to64(fs_seq[0, h])))
    say("  err_o %.3e err_state %.3e (elementwise %.3e / %.3e) | segmented vs sequential worst %.3e"
        % (eo, es, w["elem_o"], w["elem_state"], worst))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and worst <= TOL["bf16"]
    assert worst > 0.0  # the schedules really differ here
    del inp, o, fs, o_seq, fs_seq
    torch.cuda.empty_cache()


def _slice_errs(y, r):
    """Normwise error of every slice of the last axes: max|y - r| / max|r|
    over the trailing dimensions, vectorised (0 where both are zero)."""
    axes = tuple(range(2, y.ndim))
    num = np.abs(y - r).max(axis=axes)
    den = np.abs(r).max(axis=axes)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))


@pytest.mark.timeout(900)
def test_decode_N256_H96_64_steps_all_pairs():
    say("workload 3: decode N=256 H=96, 64 steps, every (n, h): all outputs and the final state")
    d = kda_inputs.make_workload(3, device=DEV)
    ref_state = to64(d["state"])
    state = d["state"]
    worst_o = 0.0
    for s in range(64):
        o = kda.decode_step(state, d["q"][s], d["k"][s], d["v"][s], d["log_alpha"][s], d["beta"][s])
        sync()
        o_ref = oracle.decode_step(ref_state, to64(d["q"][s]), to64(d["k"][s]), to64(d["v"][s]),
                                   to64(d["log_alpha"][s]), to64(d["beta"][s]))
        e = float(_slice_errs(to64(o)[..., None], o_ref[..., None]).max())
        worst_o = max(worst_o, e)
        if s % 16 == 15:
            say("  step %d: worst output slice error so far %.3e" % (s, worst_o))
    worst_s = 0.0
    for n0 in range(0, 256, 32):  # the final state, 32 sequences at a time
        worst_s = max(worst_s, float(_slice_errs(to64(state[n0:n0 + 32]), ref_state[n0:n0 + 32]).max()))
    say("  all 24576 pairs: worst output %.3e, worst final state %.3e" % (worst_o, worst_s))
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]
    del d, state
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_varlen_fused_64_sequences_all_heads():
    say("workload 4: varlen 64 sequences, fused prologue/epilogue; every head of the longest, shortest and first")
    inp, o, fs = run_workload(4)
    lengths = inp["lengths"]
    longest = int(np.argmax(lengths))
    shortest = int(np.argmin(lengths))
    say("  T=%d, longest %d, shortest %d" % (inp["T"], lengths[longest], lengths[shortest]))
    check_all(inp, o, fs, seqs=sorted({longest, shortest, 0}))
    del inp, o, fs
    torch.cuda.empty_cache()
