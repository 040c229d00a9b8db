"""Prefill with unbounded decay (kda_chunk_fwd with unbounded_decay set)
against the fp64 oracle (run with -m gpu on an MI355X).

Kimi Linear's negative-softplus gate ("Kimi K3 架构…" section 4.2.5) lets
log_alpha go arbitrarily low, so a 16-token tile's cumulative decay leaves
the (-80, 0) range that the bounded tile path relies on; with the flag the
diagonal tiles are formed position pair by position pair.  Same metric and
bars as the other parity tests (normwise per (sequence, head) slice; 2e-2
bf16, 1e-4 fp32).  The cases cover both I/O types (their 32- and 64-token
chunks), ragged and empty sequences, the fused prologue and epilogue, the
segmented schedule, decays far beyond the bound (-1e4 and -inf, a full reset
of the channel), no decay at all, and the bounded inputs through both paths.
"""
import sys
import zlib

import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
from kda_testlib import TOL, compare_prefill, library_inputs, sync, to64, slice_err
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(inp, **extra):
    kw = library_inputs(inp)
    kw.update(extra)
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], unbounded_decay=True, **kw)
    sync()
    return o, fs


CASES = [
    # (name, H, lengths, dtype, s0_std, fused)
    ("f32_T1", 2, [1], "f32", 0.5, False),
    ("f32_T100_ragged", 2, [100], "f32", 0.5, False),
    ("f32_varlen", 3, [5, 0, 64, 1, 100], "f32", 0.3, False),
    ("bf16_T17", 4, [17], "bf16", 0.02, False),
    ("bf16_T1000", 4, [1000], "bf16", 0.02, False),
    ("bf16_varlen_empty_ones", 5, [0, 1, 130, 0, 77, 2], "bf16", 0.5, False),
    ("bf16_fused_varlen", 3, [200, 0, 65, 3], "bf16", 0.0, True),
    ("f32_fused", 2, [150, 40], "f32", 0.3, True),
]


@pytest.mark.parametrize("name,H,lengths,dtype,s0,fused", CASES, ids=[c[0] for c in CASES])
def test_unbounded_parity(name, H, lengths, dtype, s0, fused):
    say("case unbounded %s H=%d lengths=%s dtype=%s fused=%s" % (name, H, lengths, dtype, fused))
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, fused, DEV, seed=zlib.crc32(name.encode()) & 0xFFFF,
                                  decay="softplus")
    assert float(inp["log_alpha"].min()) < -5.0
    o, fs = run(inp)
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_extreme_decays(dtype):
    """Decays of -1e4 and -inf (the channel forgets everything) next to tokens
    with no decay at all, so that prefix sums of very different magnitudes meet
    in one tile; the outputs stay finite and match the oracle."""
    say("case unbounded extreme decays %s" % dtype)
    inp = kda_inputs.make_prefill(3, [150, 70], dtype, 0.3, False, DEV, seed=77, decay="softplus")
    la = inp["log_alpha"]
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    u = torch.rand(la.shape, generator=g, device=DEV)
    la[u < 0.15] = 0.0
    la[(u >= 0.15) & (u < 0.20)] = -1.0e4
    la[(u >= 0.20) & (u < 0.22)] = float("-inf")
    la[40:56, 1] = 0.0           # a whole tile with no decay in head 1
    la[40, 1, :64] = -1.0e4      # ... after a huge decay on half the channels
    o, fs = run(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(fs).all()
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segmented_schedule(dtype):
    """Few chains and a long sequence, forced onto the segmented schedule:
    the affine pairs (M_j, B_j) of every segment come from the same factors."""
    say("case unbounded segmented %s" % dtype)
    inp = kda_inputs.make_prefill(2, [1500], dtype, 0.3, False, DEV, seed=79, decay="softplus")
    inp["log_alpha"].mul_(0.01)  # keep some state across chunk boundaries
    o, fs = run(inp, segment_tokens=256)
    o2, fs2 = run(inp, segment_tokens=-1)
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    eo2, es2 = compare_prefill(inp, o2, fs2)
    assert eo2 <= TOL[dtype] and es2 <= TOL[dtype], (eo2, es2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bounded_inputs_both_paths(dtype):
    """Inputs inside the bound: the per-position diagonal and the dense tile
    path both match the oracle."""
    say("case bounded inputs through both paths %s" % dtype)
    inp = kda_inputs.make_prefill(3, [300, 45], dtype, 0.3, False, DEV, seed=80)
    o_u, fs_u = run(inp)
    kw = library_inputs(inp)
    o_b, fs_b = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **kw)
    sync()
    for o, fs in ((o_u, fs_u), (o_b, fs_b)):
        eo, es = compare_prefill(inp, o, fs)
        say("  err_o %.3e err_state %.3e" % (eo, es))
        assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def test_full_layer_sampled_heads():
    """The K3 layer shape (H = 96, T = 8192, bf16) with the softplus decay,
    checked on sampled heads."""
    say("case unbounded full layer H=96 T=8192")
    inp = kda_inputs.make_workload(7, device=DEV)
    o, fs = run(inp)
    eo, es = compare_prefill(inp, o, fs, heads=[0, 31, 64, 95])
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


def test_decode_step_unbounded():
    """One decode step needs no bound: decays of -1e4 and -inf per channel."""
    say("case decode step, unbounded decay")
    d = kda_inputs.make_decode(3, 2, 1, "f32", 0.3, DEV, seed=81)
    la = d["log_alpha"][0]
    la[0, 0, :10] = -1.0e4
    la[1, 1, 5:20] = float("-inf")
    la[2, 0] = -40.0
    st = d["state"].clone()
    o = kda.decode_step(st, d["q"][0], d["k"][0], d["v"][0], la, d["beta"][0])
    sync()
    st_ref = to64(d["state"]).copy()
    o_ref = oracle.decode_step(st_ref, to64(d["q"][0]), to64(d["k"][0]), to64(d["v"][0]), to64(la),
                               to64(d["beta"][0]))
    e = max(max(slice_err(to64(o)[n, h], o_ref[n, h]), slice_err(to64(st)[n, h], st_ref[n, h]))
            for n in range(3) for h in range(2))
    say("  err %.3e" % e)
    assert e <= TOL["f32"], e

