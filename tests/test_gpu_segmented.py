"""GPU parity of the segmented schedule (in-device context parallelism).

A sequence is cut into segments; each segment's affine pair (M_j, B_j) is
computed from a zero state and from the identity, a scan composes the pairs
into incoming states, and a last pass writes the outputs ("Kimi K3 架构、训练与
系统全景解析", section 7.1).  The results must match the fp64 oracle, which
runs every sequence token by token, to the same bars as the sequential
schedule (metric in tests/kda_testlib.py).  segment_tokens forces the form at
sizes the oracle finishes quickly; one case checks the automatic choice.
"""
import sys
import zlib

import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
from kda_testlib import TOL, compare_prefill, library_inputs, slice_err, sync, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(inp, **extra):
    kw = library_inputs(inp)
    kw.update(extra)
    o, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], **kw)
    sync()
    return o, fs


SEG_CASES = [
    # (name, H, lengths, dtype, s0_std, fused, segment_tokens)
    ("bf16_T1000_seg64", 4, [1000], "bf16", 0.02, False, 64),
    ("bf16_T1000_seg256", 4, [1000], "bf16", 0.02, False, 256),
    ("bf16_T1024_seg512_exact", 2, [1024], "bf16", 0.5, False, 512),
    ("bf16_T40_one_short_segment", 2, [40], "bf16", 0.5, False, 64),
    ("f32_T300_seg64", 2, [300], "f32", 0.3, False, 64),
    ("bf16_varlen_seg128", 3, [0, 1, 130, 0, 777, 64, 65, 128], "bf16", 0.3, False, 128),
    ("f32_varlen_seg64", 2, [33, 0, 200], "f32", 0.3, False, 64),
    ("bf16_fused_seg128", 3, [700, 5, 300], "bf16", 0.0, True, 128),
    ("f32_fused_seg64", 2, [200, 33], "f32", 0.0, True, 64),
]


@pytest.mark.parametrize("name,H,lengths,dtype,s0,fused,seg", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_segmented_parity(name, H, lengths, dtype, s0, fused, seg):
    say("case %s H=%d lengths=%s dtype=%s fused=%s segment_tokens=%d" % (name, H, lengths, dtype, fused, seg))
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, fused, DEV, seed=zlib.crc32(name.encode()) & 0xFFFF)
    if fused:
        inp["norm_w"] = 1.0 + 0.1 * torch.randn(128, device=DEV)
    o, fs = run(inp, segment_tokens=seg)
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def test_segmented_matches_sequential_and_inplace():
    """Same inputs through both schedules; the in-place continuation
    (initial_state is final_state) also works in the segmented form."""
    say("case segmented vs sequential, H=4 lengths [900, 0, 333] bf16, in place")
    inp = kda_inputs.make_prefill(4, [900, 0, 333], "bf16", 0.5, False, DEV, seed=4242)
    o_seq, fs_seq = run(inp, segment_tokens=-1)
    s = inp["initial_state"].clone()
    kw = library_inputs(inp)
    kw["initial_state"] = s
    kw["final_state"] = s
    o_seg, fs_seg = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                  segment_tokens=128, **kw)
    sync()
    assert fs_seg.data_ptr() == s.data_ptr()
    cu = inp["cu_host"].tolist()
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(4):
            if cu[n + 1] > cu[n]:
                worst = max(worst, slice_err(to64(o_seg[cu[n]:cu[n + 1], h]), to64(o_seq[cu[n]:cu[n + 1], h])))
            worst = max(worst, slice_err(to64(fs_seg[n, h]), to64(fs_seq[n, h])))
    say("  worst %.3e" % worst)
    assert worst <= TOL["bf16"]
    # the empty sequence keeps its initial state exactly
    assert torch.equal(fs_seg[1], inp["initial_state"][1])


def test_automatic_segmentation_few_heads():
    """H=8, T=8192: the sequential schedule would keep 16 of the compute units
    busy, so the library picks the segmented form by itself."""
    say("case auto: bf16 H=8 T=8192, heads 0, 5")
    need = kda.chunk_fwd_workspace_bytes(1, 8192, 8, torch.bfloat16)
    say("  workspace %d bytes" % need)
    assert need > 0
    inp = kda_inputs.make_prefill(8, [8192], "bf16", 0.02, False, DEV, seed=808)
    o, fs = run(inp)
    eo, es = compare_prefill(inp, o, fs, heads=[0, 5])
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


WINDOW_CASES = [
    # (name, H, lengths, dtype, s0_std, fused, segment_tokens): run with a 1 MiB
    # factor-store budget, so every case spans several windows
    ("bf16_T3000_windows_seg256", 3, [3000], "bf16", 0.3, False, 256),
    ("bf16_varlen_windows_seg64", 2, [1000, 0, 2500, 70], "bf16", 0.3, False, 64),
    ("bf16_fused_windows_seg128", 2, [900, 300], "bf16", 0.0, True, 128),
    ("f32_T700_windows_seg64", 2, [700], "f32", 0.3, False, 64),
    ("bf16_varlen_windows_sequential", 2, [2000, 333], "bf16", 0.3, False, -1),
]


@pytest.mark.parametrize("name,H,lengths,dtype,s0,fused,seg", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_windows_parity(name, H, lengths, dtype, s0, fused, seg):
    """Inputs longer than the factor-store budget run in windows; the state
    crosses them through the final-state buffer (or the workspace), and in the
    segmented form each window scans its own segments from that state."""
    say("case %s H=%d lengths=%s dtype=%s fused=%s segment_tokens=%d budget 1 MiB"
        % (name, H, lengths, dtype, fused, seg))
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, fused, DEV, seed=zlib.crc32(name.encode()) & 0xFFFF)
    if fused:
        inp["norm_w"] = 1.0 + 0.1 * torch.randn(128, device=DEV)
    T = sum(lengths)
    big = kda.chunk_fwd_workspace_bytes(len(lengths), T, H, kda_inputs.torch_dtype(dtype), gated=fused,
                                        segment_tokens=seg, factor_budget_mib=1)
    one = kda.chunk_fwd_workspace_bytes(len(lengths), T, H, kda_inputs.torch_dtype(dtype), gated=fused,
                                        segment_tokens=seg)
    assert big < one, (big, one)  # several windows: a smaller factor store
    o, fs = run(inp, segment_tokens=seg, factor_budget_mib=1)
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


SLOW_CASES = [
    # (name, H, lengths, dtype, segment_tokens, budget MiB or None): log_alpha scaled
    # into (-0.01, 0), so the state is carried across many chunks and segments
    ("bf16_slow_sequential", 4, [2000, 700], "bf16", -1, None),
    ("f32_slow_sequential", 2, [1500], "f32", -1, None),
    ("bf16_slow_seg256", 4, [2000, 700], "bf16", 256, None),
    ("f32_slow_seg128", 2, [1500], "f32", 128, None),
    ("bf16_slow_seg256_windows", 3, [3000, 1100], "bf16", 256, "1"),
    ("bf16_slow_sequential_windows", 3, [3000, 1100], "bf16", -1, "1"),
]


@pytest.mark.parametrize("name,H,lengths,dtype,seg,budget", SLOW_CASES, ids=[c[0] for c in SLOW_CASES])
def test_slow_decay_parity(name, H, lengths, dtype, seg, budget):
    """With the workloads' decay (log_alpha = -5 sigmoid(N(0,1))) a 64-token
    chunk decays by ~e^-160, so little state crosses chunk boundaries; here
    the decay is ~500x slower and the carried state dominates the outputs."""
    say("case %s H=%d lengths=%s dtype=%s segment_tokens=%d budget %s" % (name, H, lengths, dtype, seg, budget))
    inp = kda_inputs.make_prefill(H, lengths, dtype, 0.3, False, DEV, seed=zlib.crc32(name.encode()) & 0xFFFF)
    inp["log_alpha"].mul_(0.002)
    o, fs = run(inp, segment_tokens=seg, factor_budget_mib=int(budget or 0))
    eo, es = compare_prefill(inp, o, fs)
    say("  err_o %.3e err_state %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
