"""GPU parity of the backward pass (kda_chunk_bwd) against the fp64 oracle's
backward (oracle.chunk_bwd), through the C ABI (Python binding).

Every gradient is compared per (sequence, head) slice with the normwise
metric of tests/kda_testlib.py (bars 2e-2 for bf16 I/O, 1e-4 for fp32): dq,
dk, dv, dlog_alpha ([tokens, 128] slices), dbeta ([tokens] slices) and
d_initial_state ([128, 128]).  The loss seeds d_o and d_final_state are
drawn by kda_inputs.make_grad_seeds.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda
import oracle
from kda_testlib import TOL, elem_err, slice_err, sync, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "d_initial_state"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_bwd(inp, d_o, dsT):
    out = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], d_o,
                        initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], d_final_state=dsT)
    sync()
    return out


def compare_bwd(inp, d_o, dsT, got, heads=None):
    """Worst normwise (and secondary elementwise) slice error per gradient,
    the oracle run per sequence on the selected heads."""
    cu = inp["cu_host"].numpy().astype(np.int64)
    H = inp["H"]
    hs = list(range(H)) if heads is None else list(heads)
    worst = {k: 0.0 for k in NAMES}
    welem = {k: 0.0 for k in NAMES}
    for n in range(len(cu) - 1):
        a, e = int(cu[n]), int(cu[n + 1])
        sl = slice(a, e)
        s0 = None if inp["initial_state"] is None else to64(inp["initial_state"][n:n + 1, hs])
        dst = None if dsT is None else to64(dsT[n:n + 1, hs])
        ref = oracle.chunk_bwd(to64(inp["q"][sl][:, hs]), to64(inp["k"][sl][:, hs]), to64(inp["v"][sl][:, hs]),
                               to64(inp["log_alpha"][sl][:, hs]), to64(inp["beta"][sl][:, hs]),
                               to64(d_o[sl][:, hs]), initial_state=s0, d_final_state=dst)
        for idx, name in enumerate(NAMES):
            y = to64(got[idx][n:n + 1, hs])[0] if name == "d_initial_state" else to64(got[idx][sl][:, hs])
            r = ref[idx][0] if name == "d_initial_state" else ref[idx]
            for j in range(len(hs)):
                yy = y[j] if name == "d_initial_state" else y[:, j]
                rr = r[j] if name == "d_initial_state" else r[:, j]
                if yy.size == 0:
                    continue
                worst[name] = max(worst[name], slice_err(yy, rr))
                welem[name] = max(welem[name], elem_err(yy, rr))
    return worst, welem


CASES = [
    # (name, H, lengths, dtype, s0_std, ds_std, log_alpha scale)
    ("f32_T256_config0_shape", 2, [256], "f32", 0.0, 1.0, 1.0),
    ("f32_T1", 2, [1], "f32", 0.5, 1.0, 1.0),
    ("f32_T33_ragged", 2, [33], "f32", 0.5, 0.0, 1.0),
    ("f32_varlen_empty", 2, [70, 0, 1, 45], "f32", 0.3, 1.0, 1.0),
    ("f32_slow_decay", 2, [300], "f32", 0.3, 1.0, 0.002),
    ("bf16_T64_one_chunk", 2, [64], "bf16", 0.02, 1.0, 1.0),
    ("bf16_T200_ragged", 3, [200], "bf16", 0.02, 1.0, 1.0),
    ("bf16_varlen_empty", 2, [100, 0, 37, 1], "bf16", 0.3, 1.0, 1.0),
    ("bf16_slow_decay", 2, [700], "bf16", 0.3, 1.0, 0.002),
    ("bf16_no_final_grad", 2, [150], "bf16", 0.3, 0.0, 1.0),
]


@pytest.mark.parametrize("name,H,lengths,dtype,s0,ds,scale", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(name, H, lengths, dtype, s0, ds, scale):
    say("case %s H=%d lengths=%s dtype=%s S0 std %g dS_T std %g decay x%g" % (name, H, lengths, dtype, s0, ds, scale))
    seed = zlib.crc32(name.encode()) & 0xFFFF
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, False, DEV, seed=seed)
    inp["log_alpha"].mul_(scale)
    d_o, dsT = kda_inputs.make_grad_seeds(H, len(lengths), sum(lengths), dtype, ds, DEV, seed=seed + 1)
    got = run_bwd(inp, d_o, dsT)
    for t in got:
        assert torch.isfinite(t.float()).all()
    worst, welem = compare_bwd(inp, d_o, dsT, got)
    say("  " + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
    say("  elementwise " + " ".join("%s %.2e" % (k, welem[k]) for k in NAMES))
    for k in NAMES:
        assert worst[k] <= TOL[dtype], (k, worst[k])


def test_bwd_worst_case_decay():
    """log_alpha = -5 everywhere: the diagonal tiles' factors reach exactly
    e^80, the decay bound's limit."""
    say("case worst-case decay: bf16 H=2 T=128, log_alpha = -5")
    inp = kda_inputs.make_prefill(2, [128], "bf16", 0.3, False, DEV, seed=77)
    inp["log_alpha"].fill_(-5.0)
    d_o, dsT = kda_inputs.make_grad_seeds(2, 1, 128, "bf16", 1.0, DEV, seed=78)
    got = run_bwd(inp, d_o, dsT)
    for t in got:
        assert torch.isfinite(t.float()).all()
    worst, _ = compare_bwd(inp, d_o, dsT, got)
    say("  " + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
    for k in NAMES:
        assert worst[k] <= TOL["bf16"], (k, worst[k])


@pytest.mark.timeout(900)
def test_bwd_one_layer_T8192_all_heads():
    """The K3 layer's shape (H=96, T=8192, bf16), every head against the oracle."""
    say("workload 1 backward: bf16 H=96 T=8192, every head")
    inp = kda_inputs.make_workload(1, device=DEV)
    d_o, dsT = kda_inputs.make_grad_seeds(96, 1, 8192, "bf16", 1.0, DEV)
    got = run_bwd(inp, d_o, dsT)
    for t in got:
        assert torch.isfinite(t.float()).all()
    total = {k: 0.0 for k in NAMES}
    for h0 in range(0, 96, 16):
        worst, welem = compare_bwd(inp, d_o, dsT, got, heads=range(h0, h0 + 16))
        say("  heads %d..%d: " % (h0, h0 + 15) + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
        for k in NAMES:
            total[k] = max(total[k], worst[k])
    for k in NAMES:
        assert total[k] <= TOL["bf16"], (k, total[k])


def test_bwd_errors():
    inp = kda_inputs.make_prefill(2, [10], "bf16", 0.0, False, DEV, seed=5)
    d_o, _ = kda_inputs.make_grad_seeds(2, 1, 10, "bf16", 0.0, DEV)
    with pytest.raises(ValueError):
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], d_o[:5])


def test_bwd_bitwise_repeatable_and_optional_state_gradient():
    """Every gradient is a fixed-order sum: two calls give the same bits (the
    per-token dbeta is assembled from per-tile parts in a fixed order, not by
    atomics). need_d_initial_state=False skips only that output."""
    say("case repeatability: bf16 H=4 lengths [300, 77, 0, 129], S0 and d_final_state given")
    inp = kda_inputs.make_prefill(4, [300, 77, 0, 129], "bf16", 0.3, False, DEV, seed=91)
    d_o, dsT = kda_inputs.make_grad_seeds(4, 4, 506, "bf16", 1.0, DEV, seed=92)
    first = run_bwd(inp, d_o, dsT)
    for rep in range(3):
        again = run_bwd(inp, d_o, dsT)
        for name, a, b in zip(NAMES, first, again):
            assert torch.equal(a, b), (rep, name)
    no_ds0 = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], d_o,
                           initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], d_final_state=dsT,
                           need_d_initial_state=False)
    sync()
    assert no_ds0[5] is None
    for name, a, b in zip(NAMES[:5], first[:5], no_ds0[:5]):
        assert torch.equal(a, b), name


VARLEN_LENGTHS = [1, 31, 32, 33, 63, 64, 65, 128, 0, 1000, 2, 97]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_varlen_chunk_boundaries(dtype):
    """Twelve sequences whose lengths sit on both sides of the 32- and
    64-token chunk edges (and an empty one), every head against the oracle."""
    say("case varlen chunk edges: %s H=3 lengths=%s" % (dtype, VARLEN_LENGTHS))
    inp = kda_inputs.make_prefill(3, VARLEN_LENGTHS, dtype, 0.3, False, DEV, seed=93)
    d_o, dsT = kda_inputs.make_grad_seeds(3, len(VARLEN_LENGTHS), sum(VARLEN_LENGTHS), dtype, 1.0, DEV, seed=94)
    got = run_bwd(inp, d_o, dsT)
    for t in got:
        assert torch.isfinite(t.float()).all()
    worst, welem = compare_bwd(inp, d_o, dsT, got)
    say("  " + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
    for k in NAMES:
        assert worst[k] <= TOL[dtype], (k, worst[k])


@pytest.mark.timeout(900)
def test_bwd_one_layer_T8192_all_heads_fp32():
    """The K3 layer's shape in fp32 I/O (32-token chunks), every head."""
    say("workload 1 shape in fp32: H=96 T=8192, every head")
    inp = kda_inputs.make_prefill(96, [8192], "f32", 0.02, False, DEV, seed=95)
    d_o, dsT = kda_inputs.make_grad_seeds(96, 1, 8192, "f32", 1.0, DEV, seed=96)
    got = run_bwd(inp, d_o, dsT)
    for t in got:
        assert torch.isfinite(t.float()).all()
    total = {k: 0.0 for k in NAMES}
    for h0 in range(0, 96, 16):
        worst, _ = compare_bwd(inp, d_o, dsT, got, heads=range(h0, h0 + 16))
        for k in NAMES:
            total[k] = max(total[k], worst[k])
    say("  " + " ".join("%s %.2e" % (k, total[k]) for k in NAMES))
    for k in NAMES:
        assert total[k] <= TOL["f32"], (k, total[k])


def test_chunk_kda_autograd_matches_the_two_calls():
    """chunk_kda (torch.autograd) gives chunk_fwd's outputs and, for the loss
    <d_o, o> + <d_final_state, S_T>, chunk_bwd's gradients bit for bit; with
    an initial state that needs no gradient its gradient is not formed."""
    say("case autograd: bf16 H=2 lengths [90, 40], S0 given")
    inp = kda_inputs.make_prefill(2, [90, 40], "bf16", 0.3, False, DEV, seed=97)
    d_o, dsT = kda_inputs.make_grad_seeds(2, 2, 130, "bf16", 1.0, DEV, seed=98)
    leaves = [inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "log_alpha", "beta", "initial_state")]
    o, fs = kda.chunk_kda(*leaves, inp["cu_seqlens"])
    o_ref, fs_ref = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                  inp["initial_state"], inp["cu_seqlens"])
    sync()
    assert torch.equal(o.detach(), o_ref) and torch.equal(fs.detach(), fs_ref)
    ((o.float() * d_o.float()).sum() + (fs * dsT).sum()).backward()
    sync()
    ref = run_bwd(inp, d_o, dsT)
    for name, leaf, r in zip(NAMES, leaves, ref):
        assert leaf.grad is not None and torch.equal(leaf.grad, r), name
    # no gradient wanted for the initial state
    leaves2 = [inp[n].clone().requires_grad_(n != "initial_state")
               for n in ("q", "k", "v", "log_alpha", "beta", "initial_state")]
    o2, _ = kda.chunk_kda(*leaves2, inp["cu_seqlens"])
    (o2.float() * d_o.float()).sum().backward()
    sync()
    assert leaves2[5].grad is None and leaves2[0].grad is not None


def test_bwd_all_sequences_empty():
    """T = 0 with two empty sequences: no token gradients, and the state
    gradient passes through unchanged (d_initial_state = d_final_state)."""
    say("case empty batch: bf16 H=2 lengths [0, 0]")
    inp = kda_inputs.make_prefill(2, [0, 0], "bf16", 0.3, False, DEV, seed=99)
    d_o, dsT = kda_inputs.make_grad_seeds(2, 2, 0, "bf16", 1.0, DEV, seed=100)
    got = run_bwd(inp, d_o, dsT)
    for t in got[:5]:
        assert t.shape[0] == 0
    assert torch.equal(got[5], dsT)
    got0 = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], d_o,
                         initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"], d_final_state=None)
    sync()
    assert torch.count_nonzero(got0[5]).item() == 0


SAVE_CASES = [
    # (name, H, lengths, dtype, s0_std, ds_std, in_place)
    ("bf16_varlen_empty", 3, [200, 0, 65, 1], "bf16", 0.3, 1.0, False),
    ("bf16_in_place", 2, [150, 77], "bf16", 0.02, 1.0, True),
    ("f32_T100_no_final_grad", 2, [100], "f32", 0.5, 0.0, False),
    ("f32_varlen_no_state", 2, [64, 33], "f32", 0.0, 1.0, False),
]


@pytest.mark.parametrize("name,H,lengths,dtype,s0,ds,in_place", SAVE_CASES, ids=[c[0] for c in SAVE_CASES])
def test_fwd_save_then_bwd_saved(name, H, lengths, dtype, s0, ds, in_place):
    """kda_chunk_fwd_save gives kda_chunk_fwd's outputs and final state bit for
    bit (the sequential schedule in one window runs the same kernels), and
    kda_chunk_bwd_saved from its residuals gives kda_chunk_bwd's gradients bit
    for bit; an in-place forward overwrites the initial state, which the saved
    backward does not read."""
    say("case fwd_save + bwd_saved %s H=%d lengths=%s dtype=%s in_place=%s" % (name, H, lengths, dtype, in_place))
    seed = zlib.crc32(name.encode()) & 0xFFFF
    inp = kda_inputs.make_prefill(H, lengths, dtype, s0, False, DEV, seed=seed)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    s0_orig = None if inp["initial_state"] is None else inp["initial_state"].clone()
    o_ref, fs_ref = kda.chunk_fwd(*args, s0_orig, inp["cu_seqlens"], segment_tokens=-1)
    if in_place:
        st = s0_orig.clone()
        o, fs, ws = kda.chunk_fwd_save(*args, st, inp["cu_seqlens"], final_state=st)
        assert fs is st
    else:
        o, fs, ws = kda.chunk_fwd_save(*args, inp["initial_state"], inp["cu_seqlens"])
    sync()
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref)
    d_o, dsT = kda_inputs.make_grad_seeds(H, len(lengths), sum(lengths), dtype, ds, DEV, seed=seed + 1)
    ref = kda.chunk_bwd(*args, d_o, s0_orig, inp["cu_seqlens"], dsT)
    got = kda.chunk_bwd(*args, d_o, fs if in_place else inp["initial_state"], inp["cu_seqlens"], dsT, saved=ws)
    sync()
    for n, g, r in zip(NAMES, got, ref):
        assert (g is None and r is None) or torch.equal(g, r), n
    # and against the oracle
    inp["initial_state"] = s0_orig
    worst, _ = compare_bwd(inp, d_o, dsT, got)
    say("  " + " ".join("%s %.2e" % (k, worst[k]) for k in NAMES))
    for k in NAMES:
        assert worst[k] <= TOL[dtype], (k, worst[k])


def test_chunk_kda_save_residuals():
    """chunk_kda with save_residuals (the training forward and the backward
    from its workspace) gives the default path's outputs and gradients bit
    for bit."""
    say("case autograd with saved residuals: bf16 H=2 lengths [90, 40]")
    inp = kda_inputs.make_prefill(2, [90, 40], "bf16", 0.3, False, DEV, seed=97)
    d_o, dsT = kda_inputs.make_grad_seeds(2, 2, 130, "bf16", 1.0, DEV, seed=98)
    grads = []
    for save in (False, True):
        leaves = [inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "log_alpha", "beta", "initial_state")]
        o, fs = kda.chunk_kda(*leaves, inp["cu_seqlens"], save_residuals=save)
        ((o.float() * d_o.float()).sum() + (fs * dsT).sum()).backward()
        sync()
        grads.append([o.detach(), fs.detach()] + [leaf.grad for leaf in leaves])
    for a, b in zip(*grads):
        assert torch.equal(a, b)


def test_fwd_save_and_bwd_saved_all_sequences_empty():
    """T = 0 with two empty sequences: the training forward passes the initial
    state through as the plain forward does, and the saved backward gives
    d_initial_state = d_final_state."""
    say("case empty batch, training pair: bf16 H=2 lengths [0, 0]")
    inp = kda_inputs.make_prefill(2, [0, 0], "bf16", 0.3, False, DEV, seed=101)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    o_ref, fs_ref = kda.chunk_fwd(*args, inp["initial_state"], inp["cu_seqlens"], segment_tokens=-1)
    o, fs, ws = kda.chunk_fwd_save(*args, inp["initial_state"], inp["cu_seqlens"])
    d_o, dsT = kda_inputs.make_grad_seeds(2, 2, 0, "bf16", 1.0, DEV, seed=102)
    got = kda.chunk_bwd(*args, d_o, inp["initial_state"], inp["cu_seqlens"], dsT, saved=ws)
    sync()
    assert o.shape[0] == 0 and torch.equal(fs, fs_ref) and torch.equal(fs, inp["initial_state"])
    for t in got[:5]:
        assert t.shape[0] == 0
    assert torch.equal(got[5], dsT)
