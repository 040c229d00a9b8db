"""Shared helpers for the GPU parity tests: run the library and the oracle on
the same bytes and compare with the tolerance metric.

Tolerance metric: for each (sequence, head) slice of an output tensor,
max|y - r| / max|r| (normwise relative error of the slice).  Bars: 2e-2 for
bf16 inputs, 1e-4 for fp32 inputs.  A pure elementwise relative error is not
used: outputs that are near zero would dominate it.  A secondary elementwise
figure is reported beside it: max over elements of |y - r| / (|r| + rms(r)),
with rms(r) the root mean square of the slice.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to64(t):
    if t is None:
        return None
    return t.detach().float().cpu().double().numpy()


def slice_err(y, r):
    """Normwise relative error of one slice; 0 when both are all zero."""
    den = np.abs(r).max() if r.size else 0.0
    num = np.abs(y - r).max() if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def elem_err(y, r):
    """Secondary elementwise figure of one slice: max |y - r| / (|r| + rms(r))."""
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(np.square(r))))
    d = np.abs(y - r)
    if rms == 0.0:
        return 0.0 if float(d.max()) == 0.0 else float("inf")
    return float((d / (np.abs(r) + rms)).max())


def prefill_errors(o, fs, o_ref, fs_ref, cu):
    """Max slice error over (sequence, head) for outputs and final states."""
    H = o.shape[1]
    eo, es = 0.0, 0.0
    for n in range(len(cu) - 1):
        a, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            if e > a:
                eo = max(eo, slice_err(o[a:e, h], o_ref[a:e, h]))
            if fs is not None:
                es = max(es, slice_err(fs[n, h], fs_ref[n, h]))
    return eo, es


def oracle_prefill(inp, heads=None, seqs=None):
    """Run the oracle on the exact device bytes of `inp` (optionally only some
    heads / sequences, each sliced out and run on its own)."""
    cu = inp["cu_host"].numpy().astype(np.int64)
    H = inp["H"]
    heads = list(range(H)) if heads is None else list(heads)
    seqs = list(range(len(cu) - 1)) if seqs is None else list(seqs)
    res = {}
    for n in seqs:
        a, e = int(cu[n]), int(cu[n + 1])
        sl = slice(a, e)
        hs = heads
        q = to64(inp["q"][sl][:, hs])
        k = to64(inp["k"][sl][:, hs])
        v = to64(inp["v"][sl][:, hs])
        la = to64(inp["log_alpha"][sl][:, hs])
        b = to64(inp["beta"][sl][:, hs])
        s0 = None if inp["initial_state"] is None else to64(inp["initial_state"][n:n + 1, hs])
        kw = {}
        if inp.get("conv_q_w") is not None:
            w = inp["conv_q_w"].view(H, 128, 4)[hs].reshape(-1, 4)
            kw["conv_q_w"] = to64(w)
        if inp.get("conv_k_w") is not None:
            w = inp["conv_k_w"].view(H, 128, 4)[hs].reshape(-1, 4)
            kw["conv_k_w"] = to64(w)
        if inp.get("gate") is not None:
            kw["gate"] = to64(inp["gate"][sl][:, hs])
        if inp.get("norm_w") is not None:
            kw["norm_w"] = to64(inp["norm_w"])
        o, fs = oracle.chunk_fwd(q, k, v, la, b, initial_state=s0, **kw)
        res[n] = (o, fs[0])
    return res, heads


def library_inputs(inp):
    """Keyword arguments of gated_delta_rule_25_amd.chunk_fwd for a generated input dict."""
    kw = dict(initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    for key in ("conv_q_w", "conv_k_w", "gate", "norm_w"):
        if inp.get(key) is not None:
            kw[key] = inp[key]
    return kw


def compare_prefill_full(inp, o, fs, heads=None, seqs=None):
    """Compare library outputs against the oracle: the normwise slice errors
    (err_o, err_state) and the secondary elementwise ones (elem_o, elem_state)."""
    ref, hs = oracle_prefill(inp, heads, seqs)
    cu = inp["cu_host"].numpy()
    r = dict(err_o=0.0, err_state=0.0, elem_o=0.0, elem_state=0.0)
    for n, (o_ref, fs_ref) in ref.items():
        a, e = int(cu[n]), int(cu[n + 1])
        if e > a:
            y = to64(o[a:e][:, hs])
            for j in range(len(hs)):
                r["err_o"] = max(r["err_o"], slice_err(y[:, j], o_ref[:, j]))
                r["elem_o"] = max(r["elem_o"], elem_err(y[:, j], o_ref[:, j]))
        if fs is not None:
            ys = to64(fs[n][hs])
            for j in range(len(hs)):
                r["err_state"] = max(r["err_state"], slice_err(ys[j], fs_ref[j]))
                r["elem_state"] = max(r["elem_state"], elem_err(ys[j], fs_ref[j]))
    return r


def compare_prefill(inp, o, fs, heads=None, seqs=None):
    """Compare library outputs against the oracle; returns (err_o, err_state)."""
    r = compare_prefill_full(inp, o, fs, heads, seqs)
    return r["err_o"], r["err_state"]


def compare_all_heads(inp, o, fs, seqs=None, group=16, say=None):
    """compare_prefill_full over every head, `group` heads per oracle call (so
    host memory stays bounded at long contexts); the worst of each figure."""
    H = inp["H"]
    worst = dict(err_o=0.0, err_state=0.0, elem_o=0.0, elem_state=0.0)
    for h0 in range(0, H, group):
        r = compare_prefill_full(inp, o, fs, heads=range(h0, min(H, h0 + group)), seqs=seqs)
        for key in worst:
            worst[key] = max(worst[key], r[key])
        if say:
            say("  heads %d..%d: err_o %.3e err_state %.3e (elementwise %.3e / %.3e)"
                % (h0, min(H, h0 + group) - 1, r["err_o"], r["err_state"], r["elem_o"], r["elem_state"]))
    return worst


def sync():
    torch.cuda.synchronize()
