"""Seeded synthetic inputs for the KDA hot path (shared by tests and bench).

This module only draws random inputs with the shapes and distributions of
the K3 KDA layers ("Kimi K3 架构、训练与系统全景解析", section 2.1: 96 heads,
head_dim 128, ShortConv kernel 4, gate_lower_bound -5; contexts up to 1M
tokens).  It contains none of the recurrence's arithmetic; the library and
the fp64 oracle both consume what it produces, and the oracle always reads
back the exact bytes the library was given.

Recipe (every draw uses torch's counter-based generator on the target
device, seeded per workload; slices are drawn in a fixed order so the result
is deterministic for a given device type):
  q, k     N(0,1) fp32, then L2-normalised over the 128 channels of each
           (token, head) in fp32, then cast to the I/O dtype (RNE).  With
           the fused prologue q and k are the raw N(0,1) projections instead.
  v        N(0,1), cast to the I/O dtype.
  beta     sigmoid(N(0,1)) fp32, [T, H].
  log_alpha  -5 * sigmoid(N(0,1)) fp32, [T, H, 128]  (values in (-5, 0)).
           Unbounded variant (decay="softplus"): -a_h * softplus(N(0,1)),
           the negative-softplus gate that "Kimi K3 架构…" section 4.2.5
           attributes to Kimi Linear (its formula is lost from the page; read
           as Mamba-2's form, a positive per-head rate times a softplus), with
           a_h = 16**u_h, u_h ~ U[0,1) per head from a generator of its own
           (so every other tensor matches the bounded draw); over one
           96-head, 8192-token layer values reach about -76 per token and a
           16-token tile's sum about -360, far below -80.
  S0       std * N(0,1) fp32 [N, H, 128, 128], or None (zeros) when std = 0.
  prologue conv weights 0.5 * N(0,1) fp32 [H*128, 4] for each of q and k.
  epilogue gate logits N(0,1) in the I/O dtype, norm weight = ones (None).
  varlen   L_n = floor(1024 * 64**u_n), u_n ~ U[0,1) from numpy's Philox
           generator (log-uniform in [1024, 65536]).
  replay   (multi-token decode of cached draft tokens, "Kimi K3 架构…"
           section 7.4; drafts of up to 7 steps: the study notes' section
           4-7, EAGLE-3-style draft model, and "Kimi K3 架构…" section 4.9)
           N sequences x L = 8 cached tokens (7 drafts and the bonus token), [N, L, H, 128] token-major per sequence, drawn
           like the prefill inputs with the prologue (raw q, k); convolution
           histories [N, 3, H, 128] N(0,1) in the I/O dtype (the raw rows
           before the drafts); S0 std * N(0,1).  Tokens run per sequence on
           commit: uniform on {1, ..., L} from numpy's Philox generator (the
           pages give no acceptance rate).
  backward seeds (the loss gradients a training step feeds the backward
           pass): d_o N(0,1) in the I/O dtype [T, H, 128]; d_final_state
           std * N(0,1) fp32 [N, H, 128, 128], or None when std = 0.
"""
from __future__ import annotations

import math

import numpy as np
import torch

D = 128
SEED_BASE = 0x4B444100

# The five workloads (shapes of one K3 KDA layer, and the small fp32 case),
# plus a few-head long prefill that exercises the segmented schedule.
WORKLOADS = {
    0: dict(name="kda_fp32_H2_T256", kind="prefill", dtype="f32", H=2, lengths=[256], s0_std=0.0,
            fused=False),
    1: dict(name="kda_prefill_H96_T8192", kind="prefill", dtype="bf16", H=96, lengths=[8192],
            s0_std=0.02, fused=False),
    2: dict(name="kda_prefill_H96_T131072", kind="prefill", dtype="bf16", H=96, lengths=[131072],
            s0_std=0.02, fused=False),
    3: dict(name="kda_decode_N256_H96_64steps", kind="decode", dtype="bf16", N=256, H=96, steps=64,
            s0_std=0.02),
    4: dict(name="kda_varlen64_fused_H96", kind="prefill", dtype="bf16", H=96, lengths="loguniform64",
            s0_std=0.0, fused=True),
    # few chains: 8 heads of one long sequence fill 16 of 256 compute units
    # sequentially, so the library cuts the sequence into segments
    5: dict(name="kda_prefill_H8_T131072", kind="prefill", dtype="bf16", H=8, lengths=[131072],
            s0_std=0.02, fused=False),
    # speculative decoding at the decode workload's batch: a verification
    # pass over 7 draft tokens + the bonus token, then the replay commit
    6: dict(name="kda_replay_N256_H96_L8", kind="replay", dtype="bf16", N=256, H=96, L=8, s0_std=0.02,
            fused=True),
    # the K3 layer shape with Kimi Linear's unbounded negative-softplus decay
    # (the per-position diagonal tiles that the decay bound removes)
    7: dict(name="kda_prefill_H96_T8192_softplus", kind="prefill", dtype="bf16", H=96, lengths=[8192],
            s0_std=0.02, fused=False, decay="softplus"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def varlen_lengths(seed: int, n: int = 64, lo: int = 1024, hi: int = 65536) -> list:
    rng = np.random.Generator(np.random.Philox(seed))
    u = rng.random(n)
    ratio = hi / lo
    return [int(math.floor(lo * ratio ** x)) for x in u]


def workload_lengths(wid: int) -> list:
    w = WORKLOADS[wid]
    if w["lengths"] == "loguniform64":
        return varlen_lengths(SEED_BASE + wid)
    return list(w["lengths"])


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _fill_unit(dst, g, device, normalise, slab):
    """Fill dst [T, H, 128] slab by slab with N(0,1) draws (L2-normalised per row if asked)."""
    T = dst.shape[0]
    for a in range(0, T, slab):
        e = min(T, a + slab)
        x = _randn((e - a,) + tuple(dst.shape[1:]), g, device)
        if normalise:
            x = x / x.norm(dim=-1, keepdim=True)
        dst[a:e].copy_(x)
        del x


def make_prefill(H, lengths, dtype="bf16", s0_std=0.0, fused=False, device="cpu", seed=SEED_BASE,
                 slab_tokens=16384, decay="bounded"):
    """Packed prefill inputs.  Returns a dict of tensors on ``device``.
    decay: "bounded" (-5 sigmoid) or "softplus" (unbounded, see the recipe)."""
    if decay not in ("bounded", "softplus"):
        raise ValueError("decay must be 'bounded' or 'softplus'")
    dt = torch_dtype(dtype)
    g = _gen(device, seed)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T = int(sum(lengths))
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    out = {"H": H, "N": N, "T": T, "lengths": lengths, "dtype": dtype}
    q = torch.empty((T, H, D), dtype=dt, device=device)
    k = torch.empty((T, H, D), dtype=dt, device=device)
    v = torch.empty((T, H, D), dtype=dt, device=device)
    la = torch.empty((T, H, D), dtype=torch.float32, device=device)
    _fill_unit(q, g, device, not fused, slab_tokens)
    _fill_unit(k, g, device, not fused, slab_tokens)
    _fill_unit(v, g, device, False, slab_tokens)
    rate = None
    if decay == "softplus":
        rate = torch.pow(16.0, torch.rand((H, 1), generator=_gen(device, seed + 0x5F0), device=device))
    for a in range(0, T, slab_tokens):
        e = min(T, a + slab_tokens)
        z = _randn((e - a, H, D), g, device)
        la[a:e] = -5.0 * torch.sigmoid(z) if rate is None else -rate * torch.nn.functional.softplus(z)
        del z
    beta = torch.sigmoid(_randn((T, H), g, device))
    s0 = None
    if s0_std > 0:
        s0 = s0_std * _randn((N, H, D, D), g, device)
    out.update(q=q, k=k, v=v, log_alpha=la, beta=beta, initial_state=s0,
               cu_seqlens=cu.to(device) if N > 1 else None, cu_host=cu, decay=decay)
    if fused:
        out["conv_q_w"] = 0.5 * _randn((H * D, 4), g, device)
        out["conv_k_w"] = 0.5 * _randn((H * D, 4), g, device)
        gate = torch.empty((T, H, D), dtype=dt, device=device)
        _fill_unit(gate, g, device, False, slab_tokens)
        out["gate"] = gate
        out["norm_w"] = None
    return out


def make_grad_seeds(H, N, T, dtype="bf16", ds_std=1.0, device="cpu", seed=SEED_BASE + 0x6B):
    """Gradients of the loss with respect to o and to the final state."""
    g = _gen(device, seed)
    d_o = torch.empty((T, H, D), dtype=torch_dtype(dtype), device=device)
    _fill_unit(d_o, g, device, False, 16384)
    dsT = ds_std * _randn((N, H, D, D), g, device) if ds_std > 0 else None
    return d_o, dsT


def make_decode(N, H, steps, dtype="bf16", s0_std=0.02, device="cpu", seed=SEED_BASE):
    """Decode inputs: state [N,H,128,128] and `steps` distinct tokens per sequence."""
    dt = torch_dtype(dtype)
    g = _gen(device, seed)
    state = s0_std * _randn((N, H, D, D), g, device)
    q = torch.empty((steps, N, H, D), dtype=dt, device=device)
    k = torch.empty((steps, N, H, D), dtype=dt, device=device)
    v = torch.empty((steps, N, H, D), dtype=dt, device=device)
    la = torch.empty((steps, N, H, D), dtype=torch.float32, device=device)
    beta = torch.empty((steps, N, H), dtype=torch.float32, device=device)
    for s in range(steps):
        x = _randn((N, H, D), g, device)
        q[s] = x / x.norm(dim=-1, keepdim=True)
        x = _randn((N, H, D), g, device)
        k[s] = x / x.norm(dim=-1, keepdim=True)
        v[s] = _randn((N, H, D), g, device)
        la[s] = -5.0 * torch.sigmoid(_randn((N, H, D), g, device))
        beta[s] = torch.sigmoid(_randn((N, H), g, device))
    return dict(N=N, H=H, steps=steps, dtype=dtype, state=state, q=q, k=k, v=v, log_alpha=la,
                beta=beta)


def accepted_counts(seed: int, n: int, L: int) -> list:
    """Tokens run per sequence on commit: uniform on {1, ..., L}."""
    rng = np.random.Generator(np.random.Philox(seed))
    return [int(x) for x in rng.integers(1, L + 1, size=n)]


def make_replay(N, H, L, dtype="bf16", s0_std=0.02, fused=True, device="cpu", seed=SEED_BASE, decay="bounded"):
    """Cached draft-token inputs [N, L, H, 128] plus the verified state, the
    convolution histories and the per-sequence counts of tokens to commit.
    decay: "bounded" (-5 sigmoid) or "softplus" (unbounded, as make_prefill)."""
    if decay not in ("bounded", "softplus"):
        raise ValueError("decay must be 'bounded' or 'softplus'")
    dt = torch_dtype(dtype)
    g = _gen(device, seed)
    out = {"N": N, "H": H, "L": L, "dtype": dtype, "fused": fused}
    out["state"] = s0_std * _randn((N, H, D, D), g, device) if s0_std > 0 else None
    rows = N * L
    q = torch.empty((rows, H, D), dtype=dt, device=device)
    k = torch.empty((rows, H, D), dtype=dt, device=device)
    v = torch.empty((rows, H, D), dtype=dt, device=device)
    _fill_unit(q, g, device, not fused, 16384)
    _fill_unit(k, g, device, not fused, 16384)
    _fill_unit(v, g, device, False, 16384)
    z = _randn((N, L, H, D), g, device)
    if decay == "softplus":
        rate = torch.pow(16.0, torch.rand((H, 1), generator=_gen(device, seed + 0x5F0), device=device))
        la = -rate * torch.nn.functional.softplus(z)
    else:
        la = -5.0 * torch.sigmoid(z)
    beta = torch.sigmoid(_randn((N, L, H), g, device))
    out.update(q=q.view(N, L, H, D), k=k.view(N, L, H, D), v=v.view(N, L, H, D), log_alpha=la, beta=beta,
               decay=decay)
    if fused:
        out["conv_q_w"] = 0.5 * _randn((H * D, 4), g, device)
        out["conv_k_w"] = 0.5 * _randn((H * D, 4), g, device)
        out["conv_q_state"] = _randn((N, 3, H, D), g, device).to(dt)
        out["conv_k_state"] = _randn((N, 3, H, D), g, device).to(dt)
        gate = torch.empty((rows, H, D), dtype=dt, device=device)
        _fill_unit(gate, g, device, False, 16384)
        out["gate"] = gate.view(N, L, H, D)
        out["norm_w"] = None
    out["num_tokens_host"] = accepted_counts(seed, N, L)
    out["num_tokens"] = torch.tensor(out["num_tokens_host"], dtype=torch.int32, device=device)
    return out


def make_workload(wid: int, device="cpu", **overrides):
    """Inputs of one of the workloads above (overrides: e.g. lengths or steps)."""
    w = dict(WORKLOADS[wid])
    w.update(overrides)
    seed = SEED_BASE + wid
    if w["kind"] == "decode":
        return make_decode(w["N"], w["H"], w["steps"], w["dtype"], w["s0_std"], device, seed)
    if w["kind"] == "replay":
        return make_replay(w["N"], w["H"], w["L"], w["dtype"], w["s0_std"], w["fused"], device, seed)
    lengths = w["lengths"] if w["lengths"] != "loguniform64" else varlen_lengths(seed)
    return make_prefill(w["H"], lengths, w["dtype"], w["s0_std"], w["fused"], device, seed,
                        decay=w.get("decay", "bounded"))
