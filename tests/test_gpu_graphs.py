"""The compute entry points under HIP graph capture and on concurrent streams.

Every compute path of the library only launches kernels on the caller's
stream (no memsets, copies or host waits), so a serving loop can capture it
once and replay it (the unbounded-decay prefill and the training pair included).  Each graph case captures one call, then replays the
graph several times with eager work and synchronisations in between, and
checks every replay bit for bit against the same call run eagerly (the
kernels are deterministic).  The last case runs calls on three streams at
once: the library keeps no state between calls.
"""
import sys

import pytest
import torch

import kda_inputs
import gated_delta_rule_25_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def capture(fn):
    """Warm up fn on a side stream (default priority), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(False)
    torch.cuda.synchronize()
    return g


def test_decode_step_graph():
    say("case graph: decode_step, state in place")
    d = kda_inputs.make_decode(4, 3, 1, "bf16", 0.02, DEV, seed=91)
    q, k, v, la, b = (d[x][0] for x in ("q", "k", "v", "log_alpha", "beta"))
    st_g, st_e = d["state"].clone(), d["state"].clone()
    o_g = torch.empty_like(v)
    scratch = d["state"].clone()

    def step(warm):
        kda.decode_step(scratch if warm else st_g, q, k, v, la, b, out=o_g)

    g = capture(step)
    assert torch.equal(st_g, d["state"]), "capture ran the step"
    for i in range(REPLAYS):
        g.replay()
        o_e = kda.decode_step(st_e, q, k, v, la, b)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), i
        assert torch.equal(st_g, st_e), i


@pytest.mark.parametrize("segment_tokens,unbounded", [(0, False), (64, False), (0, True)])
def test_chunk_fwd_graph(segment_tokens, unbounded):
    say("case graph: chunk_fwd segment_tokens=%d unbounded_decay=%s" % (segment_tokens, unbounded))
    inp = kda_inputs.make_prefill(3, [300, 37], "bf16", 0.02, False, DEV, seed=92,
                                  decay="softplus" if unbounded else "bounded")
    N, T, H = inp["N"], inp["T"], inp["H"]
    ws = torch.empty(max(1, kda.chunk_fwd_workspace_bytes(N, T, H, torch.bfloat16, segment_tokens=segment_tokens)),
                     dtype=torch.uint8, device=DEV)
    o_g = torch.empty_like(inp["v"])
    fs_g = torch.empty((N, H, 128, 128), dtype=torch.float32, device=DEV)

    def call(warm):
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["initial_state"],
                      inp["cu_seqlens"], out=o_g, final_state=fs_g, workspace=ws, segment_tokens=segment_tokens,
                      unbounded_decay=unbounded)

    g = capture(call)
    for i in range(REPLAYS):
        o_g.zero_()
        fs_g.zero_()
        g.replay()
        o_e, fs_e = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["initial_state"],
                                  inp["cu_seqlens"], segment_tokens=segment_tokens, unbounded_decay=unbounded)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), i
        assert torch.equal(fs_g, fs_e), i


def test_training_step_graph():
    """kda_chunk_fwd_save and kda_chunk_bwd_saved captured together: every
    replay gives the eager kda_chunk_fwd outputs and kda_chunk_bwd gradients."""
    say("case graph: chunk_fwd_save + chunk_bwd(saved)")
    inp = kda_inputs.make_prefill(2, [150, 77], "bf16", 0.02, False, DEV, seed=94)
    N, T, H = inp["N"], inp["T"], inp["H"]
    d_o, dsT = kda_inputs.make_grad_seeds(H, N, T, "bf16", 1.0, DEV, seed=95)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(N, T, H, torch.bfloat16), dtype=torch.uint8, device=DEV)
    o_g = torch.empty_like(inp["v"])
    fs_g = torch.empty((N, H, 128, 128), dtype=torch.float32, device=DEV)
    res = {}

    def call(warm):
        kda.chunk_fwd_save(*args, inp["initial_state"], inp["cu_seqlens"], out=o_g, final_state=fs_g, workspace=ws)
        res["grads"] = kda.chunk_bwd(*args, d_o, inp["initial_state"], inp["cu_seqlens"], dsT, saved=ws)

    g = capture(call)
    grads_g = res["grads"]
    for i in range(REPLAYS):
        o_g.zero_()
        fs_g.zero_()
        for t in grads_g:
            t.zero_()
        g.replay()
        o_e, fs_e = kda.chunk_fwd(*args, inp["initial_state"], inp["cu_seqlens"], segment_tokens=-1)
        grads_e = kda.chunk_bwd(*args, d_o, inp["initial_state"], inp["cu_seqlens"], dsT)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(fs_g, fs_e), i
        for x, y in zip(grads_g, grads_e):
            assert torch.equal(x, y), i


def test_decode_replay_graph():
    say("case graph: decode_replay verify + in-place commit")
    r = kda_inputs.make_replay(3, 2, 6, "bf16", 0.02, True, DEV, seed=93)
    kw = dict(conv_q_w=r["conv_q_w"], conv_k_w=r["conv_k_w"], gate=r["gate"])
    st_g, hq_g, hk_g = r["state"].clone(), r["conv_q_state"].clone(), r["conv_k_state"].clone()
    st_e, hq_e, hk_e = r["state"].clone(), r["conv_q_state"].clone(), r["conv_k_state"].clone()
    o_g = torch.empty_like(r["v"])
    scratch = (r["state"].clone(), r["conv_q_state"].clone(), r["conv_k_state"].clone())

    def round_(warm):
        st, a, b = scratch if warm else (st_g, hq_g, hk_g)
        kda.decode_replay(st, r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], conv_q_state=a, conv_k_state=b,
                          out=o_g, **kw)
        kda.decode_replay(st, r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], r["num_tokens"], state_out=st,
                          conv_q_state=a, conv_k_state=b, out=False, **kw)

    g = capture(round_)
    for i in range(REPLAYS):
        g.replay()
        o_e, _ = kda.decode_replay(st_e, r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], conv_q_state=hq_e,
                                   conv_k_state=hk_e, **kw)
        kda.decode_replay(st_e, r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], r["num_tokens"], state_out=st_e,
                          conv_q_state=hq_e, conv_k_state=hk_e, out=False, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), i
        assert torch.equal(st_g, st_e), i
        assert torch.equal(hq_g, hq_e) and torch.equal(hk_g, hk_e), i


def test_concurrent_streams():
    """Two prefill calls with their own workspaces on two streams (default
    priority) at once, plus a replay on a third: the library keeps no state
    between calls, so each matches the same call run alone."""
    say("case two streams")
    a = kda_inputs.make_prefill(4, [500, 200], "bf16", 0.02, False, DEV, seed=94)
    b = kda_inputs.make_prefill(3, [700], "bf16", 0.02, True, DEV, seed=95)
    r = kda_inputs.make_replay(4, 2, 8, "bf16", 0.02, True, DEV, seed=96)
    kw_b = dict(conv_q_w=b["conv_q_w"], conv_k_w=b["conv_k_w"], gate=b["gate"])
    kw_r = dict(conv_q_w=r["conv_q_w"], conv_k_w=r["conv_k_w"], gate=r["gate"], conv_q_state=r["conv_q_state"],
                conv_k_state=r["conv_k_state"])
    ref_a = kda.chunk_fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"], a["cu_seqlens"])
    ref_b = kda.chunk_fwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], **kw_b)
    ref_r, _ = kda.decode_replay(r["state"], r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], **kw_r)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(streams[0]):
            out_a = kda.chunk_fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"],
                                  a["cu_seqlens"])
        with torch.cuda.stream(streams[1]):
            out_b = kda.chunk_fwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], **kw_b)
        with torch.cuda.stream(streams[2]):
            out_r, _ = kda.decode_replay(r["state"], r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], **kw_r)
        torch.cuda.synchronize()
        assert torch.equal(out_a[0], ref_a[0]) and torch.equal(out_a[1], ref_a[1])
        assert torch.equal(out_b[0], ref_b[0]) and torch.equal(out_b[1], ref_b[1])
        assert torch.equal(out_r, ref_r)
