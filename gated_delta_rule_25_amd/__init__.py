"""MI355X (gfx950) Kimi Delta Attention: Python binding of libkda.so.

Thin ctypes marshalling over the C ABI declared in include/kda.h: checks
dtypes, devices, shapes and contiguity of torch tensors, allocates outputs
and workspace with torch (device memory and streams only), and passes raw
pointers plus torch's current HIP stream.  Every step of the computation
runs in the HIP kernels of libkda.so; there is no fallback path.  If the
library is not built this module raises on first use.

    o, final_state = chunk_fwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens)
    dq, dk, dv, dlog_alpha, dbeta, d_initial_state = chunk_bwd(q, k, v, log_alpha, beta, d_o, ...)
    o, final_state = chunk_kda(q, k, v, log_alpha, beta, initial_state)   # torch.autograd: forward + backward
    o = decode_step(state, q, k, v, log_alpha, beta)      # state updated in place
    o, state_out = decode_replay(state, q, k, v, log_alpha, beta, num_tokens, state_out=state)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_save", "chunk_bwd", "chunk_bwd_workspace_bytes", "chunk_kda",
           "decode_step",
           "decode_replay", "chunk_fwd_workspace_bytes", "status_string", "KDAError", "last_precondition_flags",
           "library_path", "D", "REPLAY_MAX_TOKENS"]

D = 128
REPLAY_MAX_TOKENS = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

(KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP, KDA_ERR_PRECONDITION,
 KDA_ERR_SCRATCH) = range(7)
# size of the device scratch array behind chunk_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20
# KDA_DEBUG_CHECKS precondition bits (kda_last_precondition_flags)
CHECK_LOG_ALPHA, CHECK_BETA, CHECK_Q_NORM, CHECK_K_NORM, CHECK_CU_SEQLENS = 1, 2, 4, 8, 16
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class KDAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (kda_status %d)" % (where, status_string(code), code))


class _FusedOpts(ctypes.Structure):
    _fields_ = [("conv_q_w", ctypes.c_void_p), ("conv_k_w", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("segment_tokens", ctypes.c_int), ("unbounded_decay", ctypes.c_int),
                ("factor_budget_mib", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libkda.so is not built (%s); run `python -m gated_delta_rule_25_amd.build`"
                           % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, vp,
                                  sz, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_chunk_bwd.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32] + [vp] * 7 + [sz, vp]
    lib.kda_chunk_bwd_saved.restype = i32
    lib.kda_chunk_bwd_saved.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32] + [vp] * 7 + [sz, vp]
    lib.kda_chunk_fwd_save.restype = i32
    lib.kda_chunk_fwd_save.argtypes = [vp] * 7 + [i32, i64, i32, i32, i32, i32] + [vp] * 3 + [sz, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.kda_last_precondition_flags.restype = ctypes.c_uint32
    lib.kda_last_precondition_flags.argtypes = []
    lib.kda_decode_replay.restype = i32
    lib.kda_decode_replay.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                      vp, vp]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return _load().kda_status_string(int(code)).decode()


def last_precondition_flags() -> int:
    """CHECK_* bits that failed in this thread's last call made with the
    environment variable KDA_DEBUG_CHECKS set (0 when all passed)."""
    return int(_load().kda_last_precondition_flags())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int,
                              dtype: torch.dtype = torch.bfloat16, *, gated: bool = False,
                              segment_tokens: int = 0, factor_budget_mib: int = 0) -> int:
    """Workspace bytes of chunk_fwd on the current device.  Of the fused
    options only whether an output gate is given matters (gated=True); the
    address passed for it here is a placeholder that is never read."""
    opts = None
    if gated or segment_tokens != 0 or factor_budget_mib != 0:
        opts = ctypes.byref(_FusedOpts(None, None, 16 if gated else None, None, 1e-6, 1e-6, int(segment_tokens),
                                       0, int(factor_budget_mib)))
    return int(_load().kda_chunk_fwd_workspace_bytes(num_seqs, total_tokens, num_heads, D, D,
                                                     _DTYPES[dtype], opts))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor, beta: torch.Tensor,
              initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
              conv_q_w: Optional[torch.Tensor] = None, conv_k_w: Optional[torch.Tensor] = None,
              gate: Optional[torch.Tensor] = None, norm_w: Optional[torch.Tensor] = None,
              l2_eps: float = 1e-6, rms_eps: float = 1e-6, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
              workspace: Optional[torch.Tensor] = None,
              segment_tokens: int = 0, unbounded_decay: bool = False,
              factor_budget_mib: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KDA prefill over a packed batch (kda_chunk_fwd).

    q, k, v: [T, H, 128] float32 or bfloat16; log_alpha [T, H, 128] float32;
    beta [T, H] float32; initial_state [N, H, 128, 128] float32 or None;
    cu_seqlens int32 [N+1] on the device or None.  Optional fused prologue
    (conv_q_w / conv_k_w [H*128, 4] float32) and epilogue (gate [T, H, 128],
    norm_w [128] float32).  segment_tokens: 0 lets the library choose between
    the sequential and the segmented schedule, a positive multiple of 64
    forces segments of that length, a negative value keeps the sequential
    one.  unbounded_decay: accept any log_alpha <= 0 (the negative-softplus
    decay) instead of the bound [-5, 0]; the diagonal tiles then run position
    pair by position pair.  factor_budget_mib: cap on one window's factor
    store in MiB (0: 16384); longer inputs run in several windows.  Returns
    (o, final_state); final_state may be the same tensor as initial_state
    (in-place continuation).
    """
    lib = _load()
    a = _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens, conv_q_w, conv_k_w, gate, norm_w,
                      l2_eps, rms_eps, out, final_state, output_final_state, segment_tokens, unbounded_decay,
                      factor_budget_mib)
    N, T, H, dtc, opts_p = a["N"], a["T"], a["H"], a["dtc"], a["opts_p"]
    dev = q.device
    need = int(lib.kda_chunk_fwd_workspace_bytes(N, T, H, D, D, dtc, opts_p))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), N, T, H, D, D, dtc, opts_p, _ptr(a["out"]), _ptr(a["final_state"]),
                           _ptr(workspace), ws_bytes, _stream(dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd")
    return a["out"], a["final_state"]


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                      beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, *, out: torch.Tensor,
                      final_state: Optional[torch.Tensor] = None, conv_q_w: Optional[torch.Tensor] = None,
                      conv_k_w: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                      norm_w: Optional[torch.Tensor] = None, l2_eps: float = 1e-6, rms_eps: float = 1e-6,
                      segment_tokens: int = 0, unbounded_decay: bool = False,
                      factor_budget_mib: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """chunk_fwd without a workspace (kda_chunk_fwd_noalloc): the library's
    own NOALLOC_SCRATCH_BYTES device array takes its place and the factor
    store runs in windows that fit it.  The caller passes the outputs (`out`,
    and `final_state` or None), so this function allocates nothing on the
    device.  Calls that overlap in time on one GPU share that GPU's array and
    race.  Raises KDAError with KDA_ERR_SCRATCH when the sizes need more."""
    lib = _load()
    a = _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens, conv_q_w, conv_k_w, gate, norm_w,
                      l2_eps, rms_eps, out, final_state, False, segment_tokens, unbounded_decay,
                      factor_budget_mib)
    rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
                                   _ptr(cu_seqlens), a["N"], a["T"], a["H"], D, D, a["dtc"], a["opts_p"],
                                   _ptr(a["out"]), _ptr(a["final_state"]), _stream(q.device))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_noalloc")
    return a["out"], a["final_state"]


def chunk_bwd_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int,
                              dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of chunk_bwd (every chunk of the input at once)."""
    return int(_load().kda_chunk_bwd_workspace_bytes(num_seqs, total_tokens, num_heads, D, D, _DTYPES[dtype]))


def chunk_fwd_save(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor, beta: torch.Tensor,
                   initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                   out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                   output_final_state: bool = True, workspace: Optional[torch.Tensor] = None):
    """Forward pass for training (kda_chunk_fwd_save): (o, final_state,
    workspace), o and final_state as chunk_fwd gives them without fused
    options, and workspace the backward's residuals, to be passed unchanged
    as chunk_bwd(..., saved=workspace) for the same inputs.  final_state may
    be initial_state (in place)."""
    lib = _load()
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [T, H, 128]")
    T, H, _ = q.shape
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (T, H, D), dt, dev)
    _check(log_alpha, "log_alpha", (T, H, D), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens is None:
        N = 1
    else:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N+1]")
        N = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, D, D), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=dt, device=dev)
    _check(out, "out", (T, H, D), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, D, D), torch.float32, dev)
    dtc = _DTYPES[dt]
    need = int(lib.kda_chunk_bwd_workspace_bytes(N, T, H, D, D, dtc))
    if need == 0:
        raise ValueError("chunk_fwd_save: unsupported sizes")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
                                _ptr(cu_seqlens), N, T, H, D, D, dtc, _ptr(out), _ptr(final_state), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_save")
    return out, final_state, workspace


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor, beta: torch.Tensor,
              d_o: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, d_final_state: Optional[torch.Tensor] = None, *,
              need_d_initial_state: bool = True, workspace: Optional[torch.Tensor] = None,
              saved: Optional[torch.Tensor] = None):
    """Gradients of sum <d_o, o> + <d_final_state, S_T> through chunk_fwd
    (kda_chunk_bwd; no fused prologue or epilogue, log_alpha in [-5, 0]).

    Inputs as chunk_fwd; d_o [T, H, 128] in the I/O dtype; d_final_state
    [N, H, 128, 128] float32 or None (zero).  Returns (dq, dk, dv, dlog_alpha,
    dbeta, d_initial_state) with the shapes and dtypes of q, k, v, log_alpha,
    beta and the initial state (float32; None when need_d_initial_state is
    False).  saved: the workspace chunk_fwd_save returned for these inputs
    (kda_chunk_bwd_saved: the forward is not recomputed; the same bits)."""
    lib = _load()
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [T, H, 128]")
    T, H, _ = q.shape
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o)):
        _check(t, name, (T, H, D), dt, dev)
    _check(log_alpha, "log_alpha", (T, H, D), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens is None:
        N = 1
    else:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N+1]")
        N = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(t, name, (N, H, D, D), torch.float32, dev)
    dq, dk, dv = (torch.empty((T, H, D), dtype=dt, device=dev) for _ in range(3))
    dla = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    db = torch.empty((T, H), dtype=torch.float32, device=dev)
    ds0 = torch.empty((N, H, D, D), dtype=torch.float32, device=dev) if need_d_initial_state else None
    dtc = _DTYPES[dt]
    need = int(lib.kda_chunk_bwd_workspace_bytes(N, T, H, D, D, dtc))
    if need == 0:
        raise ValueError("chunk_bwd: unsupported sizes")
    if saved is not None:
        if saved.device != dev or saved.numel() * saved.element_size() < need:
            raise ValueError("chunk_bwd: saved must be the workspace chunk_fwd_save returned for these inputs")
        workspace, fn, name = saved, lib.kda_chunk_bwd_saved, "kda_chunk_bwd_saved"
    else:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        fn, name = lib.kda_chunk_bwd, "kda_chunk_bwd"
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o),
            _ptr(d_final_state), N, T, H, D, D, dtc, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dla), _ptr(db), _ptr(ds0),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    if rc != KDA_OK:
        raise KDAError(rc, name)
    return dq, dk, dv, dla, db, ds0


class _ChunkKDA(torch.autograd.Function):
    """chunk_fwd forward, chunk_bwd backward (the plain recurrence with the
    bounded decay).  By default the forward saves only its inputs and the
    backward recomputes the chunk states; with save_residuals the forward is
    chunk_fwd_save and the backward starts from its workspace."""

    @staticmethod
    def forward(ctx, q, k, v, log_alpha, beta, initial_state, cu_seqlens, save_residuals):
        ctx.residuals = None
        if save_residuals:
            o, final_state, ctx.residuals = chunk_fwd_save(q, k, v, log_alpha, beta, initial_state, cu_seqlens)
        else:
            o, final_state = chunk_fwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens, output_final_state=True)
        ctx.save_for_backward(q, k, v, log_alpha, beta, initial_state, cu_seqlens)
        ctx.mark_non_differentiable(*(t for t in (cu_seqlens,) if t is not None))
        return o, final_state

    @staticmethod
    def backward(ctx, d_o, d_final_state):
        q, k, v, log_alpha, beta, initial_state, cu_seqlens = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(q)
        d_o = d_o.to(q.dtype).contiguous()
        if d_final_state is not None:
            d_final_state = d_final_state.to(torch.float32).contiguous()
        need_ds0 = initial_state is not None and ctx.needs_input_grad[5]
        dq, dk, dv, dla, db, ds0 = chunk_bwd(q, k, v, log_alpha, beta, d_o, initial_state, cu_seqlens, d_final_state,
                                             need_d_initial_state=need_ds0, saved=ctx.residuals)
        ctx.residuals = None
        return dq, dk, dv, dla, db, ds0, None, None


def chunk_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor, beta: torch.Tensor,
              initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
              save_residuals: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable KDA prefill (torch.autograd): (o, final_state) as
    chunk_fwd, with gradients for q, k, v, log_alpha, beta and the initial
    state from chunk_bwd.  Plain recurrence only (no fused prologue or
    epilogue), log_alpha in [-5, 0].  save_residuals keeps the backward's
    workspace (chunk_bwd_workspace_bytes) from the forward to the backward
    instead of recomputing the chunk states: faster, and that much memory
    held in between."""
    return _ChunkKDA.apply(q, k, v, log_alpha, beta, initial_state, cu_seqlens, save_residuals)


def _prefill_args(q, k, v, log_alpha, beta, initial_state, cu_seqlens, conv_q_w, conv_k_w, gate, norm_w, l2_eps,
                  rms_eps, out, final_state, output_final_state, segment_tokens, unbounded_decay,
                  factor_budget_mib) -> dict:
    """Checks the prefill's tensors, allocates the outputs the caller left
    out (only when asked) and builds the options struct."""
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [T, H, 128]")
    T, H, _ = q.shape
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (T, H, D), dt, dev)
    _check(log_alpha, "log_alpha", (T, H, D), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens is None:
        N = 1
    else:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N+1]")
        N = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, D, D), torch.float32, dev)
    if conv_q_w is not None:
        _check(conv_q_w, "conv_q_w", (H * D, 4), torch.float32, dev)
    if conv_k_w is not None:
        _check(conv_k_w, "conv_k_w", (H * D, 4), torch.float32, dev)
    if gate is not None:
        _check(gate, "gate", (T, H, D), dt, dev)
    if norm_w is not None:
        _check(norm_w, "norm_w", (D,), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=dt, device=dev)
    else:
        _check(out, "out", (T, H, D), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (N, H, D, D), torch.float32, dev)
    opts = None
    if (any(x is not None for x in (conv_q_w, conv_k_w, gate, norm_w)) or segment_tokens != 0 or unbounded_decay
            or factor_budget_mib != 0):
        opts = _FusedOpts(_ptr(conv_q_w), _ptr(conv_k_w), _ptr(gate), _ptr(norm_w), float(l2_eps),
                          float(rms_eps), int(segment_tokens), int(bool(unbounded_decay)), int(factor_budget_mib))
    # the struct must outlive the call: keep it in the returned dict
    return dict(N=N, T=T, H=H, dtc=_DTYPES[dt], opts=opts, opts_p=ctypes.byref(opts) if opts is not None else None,
                out=out, final_state=final_state)


def decode_step(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                log_alpha: torch.Tensor, beta: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token for every (sequence, head); ``state`` [N, H, 128, 128] float32
    is advanced in place (kda_decode_step).  q, k, v [N, H, 128] float32 or
    bfloat16, log_alpha [N, H, 128] float32, beta [N, H] float32.  Returns o."""
    lib = _load()
    if state.dim() != 4:
        raise ValueError("state must be [N, H, 128, 128]")
    N, H = state.shape[0], state.shape[1]
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    _check(state, "state", (N, H, D, D), torch.float32, dev)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (N, H, D), dt, dev)
    _check(log_alpha, "log_alpha", (N, H, D), torch.float32, dev)
    _check(beta, "beta", (N, H), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, D), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, H, D), dt, dev)
    rc = lib.kda_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), N, H, D, D,
                             _DTYPES[dt], _ptr(out), _stream(dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_step")
    return out


def decode_replay(state_in: Optional[torch.Tensor], q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  log_alpha: torch.Tensor, beta: torch.Tensor, num_tokens: Optional[torch.Tensor] = None, *,
                  state_out=None, conv_q_w: Optional[torch.Tensor] = None,
                  conv_k_w: Optional[torch.Tensor] = None, conv_q_state: Optional[torch.Tensor] = None,
                  conv_k_state: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                  norm_w: Optional[torch.Tensor] = None, l2_eps: float = 1e-6, rms_eps: float = 1e-6,
                  out=None, unbounded_decay: bool = False) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Multi-token decode from cached token inputs (kda_decode_replay).

    q, k, v: [N, L, H, 128] float32 or bfloat16 (L <= 16), log_alpha
    [N, L, H, 128] float32, beta [N, L, H] float32; num_tokens int32 [N] on the
    device (tokens to run per sequence, clamped to [0, L]) or None (all L).
    state_in [N, H, 128, 128] float32 or None (zeros).  state_out: None (the
    state is not written: a verification pass), a tensor (may be state_in
    itself) or the string "new" to allocate one.  conv_*_state [N, 3, H, 128]
    in the I/O dtype hold the raw rows before token 0 and are advanced in
    place when state_out is given.  out: None allocates the outputs, False
    skips them.  unbounded_decay: accept any log_alpha <= 0 (the
    negative-softplus decay) instead of the bound [-5, 0].  Returns (o or
    None, state_out or None).
    """
    lib = _load()
    if q.dim() != 4 or q.shape[3] != D:
        raise ValueError("q must be [N, L, H, 128]")
    N, L, H, _ = q.shape
    dev, dt = q.device, q.dtype
    if dt not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (N, L, H, D), dt, dev)
    _check(log_alpha, "log_alpha", (N, L, H, D), torch.float32, dev)
    _check(beta, "beta", (N, L, H), torch.float32, dev)
    if num_tokens is not None:
        _check(num_tokens, "num_tokens", (N,), torch.int32, dev)
    if state_in is not None:
        _check(state_in, "state_in", (N, H, D, D), torch.float32, dev)
    if isinstance(state_out, str):
        if state_out != "new":
            raise ValueError('state_out must be None, a tensor or "new"')
        state_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _check(state_out, "state_out", (N, H, D, D), torch.float32, dev)
    for name, t in (("conv_q_w", conv_q_w), ("conv_k_w", conv_k_w)):
        if t is not None:
            _check(t, name, (H * D, 4), torch.float32, dev)
    for name, t in (("conv_q_state", conv_q_state), ("conv_k_state", conv_k_state)):
        if t is not None:
            _check(t, name, (N, 3, H, D), dt, dev)
    if gate is not None:
        _check(gate, "gate", (N, L, H, D), dt, dev)
    if norm_w is not None:
        _check(norm_w, "norm_w", (D,), torch.float32, dev)
    if out is None:
        out = torch.empty((N, L, H, D), dtype=dt, device=dev)
    elif out is False:
        out = None
    else:
        _check(out, "out", (N, L, H, D), dt, dev)
    opts = None
    if any(x is not None for x in (conv_q_w, conv_k_w, gate, norm_w)) or unbounded_decay:
        opts = ctypes.byref(_FusedOpts(_ptr(conv_q_w), _ptr(conv_k_w), _ptr(gate), _ptr(norm_w), float(l2_eps),
                                       float(rms_eps), 0, int(bool(unbounded_decay)), 0))
    rc = lib.kda_decode_replay(_ptr(state_in), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(beta), _ptr(num_tokens), N, L, H, D, D, _DTYPES[dt], opts,
                               _ptr(conv_q_state), _ptr(conv_k_state), _ptr(out), _stream(dev))
    if rc != KDA_OK:
        raise KDAError(rc, "kda_decode_replay")
    return out, state_out
