"""ctypes binding of libkda.so (C ABI in include/kda.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  Torch provides device memory and the current HIP stream.  The
functions carry the C entry points' names and raise ``KdaError`` on any non-OK
status.  There is no fallback: if ``libkda.so`` is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_HEAD, KDA_GATE_PROJ = 0, 1, 2


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_HIP"}

_vp = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float

_SIGNATURES = {
    "kda_status_string": (ctypes.c_char_p, [_i32]),
    "kda_last_error_detail": (ctypes.c_char_p, []),
    "kda_state_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "kda_state_init": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _i32, _vp]),
    "kda_prefill_chunked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32,
                                   _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                   ctypes.c_size_t, _vp]),
    "kda_prefill_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "kda_prefill_workspace_bytes_batch": (ctypes.c_size_t, [_vp, _i32, _i32, _i32, _i32, _i32,
                                                            _i32]),
    "kda_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp,
                               _i32, _i32, _i32, _i32, _vp, _vp]),
    "kda_decode_tokens": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "kda_short_conv_prefill": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32, _vp,
                                      _vp, _vp, _vp]),
    "kda_short_conv_decode": (_i32, [_vp, _vp, _i32, _vp, _i64, _vp, _i32, _i32, _i32, _f32,
                                     _vp, _vp]),
}
EXPORTS = tuple(_SIGNATURES)

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m gated_delta_rule_99_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != KDA_OK:
        detail = load().kda_last_error_detail().decode(errors="replace")
        raise KdaError(status, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gate_code(g, q, a_log=None) -> int:
    """Per-channel log decay has q's shape; per-head decay drops the channel axis.
    With a_log, g is the decay projection (q's shape and dtype) and beta logits."""
    if a_log is not None:
        if g.shape != q.shape or g.dtype != q.dtype:
            raise ValueError("with a_log, g is the decay projection: q's shape and dtype")
        return KDA_GATE_PROJ
    if g.dim() == q.dim():
        return KDA_GATE_CHANNEL
    if g.dim() == q.dim() - 1:
        return KDA_GATE_HEAD
    raise ValueError(f"g must have shape {tuple(q.shape)} or {tuple(q.shape[:-1])}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _cu_pair(cu_seqlens, cu_seqlens_host, T, device):
    """Device int32 cu_seqlens and a host int32 copy (both required by the ABI)."""
    if cu_seqlens is None:
        host = torch.tensor([0, T], dtype=torch.int32)
    elif isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        host = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.cpu()
        host = torch.as_tensor(host, dtype=torch.int32).contiguous()
        return cu_seqlens.to(torch.int32).contiguous(), host
    else:
        host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
    return host.to(device), host


def kda_state_bytes(H: int, dk: int, dv: int, state_dtype=torch.float32) -> int:
    return int(load().kda_state_bytes(H, dk, dv, _STATE_DTYPES[state_dtype]))


_STATE_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


def _state_code(t: torch.Tensor) -> int:
    if t.dtype not in _STATE_DTYPES:
        raise TypeError(f"state dtype {t.dtype}: expected float32 or bfloat16")
    return _STATE_DTYPES[t.dtype]


def kda_state_init(state: torch.Tensor, src: torch.Tensor | None = None, stream=None):
    """Zero-fill (src None) or copy src into state [n_slots, H, dk, dv], each
    fp32 or bf16 (converted; fp32 -> bf16 rounds to nearest even)."""
    n_slots, H, dk, dv = state.shape
    _check(load().kda_state_init(_ptr(state), _state_code(state), n_slots, H, dk, dv, _ptr(src),
                                 _state_code(src) if src is not None else KDA_F32,
                                 _stream(stream)))
    return state


def kda_prefill_workspace_bytes(n_seqs: int, H: int, dk: int, dv: int, chunk: int,
                                dtype: torch.dtype) -> int:
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_prefill_workspace_bytes(n_seqs, H, dk, dv, chunk, code))


def kda_prefill_workspace_bytes_batch(cu_seqlens_host, H: int, dk: int, dv: int, chunk: int,
                                      dtype: torch.dtype) -> int:
    """Workspace for the longest windows of this batch (cu_seqlens_host: int32
    CPU tensor)."""
    cu = cu_seqlens_host.to(torch.int32).contiguous()
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_prefill_workspace_bytes_batch(cu.data_ptr(), cu.numel() - 1, H, dk, dv,
                                                        chunk, code))


_ws_cache: dict = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes (one per device; reused by
    later calls, which the ABI allows when they are ordered on one stream)."""
    key = torch.device(device)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=None, chunk: int = 64,
                        initial_state=None, final_state=None, o=None,
                        output_final_state: bool = True, cu_seqlens_host=None,
                        workspace="auto", snapshots=None, snap_interval: int = 0,
                        a_log=None, stream=None):
    """Chunked prefill over packed sequences.  q, k: [T, H, dk]; v: [T, H, dv];
    g: [T, H, dk] (per-channel decay) or [T, H] (per-head decay); beta: [T, H].
    With a_log ([H] fp32), g is the decay projection f (q's dtype) and beta the
    write-strength logits: log alpha = -exp(a_log) softplus(f), beta = sigmoid.
    Returns (o, final_state or None), or (o, final_state, snapshots) when
    snapshots is given.

    workspace: "auto" (a cached device buffer of kda_prefill_workspace_bytes_batch),
    a uint8 device tensor, or None (no workspace: the fused kernel).
    snapshots: None, True (allocate [n_seqs, longest // snap_interval, H, dk, dv]
    fp32 zeros) or such a tensor; entry [n, j] receives sequence n's state after
    (j + 1) * snap_interval tokens where it has that many."""
    T, H, dk = q.shape
    dv = v.shape[2]
    cu_dev, cu_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, q.device)
    n_seqs = cu_host.numel() - 1
    want_snaps = snapshots is not None
    if snapshots is True:
        if snap_interval <= 0:
            raise ValueError("snap_interval must be positive")
        lens = cu_host[1:] - cu_host[:-1]
        cap = int(lens.max()) // snap_interval if n_seqs else 0
        snapshots = torch.zeros((n_seqs, cap, H, dk, dv), dtype=torch.float32, device=q.device)
    snap_cap = 0 if snapshots is None else int(snapshots.shape[1])
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', a tensor or None")
        need = kda_prefill_workspace_bytes_batch(cu_host, H, dk, dv, chunk, q.dtype)
        workspace = _workspace(need, q.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kda_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q),
        _gate_code(g, q, a_log), _ptr(a_log), _ptr(cu_dev), cu_host.data_ptr(), n_seqs, H, dk, dv, int(chunk), _ptr(initial_state),
        _ptr(final_state), _ptr(o), _ptr(snapshots), int(snap_interval), snap_cap,
        _ptr(workspace), ws_bytes, _stream(stream)))
    if want_snaps:
        return o, final_state, snapshots
    return o, final_state


def kda_decode_step(q, k, v, g, beta, state, slot_idx=None, o=None, a_log=None, stream=None):
    """One token per sequence.  q, k: [B, H, dk]; g: [B, H, dk] or [B, H] (or the
    decay projection with a_log, as in kda_prefill_chunked); v: [B, H, dv]; beta: [B, H];
    state [n_slots, H, dk, dv] fp32 or bf16, updated in place.  Returns o [B, H, dv]."""
    B, H, dk = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _check(load().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q), _gate_code(g, q, a_log),
        _ptr(a_log), _ptr(state), _state_code(state), state.shape[0], _ptr(slot_idx), B, H, dk,
        dv, _ptr(o),
        _stream(stream)))
    return o


def kda_decode_tokens(q, k, v, g, beta, state, slot_idx=None, o=None, token_states=None,
                      a_log=None, stream=None):
    """n_tok consecutive tokens per sequence.  q, k: [B, n_tok, H, dk]; g: the same
    shape or [B, n_tok, H]; v: [B, n_tok, H, dv]; beta: [B, n_tok, H]; state
    [n_slots, H, dk, dv] fp32 or bf16, updated in place.  token_states: None,
    True (allocate [B, n_tok, H, dk, dv] of the state's dtype) or such a tensor.
    Returns (o [B, n_tok, H, dv], token_states)."""
    B, n_tok, H, dk = q.shape
    dv = v.shape[3]
    if o is None:
        o = torch.empty((B, n_tok, H, dv), dtype=q.dtype, device=q.device)
    if token_states is True:
        token_states = torch.empty((B, n_tok, H, dk, dv), dtype=state.dtype, device=q.device)
    _check(load().kda_decode_tokens(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q), _gate_code(g, q, a_log),
        _ptr(a_log), _ptr(state), _state_code(state), state.shape[0], _ptr(slot_idx), B, n_tok,
        H, dk, dv,
        _ptr(o), _ptr(token_states) if token_states is not None else None, _stream(stream)))
    return o, token_states


def kda_short_conv_prefill(x, w, cu_seqlens=None, l2_head_dim: int = 0, l2_eps: float = 1e-6,
                           conv_tail_in=None, conv_tail_out=None, y=None, cu_seqlens_host=None,
                           stream=None):
    """Width-4 causal depthwise conv (+ per-head L2 norm) over x [T, channels]."""
    T, channels = x.shape
    cu_dev, cu_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, x.device)
    n_seqs = cu_host.numel() - 1
    if y is None:
        y = torch.empty_like(x)
    _check(load().kda_short_conv_prefill(
        _ptr(x), _ptr(w), _dtype_code(x), _ptr(cu_dev), cu_host.data_ptr(), n_seqs, channels,
        int(l2_head_dim), float(l2_eps), _ptr(conv_tail_in), _ptr(conv_tail_out), _ptr(y),
        _stream(stream)))
    return y


def kda_short_conv_decode(x, w, conv_tail, slot_idx=None, l2_head_dim: int = 0,
                          l2_eps: float = 1e-6, y=None, stream=None):
    """One token per sequence: x [B, channels]; conv_tail [n_slots, 3, channels]
    updated in place.  Returns y [B, channels]."""
    B, channels = x.shape
    if y is None:
        y = torch.empty_like(x)
    _check(load().kda_short_conv_decode(
        _ptr(x), _ptr(w), _dtype_code(x), _ptr(conv_tail), conv_tail.shape[0], _ptr(slot_idx),
        B, channels, int(l2_head_dim), float(l2_eps), _ptr(y), _stream(stream)))
    return y
