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
KDA_ERR_WORKSPACE_TOO_SMALL = 4
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_HEAD, KDA_GATE_PROJ = 0, 1, 2


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_HIP", 4: "KDA_ERR_WORKSPACE_TOO_SMALL"}

_vp = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float

_SIGNATURES = {
    "kda_status_string": (ctypes.c_char_p, [_i32]),
    "kda_last_error_detail": (ctypes.c_char_p, []),
    "kda_state_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "kda_state_init": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _i32, _vp]),
    "kda_prefill_chunked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32,
                                   _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                   _vp, ctypes.c_size_t, _vp]),
    "kda_prefill_chunked_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                           _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                           _vp, _i32, _i32, _vp]),
    "kda_prefill_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "kda_prefill_workspace_bytes_batch": (ctypes.c_size_t, [_vp, _i32, _i32, _i32, _i32, _i32,
                                                            _i32]),
    "kda_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp,
                               _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "kda_decode_tokens": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kda_short_conv_prefill": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32, _vp,
                                      _vp, _vp, _vp]),
    "kda_short_conv_decode": (_i32, [_vp, _vp, _i32, _vp, _i64, _vp, _i32, _i32, _i32, _f32,
                                     _vp, _vp]),
    "kda_device_copy": (_i32, [_vp, _vp, ctypes.c_size_t, _vp]),
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


def _stream(stream, device=None):
    """(HIP stream handle, torch stream object or None).  None: torch's current
    stream on `device`; a torch stream, or a raw handle (int)."""
    if stream is None:
        if device is None or device.type != "cuda":
            return 0, None
        st = torch.cuda.current_stream(device)
        return st.cuda_stream, st
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream, stream
    handle = int(stream)
    if device is None or device.type != "cuda":
        return handle, None
    if handle == 0:
        return 0, torch.cuda.default_stream(device)
    return handle, torch.cuda.ExternalStream(handle, device=device)


def _on_stream(t, st):
    """Tell torch's caching allocator that a buffer the binding allocated is used
    on stream st (when st is not the current stream), so that its memory is not
    handed out again before st's work on it has finished."""
    if t is not None and st is not None and t.is_cuda and st != torch.cuda.current_stream(t.device):
        t.record_stream(st)
    return t


# ------------------------------------------------------------------ argument checks
# What the C ABI cannot see from raw pointers (the tensors' sizes, dtypes and
# devices) is checked here, before any call: a mismatch would otherwise make a
# kernel read or write past an allocation.
def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _shape(name, t, shape):
    _need(tuple(t.shape) == tuple(shape),
          f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype(name, t, dtypes):
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")


def _same_device(ref, **tensors):
    """Every given tensor on ref's device, and that device a GPU."""
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if ref.device.type != "cuda":
        raise ValueError(f"tensors are on {ref.device}: the library runs on a GPU")


def _gate_check(g, q, a_log, lead):
    """g: the log decay per channel (fp32, q's shape), per head (fp32, q's
    shape without the channel axis), or with a_log the decay projection (q's
    shape and dtype); a_log [H] fp32."""
    H = q.shape[-2]
    if a_log is not None:
        _shape("a_log", a_log, (H,))
        _dtype("a_log", a_log, torch.float32)
        _shape("g", g, q.shape)
        _dtype("g", g, q.dtype)
    else:
        _dtype("g", g, torch.float32)
        _need(tuple(g.shape) in (tuple(q.shape), tuple(lead) + (H,)),
              f"g has shape {tuple(g.shape)}, expected {tuple(q.shape)} or "
              f"{tuple(lead) + (H,)}")


def _cu_pair(cu_seqlens, cu_seqlens_host, T, device):
    """Device int32 cu_seqlens and a host int32 copy (both required by the ABI).
    The host copy must end at T (the tokens of the tensors), and the device copy
    must have as many entries."""
    if cu_seqlens is None:
        host = torch.tensor([0, T], dtype=torch.int32)
        dev_cu = host.to(device)
    elif isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        host = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.cpu()
        host = torch.as_tensor(host, dtype=torch.int32).contiguous()
        _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() == host.numel(),
              "cu_seqlens and cu_seqlens_host differ in length")
        _need(cu_seqlens.device == device, f"cu_seqlens is on {cu_seqlens.device}, expected {device}")
        dev_cu = cu_seqlens.to(torch.int32).contiguous()
    else:
        host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
        dev_cu = host.to(device) if device.type == "cuda" else host
    _need(host.dim() == 1 and host.numel() >= 1, "cu_seqlens must be 1-D with n_seqs + 1 entries")
    _need(int(host[-1]) == T, f"cu_seqlens ends at {int(host[-1])}, but the tensors hold {T} tokens")
    return dev_cu, host


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
    _need(state.dim() == 4, "state must be [n_slots, H, dk, dv]")
    n_slots, H, dk, dv = state.shape
    if src is not None:
        _shape("src", src, state.shape)
        _state_code(src)
    _same_device(state, src=src)
    handle, _ = _stream(stream, state.device)
    _check(load().kda_state_init(_ptr(state), _state_code(state), n_slots, H, dk, dv, _ptr(src),
                                 _state_code(src) if src is not None else KDA_F32, handle))
    return state


def kda_device_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> torch.Tensor:
    """Copy src into dst (same number of bytes, contiguous, on one GPU) with the
    library's 16-byte non-temporal streaming copy: the bandwidth reference of
    the HBM-bound kernels."""
    _need(dst.is_contiguous() and src.is_contiguous(), "dst and src must be contiguous")
    nbytes = dst.numel() * dst.element_size()
    _need(src.numel() * src.element_size() == nbytes, "dst and src must hold the same bytes")
    _same_device(dst, src=src)
    handle, _ = _stream(stream, dst.device)
    _check(load().kda_device_copy(_ptr(dst), _ptr(src), nbytes, handle))
    return dst


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


def _workspace(nbytes: int, device, handle: int, st) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes, one per (device, stream):
    calls on one stream are ordered, so they may share it (the ABI allows that),
    while calls on different streams get different buffers.  A buffer that
    grows is replaced; the old one goes back to torch's allocator marked as used
    on its stream, so its memory is not reused before that stream's work on it
    has finished."""
    key = (torch.device(device), handle)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = _on_stream(torch.empty(nbytes, dtype=torch.uint8, device=device), st)
        _ws_cache[key] = buf
    return buf


def kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=None, chunk: int = 64,
                        initial_state=None, final_state=None, o=None,
                        output_final_state: bool = True, cu_seqlens_host=None,
                        workspace="auto", snapshots=None, snap_interval: int = 0,
                        a_log=None, out_gate=None, stream=None):
    """Chunked prefill over packed sequences.  q, k: [T, H, dk]; v: [T, H, dv];
    g: [T, H, dk] (per-channel decay) or [T, H] (per-head decay); beta: [T, H].
    With a_log ([H] fp32), g is the decay projection f (q's dtype) and beta the
    write-strength logits: log alpha = -exp(a_log) softplus(f), beta = sigmoid.
    out_gate: None, or the output gate's projection z [T, H, dv] in q's dtype:
    o is then o * sigmoid(z).
    Returns (o, final_state or None), or (o, final_state, snapshots) when
    snapshots is given.

    workspace: "auto" (a cached device buffer of kda_prefill_workspace_bytes_batch,
    one per device and stream), a uint8 device tensor, None (no workspace:
    the fused kernel), or "static": kda_prefill_chunked_noalloc, which runs the
    two-kernel path on the library's static scratch and allocates nothing (the
    binding still allocates o and final_state when they are not given).
    snapshots: None, True (allocate [n_seqs, longest // snap_interval, H, dk, dv]
    fp32 zeros) or such a tensor; entry [n, j] receives sequence n's state after
    (j + 1) * snap_interval tokens where it has that many."""
    _need(q.dim() == 3, "q must be [T, H, dk]")
    T, H, dk = q.shape
    _dtype("q", q, (torch.float32, torch.bfloat16))
    _shape("k", k, q.shape)
    _dtype("k", k, q.dtype)
    _need(v.dim() == 3 and tuple(v.shape[:2]) == (T, H), f"v must be [{T}, {H}, dv]")
    _dtype("v", v, q.dtype)
    dv = v.shape[2]
    _gate_check(g, q, a_log, (T,))
    _shape("beta", beta, (T, H))
    _dtype("beta", beta, torch.float32)
    cu_dev, cu_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, q.device)
    n_seqs = cu_host.numel() - 1
    for name, st_t in (("initial_state", initial_state), ("final_state", final_state)):
        if st_t is not None:
            _shape(name, st_t, (n_seqs, H, dk, dv))
            _dtype(name, st_t, torch.float32)
    if o is not None:
        _shape("o", o, (T, H, dv))
        _dtype("o", o, q.dtype)
    if out_gate is not None:
        _shape("out_gate", out_gate, (T, H, dv))
        _dtype("out_gate", out_gate, q.dtype)
    if isinstance(snapshots, torch.Tensor):
        _need(snapshots.dim() == 5 and tuple(snapshots.shape[:1]) == (n_seqs,) and
              tuple(snapshots.shape[2:]) == (H, dk, dv),
              f"snapshots must be [{n_seqs}, capacity, {H}, {dk}, {dv}]")
        _dtype("snapshots", snapshots, torch.float32)
    if isinstance(workspace, torch.Tensor):
        _dtype("workspace", workspace, torch.uint8)
    _same_device(q, k=k, v=v, g=g, beta=beta, a_log=a_log, initial_state=initial_state,
                 final_state=final_state, o=o, out_gate=out_gate,
                 snapshots=snapshots if isinstance(snapshots, torch.Tensor) else None,
                 workspace=workspace if isinstance(workspace, torch.Tensor) else None)
    handle, st = _stream(stream, q.device)
    want_snaps = snapshots is not None
    if snapshots is True:
        if snap_interval <= 0:
            raise ValueError("snap_interval must be positive")
        lens = cu_host[1:] - cu_host[:-1]
        cap = int(lens.max()) // snap_interval if n_seqs else 0
        snapshots = _on_stream(torch.zeros((n_seqs, cap, H, dk, dv), dtype=torch.float32,
                                           device=q.device), st)
    snap_cap = 0 if snapshots is None else int(snapshots.shape[1])
    if o is None:
        o = _on_stream(torch.empty((T, H, dv), dtype=q.dtype, device=q.device), st)
    if final_state is None and output_final_state:
        final_state = _on_stream(torch.empty((n_seqs, H, dk, dv), dtype=torch.float32,
                                             device=q.device), st)
    if workspace == "static":
        _check(load().kda_prefill_chunked_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q),
            _gate_code(g, q, a_log), _ptr(a_log), _ptr(cu_dev), cu_host.data_ptr(), n_seqs, H,
            dk, dv, int(chunk), _ptr(initial_state), _ptr(final_state), _ptr(out_gate), _ptr(o),
            _ptr(snapshots), int(snap_interval), snap_cap, handle))
        return (o, final_state, snapshots) if want_snaps else (o, final_state)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', 'static', a tensor or None")
        need = kda_prefill_workspace_bytes_batch(cu_host, H, dk, dv, chunk, q.dtype)
        workspace = _workspace(need, q.device, handle, st) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kda_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q),
        _gate_code(g, q, a_log), _ptr(a_log), _ptr(cu_dev), cu_host.data_ptr(), n_seqs, H, dk,
        dv, int(chunk), _ptr(initial_state), _ptr(final_state), _ptr(out_gate), _ptr(o),
        _ptr(snapshots), int(snap_interval), snap_cap, _ptr(workspace), ws_bytes, handle))
    if want_snaps:
        return o, final_state, snapshots
    return o, final_state


def _decode_checks(q, k, v, g, beta, state, slot_idx, o, a_log, lead, out_gate=None):
    """Shapes, dtypes and devices of a decode call; lead = (B,) or (B, n_tok)."""
    _dtype("q", q, (torch.float32, torch.bfloat16))
    _shape("k", k, q.shape)
    _dtype("k", k, q.dtype)
    H, dk = q.shape[-2], q.shape[-1]
    _need(v.dim() == q.dim() and tuple(v.shape[:-1]) == tuple(lead) + (H,),
          f"v must be {tuple(lead) + (H,)} + (dv,)")
    _dtype("v", v, q.dtype)
    dv = v.shape[-1]
    _gate_check(g, q, a_log, lead)
    _shape("beta", beta, tuple(lead) + (H,))
    _dtype("beta", beta, torch.float32)
    _need(state.dim() == 4 and tuple(state.shape[1:]) == (H, dk, dv),
          f"state must be [n_slots, {H}, {dk}, {dv}]")
    _state_code(state)
    if slot_idx is not None:
        _shape("slot_idx", slot_idx, (lead[0],))
        _dtype("slot_idx", slot_idx, torch.int32)
    for name, t in (("o", o), ("out_gate", out_gate)):
        if t is not None:
            _shape(name, t, tuple(lead) + (H, dv))
            _dtype(name, t, q.dtype)
    _same_device(q, k=k, v=v, g=g, beta=beta, a_log=a_log, state=state, slot_idx=slot_idx, o=o,
                 out_gate=out_gate)
    return H, dk, dv


def kda_decode_step(q, k, v, g, beta, state, slot_idx=None, o=None, a_log=None, out_gate=None,
                    stream=None):
    """One token per sequence.  q, k: [B, H, dk]; g: [B, H, dk] or [B, H] (or the
    decay projection with a_log, as in kda_prefill_chunked); v: [B, H, dv]; beta: [B, H];
    state [n_slots, H, dk, dv] fp32 or bf16, updated in place; slot_idx: int32
    [B] or None; out_gate: None or z [B, H, dv] (o * sigmoid(z)).  Returns
    o [B, H, dv]."""
    _need(q.dim() == 3, "q must be [B, H, dk]")
    B = q.shape[0]
    H, dk, dv = _decode_checks(q, k, v, g, beta, state, slot_idx, o, a_log, (B,), out_gate)
    handle, st = _stream(stream, q.device)
    if o is None:
        o = _on_stream(torch.empty((B, H, dv), dtype=q.dtype, device=q.device), st)
    _check(load().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q), _gate_code(g, q, a_log),
        _ptr(a_log), _ptr(state), _state_code(state), state.shape[0], _ptr(slot_idx), B, H, dk,
        dv, _ptr(out_gate), _ptr(o), handle))
    return o


def kda_decode_tokens(q, k, v, g, beta, state, slot_idx=None, o=None, token_states=None,
                      a_log=None, out_gate=None, stream=None):
    """n_tok consecutive tokens per sequence.  q, k: [B, n_tok, H, dk]; g: the same
    shape or [B, n_tok, H]; v: [B, n_tok, H, dv]; beta: [B, n_tok, H]; state
    [n_slots, H, dk, dv] fp32 or bf16, updated in place.  token_states: None,
    True (allocate [B, n_tok, H, dk, dv] of the state's dtype) or such a tensor.
    out_gate: None or z [B, n_tok, H, dv] (o * sigmoid(z)).
    Returns (o [B, n_tok, H, dv], token_states)."""
    _need(q.dim() == 4, "q must be [B, n_tok, H, dk]")
    B, n_tok = q.shape[0], q.shape[1]
    H, dk, dv = _decode_checks(q, k, v, g, beta, state, slot_idx, o, a_log, (B, n_tok),
                               out_gate)
    if isinstance(token_states, torch.Tensor):
        _shape("token_states", token_states, (B, n_tok, H, dk, dv))
        _dtype("token_states", token_states, state.dtype)
        _same_device(q, token_states=token_states)
    handle, st = _stream(stream, q.device)
    if o is None:
        o = _on_stream(torch.empty((B, n_tok, H, dv), dtype=q.dtype, device=q.device), st)
    if token_states is True:
        token_states = _on_stream(torch.empty((B, n_tok, H, dk, dv), dtype=state.dtype,
                                              device=q.device), st)
    _check(load().kda_decode_tokens(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q), _gate_code(g, q, a_log),
        _ptr(a_log), _ptr(state), _state_code(state), state.shape[0], _ptr(slot_idx), B, n_tok,
        H, dk, dv, _ptr(out_gate), _ptr(o), _ptr(token_states) if token_states is not None else None,
        handle))
    return o, token_states


def _conv_checks(x, w, y, tails):
    _need(x.dim() == 2, "x must be [tokens, channels]")
    _dtype("x", x, (torch.float32, torch.bfloat16))
    channels = x.shape[1]
    _shape("w", w, (channels, 4))
    _dtype("w", w, torch.float32)
    if y is not None:
        _shape("y", y, x.shape)
        _dtype("y", y, x.dtype)
    for name, t in tails.items():
        if t is not None:
            _need(t.dim() == 3 and tuple(t.shape[1:]) == (3, channels),
                  f"{name} must be [slots, 3, {channels}]")
            _dtype(name, t, x.dtype)


def kda_short_conv_prefill(x, w, cu_seqlens=None, l2_head_dim: int = 0, l2_eps: float = 1e-6,
                           conv_tail_in=None, conv_tail_out=None, y=None, cu_seqlens_host=None,
                           stream=None):
    """Width-4 causal depthwise conv (+ per-head L2 norm) over x [T, channels]."""
    _conv_checks(x, w, y, {"conv_tail_in": conv_tail_in, "conv_tail_out": conv_tail_out})
    T, channels = x.shape
    cu_dev, cu_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, x.device)
    n_seqs = cu_host.numel() - 1
    for name, t in (("conv_tail_in", conv_tail_in), ("conv_tail_out", conv_tail_out)):
        if t is not None:
            _need(t.shape[0] == n_seqs, f"{name} must hold {n_seqs} sequences")
    _same_device(x, w=w, y=y, conv_tail_in=conv_tail_in, conv_tail_out=conv_tail_out)
    handle, st = _stream(stream, x.device)
    if y is None:
        y = _on_stream(torch.empty_like(x), st)
    _check(load().kda_short_conv_prefill(
        _ptr(x), _ptr(w), _dtype_code(x), _ptr(cu_dev), cu_host.data_ptr(), n_seqs, channels,
        int(l2_head_dim), float(l2_eps), _ptr(conv_tail_in), _ptr(conv_tail_out), _ptr(y),
        handle))
    return y


def kda_short_conv_decode(x, w, conv_tail, slot_idx=None, l2_head_dim: int = 0,
                          l2_eps: float = 1e-6, y=None, stream=None):
    """One token per sequence: x [B, channels]; conv_tail [n_slots, 3, channels]
    updated in place; slot_idx int32 [B] or None.  Returns y [B, channels]."""
    _conv_checks(x, w, y, {"conv_tail": conv_tail})
    B, channels = x.shape
    if slot_idx is not None:
        _shape("slot_idx", slot_idx, (B,))
        _dtype("slot_idx", slot_idx, torch.int32)
    _same_device(x, w=w, y=y, conv_tail=conv_tail, slot_idx=slot_idx)
    handle, st = _stream(stream, x.device)
    if y is None:
        y = _on_stream(torch.empty_like(x), st)
    _check(load().kda_short_conv_decode(
        _ptr(x), _ptr(w), _dtype_code(x), _ptr(conv_tail), conv_tail.shape[0], _ptr(slot_idx),
        B, channels, int(l2_head_dim), float(l2_eps), _ptr(y), handle))
    return y
