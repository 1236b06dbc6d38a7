"""The C ABI without a GPU: the library loads, exports every symbol that
include/kda.h declares, and rejects bad arguments on the host before anything
is enqueued.  Fake (never dereferenced) device addresses are used, and every
call here fails validation, so no HIP call is made."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_99_amd as kda_pkg
from gated_delta_rule_99_amd.kda import (KDA_BF16, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED,
                                          KDA_ERR_WORKSPACE_TOO_SMALL, KDA_F32)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

A = 0x10000  # fake 16-byte-aligned addresses, never dereferenced
Bp = 0x20000000
Cp = 0x40000000
Dp = 0x60000000
Ep = 0x80000000
Fp = 0xA0000000
Gp = 0xC0000000
Hp = 0xE0000000


@pytest.fixture(scope="module")
def lib():
    return kda_pkg.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(kda_pkg.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_state_bytes(lib):
    assert lib.kda_state_bytes(64, 128, 128, KDA_F32) == 4194304
    assert lib.kda_state_bytes(64, 128, 128, KDA_BF16) == 2097152
    assert lib.kda_state_bytes(0, 128, 128, KDA_F32) == 0
    assert lib.kda_state_bytes(64, 128, 128, 7) == 0
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(4) == b"KDA_ERR_WORKSPACE_TOO_SMALL"


def cu_arr(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def prefill(lib, **kw):
    a = dict(q=A, k=Bp, v=Cp, g=Dp, beta=Ep, dtype=KDA_BF16, gate=0, a_log=None, cu_dev=Fp,
             cu_host=cu_arr([0, 8]), n=1, H=2, dk=128, dv=128, chunk=64, s0=None, sf=None, og=None,
             o=Gp, snaps=None, snap_interval=0, snap_capacity=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kda_prefill_chunked(a["q"], a["k"], a["v"], a["g"], a["beta"], a["dtype"],
                                   a["gate"], a["a_log"], a["cu_dev"], a["cu_host"], a["n"], a["H"], a["dk"],
                                   a["dv"],
                                   a["chunk"], a["s0"], a["sf"], a["og"], a["o"], a["snaps"],
                                   a["snap_interval"], a["snap_capacity"], a["ws"], a["ws_bytes"],
                                   a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dk=96, dv=96), KDA_ERR_UNSUPPORTED, "head dim"),
    (dict(dk=128, dv=64), KDA_ERR_UNSUPPORTED, "dk != dv"),
    (dict(H=0), KDA_ERR_INVALID_ARGUMENT, "positive"),
    (dict(chunk=48), KDA_ERR_INVALID_ARGUMENT, "chunk"),
    (dict(dtype=7), KDA_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(gate=3), KDA_ERR_INVALID_ARGUMENT, "gate layout"),
    (dict(gate=2), KDA_ERR_INVALID_ARGUMENT, "needs a_log"),
    (dict(gate=2, a_log=Hp + 2), KDA_ERR_INVALID_ARGUMENT, "needs a_log"),
    (dict(gate=0, a_log=Hp), KDA_ERR_INVALID_ARGUMENT, "only taken"),
    (dict(gate=2, a_log=Gp + 64), KDA_ERR_INVALID_ARGUMENT, "o overlaps"),
    (dict(n=-1), KDA_ERR_INVALID_ARGUMENT, "n_seqs"),
    (dict(cu_host=None), KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host"),
    (dict(cu_host=cu_arr([1, 8])), KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0]"),
    (dict(cu_host=cu_arr([0, 8, 4]), n=2), KDA_ERR_INVALID_ARGUMENT, "decreases"),
    (dict(cu_dev=None), KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_dev"),
    (dict(q=None), KDA_ERR_INVALID_ARGUMENT, "required"),
    (dict(k=Bp + 8), KDA_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(o=A + 64), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(s0=0x7000000, sf=0x7000040), KDA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(sf=A), KDA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(ws=0x9000000, ws_bytes=1024), KDA_ERR_WORKSPACE_TOO_SMALL, "needed"),
    (dict(ws=0x9000008, ws_bytes=1 << 30), KDA_ERR_INVALID_ARGUMENT, "misaligned workspace"),
    (dict(ws=A - 4096, ws_bytes=1 << 30), KDA_ERR_INVALID_ARGUMENT, "workspace overlaps"),
    (dict(snaps=Hp, snap_interval=48, snap_capacity=1), KDA_ERR_INVALID_ARGUMENT,
     "positive multiple of chunk"),
    (dict(snaps=Hp, snap_interval=0, snap_capacity=1), KDA_ERR_INVALID_ARGUMENT,
     "positive multiple of chunk"),
    (dict(snaps=Hp, snap_interval=64, snap_capacity=-1), KDA_ERR_INVALID_ARGUMENT,
     "snap_capacity"),
    (dict(snaps=Hp + 8, snap_interval=64, snap_capacity=1), KDA_ERR_INVALID_ARGUMENT,
     "misaligned snapshots"),
    (dict(snaps=Gp - 65536, snap_interval=64, snap_capacity=1), KDA_ERR_INVALID_ARGUMENT,
     "snapshots overlap"),
    (dict(snaps=Hp, snap_interval=64, snap_capacity=2, s0=Hp + 2 * 65536),
     KDA_ERR_INVALID_ARGUMENT, "snapshots overlap"),
    (dict(og=Hp + 8), KDA_ERR_INVALID_ARGUMENT, "misaligned out_gate"),
    (dict(og=Gp + 16), KDA_ERR_INVALID_ARGUMENT, "o overlaps"),
    (dict(og=Hp, sf=Hp + 64), KDA_ERR_INVALID_ARGUMENT, "final_state overlaps out_gate"),
])
def test_prefill_rejects(lib, kw, status, needle):
    assert prefill(lib, **kw) == status
    assert needle in lib.kda_last_error_detail().decode()


def test_prefill_workspace_bytes(lib):
    """State carry (64 KiB per sequence and head), the rank table (4 bytes per
    sequence, rounded up to 256) and a window of 58 112-byte chunk tiles; 0 for
    shapes that run without a workspace."""
    f = lib.kda_prefill_workspace_bytes
    # one sequence, 64 heads: a full 32-chunk window is below the 192 MiB budget
    assert f(1, 64, 128, 128, 64, KDA_BF16) == 64 * 65536 + 256 + 32 * 64 * 58112
    # four sequences, 64 heads: the 192 MiB budget
    assert f(4, 64, 128, 128, 64, KDA_BF16) == 4 * 64 * 65536 + 256 + (192 << 20)
    # large batches keep one chunk per sequence and head
    assert f(256, 64, 128, 128, 64, KDA_BF16) == 256 * 64 * (65536 + 58112) + 1024
    assert f(1, 64, 128, 128, 64, KDA_F32) == 0
    assert f(1, 64, 64, 64, 64, KDA_BF16) == 0
    assert f(1, 64, 128, 128, 32, KDA_BF16) == 0
    assert f(0, 64, 128, 128, 64, KDA_BF16) == 0


def test_prefill_workspace_bytes_batch(lib):
    """Windows of min(32, longest) chunks of every sequence while those tiles
    stay within 4 GiB; never below the minimum; the minimum for an invalid
    cu_seqlens_host; 0 for shapes without a workspace."""
    f = lib.kda_prefill_workspace_bytes_batch
    fixed = lambda n: n * 64 * 65536 + ((n * 4 + 255) // 256) * 256
    # 64 sequences of 8 chunks: all 8 chunks of each
    cu = cu_arr([512 * i for i in range(65)])
    assert f(cu, 64, 64, 128, 128, 64, KDA_BF16) == fixed(64) + 8 * 64 * 64 * 58112
    # 24 sequences of 2048 tokens: 32-chunk windows (2.86 GB of tiles)
    cu = cu_arr([2048 * i for i in range(25)])
    assert f(cu, 24, 64, 128, 128, 64, KDA_BF16) == fixed(24) + 32 * 24 * 64 * 58112
    # 256 sequences of 4096 tokens: capped at 4 GiB of tiles (4 chunks)
    cu = cu_arr([4096 * i for i in range(257)])
    assert f(cu, 256, 64, 128, 128, 64, KDA_BF16) == fixed(256) + 4 * 256 * 64 * 58112
    # one short sequence: the minimum (the 192 MiB budget's 32-chunk window)
    cu = cu_arr([0, 100])
    assert f(cu, 1, 64, 128, 128, 64, KDA_BF16) == \
        lib.kda_prefill_workspace_bytes(1, 64, 128, 128, 64, KDA_BF16)
    bad = cu_arr([0, 8, 4])
    assert f(bad, 2, 64, 128, 128, 64, KDA_BF16) == \
        lib.kda_prefill_workspace_bytes(2, 64, 128, 128, 64, KDA_BF16)
    assert f(cu_arr([0, 100]), 1, 64, 64, 64, 64, KDA_BF16) == 0


def test_prefill_nothing_to_do(lib):
    """n_seqs = 0 is valid and enqueues nothing."""
    assert prefill(lib, n=0, cu_host=cu_arr([0]), q=None, k=None, v=None, g=None, beta=None,
                   o=None) == 0


def decode(lib, **kw):
    a = dict(q=A, k=Bp, v=Cp, g=Dp, beta=Ep, dtype=KDA_F32, gate=0, a_log=None, state=Fp,
             sdt=KDA_F32, n_slots=4, slot=None, B=4, H=2, dk=64, dv=64, og=None, o=Gp, stream=None)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["dtype"], a["gate"],
                               a["a_log"], a["state"], a["sdt"], a["n_slots"], a["slot"], a["B"], a["H"],
                               a["dk"], a["dv"], a["og"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dk=48, dv=48), KDA_ERR_UNSUPPORTED, "head dim"),
    (dict(gate=-1), KDA_ERR_INVALID_ARGUMENT, "gate layout"),
    (dict(gate=2), KDA_ERR_INVALID_ARGUMENT, "needs a_log"),
    (dict(gate=1, a_log=Hp), KDA_ERR_INVALID_ARGUMENT, "only taken"),
    (dict(gate=2, a_log=Fp + 256), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(B=-1), KDA_ERR_INVALID_ARGUMENT, ">= 0"),
    (dict(n_slots=3), KDA_ERR_INVALID_ARGUMENT, "n_slots"),
    (dict(state=None), KDA_ERR_INVALID_ARGUMENT, "required"),
    (dict(state=Fp + 4), KDA_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(slot=Gp + 2, n_slots=8), KDA_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(o=A), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(state=Dp), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(sdt=3), KDA_ERR_INVALID_ARGUMENT, "state dtype"),
    # a bf16 state is half the bytes: this one ends just below o, an fp32 one would not
    (dict(state=Gp - 4 * 2 * 64 * 64 * 2, sdt=KDA_F32), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(og=Hp + 4), KDA_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(og=Gp + 64), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
])
def test_decode_rejects(lib, kw, status, needle):
    assert decode(lib, **kw) == status
    assert needle in lib.kda_last_error_detail().decode()


def decode_tokens(lib, **kw):
    a = dict(q=A, k=Bp, v=Cp, g=Dp, beta=Ep, dtype=KDA_BF16, gate=1, a_log=None, state=Fp,
             sdt=KDA_BF16, n_slots=4, slot=None, B=4, n_tok=3, H=2, dk=128, dv=128, og=None,
             o=Gp, snaps=None, stream=None)
    a.update(kw)
    return lib.kda_decode_tokens(a["q"], a["k"], a["v"], a["g"], a["beta"], a["dtype"],
                                 a["gate"], a["a_log"], a["state"], a["sdt"], a["n_slots"], a["slot"], a["B"],
                                 a["n_tok"], a["H"], a["dk"], a["dv"], a["og"], a["o"], a["snaps"],
                                 a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n_tok=0), KDA_ERR_INVALID_ARGUMENT, "n_tok"),
    (dict(n_tok=65), KDA_ERR_INVALID_ARGUMENT, "n_tok"),
    (dict(snaps=0x9000008), KDA_ERR_INVALID_ARGUMENT, "misaligned"),
    (dict(snaps=Fp + 4096), KDA_ERR_INVALID_ARGUMENT, "token_states overlaps"),
    (dict(dk=96, dv=96), KDA_ERR_UNSUPPORTED, "head dim"),
    (dict(n_slots=3), KDA_ERR_INVALID_ARGUMENT, "n_slots"),
    (dict(gate=2, a_log=None), KDA_ERR_INVALID_ARGUMENT, "needs a_log"),
])
def test_decode_tokens_rejects(lib, kw, status, needle):
    assert decode_tokens(lib, **kw) == status
    assert needle in lib.kda_last_error_detail().decode()


def test_state_init_rejects(lib):
    f = lib.kda_state_init
    assert f(None, KDA_F32, 2, 2, 64, 64, None, KDA_F32, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, KDA_F32, 2, 2, 64, 32, None, KDA_F32, None) == KDA_ERR_UNSUPPORTED
    assert f(A, KDA_F32, -1, 2, 64, 64, None, KDA_F32, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, KDA_F32, 2, 2, 64, 64, A + 16, KDA_F32, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, 5, 2, 2, 64, 64, None, KDA_F32, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, KDA_BF16, 2, 2, 64, 64, Bp, 5, None) == KDA_ERR_INVALID_ARGUMENT
    # 2 fp32 states of 2 x 64 x 64 end 64 KiB after A; a bf16 source there overlaps
    assert f(A, KDA_F32, 2, 2, 64, 64, A + 65536 - 16, KDA_BF16, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, KDA_F32, 0, 2, 64, 64, None, KDA_F32, None) == 0


def conv(lib, **kw):
    a = dict(x=A, w=Bp, dtype=KDA_BF16, cu_dev=Cp, cu_host=cu_arr([0, 10]), n=1, ch=256, l2=128,
             eps=1e-6, tin=None, tout=None, y=Dp, stream=None)
    a.update(kw)
    return lib.kda_short_conv_prefill(a["x"], a["w"], a["dtype"], a["cu_dev"], a["cu_host"], a["n"],
                                      a["ch"], a["l2"], a["eps"], a["tin"], a["tout"], a["y"],
                                      a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ch=255), KDA_ERR_INVALID_ARGUMENT, "even"),
    (dict(l2=96), KDA_ERR_INVALID_ARGUMENT, "l2_head_dim"),
    (dict(ch=1024, l2=512), KDA_ERR_UNSUPPORTED, "256"),
    (dict(w=None), KDA_ERR_INVALID_ARGUMENT, "w must"),
    (dict(eps=-1.0), KDA_ERR_INVALID_ARGUMENT, "l2_eps"),
    (dict(y=A), KDA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(tin=Ep, tout=Ep + 16), KDA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(cu_host=cu_arr([0, 5, 2]), n=2), KDA_ERR_INVALID_ARGUMENT, "decreases"),
])
def test_conv_prefill_rejects(lib, kw, status, needle):
    assert conv(lib, **kw) == status
    assert needle in lib.kda_last_error_detail().decode()


def test_dispatch_size_rejects(lib):
    """Launches beyond 2^32 work-items are refused before any HIP call: decode
    spends up to 1024 work-items per (sequence, head), prefill up to 1024 per
    workgroup (4 workgroups per head of d = 128), the convolution 256 per 16
    tokens and 64 per decoded sequence."""
    assert decode(lib, B=4194304, H=1, slot=Hp, n_slots=8) == KDA_ERR_UNSUPPORTED
    assert "dispatch" in lib.kda_last_error_detail().decode()
    n = 4194304 // (64 * 4)
    assert prefill(lib, n=n, H=64, cu_host=cu_arr([0] * (n + 1))) == KDA_ERR_UNSUPPORTED
    assert "dispatch" in lib.kda_last_error_detail().decode()
    assert conv(lib, cu_host=cu_arr([0, 1 << 28])) == KDA_ERR_UNSUPPORTED
    assert "dispatch" in lib.kda_last_error_detail().decode()
    assert lib.kda_short_conv_decode(A, Bp, KDA_BF16, Cp, 4, Ep, 1 << 26, 256, 128, 1e-6, Dp,
                                     None) == KDA_ERR_UNSUPPORTED
    assert "dispatch" in lib.kda_last_error_detail().decode()


def test_conv_decode_rejects(lib):
    f = lib.kda_short_conv_decode
    assert f(A, Bp, KDA_BF16, None, 4, None, 2, 256, 128, 1e-6, Dp, None) == \
        KDA_ERR_INVALID_ARGUMENT
    assert f(A, Bp, KDA_BF16, Cp, 1, None, 2, 256, 128, 1e-6, Dp, None) == \
        KDA_ERR_INVALID_ARGUMENT
    assert f(A, Bp, KDA_BF16, Cp, 4, None, 2, 256, 128, 1e-6, A, None) == \
        KDA_ERR_INVALID_ARGUMENT


def test_device_copy_rejects(lib):
    f = lib.kda_device_copy
    assert f(A, Bp, 0, None) == 0  # nothing to copy: no HIP call
    assert f(None, Bp, 64, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, None, 64, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A + 8, Bp, 64, None) == KDA_ERR_INVALID_ARGUMENT
    assert f(A, Bp, 72, None) == KDA_ERR_INVALID_ARGUMENT
    assert "aligned" in lib.kda_last_error_detail().decode()
    assert f(A, A + 32, 64, None) == KDA_ERR_INVALID_ARGUMENT
    assert "overlap" in lib.kda_last_error_detail().decode()


def test_python_binding_raises_on_error(lib):
    """The binding turns a non-OK status into KdaError with the library's detail
    (no fallback)."""
    from gated_delta_rule_99_amd import kda as binding
    assert prefill(lib, dk=96, dv=96) == KDA_ERR_UNSUPPORTED
    with pytest.raises(kda_pkg.KdaError) as ei:
        binding._check(KDA_ERR_UNSUPPORTED)
    assert ei.value.status == KDA_ERR_UNSUPPORTED and "head dim" in ei.value.detail


def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float32)


def _prefill_args(T=8, H=2, d=128, n=1, bf16=True):
    import torch
    dt = torch.bfloat16 if bf16 else torch.float32
    cu = torch.tensor([0, T] if n == 1 else [0, T // 2, T], dtype=torch.int32)
    return dict(q=_t(T, H, d, dtype=dt), k=_t(T, H, d, dtype=dt), v=_t(T, H, d, dtype=dt),
                g=_t(T, H, d), beta=_t(T, H), cu_seqlens=cu)


def _call_prefill(args, **kw):
    a = dict(args)
    a.update(kw)
    return kda_pkg.kda_prefill_chunked(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"),
                                       a.pop("beta"), **a)


@pytest.mark.parametrize("change,err,needle", [
    # the host cu_seqlens must end at the tokens the tensors hold
    (dict(cu_seqlens="long"), ValueError, "cu_seqlens ends at"),
    (dict(k="f32"), TypeError, "k has dtype"),
    (dict(v="short"), ValueError, "v must be"),
    (dict(g="bf16"), TypeError, "g has dtype"),
    (dict(g="wide"), ValueError, "g has shape"),
    (dict(beta="bf16"), TypeError, "beta has dtype"),
    (dict(beta="short"), ValueError, "beta has shape"),
    (dict(o="f32"), TypeError, "o has dtype"),
    (dict(final_state="short"), ValueError, "final_state has shape"),
    (dict(initial_state="bf16"), TypeError, "initial_state has dtype"),
    (dict(a_log="f32 g"), TypeError, "g has dtype"),
    (dict(), ValueError, "runs on a GPU"),
])
def test_binding_checks_prefill_arguments(change, err, needle):
    """What the C ABI cannot see from raw pointers (sizes, dtypes, devices) is
    checked by the binding before any call: each mismatch raises, none reaches
    a kernel.  CPU tensors stop at the device check, which runs last."""
    import torch
    a = _prefill_args()
    T, H, d = a["q"].shape
    if change.get("cu_seqlens") == "long":
        a["cu_seqlens"] = torch.tensor([0, T + 8], dtype=torch.int32)
    if change.get("k") == "f32":
        a["k"] = a["k"].float()
    if change.get("v") == "short":
        a["v"] = _t(T - 1, H, d, dtype=torch.bfloat16)
    if change.get("g") == "bf16":
        a["g"] = a["g"].bfloat16()
    if change.get("g") == "wide":
        a["g"] = _t(T, H, 2 * d)
    if change.get("beta") == "bf16":
        a["beta"] = a["beta"].bfloat16()
    if change.get("beta") == "short":
        a["beta"] = _t(T, H - 1)
    if change.get("o") == "f32":
        a["o"] = _t(T, H, d)
    if change.get("final_state") == "short":
        a["final_state"] = _t(1, H, d, d // 2)
    if change.get("initial_state") == "bf16":
        a["initial_state"] = _t(1, H, d, d, dtype=torch.bfloat16)
    if change.get("a_log") == "f32 g":
        a["a_log"] = _t(H)  # then g must be the bf16 projection, not fp32
    with pytest.raises(err) as ei:
        _call_prefill(a, workspace=None)
    assert needle in str(ei.value)


@pytest.mark.parametrize("change,err,needle", [
    (dict(slot_idx="int64"), TypeError, "slot_idx has dtype"),
    (dict(slot_idx="short"), ValueError, "slot_idx has shape"),
    (dict(state="bad"), ValueError, "state must be"),
    (dict(v="bad"), ValueError, "v must be"),
    (dict(), ValueError, "runs on a GPU"),
])
def test_binding_checks_decode_arguments(change, err, needle):
    import torch
    B, H, d = 3, 2, 64
    bf = torch.bfloat16
    a = dict(q=_t(B, H, d, dtype=bf), k=_t(B, H, d, dtype=bf), v=_t(B, H, d, dtype=bf),
             g=_t(B, H, d), beta=_t(B, H), state=_t(5, H, d, d),
             slot_idx=torch.zeros(B, dtype=torch.int32))
    if change.get("slot_idx") == "int64":
        a["slot_idx"] = torch.zeros(B, dtype=torch.int64)
    if change.get("slot_idx") == "short":
        a["slot_idx"] = torch.zeros(B - 1, dtype=torch.int32)
    if change.get("state") == "bad":
        a["state"] = _t(5, H, d, d + 1)
    if change.get("v") == "bad":
        a["v"] = _t(B + 1, H, d, dtype=bf)
    with pytest.raises(err) as ei:
        kda_pkg.kda_decode_step(**a)
    assert needle in str(ei.value)
    tok = {k_: (v_.unsqueeze(1) if k_ not in ("state", "slot_idx") else v_) for k_, v_ in a.items()}
    with pytest.raises(err):
        kda_pkg.kda_decode_tokens(**tok)


def test_noalloc_rejects_beyond_its_scratch(lib):
    """The no-allocation prefill rejects, before any HIP call, a batch whose
    workspace exceeds the static scratch (128 MiB): 64 sequences x 64 heads
    need 64 * 64 * (65536 + 58112) bytes and more."""
    f = lib.kda_prefill_chunked_noalloc
    n = 64
    cu = cu_arr(list(range(0, 64 * (n + 1), 64)))
    st = f(A, Bp, Cp, Dp, Ep, KDA_BF16, 0, None, Fp, cu, n, 64, 128, 128, 64, None, None, None,
           Gp, None, 0, 0, None)
    assert st == KDA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch holds 134217728" in lib.kda_last_error_detail().decode()
