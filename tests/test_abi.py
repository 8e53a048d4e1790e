"""The C-ABI library loads, exports every entry point of include/fa.h, and
rejects bad arguments on the host before any GPU work (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import exact_attention_forward_04_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_ex", "fa_exp2_emu", "fa_schedule", "fa_status_string"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for st in (0, -1, -2, -3, -4, -5):
        assert fa.status_string(st).startswith(("FA_OK", "FA_ERR"))
    assert fa.status_string(12345) == "unknown fa_status"
    assert fa.version() >= 100


def test_default_tuning():
    t = fa.default_tuning()
    assert t.tau == 8.0 and t.exp2_emu == 0 and t.schedule == 0 and not t.counters


# Fake, 16-byte aligned, never-dereferenced addresses: validation must reject
# the call before anything touches them.
A = 0x10000


def call(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, S=8, D=128, scale=0.1, causal=0, cu=None):
    lib = fa.load()
    return lib.fa_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, cu, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(S=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(D=512), fa.FA_ERR_UNSUPPORTED),
])
def test_validation_rejects(kw, expect):
    assert call(**kw) == expect


def test_tuning_validation():
    lib = fa.load()
    for field, val in (("tau", -1.0), ("tau", float("nan")), ("tau", 64.5), ("tau", float("inf")),
                       ("exp2_emu", 3), ("schedule", 2)):
        t = fa.default_tuning()
        setattr(t, field, val)
        rc = lib.fa_fwd_ex(A, A, A, A, A, 1, 1, 8, 128, 0.1, 0, None, None, ctypes.byref(t))
        assert rc == fa.FA_ERR_INVALID_ARG, (field, val)
    # the largest accepted threshold passes validation (then finds no device here)
    t = fa.default_tuning()
    t.tau = 64.0
    rc = lib.fa_fwd_ex(A, A, A, A, A, 1, 1, 8, 128, 0.1, 0, None, None, ctypes.byref(t))
    assert rc != fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("H,H_kv,expect", [
    (4, 3, fa.FA_ERR_INVALID_ARG),   # K/V heads must divide the query heads
    (4, 0, fa.FA_ERR_INVALID_ARG),
    (4, -2, fa.FA_ERR_INVALID_ARG),
    (2, 4, fa.FA_ERR_INVALID_ARG),   # more K/V heads than query heads
])
def test_gqa_head_validation(H, H_kv, expect):
    lib = fa.load()
    rc = lib.fa_fwd_gqa(A, A, A, A, A, 1, H, H_kv, 8, 128, 0.1, 1, None, None, None)
    assert rc == expect


@pytest.mark.parametrize("D,D_v,expect", [
    (192, 192, fa.FA_ERR_UNSUPPORTED),
    (128, 64, fa.FA_ERR_UNSUPPORTED),
    (256, 128, fa.FA_ERR_UNSUPPORTED),
    (192, 0, fa.FA_ERR_INVALID_ARG),
])
def test_head_dim_pair_validation(D, D_v, expect):
    lib = fa.load()
    rc = lib.fa_fwd_hd(A, A, A, A, A, 1, 2, 2, 8, D, D_v, 0.1, 1, None, None, None)
    assert rc == expect


def test_general_entry_validation():
    lib = fa.load()
    # one offset array without the other
    assert lib.fa_fwd_general(A, A, A, A, A, 2, 4, 2, 8, 16, 128, 128, 0.1, 1, A, None, None,
                              None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_general(A, A, A, A, A, 2, 4, 2, 8, 16, 128, 128, 0.1, 1, None, A, None,
                              None) == fa.FA_ERR_INVALID_ARG
    # key length must be positive
    assert lib.fa_fwd_general(A, A, A, A, A, 2, 4, 2, 8, 0, 128, 128, 0.1, 1, None, None, None,
                              None) == fa.FA_ERR_INVALID_ARG


def test_fa_fwd_rejects_d192_without_a_value_dimension():
    assert call(D=192) == fa.FA_ERR_UNSUPPORTED


def test_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == fa.FA_ERR_NO_DEVICE
    assert fa.load().fa_exp2_emu(A, A, 16, None) == fa.FA_ERR_NO_DEVICE
    assert fa.load().fa_fwd_gqa(A, A, A, A, A, 1, 8, 2, 8, 128, 0.1, 1, None, None,
                                None) == fa.FA_ERR_NO_DEVICE
    assert fa.load().fa_fwd_hd(A, A, A, A, A, 1, 8, 2, 8, 192, 128, 0.1, 1, None, None,
                               None) == fa.FA_ERR_NO_DEVICE
    assert fa.load().fa_fwd_general(A, A, A, A, A, 1, 8, 2, 3, 900, 128, 128, 0.1, 1, None,
                                    None, None, None) == fa.FA_ERR_NO_DEVICE


def test_exp2_emu_argument_checks():
    lib = fa.load()
    assert lib.fa_exp2_emu(A, A, -1, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_exp2_emu(None, A, 4, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_exp2_emu(A + 1, A, 4, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_exp2_emu(None, None, 0, None) == fa.FA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)


def bwd_call(**kw):
    """fa_bwd with valid arguments except those overridden."""
    a = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, delta=A, B=1, H=8, H_kv=2,
             S=64, D=128, scale=0.1, causal=1, cu=None)
    a.update(kw)
    return fa.load().fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"],
                            a["dk"], a["dv"], a["delta"], a["B"], a["H"], a["H_kv"], a["S"],
                            a["D"], a["scale"], a["causal"], a["cu"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dout=None), fa.FA_ERR_INVALID_ARG),
    (dict(delta=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=A + 8), fa.FA_ERR_INVALID_ARG),        # not 16-byte aligned
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),       # not 4-byte aligned
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(S=-1), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),          # does not divide H
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(D=192), fa.FA_ERR_UNSUPPORTED),           # (192, 192): only fa_bwd_hd's (192, 128)
    (dict(S=1 << 30, H=8), fa.FA_ERR_UNSUPPORTED),  # beyond 32-bit row indexing
])
def test_backward_validation_rejects(kw, expect):
    assert bwd_call(**kw) == expect


def test_backward_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bwd_call() == fa.FA_ERR_NO_DEVICE
    assert bwd_call(D=64, H_kv=8, causal=0) == fa.FA_ERR_NO_DEVICE
    assert bwd_call(D=256) == fa.FA_ERR_NO_DEVICE


def test_backward_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        fa.attention_backward(q, q, q, q, lse, q)


def test_splitkv_workspace_size():
    lib = fa.load()
    # splits x B x S_q x H x (D_v + 1) x 4 bytes; one split (or fewer key
    # blocks than two) needs none
    assert lib.fa_splitkv_workspace_size(2, 4, 1, 1000, 128, 4) == 4 * 2 * 1 * 4 * 129 * 4
    assert lib.fa_splitkv_workspace_size(2, 4, 1, 1000, 128, 1) == 0
    assert lib.fa_splitkv_workspace_size(1, 1, 1, 64, 128, 8) == 0       # one key block
    # 1000 keys = 16 blocks: 5 requested -> 4 blocks per split -> 4 splits
    assert lib.fa_splitkv_workspace_size(1, 1, 1, 1000, 64, 5) == 4 * 1 * 1 * 1 * 65 * 4
    assert lib.fa_splitkv_workspace_size(0, 4, 1, 1000, 128, 4) == 0
    assert lib.fa_splitkv_workspace_size(1, 4, 1, 1000, 128, -1) == 0


def splitkv_call(**kw):
    a = dict(B=1, H=8, H_kv=2, S_q=1, S_k=4096, D=128, D_v=128, scale=0.1, causal=1,
             splits=4, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return fa.load().fa_fwd_splitkv(A, A, A, A, A, a["B"], a["H"], a["H_kv"], a["S_q"], a["S_k"],
                                    a["D"], a["D_v"], a["scale"], a["causal"], None, None,
                                    a["splits"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=65), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws=A + 4), fa.FA_ERR_INVALID_ARG),        # misaligned workspace
    (dict(ws_bytes=100), fa.FA_ERR_INVALID_ARG),     # too small
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(D=96, D_v=96), fa.FA_ERR_UNSUPPORTED),
])
def test_splitkv_validation_rejects(kw, expect):
    assert splitkv_call(**kw) == expect


def test_splitkv_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert splitkv_call() == fa.FA_ERR_NO_DEVICE
    n = ctypes.c_int(0)
    assert fa.load().fa_splitkv_auto_splits(1, 8, 1, 4096, 128, ctypes.byref(n)) == fa.FA_ERR_NO_DEVICE


def splitkv_noalloc_call(**kw):
    a = dict(B=1, H=8, H_kv=2, S_q=1, S_k=4096, D=128, D_v=128, scale=0.1, causal=1, splits=4)
    a.update(kw)
    return fa.load().fa_fwd_splitkv_noalloc(A, A, A, A, A, a["B"], a["H"], a["H_kv"], a["S_q"],
                                            a["S_k"], a["D"], a["D_v"], a["scale"], a["causal"],
                                            None, None, a["splits"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=65), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(D=96, D_v=96), fa.FA_ERR_UNSUPPORTED),
    # 64 splits x 32 x 1 x 32 rows x 129 floats = 33.8 MB > the 16 MiB scratch
    (dict(B=32, H=32, H_kv=8, S_k=8192, splits=64), fa.FA_ERR_TOO_LARGE),
])
def test_splitkv_noalloc_validation_rejects(kw, expect):
    assert splitkv_noalloc_call(**kw) == expect


def test_splitkv_noalloc_limit_matches_workspace_size():
    """The scratch limit is checked against the same byte count the
    workspace variant asks for: the largest batch that fits is accepted (it
    reaches the device check), one more sequence is refused."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = fa.load()
    per_seq = lib.fa_splitkv_workspace_size(1, 32, 1, 8192, 128, 64)
    fit = fa.SPLITKV_SCRATCH_BYTES // per_seq
    assert lib.fa_splitkv_workspace_size(fit, 32, 1, 8192, 128, 64) <= fa.SPLITKV_SCRATCH_BYTES
    assert splitkv_noalloc_call(B=fit, H=32, H_kv=8, S_k=8192, splits=64) == fa.FA_ERR_NO_DEVICE
    assert splitkv_noalloc_call(B=fit + 1, H=32, H_kv=8, S_k=8192, splits=64) == fa.FA_ERR_TOO_LARGE
    # one split needs no scratch at any size
    assert splitkv_noalloc_call(B=4096, H=32, H_kv=8, S_k=8192, splits=1) == fa.FA_ERR_NO_DEVICE


def test_binding_static_workspace_needs_splits():
    import torch
    q = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="only with num_splits"):
        fa.attention(q, q, q, workspace="static")


def bwd_general_call(**kw):
    """fa_bwd_general with valid arguments except those overridden."""
    a = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, delta=A, B=1, H=8, H_kv=2,
             S_q=5, S_k=300, D=128, scale=0.1, causal=1, cu=None, cu_k=None)
    a.update(kw)
    return fa.load().fa_bwd_general(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"],
                                    a["dq"], a["dk"], a["dv"], a["delta"], a["B"], a["H"],
                                    a["H_kv"], a["S_q"], a["S_k"], a["D"], a["scale"],
                                    a["causal"], a["cu"], a["cu_k"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(S_k=0), fa.FA_ERR_INVALID_ARG),
    (dict(S_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(cu=A), fa.FA_ERR_INVALID_ARG),            # one offset array without the other
    (dict(cu_k=A), fa.FA_ERR_INVALID_ARG),
    (dict(dv=None), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(D=320), fa.FA_ERR_UNSUPPORTED),
    (dict(S_k=1 << 30), fa.FA_ERR_UNSUPPORTED),     # the longer length sets the index bound
])
def test_backward_general_validation_rejects(kw, expect):
    assert bwd_general_call(**kw) == expect


def bwd_hd_call(D, Dv):
    return fa.load().fa_bwd_hd(A, A, A, A, A, A, A, A, A, A, 1, 8, 2, 5, 300, D, Dv, 0.1, 1,
                               None, None, None)


@pytest.mark.parametrize("D,Dv,supported", [
    (64, 64, True), (128, 128, True), (256, 256, True), (192, 128, True),
    (192, 192, False), (128, 64, False), (256, 128, False), (96, 96, False),
])
def test_backward_head_dim_pairs(D, Dv, supported):
    import torch
    rc = bwd_hd_call(D, Dv)
    if not supported:
        assert rc == fa.FA_ERR_UNSUPPORTED
    elif not torch.cuda.is_available():
        assert rc == fa.FA_ERR_NO_DEVICE
    assert bwd_hd_call(D, 0) == fa.FA_ERR_INVALID_ARG


def test_backward_general_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bwd_general_call() == fa.FA_ERR_NO_DEVICE
    assert bwd_general_call(cu=A, cu_k=A, causal=0) == fa.FA_ERR_NO_DEVICE


def test_backward_binding_checks_key_offsets():
    import torch
    q = torch.zeros(8, 1, 64, dtype=torch.bfloat16)
    k = torch.zeros(5, 1, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 8)
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, k, q, lse, q, cu_seqlens=torch.zeros(2, dtype=torch.int32),
                              max_seqlen=8)


def test_output_buffer_checks():
    """Caller-supplied outputs and scratch (out, lse_out, dq/dk/dv, delta) are
    written through raw pointers: a wrong shape, dtype, layout or device is
    rejected before any launch."""
    import torch
    cpu = torch.device("cpu")
    fa._require_buffer(torch.empty((2, 3, 4)), "lse_out", (2, 3, 4), torch.float32, cpu)
    bad = [
        torch.empty((2, 3, 3)),                              # too small
        torch.empty((2, 3, 5)),                              # too large
        torch.empty((2, 3, 4), dtype=torch.bfloat16),        # wrong dtype
        torch.empty((2, 4, 3)).transpose(1, 2),              # right shape, not contiguous
        torch.empty((2, 3, 4), device="meta"),               # another device
    ]
    for t in bad:
        with pytest.raises(ValueError):
            fa._require_buffer(t, "lse_out", (2, 3, 4), torch.float32, cpu)


def test_mfma_ceiling_argument_checks():
    lib = fa.load()
    r = fa.MfmaRate()
    for mode, blocks, reps in ((2, 10, 1), (-1, 10, 1), (0, 0, 1), (0, (1 << 20) + 1, 1),
                               (0, 10, 0), (1, 10, 1001)):
        assert lib.fa_mfma_ceiling(mode, blocks, reps, ctypes.byref(r)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_mfma_ceiling(0, 10, 1, None) == fa.FA_ERR_INVALID_ARG
    import torch
    if not torch.cuda.is_available():
        assert lib.fa_mfma_ceiling(0, 10, 1, ctypes.byref(r)) == fa.FA_ERR_NO_DEVICE
