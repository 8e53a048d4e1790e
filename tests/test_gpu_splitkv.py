"""GPU parity of split-KV attention (fa_fwd_splitkv, through the C ABI)
against the fp64 oracle.

Decode-like shapes (one or a few query rows against long key ranges), dense
and variable-length, with grouped K/V heads and the (192, 128) head
dimensions; split counts that leave some splits without keys (short
sequences, causal rows); rows that may use no key at all.  The gate is the
forward's (parity.py); rows without keys must be exactly O = 0, LSE = -inf.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
import oracle
from attn_inputs import WORKLOADS, cu_seqlens_of, draw_qkv, make_qk
from parity import assert_close, compare, tensor_to_f64

pytestmark = pytest.mark.gpu


def note(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield
    torch.cuda.synchronize()


def split_check(q, k, v, causal, scale, splits, cu_q=None, cu_k=None, Sq=None, Sk=None, what=""):
    note(what, "q", tuple(q.shape), "k", tuple(k.shape), "causal", causal, "splits", splits)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    kw = {}
    if cu_q is not None:
        kw = dict(cu_seqlens=torch.from_numpy(np.asarray(cu_q, np.int32)).cuda(), max_seqlen=Sq,
                  cu_seqlens_k=torch.from_numpy(np.asarray(cu_k, np.int32)).cuda(),
                  max_seqlen_k=Sk)
    o, lse = fa.attention(dq, dk, dv, causal=causal, scale=scale, num_splits=splits, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_bf16(q, k, v, scale, causal, cu_q, cu_k)
    lse_g = tensor_to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_g), empty), what
    o_g = tensor_to_f64(o)
    if empty.any():
        rows_o = o_g.transpose(0, 2, 1, 3)[empty] if cu_q is None else o_g.transpose(1, 0, 2)[empty]
        assert np.all(rows_o == 0.0), what
    st = compare(o_g, np.where(empty, 0.0, lse_g), o_ref, np.where(empty, 0.0, lse_ref))
    note(what, st, "empty rows", int(empty.sum()))
    assert_close(st, what)
    return o, lse


SPLIT_DENSE = [
    # (B, Sq, Sk, H, H_kv, D, D_v, splits)
    (2, 1, 1000, 4, 2, 128, 128, 4),
    (2, 1, 4097, 4, 1, 128, 128, 16),     # MQA decode, ragged last block
    (1, 5, 2049, 4, 4, 64, 64, 7),
    (1, 300, 300, 2, 2, 128, 128, 3),     # prefill: causal splits past a row's last key are empty
    (1, 700, 300, 2, 2, 128, 128, 2),     # more queries than keys: rows without keys
    (1, 2, 1500, 2, 2, 192, 128, 5),
    (1, 1, 640, 2, 2, 256, 256, 64),      # more splits requested than key blocks
    # query heads of a K/V group packed into one tile (S_q * H/H_kv <= 256):
    (1, 60, 900, 8, 2, 128, 128, 3),      # 240 packed rows over 8 waves, per-row causal limits
    (2, 7, 530, 8, 1, 64, 64, 5),         # MQA, D = 64
    (1, 3, 800, 4, 2, 192, 128, 4),       # (192, 128) head dimensions
    (1, 1, 700, 4, 2, 256, 256, 3),       # D = 256
    # a full 256-row tile and a ragged one over 8 splits
    (1, 300, 2000, 2, 2, 128, 128, 8),
]


@pytest.mark.parametrize("shape", SPLIT_DENSE, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_dense(shape, causal):
    B, Sq, Sk, H, Hkv, D, Dv, splits = shape
    q, _, _ = draw_qkv((B, Sq, H, D), seed=201 + Sq)
    _, k, v = draw_qkv((B, Sk, H, D), seed=202 + Sk, kv_heads=Hkv, v_dim=Dv)
    split_check(q, k, v, causal, D ** -0.5, splits, what="split-dense")


@pytest.mark.parametrize("splits", [4, 0])
def test_splitkv_varlen_decode(splits):
    """A packed decode batch: 1-3 query rows per sequence, keys from 1 to 2500
    (some sequences shorter than one split, one shorter than one block)."""
    lq, lk = [1, 1, 3, 1, 2], [700, 64, 2500, 1, 1300]
    cu_q, cu_k = cu_seqlens_of(lq), cu_seqlens_of(lk)
    H, Hkv, D = 4, 2, 128
    q, _, _ = draw_qkv((int(cu_q[-1]), H, D), seed=203)
    _, k, v = draw_qkv((int(cu_k[-1]), H, D), seed=204, kv_heads=Hkv)
    split_check(q, k, v, True, D ** -0.5, splits, cu_q, cu_k, max(lq), max(lk),
                what="split-varlen")


def test_splitkv_matches_one_split():
    """Splitting changes only the rounding: the split result stays within the
    gate of the unsplit one, and one split is the unsplit path exactly."""
    B, Sq, Sk, H, D = 2, 1, 3000, 8, 128
    q, _, _ = draw_qkv((B, Sq, H, D), seed=205)
    _, k, v = draw_qkv((B, Sk, H, D), seed=206)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o1, l1 = fa.attention(dq, dk, dv, causal=True)
    o8, l8 = fa.attention(dq, dk, dv, causal=True, num_splits=8)
    os_, ls_ = fa.attention(dq, dk, dv, causal=True, num_splits=1)
    torch.cuda.synchronize()
    st = compare(tensor_to_f64(o8), tensor_to_f64(l8), tensor_to_f64(o1), tensor_to_f64(l1))
    note("split-vs-one", st)
    assert st["o_max"] <= 1e-2 and st["lse_max"] <= 1e-5
    assert torch.equal(o1.view(torch.int16), os_.view(torch.int16))
    assert torch.equal(l1, ls_)


def test_splitkv_mixed_workload_sampled():
    """The mixed prefill/decode workload through split-KV (auto count),
    sampled rows against the oracle."""
    w = WORKLOADS["mixed_16x_q1to2048_k512to8192_h16d128_causal"]
    q, k, v, cu_q, cu_k, Sq, Sk = make_qk(w)
    dcu_q = torch.from_numpy(cu_q).cuda()
    dcu_k = torch.from_numpy(cu_k).cuda()
    note("split-mixed gpu run")
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=w.scale,
                          cu_seqlens=dcu_q, max_seqlen=Sq, cu_seqlens_k=dcu_k, max_seqlen_k=Sk,
                          num_splits=0)
    torch.cuda.synchronize()
    T = int(cu_q[-1])
    rng = np.random.default_rng(207)
    rows = np.unique(np.concatenate([rng.integers(0, T * w.H, 300), [0, T * w.H - 1]]))
    o_ref, lse_ref = oracle.attention_rows_bf16(q, k, v, rows, w.scale, True, cu_q, cu_k)
    o_g = tensor_to_f64(o)       # [T, H, D]
    l_g = tensor_to_f64(lse)     # [H, T]
    h, t = rows // T, rows % T
    st = compare(o_g[t, h], l_g[h, t], o_ref, lse_ref)
    note("split-mixed", st)
    assert_close(st, "split-mixed")


def test_splitkv_long_context_decode_auto():
    """The long-context decode workload (one row per head against 32768
    keys) through the automatic split count, every output against the oracle."""
    w = WORKLOADS["decode_1x_q1_k32768_h32kv8d128"]
    q, k, v, cu_q, cu_k, Sq, Sk = make_qk(w)
    split_check(q, k, v, True, w.scale, 0, cu_q, cu_k, Sq, Sk, what="split-decode-32k")


def test_splitkv_workspace_needs_no_clearing():
    """The workspace's contents on entry do not matter: a workspace full of
    stale bytes (all ones, then what a previous call left) gives the same
    result call after call."""
    B, Sq, Sk, H, Hkv, D = 2, 1, 3000, 8, 2, 128
    q, _, _ = draw_qkv((B, Sq, H, D), seed=211)
    _, k, v = draw_qkv((B, Sk, H, D), seed=212, kv_heads=Hkv)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    splits = 6
    need = fa.splitkv_workspace_size(B, H, Sq, Sk, D, splits)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        o, lse = fa.attention(dq, dk, dv, causal=True, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse, outs[0][1])
    o_ref, lse_ref = oracle.attention_bf16(q, k, v, D ** -0.5, True)
    st = compare(tensor_to_f64(outs[0][0]), tensor_to_f64(outs[0][1]), o_ref, lse_ref)
    note("split-stale-workspace", st)
    assert_close(st, "split-stale-workspace")
