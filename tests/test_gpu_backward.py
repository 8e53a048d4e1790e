"""GPU parity of the backward pass: fa_bwd (through the C ABI) against the
fp64 oracle's gradients.

The forward runs on the GPU first (its o and lse are fa_bwd's inputs, as in
training); dO is drawn from its own seeded stream.  Small shapes are
compared element by element on every gradient (several row and key tiles,
ragged tails, both masks, D = 64, 128, 256 and (192, 128), grouped K/V heads, packed
variable-length batches); the 8k causal shape is compared on sampled query
and key rows.  The gate, derived from the arithmetic, is in parity.py.
Run-to-run reproducibility is checked bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
import oracle
from attn_inputs import WORKLOADS, cu_seqlens_of, draw_dout, draw_qkv
from parity import assert_grad_close, compare_grad, tensor_to_f64

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


def gpu_grads(q, k, v, g, causal, scale, cu=None, S=None):
    """Forward then backward on the GPU; returns CPU (dq, dk, dv) tensors."""
    dq_, dk_, dv_, dg = (t.cuda() for t in (q, k, v, g))
    dcu = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    o, lse = fa.attention(dq_, dk_, dv_, causal=causal, scale=scale, cu_seqlens=dcu,
                          max_seqlen=S)
    grads = fa.attention_backward(dq_, dk_, dv_, o, lse, dg, causal=causal, scale=scale,
                                  cu_seqlens=dcu, max_seqlen=S)
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in grads)


def full_bwd_check(q, k, v, g, causal, scale, cu=None, S=None, what=""):
    note(what, "q", tuple(q.shape), "k", tuple(k.shape), "causal", causal)
    got = gpu_grads(q, k, v, g, causal, scale, cu, S)
    ref = oracle.attention_backward(q, k, v, g, scale, causal, cu, magnitudes=True)
    for name, gg, rr, mm in zip(("dq", "dk", "dv"), got, ref[:3], ref[3:]):
        st = compare_grad(tensor_to_f64(gg), rr, mm)
        note(what, name, st)
        assert_grad_close(st, (what, name))
    return got


# ---- full element-by-element parity on shapes the oracle finishes quickly
# S = 333: one and a half 256-row query tiles, two or three key tiles, five
# 64-row blocks and a ragged tail of 13 rows.
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small(D, causal):
    B, S, H = 2, 333, 3
    q, k, v = draw_qkv((B, S, H, D), seed=101 + D)
    g = draw_dout((B, S, H, D), seed=101 + D)
    full_bwd_check(q, k, v, g, causal, D ** -0.5, what="bwd-small D%d" % D)


# S = 512: whole 64-row blocks, so a dense non-causal D = 128 launch takes the
# dK/dV instance without the entry mask, and D = 64 runs every block of a key
# tile through the mask-free body; causal, each wave's diagonal blocks sit
# between mask-free runs, over two query heads per K/V head.
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_whole_blocks(D, causal):
    B, S, H, H_kv = 1, 512, 4, 2
    q, k, v = draw_qkv((B, S, H, D), seed=131 + D, kv_heads=H_kv)
    g = draw_dout((B, S, H, D), seed=132 + D)
    full_bwd_check(q, k, v, g, causal, D ** -0.5, what="bwd-whole-blocks D%d" % D)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_short_sequences(D):
    """S below one block (and a single row): tails only."""
    for S in (1, 37):
        q, k, v = draw_qkv((1, S, 2, D), seed=103 + S)
        g = draw_dout((1, S, 2, D), seed=103 + S)
        full_bwd_check(q, k, v, g, True, D ** -0.5, what="bwd-short S%d" % S)


@pytest.mark.parametrize("H_kv", [1, 2])
def test_backward_grouped_kv_heads(H_kv):
    """GQA / MQA: dK and dV sum the contributions of every query head of the group."""
    B, S, H, D = 2, 300, 4, 128
    q, k, v = draw_qkv((B, S, H, D), seed=105, kv_heads=H_kv)
    g = draw_dout((B, S, H, D), seed=105)
    full_bwd_check(q, k, v, g, True, D ** -0.5, what="bwd-gqa Hkv%d" % H_kv)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_varlen(D):
    lengths = [1, 64, 200, 333, 65, 129]
    cu = cu_seqlens_of(lengths)
    T, H = int(cu[-1]), 2
    q, k, v = draw_qkv((T, H, D), seed=107)
    g = draw_dout((T, H, D), seed=107)
    full_bwd_check(q, k, v, g, True, D ** -0.5, cu=cu, S=max(lengths), what="bwd-varlen D%d" % D)


def test_backward_spread_logits():
    """Q with std 3: peaked rows (few keys carry the weight), non-causal."""
    B, S, H, D = 1, 260, 2, 128
    q, k, v = draw_qkv((B, S, H, D), seed=109, q_std=3.0)
    g = draw_dout((B, S, H, D), seed=109)
    full_bwd_check(q, k, v, g, False, D ** -0.5, what="bwd-spread")


def test_backward_is_reproducible():
    """Every gradient row is reduced by one workgroup in a fixed order: two
    runs give identical bits."""
    B, S, H, D = 1, 700, 4, 128
    q, k, v = draw_qkv((B, S, H, D), seed=111, kv_heads=2)
    g = draw_dout((B, S, H, D), seed=111)
    a = gpu_grads(q, k, v, g, True, D ** -0.5)
    b = gpu_grads(q, k, v, g, True, D ** -0.5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_autograd_function_matches_backward_entry():
    """attention_fn(...).backward(dO) runs the same kernels as attention_backward."""
    B, S, H, D = 1, 200, 2, 64
    q, k, v = draw_qkv((B, S, H, D), seed=113)
    g = draw_dout((B, S, H, D), seed=113)
    ref = gpu_grads(q, k, v, g, True, None)
    tq, tk, tv = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = fa.attention_fn(tq, tk, tv, causal=True)
    o.backward(g.cuda())
    torch.cuda.synchronize()
    for x, y in zip((tq.grad, tk.grad, tv.grad), ref):
        assert torch.equal(x.cpu().view(torch.int16), y.view(torch.int16))


def test_backward_8k_causal_sampled():
    """B=2, H=16, S=8192, D=128, causal (the 8k causal forward workload):
    query rows and key rows sampled from one (sequence, head) slice and the
    edges of others, compared with the oracle row by row."""
    w = WORKLOADS["causal_b2h16s8192d128"]
    B, S, H, D = w.B, w.S, w.H, w.D
    q, k, v = draw_qkv((B, S, H, D), seed=w.seed)
    g = draw_dout((B, S, H, D), seed=w.seed)
    note("bwd-8k gpu run")
    dq, dk, dv = gpu_grads(q, k, v, g, True, w.scale)
    rng = np.random.default_rng(115)
    # key rows of slice (b=1, h=5): first, last, block edges and random
    b, h = 1, 5
    js = sorted(set([0, 1, 63, 64, 127, 128, 255, 256, S - 1, S - 64]
                    + list(rng.integers(0, S, 24))))
    k_rows = [(b * H + h) * S + j for j in js]
    # query rows of the same slice plus a few in other slices
    is_ = sorted(set([0, 1, 255, 256, S - 1] + list(rng.integers(0, S, 24))))
    q_rows = [(b * H + h) * S + i for i in is_] + [(0 * H + 0) * S + 0, (0 * H + 15) * S + S - 1]
    note("bwd-8k oracle rows", len(q_rows), len(k_rows))
    rdq, rdqm, rdk, rdv, rdkm, rdvm = oracle.attention_backward_rows_bf16(
        q, k, v, g, q_rows, k_rows, w.scale, True)
    gdq = tensor_to_f64(dq)
    gdk, gdv = tensor_to_f64(dk), tensor_to_f64(dv)
    sel_q = np.stack([gdq[r // (H * S), r % S, (r // S) % H] for r in q_rows])
    sel_k = np.stack([gdk[b, j, h] for j in js])
    sel_v = np.stack([gdv[b, j, h] for j in js])
    for name, gg, rr, mm in (("dq", sel_q, rdq, rdqm), ("dk", sel_k, rdk, rdkm),
                             ("dv", sel_v, rdv, rdvm)):
        st = compare_grad(gg, rr, mm)
        note("bwd-8k", name, st)
        assert_grad_close(st, ("bwd-8k", name))


def test_backward_largest_tensors_sampled():
    """1040 sequences of 1024 tokens, 8 query heads on one K/V head, causal:
    Q, O, dO and dQ hold 2.18e9 bytes, and the rows at the end of the last
    sequence sit past 2^31 bytes from the tensor start.  Gradient rows are
    gathered on the device and compared with the oracle row by row."""
    B, S, H, Hkv, D = 1040, 1024, 8, 1, 128
    scale = D ** -0.5
    q, k, v = draw_qkv((B, S, H, D), seed=141, kv_heads=Hkv)
    g = draw_dout((B, S, H, D), seed=141)
    note("bwd-largest gpu run")
    dq_, dk_, dv_, dg = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(dq_, dk_, dv_, causal=True, scale=scale)
    dq, dk, dv = fa.attention_backward(dq_, dk_, dv_, o, lse, dg, causal=True, scale=scale)
    torch.cuda.synchronize()
    last = B - 1
    q_idx = [(last, H - 1, i) for i in (0, 1, 511, S - 2, S - 1)] + \
            [(last, 3, 700), (0, 0, 0), (517, 2, 33)]
    k_idx = [(last, j) for j in (0, 63, 64, 700, S - 1)] + [(3, 10)]
    q_rows = [(b * H + h) * S + i for b, h, i in q_idx]
    k_rows = [(b * Hkv) * S + j for b, j in k_idx]
    note("bwd-largest oracle rows", len(q_rows), len(k_rows))
    rdq, rdqm, rdk, rdv, rdkm, rdvm = oracle.attention_backward_rows_bf16(
        q, k, v, g, q_rows, k_rows, scale, True)

    def take(x, idx):
        cols = [torch.as_tensor(c, device=x.device) for c in zip(*idx)]
        return tensor_to_f64(x[tuple(cols)])
    sel_q = take(dq, [(b, i, h) for b, h, i in q_idx])
    sel_k = take(dk, [(b, j, 0) for b, j in k_idx])
    sel_v = take(dv, [(b, j, 0) for b, j in k_idx])
    for name, gg, rr, mm in (("dq", sel_q, rdq, rdqm), ("dk", sel_k, rdk, rdkm),
                             ("dv", sel_v, rdv, rdvm)):
        st = compare_grad(gg, rr, mm)
        note("bwd-largest", name, st)
        assert_grad_close(st, ("bwd-largest", name))


# ---- query and key lengths that differ (fa_bwd_general; bottom-right causal)
def gpu_grads_general(q, k, v, g, causal, scale, cu=None, cu_k=None, S=None, S_k=None):
    dq_, dk_, dv_, dg = (t.cuda() for t in (q, k, v, g))
    dcu = dcu_k = None
    if cu is not None:
        dcu = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
        dcu_k = torch.from_numpy(np.asarray(cu_k, np.int32)).cuda()
    o, lse = fa.attention(dq_, dk_, dv_, causal=causal, scale=scale, cu_seqlens=dcu,
                          max_seqlen=S, cu_seqlens_k=dcu_k, max_seqlen_k=S_k)
    grads = fa.attention_backward(dq_, dk_, dv_, o, lse, dg, causal=causal, scale=scale,
                                  cu_seqlens=dcu, max_seqlen=S, cu_seqlens_k=dcu_k,
                                  max_seqlen_k=S_k)
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in grads)


def full_bwd_check_general(q, k, v, g, causal, scale, cu=None, cu_k=None, S=None, S_k=None,
                           what=""):
    note(what, "q", tuple(q.shape), "k", tuple(k.shape), "causal", causal, "cu", cu, "cu_k", cu_k)
    got = gpu_grads_general(q, k, v, g, causal, scale, cu, cu_k, S, S_k)
    ref = oracle.attention_backward(q, k, v, g, scale, causal, cu, cu_k, magnitudes=True)
    for name, gg, rr, mm in zip(("dq", "dk", "dv"), got, ref[:3], ref[3:]):
        st = compare_grad(tensor_to_f64(gg), rr, mm)
        note(what, name, st)
        assert_grad_close(st, (what, name))
    return got


# (S_q, S_k): fewer queries than keys (chunked prefill), one query (decode),
# more queries than keys (causal rows without keys), and tails of each
QK_BWD = [(100, 333), (1, 300), (333, 130), (64, 64 + 257)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", QK_BWD, ids=lambda s: "q%dk%d" % s)
def test_backward_qk_lengths_dense(lens, causal, D):
    S_q, S_k = lens
    B, H, H_kv = 2, 4, 2
    q, _, _ = draw_qkv((B, S_q, H, D), seed=111 + S_q + D)
    _, k, v = draw_qkv((B, S_k, H, D), seed=112 + S_k + D, kv_heads=H_kv)
    g = draw_dout((B, S_q, H, D), seed=113 + S_q)
    got = full_bwd_check_general(q, k, v, g, causal, D ** -0.5,
                                 what="bwd-qk q%d k%d D%d" % (S_q, S_k, D))
    if causal and S_q > S_k:
        assert torch.all(got[0][:, :S_q - S_k].float() == 0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_qk_lengths_varlen(causal, D):
    """Packed sequences with key lengths of their own, including a sequence
    without queries, one without keys and one-query (decode) rows."""
    lq = [5, 0, 130, 1, 70, 9]
    lk = [40, 17, 66, 300, 0, 9]
    cu, cu_k = cu_seqlens_of(lq), cu_seqlens_of(lk)
    H, H_kv = 4, 1
    q, _, _ = draw_qkv((int(cu[-1]), H, D), seed=121 + D)
    _, k, v = draw_qkv((int(cu_k[-1]), H, D), seed=122 + D, kv_heads=H_kv)
    g = draw_dout((int(cu[-1]), H, D), seed=123 + D)
    got = full_bwd_check_general(q, k, v, g, causal, D ** -0.5, cu=cu, cu_k=cu_k, S=max(lq),
                                 S_k=max(lk), what="bwd-qk-varlen D%d" % D)
    # the sequence without keys: zero query gradient
    a = int(cu[4])
    assert torch.all(got[0][a:a + lq[4]].float() == 0)
    # keys of the sequence without queries: zero key and value gradients
    c = int(cu_k[1])
    assert torch.all(got[1][c:c + lk[1]].float() == 0)
    assert torch.all(got[2][c:c + lk[1]].float() == 0)


def test_backward_general_equal_lengths_is_fa_bwd():
    """fa_bwd_general with S_q = S_k and the same offsets is fa_bwd, bit for bit."""
    D, S, H = 128, 333, 2
    q, k, v = draw_qkv((1, S, H, D), seed=131)
    g = draw_dout((1, S, H, D), seed=131)
    dq_, dk_, dv_, dg = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(dq_, dk_, dv_, causal=True)
    lib = fa.load()
    outs = []
    for general in (False, True):
        dq, dk, dv = (torch.empty_like(t) for t in (dq_, dk_, dv_))
        delta = torch.empty_like(lse)
        ptrs = [t.data_ptr() for t in (dq_, dk_, dv_, o, dg, lse, dq, dk, dv, delta)]
        stream = torch.cuda.current_stream().cuda_stream
        if general:
            rc = lib.fa_bwd_general(*ptrs, 1, H, H, S, S, D, D ** -0.5, 1, None, None, stream)
        else:
            rc = lib.fa_bwd(*ptrs, 1, H, H, S, D, D ** -0.5, 1, None, stream)
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((dq.cpu(), dk.cpu(), dv.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_autograd_function_with_key_offsets():
    """attention_fn with key offsets of their own runs fa_bwd_general: the
    same bits as attention_backward on the same call."""
    D, H = 64, 2
    lq, lk = [3, 90, 1], [50, 40, 129]
    cu, cu_k = cu_seqlens_of(lq), cu_seqlens_of(lk)
    q, _, _ = draw_qkv((int(cu[-1]), H, D), seed=141)
    _, k, v = draw_qkv((int(cu_k[-1]), H, D), seed=142)
    g = draw_dout((int(cu[-1]), H, D), seed=143)
    ref = gpu_grads_general(q, k, v, g, True, None, cu, cu_k, max(lq), max(lk))
    dcu = torch.from_numpy(cu).cuda()
    dcu_k = torch.from_numpy(cu_k).cuda()
    tq, tk, tv = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = fa.attention_fn(tq, tk, tv, causal=True, cu_seqlens=dcu, max_seqlen=max(lq),
                        cu_seqlens_k=dcu_k, max_seqlen_k=max(lk))
    o.backward(g.cuda())
    torch.cuda.synchronize()
    for x, y in zip((tq.grad, tk.grad, tv.grad), ref):
        assert torch.equal(x.cpu().view(torch.int16), y.view(torch.int16))


def test_backward_chunked_prefill_sampled():
    """A chunked-prefill batch at full size: B=2, H=16 query heads over 4 K/V
    heads, 1024 queries against 8192 keys, D=128, causal (bottom-right: the
    chunk's queries follow 7168 earlier keys).  Query rows and key rows
    around the diagonal's start, block edges and random ones, compared with
    the oracle row by row."""
    B, H, H_kv, S_q, S_k, D = 2, 16, 4, 1024, 8192, 128
    scale = D ** -0.5
    q, _, _ = draw_qkv((B, S_q, H, D), seed=151)
    _, k, v = draw_qkv((B, S_k, H, D), seed=152, kv_heads=H_kv)
    g = draw_dout((B, S_q, H, D), seed=153)
    note("bwd-chunk gpu run")
    dq, dk, dv = gpu_grads_general(q, k, v, g, True, scale)
    rng = np.random.default_rng(155)
    off = S_k - S_q
    b, hk = 1, 2
    js = sorted(set([0, 63, 64, off - 1, off, off + 1, off + 255, off + 256, S_k - 64, S_k - 1]
                    + list(rng.integers(0, S_k, 20))))
    k_rows = [(b * H_kv + hk) * S_k + j for j in js]
    h = hk * (H // H_kv) + 1
    is_ = sorted(set([0, 1, 255, 256, S_q - 1] + list(rng.integers(0, S_q, 20))))
    q_rows = [(b * H + h) * S_q + i for i in is_] + [(0 * H + 0) * S_q + 0,
                                                      (0 * H + 15) * S_q + S_q - 1]
    note("bwd-chunk oracle rows", len(q_rows), len(k_rows))
    rdq, rdqm, rdk, rdv, rdkm, rdvm = oracle.attention_backward_rows_bf16(
        q, k, v, g, q_rows, k_rows, scale, True)
    gdq = tensor_to_f64(dq)
    gdk, gdv = tensor_to_f64(dk), tensor_to_f64(dv)
    sel_q = np.stack([gdq[r // (H * S_q), r % S_q, (r // S_q) % H] for r in q_rows])
    sel_k = np.stack([gdk[b, j, hk] for j in js])
    sel_v = np.stack([gdv[b, j, hk] for j in js])
    for name, gg, rr, mm in (("dq", sel_q, rdq, rdqm), ("dk", sel_k, rdk, rdkm),
                             ("dv", sel_v, rdv, rdvm)):
        st = compare_grad(gg, rr, mm)
        note("bwd-chunk", name, st)
        assert_grad_close(st, ("bwd-chunk", name))


# ---- wide heads: D = 256 and the (192, 128) pair (one wave per SIMD, dK/dV
# columns split over two workgroups at D = 256)
WIDE = [(256, 256), (192, 128)]


def _wide_id(d):
    return "D%dDv%d" % d


@pytest.mark.parametrize("dims", WIDE, ids=_wide_id)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_wide_small(dims, causal):
    """S = 333: three 128-row query and key tiles, six 64-row blocks, a
    ragged tail of 13 rows."""
    D, Dv = dims
    B, S, H = 2, 333, 2
    q, k, v = draw_qkv((B, S, H, D), seed=141 + D, v_dim=Dv)
    g = draw_dout((B, S, H, Dv), seed=141 + D)
    full_bwd_check(q, k, v, g, causal, D ** -0.5, what="bwd-wide D%d/%d" % dims)


@pytest.mark.parametrize("dims", WIDE, ids=_wide_id)
def test_backward_wide_short_and_grouped(dims):
    """Sequences below one block, and grouped K/V heads (MQA)."""
    D, Dv = dims
    for S in (1, 37):
        q, k, v = draw_qkv((1, S, 2, D), seed=143 + S, v_dim=Dv)
        g = draw_dout((1, S, 2, Dv), seed=143 + S)
        full_bwd_check(q, k, v, g, True, D ** -0.5, what="bwd-wide-short S%d" % S)
    q, k, v = draw_qkv((1, 200, 4, D), seed=145, kv_heads=1, v_dim=Dv)
    g = draw_dout((1, 200, 4, Dv), seed=145)
    full_bwd_check(q, k, v, g, True, D ** -0.5, what="bwd-wide-mqa D%d" % D)


@pytest.mark.parametrize("dims", WIDE, ids=_wide_id)
def test_backward_wide_varlen_and_lengths(dims):
    """A packed batch, then query and key lengths of their own (a sequence
    without queries, one without keys, one-query rows)."""
    D, Dv = dims
    lengths = [1, 64, 200, 333, 65, 129]
    cu = cu_seqlens_of(lengths)
    q, k, v = draw_qkv((int(cu[-1]), 2, D), seed=147, v_dim=Dv)
    g = draw_dout((int(cu[-1]), 2, Dv), seed=147)
    full_bwd_check(q, k, v, g, True, D ** -0.5, cu=cu, S=max(lengths),
                   what="bwd-wide-varlen D%d" % D)
    lq = [5, 0, 130, 1, 70, 9]
    lk = [40, 17, 66, 300, 0, 9]
    cu_q, cu_k = cu_seqlens_of(lq), cu_seqlens_of(lk)
    q, _, _ = draw_qkv((int(cu_q[-1]), 4, D), seed=149)
    _, k, v = draw_qkv((int(cu_k[-1]), 4, D), seed=150, kv_heads=2, v_dim=Dv)
    g = draw_dout((int(cu_q[-1]), 4, Dv), seed=151)
    got = full_bwd_check_general(q, k, v, g, True, D ** -0.5, cu=cu_q, cu_k=cu_k, S=max(lq),
                                 S_k=max(lk), what="bwd-wide-qk-varlen D%d" % D)
    a = int(cu_q[4])
    assert torch.all(got[0][a:a + lq[4]].float() == 0)
    c = int(cu_k[1])
    assert torch.all(got[1][c:c + lk[1]].float() == 0)
    assert torch.all(got[2][c:c + lk[1]].float() == 0)


@pytest.mark.parametrize("dims", WIDE, ids=_wide_id)
def test_backward_wide_dense_lengths_and_reproducible(dims):
    """Fewer queries than keys (chunked prefill), bottom-right causal; two
    runs give identical bits."""
    D, Dv = dims
    q, _, _ = draw_qkv((2, 100, 4, D), seed=153)
    _, k, v = draw_qkv((2, 333, 4, D), seed=154, kv_heads=2, v_dim=Dv)
    g = draw_dout((2, 100, 4, Dv), seed=155)
    a = full_bwd_check_general(q, k, v, g, True, D ** -0.5, what="bwd-wide-qk D%d" % D)
    b = gpu_grads_general(q, k, v, g, True, D ** -0.5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
