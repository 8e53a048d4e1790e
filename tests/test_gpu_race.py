"""Race check of the forward's hand-synchronised pipeline.

The forward overlaps global->LDS copies of later key blocks with the matrix
products and softmax of the current one: copies are issued from inline asm
that the compiler does not track, waited for with hand-counted
`s_waitcnt vmcnt(N)`, and published with fenceless barriers.  The
race-check build (libfa_mi355x_syncdebug.so, compiled with FA_SYNC_DEBUG)
runs the same kernels with every wait draining every counter, each copy
waited for as soon as it is issued, and a barrier between the ping-pong
phases.  Both builds compute the same values in the same order, so a block
read before its copy landed, or overwritten while another wave still read
it, would make their outputs differ.  Every case below must be bitwise
equal, through the C ABI of each library.

The backward's rings (the dQ kernel's K/V ring, the dK/dV kernels' Q/dO
ring with their LSE and Delta copies) use the same waits and barriers, and
the race-check library holds them too: its dQ, dK, dV and Delta must equal
the pipelined build's bit for bit as well.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
from attn_inputs import WORKLOADS, cu_seqlens_of, draw_dout, draw_qkv, make, make_qk

pytestmark = pytest.mark.gpu


def note(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield fa.load(), fa.load_sync_debug()
    torch.cuda.synchronize()


def run_general(lib, q, k, v, B, H, Hkv, Sq, Sk, D, Dv, causal, cu_q=None, cu_k=None,
                splits=None):
    o = torch.full(tuple(q.shape[:-1]) + (Dv,), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    T = q.shape[0]
    lse_shape = (B, H, Sq) if cu_q is None else (H, T)
    lse = torch.full(lse_shape, float("nan"), dtype=torch.float32, device="cuda")
    cq = cu_q.data_ptr() if cu_q is not None else None
    ck = cu_k.data_ptr() if cu_k is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv,
            Sq, Sk, D, Dv, D ** -0.5, int(causal), cq, ck)
    if splits is None:
        rc = lib.fa_fwd_general(*args, stream, None)
    else:
        need = lib.fa_splitkv_workspace_size(B, H, Sq, Sk, Dv, splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        rc = lib.fa_fwd_splitkv(*args, splits, ws.data_ptr(), ws.numel(), stream)
        torch.cuda.synchronize()
    assert rc == fa.FA_OK, fa.status_string(rc)
    torch.cuda.synchronize()
    return o, lse


def assert_same(libs, what, *args, **kw):
    fast, debug = libs
    o1, l1 = run_general(fast, *args, **kw)
    o2, l2 = run_general(debug, *args, **kw)
    diff = int((o1.view(torch.int16) != o2.view(torch.int16)).sum().item())
    ldiff = int((l1.view(torch.int32) != l2.view(torch.int32)).sum().item())
    note(what, "O elements differing", diff, "LSE rows differing", ldiff, "of", o1.numel(),
         l1.numel())
    assert diff == 0 and ldiff == 0, what


def dense_case(B, S, H, D, Dv, causal, seed, Hkv=None, q_std=1.0):
    q, k, v = draw_qkv((B, S, H, D), seed, q_std=q_std, kv_heads=Hkv, v_dim=Dv)
    return [t.cuda() for t in (q, k, v)]


@pytest.mark.parametrize("name", ["dense_b2h16s2048d128_causal", "causal_b2h16s8192d128",
                                  "dense_b2h16s2048d128", "gqa_b2h32kv8s8192d128_causal",
                                  "causal_b2h16s8192d256"])
def test_race_check_dense_workloads(libs, name):
    w = WORKLOADS[name]
    note("race-check", name)
    q, k, v, _, S = make(w)
    q, k, v = (t.cuda() for t in (q, k, v))
    assert_same(libs, name, q, k, v, w.B, w.H, w.kv_heads, S, S, w.D, w.head_dim_v, w.causal)


@pytest.mark.parametrize("D,Dv,causal,S", [
    (192, 128, True, 2000),     # two-part K layout, 3-slot K ring
    (192, 128, False, 1100),
    (256, 256, False, 2000),    # the pipelined single-wave body
    (256, 256, True, 1500),     # the same body under a causal mask
    (64, 64, True, 1500),
])
def test_race_check_head_dims(libs, D, Dv, causal, S):
    note("race-check D", D, "Dv", Dv, "causal", causal, "S", S)
    q, k, v = dense_case(1, S, 4, D, Dv, causal, seed=400 + D + S)
    assert_same(libs, "D%d/%d causal=%s S=%d" % (D, Dv, causal, S), q, k, v, 1, 4, 4, S, S, D,
                Dv, causal)


@pytest.mark.parametrize("D", [128, 256])   # D = 256 varlen: the serial single-wave body
def test_race_check_small_varlen(libs, D):
    lens = [1, 63, 64, 65, 300, 1000, 2049, 0, 130]
    cu = cu_seqlens_of(lens)
    H = 4
    note("race-check varlen", lens, "D", D)
    q, k, v = draw_qkv((int(cu[-1]), H, D), seed=410)
    dcu = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    q, k, v = (t.cuda() for t in (q, k, v))
    assert_same(libs, "varlen", q, k, v, len(lens), H, H, max(lens), max(lens), D, D, True,
                cu_q=dcu, cu_k=dcu)


def test_race_check_mixed_and_splitkv(libs):
    w = WORKLOADS["mixed_16x_q1to2048_k512to8192_h16d128_causal"]
    note("race-check mixed")
    q, k, v, cu_q, cu_k, Sq, Sk = make_qk(w)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    dcq = torch.from_numpy(cu_q).cuda()
    dck = torch.from_numpy(cu_k).cuda()
    B = len(cu_q) - 1
    assert_same(libs, "mixed", dq, dk, dv, B, w.H, w.kv_heads, Sq, Sk, w.D, w.D, True,
                cu_q=dcq, cu_k=dck)
    assert_same(libs, "mixed split-KV x4", dq, dk, dv, B, w.H, w.kv_heads, Sq, Sk, w.D, w.D,
                True, cu_q=dcq, cu_k=dck, splits=4)


def run_backward(lib, q, k, v, o, lse, g, B, H, Hkv, Sq, Sk, D, Dv, causal, cu_q=None,
                 cu_k=None):
    nan = float("nan")
    dq, dk, dv = (torch.full_like(t, nan) for t in (q, k, v))
    delta = torch.full_like(lse, nan)
    cq = cu_q.data_ptr() if cu_q is not None else None
    ck = cu_k.data_ptr() if cu_k is not None else None
    rc = lib.fa_bwd_hd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       delta.data_ptr(), B, H, Hkv, Sq, Sk, D, Dv, D ** -0.5, int(causal), cq, ck,
                       torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.status_string(rc)
    torch.cuda.synchronize()
    return dq, dk, dv, delta


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# (D, D_v, causal, H, H_kv, query lengths, key lengths); one length each is a
# dense batch of one sequence, several a packed (varlen) batch.
BWD_CASES = [
    (128, 128, True, 4, 2, [2000], [2000]),        # dQ ring; dK/dV D=128 with the score mask
    (128, 128, False, 4, 4, [2048], [2048]),       # dK/dV instance with no masked block
    (128, 128, True, 4, 1, [333, 1, 700, 64, 0], [130, 50, 900, 64, 10]),  # rows without keys
    (64, 64, True, 4, 2, [1500], [1500]),          # masked and mask-free runs
    (64, 64, True, 2, 2, [700, 257, 1024], [300, 257, 1500]),
    (256, 256, True, 2, 2, [1100], [1100]),        # the wide kernels' two-slot rings
    (192, 128, True, 2, 1, [1000], [1000]),
]


def _bwd_id(c):
    D, Dv, causal, H, Hkv, lq, lk = c
    lay = "s%d" % lq[0] if len(lq) == 1 else "varlen%d" % len(lq)
    own = "" if lq == lk else "-ownk"
    return "d%dv%d-%s-h%dkv%d-%s%s" % (D, Dv, "c" if causal else "n", H, Hkv, lay, own)


@pytest.mark.parametrize("case", BWD_CASES, ids=_bwd_id)
def test_race_check_backward(libs, case):
    fast, debug = libs
    D, Dv, causal, H, Hkv, lq, lk = case
    what = "backward " + _bwd_id(case)
    note("race-check", what)
    seed = 420 + D + sum(lq)
    if len(lq) == 1:
        B, Sq, Sk = 1, lq[0], lk[0]
        q, _, _ = draw_qkv((B, Sq, H, D), seed)
        _, k, v = draw_qkv((B, Sk, H, D), seed + 1, kv_heads=Hkv, v_dim=Dv)
        dcq = dck = None
    else:
        B, Sq, Sk = len(lq), max(lq), max(lk)
        cq, ck = cu_seqlens_of(lq), cu_seqlens_of(lk)
        q, _, _ = draw_qkv((int(cq[-1]), H, D), seed)
        _, k, v = draw_qkv((int(ck[-1]), H, D), seed + 1, kv_heads=Hkv, v_dim=Dv)
        dcq = torch.from_numpy(np.asarray(cq, np.int32)).cuda()
        dck = torch.from_numpy(np.asarray(ck, np.int32)).cuda()
    q, k, v = (t.cuda() for t in (q, k, v))
    o, lse = run_general(fast, q, k, v, B, H, Hkv, Sq, Sk, D, Dv, causal, cu_q=dcq, cu_k=dck)
    g = draw_dout(tuple(o.shape), seed + 2).cuda()
    r1 = run_backward(fast, q, k, v, o, lse, g, B, H, Hkv, Sq, Sk, D, Dv, causal, dcq, dck)
    r2 = run_backward(debug, q, k, v, o, lse, g, B, H, Hkv, Sq, Sk, D, Dv, causal, dcq, dck)
    for name, a, b in zip(("dq", "dk", "dv", "delta"), r1, r2):
        diff = int((bits(a) != bits(b)).sum().item())
        note(what, name, "elements differing", diff, "of", a.numel())
        assert diff == 0, (what, name)
        # the buffers start as NaN: every element must have been written
        assert not torch.isnan(a.float()).any(), (what, name, "unwritten elements")


@pytest.mark.parametrize("name", ["causal_b2h16s8192d128", "gqa_b2h32kv8s8192d128_causal"])
def test_race_check_backward_workloads(libs, name):
    """The 8k backward workloads: every CU runs many key and query tiles."""
    fast, debug = libs
    w = WORKLOADS[name]
    what = "backward " + name
    note("race-check", what)
    q, k, v, _, S = make(w)
    q, k, v = (t.cuda() for t in (q, k, v))
    o, lse = run_general(fast, q, k, v, w.B, w.H, w.kv_heads, S, S, w.D, w.D, w.causal)
    g = draw_dout(tuple(o.shape), 430).cuda()
    args = (w.B, w.H, w.kv_heads, S, S, w.D, w.D, w.causal)
    r1 = run_backward(fast, q, k, v, o, lse, g, *args)
    r2 = run_backward(debug, q, k, v, o, lse, g, *args)
    for name_, a, b in zip(("dq", "dk", "dv", "delta"), r1, r2):
        diff = int((bits(a) != bits(b)).sum().item())
        note(what, name_, "elements differing", diff, "of", a.numel())
        assert diff == 0, (what, name_)
        assert not torch.isnan(a.float()).any(), (what, name_, "unwritten elements")
