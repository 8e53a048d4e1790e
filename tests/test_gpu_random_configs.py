"""GPU parity over seeded random configurations (forward and backward).

The other parity tests pick their shapes by hand; this one draws 96
configurations from a fixed seed, across every axis the entry points take
together: head dimensions (64, 128, 256 and the (192, 128) pair), the mask,
dense or packed (varlen) batches, key lengths of their own (bottom-right
causal), grouped K/V heads, the tuning knobs (tau, the exp2 split, the
schedule, split levels) and split-KV.  Lengths stay small (at most 600 rows
per sequence), so the oracle compares every output, and every gradient of
the configurations that also run the backward.  Rows that may use no key
must be exactly O = 0 and LSE = -inf.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
import oracle
from attn_inputs import cu_seqlens_of, draw_dout, draw_qkv
from parity import (assert_close, assert_grad_close, compare, compare_grad, tensor_to_f64)

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (256, 256), (192, 128)]


def _configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D, Dv = DIMS[i % len(DIMS)]
        causal = bool(rng.integers(2))
        G = int(rng.choice([1, 1, 2, 4]))
        Hkv = int(rng.choice([1, 2]))
        H = G * Hkv
        varlen = bool(rng.integers(2))
        own_k = bool(rng.integers(3) == 0)
        if varlen:
            n_seq = int(rng.integers(1, 6))
            lq = [int(x) for x in rng.integers(0, 601, n_seq)]
            if max(lq) == 0:
                lq[0] = 1
            lk = [int(x) for x in rng.integers(0, 601, n_seq)] if own_k else list(lq)
            if max(lk) == 0:
                lk[0] = 1
            shape = dict(lq=lq, lk=lk)
        else:
            B = int(rng.integers(1, 4))
            Sq = int(rng.integers(1, 601))
            Sk = int(rng.integers(1, 601)) if own_k else Sq
            shape = dict(B=B, Sq=Sq, Sk=Sk)
        mode = str(rng.choice(["default", "tuning", "splitkv"]))
        tun = None
        if mode == "tuning":
            tun = dict(tau=float(rng.choice([0.0, 8.0])), exp2_emu=int(rng.choice([0, 4, 8])),
                       schedule=int(rng.integers(2)), split_levels=int(rng.choice([-1, 0, 3])))
        splits = int(rng.choice([2, 3, 8])) if mode == "splitkv" else None
        backward = bool(rng.integers(2))
        out.append(dict(idx=i, D=D, Dv=Dv, causal=causal, H=H, Hkv=Hkv, varlen=varlen,
                        own_k=own_k, tuning=tun, splits=splits, backward=backward, **shape))
    return out


CONFIGS = _configs(96, seed=20261203)


def _id(c):
    lay = ("varlen%s" % "-".join(map(str, c["lq"]))) if c["varlen"] else \
        "b%ds%dk%d" % (c["B"], c["Sq"], c["Sk"])
    extra = "split%d" % c["splits"] if c["splits"] else ("tun" if c["tuning"] else "")
    return "%02d-d%dv%d-%s-h%dkv%d-%s%s%s" % (c["idx"], c["D"], c["Dv"], "c" if c["causal"] else "n",
                                            c["H"], c["Hkv"], lay, "-" + extra if extra else "",
                                            "-bwd" if c["backward"] else "")


def note(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("c", CONFIGS, ids=_id)
def test_random_config(c):
    note(_id(c))
    D, Dv, H, Hkv = c["D"], c["Dv"], c["H"], c["Hkv"]
    scale = D ** -0.5
    seed = 900 + c["idx"]
    if c["varlen"]:
        cu, cu_k = cu_seqlens_of(c["lq"]), cu_seqlens_of(c["lk"])
        Tq, Tk = int(cu[-1]), int(cu_k[-1])
        q, _, _ = draw_qkv((Tq, H, D), seed=seed)
        _, k, v = draw_qkv((Tk, H, D), seed=seed + 1, kv_heads=Hkv, v_dim=Dv)
        S, S_k = max(c["lq"]), max(c["lk"])
        dcu = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
        # shared lengths: no key offsets (the self-attention varlen path)
        dcu_k = torch.from_numpy(np.asarray(cu_k, np.int32)).cuda() if c["own_k"] else None
        ocu, ocu_k = cu, (cu_k if c["own_k"] else None)
    else:
        q, _, _ = draw_qkv((c["B"], c["Sq"], H, D), seed=seed)
        _, k, v = draw_qkv((c["B"], c["Sk"], H, D), seed=seed + 1, kv_heads=Hkv, v_dim=Dv)
        S, S_k = c["Sq"], c["Sk"]
        dcu = dcu_k = None
        ocu = ocu_k = None
    kw = dict(causal=c["causal"], scale=scale, cu_seqlens=dcu, cu_seqlens_k=dcu_k)
    if c["varlen"]:
        kw.update(max_seqlen=S, max_seqlen_k=S_k if c["own_k"] else None)
    if c["tuning"]:
        t = fa.default_tuning()
        for name, val in c["tuning"].items():
            setattr(t, name, val)
        kw["tuning"] = t
    if c["splits"]:
        kw["num_splits"] = c["splits"]
    dq_, dk_, dv_ = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.attention(dq_, dk_, dv_, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_bf16(q, k, v, scale, c["causal"], ocu, ocu_k)
    o_g, lse_g = tensor_to_f64(o), tensor_to_f64(lse)
    # rows that may use no key (causal, more queries than keys): exactly
    # O = 0 and LSE = -inf; the other rows go through the gate
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_g), empty), _id(c)
    if empty.any():
        rows_o = o_g.transpose(1, 0, 2)[empty] if c["varlen"] else o_g.transpose(0, 2, 1, 3)[empty]
        assert np.all(rows_o == 0.0), _id(c)
    st = compare(o_g, np.where(empty, 0.0, lse_g), o_ref, np.where(empty, 0.0, lse_ref))
    note(_id(c), st, "empty rows", int(empty.sum()))
    assert_close(st, _id(c))
    if not c["backward"]:
        return
    g = draw_dout(tuple(o.shape), seed=seed + 2)
    bkw = dict(causal=c["causal"], scale=scale, cu_seqlens=dcu, cu_seqlens_k=dcu_k)
    if c["varlen"]:
        bkw.update(max_seqlen=S, max_seqlen_k=S_k if c["own_k"] else None)
    grads = fa.attention_backward(dq_, dk_, dv_, o, lse, g.cuda(), **bkw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, g, scale, c["causal"], ocu, ocu_k, magnitudes=True)
    for name, gg, rr, mm in zip(("dq", "dk", "dv"), grads, ref[:3], ref[3:]):
        stg = compare_grad(tensor_to_f64(gg), rr, mm)
        note(_id(c), name, stg)
        assert_grad_close(stg, (_id(c), name))
