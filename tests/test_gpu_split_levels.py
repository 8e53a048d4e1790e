"""GPU parity of dense causal launches with split levels.

The persistent kernel runs the costliest m-blocks of a dense causal batch
with few tiles as two parts over the two halves of their key blocks; the
part that finishes second merges both partial results.  Each case is
compared with the fp64 oracle element by element (the gate of parity.py),
with the unsplit launch of the same inputs, and across repeated launches,
whose results must be identical whichever part arrived second.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
import oracle
from attn_inputs import WORKLOADS, draw_qkv, make
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


def tuning(levels):
    t = fa.default_tuning()
    t.split_levels = levels
    return t


def run(q, k, v, scale, levels, stream=None, return_lse=True):
    o, lse = fa.attention(q, k, v, causal=True, scale=scale, tuning=tuning(levels),
                          stream=stream, return_lse=return_lse)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, S, H, D, D_v, split levels): ragged tails, every head dimension
    # that splits (D = 256 never does), some and all m-blocks split
    (1, 1500, 4, 128, 128, -1),   # the library's own choice (one level)
    (1, 1000, 2, 64, 64, 3),
    (1, 1500, 4, 128, 128, 6),
    (2, 1100, 2, 192, 128, 5),
    (1, 300, 2, 128, 128, 2),
    (1, 65, 1, 128, 128, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dH%dD%dv%d_n%d" % c)
def test_split_levels_full_parity(case):
    B, S, H, D, Dv, levels = case
    workers = fa.num_workers(D)
    n = fa.split_plan(B, H, S, D, workers, levels)
    assert n > 0, "the case must exercise split levels"
    note("split levels", case, "plan", n)
    q, k, v = draw_qkv((B, S, H, D), seed=600 + S + D, v_dim=Dv)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    o, lse = run(dq, dk, dv, scale, levels)
    o_ref, lse_ref = oracle.attention_bf16(q, k, v, scale, True)
    st = compare(tensor_to_f64(o), tensor_to_f64(lse), o_ref, lse_ref)
    note("split levels", case, st)
    assert_close(st, "split levels %s" % (case,))
    # the unsplit launch: the same values up to the merge's fp32 rounding
    o0, l0 = run(dq, dk, dv, scale, 0)
    st0 = compare(tensor_to_f64(o), tensor_to_f64(lse), tensor_to_f64(o0), tensor_to_f64(l0))
    note("split vs unsplit", st0)
    assert st0["o_max"] <= 1e-2 and st0["lse_max"] <= 1e-5


def test_split_levels_repeat_is_bitwise_stable():
    """Launches that follow each other (the arrival counters must be back at
    zero after each), with another shape in between and on another stream
    (a workspace of its own), give identical bits."""
    q, k, v = (t.cuda() for t in draw_qkv((2, 2048, 16, 128), seed=611))
    q2, k2, v2 = (t.cuda() for t in draw_qkv((1, 900, 3, 128), seed=612))
    scale = 1.0 / math.sqrt(128)
    first = run(q, k, v, scale, 4)
    outs = []
    for i in range(3):
        run(q2, k2, v2, scale, 2)
        outs.append(run(q, k, v, scale, 4))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o_s, l_s = fa.attention(q, k, v, causal=True, scale=scale, stream=side, tuning=tuning(4))
    side.synchronize()
    outs.append((o_s, l_s))
    outs.append(run(q, k, v, scale, 4, return_lse=False))
    for i, (o, lse) in enumerate(outs):
        note("repeat", i)
        assert torch.equal(o.view(torch.int16), first[0].view(torch.int16)), i
        if lse is not None:
            assert torch.equal(lse, first[1]), i


def test_split_levels_2k_causal_config_sampled():
    """The dense 2k causal workload (B=2, H=16, D=128) with every level split
    (a request: by default it fills the workers and runs whole): sampled rows
    against the oracle, every output against the unsplit launch."""
    w = WORKLOADS["dense_b2h16s2048d128_causal"]
    q, k, v, _, S = make(w)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o, lse = run(dq, dk, dv, w.scale, 8)
    o0, l0 = run(dq, dk, dv, w.scale, 0)
    st0 = compare(tensor_to_f64(o), tensor_to_f64(lse), tensor_to_f64(o0), tensor_to_f64(l0))
    note("2k causal split vs unsplit", st0)
    assert st0["o_max"] <= 1e-2 and st0["lse_max"] <= 1e-5
    # rows in the oracle's numbering (b*H + h)*S + i: every head's first and
    # last rows and a seeded random sample
    rng = np.random.default_rng(613)
    heads = np.arange(w.B * w.H) * S
    rows = np.unique(np.concatenate([heads, heads + S - 1, heads + 1000,
                                     rng.choice(w.B * w.H * S, 256, replace=False)]))
    o_ref, lse_ref = oracle.attention_rows_bf16(q, k, v, rows, w.scale, True)
    b, h, i = rows // (w.H * S), (rows // S) % w.H, rows % S
    o_g = tensor_to_f64(o)[b, i, h]
    l_g = tensor_to_f64(lse)[b, h, i]
    st = compare(o_g, l_g, o_ref, lse_ref)
    note("2k causal split sampled", st)
    assert_close(st, "2k causal split, sampled rows")
