"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic: it only draws random numbers and
names the workloads.  Both the parity tests and bench.py build Q/K/V here, so
the two sides always see the same bf16 bits.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
standard normals in float32 in the order Q, K, V (shape [B,S,H,D], or
[T,H,D] for packed variable-length batches; K and V have H_kv heads for
grouped-query workloads, and V has Dv columns where the value head
dimension differs); each tensor is multiplied by its standard deviation and
rounded to bfloat16 with round-to-nearest-even.
Variable-length batches draw their lengths first from
``numpy.random.default_rng(seed).integers(lo, hi, n, endpoint=True)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One synthetic attention-forward problem."""
    name: str
    B: int                      # batch size, or number of packed sequences
    S: int                      # sequence length (varlen: the maximum length)
    H: int
    D: int
    causal: bool
    seed: int
    q_std: float = 1.0
    kv_std: float = 1.0
    varlen: Optional[tuple] = None   # (n_seqs, lo, hi) drawn uniformly, inclusive
    lengths: tuple = field(default=())
    Hkv: int = 0                     # K/V heads for grouped-query attention (0: same as H)
    Dv: int = 0                      # value/output head dimension (0: same as D)
    q_range: tuple = field(default=())  # varlen with query lengths of their own: (lo, hi)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def head_dim_v(self) -> int:
        return self.Dv or self.D

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths uniform on [lo, hi] (inclusive), seeded."""
    return np.random.default_rng(seed).integers(lo, hi, n, endpoint=True).astype(np.int64)


def cu_seqlens_of(lengths) -> np.ndarray:
    """int32 prefix sums [0, L0, L0+L1, ...]."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def draw_qkv(shape, seed: int, q_std: float = 1.0, kv_std: float = 1.0, kv_heads=None,
             v_dim=None):
    """Q, K, V as CPU bf16 tensors (drawn in that order).  Q has the given
    shape; K and V too, or kv_heads heads on the head axis (second to last);
    V has v_dim columns when given."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    kv_shape = list(shape)
    if kv_heads is not None:
        kv_shape[-2] = int(kv_heads)
    v_shape = list(kv_shape)
    if v_dim is not None:
        v_shape[-1] = int(v_dim)
    out = []
    for std, shp in ((q_std, shape), (kv_std, kv_shape), (kv_std, v_shape)):
        x = torch.randn(*shp, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def draw_dout(shape, seed: int, std: float = 1.0):
    """The output gradient dO of a backward problem as a CPU bf16 tensor of
    the given shape (o's), N(0, std^2), from its own seeded stream."""
    g = torch.Generator(device="cpu").manual_seed(int(seed) + 7919)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def io_bytes(w: Workload, cu=None) -> float:
    """Bytes the method must move: read Q, K, V, write O (bf16) and LSE (fp32)."""
    Dv = w.head_dim_v
    if w.q_range:
        lq, lk = qk_lengths(w)
        tq, tk = float(np.sum(lq)), float(np.sum(lk))
    elif cu is not None:
        tq = tk = float(cu[-1])
    else:
        tq = tk = float(w.B * w.S)
    return tq * w.H * (2 * w.D + 2 * Dv + 4) + tk * w.kv_heads * 2 * (w.D + Dv)


def qk_lengths(w: Workload):
    """(query lengths, key lengths) of a workload whose queries have lengths of
    their own: key lengths as for varlen, query lengths uniform on q_range
    (inclusive, drawn with seed + 1) and capped at the key length."""
    n, lo, hi = w.varlen
    lens_k = varlen_lengths(n, lo, hi, w.seed)
    qlo, qhi = w.q_range
    lens_q = np.minimum(varlen_lengths(n, qlo, qhi, w.seed + 1), lens_k)
    return lens_q, lens_k


def make_qk(w: Workload):
    """(q, k, v, cu_q, cu_k, Sq, Sk) for a workload with separate query and key
    lengths; Q is drawn with the query token count, K and V with the key's."""
    lens_q, lens_k = qk_lengths(w)
    cu_q, cu_k = cu_seqlens_of(lens_q), cu_seqlens_of(lens_k)
    g = torch.Generator(device="cpu").manual_seed(int(w.seed))
    shapes = ((int(cu_q[-1]), w.H, w.D), (int(cu_k[-1]), w.kv_heads, w.D),
              (int(cu_k[-1]), w.kv_heads, w.head_dim_v))
    out = []
    for std, shp in zip((w.q_std, w.kv_std, w.kv_std), shapes):
        x = torch.randn(*shp, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        out.append(x.to(torch.bfloat16))
    return out[0], out[1], out[2], cu_q, cu_k, int(lens_q.max()), int(lens_k.max())


def make(w: Workload):
    """(q, k, v, cu_seqlens or None, S) for a workload; tensors are CPU bf16."""
    assert not w.q_range, "workloads with their own query lengths use make_qk"
    if w.varlen is not None:
        n, lo, hi = w.varlen
        lens = varlen_lengths(n, lo, hi, w.seed)
        cu = cu_seqlens_of(lens)
        q, k, v = draw_qkv((int(cu[-1]), w.H, w.D), w.seed, w.q_std, w.kv_std, w.kv_heads,
                           w.head_dim_v)
        return q, k, v, cu, int(lens.max())
    if w.lengths:
        cu = cu_seqlens_of(w.lengths)
        q, k, v = draw_qkv((int(cu[-1]), w.H, w.D), w.seed, w.q_std, w.kv_std, w.kv_heads,
                           w.head_dim_v)
        return q, k, v, cu, int(max(w.lengths))
    q, k, v = draw_qkv((w.B, w.S, w.H, w.D), w.seed, w.q_std, w.kv_std, w.kv_heads,
                       w.head_dim_v)
    return q, k, v, None, w.S


def flops(w: Workload, cu=None) -> float:
    """Algorithmic flops: 2*B*H*S^2*(D + Dv) (= 4*B*H*S^2*D for equal head
    dimensions), halved for causal (varlen: sum over sequences).  With query
    lengths of their own: 2*H*(D + Dv)*sum(Lq*Lk), causal keeping Lq*Lk -
    Lq^2/2 per sequence (the bottom-right triangle, the same convention)."""
    dsum = w.D + w.head_dim_v
    if w.q_range:
        lq, lk = (x.astype(np.float64) for x in qk_lengths(w))
        pairs = lq * lk - (lq * lq / 2.0 if w.causal else 0.0)
        return float(np.sum(pairs)) * 2.0 * w.H * dsum
    if cu is not None:
        lens = np.diff(np.asarray(cu, np.int64))
        tot = float(np.sum(lens.astype(np.float64) ** 2)) * 2.0 * w.H * dsum
    else:
        tot = 2.0 * w.B * w.H * float(w.S) ** 2 * dsum
    return tot / 2.0 if w.causal else tot


# The workloads: a tiny non-causal case the oracle finishes instantly; dense
# 2k heads (both masks); 32k causal long context; a packed variable-length
# causal batch; wide heads with high-spread logits; 8k causal (the other
# sequence length the throughput metric names); the install-check shape
# (1, 8, 512, 64) causal from the FlashAttention-4 usage guide; and
# grouped-query attention at 8k causal (32 query heads sharing 8 K/V heads);
# the (192, 128) head dimensions of DeepSeek V3 at 8k causal; and a mixed
# prefill/decode batch whose queries are shorter than their keys.
WORKLOADS = {
    "tiny_b1h2s128d64": Workload("tiny_b1h2s128d64", 1, 128, 2, 64, False, seed=1),
    "dense_b2h16s2048d128": Workload("dense_b2h16s2048d128", 2, 2048, 16, 128, False, seed=2),
    "dense_b2h16s2048d128_causal": Workload("dense_b2h16s2048d128_causal", 2, 2048, 16, 128,
                                            True, seed=2),
    "long_b1h16s32768d128_causal": Workload("long_b1h16s32768d128_causal", 1, 32768, 16, 128,
                                            True, seed=3),
    "varlen_16x512to8192_h32d128_causal": Workload("varlen_16x512to8192_h32d128_causal", 16,
                                                   8192, 32, 128, True, seed=4,
                                                   varlen=(16, 512, 8192)),
    "wide_b2h16s8192d256_spread3": Workload("wide_b2h16s8192d256_spread3", 2, 8192, 16, 256,
                                            False, seed=5, q_std=3.0),
    "causal_b2h16s8192d128": Workload("causal_b2h16s8192d128", 2, 8192, 16, 128, True, seed=6),
    "smoke_b1h8s512d64_causal": Workload("smoke_b1h8s512d64_causal", 1, 512, 8, 64, True, seed=7),
    "gqa_b2h32kv8s8192d128_causal": Workload("gqa_b2h32kv8s8192d128_causal", 2, 8192, 32, 128,
                                             True, seed=8, Hkv=8),
    "hd192v128_b2h16s8192_causal": Workload("hd192v128_b2h16s8192_causal", 2, 8192, 16, 192,
                                            True, seed=9, Dv=128),
    "mixed_16x_q1to2048_k512to8192_h16d128_causal": Workload(
        "mixed_16x_q1to2048_k512to8192_h16d128_causal", 16, 8192, 16, 128, True, seed=10,
        varlen=(16, 512, 8192), q_range=(1, 2048)),
    # A long-context decode step: one sequence, one query row against 32768
    # cached keys, 32 query heads over 8 K/V heads.  It has far fewer query
    # tiles than the GPU has CUs: the shape split-KV is for.
    "decode_1x_q1_k32768_h32kv8d128": Workload(
        "decode_1x_q1_k32768_h32kv8d128", 1, 32768, 32, 128, True, seed=11,
        varlen=(1, 32768, 32768), q_range=(1, 1), Hkv=8),
    # The wide head under a causal mask (the shape of a long-context model
    # with 256-wide heads), N(0, 1).
    "causal_b2h16s8192d256": Workload("causal_b2h16s8192d256", 2, 8192, 16, 256, True, seed=12),
}
