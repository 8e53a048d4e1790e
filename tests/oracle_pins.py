"""Checks that pin the fp64 oracle to facts it does not compute itself.

Each check takes an ``OracleLib``-like object (``attention_f64`` method) and
raises AssertionError when the oracle disagrees with what the definition of
attention fixes.  The checks come from closed forms, invariances and an
independent 50-digit brute force; none re-types the oracle's own formula.
They are used on the real oracle (test_oracle_pins.py) and on deliberately
broken copies of it (test_oracle_mutants.py), which every one of these
mistakes must trip.
"""
from __future__ import annotations

import numpy as np

from oracle import brute


def _bf16_grid(rng, shape, std=1.0):
    """Random values that are exactly representable in bf16 (8-bit mantissa)."""
    x = rng.standard_normal(shape) * std
    m, e = np.frexp(x)
    m = np.round(m * 256.0) / 256.0
    return np.ldexp(m, e)


def check_brute_force_tiny(o):
    """Two-pass oracle == 50-digit exp-without-max-subtraction on tiny inputs."""
    rng = np.random.default_rng(11)
    for causal in (False, True):
        B, S, H, D = 2, 7, 2, 5
        q, k, v = (_bf16_grid(rng, (B, S, H, D)) for _ in range(3))
        scale = 0.37
        got_o, got_l = o.attention_f64(q, k, v, scale, causal)
        ref_o, ref_l = brute.attention(q, k, v, scale, causal)
        assert np.max(np.abs(got_o - ref_o)) <= 1e-12, ("brute O", causal)
        assert np.max(np.abs(got_l - ref_l)) <= 1e-12, ("brute LSE", causal)
    # packed variable-length batch, causal
    cu = [0, 3, 9, 10]
    q, k, v = (_bf16_grid(rng, (10, 2, 4)) for _ in range(3))
    got_o, got_l = o.attention_f64(q, k, v, 0.5, True, cu)
    ref_o, ref_l = brute.attention(q, k, v, 0.5, True, cu)
    assert np.max(np.abs(got_o - ref_o)) <= 1e-12, "brute varlen O"
    assert np.max(np.abs(got_l - ref_l)) <= 1e-12, "brute varlen LSE"


def check_equal_logits_mean_of_v(o):
    """Q = 0 makes every logit equal: O_i is the mean of the allowed V rows
    and LSE_i = ln(number of allowed keys)."""
    rng = np.random.default_rng(12)
    B, S, H, D = 2, 9, 3, 6
    q = np.zeros((B, S, H, D))
    k, v = rng.standard_normal((B, S, H, D)), rng.standard_normal((B, S, H, D))
    for causal in (False, True):
        got_o, got_l = o.attention_f64(q, k, v, 0.3, causal)
        for i in range(S):
            n = i + 1 if causal else S
            mean = v[:, :n].mean(axis=1)
            assert np.allclose(got_o[:, i], mean, rtol=0, atol=1e-13), ("mean of V", causal, i)
            assert np.allclose(got_l[:, :, i], np.log(n), rtol=0, atol=1e-13), ("ln n", causal, i)


def check_dominant_logit_selects_row(o):
    """One logit 60 above all others: O_i = v_{j*} (to e^-60) and LSE_i = 60."""
    rng = np.random.default_rng(13)
    S, D, scale = 12, 12, 0.25
    for causal in (False, True):
        target = np.array([rng.integers(0, (i + 1) if causal else S) for i in range(S)])
        q = np.zeros((1, S, 1, D))
        k = np.zeros((1, S, 1, D))
        for i in range(S):
            q[0, i, 0, target[i]] = 1.0          # query i points at key target[i]
        for j in range(S):
            k[0, j, 0, j] = 60.0 / scale          # key j answers only direction j
        v = rng.standard_normal((1, S, 1, D))
        got_o, got_l = o.attention_f64(q, k, v, scale, causal)
        for i in range(S):
            assert np.allclose(got_o[0, i, 0], v[0, target[i], 0], rtol=0, atol=1e-20), \
                ("dominant O", causal, i)
            assert abs(got_l[0, 0, i] - 60.0) <= 1e-12, ("dominant LSE", causal, i)


def check_causal_row0(o):
    """Causal row 0 sees only key 0: O_0 = v_0 exactly, LSE_0 = scale*q_0.k_0."""
    rng = np.random.default_rng(14)
    B, S, H, D = 2, 8, 2, 7
    q, k, v = (_bf16_grid(rng, (B, S, H, D)) for _ in range(3))
    got_o, got_l = o.attention_f64(q, k, v, 0.21, True)
    assert np.array_equal(got_o[:, 0], v[:, 0]), "causal row 0 O"
    s00 = 0.21 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    assert np.allclose(got_l[:, :, 0], s00, rtol=0, atol=1e-14), "causal row 0 LSE"


def check_kv_permutation_invariance(o):
    """Non-causal attention does not depend on the order of the (k_j, v_j) pairs."""
    rng = np.random.default_rng(15)
    B, S, H, D = 2, 11, 2, 6
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    perm = rng.permutation(S)
    o1, l1 = o.attention_f64(q, k, v, 0.4, False)
    o2, l2 = o.attention_f64(q, k[:, perm], v[:, perm], 0.4, False)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13), "permutation O"
    assert np.allclose(l1, l2, rtol=0, atol=1e-13), "permutation LSE"
    # and it does depend on pairing: permuting V alone changes O
    o3, _ = o.attention_f64(q, k, v[:, perm], 0.4, False)
    assert not np.allclose(o1, o3, rtol=0, atol=1e-6), "pairing of K and V rows"


def check_key_shift(o):
    """k_j += u for all j: O unchanged, LSE_i += scale * q_i . u."""
    rng = np.random.default_rng(16)
    B, S, H, D = 1, 10, 2, 5
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    u = rng.standard_normal((H, D))
    for causal in (False, True):
        o1, l1 = o.attention_f64(q, k, v, 0.5, causal)
        o2, l2 = o.attention_f64(q, k + u[None, None], v, 0.5, causal)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12), ("shift O", causal)
        shift = 0.5 * np.einsum("bshd,hd->bhs", q, u)
        assert np.allclose(l2 - l1, shift, rtol=0, atol=1e-12), ("shift LSE", causal)


def check_affine_v(o):
    """V -> V A + 1 b^T maps O -> O A + 1 b^T (softmax rows sum to one)."""
    rng = np.random.default_rng(17)
    B, S, H, D = 2, 9, 1, 4
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    A = rng.standard_normal((D, D))
    bvec = rng.standard_normal(D)
    for causal in (False, True):
        o1, l1 = o.attention_f64(q, k, v, 0.7, causal)
        o2, l2 = o.attention_f64(q, k, v @ A + bvec, 0.7, causal)
        assert np.allclose(o2, o1 @ A + bvec, rtol=0, atol=1e-12), ("affine O", causal)
        assert np.allclose(l1, l2, rtol=0, atol=0), ("affine LSE", causal)


def check_causal_prefix(o):
    """Causal row i equals non-causal attention over the first i+1 keys."""
    rng = np.random.default_rng(18)
    B, S, H, D = 1, 9, 2, 5
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    oc, lc = o.attention_f64(q, k, v, 0.45, True)
    for i in range(S):
        on, ln = o.attention_f64(q[:, :i + 1], k[:, :i + 1], v[:, :i + 1], 0.45, False)
        assert np.allclose(oc[:, i], on[:, i], rtol=0, atol=1e-13), ("prefix O", i)
        assert np.allclose(lc[:, :, i], ln[:, :, i], rtol=0, atol=1e-13), ("prefix LSE", i)


def check_varlen_equals_dense_runs(o):
    """A packed batch equals each sequence run on its own."""
    rng = np.random.default_rng(19)
    lens = [5, 1, 8, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, D = 2, 4
    q, k, v = (rng.standard_normal((cu[-1], H, D)) for _ in range(3))
    for causal in (False, True):
        op, lp = o.attention_f64(q, k, v, 0.6, causal, cu)
        for b, L in enumerate(lens):
            sl = slice(cu[b], cu[b + 1])
            od, ld = o.attention_f64(q[None, sl], k[None, sl], v[None, sl], 0.6, causal)
            assert np.array_equal(op[sl], od[0]), ("varlen O", causal, b)
            assert np.array_equal(lp[:, sl], ld[0]), ("varlen LSE", causal, b)


def check_scale_is_a_logit_multiplier(o):
    """attention(Q, scale=a) == attention(a*Q, scale=1) for a power of two a."""
    rng = np.random.default_rng(20)
    B, S, H, D = 1, 6, 2, 3
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    o1, l1 = o.attention_f64(q, k, v, 0.125, True)
    o2, l2 = o.attention_f64(q * 0.125, k, v, 1.0, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "scale"


def check_gqa_brute_force_tiny(o):
    """Grouped-query attention (Hkv < H) == the 50-digit brute force, dense and varlen."""
    rng = np.random.default_rng(21)
    for causal in (False, True):
        B, S, H, Hkv, D = 1, 6, 4, 2, 3
        q = _bf16_grid(rng, (B, S, H, D))
        k, v = (_bf16_grid(rng, (B, S, Hkv, D)) for _ in range(2))
        got_o, got_l = o.attention_f64(q, k, v, 0.41, causal)
        ref_o, ref_l = brute.attention(q, k, v, 0.41, causal)
        assert np.max(np.abs(got_o - ref_o)) <= 1e-12, ("gqa brute O", causal)
        assert np.max(np.abs(got_l - ref_l)) <= 1e-12, ("gqa brute LSE", causal)
    cu = [0, 4, 5, 9]                 # multi-query (one K/V head), varlen, causal
    q = _bf16_grid(rng, (9, 3, 4))
    k, v = (_bf16_grid(rng, (9, 1, 4)) for _ in range(2))
    got_o, got_l = o.attention_f64(q, k, v, 0.5, True, cu)
    ref_o, ref_l = brute.attention(q, k, v, 0.5, True, cu)
    assert np.max(np.abs(got_o - ref_o)) <= 1e-12, "mqa brute varlen O"
    assert np.max(np.abs(got_l - ref_l)) <= 1e-12, "mqa brute varlen LSE"


def check_gqa_equals_repeated_kv(o):
    """Sharing a K/V head among H/Hkv consecutive query heads is the same as
    multi-head attention on K and V with each head repeated H/Hkv times in a
    row: the multi-head path gives the identical result, bit for bit."""
    rng = np.random.default_rng(22)
    B, S, H, D = 2, 7, 6, 4
    q = rng.standard_normal((B, S, H, D))
    for Hkv in (1, 2, 3):
        k, v = (rng.standard_normal((B, S, Hkv, D)) for _ in range(2))
        kr, vr = (np.repeat(x, H // Hkv, axis=2) for x in (k, v))
        for causal in (False, True):
            o1, l1 = o.attention_f64(q, k, v, 0.3, causal)
            o2, l2 = o.attention_f64(q, kr, vr, 0.3, causal)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), ("gqa repeat", Hkv, causal)


def check_value_dim_brute_force_tiny(o):
    """A value head dimension Dv different from the q/k one == the 50-digit brute force."""
    rng = np.random.default_rng(23)
    for causal in (False, True):
        B, S, H, Hkv, D, Dv = 1, 6, 2, 1, 5, 3
        q = _bf16_grid(rng, (B, S, H, D))
        k = _bf16_grid(rng, (B, S, Hkv, D))
        v = _bf16_grid(rng, (B, S, Hkv, Dv))
        got_o, got_l = o.attention_f64(q, k, v, 0.45, causal)
        ref_o, ref_l = brute.attention(q, k, v, 0.45, causal)
        assert got_o.shape == (B, S, H, Dv)
        assert np.max(np.abs(got_o - ref_o)) <= 1e-12, ("dv brute O", causal)
        assert np.max(np.abs(got_l - ref_l)) <= 1e-12, ("dv brute LSE", causal)


def check_value_columns_are_independent(o):
    """Each output column depends only on the same column of V: attention on V
    equals the first Dv columns of attention on V padded with extra columns,
    and the LSE ignores V entirely (bit for bit in both cases)."""
    rng = np.random.default_rng(24)
    B, S, H, D, Dv = 2, 7, 2, 6, 3
    q, k = (rng.standard_normal((B, S, H, D)) for _ in range(2))
    v = rng.standard_normal((B, S, H, Dv))
    vpad = np.concatenate([v, rng.standard_normal((B, S, H, 5))], axis=-1)
    for causal in (False, True):
        o1, l1 = o.attention_f64(q, k, v, 0.2, causal)
        o2, l2 = o.attention_f64(q, k, vpad, 0.2, causal)
        assert np.array_equal(o1, o2[..., :Dv]) and np.array_equal(l1, l2), ("dv columns", causal)


def check_qk_lengths_brute_force_tiny(o):
    """Query and key lengths that differ (bottom-right causal alignment,
    rows with no key) == the 50-digit brute force, dense and varlen."""
    rng = np.random.default_rng(25)
    for (Sq, Sk) in ((3, 7), (7, 4)):
        for causal in (False, True):
            q = _bf16_grid(rng, (2, Sq, 2, 3))
            k, v = (_bf16_grid(rng, (2, Sk, 1, 3)) for _ in range(2))
            got_o, got_l = o.attention_f64(q, k, v, 0.6, causal)
            ref_o, ref_l = brute.attention(q, k, v, 0.6, causal)
            assert np.max(np.abs(got_o - ref_o)) <= 1e-12, ("qk brute O", Sq, Sk, causal)
            assert np.array_equal(np.isinf(got_l), np.isinf(ref_l)), ("qk brute empty", Sq, Sk)
            fin = np.isfinite(ref_l)
            assert np.max(np.abs(got_l[fin] - ref_l[fin])) <= 1e-12, ("qk brute LSE", Sq, Sk)
    cu_q, cu_k = [0, 2, 5, 6, 6], [0, 4, 5, 9, 11]
    q = _bf16_grid(rng, (6, 2, 4))
    k, v = (_bf16_grid(rng, (11, 2, 4)) for _ in range(2))
    for causal in (False, True):
        got_o, got_l = o.attention_f64(q, k, v, 0.5, causal, cu_q, cu_k)
        ref_o, ref_l = brute.attention(q, k, v, 0.5, causal, cu_q, cu_k)
        assert np.max(np.abs(got_o - ref_o)) <= 1e-12, ("qk brute varlen O", causal)
        fin = np.isfinite(ref_l)
        assert np.array_equal(fin, np.isfinite(got_l)), "qk brute varlen empty"
        assert np.max(np.abs(got_l[fin] - ref_l[fin])) <= 1e-12, ("qk brute varlen LSE", causal)


def check_short_queries_are_the_last_rows_of_self_attention(o):
    """Lq queries against Lk >= Lq keys (bottom-right causal) are exactly the
    last Lq rows of self-attention over Lk queries that end with them (the
    earlier queries are arbitrary), bit for bit; non-causal likewise."""
    rng = np.random.default_rng(26)
    Lk, Lq, H, D = 9, 3, 2, 4
    k, v = (rng.standard_normal((1, Lk, H, D)) for _ in range(2))
    qfull = rng.standard_normal((1, Lk, H, D))
    for causal in (False, True):
        o1, l1 = o.attention_f64(qfull[:, Lk - Lq:], k, v, 0.4, causal)
        o2, l2 = o.attention_f64(qfull, k, v, 0.4, causal)
        assert np.array_equal(o1, o2[:, Lk - Lq:]), ("suffix O", causal)
        assert np.array_equal(l1, l2[:, :, Lk - Lq:]), ("suffix LSE", causal)


def check_rows_without_keys(o):
    """Causal with more queries than keys: the first Lq - Lk rows may use no
    key and are O = 0, LSE = -inf exactly; the others attend normally."""
    rng = np.random.default_rng(27)
    Lq, Lk = 6, 2
    q = rng.standard_normal((1, Lq, 1, 3))
    k, v = (rng.standard_normal((1, Lk, 1, 3)) for _ in range(2))
    got_o, got_l = o.attention_f64(q, k, v, 0.5, True)
    assert np.all(got_o[0, :Lq - Lk] == 0.0) and np.all(got_l[0, 0, :Lq - Lk] == -np.inf)
    assert np.all(np.isfinite(got_l[0, 0, Lq - Lk:]))
    # row Lq-Lk sees exactly key 0: its output is v_0
    assert np.array_equal(got_o[0, Lq - Lk, 0], v[0, 0, 0]), "first non-empty row"


# ---------------------------------------------------------------------------
# Backward pass: gradients of F = sum <dO, O> with respect to Q, K and V.
# ---------------------------------------------------------------------------

def _objective(o, q, k, v, g, scale, causal, cu=None, cu_k=None):
    out, _ = o.attention_f64(q, k, v, scale, causal, cu, cu_k)
    return float(np.sum(out * g))


def _bwd_cases(rng):
    """(name, q, k, v, dout, scale, causal, cu_q, cu_k) covering MHA, GQA,
    D != Dv, varlen and query/key lengths that differ."""
    cases = []
    for causal in (False, True):
        B, S, H, D = 2, 6, 2, 4
        q, k, v, g = (rng.standard_normal((B, S, H, D)) for _ in range(4))
        cases.append(("mha", q, k, v, g, 0.45, causal, None, None))
    q = rng.standard_normal((1, 5, 4, 3))
    k, v = rng.standard_normal((1, 5, 2, 3)), rng.standard_normal((1, 5, 2, 2))
    cases.append(("gqa_dv", q, k, v, rng.standard_normal((1, 5, 4, 2)), 0.6, True, None, None))
    cu = [0, 3, 7, 8]
    q, k, v, g = (rng.standard_normal((8, 2, 3)) for _ in range(4))
    cases.append(("varlen", q, k, v, g, 0.5, True, cu, None))
    q, g = rng.standard_normal((1, 3, 1, 3)), rng.standard_normal((1, 3, 1, 3))
    k, v = rng.standard_normal((1, 5, 1, 3)), rng.standard_normal((1, 5, 1, 3))
    cases.append(("qk_lengths", q, k, v, g, 0.7, True, None, None))
    # varlen with key offsets of their own (every row keeps at least one key)
    cu_q, cu_k = [0, 2, 5, 9], [0, 4, 8, 13]
    q, g = rng.standard_normal((9, 2, 3)), rng.standard_normal((9, 2, 3))
    k, v = rng.standard_normal((13, 1, 3)), rng.standard_normal((13, 1, 3))
    cases.append(("qk_lengths_varlen", q, k, v, g, 0.55, True, cu_q, cu_k))
    # more queries than keys, causal: the first two rows may use no key
    q, g = rng.standard_normal((1, 5, 2, 3)), rng.standard_normal((1, 5, 2, 3))
    k, v = rng.standard_normal((1, 3, 2, 3)), rng.standard_normal((1, 3, 2, 3))
    cases.append(("nokey_rows", q, k, v, g, 0.65, True, None, None))
    return cases


def check_bwd_finite_differences(o):
    """<dF/dX, U> of the backward equals the central difference of the
    forward oracle along a random direction U, for X = Q, K, V (fp64:
    the difference quotient is exact to O(eps^2))."""
    rng = np.random.default_rng(31)
    eps = 1e-5
    for name, q, k, v, g, scale, causal, cu, cu_k in _bwd_cases(rng):
        grads = o.attention_backward(q, k, v, g, scale, causal, cu, cu_k)
        for idx, x in enumerate((q, k, v)):
            u = rng.standard_normal(x.shape)
            args = [q, k, v]
            args[idx] = x + eps * u
            fp = _objective(o, *args, g, scale, causal, cu, cu_k)
            args[idx] = x - eps * u
            fm = _objective(o, *args, g, scale, causal, cu, cu_k)
            fd = (fp - fm) / (2 * eps)
            an = float(np.sum(grads[idx] * u))
            assert abs(fd - an) <= 1e-7 * (1 + abs(fd)), (name, "dq dk dv".split()[idx], fd, an)


def check_bwd_torch_autograd(o):
    """The backward equals torch's float64 autograd through a masked softmax
    (a library differentiation of the textbook formula), with grouped K/V
    heads expanded by repetition and the causal mask bottom-right aligned."""
    import torch
    rng = np.random.default_rng(32)
    for name, q, k, v, g, scale, causal, cu, cu_k in _bwd_cases(rng):
        if name.startswith("nokey"):
            continue  # torch's softmax of an all-masked row is NaN; pinned below
        got = o.attention_backward(q, k, v, g, scale, causal, cu, cu_k)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        tg = torch.tensor(g, dtype=torch.float64)
        if cu is None:
            segs = [(tq, tk, tv, tg)]
        else:
            ck = cu if cu_k is None else cu_k
            segs = [(tq[None, a:b], tk[None, c:d], tv[None, c:d], tg[None, a:b])
                    for a, b, c, d in zip(cu[:-1], cu[1:], ck[:-1], ck[1:])]
        total = 0
        for sq, sk, sv, sg in segs:
            G = sq.shape[2] // sk.shape[2]
            kk = sk.repeat_interleave(G, dim=2)
            vv = sv.repeat_interleave(G, dim=2)
            logits = torch.einsum("bihd,bjhd->bhij", sq, kk) * scale
            Lq, Lk = sq.shape[1], sk.shape[1]
            if causal:
                ii = torch.arange(Lq)[:, None]
                jj = torch.arange(Lk)[None, :]
                logits = logits.masked_fill(jj > ii + (Lk - Lq), -float("inf"))
            p = torch.softmax(logits, dim=-1)
            out = torch.einsum("bhij,bjhd->bihd", p, vv)
            total = total + (out * sg).sum()
        total.backward()
        for got_x, ref_x, nm in zip(got, (tq.grad, tk.grad, tv.grad), ("dq", "dk", "dv")):
            assert np.max(np.abs(got_x - ref_x.numpy())) <= 1e-12, (name, nm)


def check_bwd_rows_without_keys(o):
    """Rows that may use no key (causal, more queries than keys) get a zero
    query gradient and add nothing to dK and dV: the backward of the same
    batch without those rows gives the same key gradients."""
    rng = np.random.default_rng(33)
    q, g = rng.standard_normal((1, 6, 2, 4)), rng.standard_normal((1, 6, 2, 4))
    k, v = rng.standard_normal((1, 4, 2, 4)), rng.standard_normal((1, 4, 2, 4))
    dq, dk, dv = o.attention_backward(q, k, v, g, 0.5, True)
    assert np.all(dq[0, :2] == 0.0)
    assert np.any(dq[0, 2:] != 0.0)
    dq2, dk2, dv2 = o.attention_backward(q[:, 2:], k, v, g[:, 2:], 0.5, True)
    assert np.max(np.abs(dq[0, 2:] - dq2[0])) <= 1e-12
    assert np.max(np.abs(dk - dk2)) <= 1e-12 and np.max(np.abs(dv - dv2)) <= 1e-12


def check_bwd_single_key(o):
    """With one key every probability is 1: O_i = v_0 whatever Q and K are,
    so dQ = dK = 0 and dV_0 = sum_i dO_i."""
    rng = np.random.default_rng(33)
    q, g = rng.standard_normal((2, 1, 3, 4)), rng.standard_normal((2, 1, 3, 4))
    k, v = rng.standard_normal((2, 1, 3, 4)), rng.standard_normal((2, 1, 3, 4))
    for causal in (False, True):
        dq, dk, dv = o.attention_backward(q, k, v, g, 0.5, causal)
        assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15, causal
        assert np.allclose(dv, g, rtol=0, atol=1e-15), causal


def check_bwd_uniform_probabilities(o):
    """Q = 0 makes every allowed probability 1/n_i: then dK = 0,
    dV_j = sum over the rows i that use j of dO_i / n_i, and
    dQ_i = scale * (mean_j <dO_i, v_j> k_j - mean_j <dO_i, v_j> * mean_j k_j),
    the covariance form of the softmax Jacobian at equal logits."""
    rng = np.random.default_rng(34)
    B, S, H, D = 1, 5, 1, 3
    q = np.zeros((B, S, H, D))
    k, v, g = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    scale = 0.8
    for causal in (False, True):
        dq, dk, dv, dqm, dkm, dvm = o.attention_backward(q, k, v, g, scale, causal,
                                                         magnitudes=True)
        assert np.max(np.abs(dk)) <= 1e-14, causal
        for j in range(S):
            rows = [i for i in range(S) if not causal or j <= i]
            n = [(i + 1) if causal else S for i in rows]
            ref = sum(g[0, i, 0] / ni for i, ni in zip(rows, n))
            ref_mag = sum(np.abs(g[0, i, 0]) / ni for i, ni in zip(rows, n))
            assert np.allclose(dv[0, j, 0], ref, rtol=0, atol=1e-14), ("dv", causal, j)
            assert np.allclose(dvm[0, j, 0], ref_mag, rtol=0, atol=1e-14), ("|dv|", causal, j)
        for i in range(S):
            n = i + 1 if causal else S
            kk, vv = k[0, :n, 0], v[0, :n, 0]
            dp = vv @ g[0, i, 0]
            ref = scale * ((dp[:, None] * kk).mean(0) - dp.mean() * kk.mean(0))
            assert np.allclose(dq[0, i, 0], ref, rtol=0, atol=1e-14), ("dq", causal, i)
        for got, mag in ((dq, dqm), (dk, dkm), (dv, dvm)):
            assert np.all(np.abs(got) <= mag + 1e-15), "a gradient exceeds its magnitude"


def check_bwd_magnitudes_single_key(o):
    """The magnitude A that bounds each gradient element is the sum of the
    absolute values of its terms, where the term of key j in dQ_i (and of row
    i in dK_j) is scale * (|dS_ij| + P_ij * E_i) * |k_jd| (|q_id|), E_i being
    the bound sum_d |dO_id| |O_id| of |Delta_i|.  With one key P = 1 and
    dS = 0, and O_i = v_0, so in closed form
    |dQ|_id = scale * E_i * |k_0d| and |dK|_0d = scale * sum_i E_i |q_id|,
    with E_i = sum_d |dO_id| |v_0d|."""
    rng = np.random.default_rng(36)
    B, S, H, D = 2, 1, 3, 4
    q, k, v, g = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    scale = 0.6
    for causal in (False, True):
        res = o.attention_backward(q, k, v, g, scale, causal, magnitudes=True)
        dqm, dkm = res[3], res[4]
        for b in range(B):
            for h in range(H):
                e = np.sum(np.abs(g[b, 0, h]) * np.abs(v[b, 0, h]))
                ref_q = scale * e * np.abs(k[b, 0, h])
                ref_k = scale * e * np.abs(q[b, 0, h])
                assert np.allclose(dqm[b, 0, h], ref_q, rtol=1e-13, atol=0), ("|dq|", causal, b, h)
                assert np.allclose(dkm[b, 0, h], ref_k, rtol=1e-13, atol=0), ("|dk|", causal, b, h)
    # grouped K/V: the one key of a K/V head collects every query head of its group
    q, g = rng.standard_normal((1, 1, 4, 3)), rng.standard_normal((1, 1, 4, 3))
    k, v = rng.standard_normal((1, 1, 2, 3)), rng.standard_normal((1, 1, 2, 3))
    res = o.attention_backward(q, k, v, g, scale, True, magnitudes=True)
    for hk in range(2):
        ref = 0.0
        for h in (2 * hk, 2 * hk + 1):
            e = np.sum(np.abs(g[0, 0, h]) * np.abs(v[0, 0, hk]))
            ref = ref + scale * e * np.abs(q[0, 0, h])
        assert np.allclose(res[4][0, 0, hk], ref, rtol=1e-13, atol=0), ("gqa |dk|", hk)


def check_bwd_magnitudes_equal_logits(o):
    """Equal logits make P_ij = 1/n_i exactly (n_i: the keys row i may use),
    which fixes every term of the magnitudes in closed form.  Q = 0 gives
    |dQ|_id = scale/n_i * sum_j (|dp_ij - Delta_i| + E_i) |k_jd|; K = 0
    gives |dK|_jd = scale * sum_(i uses j) (|dp_ij - Delta_i| + E_i)/n_i |q_id|,
    with dp_ij = <dO_i, v_j>, Delta_i = mean_j dp_ij, O_i = mean_j v_j and
    E_i = sum_d |dO_id| |O_id|."""
    rng = np.random.default_rng(37)
    S, D = 6, 3
    scale = 0.7
    for causal in (False, True):
        v, g, kq = (rng.standard_normal((1, S, 1, D)) for _ in range(3))
        zero = np.zeros((1, S, 1, D))

        def row_terms(i):
            n = i + 1 if causal else S
            dp = v[0, :n, 0] @ g[0, i, 0]
            delta = dp.mean()
            e = np.sum(np.abs(g[0, i, 0]) * np.abs(v[0, :n, 0].mean(0)))
            return n, np.abs(dp - delta), e

        # Q = 0, keys kq: dQ magnitudes
        res = o.attention_backward(zero, kq, v, g, scale, causal, magnitudes=True)
        for i in range(S):
            n, adp, e = row_terms(i)
            ref = scale / n * ((adp + e)[:, None] * np.abs(kq[0, :n, 0])).sum(0)
            assert np.allclose(res[3][0, i, 0], ref, rtol=1e-12, atol=0), ("|dq|", causal, i)
        # K = 0, queries kq: dK magnitudes
        res = o.attention_backward(kq, zero, v, g, scale, causal, magnitudes=True)
        for j in range(S):
            ref = np.zeros(D)
            for i in range(S):
                if causal and j > i:
                    continue
                n, adp, e = row_terms(i)
                ref += scale * (adp[j] + e) / n * np.abs(kq[0, i, 0])
            assert np.allclose(res[4][0, j, 0], ref, rtol=1e-12, atol=0), ("|dk|", causal, j)


def check_bwd_rows_match_full(o):
    """The row-list entry point returns the rows of the full backward, for
    dense and varlen inputs with grouped K/V heads."""
    rng = np.random.default_rng(35)

    def bits(x):
        return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    for cu in (None, [0, 4, 9]):
        shape_q = (2, 5, 4, 8) if cu is None else (9, 4, 8)
        shape_k = shape_q[:-2] + (2, 8)
        q, g = bits(_bf16_grid(rng, shape_q)), bits(_bf16_grid(rng, shape_q))
        k, v = bits(_bf16_grid(rng, shape_k)), bits(_bf16_grid(rng, shape_k))
        full = o.attention_backward(q, k, v, g, 0.35, True, cu, magnitudes=True)
        dq, dk, dv, dqm, dkm, dvm = full
        H, Hk = 4, 2
        if cu is None:
            qrows = [(b * H + h) * 5 + i for b, h, i in ((0, 0, 0), (1, 3, 4), (0, 2, 3))]
            krows = [(b * Hk + h) * 5 + j for b, h, j in ((0, 0, 0), (1, 1, 4), (1, 0, 2))]
            qsel = [dq[0, 0, 0], dq[1, 4, 3], dq[0, 3, 2]]
            ksel = [(0, 0, 0), (1, 4, 1), (1, 2, 0)]
        else:
            T = 9
            qrows = [h * T + t for h, t in ((0, 0), (3, 8), (2, 5))]
            krows = [h * T + t for h, t in ((0, 0), (1, 8), (0, 4))]
            qsel = [dq[0, 0], dq[8, 3], dq[5, 2]]
            ksel = [(0, 0), (8, 1), (4, 0)]
        r = o.attention_backward_rows_bf16(q, k, v, g, qrows, krows, 0.35, True, cu)
        assert np.array_equal(r[0], np.stack(qsel)), ("dq rows", cu)
        assert np.array_equal(r[2], np.stack([dk[t] for t in ksel])), ("dk rows", cu)
        assert np.array_equal(r[3], np.stack([dv[t] for t in ksel])), ("dv rows", cu)
        assert np.array_equal(r[5], np.stack([dvm[t] for t in ksel])), ("|dv| rows", cu)


ALL_CHECKS = [
    check_brute_force_tiny,
    check_equal_logits_mean_of_v,
    check_dominant_logit_selects_row,
    check_causal_row0,
    check_kv_permutation_invariance,
    check_key_shift,
    check_affine_v,
    check_causal_prefix,
    check_varlen_equals_dense_runs,
    check_scale_is_a_logit_multiplier,
    check_gqa_brute_force_tiny,
    check_gqa_equals_repeated_kv,
    check_value_dim_brute_force_tiny,
    check_value_columns_are_independent,
    check_qk_lengths_brute_force_tiny,
    check_short_queries_are_the_last_rows_of_self_attention,
    check_rows_without_keys,
    check_bwd_finite_differences,
    check_bwd_torch_autograd,
    check_bwd_rows_without_keys,
    check_bwd_single_key,
    check_bwd_uniform_probabilities,
    check_bwd_magnitudes_single_key,
    check_bwd_magnitudes_equal_logits,
    check_bwd_rows_match_full,
]
