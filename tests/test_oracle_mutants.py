"""Plausible mistakes planted in a copy of the oracle must fail a pin.

Each mutant is the oracle's C source with one small, realistic error (an
off-by-one mask, a dropped scale, a transposed or mis-indexed operand, a
wrong sign, a missing normalisation).  It is compiled to a temporary library
on the CPU and run through the pins of oracle_pins.py; the test passes only
if at least one pin rejects it.  This shows the pins would catch such a
mistake in the real oracle.
"""
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (os.path.dirname(_HERE), _HERE):   # also run as a child script
    if _p not in sys.path:
        sys.path.insert(0, _p)

import pytest  # noqa: E402

import oracle  # noqa: E402
import oracle_pins  # noqa: E402

# (name, text in attn_oracle.c, replacement)
MUTANTS = [
    ("mask_excludes_diagonal", "const int last = i + spk.len - spq.len;",
     "const int last = i + spk.len - spq.len - 1;"),
    ("mask_admits_next_key", "const int last = i + spk.len - spq.len;",
     "const int last = i + spk.len - spq.len + 1;"),
    ("causal_top_left_alignment", "const int last = i + spk.len - spq.len;", "const int last = i;"),
    ("empty_row_not_special", "if (nkeys == 0) {", "if (0) {"),
    ("key_span_from_query_offsets", "seq_span spk = span_of(b, sh->Sk, sh->cu_k);",
     "seq_span spk = span_of(b, sh->Sq, sh->cu_q);"),
    ("scale_dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("k_read_at_query_row", "dot += at(q, qbase + d) * at(k, kbase + d);",
     "dot += at(q, qbase + d) * at(k, qbase + d);"),
    ("exp_sign_flipped", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("lse_missing_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("normalisation_dropped", "o_row[d] = acc / l;", "o_row[d] = acc;"),
    ("v_head_ignored", "acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv + d);",
     "acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + 0) * (int64_t)Dv + d);"),
    ("v_read_at_query_row", "acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv + d);",
     "acc += s[j] * at(v, ((spk.tok0 + i) * Hkv + hk) * (int64_t)Dv + d);"),
    ("v_row_stride_of_q", "acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)Dv + d);",
     "acc += s[j] * at(v, ((spk.tok0 + j) * Hkv + hk) * (int64_t)D + d);"),
    ("kv_head_interleaved", "const int hk = h / (H / Hkv);", "const int hk = h % Hkv;"),
    ("kv_head_stride_of_q", "const int64_t kbase = ((spk.tok0 + j) * Hkv + hk) * (int64_t)D;",
     "const int64_t kbase = ((spk.tok0 + j) * H + hk) * (int64_t)D;"),
    ("dense_batch_offset_wrong", "sp.tok0 = (int64_t)b * S;", "sp.tok0 = (int64_t)b;"),
    ("varlen_length_short", "sp.len = cu[b + 1] - cu[b];", "sp.len = cu[b + 1] - cu[b] - (b > 0);"),
    ("row_decode_swaps_h_i", "*i = (int)(row % S);\n        *h = (int)((row / S) % H);",
     "*h = (int)(row % H);\n        *i = (int)((row / H) % S);"),
    ("sum_skips_first_key", "for (int j = 0; j < nkeys; ++j) {\n        s[j] = exp(s[j] - m);\n        l += s[j];",
     "for (int j = 0; j < nkeys; ++j) {\n        s[j] = exp(s[j] - m);\n        if (j) l += s[j];"),
    ("bwd_delta_dropped_in_dq", "const double ds = p[j] * (dp[j] - delta);",
     "const double ds = p[j] * dp[j];"),
    ("bwd_delta_dropped_in_dk", "const double ds = p * (dp - st->delta);", "const double ds = p * dp;"),
    ("bwd_dk_scale_dropped", "dk_row[d] += scale * ds * qd;", "dk_row[d] += ds * qd;"),
    ("bwd_dq_scale_dropped", "dq_row[d] = scale * g;", "dq_row[d] = g;"),
    ("bwd_dv_weighted_by_ds", "dv_row[d] += p * gd;", "dv_row[d] += ds * gd;"),
    ("bwd_dp_reads_k", "acc += at(dout, obase + d) * at(v, vbase + d);",
     "acc += at(dout, obase + d) * at(k, vbase + d);"),
    ("bwd_key_rows_start_late", "i0 = j - (spk.len - spq.len);", "i0 = j - (spk.len - spq.len) + 1;"),
    ("bwd_key_rows_top_left", "i0 = j - (spk.len - spq.len);", "i0 = j;"),
    ("bwd_key_span_from_query_offsets", "const seq_span spk = span_of(b, sh->Sk, sh->cu_k);",
     "const seq_span spk = span_of(b, sh->Sq, sh->cu_q);"),
    ("bwd_group_first_head_only", "const int h = hk * G + g;", "const int h = hk * G;"),
    ("bwd_probs_unnormalised", "p[j] = exp(p[j] - *lse);", "p[j] = exp(p[j] - m);"),
    ("bwd_lse_sign", "const double p = exp(scale * s - st->lse);",
     "const double p = exp(scale * s + st->lse);"),
    ("bwd_dq_magnitude_x4", "dq_mag[d] = scale * mag;", "dq_mag[d] = 4 * scale * mag;"),
    ("bwd_dk_magnitude_x4", "dk_mag[d] += scale * (fabs(ds) + p * st->e) * fabs(qd);",
     "dk_mag[d] += 4 * scale * (fabs(ds) + p * st->e) * fabs(qd);"),
    ("bwd_dq_delta_bound_x8", "mag += (fabs(ds) + p[j] * e) * fabs(kd);",
     "mag += (fabs(ds) + 8 * p[j] * e) * fabs(kd);"),
    ("bwd_dk_delta_bound_x8", "dk_mag[d] += scale * (fabs(ds) + p * st->e) * fabs(qd);",
     "dk_mag[d] += scale * (fabs(ds) + 8 * p * st->e) * fabs(qd);"),
    ("bwd_dq_magnitude_drops_ds", "mag += (fabs(ds) + p[j] * e) * fabs(kd);",
     "mag += (p[j] * e) * fabs(kd);"),
    ("bwd_dk_magnitude_drops_ds", "dk_mag[d] += scale * (fabs(ds) + p * st->e) * fabs(qd);",
     "dk_mag[d] += scale * (p * st->e) * fabs(qd);"),
    ("bwd_delta_bound_unsigned_o", "e += fabs(at(dout, obase + d)) * fabs(od);",
     "e += fabs(at(dout, obase + d)) * od;"),
    ("bwd_dq_magnitude_key_index", "mag += (fabs(ds) + p[j] * e) * fabs(kd);",
     "mag += (fabs(ds) + p[j] * e) * fabs(at(k, ((spk.tok0 + j) * Hkv + hk) * (int64_t)D));"),
    ("bwd_key_row_decode_swaps", "*j = (int)(row % S);\n        *hk = (int)((row / S) % Hkv);",
     "*hk = (int)(row % Hkv);\n        *j = (int)((row / Hkv) % S);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.build(force=True, src=path, out=os.path.join(tmp_path, "libmutant.so"))
    r = subprocess.run([sys.executable, os.path.abspath(__file__), lib],
                       capture_output=True, text=True, timeout=300)
    assert "Error" not in r.stderr or r.returncode < 0, r.stderr[-2000:]
    caught = r.returncode != 0 or r.stdout.strip() != ""
    assert caught, "no pin caught mutant " + name


def _run_pins(lib_path):
    """Child-process entry: print the names of the pins the library fails."""
    lib = oracle.OracleLib(lib_path)
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, FloatingPointError):
            print(check.__name__)


if __name__ == "__main__":
    _run_pins(sys.argv[1])
