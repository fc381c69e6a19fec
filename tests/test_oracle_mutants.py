"""Plant plausible mistakes in copies of the oracle's C source and check that the pins catch
every one of them (CPU only; the real oracle is never modified)."""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# (name, original text, mutated text): each original must occur in the source.
MUTANTS = [
    ("gqa_interleaved", "int64_t kv = hq / group;", "int64_t kv = hq % Hkv;"),
    ("causal_strict", "if (causal && j > i)", "if (causal && j >= i)"),
    ("causal_reversed", "if (causal && j > i)", "if (causal && j < i)"),
    ("padding_off_by_one", "if (j >= valid)", "if (j > valid)"),
    ("padding_by_query", "if (j >= valid)", "if (i >= valid)"),
    ("no_scale", "scores[j] = scale * dot;", "scores[j] = dot;"),
    ("scale_twice", "scores[j] = scale * dot;", "scores[j] = scale * scale * dot;"),
    ("no_max_shift", "l += exp(scores[j] - m);", "l += exp(scores[j]);"),
    ("max_init_zero", "double m = -INFINITY, l = 0.0;", "double m = 0.0, l = 0.0;"),
    ("sum_init_one", "double m = -INFINITY, l = 0.0;", "double m = -INFINITY, l = 1.0;"),
    ("lse_without_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("lse_base2", "*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    ("no_normalisation", "double w = exp(scores[j] - m) / l;", "double w = exp(scores[j] - m);"),
    ("key_row_from_query_index", "const double *k_row = k_head + j * D;",
     "const double *k_row = k_head + i * D;"),
    ("value_row_from_query_index", "const double *v_row = v_head + j * D;",
     "const double *v_row = v_head + i * D;"),
    ("dot_drops_last_term", "for (d = 0; d < D; ++d)\n            dot +=",
     "for (d = 0; d < D - 1; ++d)\n            dot +="),
    ("empty_row_lse_zero", "*lse_out = -INFINITY;", "*lse_out = 0.0;"),
    ("empty_row_not_zeroed", "o_row[d] = 0.0;\n        *lse_out", "o_row[d] = 1.0;\n        *lse_out"),
    ("batch_index_swapped", "int64_t b = bh / Hq;", "int64_t b = bh % B;"),
    ("head_index_swapped", "int64_t hq = bh % Hq;", "int64_t hq = bh / B % Hq;"),
    ("no_valid_len_clamp_high", "if (valid > N)\n                    valid = N;",
     "if (valid > N)\n                    valid = N - 1;"),
    ("kv_head_stride_uses_hq", "k + (b * Hkv + kv) * N * D", "k + (b * Hq + kv) * N * D"),
    ("keep_mask_ignored", "if (mr->kind == 1 && mr->keep[j] == 0)", "if (0 && mr->keep[j] == 0)"),
    ("keep_mask_inverted", "if (mr->kind == 1 && mr->keep[j] == 0)",
     "if (mr->kind == 1 && mr->keep[j] != 0)"),
    ("add_mask_ignored", "scores[j] += mr->add[j];", "scores[j] += 0.0;"),
    ("add_mask_subtracted", "scores[j] += mr->add[j];", "scores[j] -= mr->add[j];"),
    ("add_mask_scaled", "scores[j] += mr->add[j];", "scores[j] += scale * mr->add[j];"),
    ("add_neginf_kept", "if (mr->kind == 2 && mr->add[j] == -INFINITY)", "if (0)"),
    ("mask_row_ignored", "hq * mask_strides[1] + i * mask_strides[2]",
     "hq * mask_strides[1] + 0 * mask_strides[2]"),
    ("mask_head_ignored", "hq * mask_strides[1] + i * mask_strides[2]",
     "0 * mask_strides[1] + i * mask_strides[2]"),
    ("mask_batch_ignored", "int64_t off = b * mask_strides[0]", "int64_t off = 0 * mask_strides[0]"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, orig, mut):
    assert orig in source, "mutation site for %s no longer in the oracle source" % name
    text = source.replace(orig, mut, 1)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(text)
        lib = oracle.load(oracle.build(src, os.path.join(d, "libmutant.so")))

        def fn(q, k, v, scale, causal, valid_len=None, rows=None, keep_mask=None,
               add_mask=None):
            return oracle.attn_fwd(q, k, v, scale, causal, valid_len, rows=rows, threads=2,
                                   lib=lib, keep_mask=keep_mask, add_mask=add_mask)

        caught = []
        for pin in oracle_pins.ALL_PINS + oracle_pins.MASK_PINS:
            try:
                pin(fn)
            except (AssertionError, ValueError, FloatingPointError) as e:
                caught.append(pin.__name__)
        assert caught, "no pin caught the planted mistake %s" % name


# Planted mistakes in the backward (oracle_attn_bwd); the backward pins must catch each.
BWD_MUTANTS = [
    ("bwd_no_delta", "const double ds = w[j] * (dp[j] - delta);", "const double ds = w[j] * dp[j];"),
    ("bwd_delta_sign", "const double ds = w[j] * (dp[j] - delta);",
     "const double ds = w[j] * (dp[j] + delta);"),
    ("bwd_dq_unscaled", "dq_row[d] += scale * ds * k_head[j * D + d];",
     "dq_row[d] += ds * k_head[j * D + d];"),
    ("bwd_dk_unscaled", "dk_head[j * D + d] += scale * ds * q_row[d];",
     "dk_head[j * D + d] += ds * q_row[d];"),
    ("bwd_dq_uses_v", "dq_row[d] += scale * ds * k_head[j * D + d];",
     "dq_row[d] += scale * ds * v_head[j * D + d];"),
    ("bwd_dv_uses_ds", "dv_head[j * D + d] += w[j] * do_row[d];",
     "dv_head[j * D + d] += ds * do_row[d];"),
    ("bwd_dp_uses_k", "dot += do_row[d] * v_head[j * D + d];",
     "dot += do_row[d] * k_head[j * D + d];"),
    ("bwd_delta_unweighted", "delta += w[j] * dot;", "delta += dot;"),
    ("bwd_first_head_only", "for (int64_t hq = kv * group; hq < (kv + 1) * group; ++hq)",
     "for (int64_t hq = kv * group; hq < kv * group + 1; ++hq)"),
    ("bwd_unnormalised_weights", "w[j] = exp(w[j] - m) / l;", "w[j] = exp(w[j] - m);"),
    # explicit masks in the backward
    ("bwd_mask_ignored", "const mask_row *mrp = &mr;",
     "const mask_row none = {0, NULL, NULL};\n                    const mask_row *mrp = &none;"),
    ("bwd_add_mask_dropped", "                            w[j] += mr.add[j];",
     "                            w[j] += 0.0;"),
    ("bwd_add_mask_subtracted", "                            w[j] += mr.add[j];",
     "                            w[j] -= mr.add[j];"),
    ("bwd_mask_row_index", "                                      i * mask_strides[2];",
     "                                      0 * mask_strides[2];"),
    ("bwd_mask_head_index", "int64_t off = b * mask_strides[0] + hq * mask_strides[1] +\n",
     "int64_t off = b * mask_strides[0] + 0 * mask_strides[1] +\n"),
]


@pytest.mark.parametrize("name,orig,mut", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_mutant_is_caught(source, name, orig, mut):
    assert orig in source, "mutation site for %s no longer in the oracle source" % name
    text = source.replace(orig, mut, 1)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(text)
        lib = oracle.load(oracle.build(src, os.path.join(d, "libmutant.so")))

        def fn(q, k, v, scale, causal, valid_len=None, rows=None, **mask):
            return oracle.attn_fwd(q, k, v, scale, causal, valid_len, rows=rows, threads=2,
                                   lib=lib, **mask)

        def fn_bwd(q, k, v, dout, scale, causal, valid_len=None, **mask):
            return oracle.attn_bwd(q, k, v, dout, scale, causal, valid_len, threads=2, lib=lib,
                                   **mask)

        caught = []
        for pin in oracle_pins.BWD_PINS + oracle_pins.BWD_MASK_PINS:
            try:
                pin(fn_bwd, fn)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, "no pin caught the planted mistake %s" % name
