"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a wrong stride or offset, a reversed tie-break, an
off-by-one mask).  Each is compiled from a patched copy of li_oracle.c into a
temporary directory and the whole pin list runs against it.  All mutants keep
their memory accesses in bounds, so they fail by value, never by crashing.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "li_oracle.c")

MUTANTS = {
    "relu_dropped": ("double r = x > 0.0 ? x : 0.0;", "double r = x;"),
    "weight_of_head0": ("total += wrow[h] * r;", "total += wrow[0] * r;"),
    "weight_sign": ("total += wrow[h] * r;", "total -= wrow[h] * r;"),
    "tie_break_reversed": ("return (x->key > y->key) - (x->key < y->key);",
                           "return (x->key < y->key) - (x->key > y->key);"),
    "causal_off_by_one": ("long long last = (long long)i + S2 - S1;",
                          "long long last = (long long)i + S2 - S1 - 1;"),
    "q_transposed": ("x += qrow[(int64_t)h * p->d + d] * krow[d];",
                     "x += qrow[(int64_t)d * p->n1 + h] * krow[d];"),
    "pool_stride_ignored": ("return (int64_t)blk * p->k_block_stride + (int64_t)row * p->d;",
                            "return (int64_t)blk * p->block_size * p->d + (int64_t)row * p->d;"),
    "k_descale_dropped": ("double kd = (p->qk_dtype == LIO_E4M3) ? (double)in->k_descale[dsc] : 1.0;",
                          "double kd = 1.0;"),
    "q_descale_dropped": ("double qd = (p->qk_dtype == LIO_E4M3) ? (double)in->q_descale[t] : 1.0;",
                          "double qd = 1.0;"),
    "value_padding": ("ov[j] = -INFINITY;", "ov[j] = 0.0f;"),
    "index_padding": ("oi[j] = -1;", "oi[j] = 0;"),
    "last_head_dropped": ("for (int h = 0; h < p->n1; ++h) {\n    double x = 0.0;",
                          "for (int h = 0; h < p->n1 - 1; ++h) {\n    double x = 0.0;"),
    "first_dim_dropped": ("for (int d = 0; d < p->d; ++d) {", "for (int d = 1; d < p->d; ++d) {"),
    "tnd_k_offset": ("? prev_cu(in->cu_seqlens_k, b) + s", "? s"),
    "tnd_q_offset": ("if (p->layout_q == LIO_TND) return prev_cu(in->cu_seqlens_q, b) + i;",
                     "if (p->layout_q == LIO_TND) return i;"),
    "e4m3_bias": ("else v = ldexp((double)(8 + m), e - 10);",
                  "else v = ldexp((double)(8 + m), e - 9);"),
    "bf16_low_bit": ("uint32_t bits = ((uint32_t)u) << 16;",
                     "uint32_t bits = ((uint32_t)(u & 0xFFFE)) << 16;"),
    "ascending_sort": ("if (x->score > y->score) return -1;      /* higher score first */\n"
                       "  if (x->score < y->score) return 1;",
                       "if (x->score > y->score) return 1;\n  if (x->score < y->score) return -1;"),
    "block_table_batch": ("int blk = in->block_table[(int64_t)b * p->max_blocks_per_seq + s / p->block_size];",
                          "int blk = in->block_table[s / p->block_size];"),
    "cmp_block_start": ("if ((long long)j * r + r - 1 <= pos) ++n;", "if ((long long)j * r <= pos) ++n;"),
    "cmp_residual_dropped": ("(long long)S2 * r + in->cmp_residual_k[b] - S1;",
                             "(long long)S2 * r - S1;"),
    "idx_offset_dropped": ("oi[j] = c[j].key + off;", "oi[j] = c[j].key;"),
    "negative_zero_kept": ("ov[j] = (float)c[j].score + 0.0f;", "ov[j] = (float)c[j].score;"),
    "w_not_per_token": ("wrow[h] = lio_decode(p->w_dtype, in->w, t * p->n1 + h);",
                        "wrow[h] = lio_decode(p->w_dtype, in->w, h);"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique / missing"
    src = tmp_path / "li_oracle.c"
    src.write_text(source.replace(old, new))
    hdr = os.path.join(os.path.dirname(SRC), "li_oracle.h")
    (tmp_path / "li_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(src),
                           "-lpthread", "-lm"])
    failed = []
    with oracle.use_library(str(so)):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# Planted mistakes in the gather oracle (oracle/gather.py): each must fail its pin.
GATHER_SRC = os.path.join(os.path.dirname(oracle.__file__), "gather.py")
GATHER_MUTANTS = {
    "tnd_offset_dropped": ("src = kv[k0 + s]", "src = kv[s]"),
    "block_size_ignored": ("s = sel * select_block + u", "s = sel + u"),
    "pool_row_wrong": ("src = kv[blk, s % bs]", "src = kv[blk, s // bs]"),
    "padding_index_used": ("if sel < 0:\n                    continue", "if sel < -1:\n                    continue"),
}


@pytest.mark.parametrize("name", sorted(GATHER_MUTANTS))
def test_gather_mutant_is_caught(name, monkeypatch):
    import oracle.gather as og
    old, new = GATHER_MUTANTS[name]
    src = open(GATHER_SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique / missing"
    ns = {}
    exec(compile(src.replace(old, new), "gather_mutant", "exec"), ns)
    monkeypatch.setattr(og, "gather", ns["gather"])
    with pytest.raises((AssertionError, IndexError)):
        oracle_pins.pin_gather_closed_form()
