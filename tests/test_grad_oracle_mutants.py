"""Planted mistakes in copies of the backward + KL-loss oracle must each fail at
least one pin of tests/grad_pins.py.  Every mutant keeps its memory accesses in
bounds, so it fails by value, never by crashing."""
import os
import subprocess

import pytest

from oracle import grad
from tests import grad_pins

SRC = os.path.join(os.path.dirname(grad.__file__), "li_grad_oracle.c")
HDR = os.path.join(os.path.dirname(grad.__file__), "li_grad_oracle.h")

MUTANTS = {
    "kl_reversed": ("if (pj > 0.0) loss += pj * (log(pj) - log_pi);",
                    "loss += exp(log_pi) * (log_pi - log(pj));"),
    "no_l1_normalisation": ("const double pj = ph[j] / z;", "const double pj = ph[j];"),
    "dI_sign": ("dI_row[j] = exp(log_pi) - pj;", "dI_row[j] = pj - exp(log_pi);"),
    "relu_gradient_gate_dropped": ("if (d_qi && x > 0.0) {", "if (d_qi) {"),
    "dki_gate_dropped": ("if (!(x > 0.0)) continue;", "if (0) continue;"),
    "dw_without_relu": ("if (d_w) d_w[t * Ni + h] += dI_row[j] * (x > 0.0 ? x : 0.0);",
                        "if (d_w) d_w[t * Ni + h] += dI_row[j] * x;"),
    "dqi_from_qi": ("d_qi[(t * Ni + h) * Di + d] += ds * liog_decode(p->dtype, in->ki, key * Di + d);",
                    "d_qi[(t * Ni + h) * Di + d] += ds * liog_decode(p->dtype, in->qi, (t * Ni + h) * Di + d);"),
    "dki_from_ki": ("kj->d_ki[key * Di + d] += ds * liog_decode(p->dtype, in->qi, (t * Ni + h) * Di + d);",
                    "kj->d_ki[key * Di + d] += ds * liog_decode(p->dtype, in->ki, key * Di + d);"),
    "stats_of_head0": ("psum += exp(p->scale * x - (double)in->softmax_max[t * G + g]) /\n"
                       "              (double)in->softmax_sum[t * G + g];",
                       "psum += exp(p->scale * x - (double)in->softmax_max[t * G]) /\n"
                       "              (double)in->softmax_sum[t * G];"),
    "rope_dropped": ("      if (p->d_rope > 0)\n        x += dot(", "      if (0)\n        x += dot("),
    "scale_dropped": ("psum += exp(p->scale * x -", "psum += exp(x -"),
    "index_weight_head0": ("acc += liog_decode(p->w_dtype, in->w, t * Ni + h) * (x > 0.0 ? x : 0.0);",
                           "acc += liog_decode(p->w_dtype, in->w, t * Ni) * (x > 0.0 ? x : 0.0);"),
    "index_relu_dropped": ("acc += liog_decode(p->w_dtype, in->w, t * Ni + h) * (x > 0.0 ? x : 0.0);",
                           "acc += liog_decode(p->w_dtype, in->w, t * Ni + h) * x;"),
    "dki_wrong_key_row": ("kj->d_ki[key * Di + d] +=", "kj->d_ki[(key - sel[j] + j % (s2 > 0 ? s2 : 1)) * Di + d] +="),
    "tnd_key_offset": ("*k_off = prev_cu(in->cu_seqlens_k, b);", "*k_off = prev_cu(in->cu_seqlens_k, 0);"),
    "softmax_max_added": ("exp(p->scale * x - (double)in->softmax_max[t * G + g])",
                          "exp(p->scale * x + (double)in->softmax_max[t * G + g])"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_grad_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique / missing"
    src = tmp_path / "li_grad_oracle.c"
    src.write_text(source.replace(old, new))
    (tmp_path / "li_grad_oracle.h").write_text(open(HDR).read())
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(src),
                           "-lpthread", "-lm"])
    failed = []
    with grad.use_library(str(so)):
        for pin in grad_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
