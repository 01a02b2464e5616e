"""The oracle's pins must catch plausible mistakes: each case below plants one
mistake in a copy of ring_oracle.c (built into a temporary directory, on the
CPU), points the oracle at that copy and runs the pin suite, which must fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ring_oracle.c")

MUTANTS = {
    "causal_excludes_diagonal": ("if (tk > t) return 0;", "if (tk >= t) return 0;"),
    "gqa_head_map_modulo": ("h / group, d, scale, idx, n, sbuf, obuf", "h % Hkv, d, scale, idx, n, sbuf, obuf"),
    "scale_dropped": ("s *= scale;", ""),
    "striped_block_index": ("return t % r->n_blocks;", "return t / r->n_blocks;"),
    "pass_limit_off_by_one": ("return step < r->passes;", "return step <= r->passes;"),
    "ring_direction_reversed": ("((block_of(r, t) - block_of(r, tk))", "((block_of(r, tk) - block_of(r, t))"),
    "lse_without_max": ("*lse = M + log(L);", "*lse = log(L);"),
    "doc_boundary_ignored": ("if (mask == RO_MASK_DOC_CAUSAL && doc_of[tk] != doc_of[t]) return 0;", ""),
    "striped_tally_key_block": ("w * N + j : j * B + w", "w * N + i : j * B + w"),
    "empty_row_lse_zero": ("*lse = -INFINITY;\n        *m_out", "*lse = 0;\n        *m_out"),
    "value_index_transposed": ("w * view_at(v, idx[a], g, c)", "w * view_at(v, idx[a], g, d - 1 - c)"),
    "denominator_missing_term": ("L += w;", "if (a > 0) L += w;"),
    "key_padding_ignored": ("(!key_valid || key_valid[tk]))\n                        idx[n++] = tk;",
                            "1)\n                        idx[n++] = tk;"),
    "block_key_padding_inverted": ("(!key_valid || key_valid[w])", "(!key_valid || !key_valid[w])"),
}


# Mistakes in the backward, caught by its own pins.
MUTANTS_BWD = {
    "bwd_softmax_jacobian_diagonal_only": ("double ds = p * (dp - D);", "double ds = p * dp;"),
    "bwd_dk_without_scale": ("dkr[x] += c->scale * ds * view_at(c->q, t, h, x);",
                             "dkr[x] += ds * view_at(c->q, t, h, x);"),
    "bwd_dv_uses_dp": ("dvr[x] += p * view_at(c->dout, t, h, x);", "dvr[x] += dp * view_at(c->dout, t, h, x);"),
    "bwd_dq_uses_value": ("dq_row[x] += c->scale * ds * view_at(c->k, j, g, x);",
                          "dq_row[x] += c->scale * ds * view_at(c->v, j, g, x);"),
    "bwd_D_from_state": ("D += view_at(c->dout, t, h, x) * obuf[x];", "D += view_at(c->dout, t, h, x) * Obuf[x];"),
    "bwd_key_padding_ignored": ("(!c->key_valid || c->key_valid[tk]))", "1)"),
}


def _build_mutant(tmp_path, name, before, after):
    src = open(SRC).read()
    assert before in src, "mutation site vanished: update the mutant table"
    c_path = tmp_path / (name + ".c")
    c_path.write_text(src.replace(before, after, 1))
    so = tmp_path / ("lib_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", str(c_path),
                           "-o", str(so), "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    so = _build_mutant(tmp_path, name, *MUTANTS_BWD[name])
    env = dict(os.environ, RING_ORACLE_LIB=str(so), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_backward_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=600)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    before, after = MUTANTS[name]
    assert before in src, "mutation site vanished: update the mutant table"
    c_path = tmp_path / (name + ".c")
    c_path.write_text(src.replace(before, after, 1))
    so = tmp_path / ("lib_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", str(c_path),
                           "-o", str(so), "-lm"])
    env = dict(os.environ, RING_ORACLE_LIB=str(so), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=600)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])
