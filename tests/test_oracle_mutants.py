"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Every mutant below is a plausible slip (a dropped term, a wrong sign, a wrong
operand or index, a missing rounding or check). The source copy is edited
textually, built with the same flags as the oracle, and the pins run against it
in a child process; the test passes only when some pin rejects the mutant.
Every mutant keeps all memory accesses inside the arrays the pins pass.
"""

import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

# (name, text in kda_oracle.c, replacement, number of occurrences replaced)
MUTANTS = [
    ("drop_decay", "S[i * dv + j] = at[i] * S[i * dv + j];", "S[i * dv + j] = S[i * dv + j];", 1),
    ("decay_per_value_channel", "S[i * dv + j] = at[i] * S[i * dv + j];",
     "S[i * dv + j] = at[j % dk] * S[i * dv + j];", 1),
    ("delta_sign", "(vt[j] - u[j])", "(u[j] - vt[j])", 1),
    ("drop_beta", "S[i * dv + j] += bt * kt[i] * (vt[j] - u[j]);",
     "S[i * dv + j] += kt[i] * (vt[j] - u[j]);", 1),
    ("delta_read_with_q", "acc += S[i * dv + j] * kt[i];", "acc += S[i * dv + j] * (qt ? qt[i] : kt[i]);", 1),
    ("read_out_with_k", "acc += S[i * dv + j] * qt[i];", "acc += S[i * dv + j] * kt[i];", 1),
    ("write_uses_q", "S[i * dv + j] += bt * kt[i] * (vt[j] - u[j]);",
     "S[i * dv + j] += bt * (qt ? qt[i] : kt[i]) * (vt[j] - u[j]);", 1),
    ("no_fp32_state_rounding", "S[e] = (double)(float)S[e];", "S[e] = S[e];", 1),
    ("cache_transposed", "return slot * c->slot_stride + ((int64_t)h * c->dv + j) * c->dk + i;",
     "return slot * c->slot_stride + ((int64_t)h * c->dv + (i % c->dv)) * c->dk + (j % c->dk);", 1),
    ("cache_head_ignored", "return slot * c->slot_stride + ((int64_t)h * c->dv + j) * c->dk + i;",
     "return slot * c->slot_stride + ((int64_t)0 * c->dv + j) * c->dk + i;", 1),
    ("token_row_ignores_t", "const int64_t r = (row0 + t) * H + h;", "const int64_t r = (row0) * H + h;", 3),
    ("replay_offset_ignores_t", "const int64_t d = ((int64_t)b * c->T_max + t) * H + h;",
     "const int64_t d = ((int64_t)b * c->T_max) * H + h;", 1),
    ("commit_one_token_extra", "n = a;", "n = a < Tb ? a + 1 : a;", 1),
    ("accepted_not_checked", "if (a < 0 || a > Tb)", "if (a < 0)", 1),
    ("padding_uses_slot0", "const int64_t slot = c->slot_ids[b];",
     "const int64_t slot = c->slot_ids[b] < 0 ? 0 : c->slot_ids[b];", 1),
    ("prefill_checkpoint_off_by_one", "kda_oracle_unit(S, dk, dv, (int)ckpt_at, q, k, v, a, be, c->state_fp32, o, NULL);",
     "kda_oracle_unit(S, dk, dv, (int)(ckpt_at > 0 ? ckpt_at - 1 : 0), q, k, v, a, be, c->state_fp32, o, NULL);", 1),
    ("prefill_slot_not_written", "c->kind == KIND_COMMIT || c->kind == KIND_PREFILL ||",
     "c->kind == KIND_COMMIT ||", 1),
    ("gate_sum_not_mean", "ms /= (double)dv;", "ms /= 1.0;", 1),
    ("gate_sigmoid_sign", "exp(-g[j])", "exp(g[j])", 1),
    ("gate_eps_dropped", "sqrt(ms + eps)", "sqrt(ms)", 1),
    ("prologue_q_unscaled", "sqrt(qq + 1e-12) / sqrt((double)dk)", "sqrt(qq + 1e-12)", 1),
    ("prologue_k_not_normalized", "k[i] *= kn;", "k[i] *= 1.0;", 1),
    ("prologue_q_norm_from_k", "qq += q[i] * q[i];", "qq += k[i] * k[i];", 1),
    ("prologue_half_norm", "kk += k[i] * k[i];", "kk += i < dk / 2 ? k[i] * k[i] : 0.0;", 1),
    ("prologue_alpha_as_exp", "exp(-log1p(exp(alpha[i])))", "exp(-alpha[i])", 1),
    ("prologue_alpha_as_sigmoid", "exp(-log1p(exp(alpha[i])))", "1.0 / (1.0 + exp(-alpha[i]))", 1),
    ("prologue_beta_sign", "1.0 / (1.0 + exp(-*beta))", "1.0 / (1.0 + exp(*beta))", 1),
    ("prologue_ignored", "if (c->prologue)", "if (0)", 1),
    ("inplace_rows_not_written", "const int inplace_row = c->kind == KIND_VERIFY && Tb == 1 && c->t1_inplace;",
     "const int inplace_row = 0;", 1),
    ("inplace_flag_ignored_for_perpos", "c->mode == ORACLE_PER_POSITION && !inplace_row;",
     "c->mode == ORACLE_PER_POSITION;", 1),
    ("inplace_slot_not_written", "c->kind == KIND_PREFILL ||\n                           inplace_row;",
     "c->kind == KIND_PREFILL;", 1),
    ("inplace_ignores_token_count", "c->kind == KIND_VERIFY && Tb == 1 && c->t1_inplace;",
     "c->kind == KIND_VERIFY && Tb >= 1 && c->t1_inplace;", 1),
    ("gate_only_first_token", "if (c->gate) {", "if (c->gate && t == 0) {", 1),
    ("gate_only_single_token_rows", "if (c->gate) {", "if (c->gate && n == 1) {", 1),
    ("ckpt_negative_exports_start", "ckpt_at = c->ckpt_pos[b];",
     "ckpt_at = c->ckpt_pos[b] < 0 ? 0 : c->ckpt_pos[b];", 1),
    ("ckpt_negative_is_error", "if (ckpt_at > Tb)", "if (ckpt_at > Tb || ckpt_at < 0)", 1),
]

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
lib = oracle.load_variant({lib!r})
for check in oracle_pins.CHECKS:
    try:
        check(lib)
    except AssertionError:
        print("caught by", check.__name__)
        sys.exit(3)
print("not caught")
sys.exit(0)
"""


def _run_pins(lib_path):
    code = RUNNER.format(root=ROOT, tests=TESTS, lib=lib_path)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)


def _build_variant(tmp_path, text):
    src = tmp_path / "kda_oracle_variant.c"
    src.write_text(text)
    lib = tmp_path / "libkda_oracle_variant.so"
    oracle_build.build(out=str(lib), src=str(src))
    return str(lib)


def test_unmodified_copy_passes_every_pin(tmp_path):
    text = open(oracle_build.SRC).read()
    r = _run_pins(_build_variant(tmp_path, text))
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, count):
    text = open(oracle_build.SRC).read()
    assert text.count(old) == count, f"{name}: pattern occurs {text.count(old)} times"
    r = _run_pins(_build_variant(tmp_path, text.replace(old, new)))
    assert r.returncode == 3, f"{name}: {r.stdout} {r.stderr}"
