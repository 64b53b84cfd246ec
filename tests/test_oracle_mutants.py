"""Planted mistakes: each mutant of the oracle source must fail at least one pin.

The mutants are made by textual substitution in a temporary copy of oracle.c,
built with gcc, and the pin suite (test_oracle.py) is run against each in a
subprocess. This shows the pins are sharp enough to catch a dropped term, a
wrong sign, a wrong index or stride, a swapped operand and a wrong decoder.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "head_map_mod": ("return attend(p, qv, b, h / G, L, s, out);", "return attend(p, qv, b, h % p->Hkv, L, s, out);"),
    "offset_shift": ("*off = t % p->bs;", "*off = (t + 1) % p->bs;"),
    "block_index": ("p->table[(int64_t)b * p->MBS + t / p->bs]", "p->table[(int64_t)b * p->MBS + t % p->MBS]"),
    "scale_dropped": ("s[t] = p->scale * dot;", "s[t] = dot;"),
    "max_sign": ("double w = exp(s[t] - M);", "double w = exp(M - s[t]);"),
    "no_normalise": ("out[i] /= Z;", "out[i] /= 1.0;"),
    "strides_swapped": ("(int64_t)hk * st[1] + (int64_t)off * st[2]", "(int64_t)hk * st[2] + (int64_t)off * st[1]"),
    "k_for_v": ("load_elem(p, p->v, p->vs,", "load_elem(p, p->k, p->ks,"),
    "q_row_by_kv_head": ("((int64_t)b * p->Hq + h) * p->D", "((int64_t)b * p->Hq + h / G) * p->D"),
    "f16_bias": ("e - 25", "e - 24"),
    "f16_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "last_token_dropped": ("for (int t = 0; t < L; t++) {\n    int off;\n    int64_t phys = slot_of(p, b, t, &off);\n    if (phys < 0)",
                           "for (int t = 0; t < L - 1; t++) {\n    int off;\n    int64_t phys = slot_of(p, b, t, &off);\n    if (phys < 0)"),
    "max_not_subtracted_first_token": ("if (s[t] > M || t == 0) M = s[t];", "if (s[t] > M && t > 0) M = s[t];"),
}


# mistakes in the prefill's row -> sequence mapping and causal key range; the
# prefill pins (test_oracle_prefill.py) must catch each
PREFILL_MUTANTS = {
    "causal_no_plus_one": ("kend = L - qlen + (row - cu_q[b]) + 1;", "kend = L - qlen + (row - cu_q[b]);"),
    "causal_top_left": ("kend = L - qlen + (row - cu_q[b]) + 1;", "kend = (row - cu_q[b]) + 1;"),
    "row_seq_off_by_one": ("while (cu_q[b + 1] <= row) b++;", "while (cu_q[b + 1] < row) b++;"),
    "causal_ignored": ("    if (causal) {\n      kend", "    if (0) {\n      kend"),
    "q_row_not_packed": ("attend(&p, q + ((int64_t)row * Hq + h) * D,", "attend(&p, q + ((int64_t)b * Hq + h) * D,"),
}


def _run_pins(tmp_path, name, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant = src.replace(old, new)
    c = tmp_path / "oracle_mut.c"
    c.write_text(mutant)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    str(c), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(HERE, pins)], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_fails_some_pin(name, tmp_path):
    old, new = PREFILL_MUTANTS[name]
    r = _run_pins(tmp_path, name, old, new, "test_oracle_prefill.py")
    assert r.returncode != 0, f"mutant {name} passed every prefill pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_some_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant = src.replace(old, new)
    c = tmp_path / "oracle_mut.c"
    c.write_text(mutant)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    str(c), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
