"""Planted mistakes in the oracle, on the CPU: a copy of oracle.c with one
plausible error is built with gcc and the oracle's pins (tests/test_oracle.py)
are run against it in a fresh process. Each planted error must make at least
one pin fail; the unmodified copy, built the same way, must pass them all."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTATIONS = [
    # dequantisation x^ = s c + z with the offset's sign flipped
    ("offset_sign", "out[i] = s[i] * (double)c[i] + z[i];", "out[i] = s[i] * (double)c[i] - z[i];"),
    # query head r of KV head h read as head r Hkv + h instead of h R + r
    ("gqa_head_index", "J->q[((long)b * f->num_q_heads + (long)h * R + r) * D + d]",
     "J->q[((long)b * f->num_q_heads + (long)r * f->num_kv_heads + h) * D + d]"),
    # K codes packed from the top of each byte down instead of from bit 0 up
    ("k_bit_order", "|= (uint8_t)(c << (bit % 8));", "|= (uint8_t)(c << (8 - f->bits - bit % 8));"),
    # binary16 rounding: ties away from zero instead of to even
    ("f16_ties", "if (rem > half || (rem == half && (keep & 1u))) keep += 1u;",
     "if (rem >= half) keep += 1u;"),
    # paged channel-wise (s, z): the pair looked up in each token's own page
    # instead of the page holding the group's first token
    ("paged_pair_page", "int t0 = (t / G) * G;", "int t0 = t;"),
    # scale from 2^b levels instead of the 2^b - 1 steps between min and max
    ("scale_levels", "range / (float)qmax;", "range / (float)(qmax + 1);"),
    # binary16 subnormals decoded one binade too low
    ("f16_subnormal", "if (e == 0) v = ldexp((double)m, -24);", "if (e == 0) v = ldexp((double)m, -25);"),
    # the softmax scale left out of the reference attention
    ("softmax_scale", "      w[t] = scale * acc;", "      w[t] = acc;"),
    # V codes packed into a word from the top down
    ("v_bit_order", "|= (uint32_t)c << (f->bits * (t % tpw(f)));",
     "|= (uint32_t)c << (f->bits * (tpw(f) - 1 - t % tpw(f)));"),
    # V word position in a 64-token block: channel half chosen by the wrong bit
    ("v_block_word", "256L * ((d / 4) % 2)", "256L * ((d / 8) % 2)"),
]


def _build(tmp_path, text, tag):
    c = tmp_path / f"oracle_{tag}.c"
    c.write_text(text)
    so = tmp_path / f"liboracle_{tag}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                           "-shared", "-pthread", "-o", str(so), str(c), "-lm"])
    return so


def _run_pins(so):
    env = dict(os.environ, KVQ_ORACLE_LIB=str(so))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join("tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    r = _run_pins(_build(tmp_path, open(SRC).read(), "clean"))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"{name}: the text to change must occur once in oracle.c"
    r = _run_pins(_build(tmp_path, text.replace(old, new), name))
    # exit status 1: tests ran and at least one failed (not a usage or collection error)
    assert r.returncode == 1, (name, r.returncode, r.stdout[-3000:])
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    print(f"{name}: {failed}")
    assert failed
