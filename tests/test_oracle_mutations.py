"""The oracle's pins catch plausible mistakes in oracle.c.

Each case plants one mistake in a copy of oracle/oracle.c -- a dropped
term, a wrong sign or exponent, an index off by one, a transposed layout, a
wrong head mapping, a missing normalisation -- builds the copy into its own
library, and runs the oracle's pins (tests/test_oracle.py, then
tests/test_oracle_fp8.py, whose attention over a quantized cache also runs
through oracle.c) against it in a child process: at least one pin must
fail.  A mutation that no pin catches would be a part of the oracle that
nothing checks against the pages or the mathematics.  CPU only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, planted text); each original occurs once in oracle.c
MUTATIONS = [
    ("binary16 subnormal exponent", "v = ldexp((double)frac, -24);",
     "v = ldexp((double)frac, -25);"),
    ("binary16 normal exponent bias", "v = ldexp((double)(1024 + frac), expo - 25);",
     "v = ldexp((double)(1024 + frac), expo - 24);"),
    ("binary16 sign dropped", "return sign ? -v : v;", "return v;"),
    ("slot of a new token off by one", "int64_t p = (int64_t)ctx - n + k;",
     "int64_t p = (int64_t)ctx - n + k - 1;"),
    ("append into a [block][slot][head] layout",
     "int64_t dst = ((block * num_kv_heads + g) * block_size + offset) * head_dim + e;",
     "int64_t dst = ((block * block_size + offset) * num_kv_heads + g) * head_dim + e;"),
    ("gather reads the next row of the block",
     "int64_t base = ((block * num_kv_heads + g) * block_size + p % block_size) * head_dim;",
     "int64_t base = ((block * num_kv_heads + g) * block_size + (p + 1) % block_size) * head_dim;"),
    ("causal range leaves out the query's own position",
     "attend_range(qd, K, V, 0, pos + 1, head_dim, scale, s,",
     "attend_range(qd, K, V, 0, pos, head_dim, scale, s,"),
    ("score scale dropped", "s_scratch[p - lo] = scale * dot;", "s_scratch[p - lo] = dot;"),
    ("running max not subtracted", "double w = exp(s_scratch[p - lo] - m);",
     "double w = exp(s_scratch[p - lo]);"),
    ("output not normalised", "for (int32_t e = 0; e < head_dim; ++e) out[e] /= l;",
     "for (int32_t e = 0; e < head_dim; ++e) out[e] /= 1.0;"),
    ("query heads interleaved over KV heads",
     "for (int32_t h = g * group; h < (g + 1) * group; ++h) {",
     "for (int32_t h = g; h < num_q_heads; h += num_kv_heads) {"),
    ("merge weight without the partial's sum", "double w = l_parts[p] * exp(m_parts[p] - M);",
     "double w = exp(m_parts[p] - M);"),
    ("merge not divided by the total weight",
     "for (int32_t e = 0; e < head_dim; ++e) out[e] /= W;",
     "for (int32_t e = 0; e < head_dim; ++e) out[e] /= 1.0;"),
]


def _run_pins(name, original, planted, tmp):
    src = open(SRC).read()
    assert src.count(original) == 1, f"{name}: the original text must occur once in oracle.c"
    tag = "".join(c if c.isalnum() else "_" for c in name)
    mutated = os.path.join(tmp, f"{tag}.c")
    lib = os.path.join(tmp, f"lib{tag}.so")
    with open(mutated, "w") as f:
        f.write(src.replace(original, planted))
    oracle.build(src=mutated, out=lib)
    env = dict(os.environ, ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2")
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(HERE, "test_oracle.py"), os.path.join(HERE, "test_oracle_fp8.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, res.returncode, res.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_pins(*m, str(tmp_path)), MUTATIONS))
    survived = [(name, out) for name, rc, out in results if rc == 0]
    for name, rc, _ in results:
        print(f"[mutation] {name}: {'caught' if rc != 0 else 'SURVIVED'}", flush=True)
    assert not survived, "mutations no pin catches: " + "; ".join(n for n, _ in survived)


def test_the_unmutated_copy_passes_the_pins(tmp_path):
    """The harness itself: the same build and run of an unchanged copy passes
    (so a caught mutation fails for its planted mistake, not the harness)."""
    name, rc, out = _run_pins("unchanged", "return sign ? -v : v;", "return sign ? -v : v;",
                              str(tmp_path))
    assert rc == 0, out
