"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of oracle.c (a wrong head
group, a sign, a dropped scale or normalisation, a transposed V tile, an
off-by-one in the block walk or the causal limit, a missed copy), builds it with
gcc and runs the pin tests against that build: they must fail.  CPU only; the
real oracle is never modified.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "interleaved_head_groups": ("int h = g * G + j;", "int h = j * Hkv + g;"),
    "score_sign": ("double w = exp(x[t] - m);", "double w = exp(m - x[t]);"),
    "dropped_scale": ("x[t] = scale * acc;", "x[t] = acc;"),
    "dropped_normalisation": ("for (int d = 0; d < D; ++d) o[d] /= den;", "(void)den;"),
    "v_tile_token_major": ("return (((size_t)blk * H + h) * D + d) * BS + off;",
                           "return (((size_t)blk * H + h) * BS + off) * D + d;"),
    "block_walk_off_by_one": ("int32_t blk = table[t / BS];", "int32_t blk = table[(t + 1) / BS];"),
    "offset_off_by_one": ("int off = t % BS;\n        if (blk", "int off = (t + 1) % BS;\n        if (blk"),
    "causal_limit_off_by_one": ("attend(out + (row * Hq + h) * D, q, K, V, pos + 1, D, scale, x);",
                                "attend(out + (row * Hq + h) * D, q, K, V, pos, D, scale, x);"),
    "copy_blocks_skips_v": ("memcpy((char*)value_caches[l] + dst * bytes, (const char*)value_caches[l] + src * bytes, "
                            "bytes);", ";"),
    "f16_exponent_bias": ("v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);"),
    "query_row_of_wrong_head": ("q[d] = load(query, ((size_t)s * Hq + h) * D + d, dtype);",
                                "q[d] = load(query, ((size_t)s * Hq + g) * D + d, dtype);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", str(src), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, PKV_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout or "error" in r.stdout.lower()
