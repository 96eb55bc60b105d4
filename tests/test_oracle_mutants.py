"""The oracle's pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/oracle.c``, plants one mistake by text substitution
(a dropped term, a wrong sign, a wrong index, a swapped operand), compiles the
copy, and runs the pin suite against it in a subprocess.  The suite must fail.
Every planted mistake keeps all memory accesses inside the test's buffers.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("z[t] = scale * dot;", "z[t] = dot;"),
    "softmax_sign": ("z[t] = exp(z[t] - m);", "z[t] = exp(m - z[t]);"),
    "unnormalised": ("double p = z[t] / l;", "double p = z[t];"),
    "keys_read_from_v": ("dot += q[d] * K[(int64_t)t * head_dim + d];",
                         "dot += q[d] * V[(int64_t)t * head_dim + d];"),
    "gqa_head_map": ("int32_t kvh = h / group;\n            orc_unpage(k_cache, ks, kv_dtype, table, block_size, L,",
                     "int32_t kvh = h % num_kv_heads;\n            orc_unpage(k_cache, ks, kv_dtype, table, block_size, L,"),
    "row_offset": ("int64_t offset = t % block_size;", "int64_t offset = (t + 1) % block_size;"),
    "causal_off_by_one": ("orc_attention(qv, K, V, pos + 1,", "orc_attention(qv, K, V, pos,"),
    "write_offset": ("int64_t o = slot % block_size;", "int64_t o = (slot + 1) % block_size;"),
    "copy_k_only": ("memcpy((char *)v_cache + (dst * vs.block + vo) * elem_size,",
                    "if (0) memcpy((char *)v_cache + (dst * vs.block + vo) * elem_size,"),
    "bf16_widen": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = ((uint32_t)h << 16) | 1u;"),
    "e4m3_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "e4m3_ties_up": ("(err == best_err && (c & 1) == 0 && (best & 1) == 1)",
                     "(err == best_err)"),
    "e4m3_no_saturation": ("if (isinf(x)) return (uint8_t)(sign | 0x7E);",
                           "if (isinf(x)) return (uint8_t)(sign | 0x7F);"),
    "fp8_scale_dropped": ("K[i] *= k_scale;", "K[i] *= 1.0;"),
    "fp8_prefill_v_scale": ("V[e] *= v_scale;", "V[e] *= k_scale;"),
    "fp8_write_scale": ("orc_e4m3_encode(vx / v_scale);", "orc_e4m3_encode(vx * v_scale);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    (tmp_path / "oracle.h").write_text(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(lib),
                           str(mutant_c), "-lm"])
    env = dict(os.environ, PA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
