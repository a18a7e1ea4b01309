"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/uq_oracle.c`` (on the CPU, in a
temporary directory), builds it, and runs the oracle pin suites against that build in a
subprocess: at least one pin has to fail.  The real oracle source is never modified."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "uq_oracle.c")

MUTANTS = {
    "e4m3_bias": ("mag = ldexp((double)(8 + m), e - 10);", "mag = ldexp((double)(8 + m), e - 9);"),
    "e4m3_subnormal": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "e2m1_mantissa": ("mag = ldexp((double)(2 + m), e - 2);", "mag = ldexp((double)(1 + m), e - 1);"),
    "nibble_order": ("return uqo_e2m1((d & 1) ? (b >> 4) : (b & 15));",
                     "return uqo_e2m1((d & 1) ? (b & 15) : (b >> 4));"),
    "v_codes_offset": ("const uint8_t* vc = ks + D / 32;", "const uint8_t* vc = ks + D / 16;"),
    "scale_group": ("const int g = d / 32;", "const int g = d / 16;"),
    "rotation_signs": ("acc += q[i] * (double)signs[i] * h;", "acc += q[i] * h;"),
    "rotation_norm": ("out[j] = acc * inv;", "out[j] = acc;"),
    "slot_head_stride": ("const int64_t slot_index = (blk * block_size + t % block_size) * Hk + h;",
                         "const int64_t slot_index = (blk * block_size + t % block_size) + h;"),
    "missing_k_scale": ("s[t] = softmax_scale * k_scale * dot;", "s[t] = softmax_scale * dot;"),
    "missing_v_scale": ("for (int d = 0; d < D; ++d) o[d] = v_scale * o[d] / den;",
                        "for (int d = 0; d < D; ++d) o[d] = o[d] / den;"),
    "partition_map": ("for (int tg = p; (int64_t)tg * UQO_TILE_GROUP < L; tg += P) {\n"
                      "            for (int t = tg * UQO_TILE_GROUP; t < (tg + 1) * UQO_TILE_GROUP && t < L; ++t) {\n"
                      "              any = 1;",
                      "for (int tg = p; (int64_t)tg * UQO_TILE_GROUP < L; tg += 1) {\n"
                      "            for (int t = tg * UQO_TILE_GROUP; t < (tg + 1) * UQO_TILE_GROUP && t < L; ++t) {\n"
                      "              any = 1;"),
    "reduce_weight_sign": ("const double w = part_l[ml] * exp(part_m[ml] - M);",
                           "const double w = part_l[ml] * exp(M - part_m[ml]);"),
    "index_no_causal": ("const int64_t lim = (int64_t)L - QL + j;", "const int64_t lim = (int64_t)L - 1;"),
    "index_scale_group": ("k[d] = e2m1_at(codes, d) * uqo_e4m3(sc[d / 16]);",
                          "k[d] = e2m1_at(codes, d) * uqo_e4m3(sc[d / 32]);"),
    "index_head_stride": ("qv[d] = uqo_e4m3(q[row * q_st + h * q_sh + d]);",
                          "qv[d] = uqo_e4m3(q[row * q_st + d]);"),
    "mtp_no_causal_window": ("const int L = Lseq - QL + 1 + j > 0 ? Lseq - QL + 1 + j : 0;",
                             "const int L = Lseq;"),
    "mtp_query_row": ("const int64_t qrow = (int64_t)b * QL + j;",
                      "const int64_t qrow = (int64_t)b * QL + (QL - 1 - j);"),
    "mtp_reduce_row_map": ("double* o = out + (((int64_t)b * QL + j) * Hk * QG + h * QG + g) * D;",
                           "double* o = out + (((int64_t)b * QL) * Hk * QG + h * QR + r) * D;"),
    "tok_scale_layout": ("const int64_t si = (blk * Hk + h) * block_size + t % block_size;",
                         "const int64_t si = (blk * block_size + t % block_size) * Hk + h;"),
    "tok_scale_kv_swap": ("const double sk = k_tok[si], sv = v_tok[si];",
                          "const double sk = v_tok[si], sv = k_tok[si];"),
    "tok_scale_v_missing": ("V[(size_t)t * D + d] *= sv;", "V[(size_t)t * D + d] *= 1.0;"),
}

PIN_SUITES = ["tests/test_oracle_codecs.py", "tests/test_oracle_attention.py",
              "tests/test_oracle_index.py", "tests/test_oracle_mtp.py",
              "tests/test_oracle_pertoken.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(mutant),
                    "-lm"], check=True)
    env = dict(os.environ, UQ_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_SUITES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 1, f"no pin caught mutant {name}:\n{r.stdout[-2000:]}"
