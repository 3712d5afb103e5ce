"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (on the CPU, in a
temporary directory), builds it, and runs the pin suite against that build
in a subprocess; the suite must fail.  The exhaustive 2^32 comparison is left
out to keep this quick; the fp16 mistakes planted here are caught by the
format-point, underflow and swamping pins as well.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "m_sign": ("float m_new = m_old + m_in;", "float m_new = m_old - m_in;"),
    "beta_swap": ("float m_old = b1 * m[i];", "float m_old = b2 * m[i];"),
    "no_bias_corr_m": ("float m_hat = m_new / bc1;", "float m_hat = m_new;"),
    "no_bias_corr_v": ("float v_hat = v_new / bc2;", "float v_hat = v_new;"),
    "eps_inside_sqrt": ("float root = sqrtf(v_hat);", "float root = sqrtf(v_hat + eps) - eps;"),
    "abs_not_square": ("float g2 = g * g;", "float g2 = fabsf(g);"),
    "w_plus": ("float w_new = w[i] - step;", "float w_new = w[i] + step;"),
    "bias_t_minus_1": ("out[5] = (float)(1.0 - pow(b1, (double)t));",
                       "out[5] = (float)(1.0 - pow(b1, (double)t + 1.0));"),
    "omb1_in_fp32": ("out[2] = (float)(1.0 - b1);", "out[2] = 1.0f - (float)b1;"),
    "v_drops_old": ("float v_new = v_old + v_in;", "float v_new = v_in;"),
    "round_trunc": ("double k = nearbyint(ldexp(a, -q));", "double k = trunc(ldexp(a, -q));"),
    "round_half_up": ("double k = nearbyint(ldexp(a, -q));", "double k = floor(ldexp(a, -q) + 0.5);"),
    "subnormal_quantum": ("if (q < -24)\n        q = -24;", "if (q < -25)\n        q = -25;"),
    "overflow_at_max_finite": ("if (a >= 65520.0)", "if (a > 65504.0)"),
    "layout_floor": ("units = ((unsigned __int128)psi + unit - 1) / unit;",
                     "units = ((unsigned __int128)psi) / unit;"),
    "ledger_stage2": ("case 2: b = 2 * P + 14 * S; break;", "case 2: b = 2 * P + 12 * S; break;"),
    "ledger_stage1": ("case 1: b = 4 * P + 12 * S; break;", "case 1: b = 4 * P + 12 * P; break;"),
    "reduce_divisor": ("const float count = (float)nd;", "const float count = (float)(nd + 1);"),
    "reduce_skip_first": ("for (uint32_t r = 1; r < nd; r++)", "for (uint32_t r = 2; r < nd; r++)"),
    "reduce_reverse": ("float acc = orc_widen(fmt, slices[0][i]);\n"
                       "        for (uint32_t r = 1; r < nd; r++)\n"
                       "            acc = acc + orc_widen(fmt, slices[r][i]);",
                       "float acc = orc_widen(fmt, slices[nd - 1][i]);\n"
                       "        for (uint32_t r = nd - 1; r-- > 0;)\n"
                       "            acc = acc + orc_widen(fmt, slices[r][i]);"),
    "flag_ignores_nan": ("if (!isfinite(g))", "if (isinf(g))"),
    "flag_before_unscale": ("if (!isfinite(g))", "if (!orc_is_finite(fmt, grad16[i]))"),
    "reduce_flag_ignores_nan": ("if (!orc_is_finite(fmt, out[i]))",
                                "if (((out[i] >> 10) & 0x1f) == 31 && (out[i] & 0x3ff) == 0)"),
    "comm_stage3_two_passes": ("uint64_t passes = stage == 3 ? 3 : 2;", "uint64_t passes = 2;"),
    "comm_ring_nd_shards": ("ring = (unsigned __int128)passes * (nd - 1) * lay[1];",
                            "ring = (unsigned __int128)passes * nd * lay[1];"),
    "bf16_round_trunc": ("double quanta = nearbyint(ldexp(a, -q));",
                         "double quanta = trunc(ldexp(a, -q));"),
    "bf16_quantum": ("int q = e - 8;\n    if (q < -133)", "int q = e - 7;\n    if (q < -133)"),
    "bf16_overflow_edge": ("if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))",
                           "if (a > ldexp(2.0 - ldexp(1.0, -7), 127))"),
    "bf16_widen_bias": ("mag = ldexp(128.0 + (double)F, E - 134);",
                        "mag = ldexp(128.0 + (double)F, E - 133);"),
    "bf16_flag_exponent": ("return fmt == ORC_FMT_BF16 ? ((h >> 7) & 0xff) != 255 : orc_f16_is_finite(h);",
                           "return fmt == ORC_FMT_BF16 ? ((h >> 7) & 0xff) != 254 : orc_f16_is_finite(h);"),
    "unscale_divides": ("            g = g * unscale;", "            g = g / unscale;"),
    "unscale_sign": ("ldexp(1.0, -log2_scale)", "ldexp(1.0, log2_scale)"),
    "unscale_dropped": ("        if (scaled)\n            g = g * unscale;\n", ""),
    "unscale_off_by_one": ("ldexp(1.0, -log2_scale)", "ldexp(1.0, -log2_scale - 1)"),
    "gather_reversed": ("full[(uint64_t)r * shard_len + i] = shards[r][i];",
                        "full[(uint64_t)r * shard_len + i] = shards[nd - 1 - r][i];"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not unique"
    c = tmp_path / f"{name}.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
                    "-fno-tree-vectorize", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTANTS[name]
    so = _build(tmp_path, name, old, new)
    env = dict(os.environ, ZERO_ORACLE_LIB=str(so))
    files = [os.path.join(HERE, f) for f in (
        "test_oracle_fp16.py", "test_oracle_ledger_layout.py",
        "test_oracle_adam.py", "test_oracle_reduce.py", "test_oracle_comm.py",
        "test_oracle_bf16.py", "test_oracle_loss_scale.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not every_fp32_pattern", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
