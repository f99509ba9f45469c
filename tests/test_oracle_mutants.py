"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of oracle/mxref.c (on the CPU,
in a temporary directory), builds it, and runs tests/test_oracle.py (tests/test_oracle_routing.py for
the dispatch and combine functions) against that build in a subprocess: the
pins must fail.  The oracle itself is never
modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxref.c")

MUTANTS = {
    "scale_offset_7": ("int shared = (e - 1) - 8;", "int shared = (e - 1) - 7;"),
    "no_lower_clamp": ("if (shared < -127) shared = -127;", ""),
    "ties_away": ("code = ((E + 7) << 3) + (n - 8);", "code = ((E + 7) << 3) + ((int)round(ldexp(a, 3 - E)) - 8);"),
    "no_saturation": ("if (a > 448.0) a = 448.0;", ""),
    "unsigned_zero": ("return (uint8_t)(code | (neg << 7));", "return (uint8_t)(code | ((neg && code) << 7));"),
    "subnormal_threshold": ("if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {"),
    "bf16_subnormal_exp": ("v = ldexp((double)fr, -126 - 7);", "v = ldexp((double)fr, -126 - 8);"),
    "dequant_bias": ("return ldexp(mxref_e4m3_value(q), (int)S - 127);", "return ldexp(mxref_e4m3_value(q), (int)S - 128);"),
    "cols_pad_128": ("P[g + 1] = P[g] + 256 * ((mg + 255) / 256);", "P[g + 1] = P[g] + 128 * ((mg + 127) / 128);"),
    "pack_byte": ("int64_t byte = (b % 8) / 2;", "int64_t byte = (b % 4);"),
    "pack_lane": ("int64_t lane = 32 * (b % 2) + (r % 32);", "int64_t lane = 32 * ((b / 2) % 2) + (r % 32);"),
    "gemm_scale_index": ("acc += mxref_dequant(xr[k], xs[k / 32]) * mxref_dequant(wr[k], ws[k / 32]);",
                         "acc += mxref_dequant(xr[k], xs[k / 32]) * mxref_dequant(wr[k], ws[(k + 1) / 32]);"),
    "wgrad_skip_first": ("for (int64_t t = P[g]; t < P[g + 1]; ++t)", "for (int64_t t = P[g] + 1; t < P[g + 1]; ++t)"),
    "e4m3_bias": ("else v = ldexp((double)(8 + fr), ef - 7 - 3);", "else v = ldexp((double)(8 + fr), ef - 8 - 3);"),
    "silu_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "swiglu_roles": ("for (int64_t i = 0; i < M * I; ++i) h[i] = mxref_silu(gate[i]) * up[i];",
                     "for (int64_t i = 0; i < M * I; ++i) h[i] = mxref_silu(up[i]) * gate[i];"),
    "bwd_h_roles": ("        h[i] = mxref_silu(gate[i]) * up[i];", "        h[i] = mxref_silu(up[i]) * gate[i];"),
    "f64_signed_amax": ("if (fabs(x[i]) > amax) amax = fabs(x[i]);", "if (x[i] > amax) amax = x[i];"),
    "f64_scale_direction": ("q[i] = mxref_e4m3_encode(ldexp(x[i], 127 - (int)S));",
                            "q[i] = mxref_e4m3_encode(ldexp(x[i], (int)S - 127));"),
    "f64_block_stride": ("const double* blk = x + m * K + b * 32;", "const double* blk = x + m * K + b * 31;"),
    "dsilu_missing_term": ("return sig * (1.0 + x * (1.0 - sig));", "return sig * (1.0 + x * sig);"),
    "bwd_dup_uses_dsilu": ("dup[i] = dh[i] * mxref_silu(gate[i]);", "dup[i] = dh[i] * mxref_dsilu(gate[i]);"),
    "bwd_dgate_no_up": ("dgate[i] = dh[i] * up[i] * mxref_dsilu(gate[i]);", "dgate[i] = dh[i] * mxref_dsilu(gate[i]);"),
    "bf16_round_truncates": ("double n = nearbyint(ldexp(a, 7 - E));", "double n = floor(ldexp(a, 7 - E));"),
    "bf16_subnormal_quantum": ("int n = (int)nearbyint(ldexp(a, 133));", "int n = (int)nearbyint(ldexp(a, 134));"),
    # dispatch and combine (pinned in tests/test_oracle_routing.py)
    "plan_unstable": ("    for (int64_t j = 0; j < n; ++j) {\n        const int32_t e = experts[j];\n        if (e < 0 || e >= G) {",
                      "    for (int64_t j = n - 1; j >= 0; --j) {\n        const int32_t e = experts[j];\n        if (e < 0 || e >= G) {"),
    "plan_keeps_last_expert_id": ("        if (e < 0 || e >= G) {\n            slot_of[j] = -1;",
                                  "        if (e < 0 || e > G) {\n            slot_of[j] = -1;"),
    "f32_subnormal_quantum": ("if (E < -126) return copysign(ldexp(nearbyint(ldexp(a, 149)), -149), x);",
                              "if (E < -126) return copysign(ldexp(nearbyint(ldexp(a, 150)), -150), x);"),
    "gather_single_rounding": ("o[c] = mxref_bf16_round(mxref_f32_round(p));", "o[c] = mxref_bf16_round(p);"),
    "combine_ignores_weights": ("acc += (w ? (double)w[t * k + j] : 1.0) * mxref_bf16_value(y[(int64_t)slot * N + c]);",
                                "acc += mxref_bf16_value(y[(int64_t)slot * N + c]);"),
}
ROUTING = {"plan_unstable", "plan_keeps_last_expert_id", "f32_subnormal_quantum", "gather_single_rounding",
           "combine_ignores_weights"}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mxref.c")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        with open(os.path.join(d, "mxref.h"), "w") as f:
            f.write(open(os.path.join(ROOT, "oracle", "mxref.h")).read())
        so = os.path.join(d, "libmxref_mutant.so")
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", c, "-o", so, "-lm"])
        env = dict(os.environ, MXREF_LIB=so)
        pins = "test_oracle_routing.py" if name in ROUTING else "test_oracle.py"
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", pins)],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"mutant {name} survived the oracle pins"
