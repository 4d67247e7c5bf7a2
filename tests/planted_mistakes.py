"""Planted mistakes in the CPU oracle: each one must fail at least one pin.

Run by hand (not collected by pytest; a few minutes on 4 cores):

    python tests/planted_mistakes.py

(The output of its last run is kept in tests/planted_mistakes_result.txt.)

For every mistake below, a copy of oracle/ with that one change in
moe_oracle.c is built in a temporary directory and the oracle's pin tests
(-m "not gpu") are run against it.  A mistake "survives" when every pin test
still passes; the script then exits with status 1.  The mistakes are the
plausible slips of each part: a tie rule turned round, a renormalised or
single-precision softmax, an off-by-one capacity, a transposed slot index,
slots in the wrong token order, capped counts, inclusive offsets, the E4M3
encoder's rounding, saturation, subnormals and bias, a signed block maximum,
a wrong zero-block scale, a reciprocal-multiply scale, combine's order, an
unfused multiply-add, dropped pairs kept, a -0 start, bf16 truncation or
ties away, the group-limited router's scoring and group choice, and the
RMSNorm epilogue's residual add, mean, eps, gamma and rounding.  Changes
that compute the same values (an fp32 sum of two floats formed in double
and rounded once, say) are not mistakes and are not listed.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "moe_oracle.c")).read()
CORE_TESTS = ["tests/test_oracle_route.py", "tests/test_oracle_dispatch.py", "tests/test_oracle_packed.py",
              "tests/test_oracle_fp8.py", "tests/test_oracle_combine.py", "tests/test_oracle_sizes.py"]
GROUPED_TESTS = ["tests/test_oracle_route_grouped.py"]

Z = '''        for (int32_t e = 0; e < E; ++e)
            z += exp((double)row[e] - mx);
        for (int32_t j = 0; j < k; ++j)
            w[t * k + j] = (float)(exp((double)row[idx[t * k + j]] - mx) / z);'''
CORE = {
  'route_ties_to_higher': ('if (best < 0 || row[e] > row[best])   /* strict', 'if (best < 0 || row[e] >= row[best])   /* strict'),
  'route_smallest_first': ('if (best < 0 || row[e] > row[best])   /* strict', 'if (best < 0 || row[e] < row[best])   /* strict'),
  'route_renormalise_topk': (Z, Z.replace('for (int32_t e = 0; e < E; ++e)\n            z += exp((double)row[e] - mx);',
                                        'for (int32_t e = 0; e < k; ++e)\n            z += exp((double)row[idx[t * k + e]] - mx);')),
  'route_weights_in_float': (Z, Z.replace('(float)(exp((double)row[idx[t * k + j]] - mx) / z)',
                                        '(float)((float)expf(row[idx[t * k + j]] - (float)mx) / (float)z)')),
  'slots_capacity_one_short': ('            if (r < C) {\n                int64_t s', '            if (r <= C - 2) {\n                int64_t s'),
  'slots_descending_tokens': ('    for (int64_t t = 0; t < T; ++t) {\n        for (int32_t j = 0; j < k; ++j) {\n            int32_t e = idx[t * k + j];\n            if (e < 0 || e >= E) {\n                free(fill);',
                              '    for (int64_t t = T - 1; t >= 0; --t) {\n        for (int32_t j = 0; j < k; ++j) {\n            int32_t e = idx[t * k + j];\n            if (e < 0 || e >= E) {\n                free(fill);'),
  'slots_transposed_index': ('                int64_t s = (int64_t)e * C + r;\n                recv_src[s] = (int32_t)t;',
                             '                int64_t s = (int64_t)r * E + e;\n                recv_src[s] = (int32_t)t;'),
  'counts_capped_at_C': ('counts[e] = (int32_t)fill[e];', 'counts[e] = (int32_t)(fill[e] < C ? fill[e] : C);'),
  'packed_inclusive_offsets': ('        offsets[e] = (int32_t)run;\n        run += count[e];', '        run += count[e];\n        offsets[e] = (int32_t)run;'),
  'fp8_scale_reciprocal_mul': ('amax / 448.0f;', 'amax * (1.0f / 448.0f);'),
  'fp8_zero_block_scale_0': ('(amax == 0.0f) ? 1.0f :', '(amax == 0.0f) ? 0.0f :'),
  'fp8_rows_scale_stride': ('codes + r * H, scales + r * (H / 128));', 'codes + r * H, scales + r);'),
  'fp8_rows_code_stride': ('codes + r * H, scales + r * (H / 128));', 'codes + r * 128, scales + r * (H / 128));'),
  'fp8_amax_signed': ('float a = fabsf(bf16_bits_to_float(x[b * 128 + i]));', 'float a = bf16_bits_to_float(x[b * 128 + i]);'),
  'e4m3_no_saturation': ('    if (a > 448.0)\n        return (uint8_t)(sign | 0x7E);', '    if (a > 464.0)\n        return (uint8_t)(sign | 0x7F);'),
  'e4m3_ties_away': ('double m = rint(ldexp(a, 3 - e));', 'double m = floor(ldexp(a, 3 - e) + 0.5);'),
  'e4m3_subnormal_truncate': ('double units = rint(ldexp(a, 9));', 'double units = floor(ldexp(a, 9));'),
  'e4m3_bias_8': ('int code = ((e + 7) << 3)', 'int code = ((e + 8) << 3)'),
  'combine_reverse_order': ('            for (int32_t j = 0; j < k; ++j) {\n                if (token_slot[t * k + j] < 0)',
                            '            for (int32_t j = k - 1; j >= 0; --j) {\n                if (token_slot[t * k + j] < 0)'),
  'combine_unfused': ('acc = fmaf(w[t * k + j], y, acc);', 'acc = w[t * k + j] * y + acc;'),
  'combine_keeps_dropped': ('                if (token_slot[t * k + j] < 0)\n                    continue;\n                float y', '                float y'),
  'combine_starts_at_neg0': ('            float acc = 0.0f;\n            for (int32_t j = 0; j < k; ++j) {\n                if (token_slot',
                             '            float acc = -0.0f;\n            for (int32_t j = 0; j < k; ++j) {\n                if (token_slot'),
  'bf16_round_truncate': ('return (uint16_t)((u + 0x7FFFu + lsb) >> 16);', 'return (uint16_t)(u >> 16);'),
  'bf16_round_ties_up': ('return (uint16_t)((u + 0x7FFFu + lsb) >> 16);', 'return (uint16_t)((u + 0x8000u) >> 16);'),
}
GROUPED = {
  'top1_only': ('score[g] = a + b;', 'score[g] = a;'),
  'keep_worst': ('if (!kept[g] && (best < 0 || score[g] > score[best]))', 'if (!kept[g] && (best < 0 || score[g] < score[best]))'),
  'tie_high': ('if (!kept[g] && (best < 0 || score[g] > score[best]))', 'if (!kept[g] && (best < 0 || score[g] >= score[best]))'),
  'b2_includes_b1': ('if (e != b1 && (b2 < 0 || row[e] > row[b2]))', 'if ((b2 < 0 || row[e] > row[b2]))'),
  'group_stride': ('taken[e] = kept[e / gs] ? 0 : 1;', 'taken[e] = kept[e % G] ? 0 : 1;'),
}

NORM = {
    "sum_rounded_before_residual": ("r[h] = acc + bf16_bits_to_float(residual[t * H + h]);",
                                    "r[h] = bf16_bits_to_float(oracle_bf16_round(acc)) + "
                                    "bf16_bits_to_float(residual[t * H + h]);"),
    "mean_over_H_minus_1": ("sqrt(ss / H + (double)eps)", "sqrt(ss / (H - 1 > 0 ? H - 1 : 1) + (double)eps)"),
    "eps_outside_root": ("1.0 / sqrt(ss / H + (double)eps)", "1.0 / (sqrt(ss / H) + (double)eps)"),
    "no_gamma": ("(double)r[h] * inv * (double)bf16_bits_to_float(gamma[h])", "(double)r[h] * inv"),
    "double_rounding_via_float": ("bf16_round_double((double)r[h] * inv * (double)bf16_bits_to_float(gamma[h]))",
                                  "oracle_bf16_round((float)((double)r[h] * inv * "
                                  "(double)bf16_bits_to_float(gamma[h])))"),
    "squares_of_rounded_residual": ("ss += (double)r[h] * (double)r[h];",
                                    "ss += (double)bf16_bits_to_float(residual_out[t * H + h]) * "
                                    "(double)bf16_bits_to_float(residual_out[t * H + h]);"),
}
NORM_TESTS = ["tests/test_oracle_combine_norm.py"]


def run(job):
    name, (old, new), tests, tmp = job
    if SRC.count(old) < 1:
        return name, "NOT APPLIED", "the text to change is missing from moe_oracle.c"
    d = os.path.join(tmp, name)
    os.makedirs(os.path.join(d, "oracle"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(d, "oracle", "__init__.py"))
    with open(os.path.join(d, "oracle", "moe_oracle.c"), "w") as f:
        f.write(SRC.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(ROOT, t) for t in tests]],
                       capture_output=True, text=True, cwd=d, timeout=1800,
                       env={**os.environ, "PYTHONPATH": d + os.pathsep + ROOT})
    if not glob.glob(os.path.join(d, "oracle", "*.so")):
        return name, "NOT BUILT", (r.stdout + r.stderr)[-200:]
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    return name, ("killed" if r.returncode else "SURVIVED"), (failed[0] if failed else "")


def main() -> int:
    with tempfile.TemporaryDirectory(prefix="planted_") as tmp:
        jobs = [(n, m, CORE_TESTS, tmp) for n, m in CORE.items()]
        jobs += [(f"grouped_{n}", m, GROUPED_TESTS, tmp) for n, m in GROUPED.items()]
        jobs += [(f"norm_{n}", m, NORM_TESTS, tmp) for n, m in NORM.items()]
        bad = 0
        with ThreadPoolExecutor(4) as ex:
            for name, outcome, detail in ex.map(run, jobs):
                print(f"{name:36s} {outcome:10s} {detail[:100]}", flush=True)
                bad += outcome != "killed"
    print(f"{len(jobs) - bad} of {len(jobs)} planted mistakes fail a pin")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
