"""The oracle pins must fail on a broken oracle.

Each case plants one plausible mistake in a copy of oracle.c (CPU only),
builds it, and runs the pin suite against it; the suite has to fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "no_gdn_decay": ("S[e] *= alpha;", "S[e] *= 1.0;"),
    "delta_sign": ("const double c = bb * (vv[i] - u);",
                   "const double c = bb * (u - vv[i]);"),
    "lightning_outer_transposed": (
        "lam * S[(size_t)i * K + j] + vv[i] * kv[j];",
        "lam * S[(size_t)i * K + j] + vv[j % V] * kv[i % K];"),
    "gva_head_map": ("const int h = hv / group;", "const int h = hv % H;"),
    "kda_decay_on_rows": ("S[(size_t)i * K + j] *= ek[j];",
                          "S[(size_t)i * K + j] *= ek[i % K];"),
    "write_to_read_slot": (
        "memcpy(pool_out + ((size_t)w * HV + hv) * tile, S,",
        "memcpy(pool_out + ((size_t)r * HV + hv) * tile, S,"),
    "lightning_decay_index": ("pow(2.0, -8.0 * (double)(head + 1)",
                              "pow(2.0, -8.0 * (double)(head)"),
    "padded_output_not_zeroed": (
        "out[((tok0 + t) * HV + hv) * V + i] = 0.0;", ";"),
    "beta_sigmoid_missing": ("bb = 1.0 / (1.0 + exp(-bb));", "bb = bb;"),
    "output_reads_key": ("o += S[(size_t)i * K + j] * qv[j];",
                         "o += S[(size_t)i * K + j] * kv[j];"),
    "readout_before_decay": (
        "u += S[(size_t)i * K + j] * kv[j];",
        "u += S[(size_t)i * K + j] / (variant == ORACLE_GDN ? exp(g[bt]) "
        ": exp(g[bt * (size_t)K + j])) * kv[j];"),
    "l2norm_skipped_for_k": ("l2_normalise(kv, K);", ";"),
    "paged_seed_off_by_one": (
        "? slots[(size_t)b * slots_stride + na - 1]",
        "? slots[(size_t)b * slots_stride + na % T]"),
    "replay_decay_after_update": (
        "S[(size_t)i * K + j] * a[j] + err[i] * kk[j];",
        "(S[(size_t)i * K + j] + err[i] * kk[j]) * a[j];"),
    "factor_err_missing_beta": ("rec[2 * K + i] = c;",
                                "rec[2 * K + i] = vv[i] - u;"),
    "paged_write_wrong_token": (
        "const int ws = slots[(size_t)b * slots_stride + t];",
        "const int ws = slots[(size_t)b * slots_stride + T - 1 - t];"),
    "varlen_token_base_ignored": (
        "const size_t tok0 = cu_seqlens ? (size_t)cu_seqlens[b] : (size_t)b * T;",
        "const size_t tok0 = (size_t)b * T;"),
    "varlen_accepted_bound_is_T": ("(na >= 1 && na <= Tb)",
                                   "(na >= 1 && na <= T)"),
    "varlen_replay_dense_records": (
        "const double *rec = factors + ((tok0 + t) * HV + hv) * rsz;",
        "const double *rec = factors + (((size_t)b * T + t) * HV + hv) * rsz;"),
    "gate_softplus_sign": ("return -exp(a_log) * log1p(exp(z));",
                           "return exp(a_log) * log1p(exp(z));"),
    "gate_softplus_missing_a_log": ("return -exp(a_log) * log1p(exp(z));",
                                    "return -log1p(exp(z));"),
    "gate_sigmoid_scale_outside": (
        "return lower_bound / (1.0 + exp(-exp(a_log) * z));",
        "return lower_bound * exp(a_log) / (1.0 + exp(-z));"),
    "gate_kda_dt_bias_transposed": ("dt_bias[(size_t)hv * K + j],",
                                    "dt_bias[(size_t)j * HV + hv],"),
    "read_slot_is_batch_position": (
        "            r = read_idx[b];\n            w = write_idx",
        "            r = read_idx[b] < 0 ? -1 : b;\n            w = write_idx"),
    "state_restarts_each_token": (
        "            for (int t = 0; t < Tb; ++t) {\n                const size_t qk_off",
        "            for (int t = 0; t < Tb; ++t) {\n                memcpy(S, pool_in + "
        "((size_t)r * HV + hv) * tile, tile * sizeof(double));\n"
        "                const size_t qk_off"),
    "varlen_empty_request_skips_write": (
        "            if (w >= 0)\n                memcpy(pool_out + ((size_t)w * HV + hv) * tile, S,",
        "            if (w >= 0 && Tb > 0)\n                memcpy(pool_out + ((size_t)w * HV + hv) * tile, S,"),
}


# Indexing mistakes that the property tests over random shapes and slot
# assignments (test_oracle_properties.py) must catch on their own.
PROPERTY_MUTATIONS = ["gva_head_map", "padded_output_not_zeroed",
                      "write_to_read_slot", "read_slot_is_batch_position",
                      "state_restarts_each_token"]


def _run_against_mutant(name, tmp_path, test_file):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: " + old
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new, 1))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o",
                    str(lib), str(src), "-lm"], check=True)
    env = dict(os.environ, LA_ORACLE_LIB=str(lib))
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", test_file)],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    proc = _run_against_mutant(name, tmp_path, "test_oracle_pins.py")
    assert proc.returncode != 0, "pins did not catch " + name


@pytest.mark.parametrize("name", PROPERTY_MUTATIONS)
def test_properties_catch_planted_indexing_mistake(name, tmp_path):
    proc = _run_against_mutant(name, tmp_path, "test_oracle_properties.py")
    assert proc.returncode != 0, "properties did not catch " + name
