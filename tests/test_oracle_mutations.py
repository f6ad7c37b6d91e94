"""The pins catch plausible mistakes in the oracle (CPU only).

Each case copies oracle.c into a temporary directory, plants one mistake (a
dropped term, a wrong index or operand, an off-by-one, the other reading of
an open point), builds it with gcc and runs the pin suite against it in a
subprocess.  The suite must fail for every mutant.  Nothing here touches the
GPU or the real oracle build.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "maxvio_drops_minus_one": ("*maxvio = (float)(ratio - 1.0);", "*maxvio = (float)(ratio);"),
    "maxvio_wrong_operand": ("(double)((int64_t)tmax * E)", "(double)((int64_t)tmax * R)"),
    "count_drops_last_entry": ("for (int64_t n = 0; n < NK; ++n) {\n        const int32_t e = topk[n];\n        if (e < 0 || e >= E)\n            return ORC_ERR_EXPERT_ID;",
                               "for (int64_t n = 0; n + 1 < NK; ++n) {\n        const int32_t e = topk[n];\n        if (e < 0 || e >= E)\n            return ORC_ERR_EXPERT_ID;"),
    "spill_highest_id_first": ("for (int32_t e = r * L; e < (r + 1) * L; ++e) {\n                const int32_t give",
                               "for (int32_t e = (r + 1) * L - 1; e >= r * L; --e) {\n                const int32_t give"),
    "largest_first_ties_to_higher_id": ("(best < 0 || T[e] > T[best])", "(best < 0 || T[e] >= T[best])"),
    "largest_first_takes_smallest": ("(best < 0 || T[e] > T[best])", "(best < 0 || T[e] < T[best])"),
    "largest_first_spills_whole_expert": ("const int32_t give = T[best] < excess ? T[best] : excess;",
                                          "const int32_t give = T[best];"),
    "deficit_includes_full_ranks": ("if (p->load[r] < C) {\n            df_r[nd]", "if (p->load[r] <= C) {\n            df_r[nd]"),
    "spill_off_from_remainder": ("p->rep_spill_off[nrep] = sp_amt[i] - rem_s;", "p->rep_spill_off[nrep] = rem_s;"),
    "tie_advances_one_pointer": ("        if (rem_d == 0) {\n            ++j;", "        else if (rem_d == 0) {\n            ++j;"),
    "home_rows_sized_by_count": ("row += p->keep[e];", "row += T[e];"),
    "keep_boundary_off_by_one": ("if (pos < p->keep[e]) {", "if (pos <= p->keep[e]) {"),
    "replica_row_ignores_spill_off": ("row = p->rep_row_off[found] + (q - p->rep_spill_off[found]);",
                                      "row = p->rep_row_off[found] + q;"),
    "dispatch_wrong_token": ("const int64_t tok = n / K;\n        for (int32_t h = 0; h < H; ++h)\n            buf",
                             "const int64_t tok = n % (NK / K);\n        for (int32_t h = 0; h < H; ++h)\n            buf"),
    "expert_wrong_scale": ("const float s = scale[row_expert[r]];", "const float s = scale[r % 2];"),
    "combine_first_gate_only": ("acc += (double)gates[n] * orc_bf16_to_double(out",
                                "acc += (double)gates[t * K] * orc_bf16_to_double(out"),
    "bf16_truncates": ("double r = rint(ldexp(d, -qexp));", "double r = trunc(ldexp(d, -qexp));"),
    "bf16_one_bit_short": ("int qexp = (ex < -125 ? -125 : ex) - 8;", "int qexp = (ex < -125 ? -125 : ex) - 7;"),
    "bwd_dot_wrong_slot": ("dot += g * orc_bf16_to_double(out[row * H + h]);",
                           "dot += g * orc_bf16_to_double(out[(int64_t)slot_of[t * K] * H + h]);"),
    "bwd_dout_first_gate": ("orc_bf16_from_double((double)gates[n] * g);",
                            "orc_bf16_from_double((double)gates[t * K] * g);"),
    "dispatch_bwd_drops_last_k": ("            for (int32_t k = 0; k < K; ++k)\n                acc += orc_bf16_to_double(d_buf",
                                  "            for (int32_t k = 0; k + 1 < K; ++k)\n                acc += orc_bf16_to_double(d_buf"),
    "dispatch_bwd_ignores_slot": ("acc += orc_bf16_to_double(d_buf[(int64_t)slot_of[t * K + k] * H + h]);",
                                  "acc += orc_bf16_to_double(d_buf[(int64_t)(t * K + k) * H + h]);"),
    "weight_slot_ignores_rank_base": ("wslot[j] = d * B + b;", "wslot[j] = b;"),
    "weight_slot_cap_off_by_one": ("            if (b < B)\n                wslot[j]", "            if (b <= B)\n                wslot[j]"),
    "weight_slot_counts_other_ranks": ("            if (p->rep_host[j] != d)\n                continue;",
                                       "            if (p->rep_host[j] != d && ++b)\n                continue;"),
    "prefetch_wrong_source": ("w_home + (int64_t)p->rep_expert[j] * wbytes", "w_home + (int64_t)p->rep_host[j] * wbytes"),
    "gemm_ignores_wslot": ("w = wslot[j] >= 0 ? pool", "w = wslot[j] < -1 ? pool"),
    "gemm_transposed_weight": ("acc += orc_bf16_to_double(xr[k]) * orc_bf16_to_double(wn[k]);",
                               "acc += orc_bf16_to_double(xr[k]) * orc_bf16_to_double(w[w_offset + (int64_t)k * out_dim + n]);"),
    "gemm_ignores_offset": ("const uint16_t *wn = w + w_offset + (int64_t)n * in_dim;",
                            "const uint16_t *wn = w + (int64_t)n * in_dim;"),
    "gemm_drops_last_k": ("for (int32_t k = 0; k < in_dim; ++k)\n                    acc",
                          "for (int32_t k = 0; k + 1 < in_dim; ++k)\n                    acc"),
    "gemm_home_range_off_by_one": ("local < p->home_row_off[e] + p->keep[e])\n                w = w_home",
                                   "local <= p->home_row_off[e] + p->keep[e])\n                w = w_home"),
    "reduce_skips_home": ("double acc = (double)home[(int64_t)e * G + i];\n            for (int32_t q",
                          "double acc = 0.0;\n            for (int32_t q"),
    "reduce_keeps_replicas": ("rep[(int64_t)q * G + i] = 0.0f;", "rep[(int64_t)q * G + i] = rep[(int64_t)q * G + i];"),
    "reduce_misses_last_replica": ("for (int32_t q = p->rep_first[e]; q < p->rep_first[e] + p->rep_cnt[e]; ++q)\n                acc += (double)rep[(int64_t)q * G + i];",
                                   "for (int32_t q = p->rep_first[e]; q + 1 < p->rep_first[e] + p->rep_cnt[e]; ++q)\n                acc += (double)rep[(int64_t)q * G + i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    oracle.build(src=str(mut), out=lib)
    env = dict(os.environ, MOONEP_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
