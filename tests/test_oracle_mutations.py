"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that
every one of them fails at least one pin, i.e. the pins can tell."""
import os

import pytest

import oracle
from oracle.build import SRC, build_oracle
from oracle_pins import ALL_PINS

# (name, [(original text, replacement)]) -- each substitution must match exactly once
MUTATIONS = [
    ("drop_decay", [("S[p * N + n] = decay * S[p * N + n] +", "S[p * N + n] = S[p * N + n] +")]),
    ("first_token_not_decayed", [("const double decay = exp(delta * A[h]);",
                                  "const double decay = (t == t0) ? 1.0 : exp(delta * A[h]);")]),
    ("decay_sign", [("exp(delta * A[h])", "exp(-0.01 * delta * A[h])")]),
    ("drop_D", [("yt[p] = acc + (D ? D[h] : 0.0) * xt[p];", "yt[p] = acc;")]),
    ("wrong_group", [("const int64_t g = h / heads_per_group;", "const int64_t g = h % G;")]),
    ("swap_B_C", [("const double *Bt = B + (t * G + g) * N;", "const double *Bt = C + (t * G + g) * N;"),
                  ("const double *Ct = C + (t * G + g) * N;", "const double *Ct = B + (t * G + g) * N;")]),
    ("softplus_as_exp", [("return log1p(exp(u));", "return exp(u);")]),
    ("drop_dt_bias", [("dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0)", "dt[t * H + h]")]),
    ("input_without_delta", [("+ delta * xt[p] * Bt[n]", "+ xt[p] * Bt[n]")]),
    ("transposed_input", [("+ delta * xt[p] * Bt[n]", "+ delta * xt[n % P] * Bt[p % N]")]),
    ("output_uses_previous_C", [("const double *Ct = C + (t * G + g) * N;",
                                 "const double *Ct = C + ((t > t0 ? t - 1 : t) * G + g) * N;")]),
    ("chunk_state_off_by_one", [("if ((local + 1) % chunk_size == 0 || t == t1 - 1) {", "if (local % chunk_size == 0 || t == t1 - 1) {")]),
    ("ignore_has_init", [("init != NULL && (has_init == NULL || has_init[s] != 0);", "init != NULL && (has_init == NULL);")]),
    ("global_chunk_grid", [("t < cu_seqlens[s + 1]; t += chunk_size)",
                            "t < cu_seqlens[s + 1]; t = (t / chunk_size + 1) * chunk_size)")]),
    ("plan_missing_minus_one", [("ncomp) / chunk_size - 1;", "ncomp) / chunk_size;")]),
    ("plan_no_alignment_skip", [("if (ncomp % chunk_size == 0) {", "if (1) {")]),
    ("plan_no_final_block", [("ckpt_src[s * max_blocks + last] = (int32_t)hi;", "")]),
    ("order_tie_break", [("(lu == lv && u < v)", "(lu == lv && u > v)")]),
    # the gated delta rule
    ("gdn_drop_decay", [("                    S[i] *= a;", "                    S[i] *= 1.0;")]),
    ("gdn_write_from_undecayed_state", [("u[c] = b * (vt[c] - hk);", "u[c] = b * (vt[c] - hk / a);")]),
    ("gdn_write_without_beta", [("u[c] = b * (vt[c] - hk);", "u[c] = (vt[c] - hk);")]),
    ("gdn_beta_on_value_only", [("u[c] = b * (vt[c] - hk);", "u[c] = b * vt[c] - hk;")]),
    ("gdn_output_before_write", [("acc += S[c * dk + r] * qt[r];", "acc += (S[c * dk + r] - kt[r] * u[c]) * qt[r];")]),
    ("gdn_wrong_key_group", [("const int64_t g = hd / (H / G);\n            double *S",
                              "const int64_t g = hd % G;\n            double *S")]),
    ("gdn_read_with_key", [("acc += S[c * dk + r] * qt[r];", "acc += S[c * dk + r] * kt[r];")]),
    ("gdn_no_scale", [("ot[c] = scale * acc;", "ot[c] = acc;")]),
    ("gdn_chunk_state_off_by_one", [(
        "((local + 1) % chunk_size == 0 || t == t1 - 1)) {\n                    const int64_t c = chunk_base[s]",
        "(local % chunk_size == 0 || t == t1 - 1)) {\n                    const int64_t c = chunk_base[s]")]),
    # the scheduler's prefill bites
    ("bites_no_realign_on_final_bite", [("if (start % align != 0 && next <= last_aligned) {",
                                         "if (start % align != 0 && end < last_aligned) {")]),
    ("bites_clip_up", [("end = end / align * align;", "end = (end + align - 1) / align * align;")]),
    ("bites_realign_one_boundary_late", [("if (next < end)\n                end = next;",
                                          "if (next + align < end)\n                end = next + align;")]),
    ("bites_ignore_budget", [("int64_t end = start + budget[s] < len ? start + budget[s] : len;",
                              "int64_t end = len;")]),
    # the decode step with dual state anchors
    ("decode_drop_decay", [("hs[p * N + n] = decay * hs[p * N + n] + delta * xs[p] * Bs[n];",
                            "hs[p * N + n] = hs[p * N + n] + delta * xs[p] * Bs[n];")]),
    ("decode_y_from_entering_state", [(
        "hs[p * N + n] = decay * hs[p * N + n] + delta * xs[p] * Bs[n];\n                    acc += Cs[n] * hs[p * N + n];",
        "acc += Cs[n] * hs[p * N + n];\n                    hs[p * N + n] = decay * hs[p * N + n] + delta * xs[p] * Bs[n];")]),
    ("decode_read_slot_ignored", [("if (r >= 0)\n            memcpy(h_in", "if (0)\n            memcpy(h_in")]),
    ("decode_writes_read_anchor", [("memcpy(state_cache + (int64_t)w * per_state",
                                    "memcpy(state_cache + (int64_t)(r >= 0 ? r : w) * per_state")]),
    ("decode_wrong_group", [("const int64_t g = hd / (H / G);\n            const double delta", "const int64_t g = hd % G;\n            const double delta")]),
    ("decode_no_bias", [("dt[s * H + hd] + (dt_bias ? dt_bias[hd] : 0.0)", "dt[s * H + hd]")]),
    ("decode_drop_D", [("(D ? D[hd] : 0.0) * xs[p]", "0.0 * xs[p]")]),
    ("decode_bad_slot_not_refused", [("            bad = 1;", "            bad = 0;")]),
    # the varlen causal conv1d
    ("conv_taps_reversed", [("z += weight[c * W + k] * u;", "z += weight[c * W + (W - 1 - k)] * u;")]),
    ("conv_no_bias", [("double z = bias ? bias[c] : 0.0;", "double z = 0.0;")]),
    ("conv_silu_sign", [("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))")]),
    ("conv_cached_rows_ignored", [("if (r >= 0 && per_slot > 0)", "if (0 && per_slot > 0)")]),
    ("conv_leaks_previous_sequence", [(
        "const double u = jj >= 0 ? x[(t0 + jj) * Cn + c] : ps[(W - 1 + jj) * Cn + c];",
        "const double u = t0 + jj >= 0 ? x[(t0 + jj) * Cn + c] : ps[(W - 1 + jj) * Cn + c];")]),
    ("conv_state_rows_reversed", [("conv_states[(int64_t)w * per_slot + i * Cn + c] =",
                                   "conv_states[(int64_t)w * per_slot + (W - 2 - i) * Cn + c] =")]),
    ("conv_bad_slot_not_refused", [("bad |= 1;", "bad |= 0;")]),
]


@pytest.mark.parametrize("name,subs", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, subs, tmp_path):
    with open(SRC) as f:
        text = f.read()
    for old, new in subs:
        assert text.count(old) == 1, f"mutation {name}: pattern not unique: {old!r}"
        text = text.replace(old, new)
    src = os.path.join(tmp_path, f"oracle_{name}.c")
    with open(src, "w") as f:
        f.write(text)
    lib = oracle.load(build_oracle(out=os.path.join(tmp_path, f"liboracle_{name}.so"), src=src,
                                   werror=False))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
