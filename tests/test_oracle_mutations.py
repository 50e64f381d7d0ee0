"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them: a dropped term, a wrong sign, index or axis,
an off-by-one in the causal rule, the wrong tie rule, a skipped rounding."""
import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "kpool_oracle.py")

MUTATIONS = {
    "ape_dropped": ("a = gs + ape[None, :, :]", "a = gs + 0 * ape[None, :, :]"),
    "ape_slots_reversed": ("a = gs + ape[None, :, :]", "a = gs + ape[None, ::-1, :]"),
    "softmax_over_dims": ("pi = e / Z[:, None, :]", "pi = e / e.sum(axis=2, keepdims=True)"),
    "softmax_unnormalised": ("pi = e / Z[:, None, :]", "pi = e"),
    "no_bf16_rounding_of_pool": ("pooled[int(cuP[b]):int(cuP[b]) + n] = bf16_round(acc)",
                                 "pooled[int(cuP[b]):int(cuP[b]) + n] = acc"),
    "pool_key_from_wrong_slot": ("acc = acc + pi[:, s, :] * ks[:, s, :]",
                                 "acc = acc + pi[:, s, :] * ks[:, 0, :]"),
    "scale_dropped": ("w_t[h] * np.maximum(F32(0.0), sc * dots[h])",
                      "w_t[h] * np.maximum(F32(0.0), dots[h])"),
    "w_inside_relu": ("w_t[h] * np.maximum(F32(0.0), sc * dots[h])",
                      "np.maximum(F32(0.0), w_t[h] * sc * dots[h])"),
    "relu_dropped": ("w_t[h] * np.maximum(F32(0.0), sc * dots[h])", "w_t[h] * (sc * dots[h])"),
    "head_weight_index": ("w_t[h] * np.maximum(F32(0.0), sc * dots[h])",
                          "w_t[0] * np.maximum(F32(0.0), sc * dots[h])"),
    "causal_off_by_one_more": ("return (i + 1) // kpool", "return (i + 2) // kpool"),
    "causal_off_by_one_less": ("return (i + 1) // kpool", "return i // kpool"),
    "tail_too_short": ("row.extend(range(int(cu[b]) + n_c * kpool, t + 1))",
                       "row.extend(range(int(cu[b]) + n_c * kpool, t))"),
    "tail_ignores_doc_start": ("row.extend(range(int(cu[b]) + n_c * kpool, t + 1))",
                               "row.extend(range(n_c * kpool, t + 1))"),
    "ties_to_higher_index": ("np.lexsort((np.arange(n), -s))", "np.lexsort((-np.arange(n), -s))"),
    "selects_smallest": ("np.lexsort((np.arange(n), -s))", "np.lexsort((np.arange(n), s))"),
    "nan_not_demoted": ("s = np.where(np.isnan(s), F32(-np.inf), s)", "s = s"),
    "pool_id_not_doc_relative": ("p = int(gid) - int(cuP[b])", "p = int(gid)"),
    "pools_ceil_per_doc": ("counts = (cu[1:] - cu[:-1]) // kpool",
                           "counts = -(-(cu[1:] - cu[:-1]) // kpool)"),
    "keys_not_doc_offset": ("keys = keys_all[int(cuP[b]):int(cuP[b]) + n_c]",
                            "keys = keys_all[:n_c]"),
    "doc_of_left": ('np.searchsorted(cu, t, side="right") - 1', 'np.searchsorted(cu, t, side="left") - 1'),
    "fwht_sign": ("np.stack([a + b, a - b], axis=2)", "np.stack([a + b, b - a], axis=2)"),
    "fwht_not_normalised": ("fwht128(x) * F32(1.0 / np.sqrt(128.0))", "fwht128(x) * F32(1.0 / 128.0)"),
    "fwht_no_bf16": ("y = bf16_round(fwht128(x) * F32(1.0 / np.sqrt(128.0)))",
                     "y = (fwht128(x) * F32(1.0 / np.sqrt(128.0)))"),
    "fp8_fnuz_max": ("while amax > np.ldexp(448.0, e):\n        e += 1\n    while amax <= np.ldexp(448.0, e - 1):",
                     "while amax > np.ldexp(240.0, e):\n        e += 1\n    while amax <= np.ldexp(240.0, e - 1):"),
    "e4m3_truncates": ("val = np.rint(a / spacing) * spacing", "val = np.floor(a / spacing) * spacing"),
    "e4m3_no_subnormals": ("spacing = np.where(a >= 2.0 ** -6, np.ldexp(1.0, E - 3), 2.0 ** -9)",
                           "spacing = np.ldexp(1.0, E - 3)"),
    "fp8_keys_not_quantised": ("_, _, keys_all = fp8_quantize_rows(pooled)", "keys_all = pooled"),
    "fp8_q_not_quantised": ("_, _, q_t = fp8_quantize_rows(q_t)", "pass"),
    "bf16_truncates": ("r = (u + np.uint64(0x7FFF) + keep_lsb)", "r = (u + np.uint64(0))"),
    "bf16_ties_away": ("r = (u + np.uint64(0x7FFF) + keep_lsb)", "r = (u + np.uint64(0x8000))"),
    "ln_no_eps": ("np.sqrt(var + F32(eps))", "np.sqrt(var)"),
    "ln_var_unbiased": ("var = ((dev * dev).sum(axis=1, dtype=F32) / F32(v.shape[1]))",
                        "var = ((dev * dev).sum(axis=1, dtype=F32) / F32(v.shape[1] - 1))"),
    "ln_bias_not_added": ("+ np.asarray(beta, F32)[None, :]", "+ 0 * np.asarray(beta, F32)[None, :]"),
    "k_lin_not_rounded": ("k = bf16_round(layer_norm(linear_bf16(x, wk), k_norm_weight",
                          "k = bf16_round(layer_norm((np.asarray(x, F32) @ np.asarray(wk, F32).T), k_norm_weight"),
    "head_weights_bf16": ("w = (np.asarray(x, dtype=F32) @ np.asarray(ww, dtype=F32).T).astype(F32)",
                          "w = bf16_round((np.asarray(x, dtype=F32) @ np.asarray(ww, dtype=F32).T).astype(F32))"),
    "q_heads_transposed": ("q = linear_bf16(qr, wq_b).reshape(T, num_heads, head_dim)",
                           "q = linear_bf16(qr, wq_b).reshape(T, head_dim, num_heads).transpose(0, 2, 1)"),
    "gate_from_wk": ("gate = linear_bf16(x, wg)", "gate = linear_bf16(x, wk)"),
    "mla_scale_dropped": ("s = sm_scale * (q[t] @ rows.T)", "s = (q[t] @ rows.T)"),
    "mla_lse_log2": ("lse[t] = m + np.log(l)", "lse[t] = (m + np.log(l)) * np.log2(np.e)"),
    "mla_minus_one_wraps": ("if 0 <= int(j) < N]", "if int(j) < N]"),
    "mla_out_of_range_kept": ("if 0 <= int(j) < N]", "if 0 <= int(j)] if False else "
                              "[min(int(j), N - 1) for j in indices[t] if 0 <= int(j)]"),
    "mla_repeats_merged": ("sel = [int(j) for j in indices[t] if 0 <= int(j) < N]",
                           "sel = sorted(set(int(j) for j in indices[t] if 0 <= int(j) < N))"),
    "mla_normalised_over_heads": ("o[t] = (e @ rows[:, :d_v]) / l[:, None]",
                                  "o[t] = (e @ rows[:, :d_v]) / l.sum()"),
    "mla_values_from_tail": ("o[t] = (e @ rows[:, :d_v])", "o[t] = (e @ rows[:, d_qk - d_v:])"),
    "mla_no_max_in_lse": ("lse[t] = m + np.log(l)", "lse[t] = np.log(l)"),
    "mla_empty_lse_zero": ("lse = np.full((T, H), -np.inf)", "lse = np.zeros((T, H))"),
    "mla_head_order": ("s = sm_scale * (q[t] @ rows.T)", "s = sm_scale * (q[t][::-1] @ rows.T)"),
}


def mutated_oracle(name):
    old, new = MUTATIONS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site of {name} not found"
    mod = types.ModuleType(f"oracle_mut_{name}")
    exec(compile(src.replace(old, new), SRC + f"<{name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = mutated_oracle(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:          # any failure (assertion or crash) counts
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"
