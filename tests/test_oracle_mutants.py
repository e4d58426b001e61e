"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is the oracle's source with one plausible slip substituted in
(CPU only, nothing touches the GPU). If a mutant passed every pin, the pins
would not be strong enough to trust the oracle.
"""
import inspect
import types

import pytest

import oracle
from pins import ALL_PINS

MUTANTS = {
    "causal_off_by_one": ("ok &= j <= i", "ok &= j < i"),
    "causal_bottom_right": ("ok &= j <= i", "ok &= j <= i + (Lk - 1 - i.max())"),
    "kv_len_inclusive": ("ok &= j < n", "ok &= j <= n"),
    "kv_len_ignored": ("n = min(max(int(kv_len_b), 0), Lk)", "n = Lk"),
    "kv_len_masks_queries": ("ok &= j < n", "ok &= i < n"),
    "scale_dropped": ("s = scale * (q_bh[rows] @ k_bg.T)", "s = (q_bh[rows] @ k_bg.T)"),
    "default_scale_1_over_d": ("return 1.0 / math.sqrt(d)", "return 1.0 / d"),
    "max_wrong_axis": ("m = s.max(axis=1, keepdims=True)", "m = s.max(axis=0, keepdims=True)"),
    "sum_wrong_axis": ("z = e.sum(axis=1, keepdims=True)", "z = e.sum(axis=0, keepdims=True)"),
    "values_are_keys": ("return p @ v_bg, p", "return p @ k_bg, p"),
    "gqa_interleaved": ("g = h // group", "g = h % Hkv"),
    "gqa_rows_interleaved": ("g = h // (H // Hkv)", "g = h % Hkv"),
    "bcast_ignores_map": ("u = int(cand2user[c])", "u = int(c) % B_u"),
    "bcast_kvlen_by_candidate": ("kvl = None if kv_len is None else kv_len[u]",
                                 "kvl = None if kv_len is None else kv_len[min(c, B_u - 1)]"),
    "bcast_no_nan": ("o[n] = np.nan", "o[n] = 0.0"),
    "masked_row_not_zero": ("where=z > 0)", "where=z >= 0)"),
    "exp_base_2": ("np.exp(s - m)", "np.exp2(s - m)"),
    "jagged_kv_uses_q_offsets": ("ks, lk = _seq_bounds(kv_offsets, b)",
                                 "ks, lk = _seq_bounds(q_offsets, b)"),
    "jagged_length_short": ("return start, max(int(offsets[b + 1]) - start, 0)",
                            "return start, max(int(offsets[b + 1]) - start - 1, 0)"),
    "jagged_global_causal": ("rows = np.arange(lq)\n", "rows = np.arange(qs, qs + lq)\n"),
    "block_mask_transposed": ("ok &= np.asarray(bm, dtype=bool)[i // blk, j // blk]",
                              "ok &= np.asarray(bm, dtype=bool).T[i // blk, j // blk]"),
    "block_mask_ignored": ("ok &= np.asarray(bm, dtype=bool)[i // blk, j // blk]",
                           "ok &= np.asarray(bm, dtype=bool).any()"),
    "block_mask_first_head": ("return (bm[0] if bm.shape[0] == 1 else bm[h]), int(blk)",
                              "return bm[0], int(blk)"),
    "block_index_by_key_only": ("ok &= np.asarray(bm, dtype=bool)[i // blk, j // blk]",
                                "ok &= np.asarray(bm, dtype=bool)[0 * i, j // blk]"),
    "ikbo_concat_swapped": ("feats = np.concatenate([rep, xc], axis=1)",
                            "feats = np.concatenate([xc, rep], axis=1)"),
    "ikbo_ignores_map": ("bad = (c2u < 0) | (c2u >= B_u)",
                         "c2u = np.arange(B_c) % max(B_u, 1); bad = (c2u < 0) | (c2u >= B_u)"),
    "ikbo_weight_transposed": ("y = feats @ w.T", "y = feats @ w.reshape(w.shape[1], -1)"),
    "ikbo_bias_dropped": ("        y = y + np.asarray(bias, np.float64)[None, :]\n",
                          "        pass\n"),
    "ikbo_no_nan": ("y[bad] = np.nan", "y[bad] = 0.0"),
    "ikbo_user_partial_wrong_columns": ("z = xu @ w[:, :K_u].T", "z = xu @ w[:, -K_u:].T"),
    "rms_mean_as_sum": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                        "r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    "rms_eps_outside": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                        "r = 1.0 / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    "rms_wrong_axis": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                       "r = 1.0 / np.sqrt(np.mean(x * x, axis=-2, keepdims=True) + eps)"),
    "rms_gamma_ignored": ("        y = y * np.asarray(gamma, np.float64)\n", "        pass\n"),
    # (swapping the two gains is no mistake: scores depend on their product only)
    "qknorm_key_gain_dropped": ("return attention(rms_norm(q, gamma_q, eps), rms_norm(k, gamma_k, eps), v,",
                                "return attention(rms_norm(q, gamma_q, eps), rms_norm(k, None, eps), v,"),
    "qknorm_v_normalised": ("rms_norm(k, gamma_k, eps), v, causal=causal,",
                            "rms_norm(k, gamma_k, eps), rms_norm(v, None, eps), causal=causal,"),
    "jagged_heads_interleaved": ("o[qs:qs + lq, h], _ = _head_rows(q[qs:qs + lq, h], k[ks:ks + lk, g]",
                                 "o[qs:qs + lq, h], _ = _head_rows(q[qs:qs + lq, h], k[ks:ks + lk, h % Hkv]"),
}


def _mutant(name):
    src = inspect.getsource(oracle)
    old, new = MUTANTS[name]
    assert old in src, f"mutation anchor missing for {name}: {old!r}"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in ALL_PINS:
        if pin.__name__ in ("pin_brute_force",):   # slow; the others suffice
            continue
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
