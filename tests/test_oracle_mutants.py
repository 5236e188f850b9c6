"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
that the pins catch every one: a dropped scale, transposed bases, the wrong
row order of the joint value basis, a gather that ignores the block table,
an off-by-one causal rule, and so on."""
import json
import os
import types

import pytest

import oracle.starkv_oracle as real
import oracle_checks as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = open(real.__file__).read()

MUTANTS = {
    "drop_scale": ("s = (qh @ Kh.T) * scale", "s = (qh @ Kh.T)"),
    "scale_by_rank": ("s = (qh @ Kh.T) * scale", "s = (qh @ Kh.T) / np.sqrt(Kh.shape[1] // 2)"),
    "transpose_U_in_rebuild": ("K[:, h, :] = ck[:, h, :] @ U[h].T",
                               "K[:, h, :] = (ck[:, h, :] @ U[h].T) if U.shape[1] != U.shape[2] else ck[:, h, :] @ U[h]"),
    "W_feature_major_rows": ("V = (cv @ W.T).reshape(L, H, d)",
                             "V = (cv @ W.T).reshape(L, d, H).transpose(0, 2, 1)"),
    "gather_ignores_block_table": ("blk = int(block_table_row[t // bs])", "blk = t // bs"),
    "gather_wrong_offset": ("off = t % bs", "off = (t + 1) % bs"),
    "softmax_no_normalise": ("return e / np.sum(e, axis=-1, keepdims=True)", "return e"),
    "softmax_wrong_axis": ("return e / np.sum(e, axis=-1, keepdims=True)",
                           "return e / np.sum(e, axis=0, keepdims=True)"),
    "causal_excludes_diagonal": ("visible = key_pos <= qry_pos", "visible = key_pos < qry_pos"),
    "causal_ignores_prefix": ("qry_pos = P0 + np.arange(C)[:, None]", "qry_pos = np.arange(C)[:, None]"),
    "no_causal_mask": ("o, _ = _attend(qf[q0:q1, h], K[:, g, :], V[:, g, :], scale, visible)",
                       "o, _ = _attend(qf[q0:q1, h], K[:, g, :], V[:, g, :], scale)"),
    "append_wrong_head_basis": ("kc[blk, h, off, :] = (Uf[h].T @ kf[n, h])",
                                "kc[blk, h, off, :] = (Uf[(h + 1) % H].T @ kf[n, h])"),
    "append_v_flatten_feature_major": ("vc[blk, :, off] = (Wf.T @ vf[n].reshape(-1))",
                                       "vc[blk, :, off] = (Wf.T @ vf[n].T.reshape(-1))"),
    "append_swapped_divmod": ("blk, off = divmod(slot, bs)", "off, blk = divmod(slot, bs)"),
    "append_writes_negative_slot": ("if slot < 0:\n            continue",
                                    "if slot < -1:\n            continue"),
    "append_truncates": ("kc[blk, h, off, :] = (Uf[h].T @ kf[n, h]).astype(np.float16)",
                         "kc[blk, h, off, :] = np.trunc((Uf[h].T @ kf[n, h]) * 64) / 64"),
    "empty_sequence_nan": ("out[b] = 0.0", "out[b] = np.nan"),
    "e4m3_wrong_bias": ("vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
                        "vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "e4m3_truncates": ("q = np.round(a / step) * step", "q = np.floor(a / step) * step"),
    "e4m3_no_saturation": ("x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)",
                           "x = np.asarray(x, dtype=np.float64)"),
    "fp8_append_scale_inverted": ("quantize_e4m3((Uf[h].T @ kf[n, h]) / k_scale)",
                                  "quantize_e4m3((Uf[h].T @ kf[n, h]) * k_scale)"),
    "gqa_interleaved_groups": ("        for h in range(H):\n            g = h // G\n            o, p = _attend(",
                               "        for h in range(H):\n            g = h % (H // G)\n            o, p = _attend("),
    "gqa_prefill_first_head_only": ("            g = h // G\n            o, _ = _attend(",
                                    "            g = 0\n            o, _ = _attend("),
    "fit_bottom_eigvecs": ("order = np.argsort(w)[::-1]", "order = np.argsort(w)"),
    "fit_mean_centred": ("        Kh = kf[:, h, :]\n", "        Kh = kf[:, h, :] - kf[:, h, :].mean(axis=0)\n"),
    "fit_v_feature_major": ("Vm = vf.reshape(N, H * d)", "Vm = vf.transpose(0, 2, 1).reshape(N, H * d)"),
    "fit_wrong_head": ("        Kh = kf[:, h, :]\n", "        Kh = kf[:, (h + 1) % H, :]\n"),
    "fit_values_from_keys": ("Vm = vf.reshape(N, H * d)", "Vm = kf.reshape(N, H * d)"),
    "decode_drops_last_token": ("ck, cv = gather_sequence_latents(k_cache, v_cache, block_tables[b], L)\n        K, V = reconstruct_sequence(ck, cv, U, W)\n        ph",
                                "ck, cv = gather_sequence_latents(k_cache, v_cache, block_tables[b], max(L - 1, 1))\n        K, V = reconstruct_sequence(ck, cv, U, W)\n        L = K.shape[0]\n        ph"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _run_all(mod):
    with open(os.path.join(GOLDEN, "paging_fixture.json")) as f:
        fx = json.load(f)
    failures = []
    for chk in oc.ALL_CHECKS:
        try:
            chk(mod)
        except Exception as e:  # an assertion or a crash both count as caught
            failures.append((chk.__name__, type(e).__name__))
    try:
        oc.check_paging_fixture(mod, fx)
    except Exception as e:
        failures.append(("check_paging_fixture", type(e).__name__))
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failures = _run_all(_load_mutant(name))
    assert failures, f"no pin caught the planted mistake {name}"
