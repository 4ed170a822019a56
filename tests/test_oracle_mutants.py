"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (on the CPU,
never on the GPU path), loads the copy as a separate module and runs the pin
checks of ``oracle_checks`` against it: at least one check must fail.  The
unmodified source must pass the same checks (covered in
``test_oracle_pins.py``).
"""

import os
import types

import pytest

from tests import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "rnn_oracle.py")
PHILOX_SRC = os.path.join(ORACLE_DIR, "philox.py")

# (id, original text, mutated text, modes whose checks must catch it)
MUTANTS = [
    ("lstm_gate_order", "a_i, a_f, a_g, a_o = _blocks(gi + gh, 4)",
     "a_f, a_i, a_g, a_o = _blocks(gi + gh, 4)", ["lstm"]),
    ("lstm_drop_b_hh", "        gh = h_prev @ p[\"w_hh\"].T + p[\"b_hh\"]\n        a_i",
     "        gh = h_prev @ p[\"w_hh\"].T\n        a_i", ["lstm"]),
    ("lstm_tanh_c", "h = o * np.tanh(c)", "h = o * c", ["lstm"]),
    ("gru_reset_outside", "n = np.tanh(gi_n + r * gh_n)", "n = np.tanh(gi_n + gh_n)", ["gru"]),
    ("gru_update_swapped",
     "            h = (1.0 - z) * n + z * h_prev\n            return h, None, {\"r\": r, \"z\": z, \"n\": n, \"gh_n\": gh_n}",
     "            h = (1.0 - z) * h_prev + z * n\n            return h, None, {\"r\": r, \"z\": z, \"n\": n, \"gh_n\": gh_n}",
     ["gru"]),
    ("gru_tf_flavour_as_pytorch", "n = np.tanh(gi_n + (r * h_prev) @ w_hn.T + b_hn)",
     "n = np.tanh(gi_n + r * (h_prev @ w_hn.T + b_hn))", ["gru"]),
    ("reverse_dir_runs_forward", "order = range(T) if d == 0 else range(T - 1, -1, -1)",
     "order = range(T)", ["lstm", "gru", "rnn_tanh"]),
    ("stack_input_not_chained", "        layer_in = y_l\n",
     "        layer_in = layer_in if l == 0 and layer_in.shape[2] == y_l.shape[2] else y_l\n",
     ["rnn_tanh"]),
    ("bptt_gru_dz_sign", "    dz = dh * (h_prev - n)", "    dz = dh * (n - h_prev)", ["gru"]),
    ("bptt_gru_drop_direct", "dh = dG_h @ p[\"w_hh\"] + direct", "dh = dG_h @ p[\"w_hh\"]",
     ["gru"]),
    ("bptt_gru_dr_no_ghn", "da_r = da_n * gh_n * r * (1.0 - r)", "da_r = da_n * r * (1.0 - r)",
     ["gru"]),
    ("bptt_gru_dGh_equals_dGi", "dG_h = np.concatenate([da_r, da_z, da_n * r], axis=1)",
     "dG_h = np.concatenate([da_r, da_z, da_n], axis=1)", ["gru"]),
    ("bptt_lstm_no_c_carry", "dc = dc * f\n", "dc = dc\n", ["lstm"]),
    ("bptt_lstm_dc_missing_o", "dc = dc + dh * o * (1.0 - tau ** 2)",
     "dc = dc + dh * (1.0 - tau ** 2)", ["lstm"]),
    ("bptt_lstm_df_wrong_state", "d_f = dc * s[\"c_prev\"]", "d_f = dc * s[\"c\"]", ["lstm"]),
    ("bptt_tanh_derivative", "da = dh * (1.0 - s[\"h\"] ** 2)", "da = dh * (1.0 - s[\"h\"])",
     ["rnn_tanh"]),
    ("bptt_dW_hh_uses_new_h", "g[\"w_hh\"] += dG_h.T @ h_prev",
     "g[\"w_hh\"] += dG_h.T @ (h_prev * 0.5 + 0.5 * np.tanh(h_prev))", ["rnn_tanh"]),
    ("bptt_db_hh_from_dGi", "g[\"b_hh\"] += dG_h.sum(axis=0)", "g[\"b_hh\"] += dG_i.sum(axis=0)",
     ["gru"]),
    ("bptt_dx_missing", "dX[t] += dG_i @ p[\"w_ih\"]", "dX[t] += 0.0 * (dG_i @ p[\"w_ih\"])",
     ["lstm"]),
    ("bptt_dy_not_added", "np.where(valid, dY[t, :, d * H:(d + 1) * H], 0.0)",
     "np.where(valid, dY[t, :, 0:H], 0.0)", ["rnn_tanh"]),
    ("gru_tf_bptt_no_rh_direct", "direct = direct + d_rh * r", "direct = direct", ["gru_tf"]),
    ("gru_tf_dW_hn_uses_h", 'g["w_hh"][2 * H:] += dG_h[:, 2 * H:].T @ (s["r"] * h_prev)',
     'g["w_hh"][2 * H:] += dG_h[:, 2 * H:].T @ h_prev', ["gru_tf"]),
    ("gru_paper_dz_sign", "dn, dz, direct = dh * z, dh * (n - h_prev), dh * (1.0 - z)",
     "dn, dz, direct = dh * z, dh * (h_prev - n), dh * (1.0 - z)", ["gru_paper"]),
    ("packed_state_not_held", "h = np.where(valid, h, h_prev)", "h = np.where(valid, h, h)",
     ["gru"]),
    ("packed_bwd_no_passthrough", "direct = np.where(valid, direct, dh_carried)",
     "direct = np.where(valid, direct, 0.0)", ["rnn_tanh"]),
    ("dropout_not_scaled", "np.where(k, 1.0 / (1.0 - p) if p < 1.0 else 0.0, 0.0)",
     "np.where(k, 1.0, 0.0)", ["dropout"]),
    ("dropout_bwd_unmasked", 'dY = dX * cache["dropout"][l] if l in cache["dropout"] else dX',
     "dY = dX", ["dropout"]),
    ("dropout_drops_x", "if l > 0 and dropout > 0.0:", "if dropout > 0.0:", ["dropout"]),
    ("dropout_dW_ih_undropped_input",
     "            layer_in = layer_in * m\n            if keep:\n                cache[\"dropout\"][l] = m\n"
     "        if keep:\n            cache[\"layer_inputs\"].append(layer_in)\n",
     "            if keep:\n                cache[\"layer_inputs\"].append(layer_in)\n"
     "            layer_in = layer_in * m\n            if keep:\n                cache[\"dropout\"][l] = m\n"
     "        elif keep:\n            cache[\"layer_inputs\"].append(layer_in)\n", ["dropout"]),
    ("dropout_layer_not_in_counter", "np.full(n, layer, dtype=np.uint64)",
     "np.zeros(n, dtype=np.uint64)", ["dropout"]),
    ("dropout_keep_inverted", "w.astype(np.int64) >= dropout_threshold(p)",
     "w.astype(np.int64) < dropout_threshold(p)", ["dropout"]),
    ("dropout_word_order", "(e & np.uint64(3)).astype(np.int64)",
     "(np.uint64(3) - (e & np.uint64(3))).astype(np.int64)", ["dropout"]),
    ("dropout_seed_high_word_ignored", "seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)",
     "seed & 0xFFFFFFFF, 0)", ["dropout"]),
]

# mistakes planted in the Philox generator (the known-answer vectors catch them)
PHILOX_MUTANTS = [
    ("philox_weyl_swapped", "k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask",
     "k0, k1 = (k0 + w1) & mask, (k1 + w0) & mask"),
    ("philox_first_round_bumped", "        if r > 0:\n            k0, k1 = (k0 + w0) & mask",
     "        if r >= 0:\n            k0, k1 = (k0 + w0) & mask"),
    ("philox_words_permuted", "x = [(p1 >> bits) ^ x[1] ^ k0, p1 & mask, (p0 >> bits) ^ x[3] ^ k1, p0 & mask]",
     "x = [(p0 >> bits) ^ x[1] ^ k0, p0 & mask, (p1 >> bits) ^ x[3] ^ k1, p1 & mask]"),
    ("philox_array_lo_hi", "x = [(p1 >> u64(32)) ^ x[1] ^ u64(k0), p1 & lo32,",
     "x = [(p1 & lo32) ^ x[1] ^ u64(k0), p1 >> u64(32),"),
    ("philox_array_nine_rounds", "def philox4x32_array(c0, c1, c2, c3, k0, k1, rounds=10):",
     "def philox4x32_array(c0, c1, c2, c3, k0, k1, rounds=9):"),
]


def _load_mutant(orig, new, path=SRC):
    src = open(path).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/found: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(orig, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_fail(mod, modes):
    checks = [lambda: oc.check_gru_worked_values(mod) > 1e-11,
              lambda: oc.check_closed_forms(mod) > 1e-11,
              lambda: oc.check_bptt_closed_forms(mod) > 1e-12]
    for mode in modes:
        if mode == "dropout":
            from oracle import philox as px
            checks.append(lambda: bool(oc.dropout_mask_failures(mod, px)))
            for m, L, D in (("lstm", 3, 2), ("gru", 2, 1)):
                checks.append(lambda m=m, L=L, D=D:
                              oc.check_dropout_against_torch(mod, m, L, D, 0.3, seed=77) > 1e-11)
            continue
        if mode.startswith("gru_"):   # another GRU flavour: finite differences only
            v = mode[4:]
            checks.append(lambda v=v: oc.check_finite_differences(mod, "gru", 1, 2, T=3, B=2, I=3, H=2,
                                                                  gru_variant=v) > 1e-6)
            continue
        for L, D in ((2, 2), (1, 1)):
            checks.append(lambda mode=mode, L=L, D=D: oc.check_against_torch(mod, mode, L, D) > 1e-11)
            checks.append(lambda mode=mode, L=L, D=D:
                          oc.check_finite_differences(mod, mode, L, D, T=2, B=2, I=3, H=2) > 1e-6)
            checks.append(lambda mode=mode, L=L, D=D:
                          oc.check_against_torch(mod, mode, L, D, lengths=[4, 1, 3]) > 1e-11)
    for chk in checks:
        try:
            if chk():
                return True
        except Exception:
            return True  # a crash is also a detected mistake
    return False


@pytest.mark.parametrize("name,orig,new,modes", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, new, modes):
    assert _pins_fail(_load_mutant(orig, new), modes), f"mutant {name} survived the pins"


@pytest.mark.parametrize("name,orig,new", PHILOX_MUTANTS, ids=[m[0] for m in PHILOX_MUTANTS])
def test_planted_philox_mistake_is_caught(name, orig, new):
    mod = _load_mutant(orig, new, PHILOX_SRC)
    try:
        assert oc.philox_kat_failures(mod), f"mutant {name} survived the known answers"
    except AssertionError:
        raise
    except Exception:
        pass   # a crash is also a detected mistake


def test_unmodified_copy_passes():
    mod = _load_mutant("MODES = (", "MODES = (")
    assert not _pins_fail(mod, ["lstm", "gru", "rnn_tanh", "dropout"])
    assert not oc.philox_kat_failures(_load_mutant("CONSTANTS = {", "CONSTANTS = {", PHILOX_SRC))
