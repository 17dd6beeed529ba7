"""The oracle against its pins (CPU), and planted mistakes that the pins must catch."""
import os
import sys
import types

import pytest

import oracle_pins as P

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin):
    pin()


# (name, file, [(old, new), ...], pins that must go red)
MUTANTS = [
    ("nibble_order_swapped", "formats.py",
     [("out[..., 0::2] = lo", "out[..., 0::2] = hi"), ("out[..., 1::2] = hi", "out[..., 1::2] = lo")],
     ["pin_one_hot_columns", "pin_worked_rows"]),
    ("block_scale_off_by_one", "moe.py",
     [("np.repeat(sc, 16, axis=-1)", "np.repeat(np.roll(sc, 1, axis=-1), 16, axis=-1)")],
     ["pin_one_hot_columns", "pin_worked_rows"]),
    ("tie_break_flipped", "moe.py",
     [("np.lexsort((idx[t], -vals[t]))", "np.lexsort((-idx[t], -vals[t]))")],
     ["pin_route_brute_force"]),
    ("gate_tensor_scale_dropped", "moe.py",
     [("G = tg * (X @ Wg.T)", "G = (X @ Wg.T)")],
     ["pin_single_expert_brute_force", "pin_h_rounds_once"]),
    ("down_tensor_scale_twice", "moe.py",
     [("O = td * (H @ Wd.T)", "O = td * td * (H @ Wd.T)")],
     ["pin_single_expert_brute_force", "pin_two_expert_combine"]),
    ("h_not_rounded", "moe.py",
     [("H = F.bf16_rne(h_exact)", "H = h_exact")],
     ["pin_single_expert_brute_force"]),
    ("h_rounded_through_fp32", "moe.py",
     [("H = F.bf16_rne(h_exact)", "H = F.bf16_rne(h_exact.astype(np.float32).astype(np.float64))")],
     ["pin_h_rounds_once"]),
    ("rows_rounded_before_combine", "moe.py",
     [("O = td * (H @ Wd.T)", "O = F.bf16_rne(td * (H @ Wd.T))")],
     ["pin_two_expert_combine"]),
    ("row_list_order_reversed", "moe.py",
     [("sorted_rows = np.argsort(flat, kind=\"stable\")",
       "sorted_rows = np.argsort(flat * flat.size - np.arange(flat.size), kind=\"stable\")")],
     ["pin_row_lists_definition"]),
    ("e8m0_bias_126", "formats.py",
     [("return 2.0 ** (code - 127)", "return 2.0 ** (code - 126)")],
     ["pin_e8m0_golden_and_torch", "pin_mxfp8_one_hot_and_scale"]),
    ("e4m3_subnormal_exponent", "formats.py",
     [("mag = 2.0 ** (-6) * (m / 8.0)", "mag = 2.0 ** (-7) * (m / 8.0)")],
     ["pin_e4m3_golden_and_torch"]),
    ("swiglu_branches_swapped", "moe.py",
     [("h_exact = sg * U", "h_exact = silu(U) * G")],
     ["pin_single_expert_brute_force", "pin_gate_scale_not_linear"]),
    ("weights_not_renormalized", "moe.py",
     [("w = ex / ex.sum(axis=1, keepdims=True)", "w = ex")],
     ["pin_route_brute_force", "pin_route_k2_closed_form"]),
    ("combine_wrong_slot", "moe.py",
     [("y += w[:, j:j + 1] * y_rows[ro[:, j]]", "y += w[:, j:j + 1] * y_rows[ro[:, 0]]")],
     ["pin_two_expert_combine"]),
    ("bf16_ties_away", "formats.py",
     [("np.ldexp(np.rint(scaled), q_exp)", "np.ldexp(np.sign(scaled) * np.floor(np.abs(scaled) + 0.5), q_exp)")],
     ["pin_bf16_rne_vs_torch", "pin_bf16_rne_vs_fractions"]),
    ("token_of_row_wrong", "moe.py",
     [("tok = rl.sorted_rows[p].astype(np.int64) // k", "tok = rl.sorted_rows[p].astype(np.int64) % k")],
     ["pin_token_permutation", "pin_two_expert_combine"]),
    ("router_mass_signed", "router.py",
     [("np.abs(x) @ np.abs(w).T", "x @ w.T")],
     ["pin_router_worked_case", "pin_router_mass"]),
    ("router_experts_reversed", "router.py",
     [("return x @ w.T,", "return x @ w[::-1].T,")],
     ["pin_router_worked_case", "pin_router_scaled_identity", "pin_router_fractions"]),
    ("router_weights_as_fp16", "router.py",
     [("w = F.bf16_bits_to_f64(np.asarray(wr_bits, dtype=np.uint16))",
       "w = np.asarray(wr_bits, dtype=np.uint16).view(np.float16).astype(np.float64)")],
     ["pin_router_worked_case", "pin_router_scaled_identity"]),
    ("router_tolerance_too_tight", "router.py",
     [("return (d + 8) * U32 * mass", "return U32 * mass")],
     ["pin_router_tolerance_covers_fp32"]),
    ("policy_softmax_renormalized", "router.py",
     [("w = np.exp(sel - m) / np.exp(lg - m).sum(axis=1, keepdims=True)",
       "w = np.exp(sel - m) / np.exp(sel - m).sum(axis=1, keepdims=True)")],
     ["pin_policy_softmax_vs_scipy"]),
    ("policy_bias_in_weights", "router.py",
     [("lg = np.asarray(logits, dtype=np.float32).astype(np.float64)",
       "lg = selection_keys(logits, bias).astype(np.float64)")],
     ["pin_bias_moves_choice_only"]),
    ("policy_bias_fp64", "router.py",
     [("return (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)",
       "return lg.astype(np.float64) + np.asarray(bias, dtype=np.float64)[None, :]")],
     ["pin_bias_rounds_in_fp32"]),
    ("policy_sigmoid_renorm_dropped", "router.py",
     [("w = sg / sg.sum(axis=1, keepdims=True) if policy == SIGMOID_RENORM else sg", "w = sg")],
     ["pin_policy_sigmoid_vs_scipy"]),
    ("policy_tie_to_higher_index", "router.py",
     [("ids[t] = np.lexsort((np.arange(E), -keys[t]))[:k]", "ids[t] = np.lexsort((-np.arange(E), -keys[t]))[:k]")],
     ["pin_policy_choice_property", "pin_bias_rounds_in_fp32"]),
    ("shared_gate_not_applied", "shared.py",
     [("y = res.y + g[:, None] * S.y_rows", "y = res.y + S.y_rows")],
     ["pin_shared_identity_closed_form", "pin_shared_is_an_extra_routed_expert"]),
    ("shared_gate_sign_flipped", "shared.py",
     [("    z = x @ w\n", "    z = -(x @ w)\n")],
     ["pin_shared_is_an_extra_routed_expert"]),
    ("shared_row_rounded", "shared.py",
     [("y = res.y + g[:, None] * S.y_rows", "y = res.y + g[:, None] * F.bf16_rne(S.y_rows)")],
     ["pin_shared_is_an_extra_routed_expert"]),
    ("mxfp8_block_16", "mxfp8.py",
     [("np.repeat(F.E8M0_TABLE[s], 32, axis=-1)", "np.repeat(F.E8M0_TABLE[s], 16, axis=-1)[..., : w.shape[-1]]")],
     ["pin_mxfp8_one_hot_and_scale", "pin_mxfp8_brute_force"]),
    ("residual_added_twice", "block.py",
     [("    y = res.y + x\n", "    y = res.y + 2 * x\n")],
     ["pin_residual_closed_forms"]),
    ("residual_rounded_first", "block.py",
     [("    y = res.y + x\n", "    y = F.bf16_rne(res.y) + x\n")],
     ["pin_residual_closed_forms"]),
    ("residual_wrong_tokens", "block.py",
     [("        x = x[np.asarray(tokens, dtype=np.int64)]\n", "        x = x[: len(tokens)]\n")],
     ["pin_residual_sampled_tokens"]),
    ("e4m3_ties_away", "w8a8.py",
     [("pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))", "pick_hi = (dhi <= dlo)")],
     ["pin_e4m3_rounding_vs_torch"]),
    ("mx_emax_7", "w8a8.py",
     [("E4M3_EMAX = 8 ", "E4M3_EMAX = 7 ")],
     ["pin_mx_scale_rule"]),
    ("mx_overflow_to_nan", "w8a8.py",
     [("    code = np.where(a == _POS_VALUES[hi], hi, code)           # exact values\n",
       "    code = np.where(a == _POS_VALUES[hi], hi, code)\n    code = np.where(np.abs(v) > E4M3_MAX, 0x7F, code)\n")],
     ["pin_e4m3_rounding_vs_torch", "pin_mx_scale_rule"]),
    ("mx_scale_ceil", "w8a8.py",
     [("shared = (e - 1) - E4M3_EMAX", "shared = e - E4M3_EMAX")],
     ["pin_mx_scale_rule", "pin_mx_quantization_error_bound"]),
    # ---- the acceptance rule and its slack terms
    ("slack_h_x1024", "moe.py",
     [("sh = abs(td) * ((amb * ulp) @ aWd.T)", "sh = 1024 * abs(td) * ((amb * ulp) @ aWd.T)")],
     ["pin_slack_h_midpoint"]),
    ("band_slack_x1024", "band.py",
     [("bound = bound + np.asarray(slack)", "bound = bound + 1024 * np.asarray(slack)")] * 2,
     ["pin_band_explained_by_hand"]),
    ("amb_always_true", "moe.py",
     [("amb = (h_exact - dh <= lo_mid) | (h_exact + dh >= hi_mid)", "amb = np.ones_like(H, dtype=bool)")],
     ["pin_slack_h_midpoint", "pin_slack_h_window"]),
    ("h_ulp_doubled", "moe.py",
     [("ulp = F.bf16_ulp(H)", "ulp = 2 * F.bf16_ulp(H)")],
     ["pin_slack_h_midpoint", "pin_slack_h_window"]),
    ("acc_window_doubled", "moe.py",
     [("ACC_REL = 2.0 ** -20", "ACC_REL = 2.0 ** -19")],
     ["pin_slack_h_window"]),
    ("gate_mass_signed", "moe.py",
     [("mass_g = abs(tg) * (aX @ np.abs(Wg).T)", "mass_g = abs(tg) * (X @ Wg.T)")],
     ["pin_slack_h_window"]),
    ("mass_y_signed", "moe.py",
     [("my = abs(td) * (np.abs(H) @ aWd.T)", "my = abs(td) * (H @ Wd.T)")],
     ["pin_mass_y_brute_force"]),
    ("mass_y_signed_tensor_scale", "moe.py",
     [("my = abs(td) * (np.abs(H) @ aWd.T)", "my = td * (np.abs(H) @ aWd.T)"),
      ("sh = abs(td) * ((amb * ulp) @ aWd.T)", "sh = td * ((amb * ulp) @ aWd.T)")],
     ["pin_masses_ignore_tensor_scale_signs"]),
    ("mass_u_signed_tensor_scale", "moe.py",
     [("mass_u = abs(tu) * (aX @ np.abs(Wu).T)", "mass_u = tu * (aX @ np.abs(Wu).T)")],
     ["pin_masses_ignore_tensor_scale_signs"]),
    ("mass_share_ignored", "band.py",
     [("        bound = bound + mass_rel * np.asarray(mass)", "        bound = bound + MASS_REL * np.asarray(mass)")],
     ["pin_band_mass_share_parameter"]),
    ("mass_rel_2m10", "band.py",
     [("MASS_REL = 2.0 ** -20", "MASS_REL = 2.0 ** -10")],
     ["pin_band_explained_by_hand"]),
    ("strict_open_interval", "band.py",
     [("strict = diff <= strict_bound", "strict = diff < strict_bound")] * 2,
     ["pin_band_strict_by_hand"]),
    ("rtol_wider", "band.py",
     [("RTOL = 2e-2", "RTOL = 2.1e-2")],
     ["pin_band_strict_by_hand"]),
    ("atol_wider", "band.py",
     [("ATOL = 2e-3", "ATOL = 2.1e-3")],
     ["pin_band_strict_by_hand"]),
    ("nan_passes", "band.py",
     [("diff = np.where(np.isnan(diff), np.inf, diff)", "diff = np.where(np.isnan(diff), 0.0, diff)")] * 2,
     ["pin_band_strict_by_hand", "pin_band_explained_by_hand"]),
    ("ulp_of_gpu_value", "band.py",
     [("bound = strict_bound + F.bf16_ulp(r)", "bound = strict_bound + F.bf16_ulp(g)")],
     ["pin_band_explained_by_hand"]),
    ("ulp_term_on_f32_rows", "band.py",
     [("bound = strict_bound.copy()", "bound = strict_bound + F.bf16_ulp(r)")],
     ["pin_band_explained_by_hand"]),
    ("bf16_ulp_subnormal_floor", "formats.py",
     [("return np.ldexp(1.0, np.maximum(e, -125) - 8)", "return np.ldexp(1.0, np.maximum(e, -126) - 8)")],
     ["pin_bf16_ulp_spacing"]),
    ("bf16_ulp_doubled", "formats.py",
     [("return np.ldexp(1.0, np.maximum(e, -125) - 8)", "return np.ldexp(2.0, np.maximum(e, -125) - 8)")],
     ["pin_bf16_ulp_spacing", "pin_band_explained_by_hand"]),
    ("gate_bound_without_d", "shared.py",
     [("0.25 * (d + 8) * 2.0 ** -24", "0.25 * 2.0 ** -24")],
     ["pin_shared_gate_bound"]),
    ("mxfp8_mass_signed", "mxfp8.py",
     [("mass = np.abs(X) @ np.abs(W).T", "mass = X @ W.T")],
     ["pin_mxfp8_mass_brute_force"]),
    ("refusal_nan_scale_code_dropped", "moe.py",
     [("if np.any((s & 0x7F) == 0x7F):", "if False:")],
     ["pin_refusals"]),
    ("refusal_logit_check_dropped", "moe.py",
     [("if not np.all(np.isfinite(logits)):", "if False:")],
     ["pin_refusals"]),
    ("refusal_tensor_scale_dropped", "moe.py",
     [("if not np.all(np.isfinite(experts[nm])):", "if False:")],
     ["pin_refusals"]),
    ("refusal_e8m0_dropped", "mxfp8.py",
     [("if np.any(s == 0xFF):", "if False:")],
     ["pin_refusals"]),
]


def _exec_module(fname, edits, pkg_overrides):
    path = os.path.join(ORACLE_DIR, fname)
    src = open(path).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutant anchor not found in {fname}: {old}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant_" + fname[:-3])
    mod.__package__ = "oracle"
    mod.__file__ = path
    sys.modules[mod.__name__] = mod
    exec(compile(src, path, "exec"), mod.__dict__)
    for k, v in pkg_overrides.items():
        setattr(mod, k, v)
    return mod


@pytest.mark.parametrize("name,fname,edits,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, fname, edits, pins):
    import oracle.band as bandreal
    import oracle.block as blockreal
    import oracle.w8a8 as w8real
    import oracle.formats as Freal
    import oracle.moe as moereal
    import oracle.mxfp8 as mxreal
    import oracle.router as rtreal
    import oracle.shared as shreal
    rtm = _exec_module("router.py", edits, {}) if fname == "router.py" else rtreal
    shm = _exec_module("shared.py", edits, {}) if fname == "shared.py" else shreal
    bandm = _exec_module("band.py", edits, {}) if fname == "band.py" else bandreal
    blockm = _exec_module("block.py", edits, {}) if fname == "block.py" else blockreal
    w8m = _exec_module("w8a8.py", edits, {}) if fname == "w8a8.py" else w8real
    if fname in ("router.py", "shared.py", "band.py", "block.py", "w8a8.py"):
        Fm, moem, mxm = Freal, moereal, mxreal
    elif fname == "formats.py":
        Fm = _exec_module("formats.py", edits, {})
        moem = _exec_module("moe.py", [], {"F": Fm})
        mxm = _exec_module("mxfp8.py", [], {"F": Fm})
        bandm = _exec_module("band.py", [], {"F": Fm})
    elif fname == "moe.py":
        Fm = Freal
        moem = _exec_module("moe.py", edits, {})
        mxm = mxreal
    else:
        Fm, moem = Freal, moereal
        mxm = _exec_module("mxfp8.py", edits, {})
    monkeypatch.setattr(P, "F", Fm)
    monkeypatch.setattr(P, "moe", moem)
    monkeypatch.setattr(P, "mxfp8", mxm)
    monkeypatch.setattr(P, "router", rtm)
    monkeypatch.setattr(P, "shared", shm)
    monkeypatch.setattr(P, "band", bandm)
    monkeypatch.setattr(P, "block", blockm)
    monkeypatch.setattr(P, "w8a8", w8m)
    red = []
    for pn in pins:
        try:
            getattr(P, pn)()
        except Exception:
            red.append(pn)
    assert red, f"mutant {name} went undetected by {pins}"
