"""Plant plausible mistakes in a copy of the oracle (CPU only) and require that
at least one pin catches each of them.  This is what makes the pins a real
check: a dropped term, a wrong sign or index, an off-by-one window or a
swapped operand must not slip through."""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block.py")

MUTANTS = {
    "unbiased_variance": [("var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)",
                           "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)")],
    "eps_outside_sqrt": [("np.sqrt(var + eps)", "(np.sqrt(var) + eps)")],
    "dropped_beta": [(" + np.asarray(beta, np.float64)", "")],
    "dropped_gamma": [(" * np.asarray(gamma, np.float64)", "")],
    "gelu_tanh_form": [("0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))",
                        "0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))")],
    "gelu_missing_sqrt2": [("erf(z / math.sqrt(2.0))", "erf(z)")],
    "window_one_too_wide": [("max(0, i - W + 1)", "max(0, i - W)"),
                            ("(kj >= qi - W + 1)", "(kj >= qi - W)")],
    "window_one_too_narrow": [("(kj >= qi - W + 1)", "(kj >= qi - W + 2)")],
    "window_not_causal": [("(kj <= qi)", "(kj <= qi + 1)")],
    "scale_1_over_hd": [("1.0 / math.sqrt(hd)", "1.0 / hd")],
    "no_scale": [("scale = 1.0 / math.sqrt(hd)", "scale = 1.0")],
    "k_v_swapped": [("k = z[..., A:2 * A]", "k = z[..., 2 * A:3 * A]"),
                    ("v = z[..., 2 * A:3 * A]", "v = z[..., A:2 * A]")],
    "head_minor_layout": [("q = z[..., 0:A].reshape(*lead, H, hd)",
                           "q = z[..., 0:A].reshape(*lead, hd, H).swapaxes(-1, -2)")],
    "concat_order_swapped": [("np.concatenate([o.reshape(B, S, A), g], axis=-1)",
                              "np.concatenate([g, o.reshape(B, S, A)], axis=-1)")],
    "gelu_on_attention_too": [("ag = np.concatenate([o.reshape(B, S, A), g], axis=-1)",
                               "ag = gelu(np.concatenate([o.reshape(B, S, A), f], axis=-1))")],
    "residual_dropped": [("        y = y + x\n", "        y = y\n")],
    "residual_of_ln_output": [("        y = y + x\n", "        y = y + u\n")],
    "w_out_not_transposed": [("y = ag @ w_out.T", "y = ag @ w_out.reshape(w_out.shape[1], w_out.shape[0])")],
    "softmax_over_all_keys": [("scores = np.where(allowed[None], scores, -np.inf)", "scores = scores")],
    "serial_ln2_on_x": [("u2 = layer_norm(h, gamma2, beta2, eps)\n    return h +",
                         "u2 = layer_norm(x, gamma2, beta2, eps)\n    return h +")],
    "serial_ln2_uses_ln1_params": [("layer_norm(h, gamma2, beta2, eps)", "layer_norm(h, gamma, beta, eps)")],
    "serial_no_inner_residual": [("h = x + o.reshape(B, S, A) @ w_out[:, :A].T", "h = o.reshape(B, S, A) @ w_out[:, :A].T")],
    "serial_mlp_residual_from_x": [("    return h + gelu(u2 @ w_in[3 * A:].T) @ w_out[:, A:].T",
                                    "    return x + gelu(u2 @ w_in[3 * A:].T) @ w_out[:, A:].T")],
    "gelu_tanh_wrong_cubic": [("0.044715 * z ** 3", "0.04715 * z ** 3")],
    "gelu_form_ignored": [('act = gelu(f) if gelu_form == "erf" else gelu_tanh(f)', "act = gelu(f)")],
    "rope_half_split_pairs": [("even, odd = t[..., 0::2], t[..., 1::2]", "even, odd = t[..., :hd // 2], t[..., hd // 2:]"),
                              ("out[..., 0::2] = even * c - odd * s", "out[..., :hd // 2] = even * c - odd * s"),
                              ("out[..., 1::2] = even * s + odd * c", "out[..., hd // 2:] = even * s + odd * c")],
    "rope_rotates_backwards": [("out[..., 0::2] = even * c - odd * s", "out[..., 0::2] = even * c + odd * s"),
                               ("out[..., 1::2] = even * s + odd * c", "out[..., 1::2] = -even * s + odd * c")],
    "rope_frequency_exponent": [("(-2.0 * np.arange(hd // 2) / hd)", "(-1.0 * np.arange(hd // 2) / hd)")],
    "rope_on_v_too": [("        k = rope(k, pos, rope_base)\n", "        k = rope(k, pos, rope_base)\n        v = rope(v, pos, rope_base)\n")],
    "rope_only_q": [("        k = rope(k, pos, rope_base)\n", "")],
    "bias_in_skips_mlp": [("f = f + b_in[3 * A:]", "f = f")],
    "bias_out_dropped": [("y = y + b_out", "y = y")],
    "two_ln_swapped": [("z = u_attn @ w_in[:3 * A].T", "z = u_mlp @ w_in[:3 * A].T")],
    "gelu_grad_no_density_term": [(" + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)", "")],
    "softmax_bwd_not_centred": [("ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))", "ds = p * dp")],
    "dq_missing_scale": [("dq[s0:s1] += (ds @ kk).transpose(1, 0, 2) * scale", "dq[s0:s1] += (ds @ kk).transpose(1, 0, 2)")],
    "dv_from_ds": [("dv[j0:j1 + 1] += (p.transpose(0, 2, 1) @ dos)", "dv[j0:j1 + 1] += (ds.transpose(0, 2, 1) @ dos)")],
    "dk_dv_swapped": [("dz[b, :, A:2 * A] = dk.reshape(S, A)", "dz[b, :, A:2 * A] = dv.reshape(S, A)"),
                      ("dz[b, :, 2 * A:3 * A] = dv.reshape(S, A)", "dz[b, :, 2 * A:3 * A] = dk.reshape(S, A)")],
    "ln_bwd_no_xhat_term": [(" - xhat * (g * xhat).mean(axis=-1, keepdims=True)", "")],
    "ln_bwd_dgamma_without_xhat": [("return dx, (du * xhat).sum(axis=lead), du.sum(axis=lead)",
                                    "return dx, du.sum(axis=lead), du.sum(axis=lead)")],
    "residual_grad_dropped": [("        dx = dx + dy\n", "        dx = dx\n")],
    "dw_out_before_gelu": [("dw_out = dy.reshape(-1, d).T @ ag.reshape(-1, ag.shape[-1])",
                            "dw_out = dy.reshape(-1, d).T @ np.concatenate([o.reshape(B, S, A), f], axis=-1).reshape(-1, ag.shape[-1])")],
    "relerr_denominator_from_test": [("denom = np.abs(y_ref).max()", "denom = np.abs(y_test).max()")],
    "relerr_mean_difference": [("np.abs(y_test - y_ref).max() / denom", "np.abs(y_test - y_ref).mean() / denom")],
    "relerr_elementwise_ratio": [("np.abs(y_test - y_ref).max() / denom",
                                  "(np.abs(y_test - y_ref) / np.maximum(np.abs(y_ref), 1e-300)).max()")],
    "dw_in_from_x": [("dw_in = dz.reshape(-1, z.shape[-1]).T @ u.reshape(-1, d)",
                      "dw_in = dz.reshape(-1, z.shape[-1]).T @ x.reshape(-1, d)")],
}


def _mutant(edits):
    src = open(SRC_PATH).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


# a planted mistake may produce NaN (an empty softmax row), which numpy reports as a warning
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes():
    mod = _mutant([])
    for pin in ALL_PINS:
        pin(mod)
