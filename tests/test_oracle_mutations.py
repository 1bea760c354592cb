"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each.

A mutation is a one-place source edit of ``oracle/moe_oracle.py``: the
edited source is executed into a fresh module whose functions replace the
real ones for the duration of the test.
"""
import inspect
import types

import pytest

import oracle
import oracle.moe_oracle as om
from tests import pins

MUTATIONS = {
    "tie_break_higher_id": (
        'order = np.argsort(-key, axis=1, kind="stable")',
        'order = key.shape[1] - 1 - np.argsort(-key[:, ::-1], axis=1, kind="stable")'),
    "route_weights_renorm_over_all": (
        "        sc = sc / sc.sum(axis=1, keepdims=True)\n    return sc",
        "        sc = sc / np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)\n    return sc"),
    "route_weights_select_bias_in_scores": (
        "bias if bias_mode == LOGIT else None).astype(np.float64)\n    sel",
        "bias).astype(np.float64)\n    sel"),
    "renorm_dropped": (
        "    if renorm:\n        w = w / w.sum(axis=1, keepdims=True)\n    return ids",
        "    return ids"),
    "sigmoid_sign": (
        "        return 1.0 / (1.0 + np.exp(-z))\n    raise ValueError(score)",
        "        return 1.0 / (1.0 + np.exp(z))\n    raise ValueError(score)"),
    "select_bias_ignored": (
        "key = p + (0.0 if bias is None else _f64(bias)[None, :])", "key = p"),
    "select_bias_in_weights": (
        "z32 = biased_logits_f32(logits, bias if bias_mode == LOGIT else None)\n    T, E = z32.shape",
        "z32 = biased_logits_f32(logits, bias)\n    T, E = z32.shape"),
    "group_score_top1": ("[:, :, :min(2, eg)].sum(axis=2)", "[:, :, :1].sum(axis=2)"),
    "group_ties_higher_id": (
        'gbest = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]',
        'gbest = n_groups - 1 - np.argsort(-gscore[:, ::-1], axis=1, kind="stable")[:, :topk_groups]'),
    "aux_probs_unnormalised": ("return s / s.sum(axis=1, keepdims=True), s", "return s, s"),
    "aux_bwd_sign": ("return scale * p * (f[None, :] - inner)", "return scale * p * (f[None, :] + inner)"),
    "aux_bwd_sigmoid_missing_S": (
        "return scale * s * (1.0 - s) / S * (f[None, :] - inner)",
        "return scale * s * (1.0 - s) * (f[None, :] - inner)"),
    "route_bwd_sign": ("dz[rows, ids] = w * (dw - inner)", "dz[rows, ids] = w * (dw + inner)"),
    "route_bwd_sigmoid_renorm_missing_S": ("ds = (dw - inner) / S", "ds = (dw - inner)"),
    "route_bwd_softmax_only_selected": ("dz = -p * inner", "dz = np.zeros_like(p)"),
    "route_bwd_sigmoid_missing_derivative": (
        "dz[rows, ids] = ds * s_sel * (1.0 - s_sel)", "dz[rows, ids] = ds * s_sel"),
    "align_pads_empty_groups": (
        "group_sizes = ((counts + align - 1) // align) * align",
        "group_sizes = (counts // align + 1) * align"),
    "unstable_group_order": ("r = offsets[e] + fill[e]", "r = offsets[e] + (counts[e] - 1 - fill[e])"),
    "capacity_off_by_one": ("counts[e] < capacity:", "counts[e] <= capacity:"),
    "gmm_wrong_group_weight": ("W = _f64(rhs[g])", "W = _f64(rhs[max(g - 1, 0)])"),
    "gmm_ignores_partial": ("out = _f64(partial).copy()\n        M_out", "out = 0 * _f64(partial)\n        M_out"),
    "tgmm_drops_last_row": (
        "out[g] += _f64(lhs[start:start + n]).T @ _f64(rhs[start:start + n])",
        "out[g] += _f64(lhs[start:start + n - 1]).T @ _f64(rhs[start:start + n - 1])"),
    "swiglu_missing_z": ("return h0 * _sigmoid(h0) * _f64(h1)", "return _sigmoid(h0) * _f64(h1)"),
    "swiglu_bwd_dropped_term": ("(1.0 + h0 * (1.0 - sg))", "(1.0 + h0 * sg)"),
    "combine_bwd_missing_weight": ("d_ys[r] = w[t, j] * dy[t]", "d_ys[r] = dy[t]"),
    "permute_bwd_overwrites": ("                dx[t] += d[r]", "                dx[t] = d[r]"),
    "mlp_bias_every_chunk": ("bias=b_wi_0 if last else None", "bias=b_wi_0"),
    "mlp_bias_wrong_group": ("out[start:start + n] += _f64(bias[g])[None, :]",
                             "out[start:start + n] += _f64(bias[max(g - 1, 0)])[None, :]"),
    "group_sum_skips_first_row": ("out[g] = rows[start:start + n].sum(axis=0)",
                                  "out[g] = rows[start + 1:start + n].sum(axis=0)"),
    "bias_grad_wrong_operand": ('out["d_b_wo"] = group_sum(d_ys, gs)', 'out["d_b_wo"] = group_sum(d_act, gs)'),
    "fp8_ties_away": ("r = np.round(a / quantum) * quantum", "r = np.floor(a / quantum + 0.5) * quantum",
                      "fp8"),
    "fp8_no_saturation": ("r = np.minimum(r, top)", "r = r", "fp8"),
    "fp8_scale_inverted": ("f / np.where(am > 0, am, np.float32(1))",
                           "np.where(am > 0, am, np.float32(1)) / f", "fp8"),
    "fp8_backward_in_e4m3": ('g8 = {"d_y_sorted": F8.quantize_tensor(d_ys, F8.E5M2)}',
                             'g8 = {"d_y_sorted": F8.quantize_tensor(d_ys, F8.E4M3)}'),
    "fp8_weights_per_tensor": ("q8[name] = F8.quantize_experts(wt, F8.E4M3)",
                               "q8[name] = (None, None, F8.quantize_tensor(wt.reshape(wt.shape[0] * wt.shape[1], -1), F8.E4M3)[2].reshape(wt.shape))"),
    "backward_d_wo_wrong_operand": ('d_wo = tgmm(fwd["act"], d_ys, gs)', 'd_wo = tgmm(fwd["h1"], d_ys, gs)'),
    "backward_dx_second_gmm_not_accumulated": (
        "d_xs = gmm(d_h1, wi_1, gs, trans_rhs=True, partial=d_xs)",
        "d_xs = gmm(d_h1, wi_1, gs, trans_rhs=True)"),
    "backward_d_wi_1_transposed_role": ("d_wi_1 = tgmm(xs, d_h1, gs)", "d_wi_1 = tgmm(xs, d_h0, gs)"),
    "router_bwd_missing_term": (
        'out["dx"] = dx + d_logits @ _f64(Wg).T', 'out["dx"] = dx'),
}


def _mutant_module(old, new, base=om):
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__package__ = "oracle"          # its relative imports resolve in the oracle package
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_all_pins():
    failures = []
    for name in dir(pins):
        if name.startswith("check_"):
            try:
                getattr(pins, name)()
            except Exception as exc:   # AssertionError or a crash both count as caught
                failures.append((name, type(exc).__name__))
    return failures


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_is_caught(mutation, monkeypatch):
    old, new, *where = MUTATIONS[mutation]
    if where == ["fp8"]:
        # the FP8 module: every user (the pins and the block) sees the mutant
        mod = _mutant_module(old, new, oracle.fp8)
        monkeypatch.setattr(oracle, "fp8", mod)
        monkeypatch.setattr(om, "F8", mod)
        assert _run_all_pins(), f"no pin caught mutation {mutation}"
        return
    mod = _mutant_module(old, new)
    for fname in dir(om):
        obj = getattr(om, fname)
        if isinstance(obj, types.FunctionType) and obj.__module__ == om.__name__:
            monkeypatch.setattr(oracle, fname, getattr(mod, fname), raising=False)
    failures = _run_all_pins()
    assert failures, f"no pin caught mutation {mutation}"


def test_unmutated_passes():
    assert _run_all_pins() == []
