"""FP8 expert GEMMs at the workloads' full sizes, in the launch configuration
the benchmark times (`MoEPlan` with fp8: current scaling, e4m3 forward, e5m2
backward, one row-wise FP8 copy per weight read in both orientations).

The oracle cannot run the whole step at these sizes, so for a few sampled
experts (the largest, the smallest and the median non-empty one, and the
smallest of each weight-gradient size class):
  * the expert's FP8 weight codes and scale are checked bit for bit against
    the oracle's per-expert quantizer on the same bf16 weights;
  * every FP8 GEMM of the step is checked on that expert's rows against the
    oracle on the step's own codes and scales (its quantized inputs,
    dequantized in float64) at the bf16 tolerance: h0, h1, y_sorted, d_act,
    d_x_sorted and the weight gradients d_wo, d_wi_0, d_wi_1;
and the weight gradients of every empty expert are zero."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from mixture_experts_grouped_top_amd import MoEPlan, MoEShape
from tests.gpu_util import TOL_BF16, assert_close, host
from tests.test_gpu_fullsize import sampled_experts

pytestmark = [pytest.mark.gpu]

F8 = oracle.fp8
FULL8 = ["mixtral", "deepseek_v3"]


@pytest.fixture(scope="module", params=FULL8)
def full8(request):
    w = ms.get_workload(request.param)
    dev = ms.device_inputs(w, threads=16)
    shape = MoEShape(T=w.T, D=w.D, F=w.F, E=w.E, K=w.K, score=w.score, renorm=w.renorm,
                     align=w.align, capacity=w.capacity, fp8=True)
    plan = MoEPlan(shape)
    plan.forward(dev["x"], dev["wi_0"], dev["wi_1"], dev["wo"], Wg=dev["Wg"],
                 logits=dev["logits"], bias=dev["bias"])
    plan.backward(dev["dy"], dev["x"], dev["wi_0"], dev["wi_1"], dev["wo"], Wg=dev["Wg"],
                  bias=dev["bias"])
    torch.cuda.synchronize()
    assert int(plan.err.item()) == 0
    yield w, plan
    del dev, plan
    torch.cuda.empty_cache()


def _deq_rows(plan, name, fmt, r0, r1):
    """Rows r0..r1 of an activation's row-wise codes, dequantized (float64)."""
    qr, _, sc = plan.q8[name]
    return F8.dequantize(host(qr[r0:r1]), fmt, float(host(sc[2])[0]))


def _deq_weight(plan, name, e):
    qr, _, sc = plan.q8[name]
    return F8.dequantize(host(qr[e]), "e4m3", float(host(sc[2])[e]))


def test_full_fp8_weight_codes(full8):
    """The sampled experts' weight codes and scales equal the oracle's
    per-expert current scaling of the same bf16 weights, bit for bit."""
    w, plan = full8
    counts = host(plan.idx["counts"]).astype(np.int64)
    for e in sampled_experts(counts):
        for name in ("wi_0", "wi_1", "wo"):
            codes, si, _ = F8.quantize_experts(ms.gen_expert_weight(w, name, e)[None], "e4m3")
            qr, _, sc = plan.q8[name]
            assert (host(qr[e]) == codes[0]).all(), (name, e)
            assert host(sc[2])[e] == si[0], (name, e)


def test_full_fp8_gemms_on_step_codes(full8):
    w, plan = full8
    counts = host(plan.idx["counts"]).astype(np.int64)
    gs = host(plan.idx["group_sizes"]).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(gs)])
    for e in sampled_experts(counts):
        r0, n, kept = int(off[e]), int(gs[e]), int(counts[e])
        r1 = r0 + n
        X = _deq_rows(plan, "x", "e4m3", r0, r1)
        A = _deq_rows(plan, "act", "e4m3", r0, r1)
        DY = _deq_rows(plan, "d_y_sorted", "e5m2", r0, r1)
        DH = [_deq_rows(plan, f"d_h{i}", "e5m2", r0, r1) for i in range(2)]
        Wd = {k: _deq_weight(plan, k, e) for k in ("wi_0", "wi_1", "wo")}
        what = f"expert {e} ({kept} rows)"
        # forward: the up-projections read the [D, F] copies as [K, N], the
        # down-projection the [F, D] copy
        for i in range(2):
            got = host(getattr(plan, f"h{i}")[r0:r1]).astype(np.float64)
            assert_close(got[:kept], X[:kept] @ Wd[f"wi_{i}"], TOL_BF16, f"h{i}, {what}")
            assert (got[kept:] == 0).all(), f"h{i} padding rows, {what}"
        got = host(plan.y_sorted[r0:r1]).astype(np.float64)
        assert_close(got[:kept], A[:kept] @ Wd["wo"], TOL_BF16, f"y_sorted, {what}")
        # backward: d_lhs products read the same copies as [N, K]
        got = host(plan.d_act[r0:r1]).astype(np.float64)
        assert_close(got[:kept], DY[:kept] @ Wd["wo"].T, TOL_BF16, f"d_act, {what}")
        got = host(plan.d_x_sorted[r0:r1]).astype(np.float64)
        want = DH[0][:kept] @ Wd["wi_0"].T + DH[1][:kept] @ Wd["wi_1"].T
        assert_close(got[:kept], want, TOL_BF16, f"d_x_sorted, {what}")
        # weight gradients over the kept rows
        assert_close(host(plan.d_wo[e]).astype(np.float64), A[:kept].T @ DY[:kept], TOL_BF16,
                     f"d_wo, {what}")
        for i in range(2):
            assert_close(host(getattr(plan, f"d_wi_{i}")[e]).astype(np.float64),
                         X[:kept].T @ DH[i][:kept], TOL_BF16, f"d_wi_{i}, {what}")


def test_full_fp8_empty_expert_gradients(full8):
    w, plan = full8
    counts = plan.idx["counts"]
    empty = (counts == 0).nonzero().flatten()
    if w.n_forced_empty:
        assert empty.numel() >= w.n_forced_empty
    for name in ("d_wo", "d_wi_0", "d_wi_1"):
        g = getattr(plan, name)
        assert int(torch.count_nonzero(g[empty]).item()) == 0, name
