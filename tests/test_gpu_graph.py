"""The forward + backward step captured once into a HIP graph (torch.cuda.CUDAGraph
over the library's launches on the capture stream) and replayed.

The step issues only the library's kernels and device-to-device copies (no
host synchronisation, no allocation when the plan owns its buffers, no
memset nodes), and every kernel is deterministic (integer atomics only), so
each replay must reproduce the eager step bit for bit.  Between replays the
outputs are poisoned and unrelated eager work runs on the same device, and
every replay is checked, not only the first.  The eager step itself is
checked against the oracle by the chain tests on the same workloads."""
import pytest
import torch

import moe_synth as ms
from mixture_experts_grouped_top_amd import MoEPlan
from tests.gpu_util import dev, poison
from tests.test_gpu_block import shape_of, workload_inputs

pytestmark = pytest.mark.gpu

CASES = [("tiny", False, False), ("mini_mixtral", False, False), ("mini_deepseek", False, False),
         ("mini_token_drop", False, False), ("mini_chunked", False, False),
         ("mini_dsv3_router", False, False), ("mini_mixtral_aux", False, False),
         ("tiny_bias", False, False), ("mini_bias_chunked", False, False),
         ("mini_deepseek", True, False), ("mini_mixtral_512", True, False),
         ("mini_mixtral", False, True),
         ("mini_deepseek", False, True)]

# step outputs poisoned before each replay
OUTPUTS = ("logits", "ids", "w", "x_sorted", "y", "d_w", "dx", "d_logits", "d_Wg", "d_wo",
           "d_wi_0", "d_wi_1", "d_wi", "d_b_wo", "d_b_wi_0", "d_b_wi_1", "d_b_wi", "aux_loss")


def _buffers(plan):
    """Every device tensor the plan owns except workspaces and the error flag."""
    out = {}
    for k, v in vars(plan).items():
        if k.endswith("ws") or k == "err":
            continue
        if isinstance(v, torch.Tensor) and v.is_cuda:
            out[k] = v
        elif isinstance(v, dict):
            for kk, vv in v.items():
                if isinstance(vv, torch.Tensor) and vv.is_cuda:
                    out[f"{k}.{kk}"] = vv
                elif isinstance(vv, tuple):
                    for i, t in enumerate(vv):
                        if isinstance(t, torch.Tensor) and t.is_cuda:
                            out[f"{k}.{kk}.{i}"] = t
    return out


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (NaN payloads included)."""
    if a.dtype.is_floating_point:
        it = {2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
        return torch.equal(a.view(it), b.view(it))
    return torch.equal(a, b)


@pytest.mark.parametrize("name,fused,fp8", CASES,
                         ids=[f"{n}{'-fused_wi' if fz else ''}{'-fp8' if f8 else ''}"
                              for n, fz, f8 in CASES])
def test_graph_replay_matches_eager(name, fused, fp8):
    w = ms.get_workload(name)
    inp = workload_inputs(w)
    s = shape_of(w, fused, fp8)
    td = s.dtype
    plan = MoEPlan(s)
    x = dev(inp["x"], td)
    W = {k: dev(inp[k], td) for k in ("wi_0", "wi_1", "wo")}
    Wg = dev(inp["Wg"], td) if inp["Wg"] is not None else None
    logits = dev(inp["logits"]) if inp["logits"] is not None else None
    bias = dev(inp["bias"]) if inp["bias"] is not None else None
    dy = dev(inp["dy"], td)
    wi = torch.cat([W["wi_0"], W["wi_1"]], dim=2).contiguous() if fused else None
    mb = None
    if inp["mlp"] is not None:
        mb = {k: dev(v, td) for k, v in inp["mlp"].items()}
        if fused:
            mb["wi"] = torch.cat([mb["wi_0"], mb["wi_1"]], dim=1).contiguous()

    def step():
        plan.forward(x, W["wi_0"], W["wi_1"], W["wo"], Wg=Wg, logits=logits, bias=bias, wi=wi,
                     mlp_bias=mb)
        plan.backward(dy, x, W["wi_0"], W["wi_1"], W["wo"], Wg=Wg, bias=bias, wi=wi)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert int(plan.err.item()) == 0
    bufs = _buffers(plan)
    eager = {k: v.clone() for k, v in bufs.items()}
    # d_Wg is written only with a router GEMM (not for given logits)
    poisoned = [k for k in OUTPUTS if getattr(plan, k, None) is not None
                and (k != "d_Wg" or Wg is not None)]
    assert "y" in poisoned and "dx" in poisoned

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for k in poisoned:
            poison(getattr(plan, k))
        # unrelated eager work between replays
        z = torch.randn(1 << 20, device="cuda")
        _ = (z * z).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert int(plan.err.item()) == 0
        bad = [k for k, v in bufs.items() if not _same(v, eager[k])]
        assert not bad, f"replay {rep}: differs from the eager step in {bad}"
    del g
    torch.cuda.synchronize()
