"""The seeded input generator: determinism, bf16 rounding, workload structure."""
import numpy as np
import torch

import moe_synth as ms


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0, 65504.0],
                                 dtype=np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ms.bf16_bits(a) == want).all()
    r = ms.bf16_round(a)
    assert (ms.bf16_round(r) == r).all()


def test_deterministic_and_keyed():
    w = ms.get_workload("mini_deepseek")
    assert (ms.gen_x(w) == ms.gen_x(w)).all()
    a = ms.gen_expert_weight(w, "wi_0", 3)
    assert (ms.gen_expert_weights(w, "wi_0")[3] == a).all()
    assert not (ms.gen_expert_weight(w, "wi_0", 4) == a).all()
    assert not (ms.gen_expert_weight(w, "wi_1", 3) == a).all()
    assert ms.gen_expert_weight(w, "wo", 0).shape == (w.F, w.D)


def test_prior_structure():
    for name in ("deepseek_v3", "chunked", "mini_deepseek", "mini_chunked"):
        w = ms.get_workload(name)
        b = ms.gen_logit_bias(w)
        off = np.where(np.isneginf(b))[0]
        assert len(off) == w.n_forced_empty and off[0] == 0 and off[-1] == w.E - 1
        finite = np.sort(b[np.isfinite(b)])[::-1]
        # the remaining priors are -s ln r for distinct ranks r
        ranks = np.exp(-finite.astype(np.float64) / w.zipf_s)
        assert np.allclose(ranks, np.round(ranks), rtol=1e-5)
        assert len(set(np.round(ranks).astype(int))) == len(finite)


def test_workload_sizes():
    w = ms.get_workload("deepseek_v3")
    assert (w.T, w.D, w.F, w.E, w.K, w.align) == (4096, 7168, 2048, 256, 8, 128)
    w = ms.get_workload("token_drop")
    assert w.capacity == -(-w.T * w.K // w.E)      # capacity factor 1.0
    assert ms.chunk_bounds(ms.get_workload("chunked")) == (0, 1792, 3584, 5376, 7168)
