"""Seeded synthetic inputs for the MoE expert-FFN path (CPU, NumPy).

This module is shared by the tests, the benchmark and the oracle's callers.
It holds the workload shapes and draws random numbers; it performs none of
the MoE method's arithmetic (no routing, no permutation, no GEMM, no
activation).  Every tensor is drawn from its own PCG64 stream keyed by
(seed, workload name, tensor name, expert index), so one expert's weights
can be regenerated on their own without drawing the rest.

Workloads follow the shapes the pages use:
  * "tiny"        fp32, T=512, d_model=64, d_ff=128, 8 experts, top-2
  * "mixtral"     bf16, T=8192, d_model=4096, d_ff=14336, 8 experts, top-2
                  (the Mixtral-like shapes named in the TransformerEngine MoE
                  block pull request's multi-process test description)
  * "deepseek_v3" bf16, T=4096, d_model=7168, moe d_ff=2048, 256 experts,
                  top-8, sigmoid scores, Zipf(1.2) expert prior, align 128
                  (MaxText DeepSeek-V3 671B runs on the MaxText pages)
  * "token_drop"  bf16, T=8192, d_model=7168, d_ff=2048, 256 experts, top-1,
                  capacity factor 1.0 (MaxText grouped-GEMM pull request,
                  "Tests": token dropping with one expert per token)
  * "chunked"     bf16, T=4096, d_model=7168 in 4 contracting chunks,
                  d_ff=2048, 64 experts, top-4, Zipf(1.5) prior
                  (MaxText "Overlap moe comms with collective matmul",
                  Description: chunks along the embedding dimension)
plus "mini_*" variants of the same structure at sizes the CPU oracle
finishes in seconds.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "stream", "bf16_round",
    "bf16_bits", "bf16_from_bits", "gen_x", "gen_gate", "gen_expert_weight",
    "gen_expert_weights", "gen_logit_bias", "gen_uniform_logits", "gen_dy",
    "gen_logits_normal", "forced_empty_experts", "gen_mlp_bias",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    D: int                 # d_model (contracting dim of the up-projections)
    F: int                 # d_ff (per-expert hidden width)
    E: int                 # experts
    K: int                 # experts per token (top-k)
    dtype: str             # "f32" or "bf16": storage type of x, weights, activations
    score: str             # "softmax" or "sigmoid"
    renorm: bool           # renormalise the K selected weights to sum to 1
    align: int = 0         # align_size (0 = none)
    capacity: int = 0      # expert capacity C (0 = no dropping)
    logits: str = "gemm"   # "gemm": logits = x . Wg (+ prior); "uniform": U[0,1)
    zipf_s: Optional[float] = None   # Zipf exponent of the expert prior
    n_forced_empty: int = 0          # experts whose prior is -inf
    n_chunks: int = 1                # contracting-dim chunks of the up-projection
    pad_rows_to: int = 0             # lhs row count rounded up to this (0 = none)
    w_std: float = 0.02              # std of Wg, wi_0, wi_1, wo
    seed: int = 0
    bias_mode: str = "logit"         # "select": the bias moves only the selection
    select_bias_std: float = 0.0     # std of the per-expert selection bias ("select")
    n_groups: int = 0                # expert groups of grouped top-K (0 = none)
    topk_groups: int = 0             # groups kept per token
    aux_alpha: float = 0.0           # weight of the load-balancing loss (0 = off)
    mlp_bias_std: float = 0.0        # std of the per-expert MLP biases (0 = no biases)

    @property
    def R(self) -> int:
        return self.T * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 512, 64, 128, 8, 2, "f32", "softmax", True),
        Workload("mixtral", 8192, 4096, 14336, 8, 2, "bf16", "softmax", True),
        Workload("deepseek_v3", 4096, 7168, 2048, 256, 8, "bf16", "sigmoid", True,
                 align=128, zipf_s=1.2, n_forced_empty=8),
        Workload("token_drop", 8192, 7168, 2048, 256, 1, "bf16", "softmax", False,
                 capacity=32, logits="uniform"),
        # seed 3: the seed-0 input has a token whose 4th/5th logits differ by
        # less than twice the float32 router-GEMM rounding, so its selection
        # would not be well posed; seed 3's smallest gap is 3.2e-4
        Workload("chunked", 4096, 7168, 2048, 64, 4, "bf16", "softmax", True,
                 zipf_s=1.5, n_forced_empty=4, n_chunks=4, pad_rows_to=128, seed=3),
        # Same structure at oracle-friendly sizes: several tiles and ragged tails.
        Workload("mini_mixtral", 600, 256, 384, 8, 2, "bf16", "softmax", True),
        # groups of 512 rows or more on average (the 256-row tile regime, where
        # the fused up-projection applies SwiGLU in its epilogue)
        Workload("mini_mixtral_512", 2400, 256, 384, 8, 2, "bf16", "softmax", True),
        Workload("mini_deepseek", 300, 256, 192, 32, 8, "bf16", "sigmoid", True,
                 align=128, zipf_s=1.2, n_forced_empty=4),
        Workload("mini_token_drop", 700, 192, 160, 32, 1, "bf16", "softmax", False,
                 capacity=22, logits="uniform"),
        Workload("mini_chunked", 333, 512, 160, 16, 4, "bf16", "softmax", True,
                 zipf_s=1.5, n_forced_empty=3, n_chunks=4, pad_rows_to=128),
        Workload("mini_align8", 257, 128, 96, 16, 3, "bf16", "softmax", True,
                 align=8, zipf_s=1.2, n_forced_empty=2),
        # router variants: a selection-only expert bias with grouped top-K and
        # the load-balancing loss (sigmoid scores), and the loss with softmax
        Workload("mini_dsv3_router", 320, 256, 192, 32, 4, "bf16", "sigmoid", True,
                 align=16, bias_mode="select", select_bias_std=0.05, n_groups=8,
                 topk_groups=3, aux_alpha=0.01),
        Workload("mini_mixtral_aux", 600, 256, 384, 8, 2, "bf16", "softmax", True,
                 aux_alpha=0.02),
        Workload("tiny_grouped", 512, 64, 128, 8, 2, "f32", "softmax", True,
                 n_groups=4, topk_groups=2, aux_alpha=0.01),
        # per-expert MLP biases on wi_0, wi_1 and wo: fp32, with align_size
        # padding, and under the chunked partial sums
        Workload("tiny_bias", 512, 64, 128, 8, 2, "f32", "softmax", True, mlp_bias_std=0.1),
        Workload("mini_bias_align", 300, 256, 192, 32, 8, "bf16", "sigmoid", True,
                 align=128, zipf_s=1.2, n_forced_empty=4, mlp_bias_std=0.1),
        Workload("mini_bias_chunked", 333, 512, 160, 16, 4, "bf16", "softmax", True,
                 zipf_s=1.5, n_forced_empty=3, n_chunks=4, pad_rows_to=128, mlp_bias_std=0.1),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def _key(s: str) -> int:
    return zlib.crc32(s.encode("utf-8"))


def stream(seed: int, workload: str, tensor: str, index: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one tensor (or one expert's slice of it)."""
    ss = np.random.SeedSequence([int(seed), _key(workload), _key(tensor), int(index)])
    return np.random.Generator(np.random.PCG64(ss))


# ---- bf16 storage -----------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to the float32 values they encode (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly representable in bf16."""
    return bf16_from_bits(bf16_bits(a))


def _bf16_round_inplace(a: np.ndarray) -> np.ndarray:
    """bf16_round without temporaries of the full size but one."""
    u = a.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u &= np.uint32(0xFFFF0000)
    return a


def _store(w: Workload, a: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return _bf16_round_inplace(a) if w.dtype == "bf16" else a


# ---- tensors ----------------------------------------------------------------

def gen_x(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Token activations x [T, D] ~ N(0, 1), stored in the workload dtype."""
    s = w.seed if seed is None else seed
    g = stream(s, w.name, "x")
    return _store(w, g.standard_normal((w.T, w.D), dtype=np.float32))


def gen_gate(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Router kernel Wg [D, E] ~ N(0, w_std^2)."""
    s = w.seed if seed is None else seed
    g = stream(s, w.name, "gate")
    return _store(w, g.standard_normal((w.D, w.E), dtype=np.float32), w.w_std)


def gen_expert_weight(w: Workload, name: str, e: int, seed: Optional[int] = None) -> np.ndarray:
    """One expert's weight: wi_0/wi_1 -> [D, F], wo -> [F, D]; ~ N(0, w_std^2)."""
    s = w.seed if seed is None else seed
    shape = (w.F, w.D) if name == "wo" else (w.D, w.F)
    g = stream(s, w.name, name, e)
    return _store(w, g.standard_normal(shape, dtype=np.float32), w.w_std)


def gen_expert_weights(w: Workload, name: str, seed: Optional[int] = None) -> np.ndarray:
    """All experts' weights stacked: [E, D, F] (wi_0, wi_1) or [E, F, D] (wo)."""
    return np.stack([gen_expert_weight(w, name, e, seed) for e in range(w.E)])


def gen_mlp_bias(w: Workload, name: str, seed: Optional[int] = None) -> Optional[np.ndarray]:
    """Per-expert MLP bias of projection `name`: wi_0/wi_1 -> [E, F], wo ->
    [E, D]; ~ N(0, mlp_bias_std^2) in the workload dtype, or None."""
    if w.mlp_bias_std <= 0:
        return None
    s = w.seed if seed is None else seed
    g = stream(s, w.name, "bias_" + name)
    shape = (w.E, w.D) if name == "wo" else (w.E, w.F)
    return _store(w, g.standard_normal(shape, dtype=np.float32), w.mlp_bias_std)


def forced_empty_experts(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Sorted ids of the experts the prior switches off: 0, E-1 and seeded others."""
    if w.n_forced_empty == 0:
        return np.zeros(0, dtype=np.int64)
    s = w.seed if seed is None else seed
    g = stream(s, w.name, "forced_empty")
    ids = {0, w.E - 1}
    middle = g.permutation(np.arange(1, w.E - 1))
    for e in middle:
        if len(ids) >= w.n_forced_empty:
            break
        ids.add(int(e))
    return np.array(sorted(ids), dtype=np.int64)


def gen_logit_bias(w: Workload, seed: Optional[int] = None) -> Optional[np.ndarray]:
    """Per-expert prior added to the router logits, float32 [E], or None
    (for bias_mode "select": the selection-only bias).

    Zipf(s) popularity: expert e gets rank r(e) from a seeded permutation of
    1..E and prior p_r = r^-s (p_1 = 1), contributing ln p_r = -s ln r to its
    logit.  The forced-empty experts get -inf so they are never selected.
    """
    if w.bias_mode == "select":
        # selection-only expert bias: N(0, select_bias_std^2) per expert
        s = w.seed if seed is None else seed
        bias = (stream(s, w.name, "select_bias").standard_normal(w.E) * w.select_bias_std)
        bias = bias.astype(np.float32)
        bias[forced_empty_experts(w, seed)] = -np.inf
        return bias
    if w.zipf_s is None and w.n_forced_empty == 0:
        return None
    s = w.seed if seed is None else seed
    bias = np.zeros(w.E, dtype=np.float64)
    if w.zipf_s is not None:
        rank = stream(s, w.name, "zipf_rank").permutation(w.E) + 1
        bias = -w.zipf_s * np.log(rank.astype(np.float64))
    bias = bias.astype(np.float32)
    bias[forced_empty_experts(w, seed)] = -np.inf
    return bias


def gen_uniform_logits(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Router logits drawn directly, float32 [T, E] ~ U[0, 1)."""
    s = w.seed if seed is None else seed
    return stream(s, w.name, "uniform_logits").random((w.T, w.E), dtype=np.float32)


def gen_logits_normal(w: Workload, std: float = 1.0, seed: Optional[int] = None,
                      tensor: str = "normal_logits") -> np.ndarray:
    """Router logits drawn directly, float32 [T, E] ~ N(0, std^2)."""
    s = w.seed if seed is None else seed
    return stream(s, w.name, tensor).standard_normal((w.T, w.E), dtype=np.float32) * np.float32(std)


def gen_dy(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Upstream gradient of the block output, [T, D] ~ N(0, 1), workload dtype."""
    s = w.seed if seed is None else seed
    g = stream(s, w.name, "dy")
    return _store(w, g.standard_normal((w.T, w.D), dtype=np.float32))


def chunk_bounds(w: Workload) -> Tuple[int, ...]:
    """Start columns of the contracting-dim chunks of d_model, plus D at the end."""
    n = w.n_chunks
    assert w.D % n == 0, "d_model must split into equal chunks"
    c = w.D // n
    return tuple(i * c for i in range(n + 1))


def device_inputs(w: Workload, device="cuda", threads: int = 8, seed: Optional[int] = None):
    """Seeded inputs of a workload placed on a torch device (no arithmetic:
    values are generated here on the CPU and copied).  Expert weights are
    generated one expert at a time and copied straight into preallocated
    device tensors, so the host never holds all of them.  Returns a dict
    of device tensors (x, dy, Wg, logits, bias, wi_0, wi_1, wo) and the
    small host arrays under "host" (x, dy, Wg, logits, bias)."""
    import concurrent.futures as cf
    import torch

    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dt)

    host = dict(x=gen_x(w, seed), dy=gen_dy(w, seed),
                Wg=gen_gate(w, seed) if w.logits == "gemm" else None,
                logits=gen_uniform_logits(w, seed) if w.logits == "uniform" else None,
                bias=gen_logit_bias(w, seed))
    out = {k: (up(v) if v is not None else None) for k, v in host.items()
           if k in ("x", "dy", "Wg")}
    for k in ("logits", "bias"):
        out[k] = torch.from_numpy(host[k]).to(device) if host[k] is not None else None
    for name in ("wi_0", "wi_1", "wo"):
        shape = (w.E, w.F, w.D) if name == "wo" else (w.E, w.D, w.F)
        out[name] = torch.empty(shape, dtype=dt, device=device)

    def fill(job):
        name, e = job
        a = gen_expert_weight(w, name, e, seed)
        out[name][e].copy_(torch.from_numpy(a).to(dt), non_blocking=False)

    jobs = [(name, e) for name in ("wi_0", "wi_1", "wo") for e in range(w.E)]
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, jobs))
    out["host"] = host
    return out
