"""Each C-ABI entry point against the float64 oracle, element by element, on
seeded inputs that span several tiles, ragged tails and the degenerate
cases (empty groups, one-row groups, no rows, ties, dropped slots)."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, dev, dev_i32, host, max_rel, poison)
from tests.margins import decision_margins, selection_keys

pytestmark = pytest.mark.gpu

MODES = [("softmax", True), ("softmax", False), ("sigmoid", True), ("sigmoid", False)]


def _topk_ids(g, T, E, K, off=()):
    """K distinct experts per token from a Zipf-skewed distribution (Gumbel
    top-k), never choosing the experts in `off`."""
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    logp = np.log(p / p.sum())
    logp[list(off)] = -np.inf
    gum = g.gumbel(size=(T, E))
    return np.argsort(-(logp[None, :] + gum), axis=1, kind="stable")[:, :K].astype(np.int32)


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("E,K", [(8, 2), (33, 3), (64, 8), (256, 8), (1024, 4), (5, 5), (1, 1)])
@pytest.mark.parametrize("score,renorm", MODES)
def test_route(gpu_lib, E, K, score, renorm):
    g = np.random.default_rng(1000 * E + K)
    T = 301
    z = (g.standard_normal((T, E)) * 2).astype(np.float32)
    z[::5] = np.round(z[::5])                 # rows full of exact ties
    bias = None
    if E >= 8:
        bias = (-1.2 * np.log(g.permutation(E) + 1.0)).astype(np.float32)
        bias[[0, E - 1]] = -np.inf
    ids, w = gpu_lib.moe_route(dev(z), K, score, renorm,
                               bias=None if bias is None else dev(bias))
    oi, ow = oracle.route(z, K, score, renorm, bias)
    assert (host(ids) == oi).all()
    assert_close(host(w), ow, TOL_F32, "topk_w")


@pytest.mark.parametrize("E,K", [(8, 2), (64, 8), (256, 8), (9, 1)])
@pytest.mark.parametrize("score,renorm", MODES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_route_bwd(gpu_lib, E, K, score, renorm, dtype):
    g = np.random.default_rng(7 * E + K)
    T = 257
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (-np.log(np.arange(1, E + 1))).astype(np.float32)
    dw = g.standard_normal((T, K)).astype(np.float32)
    oi, _ = oracle.route(z, K, score, renorm, bias)
    d = gpu_lib.moe_route_bwd(dev(z), dev_i32(oi), dev(dw), score, renorm, bias=dev(bias),
                              dtype=dtype)
    want = oracle.route_bwd(z, oi, dw, score, renorm, bias)
    assert_close(host(d), want, TOL_F32 if dtype == torch.float32 else TOL_BF16, "d_logits")


VARIANTS = [
    # E, K, n_groups, topk_groups, bias_mode, score, renorm
    (256, 8, 8, 4, "select", "sigmoid", True),    # DeepSeek-V3 routing
    (256, 8, 8, 4, "logit", "softmax", True),
    (64, 6, 8, 3, "select", "softmax", False),
    (160, 6, 8, 3, "select", "sigmoid", False),
    (64, 4, 64, 4, "select", "sigmoid", True),    # one expert per group
    (32, 2, 0, 0, "select", "sigmoid", False),    # selection bias, no groups
    (8, 8, 4, 4, "logit", "softmax", True),       # every group and expert kept
    (1024, 4, 32, 2, "select", "sigmoid", True),
    (128, 3, 64, 2, "logit", "sigmoid", True),    # most groups, two experts each
]


def _valid_selection(key, sel, K, n_groups, topk_groups, tol):
    """Whether ids `sel` (length K) of one token form a (grouped) top-K of
    the float64 keys `key` [E] up to `tol`: distinct and in range; their
    groups can all be among the topk_groups best (each within tol of the
    topk_groups-th group score, at most topk_groups of them, and every group
    above the (topk_groups+1)-th score by more than tol kept); keys in
    descending order; no eligible unselected expert (in a chosen or a
    certainly kept group) above the smallest selected key by more than tol.
    Returns a reason string, or "" for a valid selection."""
    E = key.size
    sel = np.asarray(sel, dtype=np.int64)
    if len(set(sel.tolist())) != K or sel.min() < 0 or sel.max() >= E:
        return "ids not distinct and in range"
    eligible = np.ones(E, dtype=bool)
    if n_groups > 1:
        eg = E // n_groups
        gs = -np.sort(-key.reshape(n_groups, eg))[:, :min(2, eg)].sum(axis=1)
        order = np.sort(gs)[::-1]
        thr = order[topk_groups - 1]
        nxt = order[topk_groups] if topk_groups < n_groups else -np.inf
        chosen = set((sel // eg).tolist())
        certain = set(np.nonzero(gs > nxt + tol)[0].tolist())
        if len(chosen | certain) > topk_groups:
            return "more groups than topk_groups"
        if any(gs[c] < thr - tol for c in chosen):
            return "an expert from a group outside the best topk_groups"
        eligible = np.isin(np.arange(E) // eg, sorted(chosen | certain))
    ks = key[sel]
    if np.any(ks[:-1] < ks[1:] - tol):
        return "slots not in descending key order"
    rest = eligible.copy()
    rest[sel] = False
    if rest.any() and ks.min() < key[rest].max() - tol:
        return "an unselected eligible expert has a larger key"
    return ""


@pytest.mark.parametrize("case", VARIANTS, ids=[str(c) for c in VARIANTS])
def test_route_variants(gpu_lib, case):
    E, K, G, TG, mode, score, renorm = case
    g = np.random.default_rng(E * 31 + K * 7 + G)
    T = 301
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    z[::7] = np.round(z[::7])                 # exact ties in the logits
    if mode == "select":
        bias = (g.standard_normal(E) * 0.05).astype(np.float32)
    else:
        bias = (-0.5 * np.log(g.permutation(E) + 1.0)).astype(np.float32)
    if E >= 32:
        bias[[1, E - 2]] = -np.inf            # never selected
    ids, w = gpu_lib.moe_route(dev(z), K, score, renorm, bias=dev(bias), bias_mode=mode,
                               n_groups=G, topk_groups=TG)
    oi, ow = oracle.route(z, K, score, renorm, bias, bias_mode=mode, n_groups=G, topk_groups=TG)
    gi, gw = host(ids), host(w)
    # The GPU ranks float32 keys, the oracle float64 ones: their selections
    # may differ only at a token whose decision margin is below the keys'
    # float32 rounding (1e-6 here; exact for plain logit keys).  Every such
    # token must still hold a valid (grouped) top-K of the float64 keys
    # within that margin, and every token's weights must be the oracle's
    # weights of the experts the GPU chose.
    tol = 0.0 if mode == "logit" and G <= 1 else 1e-6
    keys = selection_keys(z, bias, score, mode)
    margin = decision_margins(keys, K, G, TG)
    same = (gi == oi).all(axis=1)
    assert (same | (margin < tol)).all(), np.nonzero(~(same | (margin < tol)))[0][:8]
    for t in np.nonzero(~same)[0]:
        why = _valid_selection(keys[t], gi[t], K, G, TG, tol)
        assert not why, (t, why, gi[t], oi[t])
    want = oracle.route_weights(z, gi, score, renorm, bias, bias_mode=mode)
    assert_close(gw, want, TOL_F32, "topk_w")
    assert_close(gw[same], ow[same], TOL_F32, "topk_w (oracle selection)")


@pytest.mark.parametrize("score,renorm", MODES)
def test_route_bwd_select_bias(gpu_lib, score, renorm):
    """With a selection-only bias the weights are scores of the logits
    themselves, so the gradient ignores the bias."""
    g = np.random.default_rng(5)
    T, E, K = 263, 64, 6
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (g.standard_normal(E) * 0.05).astype(np.float32)
    dw = g.standard_normal((T, K)).astype(np.float32)
    oi, _ = oracle.route(z, K, score, renorm, bias, bias_mode="select", n_groups=8, topk_groups=3)
    d = gpu_lib.moe_route_bwd(dev(z), dev_i32(oi), dev(dw), score, renorm, bias=dev(bias),
                              bias_mode="select")
    want = oracle.route_bwd(z, oi, dw, score, renorm, bias, bias_mode="select")
    assert_close(host(d), want, TOL_F32, "d_logits")


@pytest.mark.parametrize("T,D,E", [(1024, 256, 8), (777, 136, 33), (4096, 512, 256),
                                   (300, 64, 1), (0, 64, 8), (9000, 128, 64)])
@pytest.mark.parametrize("dx_dtype", [torch.float32, torch.bfloat16])
def test_router_bwd(gpu_lib, T, D, E, dx_dtype):
    """d_Wg = x^T d_logits and dx += d_logits Wg^T with float32 d_logits:
    float32 accuracy (the exact three-plane split loses nothing), including
    d_logits values with all 24 significand bits set, tiny and huge ones."""
    g = np.random.default_rng(T + 7 * D + E)
    x = ms.bf16_round(g.standard_normal((T, D)).astype(np.float32))
    Wg = ms.bf16_round((g.standard_normal((D, E)) * 0.02).astype(np.float32))
    dl = (g.standard_normal((T, E)) * 1e-3).astype(np.float32)
    if T > 8:
        dl[1] = np.float32(1 + 2.0 ** -23) * 3e-4               # full 24-bit significands
        dl[2] = (g.standard_normal(E) * 1e-30).astype(np.float32)
        dl[3] = (g.standard_normal(E) * 1e4).astype(np.float32)
    dx0 = ms.bf16_round(g.standard_normal((T, D)).astype(np.float32))
    dx = dev(dx0, dx_dtype)
    d_Wg, dx = gpu_lib.moe_router_bwd(dev(x, torch.bfloat16), dev(Wg, torch.bfloat16), dev(dl),
                                      dx=dx, accumulate_dx=True)
    want_w = oracle.tgmm(x, dl, np.array([T], np.int32))[0]
    assert_close(host(d_Wg), want_w, TOL_F32, "d_Wg")
    want_x = oracle.gmm(dl, Wg.T[None], np.array([T], np.int32), partial=dx0)
    tol = TOL_F32 if dx_dtype == torch.float32 else TOL_BF16
    if T > 0:
        assert_close(host(dx), want_x, tol, "dx")
    # deterministic
    d_Wg2, _ = gpu_lib.moe_router_bwd(dev(x, torch.bfloat16), dev(Wg, torch.bfloat16), dev(dl),
                                      dx=dev(dx0, dx_dtype), accumulate_dx=True)
    assert torch.equal(d_Wg, d_Wg2)


AUX = [
    # T, E, K, score
    (301, 8, 2, "softmax"),
    (1000, 256, 8, "sigmoid"),
    (700, 64, 6, "softmax"),
    (257, 1024, 4, "sigmoid"),          # the largest expert count, several blocks
    (1, 5, 5, "softmax"),
]


@pytest.mark.parametrize("case", AUX, ids=[str(c) for c in AUX])
def test_aux_loss(gpu_lib, case):
    T, E, K, score = case
    g = np.random.default_rng(T + E)
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    ids = _topk_ids(g, T, E, K)
    alpha = 0.01
    loss, counts, probs = gpu_lib.moe_aux_loss(dev(z), dev_i32(ids), alpha, score)
    o_loss, o_counts, o_P = oracle.aux_loss(z, ids, E, alpha, score)
    assert (host(counts) == o_counts).all()
    assert_close(host(probs), o_P, TOL_F32, "aux probs")
    assert abs(float(host(loss)[0]) - o_loss) <= TOL_F32 * abs(o_loss)
    want = oracle.aux_loss_bwd(z, o_counts, K, alpha, score)
    d = gpu_lib.moe_aux_loss_bwd(dev(z), counts, K, alpha, score)
    assert_close(host(d), want, TOL_F32, "aux d_logits")
    # accumulate onto an existing gradient, in bf16
    base = g.standard_normal((T, E)).astype(np.float32) * 1e-3
    acc = dev(base, torch.bfloat16)
    start = host(acc).astype(np.float64)
    gpu_lib.moe_aux_loss_bwd(dev(z), counts, K, alpha, score, d_logits=acc, accumulate=True)
    assert_close(host(acc), start + want, TOL_BF16, "aux d_logits accumulated")


def test_aux_loss_no_tokens(gpu_lib):
    """The loss divides by T: no tokens is an argument error, while the
    gradient of no tokens is empty and succeeds."""
    z = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.MoeError):
        gpu_lib.moe_aux_loss(z, ids, 0.01, "sigmoid")
    counts = torch.zeros(16, dtype=torch.int32, device="cuda")
    assert gpu_lib.moe_aux_loss_bwd(z, counts, 2, 0.01, "sigmoid").shape == (0, 16)


# ------------------------------------------------------------- permutation

PERMUTE_CASES = [
    # T, K, E, align, capacity, capacity_layout, extra rows, forced-empty experts
    (300, 2, 8, 0, 0, False, 0, (0,)),
    (1500, 2, 8, 0, 0, False, 0, ()),          # several histogram blocks
    (700, 8, 256, 128, 0, False, 0, (0, 5, 255)),
    (257, 3, 12, 8, 0, False, 5, (11,)),       # buffer larger than the bound
    (2000, 1, 64, 0, 20, False, 0, (3,)),      # dropping, compact layout
    (2000, 1, 64, 0, 20, True, 0, (3,)),       # dropping, capacity layout
    (2000, 2, 64, 16, 30, False, 0, ()),       # dropping + align
    (100, 1, 1, 0, 0, False, 0, ()),           # one expert
    (0, 2, 8, 0, 0, False, 0, ()),             # no tokens
    (3000, 4, 1024, 16, 0, False, 0, (1023,)),
]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=[str(c[:7]) for c in PERMUTE_CASES])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute(gpu_lib, case, dtype):
    T, K, E, a, C, lay, extra, off = case
    g = np.random.default_rng(T + 31 * E + K)
    ids = _topk_ids(g, T, E, K, off) if T else np.zeros((0, K), np.int32)
    D = 136
    x = g.standard_normal((T, D)).astype(np.float32)
    if dtype == torch.bfloat16:
        x = ms.bf16_round(x)
    rows = oracle.rows_bound(T, K, E, a, C, lay) + extra
    want = oracle.permute(x, ids, E, a, C, lay, rows=rows)
    xs = poison(torch.empty((rows, D), dtype=dtype, device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = gpu_lib.moe_permute(dev(x, dtype), dev_i32(ids), E, a, C, lay, rows=rows, x_sorted=xs,
                              err=err)
    for k in ("counts", "group_sizes", "group_offsets", "row_of_slot", "slot_of_row"):
        assert (host(got[k]) == want[k]).all(), k
    assert (host(xs) == want["x_sorted"]).all()      # a copy: bit-exact
    assert host(err)[0] == 0


def test_permute_invalid_ids_flagged(gpu_lib):
    g = np.random.default_rng(5)
    T, K, E = 200, 2, 8
    ids = _topk_ids(g, T, E, K)
    ids[3, 1] = E
    ids[77, 0] = -1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = gpu_lib.moe_permute(None, dev_i32(ids), E, err=err)
    ros = host(got["row_of_slot"])
    assert host(err)[0] & gpu_lib.MOE_DERR_EXPERT_ID
    assert ros[3 * K + 1] == -1 and ros[77 * K] == -1
    real = ros[ros >= 0]
    assert sorted(real.tolist()) == list(range(T * K - 2))


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
@pytest.mark.parametrize("case", [(300, 2, 8, 0, 0, False), (400, 8, 64, 16, 0, False),
                                  (900, 1, 32, 0, 20, False), (900, 1, 32, 0, 20, True)])
def test_combine_and_backward(gpu_lib, dtype, tol, case):
    T, K, E, a, C, lay = case
    g = np.random.default_rng(T * K)
    D = 264
    ids = _topk_ids(g, T, E, K, (1,))
    P = oracle.permute(None, ids, E, a, C, lay)
    rows = P["slot_of_row"].size
    ys = g.standard_normal((rows, D)).astype(np.float32)
    dy = g.standard_normal((T, D)).astype(np.float32)
    dxs = g.standard_normal((rows, D)).astype(np.float32)
    if dtype == torch.bfloat16:
        ys, dy, dxs = ms.bf16_round(ys), ms.bf16_round(dy), ms.bf16_round(dxs)
    w = g.random((T, K)).astype(np.float32)
    ros, sor = dev_i32(P["row_of_slot"]), dev_i32(P["slot_of_row"])
    y = gpu_lib.moe_combine(dev(ys, dtype), ros, dev(w))
    assert_close(host(y), oracle.combine(ys, P["row_of_slot"], w, T, K), tol, "combine")
    d_ys = poison(torch.empty((rows, D), dtype=dtype, device="cuda"))
    d_w = poison(torch.empty((T, K), dtype=torch.float32, device="cuda"))
    gpu_lib.moe_combine_bwd(dev(dy, dtype), dev(ys, dtype), ros, sor, dev(w), d_y_sorted=d_ys,
                            d_topk_w=d_w)
    w_ys, w_dw = oracle.combine_bwd(dy, ys, P["row_of_slot"], w, rows)
    assert_close(host(d_ys), w_ys, tol, "d_y_sorted")
    assert_close(host(d_w), w_dw, TOL_F32, "d_topk_w")
    dx = gpu_lib.moe_permute_bwd(dev(dxs, dtype), ros, T, K)
    assert_close(host(dx), oracle.permute_bwd(dxs, P["row_of_slot"], T, K), tol, "permute_bwd")
    base = g.standard_normal((T, D)).astype(np.float32)
    if dtype == torch.bfloat16:
        base = ms.bf16_round(base)
    dx2 = dev(base, dtype)
    gpu_lib.moe_permute_bwd(dev(dxs, dtype), ros, T, K, d_x=dx2, accumulate=True)
    assert_close(host(dx2), base + oracle.permute_bwd(dxs, P["row_of_slot"], T, K), tol,
                 "permute_bwd accumulate")


# ------------------------------------------------------------ grouped GEMMs

GS = {
    "ragged": [130, 0, 257, 1, 64, 0, 300],
    "empty_first": [0, 0, 128, 256],
    "one_group": [517],
    "two_big": [800, 0, 900],      # >= 512 rows per group: 256-row tiles
    "all_empty": [0, 0, 0],
    "aligned": [128, 256, 0, 384],
    # more groups than the 128-row tile variant holds (1000): 256-row tiles
    "many": [(i * 7) % 3 for i in range(1010)],
    "max_groups": [(i * 5) % 4 for i in range(1024)],
    # skewed short contractions over many tiles per workgroup
    "skewed": [(i * 37) % 300 for i in range(64)],
    # mostly small groups (128-row tiles) with some above 384 rows (256-row
    # tiles in a launch of their own)
    "mixed": [30, 700, 0, 385, 384, 1100, 5, 0, 129, 40],
    # contractions of at most 64 rows (one or two steps, full and ragged)
    "shortk": [33, 64, 47, 0, 5, 63, 32, 1, 17],
    # contractions of 65 .. 128 rows (three or four steps), beside shorter ones
    "midk": [65, 128, 96, 0, 97, 100, 127, 3, 70, 40],
    # 900 groups of 0 .. 128 rows: every short class, group tables near their limit
    "many_short": [(i * 37) % 129 for i in range(900)],
}

GMM_CASES = [
    # groups, Kdim, N, extra lhs rows, out rows short of lhs, trans, in, out, accumulate
    ("ragged", 192, 136, 7, 0, False, "bf16", "f32", False),
    ("ragged", 192, 136, 7, 0, True, "bf16", "f32", False),
    ("ragged", 200, 256, 0, 0, False, "bf16", "bf16", False),
    ("ragged", 512, 128, 3, 0, True, "bf16", "bf16", False),
    ("empty_first", 64, 264, 0, 0, False, "bf16", "f32", True),
    ("empty_first", 64, 264, 0, 0, True, "bf16", "f32", True),
    ("one_group", 136, 8, 0, 0, False, "bf16", "f32", False),     # router-like, N = 8
    ("one_group", 8, 136, 0, 0, True, "bf16", "bf16", True),      # Kdim = 8
    ("all_empty", 64, 128, 9, 0, False, "bf16", "f32", False),
    ("aligned", 128, 128, 128, 100, False, "bf16", "f32", True),  # padded lhs, shorter out
    ("ragged", 72, 40, 5, 0, False, "f32", "f32", False),
    ("ragged", 72, 40, 5, 0, True, "f32", "f32", True),
    ("one_group", 96, 8, 0, 0, False, "f32", "f32", False),
    ("aligned", 64, 24, 64, 30, True, "f32", "bf16", False),
    ("one_group", 96, 264, 0, 0, False, "bf16", "bf16", False),  # 256 x 256 tiles, odd steps
    ("one_group", 200, 264, 0, 0, False, "bf16", "f32", False),  # 128-byte row segments + tail
    ("one_group", 200, 264, 0, 0, True, "bf16", "bf16", True),
    ("one_group", 1024, 264, 3, 0, False, "bf16", "bf16", False),  # long pipelined run
    ("one_group", 1024, 136, 3, 0, True, "bf16", "f32", True),
    ("mixed", 264, 520, 3, 0, False, "bf16", "bf16", False),
    ("mixed", 256, 264, 0, 0, True, "bf16", "f32", True),
    ("mixed", 200, 136, 0, 0, False, "bf16", "f32", True),
    ("two_big", 264, 520, 0, 0, True, "bf16", "bf16", False),
    ("two_big", 136, 520, 5, 0, False, "bf16", "f32", True),
    ("one_group", 96, 264, 0, 0, True, "bf16", "f32", True),
    ("many", 64, 136, 3, 0, False, "bf16", "bf16", False),
    ("max_groups", 64, 136, 0, 0, True, "bf16", "f32", True),
]


def _draw(g, shape, dt):
    a = g.standard_normal(shape).astype(np.float32)
    return ms.bf16_round(a) if dt == "bf16" else a


TD = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("with_bias", [False, True], ids=["", "bias"])
@pytest.mark.parametrize("case", GMM_CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}-t{int(c[5])}-{c[6]}{c[7]}-a{int(c[8])}" for c in GMM_CASES])
def test_gmm(gpu_lib, case, with_bias):
    name, Kd, N, extra, short, trans, it, ot, acc = case
    gs = np.array(GS[name], dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(Kd * 1000 + N + extra)
    M_lhs = int(gs.sum()) + extra
    M_out = M_lhs - short
    lhs = _draw(g, (M_lhs, Kd), it)
    rhs = _draw(g, (G, N, Kd) if trans else (G, Kd, N), it)
    P = _draw(g, (M_out, N), ot) if acc else None
    out = dev(P, TD[ot]) if acc else poison(torch.empty((M_out, N), dtype=TD[ot], device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bias = _draw(g, (G, N), it) if with_bias else None
    gpu_lib.moe_gmm(dev(lhs, TD[it]), dev(rhs, TD[it]), dev_i32(gs), trans_rhs=trans, out=out,
                    accumulate=acc, err=err, bias=None if bias is None else dev(bias, TD[it]))
    want = oracle.gmm(lhs, rhs, gs, trans_rhs=trans, partial=P, rows_out=M_out, bias=bias)
    got = host(out)
    tol = TOL_F32 if ot == "f32" else TOL_BF16
    assert_close(got, want, tol, "gmm")
    S = int(gs.sum())
    if acc:
        assert (got[S:] == P[S:]).all()           # rows past the groups untouched
    else:
        assert (got[S:] == 0).all()               # rows past the groups zero-filled
    assert host(err)[0] == 0


GMM_VALID = [
    # group sizes, valid rows, K, N, trans, accumulate
    ([300, 0, 257, 128, 1000], [299, 0, 1, 0, 613], 264, 136, False, False),   # 128-row tiles
    ([300, 0, 257, 128, 1000], [299, 0, 1, 0, 613], 136, 264, True, True),
    ([1024, 1024], [1000, 3], 512, 264, False, False),                         # 256-row pair tiles
    ([1024, 1024], [1000, 3], 512, 264, True, False),
    ([517], [0], 64, 8, False, True),                                         # no valid row at all
    # 128-row tiles whose valid rows end at and around the 32-row fragment
    # boundaries of its waves (fragments past them take no MFMAs)
    ([128] * 10 + [384], [1, 31, 32, 33, 63, 64, 65, 96, 97, 128, 300], 264, 264, False, False),
    ([128] * 10 + [384], [1, 31, 32, 33, 63, 64, 65, 96, 97, 128, 300], 264, 264, True, True),
]


@pytest.mark.parametrize("case", GMM_VALID, ids=[str(i) for i in range(len(GMM_VALID))])
def test_gmm_valid_rows(gpu_lib, case):
    """Rows past valid_rows[g] of each group are not read (garbage here) and
    give zero products: the result equals the oracle with those rows zeroed,
    plus the bias and the partial sum on every row of the group."""
    gs, valid, K, N, trans, acc = case
    gs = np.array(gs, dtype=np.int32)
    valid = np.array(valid, dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(K + N)
    M = int(gs.sum())
    lhs = _draw(g, (M, K), "bf16")
    rhs = _draw(g, (G, N, K) if trans else (G, K, N), "bf16")
    bias = _draw(g, (G, N), "bf16")
    lhs0 = lhs.copy()
    off = np.concatenate([[0], np.cumsum(gs)])
    for e in range(G):
        lhs0[off[e] + valid[e]:off[e + 1]] = 0
    P = _draw(g, (M, N), "f32") if acc else None
    out = dev(P) if acc else poison(torch.empty((M, N), dtype=torch.float32, device="cuda"))
    gpu_lib.moe_gmm(dev(lhs, torch.bfloat16), dev(rhs, torch.bfloat16), dev_i32(gs), trans_rhs=trans,
                    out=out, accumulate=acc, bias=dev(bias, torch.bfloat16),
                    valid_rows=dev_i32(valid))
    want = oracle.gmm(lhs0, rhs, gs, trans_rhs=trans, partial=P, bias=bias)
    assert_close(host(out), want, TOL_F32, "gmm valid_rows")


SWI_CASES = [
    # group sizes, valid rows, K, F, bias, write h, extra output rows
    ([300, 0, 257, 128, 1000], None, 264, 256, False, True, 7),      # 128-row tiles
    ([300, 0, 257, 128, 1000], [299, 0, 1, 0, 613], 264, 384, True, True, 0),
    ([1024, 1024], None, 512, 256, True, True, 5),                     # 256-row pair tiles
    ([1024, 1024], [1000, 3], 544, 128, False, False, 0),              # 256-row tiles, odd steps
    ([0, 0, 128], None, 40, 128, True, True, 9),                       # one full step and a tail
    ([30, 700, 0, 385, 384, 1100, 5, 0, 129, 40], None, 264, 128, True, True, 3),   # both size classes
]


@pytest.mark.parametrize("case", SWI_CASES, ids=[str(i) for i in range(len(SWI_CASES))])
def test_gmm_swiglu(gpu_lib, case):
    """The fused up-projection with the SwiGLU epilogue: h and act equal
    moe_gmm into h followed by moe_swiglu on its halves bit for bit, and the
    oracle (product, bias, SwiGLU of the bf16-rounded h) within tolerance;
    rows past the groups are zero."""
    gs, valid, K, F, with_bias, write_h, extra = case
    gs = np.array(gs, dtype=np.int32)
    G = len(gs)
    S = int(gs.sum())
    M = S + extra
    g = np.random.default_rng(K + F + G)
    lhs = _draw(g, (M, K), "bf16")
    wi = _draw(g, (G, K, 2 * F), "bf16")
    bias = _draw(g, (G, 2 * F), "bf16") if with_bias else None
    vr = None
    lhs0 = lhs.copy()
    if valid is not None:
        vr = np.array(valid, dtype=np.int32)
        off = np.concatenate([[0], np.cumsum(gs)])
        for e in range(G):
            lhs0[off[e] + vr[e]:off[e + 1]] = 0
    x_d, w_d = dev(lhs, torch.bfloat16), dev(wi, torch.bfloat16)
    b_d = dev(bias, torch.bfloat16) if with_bias else None
    v_d = dev_i32(vr) if vr is not None else None
    h = poison(torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")) if write_h else None
    act = poison(torch.empty((M, F), dtype=torch.bfloat16, device="cuda"))
    gpu_lib.moe_gmm_swiglu(x_d, w_d, dev_i32(gs), act=act, h=h, bias=b_d, valid_rows=v_d)
    # the two-call path on the same inputs
    h2 = gpu_lib.moe_gmm(x_d, w_d, dev_i32(gs), bias=b_d, valid_rows=v_d)
    a2 = gpu_lib.moe_swiglu(h2[:, :F], h2[:, F:])
    if write_h:
        assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(act.view(torch.int16), a2.view(torch.int16))
    want_h = oracle.gmm(lhs0, wi, gs, bias=bias, rows_out=M)
    hb = ms.bf16_round(want_h)
    want_act = oracle.swiglu(hb[:, :F], hb[:, F:])
    got = host(act)
    assert_close(got[:S], want_act[:S], TOL_BF16, "gmm_swiglu act")
    assert (got[S:] == 0).all()
    if write_h:
        gh = host(h)
        assert_close(gh[:S], want_h[:S], TOL_BF16, "gmm_swiglu h")
        assert (gh[S:] == 0).all()


SWB_CASES = [
    # group sizes, valid rows, K (d_model), F, fused [rows, 2F] layouts, extra output rows
    ([300, 0, 257, 128, 1000], None, 264, 264, False, 7),            # 128-row tiles, ragged F
    ([30, 700, 0, 385, 384, 1100, 5, 0, 129, 40], [30, 650, 0, 385, 300, 1100, 1, 0, 129, 40],
     520, 256, True, 0),                                              # both size classes
    ([1024, 1024], None, 512, 384, True, 5),                          # 256-row pair tiles
    ([1024, 1024], [1000, 3], 544, 256, False, 0),                    # odd steps
]


@pytest.mark.parametrize("case", SWB_CASES, ids=[str(i) for i in range(len(SWB_CASES))])
def test_gmm_swiglu_bwd(gpu_lib, case):
    """The d_act GEMM with the SwiGLU backward epilogue equals moe_gmm into a
    bf16 d_act followed by moe_swiglu_bwd bit for bit, and the oracle within
    tolerance; rows past the groups are zero."""
    gs, valid, K, F, fused, extra = case
    gs = np.array(gs, dtype=np.int32)
    G = len(gs)
    S = int(gs.sum())
    M = S + extra
    g = np.random.default_rng(K + F + 3 * G)
    dy = _draw(g, (M, K), "bf16")
    wo = _draw(g, (G, F, K), "bf16")          # used transposed: [F, K] per group
    h = ms.bf16_round(_draw(g, (M, 2 * F), "bf16") * 3)
    vr = None
    dy0 = dy.copy()
    if valid is not None:
        vr = np.array(valid, dtype=np.int32)
        off = np.concatenate([[0], np.cumsum(gs)])
        for e in range(G):
            dy0[off[e] + vr[e]:off[e + 1]] = 0
    dy_d, wo_d = dev(dy, torch.bfloat16), dev(wo, torch.bfloat16)
    v_d = dev_i32(vr) if vr is not None else None
    if fused:
        hd = dev(h, torch.bfloat16)
        h0, h1 = hd[:, :F], hd[:, F:]
        dh = poison(torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda"))
        d0, d1 = dh[:, :F], dh[:, F:]
    else:
        h0, h1 = dev(h[:, :F], torch.bfloat16), dev(h[:, F:], torch.bfloat16)
        d0 = poison(torch.empty((M, F), dtype=torch.bfloat16, device="cuda"))
        d1 = poison(torch.empty((M, F), dtype=torch.bfloat16, device="cuda"))
    gpu_lib.moe_gmm_swiglu_bwd(dy_d, wo_d, dev_i32(gs), h0, h1, d_h0=d0, d_h1=d1, valid_rows=v_d)
    da = gpu_lib.moe_gmm(dy_d, wo_d, dev_i32(gs), trans_rhs=True, valid_rows=v_d)
    w0, w1 = gpu_lib.moe_swiglu_bwd(h0, h1, da)
    # rows of the groups bit for bit (rows past them are zero in both, the
    # two-call path's possibly as -0 from a zero d_act times a negative h)
    assert torch.equal(d0.contiguous()[:S].view(torch.int16), w0[:S].view(torch.int16))
    assert torch.equal(d1.contiguous()[:S].view(torch.int16), w1[:S].view(torch.int16))
    want_da = ms.bf16_round(oracle.gmm(dy0, wo, gs, trans_rhs=True, rows_out=M))
    o0, o1 = oracle.swiglu_bwd(h[:, :F], h[:, F:], want_da)
    g0, g1 = host(d0.contiguous()), host(d1.contiguous())
    assert_close(g0[:S], o0[:S], TOL_BF16, "d_h0")
    assert_close(g1[:S], o1[:S], TOL_BF16, "d_h1")
    assert (g0[S:] == 0).all() and (g1[S:] == 0).all()


@pytest.mark.parametrize("it", ["bf16", "f32"])
@pytest.mark.parametrize("sizes", [
    ([300, 0, 257, 128, 1000], [299, 0, 1, 0, 613]),
    # valid rows in the 33..64 and 65..128 classes, groups longer than that
    ([200, 150, 100, 90, 64, 256], [33, 65, 100, 64, 40, 128]),
], ids=["classes_short_mid_large", "classes_two_and_four_steps"])
def test_tgmm_valid_rows(gpu_lib, it, sizes):
    """With valid_rows the contraction stops after each group's first
    valid_rows[g] rows: rows past them (garbage here) must not contribute,
    and the result equals the oracle over the rows with the rest zeroed."""
    gs = np.array(sizes[0], dtype=np.int32)
    valid = np.array(sizes[1], dtype=np.int32)
    Kd, N = 264, 136
    g = np.random.default_rng(11)
    M = int(gs.sum())
    lhs = _draw(g, (M, Kd), it)
    rhs = _draw(g, (M, N), it)
    lhs0, rhs0 = lhs.copy(), rhs.copy()
    off = np.concatenate([[0], np.cumsum(gs)])
    for e in range(len(gs)):
        lhs0[off[e] + valid[e]:off[e + 1]] = 0
        rhs0[off[e] + valid[e]:off[e + 1]] = 0
    out = poison(torch.empty((len(gs), Kd, N), dtype=TD[it], device="cuda"))
    gpu_lib.moe_tgmm(dev(lhs, TD[it]), dev(rhs, TD[it]), dev_i32(gs), out=out,
                     valid_rows=dev_i32(valid))
    want = oracle.tgmm(lhs0, rhs0, gs)
    assert_close(host(out), want, TOL_F32 if it == "f32" else TOL_BF16, "tgmm valid_rows")
    for e in np.where(valid == 0)[0]:
        assert (host(out)[e] == 0).all()


@pytest.mark.parametrize("hd,ad", [("bf16", "bf16"), ("f32", "bf16"), ("f32", "f32")])
def test_swiglu_fused_halves(gpu_lib, hd, ad):
    """Gate and up halves of one [rows, 2F] product (row stride 2F), and the
    gradient written into the halves of a [rows, 2F] buffer."""
    g = np.random.default_rng(5)
    rows, F = 37, 136
    h = _draw(g, (rows, 2 * F), hd) * 3
    da = _draw(g, (rows, F), ad)
    hdev = dev(h, TD[hd])
    act = gpu_lib.moe_swiglu(hdev[:, :F], hdev[:, F:], act_dtype=TD[ad])
    tol = TOL_F32 if (hd, ad) == ("f32", "f32") else TOL_BF16
    assert_close(host(act), oracle.swiglu(h[:, :F], h[:, F:]), tol, "swiglu halves")
    dh = poison(torch.empty((rows, 2 * F), dtype=TD[ad], device="cuda"))
    gpu_lib.moe_swiglu_bwd(hdev[:, :F], hdev[:, F:], dev(da, TD[ad]), d_h0=dh[:, :F], d_h1=dh[:, F:])
    w0, w1 = oracle.swiglu_bwd(h[:, :F], h[:, F:], da)
    assert_close(host(dh)[:, :F], w0, tol, "d_h0 half")
    assert_close(host(dh)[:, F:], w1, tol, "d_h1 half")


def test_gmm_strided_chunks(gpu_lib):
    """Contracting-dim chunks of a wider lhs and rhs (views with ld > K),
    accumulated in place into a float32 partial sum = the unchunked product."""
    g = np.random.default_rng(3)
    gs = np.array([100, 0, 37, 200], dtype=np.int32)
    G, D, N, n = 4, 512, 136, 4
    M_lhs = 384                                   # padded to a 128-row tile
    x = ms.bf16_round(g.standard_normal((M_lhs, D)).astype(np.float32))
    w = ms.bf16_round(g.standard_normal((G, D, N)).astype(np.float32))
    xd, wd = dev(x, torch.bfloat16), dev(w, torch.bfloat16)
    out = poison(torch.empty((int(gs.sum()), N), dtype=torch.float32, device="cuda"))
    c = D // n
    for i in range(n):
        gpu_lib.moe_gmm(xd[:, i * c:(i + 1) * c], wd[:, i * c:(i + 1) * c, :], dev_i32(gs), out=out,
                        accumulate=i > 0)
    want = oracle.gmm(x, w, gs, rows_out=int(gs.sum()))
    assert_close(host(out), want, TOL_F32, "chunked gmm")


GROUP_SUM_CASES = [
    # groups, N, in, out, accumulate, valid rows, strided input
    ("ragged", 136, "bf16", "f32", False, False, False),
    ("ragged", 520, "f32", "f32", True, False, False),
    ("empty_first", 264, "bf16", "bf16", False, True, False),
    ("two_big", 1032, "bf16", "f32", False, True, True),    # several 256-row tiles per group
    ("one_group", 8, "bf16", "bf16", True, False, False),
    ("all_empty", 64, "bf16", "f32", False, False, False),
    ("all_empty", 64, "f32", "bf16", True, False, False),
    ("many", 136, "bf16", "f32", False, True, False),
    ("max_groups", 72, "f32", "f32", False, False, True),
]


@pytest.mark.parametrize("case", GROUP_SUM_CASES, ids=[str(c) for c in GROUP_SUM_CASES])
def test_group_sum(gpu_lib, case):
    name, N, it, ot, acc, use_valid, strided = case
    gs = np.array(GS[name], dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(N * 3 + G)
    M = int(gs.sum()) + 9                      # rows past the groups are ignored
    x = _draw(g, (M, N), it)
    valid = None
    if use_valid:
        valid = np.minimum(gs, g.integers(0, 300, G)).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(gs)])
        for e in range(G):
            x[off[e] + valid[e]:off[e + 1]] = 0    # what valid_rows asserts
    if strided:
        wide = dev(np.concatenate([x, _draw(g, (M, 8), it)], axis=1), TD[it])
        xd = wide[:, :N]
    else:
        xd = dev(x, TD[it])
    P = _draw(g, (G, N), ot) if acc else None
    out = dev(P, TD[ot]) if acc else poison(torch.empty((G, N), dtype=TD[ot], device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.moe_group_sum(xd, dev_i32(gs), out=out, accumulate=acc, err=err,
                          valid_rows=None if valid is None else dev_i32(valid))
    want = oracle.group_sum(x, gs) + (P if acc else 0)
    got = host(out)
    assert_close(got, want, TOL_F32 if ot == "f32" else TOL_BF16, "group_sum")
    for e in np.where(gs == 0)[0]:
        assert (got[e] == (P[e] if acc else 0)).all()
    assert host(err)[0] == 0


def test_group_sum_deterministic(gpu_lib):
    gs = np.array(GS["two_big"], dtype=np.int32)
    x = dev(np.random.default_rng(2).standard_normal((int(gs.sum()), 264)).astype(np.float32))
    a = gpu_lib.moe_group_sum(x, dev_i32(gs))
    b = gpu_lib.moe_group_sum(x, dev_i32(gs))
    assert torch.equal(a, b)


TGMM_CASES = [
    ("ragged", 136, 128, "bf16", "f32", False),
    ("ragged", 64, 72, "bf16", "bf16", True),
    ("empty_first", 200, 264, "bf16", "f32", True),
    ("one_group", 128, 8, "bf16", "f32", False),
    ("all_empty", 64, 64, "bf16", "f32", False),
    ("all_empty", 64, 64, "bf16", "f32", True),
    ("ragged", 40, 24, "f32", "f32", False),
    ("aligned", 16, 48, "f32", "f32", True),
    ("max_groups", 16, 136, "bf16", "f32", False),
    ("one_group", 264, 136, "bf16", "bf16", True),   # long contraction: 256-row tiles
    # bf16 out, no partial sum, short contractions (128-row tiles)
    ("ragged", 136, 264, "bf16", "bf16", False),
    ("empty_first", 200, 264, "bf16", "bf16", False),
    ("all_empty", 64, 64, "bf16", "bf16", False),
    ("max_groups", 16, 136, "bf16", "bf16", False),
    ("many", 264, 520, "bf16", "bf16", False),
    ("skewed", 520, 1032, "bf16", "bf16", False),   # full and ragged tiles, several per workgroup
    # short contractions in all three size classes (<= 64 rows, <= 384 rows, larger)
    ("mixed", 136, 264, "bf16", "bf16", False),
    ("mixed", 264, 520, "bf16", "f32", True),
    ("mixed", 200, 72, "bf16", "f32", False),
    # only contractions of at most 64 rows: ragged Kdim and N, partial sums
    ("shortk", 200, 264, "bf16", "bf16", False),
    ("shortk", 136, 520, "bf16", "f32", True),
    ("shortk", 1032, 72, "bf16", "bf16", False),
    ("shortk", 8, 8, "bf16", "bf16", True),
    # contractions of 65 .. 128 rows: ragged Kdim and N, partial sums, f32 out
    ("midk", 200, 264, "bf16", "bf16", False),
    ("midk", 136, 520, "bf16", "f32", True),
    ("midk", 1032, 72, "bf16", "bf16", False),
    ("midk", 8, 8, "bf16", "f32", False),
    ("many_short", 136, 264, "bf16", "bf16", False),
    ("many_short", 72, 136, "bf16", "f32", True),
]


@pytest.mark.parametrize("case", TGMM_CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}-{c[3]}{c[4]}-a{int(c[5])}" for c in TGMM_CASES])
def test_tgmm(gpu_lib, case):
    name, Kd, N, it, ot, acc = case
    gs = np.array(GS[name], dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(Kd * 7 + N)
    M = int(gs.sum()) + 5
    lhs = _draw(g, (M, Kd), it)
    rhs = _draw(g, (M, N), it)
    P = _draw(g, (G, Kd, N), ot) if acc else None
    out = dev(P, TD[ot]) if acc else poison(torch.empty((G, Kd, N), dtype=TD[ot], device="cuda"))
    gpu_lib.moe_tgmm(dev(lhs, TD[it]), dev(rhs, TD[it]), dev_i32(gs), out=out, accumulate=acc)
    want = oracle.tgmm(lhs, rhs, gs, partial=P)
    got = host(out)
    assert_close(got, want, TOL_F32 if ot == "f32" else TOL_BF16, "tgmm")
    for gg in range(G):
        if gs[gg] == 0:
            assert (got[gg] == (P[gg] if acc else 0)).all(), "empty group"


# ------------------------------------------------------------------ SwiGLU

@pytest.mark.parametrize("hd,ad", [("bf16", "bf16"), ("f32", "bf16"), ("f32", "f32")])
def test_swiglu(gpu_lib, hd, ad):
    g = np.random.default_rng(11)
    rows, F = 333, 136
    h0 = _draw(g, (rows, F), hd) * 3
    h0 = ms.bf16_round(h0) if hd == "bf16" else h0
    h1 = _draw(g, (rows, F), hd)
    da = _draw(g, (rows, F), ad)
    act = gpu_lib.moe_swiglu(dev(h0, TD[hd]), dev(h1, TD[hd]), act_dtype=TD[ad])
    tol = TOL_F32 if ad == "f32" else TOL_BF16
    assert_close(host(act), oracle.swiglu(h0, h1), tol, "swiglu")
    d0, d1 = gpu_lib.moe_swiglu_bwd(dev(h0, TD[hd]), dev(h1, TD[hd]), dev(da, TD[ad]))
    w0, w1 = oracle.swiglu_bwd(h0, h1, da)
    assert_close(host(d0), w0, tol, "d_h0")
    assert_close(host(d1), w1, tol, "d_h1")
