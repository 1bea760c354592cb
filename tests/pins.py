"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``check_*`` raises AssertionError on a mismatch.  They are collected
as tests in ``test_oracle_pins.py`` and re-run against deliberately broken
copies of the oracle in ``test_oracle_mutations.py`` to show that a
plausible mistake (dropped term, wrong sign or index, transposed operand,
wrong tie-break, unstable order) fails at least one of them.

None of these re-types the oracle's formula or re-calls the routine it
uses for the same step: they use brute force in plain Python loops,
closed forms, invariants, a library routine of a different algorithm, or
central finite differences.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# route
# ---------------------------------------------------------------------------

def _select_by_scan(z_row, K):
    """Repeatedly pick the largest remaining value scanning ids upward with a
    strict '>' (so the lower id wins a tie)."""
    chosen = []
    for _ in range(K):
        best = None
        for e in range(len(z_row)):
            if e in chosen:
                continue
            if best is None or z_row[e] > z_row[best]:
                best = e
        chosen.append(best)
    return chosen


def check_route_selection(seed=0):
    g = _rng(seed)
    for (T, E, K) in [(40, 8, 2), (30, 16, 8), (25, 5, 5), (20, 33, 1)]:
        # coarse values force many exact ties
        z = (g.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
        bias = np.zeros(E, dtype=np.float32)
        bias[g.integers(0, E)] = -np.inf
        if K == E:
            bias[:] = 0
        for b in (None, bias):
            ids, _ = oracle.route(z, K, "softmax", True, b)
            zz = z + (b if b is not None else 0)
            for t in range(T):
                assert list(ids[t]) == _select_by_scan(list(zz[t]), K), (t, zz[t], ids[t])


def check_route_weights(seed=1):
    g = _rng(seed)
    T, E, K = 30, 12, 4
    z = g.standard_normal((T, E)).astype(np.float32) * 2
    # softmax + renorm equals the softmax over just the K selected logits
    ids, w = oracle.route(z, K, "softmax", True)
    sel = np.take_along_axis(z.astype(np.float64), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    # softmax without renorm, K = E: the full softmax, in descending order
    ids, w = oracle.route(z, E, "softmax", False)
    full = scipy.special.softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), axis=1), rtol=1e-13)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
    # sigmoid without renorm: the logistic function of the selected logits
    ids, w = oracle.route(z, K, "sigmoid", False)
    sel = np.take_along_axis(z.astype(np.float64), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, scipy.special.expit(sel), rtol=1e-13)
    # sigmoid + renorm: sums to one, ratios are ratios of logistic values
    ids, w = oracle.route(z, K, "sigmoid", True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
    ex = scipy.special.expit(sel)
    np.testing.assert_allclose(w[:, 1:] / w[:, :1], ex[:, 1:] / ex[:, :1], rtol=1e-12)
    # weights come out in descending order of score
    assert np.all(np.diff(w, axis=1) <= 0)


def check_route_closed_forms():
    # logits 1,2,3,4; top-2 softmax renorm -> experts 3, 2 with weights
    # e^4/(e^4+e^3) = 1/(1+e^-1) and 1/(1+e)
    z = np.array([[1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    ids, w = oracle.route(z, 2, "softmax", True)
    assert list(ids[0]) == [3, 2]
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-1)), 1 / (1 + math.exp(1))], rtol=1e-15)
    # a tie between experts 1 and 3 (value ln 3): lower id first, equal weights
    z = np.array([[0.0, math.log(3), math.log(2), math.log(3)]], dtype=np.float32)
    ids, w = oracle.route(z, 2, "softmax", True)
    assert list(ids[0]) == [1, 3]
    np.testing.assert_allclose(w[0], [0.5, 0.5], rtol=1e-15)
    # sigmoid + renorm over logits 0 and 10 (expert 3 is switched off by -inf)
    z = np.array([[0.0, -1.0, 10.0, 5.0]], dtype=np.float32)
    bias = np.array([0, 0, 0, -np.inf], dtype=np.float32)
    ids, w = oracle.route(z, 2, "sigmoid", True, bias)
    assert list(ids[0]) == [2, 0]
    s10, s0 = 1 / (1 + math.exp(-10)), 0.5
    np.testing.assert_allclose(w[0], [s10 / (s10 + s0), s0 / (s10 + s0)], rtol=1e-15)
    # equal logits: top-K renormalised weights are all 1/K
    z = np.zeros((3, 6), dtype=np.float32)
    ids, w = oracle.route(z, 3, "softmax", True)
    assert (ids == np.array([0, 1, 2])).all()
    np.testing.assert_allclose(w, 1 / 3, rtol=1e-15)


def _py_scores(z_row, score):
    """Scores of one token's logits with the math module (no NumPy)."""
    if score == "softmax":
        m = max(z_row)
        ex = [math.exp(v - m) for v in z_row]
        tot = sum(ex)
        return [v / tot for v in ex]
    return [1.0 / (1.0 + math.exp(-v)) for v in z_row]


def check_route_weights_of_given_ids(seed=11):
    """Weights of an arbitrary (not top-K) selection, per token with the math
    module: every score mode, with and without renorm, a logit bias that
    enters the scores and a selection-only bias that does not."""
    g = _rng(seed)
    T, E, K = 20, 9, 3
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (g.standard_normal(E) * 0.4).astype(np.float32)
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    for score in ("softmax", "sigmoid"):
        for renorm in (True, False):
            for mode, b in (("logit", None), ("logit", bias), ("select", bias)):
                w = oracle.route_weights(z, ids, score, renorm, b, mode)
                for t in range(T):
                    zz = [float(np.float32(z[t, e]) + (np.float32(b[e]) if b is not None and
                                                      mode == "logit" else 0))
                          for e in range(E)]
                    p = _py_scores(zz, score)
                    ws = [p[e] for e in ids[t]]
                    if renorm:
                        tot = sum(ws)
                        ws = [v / tot for v in ws]
                    np.testing.assert_allclose(w[t], ws, rtol=1e-12)


def check_route_select_bias(seed=4):
    """Selection-only bias: the key is score + bias, the weights the plain
    scores of the selected experts.  Brute force per token, and with a zero
    bias the plain routing."""
    g = _rng(seed)
    T, E, K = 24, 10, 3
    z = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (g.standard_normal(E) * 0.3).astype(np.float32)
    for score in ("softmax", "sigmoid"):
        for renorm in (True, False):
            ids, w = oracle.route(z, K, score, renorm, bias, "select")
            for t in range(T):
                p = _py_scores([float(v) for v in z[t]], score)
                key = [p[e] + float(bias[e]) for e in range(E)]
                sel = _select_by_scan(key, K)
                assert list(ids[t]) == sel, (score, t)
                ws = [p[e] for e in sel]
                if renorm:
                    tot = sum(ws)
                    ws = [v / tot for v in ws]
                np.testing.assert_allclose(w[t], ws, rtol=1e-12)
            i0, w0 = oracle.route(z, K, score, renorm, np.zeros(E, np.float32), "select")
            i1, w1 = oracle.route(z, K, score, renorm)
            assert (i0 == i1).all()
            np.testing.assert_allclose(w0, w1, rtol=1e-14)


def _group_select_by_scan(key, K, n_groups, topk_groups):
    E = len(key)
    eg = E // n_groups
    gscore = []
    for gi in range(n_groups):
        vals = sorted(key[gi * eg:(gi + 1) * eg], reverse=True)
        gscore.append(sum(vals[:2]))
    chosen = _select_by_scan(gscore, topk_groups)
    masked = [key[e] if (e // eg) in chosen else -math.inf for e in range(E)]
    return _select_by_scan(masked, K), chosen


def check_route_groups(seed=5):
    """Grouped selection against a loop version, the group invariant, and the
    two settings that reduce to plain top-K."""
    g = _rng(seed)
    T, E, K = 30, 16, 4
    z = (g.integers(-4, 5, size=(T, E)) * 0.25).astype(np.float32)   # many ties
    bias = (g.integers(-2, 3, size=E) * 0.125).astype(np.float32)
    for mode in ("logit", "select"):
        for n_groups, topk_groups in ((4, 2), (8, 3), (16, 4), (2, 1)):
            ids, _ = oracle.route(z, K, "sigmoid", True, bias, mode, n_groups, topk_groups)
            for t in range(T):
                if mode == "logit":
                    key = [float(np.float32(z[t, e]) + np.float32(bias[e])) for e in range(E)]
                else:
                    p = _py_scores([float(v) for v in z[t]], "sigmoid")
                    key = [p[e] + float(bias[e]) for e in range(E)]
                sel, chosen = _group_select_by_scan(key, K, n_groups, topk_groups)
                assert list(ids[t]) == sel, (mode, n_groups, t)
                assert all((e // (E // n_groups)) in chosen for e in ids[t])
        plain, _ = oracle.route(z, K, "sigmoid", True, bias, mode)
        for n_groups, topk_groups in ((1, 1), (4, 4)):
            ids, _ = oracle.route(z, K, "sigmoid", True, bias, mode, n_groups, topk_groups)
            assert (ids == plain).all()


def check_aux_loss_closed_forms():
    alpha = 0.01
    g = _rng(6)
    T, E, K = 32, 8, 2
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    for score in ("softmax", "sigmoid"):
        # equal logits: every probability is 1/E, so the loss is alpha whatever the routing
        loss, _, P = oracle.aux_loss(np.zeros((T, E), np.float32), ids, E, alpha, score)
        assert abs(loss - alpha) < 1e-15 and np.allclose(P, 1.0 / E, rtol=1e-15)
        # perfectly balanced routing: every f_e = 1/E, so the loss is alpha whatever the logits
        bal = np.array([[(t * K + j) % E for j in range(K)] for t in range(T)], dtype=np.int32)
        z = g.standard_normal((T, E)).astype(np.float32)
        loss, counts, _ = oracle.aux_loss(z, bal, E, alpha, score)
        assert (counts == T * K // E).all() and abs(loss - alpha) < 1e-15
    # one token, two experts, logits 0 and ln 3 (softmax 1/4, 3/4), expert 1 chosen:
    # loss = alpha * 2 * (0 * 1/4 + 1 * 3/4)
    loss, _, _ = oracle.aux_loss(np.array([[0.0, math.log(3)]]), np.array([[1]], np.int32), 2,
                                 alpha, "softmax")
    assert abs(loss - 1.5 * alpha) < 1e-15


def check_aux_loss_bwd_fd(seed=7):
    g = _rng(seed)
    T, E, K = 6, 7, 2
    alpha, eps = 0.3, 1e-6
    z = g.standard_normal((T, E)) * 1.2
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    for score in ("softmax", "sigmoid"):
        _, counts, _ = oracle.aux_loss(z, ids, E, alpha, score)
        d = oracle.aux_loss_bwd(z, counts, K, alpha, score)
        fd = np.zeros_like(z)
        for t in range(T):
            for e in range(E):
                zp, zm = z.copy(), z.copy()
                zp[t, e] += eps
                zm[t, e] -= eps
                fd[t, e] = (oracle.aux_loss(zp, ids, E, alpha, score)[0]
                            - oracle.aux_loss(zm, ids, E, alpha, score)[0]) / (2 * eps)
        np.testing.assert_allclose(d, fd, rtol=1e-5, atol=1e-9)


def _margin(z32, K):
    """Smallest gap between the K-th and (K+1)-th largest value per row."""
    s = -np.sort(-z32.astype(np.float64), axis=1)
    if K >= z32.shape[1]:
        return np.inf
    gap = s[:, K - 1] - s[:, K]
    return np.nanmin(np.where(np.isfinite(gap), gap, np.inf))


def check_route_bwd_fd(seed=2):
    g = _rng(seed)
    T, E, K = 12, 9, 3
    eps = 1e-6
    for score in ("softmax", "sigmoid"):
        for renorm in (True, False):
            z = g.standard_normal((T, E)) * 1.5
            assert _margin(z.astype(np.float32), K) > 1e-3
            u = g.standard_normal((T, K))
            ids, _ = oracle.route(z, K, score, renorm)
            dz = oracle.route_bwd(z, ids, u, score, renorm)
            # float64 logits: pass through the float64 weight path only
            def L(zz):
                i2, w2 = _route_f64(zz, K, score, renorm)
                assert (i2 == ids).all()
                return float((w2 * u).sum())
            for _ in range(6):
                d = g.standard_normal((T, E))
                fd = (L(z + eps * d) - L(z - eps * d)) / (2 * eps)
                assert abs(fd - float((dz * d).sum())) < 1e-7 * max(1.0, abs(fd)), (score, renorm, fd)


def _route_f64(z, K, score, renorm):
    """Selection and weights on float64 logits, computed from scratch with
    SciPy (used only to probe route_bwd by finite differences)."""
    order = np.argsort(-z, axis=1, kind="stable")[:, :K]
    if score == "softmax":
        p = scipy.special.softmax(z, axis=1)
    else:
        p = scipy.special.expit(z)
    w = np.take_along_axis(p, order, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


# ---------------------------------------------------------------------------
# permute / permute_bwd / combine / combine_bwd
# ---------------------------------------------------------------------------

def _ids(g, T, E, K, skew=False):
    """Random distinct expert ids per token."""
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
    else:
        p = None
    out = np.zeros((T, K), dtype=np.int32)
    for t in range(T):
        out[t] = g.choice(E, size=K, replace=False, p=p)
    return out


def check_permute_argsort(seed=3):
    g = _rng(seed)
    T, E, K = 50, 7, 3
    ids = _ids(g, T, E, K, skew=True)
    P = oracle.permute(None, ids, E)
    order = np.argsort(ids.reshape(-1), kind="stable")  # rows -> slots
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert (P["row_of_slot"] == inv).all()
    assert (P["slot_of_row"] == order).all()
    assert P["counts"].sum() == T * K
    assert (P["counts"] == np.bincount(ids.reshape(-1), minlength=E)).all()


def check_permute_align(seed=4):
    g = _rng(seed)
    T, E, K, a = 40, 10, 2, 8
    ids = _ids(g, T, E, K, skew=True)
    P = oracle.permute(None, ids, E, align=a)
    cnt = np.bincount(ids.reshape(-1), minlength=E)
    assert (P["counts"] == cnt).all()
    assert (P["group_sizes"] % a == 0).all()
    assert ((P["group_sizes"] >= cnt) & (P["group_sizes"] < cnt + a)).all()
    assert ((P["group_sizes"] == 0) == (cnt == 0)).all()
    assert (P["group_offsets"] % a == 0).all()
    assert P["slot_of_row"].size == T * K + E * (a - 1)   # receive-buffer bound with align_size
    # per group: the slots of expert e in ascending order, then padding
    for e in range(E):
        o = P["group_offsets"][e]
        want = [s for s in range(T * K) if ids.reshape(-1)[s] == e]
        got = list(P["slot_of_row"][o:o + P["group_sizes"][e]])
        assert got == want + [-1] * (P["group_sizes"][e] - len(want))
    assert P["group_offsets"][-1] == P["group_sizes"].sum()
    assert (P["slot_of_row"][P["group_offsets"][-1]:] == -1).all()


def check_permute_capacity(seed=5):
    g = _rng(seed)
    T, E, K, C = 60, 6, 2, 9
    ids = _ids(g, T, E, K, skew=True)
    flat = ids.reshape(-1)
    for layout in (False, True):
        P = oracle.permute(None, ids, E, capacity=C, capacity_layout=layout)
        for e in range(E):
            slots = [s for s in range(T * K) if flat[s] == e]
            keep, drop = slots[:C], slots[C:]
            assert P["counts"][e] == len(keep)
            assert all(P["row_of_slot"][s] == -1 for s in drop)
            base = e * C if layout else P["group_offsets"][e]
            assert [P["row_of_slot"][s] for s in keep] == list(range(base, base + len(keep)))
        if layout:
            assert (P["group_sizes"] == C).all() and P["slot_of_row"].size == E * C


def check_permute_rows(seed=6):
    g = _rng(seed)
    T, E, K, D = 37, 5, 2, 6
    ids = _ids(g, T, E, K)
    x = g.standard_normal((T, D))
    for a in (0, 4):
        P = oracle.permute(x, ids, E, align=a)
        xs, ros, sor = P["x_sorted"], P["row_of_slot"], P["slot_of_row"]
        for s in range(T * K):
            assert (xs[ros[s]] == x[s // K]).all()
        assert (xs[sor < 0] == 0).all()
        real = sor[sor >= 0]
        assert sorted(real.tolist()) == list(range(T * K))   # every slot lands exactly once


def check_permute_unpermute_identity(seed=7):
    g = _rng(seed)
    T, E, D = 45, 6, 5
    x = g.standard_normal((T, D))
    # K = 1, weight 1: combine(permute(x)) = x
    ids = _ids(g, T, E, 1)
    P = oracle.permute(x, ids, E, align=4)
    y = oracle.combine(P["x_sorted"], P["row_of_slot"], np.ones((T, 1)), T, 1)
    np.testing.assert_array_equal(y, x)
    # K = 3 with renormalised weights: x * sum(w) = x
    ids = _ids(g, T, E, 3)
    z = g.standard_normal((T, E))
    ids, w = oracle.route(z, 3, "softmax", True)
    P = oracle.permute(x, ids, E)
    y = oracle.combine(P["x_sorted"], P["row_of_slot"], w, T, 3)
    np.testing.assert_allclose(y, x, rtol=1e-14, atol=1e-14)
    # permute_bwd of the sorted copy counts each token K times
    dx = oracle.permute_bwd(P["x_sorted"], P["row_of_slot"], T, 3)
    np.testing.assert_allclose(dx, 3 * x, rtol=1e-14)


def check_adjoints(seed=8):
    g = _rng(seed)
    T, E, K, D = 33, 7, 3, 4
    ids = _ids(g, T, E, K, skew=True)
    for (a, C) in [(0, 0), (4, 0), (0, 11)]:
        P0 = oracle.permute(None, ids, E, align=a, capacity=C)
        rows = P0["slot_of_row"].size
        x = g.standard_normal((T, D))
        u = g.standard_normal((rows, D))
        P = oracle.permute(x, ids, E, align=a, capacity=C)
        lhs = float((P["x_sorted"] * u).sum())
        rhs = float((x * oracle.permute_bwd(u, P["row_of_slot"], T, K)).sum())
        assert abs(lhs - rhs) < 1e-12 * max(1, abs(lhs))
        # combine is linear in y_sorted; its adjoint is combine_bwd's first output
        w = g.standard_normal((T, K))
        ys = g.standard_normal((rows, D))
        v = g.standard_normal((T, D))
        d_ys, d_w = oracle.combine_bwd(v, ys, P["row_of_slot"], w, rows)
        lhs = float((oracle.combine(ys, P["row_of_slot"], w, T, K) * v).sum())
        assert abs(lhs - float((ys * d_ys).sum())) < 1e-12 * max(1, abs(lhs))
        # combine is linear in w: exact difference quotient per weight
        base = float((oracle.combine(ys, P["row_of_slot"], w, T, K) * v).sum())
        for (t, j) in [(0, 0), (5, 2), (T - 1, 1), (17, 0)]:
            w2 = w.copy()
            w2[t, j] += 1.0
            diff = float((oracle.combine(ys, P["row_of_slot"], w2, T, K) * v).sum()) - base
            assert abs(diff - d_w[t, j]) < 1e-12 * max(1, abs(diff))
        # rows no slot maps to get zero gradient
        assert (d_ys[P["slot_of_row"] < 0] == 0).all()


# ---------------------------------------------------------------------------
# gmm / tgmm
# ---------------------------------------------------------------------------

def _brute_gmm(lhs, rhs, gs, trans, partial, rows_out, bias=None):
    N = len(rhs[0]) if trans else len(rhs[0][0])
    Kd = len(lhs[0])
    out = [[0.0] * N for _ in range(rows_out)] if partial is None else partial.tolist()
    r = 0
    for g, n in enumerate(gs):
        for _ in range(n):
            for c in range(N):
                acc = 0.0
                for k in range(Kd):
                    acc += lhs[r][k] * (rhs[g][c][k] if trans else rhs[g][k][c])
                out[r][c] += acc + (0.0 if bias is None else bias[g][c])
            r += 1
    return np.array(out)


def check_gmm_bruteforce(seed=9):
    g = _rng(seed)
    Kd, N = 5, 4
    for gs in ([3, 0, 4, 1], [0, 0, 6], [2, 5, 0], [7]):
        G = len(gs)
        M_lhs = sum(gs) + 3            # rows beyond sum(gs) (padding)
        lhs = g.standard_normal((M_lhs, Kd))
        for trans in (False, True):
            rhs = g.standard_normal((G, N, Kd) if trans else (G, Kd, N))
            got = oracle.gmm(lhs, rhs, gs, trans_rhs=trans)
            want = _brute_gmm(lhs.tolist(), rhs.tolist(), gs, trans, None, M_lhs)
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
            # partial sum with fewer output rows than lhs rows
            P = g.standard_normal((sum(gs) + 1, N))
            got = oracle.gmm(lhs, rhs, gs, trans_rhs=trans, partial=P)
            want = _brute_gmm(lhs.tolist(), rhs.tolist(), gs, trans, P, sum(gs) + 1)
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
            assert (got[sum(gs):] == P[sum(gs):]).all()
            # a per-group bias on every row of its group, with and without a partial sum
            B = g.standard_normal((G, N))
            got = oracle.gmm(lhs, rhs, gs, trans_rhs=trans, bias=B)
            want = _brute_gmm(lhs.tolist(), rhs.tolist(), gs, trans, None, M_lhs, B.tolist())
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
            assert (got[sum(gs):] == 0).all()
            got = oracle.gmm(lhs, rhs, gs, trans_rhs=trans, partial=P, bias=B)
            want = _brute_gmm(lhs.tolist(), rhs.tolist(), gs, trans, P, sum(gs) + 1, B.tolist())
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def check_group_sum(seed=17):
    """Per-group row sums by scalar loops, zero for empty groups, and the
    adjoint of the bias: <gmm(X, W, bias=B) - gmm(X, W), Y> = <B, group_sum(Y)>."""
    g = _rng(seed)
    for gs in ([3, 0, 4, 1], [0, 0, 5], [6, 0]):
        G, M, N = len(gs), sum(gs) + 2, 4
        Y = g.standard_normal((M, N))
        got = oracle.group_sum(Y, gs)
        r0 = 0
        for gg, n in enumerate(gs):
            for c in range(N):
                acc = 0.0
                for r in range(r0, r0 + n):
                    acc += Y[r, c]
                assert abs(got[gg, c] - acc) < 1e-13
                if n == 0:
                    assert got[gg, c] == 0.0
            r0 += n
        X = g.standard_normal((M, 3))
        W = g.standard_normal((G, 3, N))
        B = g.standard_normal((G, N))
        lhs = float(((oracle.gmm(X, W, gs, bias=B) - oracle.gmm(X, W, gs)) * Y).sum())
        rhs = float((B * got).sum())
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def check_tgmm_bruteforce(seed=10):
    g = _rng(seed)
    Kd, N = 4, 3
    for gs in ([3, 0, 4, 1], [0, 5], [4, 0]):
        G, M = len(gs), sum(gs) + 2
        lhs = g.standard_normal((M, Kd))
        rhs = g.standard_normal((M, N))
        got = oracle.tgmm(lhs, rhs, gs)
        want = np.zeros((G, Kd, N))
        r0 = 0
        for gg, n in enumerate(gs):
            for a in range(Kd):
                for b in range(N):
                    want[gg, a, b] = sum(lhs[r, a] * rhs[r, b] for r in range(r0, r0 + n))
            r0 += n
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
        P = g.standard_normal((G, Kd, N))
        got = oracle.tgmm(lhs, rhs, gs, partial=P)
        np.testing.assert_allclose(got, want + P, rtol=1e-13, atol=1e-13)
        for gg, n in enumerate(gs):
            if n == 0:
                assert (got[gg] == P[gg]).all()
                assert (oracle.tgmm(lhs, rhs, gs)[gg] == 0).all()


def check_gmm_adjoints(seed=11):
    """<gmm(X, W), Y> = <X, gmm(Y, W, trans)> = sum_g <W_g, tgmm(X, Y)_g>."""
    g = _rng(seed)
    gs = [5, 0, 3, 7, 1]
    G, M, Kd, N = len(gs), sum(gs), 6, 4
    X = g.standard_normal((M, Kd))
    W = g.standard_normal((G, Kd, N))
    Y = g.standard_normal((M, N))
    a = float((oracle.gmm(X, W, gs) * Y).sum())
    b = float((X * oracle.gmm(Y, W, gs, trans_rhs=True)).sum())
    c = float((W * oracle.tgmm(X, Y, gs)).sum())
    assert abs(a - b) < 1e-12 * max(1, abs(a)) and abs(a - c) < 1e-12 * max(1, abs(a))


def check_gmm_chunked(seed=12):
    g = _rng(seed)
    gs = [4, 0, 6, 2]
    G, M, Kd, N = len(gs), sum(gs), 12, 5
    X = g.standard_normal((M + 4, Kd))     # lhs padded beyond sum(gs)
    W = g.standard_normal((G, Kd, N))
    full = oracle.gmm(X, W, gs, rows_out=M)
    acc = None
    for c in range(3):
        sl = slice(4 * c, 4 * c + 4)
        acc = oracle.gmm(X[:, sl], W[:, sl, :], gs, partial=acc, rows_out=M)
    np.testing.assert_allclose(acc, full, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# swiglu
# ---------------------------------------------------------------------------

def check_swiglu(seed=13):
    # silu(1) = 1/(1+e^-1), silu(-1) = -1/(1+e), silu(0) = 0, silu(2) = 2/(1+e^-2)
    h0 = np.array([1.0, -1.0, 0.0, 2.0])
    h1 = np.array([1.0, 1.0, 5.0, -0.5])
    want = np.array([1 / (1 + math.exp(-1)), -1 / (1 + math.e), 0.0, -0.5 * 2 / (1 + math.exp(-2))])
    np.testing.assert_allclose(oracle.swiglu(h0, h1), want, rtol=1e-15, atol=1e-300)
    # at h0 = 0 the gate derivative is 1/2
    d0, d1 = oracle.swiglu_bwd(np.zeros(3), np.array([2.0, -4.0, 1.0]), np.array([1.0, 1.0, 3.0]))
    np.testing.assert_allclose(d0, [1.0, -2.0, 1.5], rtol=1e-15)
    np.testing.assert_allclose(d1, 0.0, atol=0)
    g = _rng(seed)
    h0 = g.standard_normal(50) * 3
    h1 = g.standard_normal(50)
    da = g.standard_normal(50)
    d0, d1 = oracle.swiglu_bwd(h0, h1, da)
    eps = 1e-6
    fd0 = (oracle.swiglu(h0 + eps, h1) - oracle.swiglu(h0 - eps, h1)) / (2 * eps) * da
    fd1 = (oracle.swiglu(h0, h1 + eps) - oracle.swiglu(h0, h1 - eps)) / (2 * eps) * da
    np.testing.assert_allclose(d0, fd0, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(d1, fd1, rtol=1e-7, atol=1e-8)


# ---------------------------------------------------------------------------
# the whole block
# ---------------------------------------------------------------------------

def _tiny_block(g, T=24, D=6, F=5, E=5):
    x = g.standard_normal((T, D))
    Wg = g.standard_normal((D, E)) * 0.7
    wi0 = g.standard_normal((E, D, F)) * 0.5
    wi1 = g.standard_normal((E, D, F)) * 0.5
    wo = g.standard_normal((E, F, D)) * 0.5
    return x, Wg, wi0, wi1, wo


def _dense_token_ffn(x, ids, w, wi0, wi1, wo, kept=None, biases=None):
    """Per-token sum of its experts' SwiGLU FFNs, no grouping at all
    (biases: optional per-expert b0 [E, F], b1 [E, F], bo [E, D])."""
    T, D = x.shape
    y = np.zeros((T, D))
    for t in range(T):
        for j in range(ids.shape[1]):
            if kept is not None and not kept[t, j]:
                continue
            e = ids[t, j]
            F = wi0.shape[2]
            b0, b1, bo = biases if biases is not None else (None, None, None)
            h0 = [sum(x[t, d] * wi0[e, d, f] for d in range(D)) + (b0[e, f] if b0 is not None else 0)
                  for f in range(F)]
            h1 = [sum(x[t, d] * wi1[e, d, f] for d in range(D)) + (b1[e, f] if b1 is not None else 0)
                  for f in range(F)]
            a = [h0[f] / (1 + math.exp(-h0[f])) * h1[f] for f in range(F)]
            for d in range(D):
                yo = sum(a[f] * wo[e, f, d] for f in range(F)) + (bo[e, d] if bo is not None else 0)
                y[t, d] += w[t, j] * yo
    return y


def check_block_dense(seed=14):
    g = _rng(seed)
    x, Wg, wi0, wi1, wo = _tiny_block(g)
    E = wi0.shape[0]
    for (K, score, renorm, a, C) in [(2, "softmax", True, 0, 0), (3, "sigmoid", True, 4, 0),
                                     (1, "softmax", False, 0, 3), (2, "sigmoid", False, 2, 7)]:
        f = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, score=score, renorm=renorm, align=a,
                               capacity=C)
        kept = (f["perm"]["row_of_slot"] >= 0).reshape(-1, K)
        if C == 0:
            assert kept.all()
        else:
            assert not kept.all()   # the case must actually drop something
        want = _dense_token_ffn(x, f["ids"], f["w"], wi0, wi1, wo, kept)
        np.testing.assert_allclose(f["y"], want, rtol=1e-12, atol=1e-13)
        # capacity layout computes the same output as the compact layout
        if C:
            f2 = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, score=score, renorm=renorm,
                                    capacity=C, capacity_layout=True)
            np.testing.assert_allclose(f2["y"], f["y"], rtol=1e-13, atol=1e-14)
    # per-expert MLP biases, with align padding and with dropping
    F = wi0.shape[2]
    b0 = g.standard_normal((E, F))
    b1 = g.standard_normal((E, F))
    bo = g.standard_normal((E, x.shape[1]))
    for (K, a, C) in [(2, 4, 0), (1, 0, 3)]:
        f = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, align=a, capacity=C,
                               b_wi_0=b0, b_wi_1=b1, b_wo=bo)
        kept = (f["perm"]["row_of_slot"] >= 0).reshape(-1, K)
        want = _dense_token_ffn(x, f["ids"], f["w"], wi0, wi1, wo, kept, (b0, b1, bo))
        np.testing.assert_allclose(f["y"], want, rtol=1e-12, atol=1e-13)


def check_block_chunked(seed=15):
    g = _rng(seed)
    x, Wg, wi0, wi1, wo = _tiny_block(g, D=8)
    f1 = oracle.moe_forward(x, wi0, wi1, wo, 2, Wg=Wg)
    f4 = oracle.moe_forward(x, wi0, wi1, wo, 2, Wg=Wg, n_chunks=4, lhs_rows=64)
    for k in ("h0", "h1", "y"):
        np.testing.assert_allclose(f4[k], f1[k], rtol=1e-13, atol=1e-14)
    # MLP biases enter once, whatever the number of chunks
    E, F = wi0.shape[0], wi0.shape[2]
    bk = dict(b_wi_0=g.standard_normal((E, F)), b_wi_1=g.standard_normal((E, F)),
              b_wo=g.standard_normal((E, x.shape[1])))
    f1 = oracle.moe_forward(x, wi0, wi1, wo, 2, Wg=Wg, **bk)
    f4 = oracle.moe_forward(x, wi0, wi1, wo, 2, Wg=Wg, n_chunks=4, lhs_rows=64, **bk)
    for k in ("h0", "h1", "y"):
        np.testing.assert_allclose(f4[k], f1[k], rtol=1e-13, atol=1e-14)


def check_block_grad_fd(seed=16):
    """Directional central differences of L = <y, dy> for every input."""
    g = _rng(seed)
    x, Wg, wi0, wi1, wo = _tiny_block(g)
    dy = g.standard_normal(x.shape)
    eps = 1e-6
    for (K, score, renorm, a, C, bias) in [
            (2, "softmax", True, 0, 0, None), (3, "sigmoid", True, 4, 0, np.array([0, -1, -np.inf, 0.5, 0])),
            (1, "softmax", False, 0, 4, None), (2, "sigmoid", False, 0, 0, None)]:
        b32 = None if bias is None else bias.astype(np.float32)
        kw = dict(score=score, renorm=renorm, align=a, capacity=C, bias=b32)
        E, F = wi0.shape[0], wi0.shape[2]
        # per-expert MLP biases in the cases with align padding or dropping
        mlp = a > 0 or C > 0
        b0, b1, bo = (g.standard_normal((E, F)), g.standard_normal((E, F)),
                      g.standard_normal((E, x.shape[1])))
        bk = dict(b_wi_0=b0, b_wi_1=b1, b_wo=bo) if mlp else {}
        f = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, **kw, **bk)
        z = oracle.biased_logits_f32(f["logits"], b32)
        assert _margin(z, K) > 1e-4, "selection too close to a tie for finite differences"
        grads = oracle.moe_backward(f, dy, x, wi0, wi1, wo, K, Wg=Wg, score=score, renorm=renorm,
                                    bias=b32)
        ids0 = f["ids"]

        def L(xx, Wgg, a0, a1, oo, c0, c1, co):
            # the selection must not move; weights are recomputed in float64
            lg = xx @ Wgg
            if b32 is not None:
                lg = lg + b32.astype(np.float64)
            ids, w = _route_f64(lg, K, score, renorm)
            assert (ids == ids0).all()
            P = oracle.permute(xx, ids, wi0.shape[0], align=a, capacity=C)
            h0 = oracle.gmm(P["x_sorted"], a0, P["group_sizes"], bias=c0)
            h1 = oracle.gmm(P["x_sorted"], a1, P["group_sizes"], bias=c1)
            ys = oracle.gmm(oracle.swiglu(h0, h1), oo, P["group_sizes"], bias=co)
            return float((oracle.combine(ys, P["row_of_slot"], w, xx.shape[0], K) * dy).sum())

        params = [x, Wg, wi0, wi1, wo]
        names = ["dx", "d_Wg", "d_wi_0", "d_wi_1", "d_wo"]
        if mlp:
            params += [b0, b1, bo]
            names += ["d_b_wi_0", "d_b_wi_1", "d_b_wo"]
        else:
            params += [None, None, None]
        for i, name in enumerate(names):
            d = g.standard_normal(params[i].shape)
            pp = [None if p is None else p.copy() for p in params]
            pm = [None if p is None else p.copy() for p in params]
            pp[i] = params[i] + eps * d
            pm[i] = params[i] - eps * d
            fd = (L(*pp) - L(*pm)) / (2 * eps)
            an = float((grads[name] * d).sum())
            assert abs(fd - an) < 1e-6 * max(1.0, abs(fd)), (name, score, renorm, fd, an)


# ---------------------------------------------------------------------------
# FP8 (current scaling, e4m3 forward / e5m2 backward)
# ---------------------------------------------------------------------------

def check_fp8_codes_vs_torch(seed=18):
    """Decoding every code, and encoding in-range values (random, exact ties,
    subnormals), agree with torch's float8 conversions, an independent
    implementation of the same OCP formats."""
    import torch
    F8 = oracle.fp8
    g = _rng(seed)
    for fmt, dt in ((F8.E4M3, torch.float8_e4m3fn), (F8.E5M2, torch.float8_e5m2)):
        codes = np.arange(256, dtype=np.uint8)
        mine = F8.decode(codes, fmt)
        th = torch.from_numpy(codes).view(dt).float().numpy().astype(np.float64)
        assert ((mine == th) | (np.isnan(mine) & np.isnan(th))).all(), fmt
        v = (g.standard_normal(20000) * np.exp(g.uniform(-14, 12, 20000))).astype(np.float32)
        # midpoints between neighbouring finite values (ties) and their negatives
        fin = np.sort(mine[np.isfinite(mine) & (mine >= 0)])
        mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
        v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0])])
        v = v[np.abs(v) <= F8.fmax(fmt)]
        got = F8.encode(v.astype(np.float64), fmt)
        want = torch.from_numpy(v).to(dt).view(torch.uint8).numpy()
        assert (got == want).all(), (fmt, v[got != want][:5])


def check_fp8_saturation_and_scaling():
    F8 = oracle.fp8
    # beyond the largest finite value: saturate, keep the sign
    assert list(F8.encode([449.0, 1e9, -1e9, 464.0], F8.E4M3)) == [0x7E, 0x7E, 0xFE, 0x7E]
    assert list(F8.encode([57345.0, 1e30, -61440.0], F8.E5M2)) == [0x7B, 0x7B, 0xFB]
    # ties to even: 1 + 1/16 -> 1 (mantissa 0), 1 + 3/16 -> 1.25 (mantissa 2)
    assert list(F8.encode([1.0625, 1.1875], F8.E4M3)) == [0x38, 0x3A]
    # smallest subnormals: 2^-9 (e4m3) and 2^-16 (e5m2); half of them rounds to 0
    assert list(F8.encode([2.0 ** -9, 2.0 ** -10, 2.0 ** -16], F8.E4M3)) == [0x01, 0x00, 0x00]
    assert list(F8.encode([2.0 ** -16, 3 * 2.0 ** -17], F8.E5M2)) == [0x01, 0x02]
    # scale = fmax / amax in float32; amax 0 -> 1; the amax element maps to fmax
    s, si = F8.scales(np.float32([2.0, 0.0, 3.0]), F8.E4M3)
    assert s[0] == 224.0 and s[1] == 1.0 and si[0] == np.float32(1 / 224.0)
    assert s[2] == np.float32(np.float32(448.0) / np.float32(3.0))
    x = np.array([[3.0, -1.0, 0.001]], np.float32)
    q, si, d = F8.quantize_tensor(x, F8.E4M3)
    assert q[0, 0] == 0x7E and d[0, 0] == 448.0 * float(si)
    # per-expert scaling: each expert's amax maps to fmax
    w = np.stack([np.full((2, 3), 0.5, np.float32), np.full((2, 3), -8.0, np.float32)])
    q, si, d = F8.quantize_experts(w, F8.E5M2)
    assert (q[0] == 0x7B).all() and (q[1] == 0xFB).all()
    # 57344 * float32(1 / scale) is the amax up to the rounding of 1 / scale
    np.testing.assert_allclose(d, w.astype(np.float64), rtol=1e-7)


def _fp8_deq_loop(x, fmt, per_expert=False):
    """Current scaling written out with scalar loops over the pinned
    encode/decode: amax, float32 scale, float32 product, code, value."""
    F8 = oracle.fp8
    x = np.asarray(x, dtype=np.float32)
    units = [x[e] for e in range(x.shape[0])] if per_expert else [x]
    out = []
    for u in units:
        am = np.float32(0.0)
        for val in u.reshape(-1):
            am = max(am, np.float32(abs(val)))
        s = np.float32(1.0) if am == 0 else np.float32(np.float32(F8.fmax(fmt)) / am)
        si = np.float32(np.float32(1.0) / s)
        flat = [float(F8.decode(F8.encode([float(np.float32(val * s))], fmt), fmt)[0]) * float(si)
                for val in u.reshape(-1)]
        out.append(np.array(flat).reshape(u.shape))
    return np.stack(out) if per_expert else out[0]


def check_fp8_block_bruteforce(seed=19):
    """The FP8 forward and backward of a tiny block against per-token scalar
    loops over operands quantized by ``_fp8_deq_loop``: x, act e4m3 per
    tensor, weights e4m3 per expert, the gradients d_y_sorted, d_h0, d_h1
    e5m2 per tensor."""
    g = _rng(seed)
    x, Wg, wi0, wi1, wo = _tiny_block(g, T=12, D=4, F=3, E=3)
    x, Wg = x.astype(np.float32), Wg.astype(np.float32)
    wi0, wi1, wo = (w.astype(np.float32) for w in (wi0, wi1, wo))
    dy = g.standard_normal(x.shape).astype(np.float32)
    K = 2
    f = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, align=2, fp8=True)
    b = oracle.moe_backward(f, dy, x, wi0, wi1, wo, K, Wg=Wg)
    P = f["perm"]
    gs, rows = P["group_sizes"], f["rows"]
    xs = P["x_sorted"].astype(np.float32)
    xd = _fp8_deq_loop(xs, "e4m3")
    w0d, w1d, wod = (_fp8_deq_loop(w, "e4m3", per_expert=True) for w in (wi0, wi1, wo))
    grp = np.repeat(np.arange(len(gs)), gs)            # group of each routed row
    R = len(grp)
    F, D = wi0.shape[2], wi0.shape[1]
    h0 = np.zeros((rows, F))
    h1 = np.zeros((rows, F))
    for r in range(R):
        for c in range(F):
            h0[r, c] = sum(xd[r, k] * w0d[grp[r], k, c] for k in range(D))
            h1[r, c] = sum(xd[r, k] * w1d[grp[r], k, c] for k in range(D))
    np.testing.assert_allclose(f["h0"], h0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f["h1"], h1, rtol=1e-12, atol=1e-13)
    act = h0 / (1 + np.exp(-h0)) * h1
    ad = _fp8_deq_loop(act, "e4m3")
    ys = np.zeros((rows, D))
    for r in range(R):
        for c in range(D):
            ys[r, c] = sum(ad[r, k] * wod[grp[r], k, c] for k in range(F))
    np.testing.assert_allclose(f["y_sorted"], ys, rtol=1e-12, atol=1e-13)
    # backward: d_y_sorted rows are w * dy of their token (pinned elsewhere)
    dysd = _fp8_deq_loop(b["d_y_sorted"], "e5m2")
    d_act = np.zeros((rows, F))
    d_wo = np.zeros_like(wo, dtype=np.float64)
    for r in range(R):
        for c in range(F):
            d_act[r, c] = sum(dysd[r, k] * wod[grp[r], c, k] for k in range(D))
            for k in range(D):
                d_wo[grp[r], c, k] += ad[r, c] * dysd[r, k]
    np.testing.assert_allclose(b["d_act"], d_act, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["d_wo"], d_wo, rtol=1e-12, atol=1e-13)
    sg = 1 / (1 + np.exp(-h0))
    dh0 = d_act * h1 * sg * (1 + h0 * (1 - sg))
    dh1 = d_act * h0 * sg
    dh0d, dh1d = _fp8_deq_loop(dh0, "e5m2"), _fp8_deq_loop(dh1, "e5m2")
    d_xs = np.zeros((rows, D))
    d_wi0 = np.zeros_like(wi0, dtype=np.float64)
    for r in range(R):
        for k in range(D):
            d_xs[r, k] = sum(dh0d[r, c] * w0d[grp[r], k, c] + dh1d[r, c] * w1d[grp[r], k, c]
                             for c in range(F))
            for c in range(F):
                d_wi0[grp[r], k, c] += xd[r, k] * dh0d[r, c]
    np.testing.assert_allclose(b["d_x_sorted"], d_xs, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["d_wi_0"], d_wi0, rtol=1e-12, atol=1e-13)
    # and the FP8 block stays within the formats' rounding of the exact block
    e = oracle.moe_forward(x, wi0, wi1, wo, K, Wg=Wg, align=2)
    assert np.abs(f["y"] - e["y"]).max() <= 0.15 * np.abs(e["y"]).max()
