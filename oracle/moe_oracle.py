"""Plain fp64 CPU oracle for the MoE expert-FFN path.  TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import or call this module.  The product (the HIP library and its
Python binding) never does: there is no CPU fallback.  The oracle shares no
code with the GPU path and imports nothing from it.

What it computes is the plain definition of a top-K mixture of SwiGLU
expert FFNs, forward and backward, with every intermediate kept in float64
(inputs are float32 arrays whose values are widened exactly):

  route         top-K of the router logits per token, softmax or sigmoid
                scores, optional renormalisation.  TransformerEngine MoE
                block pull request ("Add an MoE Block ... router,
                permutation, groupedGEMM and communication"), Description /
                Changes: fused top-K with optional sigmoid scoring.
  route variants  a per-expert bias that moves only the selection (the
                "pre_bias_logits" of the MaxText DeepSeek-V3 router), grouped
                top-K ("n_routing_groups" / "topk_routing_group"), and the
                optional auxiliary load-balancing loss of the TransformerEngine
                MoE block (its Description lists grouped and sigmoid scoring
                and the balancing loss as options of the fused router).
  permute       stable grouping of the routed (token, slot) pairs by expert,
                per-expert group sizes, optional align_size padding and
                capacity dropping.  Same pull request: the dispatch state
                (group_sizes, sorted_indices, routing weights, pad_offsets)
                and the align_size receive-buffer bound; MaxText grouped-GEMM
                pull request, Tests: token dropping.
  gmm / tgmm    grouped GEMM and transposed grouped GEMM with in-place
                partial sums.  MaxText "Overlap moe comms with collective
                matmul", Description and the review of the gmm backward
                rule and of the partial_sum shape assertion.
  MLP biases    optional per-expert biases on the up- and down-projection
                outputs and their gradients (per-group row sums); MaxText
                "Overlap moe comms" pull request, Testing (MLP bias with the
                chunked layer) and the chunked layer's w0/w1/wo bias arguments.
  swiglu        silu(gate_proj_out) * up_proj_out (TransformerEngine pull
                request commit notes naming the two SwiGLU projection outputs).
  combine       weighted sum of each token's K expert outputs, and its
                hand-derived backward (TransformerEngine pull request review
                of ``_combine_bwd``).

Where the pages leave a step open this module takes one reading and states
it in the docstring of the function concerned.  Every function is pinned by
tests that do not re-use its own formula (brute force, closed forms,
invariants, library routines of a different algorithm, finite differences).
"""
from __future__ import annotations

import numpy as np

from . import fp8_oracle as F8

SOFTMAX = "softmax"
SIGMOID = "sigmoid"
LOGIT = "logit"      # a per-expert bias added to the logits (selection and weights)
SELECT = "select"    # a per-expert bias added to the scores for the selection only


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def router_logits(x, Wg) -> np.ndarray:
    """logits[T, E] = x[T, D] . Wg[D, E] (the gate projection; MaxText
    explicit-sharding pull request review: the gate maps [B, S, E] to
    [B, S, num_exp])."""
    return _f64(x) @ _f64(Wg)


def biased_logits_f32(logits, bias=None) -> np.ndarray:
    """The float32 values on which experts are selected.

    Reading: the Zipf expert prior is a per-expert additive bias on the
    router logits that affects both selection and weights; the addition is
    done in float32, the precision of the logits the kernels route on.
    """
    z = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return z


def _scores(z, score: str) -> np.ndarray:
    """float64 scores of float64 logits z [T, E]: softmax over the E experts
    or the logistic function per expert."""
    if score == SOFTMAX:
        m = z.max(axis=1, keepdims=True)
        ez = np.exp(z - m)
        return ez / ez.sum(axis=1, keepdims=True)
    if score == SIGMOID:
        return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(score)


def route(logits, K: int, score: str = SOFTMAX, renorm: bool = True, bias=None,
          bias_mode: str = LOGIT, n_groups: int = 0, topk_groups: int = 0):
    """Top-K routing.  Returns (ids int32 [T, K], weights float64 [T, K]).

    Selection: experts ranked by their selection key, descending; equal keys
    rank the lower expert id first; slot j holds the j-th ranked expert.
      bias_mode "logit": the key is the float32 logit plus bias (softmax and
        sigmoid are increasing, so ranking the logits ranks the scores); the
        weights are scores of the biased logits.
      bias_mode "select": the key is score + bias with the scores of the
        unbiased logits (a bias that only moves the selection); the weights
        are the unbiased scores.
    Weights: softmax p_e = exp(z_e - max z) / sum_e' exp(z_e' - max z) over
    all E experts, or sigmoid s_e = 1 / (1 + exp(-z_e)); the K selected
    scores, divided by their sum when renorm is set.
    Grouped selection (n_groups > 1; E divisible by n_groups): the experts
    form n_groups consecutive groups of E / n_groups; a group scores the sum
    of its two largest keys (its one key for single-expert groups); the
    topk_groups best groups (ties: lower group id) stay candidates and the K
    experts are the top-K keys among them.
    """
    z32 = biased_logits_f32(logits, bias if bias_mode == LOGIT else None)
    T, E = z32.shape
    assert 1 <= K <= E
    p = _scores(z32.astype(np.float64), score)
    if bias_mode == LOGIT:
        key = z32.astype(np.float64)
    elif bias_mode == SELECT:
        key = p + (0.0 if bias is None else _f64(bias)[None, :])
    else:
        raise ValueError(bias_mode)
    if n_groups > 1:
        assert E % n_groups == 0 and 1 <= topk_groups <= n_groups
        eg = E // n_groups
        assert K <= topk_groups * eg
        kg = key.reshape(T, n_groups, eg)
        gscore = -np.sort(-kg, axis=2)[:, :, :min(2, eg)].sum(axis=2)
        gbest = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]
        keep = np.zeros((T, n_groups), dtype=bool)
        np.put_along_axis(keep, gbest, True, axis=1)
        key = np.where(np.repeat(keep, eg, axis=1), key, -np.inf)
    # stable sort of the negated keys: descending, ties keep ascending id
    order = np.argsort(-key, axis=1, kind="stable")
    ids = order[:, :K]
    w = np.take_along_axis(p, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def route_weights(logits, ids, score: str = SOFTMAX, renorm: bool = True, bias=None,
                  bias_mode: str = LOGIT) -> np.ndarray:
    """Routing weights of a given selection ids [T, K] (float64 [T, K]): the
    weights ``route`` assigns once its experts are chosen.  The scores are
    those of the float32 logits plus the bias for bias_mode "logit", of the
    logits alone for "select" (the bias only moved the selection); softmax
    over all E experts or the logistic function; the K selected scores,
    divided by their sum when renorm is set (same pull request, fused top-K
    router)."""
    z = biased_logits_f32(logits, bias if bias_mode == LOGIT else None).astype(np.float64)
    sel = np.asarray(ids, dtype=np.int64)
    if score == SOFTMAX:
        # softmax scores of the selected experts: exp(z_e - max) / sum_all
        m = z.max(axis=1, keepdims=True)
        num = np.exp(np.take_along_axis(z, sel, axis=1) - m)
        sc = num / np.exp(z - m).sum(axis=1, keepdims=True)
    elif score == SIGMOID:
        sc = 1.0 / (1.0 + np.exp(-np.take_along_axis(z, sel, axis=1)))
    else:
        raise ValueError(score)
    if renorm:
        sc = sc / sc.sum(axis=1, keepdims=True)
    return sc


def route_bwd(logits, ids, d_w, score: str = SOFTMAX, renorm: bool = True, bias=None,
              bias_mode: str = LOGIT):
    """Gradient of the routing weights with respect to the router logits,
    with the selection held fixed.  Returns d_logits float64 [T, E].

    With w_j the weight of slot j and e_j its expert:
      softmax + renorm   w_j = exp(z_ej) / sum_i exp(z_ei), so
                         d z_ej = w_j (d w_j - sum_i w_i d w_i); other experts 0.
      softmax, no renorm w_j = p_ej over all E experts, so for every expert e
                         d z_e = p_e ([e = e_j] d w_j - sum_i p_ei d w_i).
      sigmoid + renorm   w_j = s_j / S with S = sum_i s_i, so
                         d s_j = (d w_j - sum_i w_i d w_i) / S and
                         d z_ej = d s_j s_j (1 - s_j).
      sigmoid, no renorm d z_ej = d w_j s_j (1 - s_j).
    The additive prior has unit derivative, so d logits = d z.  With
    bias_mode "select" the weights are scores of the unbiased logits, so z
    is the logits themselves (the bias only moved the selection).
    """
    z = biased_logits_f32(logits, bias if bias_mode == LOGIT else None).astype(np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    dw = _f64(d_w)
    T, E = z.shape
    K = ids.shape[1]
    dz = np.zeros((T, E), dtype=np.float64)
    rows = np.arange(T)[:, None]
    if score == SOFTMAX:
        m = z.max(axis=1, keepdims=True)
        ez = np.exp(z - m)
        p = ez / ez.sum(axis=1, keepdims=True)
        p_sel = np.take_along_axis(p, ids, axis=1)
        if renorm:
            w = p_sel / p_sel.sum(axis=1, keepdims=True)
            inner = (w * dw).sum(axis=1, keepdims=True)
            dz[rows, ids] = w * (dw - inner)
        else:
            inner = (p_sel * dw).sum(axis=1, keepdims=True)
            dz = -p * inner
            dz[rows, ids] += p_sel * dw
    elif score == SIGMOID:
        s = 1.0 / (1.0 + np.exp(-z))
        s_sel = np.take_along_axis(s, ids, axis=1)
        if renorm:
            S = s_sel.sum(axis=1, keepdims=True)
            w = s_sel / S
            inner = (w * dw).sum(axis=1, keepdims=True)
            ds = (dw - inner) / S
        else:
            ds = dw
        dz[rows, ids] = ds * s_sel * (1.0 - s_sel)
    else:
        raise ValueError(score)
    assert K == dw.shape[1]
    return dz


def _aux_probs(logits, score: str):
    """Per-token expert probabilities for the balancing loss: softmax over
    the E pre-bias logits, or for sigmoid scoring the sigmoids normalised to
    sum 1 over the E experts.  Returns (p [T, E], s or None)."""
    z = _f64(logits)
    if score == SOFTMAX:
        return _scores(z, SOFTMAX), None
    s = _scores(z, SIGMOID)
    return s / s.sum(axis=1, keepdims=True), s


def aux_loss(logits, ids, E: int, alpha: float, score: str = SOFTMAX):
    """Auxiliary load-balancing loss (optional in the TransformerEngine MoE
    block; its form is not written out on the pages, so this takes the
    plainest one, the product of routed fraction and mean probability):
      f_e  = (selected slots with expert e) / (T K), counted on the
             selection before any capacity dropping;
      P_e  = (1 / T) sum_t p_te with p from ``_aux_probs``;
      loss = alpha * E * sum_e f_e P_e.
    f is a count and carries no gradient.  Returns (loss, counts int64 [E],
    P float64 [E])."""
    ids = np.asarray(ids, dtype=np.int64)
    T, K = ids.shape
    counts = np.bincount(ids.reshape(-1), minlength=E)[:E]
    p, _ = _aux_probs(logits, score)
    P = p.mean(axis=0)
    f = counts / float(T * K)
    return float(alpha * E * np.dot(f, P)), counts, P


def aux_loss_bwd(logits, counts, K: int, alpha: float, score: str = SOFTMAX):
    """d loss / d logits [T, E] for ``aux_loss`` with the counts held fixed:
      softmax:  d z_tk = (alpha E / T) p_tk (f_k - sum_e f_e p_te)
      sigmoid:  p = s / S, d p_e / d z_k = s_k (1 - s_k) / S ([e = k] - p_e), so
                d z_tk = (alpha E / T) s_k (1 - s_k) / S_t (f_k - sum_e f_e p_te)."""
    p, s = _aux_probs(logits, score)
    T, E = p.shape
    f = np.asarray(counts, dtype=np.float64) / float(T * K)
    inner = (p * f[None, :]).sum(axis=1, keepdims=True)
    scale = alpha * E / T
    if score == SOFTMAX:
        return scale * p * (f[None, :] - inner)
    S = s.sum(axis=1, keepdims=True)
    return scale * s * (1.0 - s) / S * (f[None, :] - inner)


# ---------------------------------------------------------------------------
# Permutation (dispatch) and its backward
# ---------------------------------------------------------------------------

def rows_bound(T: int, K: int, E: int, align: int = 0, capacity: int = 0,
               capacity_layout: bool = False) -> int:
    """Static row count of the expert-sorted buffers.

    T*K routed rows; with align_size a > 0 each expert can add at most a-1
    padding rows, so T*K + E*(a-1) (the worst-case receive-buffer bound the
    TransformerEngine pull request review derives for align_size > 0); in
    capacity layout every expert owns exactly C rows, so E*C.
    """
    if capacity_layout:
        return E * capacity
    return T * K + (E * (align - 1) if align > 0 else 0)


def permute(x, ids, E: int, align: int = 0, capacity: int = 0,
            capacity_layout: bool = False, rows: int | None = None):
    """Group the routed slots by expert.

    Slot s = t*K + j is token t's j-th choice.  Readings taken:
      * router order is ascending s; with capacity C > 0 a slot is kept iff
        fewer than C earlier kept slots chose the same expert (overflow is
        dropped in router order);
      * group_sizes[e] = kept count, rounded up to a multiple of align_size
        when align_size > 0 (an empty group stays empty); in capacity layout
        every group has C rows starting at e*C;
      * inside a group the kept slots keep ascending s (a stable sort);
      * padding rows of x_sorted are zero.
    Returns a dict: counts [E], group_sizes [E], group_offsets [E+1],
    row_of_slot [T*K] (-1 = dropped), slot_of_row [rows] (-1 = padding),
    x_sorted [rows, D] float64 (None if x is None).
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    assert flat.min(initial=0) >= 0 and flat.max(initial=0) < E
    kept = np.zeros(T * K, dtype=bool)
    counts = np.zeros(E, dtype=np.int64)
    for s in range(T * K):
        e = flat[s]
        if capacity == 0 or counts[e] < capacity:
            kept[s] = True
            counts[e] += 1
    if capacity_layout:
        assert capacity > 0
        group_sizes = np.full(E, capacity, dtype=np.int64)
    elif align > 0:
        group_sizes = ((counts + align - 1) // align) * align
    else:
        group_sizes = counts.copy()
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + group_sizes[e]
    bound = rows_bound(T, K, E, align, capacity, capacity_layout)
    nrows = bound if rows is None else rows
    assert nrows >= offsets[E]
    row_of_slot = np.full(T * K, -1, dtype=np.int64)
    slot_of_row = np.full(nrows, -1, dtype=np.int64)
    fill = np.zeros(E, dtype=np.int64)
    for s in range(T * K):
        if kept[s]:
            e = flat[s]
            r = offsets[e] + fill[e]
            fill[e] += 1
            row_of_slot[s] = r
            slot_of_row[r] = s
    x_sorted = None
    if x is not None:
        xf = _f64(x)
        x_sorted = np.zeros((nrows, xf.shape[1]), dtype=np.float64)
        for r in range(nrows):
            if slot_of_row[r] >= 0:
                x_sorted[r] = xf[slot_of_row[r] // K]
    return dict(counts=counts.astype(np.int32), group_sizes=group_sizes.astype(np.int32),
                group_offsets=offsets.astype(np.int32), row_of_slot=row_of_slot.astype(np.int32),
                slot_of_row=slot_of_row.astype(np.int32), x_sorted=x_sorted)


def permute_bwd(d_x_sorted, row_of_slot, T: int, K: int) -> np.ndarray:
    """dx[t] = sum over token t's kept slots of d_x_sorted[row] (the adjoint
    of the row gather; TransformerEngine pull request, sequence diagram:
    the dispatch backward returns d_inputs)."""
    d = _f64(d_x_sorted)
    ros = np.asarray(row_of_slot).reshape(T, K)
    dx = np.zeros((T, d.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(K):
            r = ros[t, j]
            if r >= 0:
                dx[t] += d[r]
    return dx


# ---------------------------------------------------------------------------
# Grouped GEMMs
# ---------------------------------------------------------------------------

def gmm(lhs, rhs, group_sizes, trans_rhs: bool = False, partial=None, rows_out: int | None = None,
        bias=None):
    """Grouped GEMM: for each group g, rows [o_g, o_g + n_g) of the output are
    lhs[those rows] . rhs[g] (rhs[g] is [K, N]; with trans_rhs it is stored
    [N, K] and used transposed).  With ``partial`` the result is added to a
    copy of it (in-place partial-sum accumulation).  The output may have
    fewer rows than lhs (lhs padded to a row tile, partial sum not).
    Rows at or beyond sum(group_sizes) are zero without ``partial`` and
    equal to ``partial`` with it.  ``bias`` [G, N] (the per-expert MLP bias
    of the MaxText "Overlap moe comms" pull request's chunked layer,
    w0_bias / w1_bias / wo_bias) adds bias[g] to every row of group g.
    """
    gs = np.asarray(group_sizes, dtype=np.int64)
    lhs = np.asarray(lhs)
    M_lhs = lhs.shape[0]
    N = rhs.shape[1] if trans_rhs else rhs.shape[2]
    M_out = M_lhs if rows_out is None else rows_out
    if partial is not None:
        out = _f64(partial).copy()
        M_out = out.shape[0]
    else:
        out = np.zeros((M_out, N), dtype=np.float64)
    assert gs.sum() <= M_out <= M_lhs
    start = 0
    for g in range(len(gs)):
        n = int(gs[g])
        if n > 0:
            W = _f64(rhs[g])
            if trans_rhs:
                W = W.T
            out[start:start + n] += _f64(lhs[start:start + n]) @ W
            if bias is not None:
                out[start:start + n] += _f64(bias[g])[None, :]
        start += n
    return out


def group_sum(rows, group_sizes) -> np.ndarray:
    """out[g] = sum of the rows of group g, [G, N]: the gradient of a
    per-group bias added to those rows (zero for an empty group)."""
    gs = np.asarray(group_sizes, dtype=np.int64)
    rows = _f64(rows)
    out = np.zeros((len(gs), rows.shape[1]), dtype=np.float64)
    start = 0
    for g in range(len(gs)):
        n = int(gs[g])
        out[g] = rows[start:start + n].sum(axis=0)
        start += n
    return out


def tgmm(lhs, rhs, group_sizes, partial=None):
    """Transposed grouped GEMM: out[g] = lhs[rows of g]^T . rhs[rows of g],
    shape [G, K, N] (MaxText "Overlap moe comms" review: the tgmm output
    is (num_local_groups, in_size, out_size)).  An empty group yields zero,
    or the partial sum unchanged when one is given (Testing: tgmm with
    zero-initialised empty expert groups)."""
    gs = np.asarray(group_sizes, dtype=np.int64)
    lhs = np.asarray(lhs)
    rhs = np.asarray(rhs)
    G, Kd, N = len(gs), lhs.shape[1], rhs.shape[1]
    out = _f64(partial).copy() if partial is not None else np.zeros((G, Kd, N), dtype=np.float64)
    start = 0
    for g in range(G):
        n = int(gs[g])
        if n > 0:
            out[g] += _f64(lhs[start:start + n]).T @ _f64(rhs[start:start + n])
        start += n
    return out


# ---------------------------------------------------------------------------
# SwiGLU
# ---------------------------------------------------------------------------

def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu(h0, h1) -> np.ndarray:
    """act = silu(h0) * h1 with silu(z) = z * sigmoid(z)."""
    h0 = _f64(h0)
    return h0 * _sigmoid(h0) * _f64(h1)


def swiglu_bwd(h0, h1, d_act):
    """d h0 = d_act * h1 * sigma (1 + h0 (1 - sigma)), d h1 = d_act * silu(h0),
    sigma = sigmoid(h0) (derivative of z * sigmoid(z))."""
    h0, h1, da = _f64(h0), _f64(h1), _f64(d_act)
    sg = _sigmoid(h0)
    return da * h1 * sg * (1.0 + h0 * (1.0 - sg)), da * h0 * sg


# ---------------------------------------------------------------------------
# Combine (unpermute) and its backward
# ---------------------------------------------------------------------------

def combine(y_sorted, row_of_slot, w, T: int, K: int) -> np.ndarray:
    """y[t] = sum_j w[t, j] * y_sorted[row of slot (t, j)]; dropped slots add
    nothing and the surviving weights are not renormalised (the einsum
    "BKE,BK -> BE" of the combine)."""
    ys = _f64(y_sorted)
    ros = np.asarray(row_of_slot).reshape(T, K)
    w = _f64(w).reshape(T, K)
    y = np.zeros((T, ys.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(K):
            r = ros[t, j]
            if r >= 0:
                y[t] += w[t, j] * ys[r]
    return y


def combine_bwd(dy, y_sorted, row_of_slot, w, rows: int):
    """Hand-derived backward of the combine:
    d_y_sorted[row of (t, j)] = w[t, j] * dy[t] (rows no slot maps to get 0),
    d_w[t, j] = <dy[t], y_sorted[row of (t, j)]> (0 for a dropped slot)."""
    dy = _f64(dy)
    ys = _f64(y_sorted)
    T = dy.shape[0]
    K = np.asarray(w).reshape(T, -1).shape[1]
    ros = np.asarray(row_of_slot).reshape(T, K)
    w = _f64(w).reshape(T, K)
    d_ys = np.zeros((rows, dy.shape[1]), dtype=np.float64)
    d_w = np.zeros((T, K), dtype=np.float64)
    for t in range(T):
        for j in range(K):
            r = ros[t, j]
            if r >= 0:
                d_ys[r] = w[t, j] * dy[t]
                d_w[t, j] = float(dy[t] @ ys[r])
    return d_ys, d_w


# ---------------------------------------------------------------------------
# The whole block, forward and backward
# ---------------------------------------------------------------------------

def moe_forward(x, wi_0, wi_1, wo, K: int, *, Wg=None, logits=None, bias=None,
                score: str = SOFTMAX, renorm: bool = True, align: int = 0,
                capacity: int = 0, capacity_layout: bool = False,
                n_chunks: int = 1, lhs_rows: int | None = None, bias_mode: str = LOGIT,
                n_groups: int = 0, topk_groups: int = 0, aux_alpha: float = 0.0,
                b_wi_0=None, b_wi_1=None, b_wo=None, fp8: bool = False):
    """Forward pass.  Either ``Wg`` (router logits = x . Wg) or ``logits``.

    With n_chunks > 1 the up-projections are computed as the in-place
    partial-sum accumulation over n_chunks equal slices of d_model (the
    chunked loop of the "Overlap moe comms" pull request); lhs_rows is the
    row count of the (padded) sorted-token buffer, the output rows being the
    routed rows.  bias_mode / n_groups / topk_groups select the routing
    variant of ``route``; aux_alpha > 0 adds ``aux_loss`` (returned as
    "aux_loss", with its counts).  b_wi_0, b_wi_1 [E, F] and b_wo [E, D] are
    optional per-expert MLP biases; under partial sums the up-projection
    biases are added once, with the last chunk.  fp8: the expert GEMMs take
    FP8 operands with current scaling (``fp8_oracle``): x_sorted and act
    e4m3 per tensor, the expert weights e4m3 per expert (no chunking).
    Returns every residual the backward needs.
    """
    x = np.asarray(x)
    T, D = x.shape
    E = wi_0.shape[0]
    if logits is None:
        logits = router_logits(x, Wg)
    ids, w = route(logits, K, score, renorm, bias, bias_mode, n_groups, topk_groups)
    aux = aux_loss(logits, ids, E, aux_alpha, score) if aux_alpha > 0 else None
    nrows = rows_bound(T, K, E, align, capacity, capacity_layout)
    P = permute(x, ids, E, align, capacity, capacity_layout,
                rows=nrows if lhs_rows is None else lhs_rows)
    xs = P["x_sorted"]
    gs = P["group_sizes"]
    q8 = {}
    if fp8:
        assert n_chunks == 1, "the FP8 variant is unchunked"
        q8["x"] = F8.quantize_tensor(xs, F8.E4M3)
        for name, wt in (("wi_0", wi_0), ("wi_1", wi_1), ("wo", wo)):
            q8[name] = F8.quantize_experts(wt, F8.E4M3)
        h0 = gmm(q8["x"][2], q8["wi_0"][2], gs, rows_out=nrows, bias=b_wi_0)
        h1 = gmm(q8["x"][2], q8["wi_1"][2], gs, rows_out=nrows, bias=b_wi_1)
    elif n_chunks > 1:
        c = D // n_chunks
        h0 = h1 = None
        for i in range(n_chunks):
            sl = slice(i * c, (i + 1) * c)
            last = i == n_chunks - 1
            h0 = gmm(xs[:, sl], wi_0[:, sl, :], gs, partial=h0, rows_out=nrows,
                     bias=b_wi_0 if last else None)
            h1 = gmm(xs[:, sl], wi_1[:, sl, :], gs, partial=h1, rows_out=nrows,
                     bias=b_wi_1 if last else None)
    else:
        h0 = gmm(xs, wi_0, gs, rows_out=nrows, bias=b_wi_0)
        h1 = gmm(xs, wi_1, gs, rows_out=nrows, bias=b_wi_1)
    act = swiglu(h0, h1)
    if fp8:
        q8["act"] = F8.quantize_tensor(act, F8.E4M3)
        y_sorted = gmm(q8["act"][2], q8["wo"][2], gs, bias=b_wo)
    else:
        y_sorted = gmm(act, wo, gs, bias=b_wo)
    y = combine(y_sorted, P["row_of_slot"], w, T, K)
    out = dict(logits=_f64(logits), ids=ids, w=w, perm=P, x_sorted=xs, h0=h0, h1=h1,
               act=act, y_sorted=y_sorted, y=y, rows=nrows, bias_mode=bias_mode,
               aux_alpha=aux_alpha,
               mlp_bias=any(b is not None for b in (b_wi_0, b_wi_1, b_wo)), fp8=q8 or None)
    if aux is not None:
        out["aux_loss"], out["aux_counts"], out["aux_probs"] = aux
    return out


def moe_backward(fwd, dy, x, wi_0, wi_1, wo, K: int, *, Wg=None, bias=None,
                 score: str = SOFTMAX, renorm: bool = True):
    """Backward pass for upstream dy (hand-derived, mirroring the forward as
    the TransformerEngine block's single custom VJP does).  Returns dict with
    dx, d_wi_0, d_wi_1, d_wo, d_logits, d_w, (if Wg given) d_Wg and (with MLP
    biases) d_b_wi_0, d_b_wi_1, d_b_wo: each bias gradient is the per-group
    sum of the gradient rows of the output it was added to."""
    x = np.asarray(x)
    T = x.shape[0]
    P = fwd["perm"]
    gs = P["group_sizes"]
    ros = P["row_of_slot"]
    nrows = fwd["rows"]
    d_ys, d_w = combine_bwd(dy, fwd["y_sorted"], ros, fwd["w"], nrows)
    q8 = fwd.get("fp8")
    if q8:
        # backward GEMMs: gradients e5m2 per tensor, the forward's e4m3
        # operands reused (the second quantized copy of each)
        g8 = {"d_y_sorted": F8.quantize_tensor(d_ys, F8.E5M2)}
        d_act = gmm(g8["d_y_sorted"][2], q8["wo"][2], gs, trans_rhs=True)
        d_wo = tgmm(q8["act"][2], g8["d_y_sorted"][2], gs)
    else:
        d_act = gmm(d_ys, wo, gs, trans_rhs=True)
        d_wo = tgmm(fwd["act"], d_ys, gs)
    d_h0, d_h1 = swiglu_bwd(fwd["h0"], fwd["h1"], d_act)
    xs = fwd["x_sorted"][:nrows]
    if q8:
        g8["d_h0"] = F8.quantize_tensor(d_h0, F8.E5M2)
        g8["d_h1"] = F8.quantize_tensor(d_h1, F8.E5M2)
        xd = q8["x"][2][:nrows]
        d_xs = gmm(g8["d_h0"][2], q8["wi_0"][2], gs, trans_rhs=True)
        d_xs = gmm(g8["d_h1"][2], q8["wi_1"][2], gs, trans_rhs=True, partial=d_xs)
        d_wi_0 = tgmm(xd, g8["d_h0"][2], gs)
        d_wi_1 = tgmm(xd, g8["d_h1"][2], gs)
    else:
        d_xs = gmm(d_h0, wi_0, gs, trans_rhs=True)
        d_xs = gmm(d_h1, wi_1, gs, trans_rhs=True, partial=d_xs)
        d_wi_0 = tgmm(xs, d_h0, gs)
        d_wi_1 = tgmm(xs, d_h1, gs)
    dx = permute_bwd(d_xs, ros, T, K)
    d_logits = route_bwd(fwd["logits"], fwd["ids"], d_w, score, renorm, bias,
                         fwd.get("bias_mode", LOGIT))
    if fwd.get("aux_alpha", 0.0) > 0:
        # the balancing loss is added to the objective with weight one
        d_logits = d_logits + aux_loss_bwd(fwd["logits"], fwd["aux_counts"], K,
                                           fwd["aux_alpha"], score)
    out = dict(dx=dx, d_wi_0=d_wi_0, d_wi_1=d_wi_1, d_wo=d_wo, d_logits=d_logits, d_w=d_w,
               d_y_sorted=d_ys, d_act=d_act, d_h0=d_h0, d_h1=d_h1, d_x_sorted=d_xs)
    if q8:
        out["fp8"] = g8
    if fwd.get("mlp_bias", False):
        out["d_b_wi_0"] = group_sum(d_h0, gs)
        out["d_b_wi_1"] = group_sum(d_h1, gs)
        out["d_b_wo"] = group_sum(d_ys, gs)
    if Wg is not None:
        out["d_Wg"] = _f64(x).T @ d_logits
        out["dx"] = dx + d_logits @ _f64(Wg).T
    return out
