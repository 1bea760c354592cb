"""The MoE expert-FFN block as a fixed sequence of libmoe.so calls.

``MoEPlan`` preallocates every buffer of one workload (sizes are static:
the sorted buffers have the worst-case row count, so nothing depends on
device-resident counts and no host synchronisation is needed), then
``forward`` and ``backward`` only enqueue kernels on the current stream.

The sequence mirrors the single hand-derived custom VJP of the
TransformerEngine MoE block (route -> dispatch -> three grouped GEMMs ->
combine, and the reverse for the backward) with the gmm backward rule of
the MaxText "Overlap moe comms with collective matmul" pull request
(d_lhs = gmm with the rhs transposed, d_rhs = tgmm, in-place partial sums).
The up-projections can run as a loop over contracting-dim chunks of
d_model accumulating into float32 partial sums (that pull request's
chunked gmm).
"""
from __future__ import annotations

import contextlib
import dataclasses
from typing import Optional

import torch

from . import _binding as B


@dataclasses.dataclass(frozen=True)
class MoEShape:
    T: int
    D: int
    F: int
    E: int
    K: int
    dtype: torch.dtype = torch.bfloat16
    score: str = "softmax"
    renorm: bool = True
    align: int = 0
    capacity: int = 0
    capacity_layout: bool = False
    n_chunks: int = 1
    pad_rows_to: int = 0
    # one [E, D, 2F] up-projection weight wi = [wi_0 | wi_1] (the fused wi
    # of the TransformerEngine MoE block): one up-projection gmm, one
    # transposed-rhs gmm over 2F for d_x_sorted, one tgmm for d_wi
    fused_wi: bool = False
    # routing variants: how the bias enters ("logit" or "select"), grouped
    # top-K (n_groups > 1), and the load-balancing loss weight (0 = off)
    bias_mode: str = "logit"
    n_groups: int = 0
    topk_groups: int = 0
    aux_alpha: float = 0.0
    # per-expert MLP biases on the up- and down-projection outputs (added in
    # the GEMM epilogues; under partial sums with the last chunk) and their
    # gradients as per-group row sums
    mlp_bias: bool = False
    # FP8 expert GEMMs with current scaling: x_sorted and act e4m3 per
    # tensor, the expert weights e4m3 per expert, the gradients d_y_sorted,
    # d_h0, d_h1 e5m2 per tensor; each operand quantized once into the
    # row-wise and transposed copies its GEMMs read (unchunked, two weights)
    fp8: bool = False


def _round_up(a: int, b: int) -> int:
    return a if b <= 0 else ((a + b - 1) // b) * b


class MoEPlan:
    """Buffers and call sequence for one MoE FFN workload on one GPU."""

    def __init__(self, shape: MoEShape, device="cuda", router: bool = True):
        s = self.s = shape
        B.load()
        dev = torch.device(device)
        self.device = dev
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        act = dict(dtype=s.dtype, device=dev)
        self.rows = B.moe_rows_bound(s.T, s.K, s.E, s.align, s.capacity, s.capacity_layout)
        self.lhs_rows = _round_up(self.rows, s.pad_rows_to)
        part = f32 if s.n_chunks > 1 else act   # chunked up-projection keeps fp32 partials
        self.router = router
        self.gs_T = torch.tensor([s.T], **i32)
        # forward
        self.logits = torch.empty((s.T, s.E), **f32)
        if s.aux_alpha > 0:
            self.aux_loss = torch.empty(1, **f32)
            self.aux_counts = torch.empty(s.E, **i32)
            self.aux_probs = torch.empty(s.E, **f32)
            self.aux_ws = torch.empty(max(B.moe_aux_loss_workspace(s.T, s.E), 256),
                                      dtype=torch.uint8, device=dev)
        self.ids = torch.empty((s.T, s.K), **i32)
        self.w = torch.empty((s.T, s.K), **f32)
        self.idx = dict(counts=torch.empty(s.E, **i32), group_sizes=torch.empty(s.E, **i32),
                        group_offsets=torch.empty(s.E + 1, **i32),
                        row_of_slot=torch.empty(s.T * s.K, **i32),
                        slot_of_row=torch.empty(self.lhs_rows, **i32))
        self.ws = torch.empty(max(B.moe_permute_workspace(s.T, s.K, s.E), 256), dtype=torch.uint8,
                              device=dev)
        self.err = torch.zeros(1, **i32)
        self.x_sorted = torch.empty((self.lhs_rows, s.D), **act)
        if s.fused_wi:
            # gate and up halves of one [rows, 2F] product
            self.h = torch.empty((self.rows, 2 * s.F), **part)
            self.h0, self.h1 = self.h[:, :s.F], self.h[:, s.F:]
        else:
            self.h0 = torch.empty((self.rows, s.F), **part)
            self.h1 = torch.empty((self.rows, s.F), **part)
        self.act = torch.empty((self.rows, s.F), **act)
        self.y_sorted = torch.empty((self.rows, s.D), **act)
        self.y = torch.empty((s.T, s.D), **act)
        # backward
        self.d_y_sorted = torch.empty((self.rows, s.D), **act)
        self.d_w = torch.empty((s.T, s.K), **f32)
        self.d_act = torch.empty((self.rows, s.F), **act)
        if s.fused_wi:
            self.d_h = torch.empty((self.rows, 2 * s.F), **act)
            self.d_h0, self.d_h1 = self.d_h[:, :s.F], self.d_h[:, s.F:]
        else:
            self.d_h0 = torch.empty((self.rows, s.F), **act)
            self.d_h1 = torch.empty((self.rows, s.F), **act)
        self.d_x_sorted = torch.empty((self.rows, s.D), **act)
        self.dx = torch.empty((s.T, s.D), **act)
        self.d_logits = torch.empty((s.T, s.E), **f32)
        if s.fused_wi:
            self.d_wi = torch.empty((s.E, s.D, 2 * s.F), **act)
            self.d_wi_0, self.d_wi_1 = self.d_wi[:, :, :s.F], self.d_wi[:, :, s.F:]
        else:
            self.d_wi_0 = torch.empty((s.E, s.D, s.F), **act)
            self.d_wi_1 = torch.empty((s.E, s.D, s.F), **act)
        self.d_wo = torch.empty((s.E, s.F, s.D), **act)
        if s.mlp_bias:
            if s.fused_wi:
                self.d_b_wi = torch.empty((s.E, 2 * s.F), **act)
                self.d_b_wi_0, self.d_b_wi_1 = self.d_b_wi[:, :s.F], self.d_b_wi[:, s.F:]
            else:
                self.d_b_wi_0 = torch.empty((s.E, s.F), **act)
                self.d_b_wi_1 = torch.empty((s.E, s.F), **act)
            self.d_b_wo = torch.empty((s.E, s.D), **act)
            self.gsum_ws = torch.empty(
                max(B.moe_group_sum_workspace(self.rows, s.E, max(2 * s.F, s.D)), 256),
                dtype=torch.uint8, device=dev)
        if s.fp8:
            self._init_fp8(dev)
        # router GEMM backward in float32 (d_logits is float32; its products
        # with x and Wg are exact-split bf16 MFMA contractions)
        self.d_Wg = torch.empty((1, s.D, s.E), **f32) if router else None
        if router and s.dtype == torch.bfloat16:
            self.router_ws = torch.empty(max(B.moe_router_bwd_workspace(s.T, s.D, s.E), 256),
                                         dtype=torch.uint8, device=dev)
        self.recorder = None   # optional callable(kind, flops, bytes) -> context manager

    def _init_fp8(self, dev):
        s = self.s
        if s.n_chunks > 1 or s.fused_wi:
            raise B.MoeError("the FP8 plan is unchunked with two up-projection weights")
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        E, D, F = s.E, s.D, s.F
        self.P8 = B.moe_fp8_padded_rows(self.lhs_rows, E)   # columns of the transposed copies
        q = self.q8 = {}
        # activations / gradients: (rows, cols) -> row-wise [rows, cols], transposed [cols, P]
        for name, rows, cols in (("x", self.lhs_rows, D), ("act", self.rows, F),
                                 ("d_y_sorted", self.rows, D), ("d_h0", self.rows, F),
                                 ("d_h1", self.rows, F)):
            q[name] = (torch.empty((rows, cols), **u8), torch.empty((cols, self.P8), **u8),
                       torch.empty((3, 1), **f32))
        # weights [E, a, b]: the row-wise copy only; the forward reads it as
        # [K, N] and the d_lhs product as [N, K]
        for name, a, b in (("wi_0", D, F), ("wi_1", D, F), ("wo", F, D)):
            q[name] = (torch.empty((E, a, b), **u8), None, torch.empty((3, E), **f32))
        self.w_rows = {D: torch.full((E,), D, dtype=torch.int32, device=dev),
                       F: torch.full((E,), F, dtype=torch.int32, device=dev)}
        ws = max(B.moe_fp8_scale_workspace(self.lhs_rows, max(D, F), 1),
                 B.moe_fp8_scale_workspace(E * max(D, F), max(D, F), E))
        self.f8_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)

    def _quant(self, name, x, fmt, stream):
        """Current scaling of an activation or gradient tensor into both copies."""
        qr, qt, sc = self.q8[name]
        # algorithmic bytes: x read twice (amax, quantize), two FP8 copies written
        nbytes = x.numel() * (2 * x.element_size() + 2)
        with self._rec("fp8_quantize", nbytes=nbytes):
            B.moe_fp8_amax_scale(x, fmt, scales=sc, workspace=self.f8_ws, stream=stream)
            B.moe_fp8_quantize(x, self.group_sizes, sc[1], fmt, q=qr, qt=qt, err=self.err,
                               stream=stream)

    def _quant_weight(self, name, w, stream):
        qr, _, sc = self.q8[name]
        E, a, b = w.shape
        w2 = w.reshape(E * a, b)
        # algorithmic bytes: w read twice (amax, quantize), one FP8 copy written
        with self._rec("fp8_quantize", nbytes=w.numel() * (2 * w.element_size() + 1)):
            B.moe_fp8_amax_scale(w2, "e4m3", G=E, scales=sc, workspace=self.f8_ws, stream=stream)
            B.moe_fp8_quantize(w2, self.w_rows[a], sc[1], "e4m3", per_group=True,
                               q=qr.view(E * a, b), err=self.err, stream=stream)

    def _forward_fp8(self, wi_0, wi_1, wo, mb, stream):
        s, q = self.s, self.q8
        gs, R = self.group_sizes, self.kept_rows
        self._quant("x", self.x_sorted, "e4m3", stream)
        for name, w in (("wi_0", wi_0), ("wi_1", wi_1), ("wo", wo)):
            self._quant_weight(name, w, stream)
        xq, _, sx = q["x"]
        for name, h in (("wi_0", self.h0), ("wi_1", self.h1)):
            wr, _, sw = q[name]
            with self._rec("gmm_nn", 2.0 * R * s.D * s.F, self._gb("gmm", s.D, s.F, in_b=1)):
                B.moe_gmm_fp8(xq, "e4m3", sx[2], wr, "e4m3", sw[2], gs, valid_rows=self.vrows, out=h, bias=mb.get(name),
                              trans_rhs=False, err=self.err, stream=stream)
        with self._rec("swiglu", nbytes=self._bytes().get("swiglu", 0) if self.recorder else 0):
            B.moe_swiglu(self.h0, self.h1, act=self.act, stream=stream)
        self._quant("act", self.act, "e4m3", stream)
        aq, _, sa = q["act"]
        wr, _, sw = q["wo"]
        with self._rec("gmm_nn", 2.0 * R * s.D * s.F, self._gb("gmm", s.F, s.D, in_b=1)):
            B.moe_gmm_fp8(aq, "e4m3", sa[2], wr, "e4m3", sw[2], gs, valid_rows=self.vact, out=self.y_sorted,
                          bias=mb.get("wo"), trans_rhs=False, err=self.err, stream=stream)

    def _backward_fp8(self, stream):
        s, q = self.s, self.q8
        gs, R, cnt = self.group_sizes, self.kept_rows, self.idx["counts"]
        self._quant("d_y_sorted", self.d_y_sorted, "e5m2", stream)
        dq, dqt, sd = q["d_y_sorted"]
        wor, _, swo = q["wo"]
        with self._rec("gmm_nt", 2.0 * R * s.D * s.F, self._gb("gmm", s.D, s.F, in_b=1)):
            B.moe_gmm_fp8(dq, "e5m2", sd[2], wor, "e4m3", swo[2], gs, valid_rows=self.vrows, out=self.d_act, err=self.err,
                          stream=stream)
        _, aqt, sa = q["act"]
        with self._rec("tgmm", 2.0 * R * s.D * s.F, self._gb("tgmm", s.F, s.D, in_b=1)):
            B.moe_tgmm_fp8(aqt, "e4m3", sa[2], dqt, "e5m2", sd[2], gs, self.rows, out=self.d_wo,
                           valid_rows=cnt, err=self.err, stream=stream)
        with self._rec("swiglu_bwd", nbytes=self._bytes().get("swiglu_bwd", 0) if self.recorder else 0):
            B.moe_swiglu_bwd(self.h0, self.h1, self.d_act, d_h0=self.d_h0, d_h1=self.d_h1,
                             stream=stream)
        _, xqt, sx = q["x"]
        for i, (gname, wname, dh, dw) in enumerate((("d_h0", "wi_0", self.d_h0, self.d_wi_0),
                                                    ("d_h1", "wi_1", self.d_h1, self.d_wi_1))):
            self._quant(gname, dh, "e5m2", stream)
            hq, hqt, sh = q[gname]
            wr, _, sw = q[wname]
            with self._rec("gmm_nt", 2.0 * R * s.D * s.F,
                           self._gb("gmm", s.F, s.D, in_b=1, rd_out=i > 0)):
                B.moe_gmm_fp8(hq, "e5m2", sh[2], wr, "e4m3", sw[2], gs, valid_rows=self.vrows, out=self.d_x_sorted,
                              accumulate=i > 0, err=self.err, stream=stream)
            with self._rec("tgmm", 2.0 * R * s.D * s.F, self._gb("tgmm", s.D, s.F, in_b=1)):
                B.moe_tgmm_fp8(xqt, "e4m3", sx[2], hqt, "e5m2", sh[2], gs, self.rows, out=dw,
                               valid_rows=cnt, err=self.err, stream=stream)

    def _rec(self, kind: str, flops: float = 0.0, nbytes: float = 0.0):
        if self.recorder is None:
            return contextlib.nullcontext()
        return self.recorder(kind, flops, nbytes)

    @property
    def group_sizes(self):
        return self.idx["group_sizes"]

    # Rows past each group's kept rows (align / capacity padding) are zero in
    # x_sorted, d_y_sorted and d_h, so the GEMMs reading them as lhs skip
    # them; act has zero padding rows only without MLP biases.
    @property
    def vrows(self):
        return self.idx["counts"]

    @property
    def vact(self):
        return None if self.s.mlp_bias else self.idx["counts"]

    # Counts of the routed data, set by a caller that has read them back from
    # the device (kept routed rows, rows of the groups including align
    # padding, non-empty groups); they only label recorded launches with
    # their algorithmic flops and bytes.  Defaults: no dropping, no padding,
    # every group non-empty.
    kept_rows_override: Optional[int] = None
    padded_rows_override: Optional[int] = None
    nonempty_groups_override: Optional[int] = None

    @property
    def kept_rows(self) -> int:
        if self.kept_rows_override is not None:
            return self.kept_rows_override
        return self.s.T * self.s.K

    @property
    def padded_rows(self) -> int:
        return self.rows if self.padded_rows_override is None else self.padded_rows_override

    @property
    def nonempty_groups(self) -> int:
        return self.s.E if self.nonempty_groups_override is None else self.nonempty_groups_override

    @property
    def _eb(self) -> int:
        return torch.finfo(self.s.dtype).bits // 8

    def _gb(self, kind: str, K: int, N: int, out_b: Optional[int] = None, in_b: Optional[int] = None,
            rd_out: bool = False, extra: int = 0) -> float:
        """Algorithmic HBM bytes of one grouped-GEMM launch (0 unless
        recording): each operand read once and the output written once.
          gmm:  the kept lhs rows (padding rows are not read), the weights of
                the non-empty groups, and every row of the groups written
                (read too when accumulating);
          tgmm: the kept rows of both operands and every group's [K, N]
                block (empty groups are written as zero)."""
        if self.recorder is None:
            return 0.0
        b = self._eb if in_b is None else in_b
        ob = self._eb if out_b is None else out_b
        R, Rp = self.kept_rows, self.padded_rows
        if kind == "gmm":
            n = R * K * b + self.nonempty_groups * K * N * b + Rp * N * ob * (2 if rd_out else 1)
        else:
            n = R * (K + N) * b + self.s.E * K * N * ob
        return float(n + extra)

    def _bytes(self) -> dict:
        """Algorithmic HBM bytes of the memory-bound calls (each tensor read or
        written once; ids and maps at 4 bytes per entry)."""
        s = self.s
        b = torch.finfo(s.dtype).bits // 8
        bh = 4 if s.n_chunks > 1 else b
        R, Rp, T, D, F, K = self.kept_rows, self.padded_rows, s.T, s.D, s.F, s.K
        return dict(
            permute=T * D * b + self.lhs_rows * D * b + T * K * 4 * 2 + self.lhs_rows * 4,
            swiglu=2 * Rp * F * bh + Rp * F * b,
            combine=R * D * b + T * D * b + T * K * 8,
            combine_bwd=T * D * b + R * D * b + self.rows * D * b + T * K * 12 + self.rows * 4,
            swiglu_bwd=2 * Rp * F * bh + 3 * Rp * F * b,
            permute_bwd=R * D * b + T * D * b + T * K * 4)

    def forward(self, x, wi_0, wi_1, wo, Wg=None, logits=None, bias=None, stream=None, wi=None,
                mlp_bias=None):
        """y = sum_j w[t,j] FFN_{e(t,j)}(x[t]).  Either Wg (router GEMM on the
        device) or precomputed float32 logits.  With fused_wi the
        up-projection weight is wi [E, D, 2F] (wi_0, wi_1 unused).  With
        mlp_bias set in the shape, mlp_bias is a dict of the per-expert biases
        "wi_0", "wi_1" [E, F] ("wi" [E, 2F] with fused_wi) and "wo" [E, D]."""
        s = self.s
        mb = mlp_bias if s.mlp_bias else {}
        if s.mlp_bias and (not mb or mb.get("wo") is None):
            raise B.MoeError("the shape has MLP biases: pass mlp_bias")
        if logits is None:
            B.moe_gmm(x, Wg.unsqueeze(0), self.gs_T, out=self.logits, err=self.err, stream=stream)
        else:
            self.logits.copy_(logits)
        B.moe_route(self.logits, s.K, s.score, s.renorm, bias, topk_ids=self.ids, topk_w=self.w,
                    stream=stream, bias_mode=s.bias_mode, n_groups=s.n_groups,
                    topk_groups=s.topk_groups)
        if s.aux_alpha > 0:
            B.moe_aux_loss(self.logits, self.ids, s.aux_alpha, s.score, loss=self.aux_loss,
                           counts=self.aux_counts, probs=self.aux_probs, workspace=self.aux_ws,
                           stream=stream)
        nb = self._bytes() if self.recorder is not None else {}
        with self._rec("permute", nbytes=nb.get("permute", 0)):
            B.moe_permute(x, self.ids, s.E, s.align, s.capacity, s.capacity_layout,
                          rows=self.lhs_rows, x_sorted=self.x_sorted, err=self.err,
                          workspace=self.ws, out=self.idx, stream=stream)
        gs = self.group_sizes
        R = self.kept_rows
        if s.fp8:
            self._forward_fp8(wi_0, wi_1, wo, mb, stream)
            with self._rec("combine", nbytes=nb.get("combine", 0)):
                B.moe_combine(self.y_sorted, self.idx["row_of_slot"], self.w, y=self.y,
                              stream=stream)
            return self.y
        if s.fused_wi:
            self._up_fused(wi, gs, R, stream, mb.get("wi"))
        elif s.n_chunks > 1:
            c = s.D // s.n_chunks
            for i in range(s.n_chunks):
                xs = self.x_sorted[:, i * c:(i + 1) * c]
                last = i == s.n_chunks - 1   # the biases enter once, with the last chunk
                with self._rec("gmm_up_chunk", 2.0 * R * c * s.F,
                               self._gb("gmm", c, s.F, out_b=4, rd_out=i > 0)):
                    B.moe_gmm(xs, wi_0[:, i * c:(i + 1) * c, :], gs, valid_rows=self.vrows, out=self.h0,
                              accumulate=i > 0, err=self.err, stream=stream,
                              bias=mb.get("wi_0") if last else None)
                with self._rec("gmm_up_chunk", 2.0 * R * c * s.F,
                               self._gb("gmm", c, s.F, out_b=4, rd_out=i > 0)):
                    B.moe_gmm(xs, wi_1[:, i * c:(i + 1) * c, :], gs, valid_rows=self.vrows, out=self.h1,
                              accumulate=i > 0, err=self.err, stream=stream,
                              bias=mb.get("wi_1") if last else None)
        else:
            with self._rec("gmm_nn", 2.0 * R * s.D * s.F, self._gb("gmm", s.D, s.F)):
                B.moe_gmm(self.x_sorted, wi_0, gs, valid_rows=self.vrows, out=self.h0, err=self.err, stream=stream,
                          bias=mb.get("wi_0"))
            with self._rec("gmm_nn", 2.0 * R * s.D * s.F, self._gb("gmm", s.D, s.F)):
                B.moe_gmm(self.x_sorted, wi_1, gs, valid_rows=self.vrows, out=self.h1, err=self.err, stream=stream,
                          bias=mb.get("wi_1"))
        if not self.swiglu_epilogue:   # else the up-projection's epilogue wrote act
            with self._rec("swiglu", nbytes=nb.get("swiglu", 0)):
                B.moe_swiglu(self.h0, self.h1, act=self.act, stream=stream)
        with self._rec("gmm_nn", 2.0 * R * s.D * s.F, self._gb("gmm", s.F, s.D)):
            B.moe_gmm(self.act, wo, gs, valid_rows=self.vact, out=self.y_sorted, err=self.err, stream=stream,
                      bias=mb.get("wo"))
        with self._rec("combine", nbytes=nb.get("combine", 0)):
            B.moe_combine(self.y_sorted, self.idx["row_of_slot"], self.w, y=self.y,
                          stream=stream)
        return self.y

    @property
    def swiglu_bwd_epilogue(self) -> bool:
        """The d_act GEMM applies the SwiGLU backward in its epilogue (bf16,
        h kept in bf16, i.e. no float32 partials of a chunked up-projection,
        d_ff above 128, d_model above one contraction step)."""
        s = self.s
        return (s.dtype == torch.bfloat16 and s.n_chunks == 1 and s.F > 128 and s.D > 32
                and s.F % 8 == 0)

    @property
    def swiglu_epilogue(self) -> bool:
        """The fused up-projection computes act in its epilogue (one launch,
        bf16, d_ff a multiple of 128, no contraction chunks), when groups
        average 512 rows or more: there the library's 256-row tiles hide the
        epilogue behind long contractions.  With smaller groups (128-row
        tiles, a weight-streaming launch) the epilogue is exposed and the
        plain product plus the SwiGLU pass is faster (DeepSeek-V3 shape:
        4.39 ms against 3.89 + 0.15 ms)."""
        s = self.s
        return (s.fused_wi and s.n_chunks == 1 and s.dtype == torch.bfloat16 and s.F % 128 == 0
                and s.T * s.K >= 512 * s.E)

    def _up_fused(self, wi, gs, R, stream, b_wi=None):
        s = self.s
        if s.n_chunks > 1:
            c = s.D // s.n_chunks
            for i in range(s.n_chunks):
                with self._rec("gmm_up_chunk", 4.0 * R * c * s.F,
                               self._gb("gmm", c, 2 * s.F, out_b=4, rd_out=i > 0)):
                    B.moe_gmm(self.x_sorted[:, i * c:(i + 1) * c], wi[:, i * c:(i + 1) * c, :],
                              gs, valid_rows=self.vrows, out=self.h, accumulate=i > 0, err=self.err, stream=stream,
                              bias=b_wi if i == s.n_chunks - 1 else None)
        elif self.swiglu_epilogue:
            # one launch: h (kept for the backward) and act = SwiGLU(h) from its epilogue
            with self._rec("gmm_nn", 4.0 * R * s.D * s.F,
                           self._gb("gmm", s.D, 2 * s.F, extra=self.padded_rows * s.F * self._eb)):
                B.moe_gmm_swiglu(self.x_sorted, wi, gs, act=self.act, h=self.h, valid_rows=self.vrows,
                                 bias=b_wi, err=self.err, stream=stream)
        else:
            with self._rec("gmm_nn", 4.0 * R * s.D * s.F, self._gb("gmm", s.D, 2 * s.F)):
                B.moe_gmm(self.x_sorted, wi, gs, valid_rows=self.vrows, out=self.h, err=self.err, stream=stream,
                          bias=b_wi)

    def backward(self, dy, x, wi_0, wi_1, wo, Wg=None, bias=None, stream=None, wi=None):
        """Gradients for upstream dy: fills dx, d_wi_0, d_wi_1 (halves of d_wi
        with fused_wi), d_wo, d_logits, (with the router) d_Wg and (with MLP
        biases) d_b_wi_0, d_b_wi_1 (halves of d_b_wi with fused_wi), d_b_wo."""
        s = self.s
        ros, sor = self.idx["row_of_slot"], self.idx["slot_of_row"]
        nb = self._bytes() if self.recorder is not None else {}
        with self._rec("combine_bwd", nbytes=nb.get("combine_bwd", 0)):
            B.moe_combine_bwd(dy, self.y_sorted, ros, sor, self.w, d_y_sorted=self.d_y_sorted,
                              d_topk_w=self.d_w, stream=stream)
        xs = self.x_sorted[:self.rows]
        if s.fp8:
            self._backward_fp8(stream)
        else:
            self._backward_gemms(wi_0, wi_1, wo, wi, xs, stream)
        self._backward_tail(dy, x, Wg, bias, stream)
        return self.dx

    def _backward_gemms(self, wi_0, wi_1, wo, wi, xs, stream):
        s = self.s
        gs = self.group_sizes
        R = self.kept_rows
        nb = self._bytes() if self.recorder is not None else {}
        if self.swiglu_bwd_epilogue:
            # d_act stays in registers: its GEMM's epilogue applies the SwiGLU
            # backward with h0, h1 and writes d_h0, d_h1
            with self._rec("gmm_nt_swiglu_bwd", 2.0 * R * s.D * s.F,
                           self._gb("gmm", s.D, s.F, extra=3 * self.padded_rows * s.F * self._eb)):
                B.moe_gmm_swiglu_bwd(self.d_y_sorted, wo, gs, self.h0, self.h1, d_h0=self.d_h0,
                                     d_h1=self.d_h1, valid_rows=self.vrows, err=self.err,
                                     stream=stream)
        else:
            with self._rec("gmm_nt", 2.0 * R * s.D * s.F, self._gb("gmm", s.D, s.F)):
                B.moe_gmm(self.d_y_sorted, wo, gs, valid_rows=self.vrows, trans_rhs=True, out=self.d_act, err=self.err,
                          stream=stream)
        with self._rec("tgmm", 2.0 * R * s.D * s.F, self._gb("tgmm", s.F, s.D)):
            # padding rows of each group (past its kept rows) are zero in
            # d_y_sorted and x_sorted: the weight gradients stop at counts
            B.moe_tgmm(self.act, self.d_y_sorted, gs, out=self.d_wo, err=self.err, stream=stream,
                       valid_rows=self.idx["counts"])
        if not self.swiglu_bwd_epilogue:
            with self._rec("swiglu_bwd", nbytes=nb.get("swiglu_bwd", 0)):
                B.moe_swiglu_bwd(self.h0, self.h1, self.d_act, d_h0=self.d_h0, d_h1=self.d_h1,
                                 stream=stream)
        if s.fused_wi:
            # the gate and up halves of the fused weight (and of d_h, d_wi) as
            # strided views through the launches of two weights: one
            # contraction over 2F and one 2F-wide tgmm measured slower than
            # two F-wide calls each on the Mixtral-8x7B shape
            wi_0, wi_1 = wi[:, :, :s.F], wi[:, :, s.F:]
        with self._rec("gmm_nt", 2.0 * R * s.D * s.F, self._gb("gmm", s.F, s.D)):
            B.moe_gmm(self.d_h0, wi_0, gs, valid_rows=self.vrows, trans_rhs=True, out=self.d_x_sorted, err=self.err,
                      stream=stream)
        with self._rec("gmm_nt", 2.0 * R * s.D * s.F, self._gb("gmm", s.F, s.D, rd_out=True)):
            B.moe_gmm(self.d_h1, wi_1, gs, valid_rows=self.vrows, trans_rhs=True, out=self.d_x_sorted,
                      accumulate=True, err=self.err, stream=stream)
        with self._rec("tgmm", 2.0 * R * s.D * s.F, self._gb("tgmm", s.D, s.F)):
            B.moe_tgmm(xs, self.d_h0, gs, out=self.d_wi_0, err=self.err, stream=stream,
                       valid_rows=self.idx["counts"])
        with self._rec("tgmm", 2.0 * R * s.D * s.F, self._gb("tgmm", s.D, s.F)):
            B.moe_tgmm(xs, self.d_h1, gs, out=self.d_wi_1, err=self.err, stream=stream,
                       valid_rows=self.idx["counts"])

    def _backward_tail(self, dy, x, Wg, bias, stream):
        s = self.s
        gs = self.group_sizes
        ros = self.idx["row_of_slot"]
        nb = self._bytes() if self.recorder is not None else {}
        if s.mlp_bias:
            # bias gradients: per-group sums of the rows of the gradient of
            # the output each bias was added to (padding rows are zero)
            cnt = self.idx["counts"]
            with self._rec("group_sum"):
                B.moe_group_sum(self.d_y_sorted, gs, out=self.d_b_wo, valid_rows=cnt,
                                workspace=self.gsum_ws, err=self.err, stream=stream)
            if s.fused_wi:
                with self._rec("group_sum"):
                    B.moe_group_sum(self.d_h, gs, out=self.d_b_wi, valid_rows=cnt,
                                    workspace=self.gsum_ws, err=self.err, stream=stream)
            else:
                for dh, db in ((self.d_h0, self.d_b_wi_0), (self.d_h1, self.d_b_wi_1)):
                    with self._rec("group_sum"):
                        B.moe_group_sum(dh, gs, out=db, valid_rows=cnt, workspace=self.gsum_ws,
                                        err=self.err, stream=stream)
        with self._rec("permute_bwd", nbytes=nb.get("permute_bwd", 0)):
            B.moe_permute_bwd(self.d_x_sorted, ros, s.T, s.K, d_x=self.dx, stream=stream)
        B.moe_route_bwd(self.logits, self.ids, self.d_w, s.score, s.renorm, bias,
                        d_logits=self.d_logits, stream=stream, bias_mode=s.bias_mode)
        if s.aux_alpha > 0:
            # the balancing loss enters the objective with weight one
            B.moe_aux_loss_bwd(self.logits, self.aux_counts, s.K, s.aux_alpha, s.score,
                               d_logits=self.d_logits, accumulate=True, stream=stream)
        if Wg is not None and self.router:
            if s.dtype == torch.bfloat16:
                B.moe_router_bwd(x, Wg, self.d_logits, d_Wg=self.d_Wg[0], dx=self.dx,
                                 accumulate_dx=True, workspace=self.router_ws, err=self.err,
                                 stream=stream)
            else:
                # float32 workloads: the float32 GEMM kernels take d_logits as is
                B.moe_tgmm(x, self.d_logits, self.gs_T, out=self.d_Wg, err=self.err,
                           stream=stream)
                B.moe_gmm(self.d_logits, Wg.unsqueeze(0), self.gs_T, trans_rhs=True,
                          out=self.dx, accumulate=True, err=self.err, stream=stream)
        return self.dx

    def expert_flops(self, kept_rows: Optional[int] = None) -> float:
        """Algorithmic expert-FFN flops of one forward+backward: 18 R D F with
        R the kept routed rows (padding rows excluded)."""
        s = self.s
        R = s.T * s.K if kept_rows is None else kept_rows
        return 18.0 * R * s.D * s.F
