"""FP8 entry points against the oracle: the current-scaling amax and scales
and the quantized codes bit for bit (both sides decide every code on the
same float32 product), and the FP8 grouped GEMMs on given codes against
float64 sums of the dequantized operands."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, dev_i32, host, poison

pytestmark = pytest.mark.gpu

F8 = oracle.fp8
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _draw(g, shape, dt, spread=3.0):
    """Normal values with a wide dynamic range (several binades)."""
    a = (g.standard_normal(shape) * np.exp(g.uniform(-spread, spread, shape))).astype(np.float32)
    return ms.bf16_round(a) if dt == "bf16" else a


def _codes(g, shape, fmt):
    """Finite FP8 codes of normal values spread over the format's range."""
    return F8.encode(g.standard_normal(shape) * (40.0 if fmt == "e4m3" else 2000.0), fmt)


def _padded_t(codes, gs, P):
    """[cols, P] transposed copy: group g's rows at 64 * (64-row tiles of
    the groups before it), zeros elsewhere (the documented layout)."""
    rows, cols = codes.shape
    out = np.zeros((cols, P), dtype=np.uint8)
    src, dst = 0, 0
    for n in gs:
        out[:, dst:dst + n] = codes[src:src + n].T
        src += n
        dst += 64 * ((n + 63) // 64)
    return out


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("G", [1, 8, 37])
def test_fp8_amax_scale(gpu_lib, dt, fmt, G):
    g = np.random.default_rng(G * 10 + len(fmt))
    rows, cols = 64 * G, 136
    x = _draw(g, (rows, cols), dt)
    if G > 1:
        x[:64] = 0                                    # a unit of zeros: scale 1
    sc = host(gpu_lib.moe_fp8_amax_scale(dev(x, TD[dt]), fmt, G=G))
    am = F8.amax_groups(x, rows // G)
    s, si = F8.scales(am, fmt)
    assert (sc[0] == am).all() and (sc[1] == s).all() and (sc[2] == si).all()


QUANT_CASES = [
    # group sizes, cols, dtype, format
    ([300, 0, 257, 1, 64, 0, 129], 136, "bf16", "e4m3"),
    ([300, 0, 257, 1, 64, 0, 129], 72, "f32", "e5m2"),
    ([0, 0, 128, 256], 264, "bf16", "e5m2"),
    ([517], 8, "bf16", "e4m3"),
    ([(i * 7) % 5 for i in range(300)], 40, "bf16", "e4m3"),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[f"G{len(c[0])}-{c[1]}-{c[2]}-{c[3]}" for c in QUANT_CASES])
def test_fp8_quantize(gpu_lib, case):
    gs, cols, dt, fmt = case
    gs = np.array(gs, dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(cols + G)
    rows = int(gs.sum()) + 5                          # rows past the groups are not touched
    x = _draw(g, (rows, cols), dt)
    xd = dev(x, TD[dt])
    sc = gpu_lib.moe_fp8_amax_scale(xd, fmt)
    P = gpu_lib.moe_fp8_padded_rows(rows, G)
    q = torch.full((rows, cols), 0xAA, dtype=torch.uint8, device="cuda")
    qt = torch.full((cols, P + 16), 0xAA, dtype=torch.uint8, device="cuda")
    gpu_lib.moe_fp8_quantize(xd, dev_i32(gs), sc[1], fmt, q=q, qt=qt)
    s, _ = F8.scales(F8.amax_groups(x), fmt)
    want = F8.quantize(x, fmt, s[0])
    S = int(gs.sum())
    got_q = host(q)
    assert (got_q[:S] == want[:S]).all()
    assert (got_q[S:] == 0xAA).all()
    got_t = host(qt)
    used = 64 * int(((gs + 63) // 64).sum())          # columns the groups own (zero-padded)
    assert (got_t[:, :used] == _padded_t(want[:S], gs, P)[:, :used]).all()
    assert (got_t[:, used:] == 0xAA).all()


def test_fp8_quantize_many_tiles(gpu_lib):
    """More 128 x 128 tiles than the quantizer's grid holds workgroups, so
    each workgroup takes several tiles (ragged groups and columns)."""
    gs = np.array([2500, 0, 1, 4095, 3000, 129, 5000, 64, 5211], dtype=np.int32)
    G, cols = len(gs), 2176
    g = np.random.default_rng(11)
    rows = int(gs.sum())
    x = _draw(g, (rows, cols), "bf16", spread=2.0)
    xd = dev(x, torch.bfloat16)
    sc = gpu_lib.moe_fp8_amax_scale(xd, "e4m3")
    P = gpu_lib.moe_fp8_padded_rows(rows, G)
    tiles = (P // 64 + 1) // 2 * ((cols + 127) // 128)
    assert tiles > 8 * torch.cuda.get_device_properties(0).multi_processor_count
    q = torch.full((rows, cols), 0xAA, dtype=torch.uint8, device="cuda")
    qt = torch.full((cols, P), 0xAA, dtype=torch.uint8, device="cuda")
    gpu_lib.moe_fp8_quantize(xd, dev_i32(gs), sc[1], "e4m3", q=q, qt=qt)
    s, _ = F8.scales(F8.amax_groups(x), "e4m3")
    want = F8.quantize(x, "e4m3", s[0])
    assert (host(q) == want).all()
    used = 64 * int(((gs + 63) // 64).sum())
    assert (host(qt)[:, :used] == _padded_t(want, gs, P)[:, :used]).all()


def _all_bf16():
    """Every finite bf16 value below 1e30 in magnitude (as float32; the
    float32 products with the test scales stay finite)."""
    v = ms.bf16_from_bits(np.arange(1 << 16, dtype=np.uint16))
    return v[np.isfinite(v) & (np.abs(v) < 1e30)]


def _f32_sweep(fmt):
    """float32 values around every FP8 code: the codes, the midpoints between
    neighbours (ties), one float32 ulp either side of them, and random bit
    patterns over the format's exponent range and beyond."""
    codes = np.arange(256, dtype=np.uint8)
    d = F8.decode(codes, fmt)
    d = np.sort(d[np.isfinite(d) & (d >= 0)])
    mids = (d[1:] + d[:-1]) / 2
    base = np.concatenate([d, mids]).astype(np.float32)
    near = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                           np.nextafter(base, np.float32(-np.inf))])
    g = np.random.default_rng(99)
    e = g.integers(-40 if fmt == "e4m3" else -50, 30 if fmt == "e5m2" else 20, 200000)
    rnd = (g.uniform(1, 2, e.size) * np.exp2(e.astype(np.float64))).astype(np.float32)
    v = np.concatenate([near, rnd, [0.0, 1e-45, 1e30]]).astype(np.float32)
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("src", ["bf16-all", "f32-sweep"])
def test_fp8_quantize_codes_exhaustive(gpu_lib, fmt, src):
    """The quantizer's codes equal the oracle's (round to nearest even of the
    float32 product, saturating, sign kept) for every finite bf16 input and
    for float32 inputs at, between and next to every FP8 value, under scales
    that keep, round and saturate them."""
    v = _all_bf16() if src == "bf16-all" else _f32_sweep(fmt)
    dt = "bf16" if src == "bf16-all" else "f32"
    cols = 128
    rows = (v.size + cols - 1) // cols
    x = np.zeros(rows * cols, dtype=np.float32)
    x[:v.size] = v
    x = x.reshape(rows, cols)
    gs = np.array([rows], dtype=np.int32)
    for scale in (1.0, 0.8125, 3.0 if fmt == "e4m3" else 1000.0):
        q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
        gpu_lib.moe_fp8_quantize(dev(x, TD[dt]), dev_i32(gs),
                                 torch.tensor([scale], dtype=torch.float32, device="cuda"), fmt, q=q)
        want = F8.quantize(x, fmt, np.float32(scale))
        got = host(q)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (scale, x.ravel()[bad[:5]], got.ravel()[bad[:5]], want.ravel()[bad[:5]])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_quantize_weights(gpu_lib, fmt):
    """Per-expert scaling of a weight stack [E, a, b]: row-wise copy and the
    per-expert transposed copy [E, b, a]; saturation past fmax."""
    g = np.random.default_rng(3)
    E, A, Bc = 5, 160, 136
    w = _draw(g, (E, A, Bc), "bf16")
    wd = dev(w.reshape(E * A, Bc), torch.bfloat16)
    sc = gpu_lib.moe_fp8_amax_scale(wd, fmt, G=E)
    gsz = dev_i32(np.full(E, A, dtype=np.int32))
    q = torch.empty((E * A, Bc), dtype=torch.uint8, device="cuda")
    qt = torch.empty((E, Bc, A), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_fp8_quantize(wd, gsz, sc[1], fmt, per_group=True, q=q, qt=qt,
                             qt_group_stride=Bc * A, ld_qt=A)
    codes, si, _ = F8.quantize_experts(w, fmt)
    assert (host(sc[2]) == si).all()
    assert (host(q).reshape(E, A, Bc) == codes).all()
    assert (host(qt) == codes.transpose(0, 2, 1)).all()
    # a scale twice the amax scale: the largest magnitudes saturate
    s2 = sc[1] * 2
    gpu_lib.moe_fp8_quantize(wd, gsz, s2, fmt, per_group=True, q=q)
    want = F8.quantize(w, fmt, host(s2))
    assert (host(q).reshape(E, A, Bc) == want).all()
    assert (np.abs(F8.decode(want, fmt)) == F8.fmax(fmt)).any()


GMM8_CASES = [
    # group sizes, K, N, lhs fmt, rhs fmt, out, accumulate, bias
    ([130, 0, 257, 1, 64, 0, 300], 192, 136, "e4m3", "e4m3", "bf16", False, False),
    ([130, 0, 257, 1, 64, 0, 300], 160, 264, "e5m2", "e4m3", "f32", True, False),   # ragged K
    ([0, 0, 128, 256], 1024, 256, "e4m3", "e4m3", "bf16", False, True),
    ([517], 64, 8, "e4m3", "e5m2", "f32", False, False),
    ([800, 0, 900], 512, 520, "e5m2", "e5m2", "bf16", True, True),
    ([(i * 7) % 3 for i in range(1000)], 64, 136, "e4m3", "e4m3", "f32", False, False),
    ([0, 0, 0], 64, 64, "e4m3", "e4m3", "f32", False, False),
    # 256-row tiles (groups of 512 rows or more on average): an odd number
    # of full contraction steps and a ragged one, and a ragged step alone
    ([700, 600], 224, 264, "e4m3", "e4m3", "bf16", True, False),
    ([600, 520], 32, 136, "e5m2", "e4m3", "f32", False, True),
]


def _kn(qb, fill=0x7F):
    """[G, N, K] codes as a [G, K, N] view whose rows are padded to a multiple
    of 16 bytes with NaN codes (0x7F: NaN in e4m3, a NaN in e5m2 too), which
    only products in columns past N may see."""
    G, N, K = qb.shape
    npad = 16 * ((N + 15) // 16)
    buf = np.full((G, K, npad), fill, dtype=np.uint8)
    buf[:, :, :N] = qb.transpose(0, 2, 1)
    return _u8(buf)[:, :, :N]


@pytest.mark.parametrize("trans", [True, False], ids=["nk", "kn"])
@pytest.mark.parametrize("case", GMM8_CASES, ids=[f"G{len(c[0])}-{c[1]}x{c[2]}-{c[3]}{c[4]}-{c[5]}-a{int(c[6])}-b{int(c[7])}" for c in GMM8_CASES])
def test_gmm_fp8(gpu_lib, case, trans):
    """Both weight orientations: B_g^T stored [N, K] (trans_rhs) or B_g stored
    [K, N] and read through transposing LDS reads."""
    gs, K, N, fa, fb, ot, acc, with_bias = case
    gs = np.array(gs, dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(K + N + G)
    M = int(gs.sum()) + 3
    qa = _codes(g, (M, K), fa)
    qb = _codes(g, (G, N, K), fb)
    sa = np.float32([0.037])
    sb = (np.float32(0.5) ** g.integers(0, 9, G) * np.float32(1.3)).astype(np.float32)
    P = (g.standard_normal((M, N)).astype(np.float32) if acc else None)
    if P is not None and ot == "bf16":
        P = ms.bf16_round(P)
    bias = ms.bf16_round(g.standard_normal((G, N)).astype(np.float32)) if with_bias else None
    out = dev(P, TD[ot]) if acc else poison(torch.empty((M, N), dtype=TD[ot], device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.moe_gmm_fp8(_u8(qa), fa, dev(sa), _u8(qb) if trans else _kn(qb), fb, dev(sb),
                        dev_i32(gs), out=out, accumulate=acc, err=err, trans_rhs=trans,
                        bias=None if bias is None else dev(bias, torch.bfloat16))
    A = F8.dequantize(qa, fa, sa[0])
    B = F8.dequantize(qb, fb, sb)
    want = oracle.gmm(A, B, gs, trans_rhs=True, partial=P, bias=bias)
    got = host(out)
    assert_close(got, want, TOL_F32 if ot == "f32" else TOL_BF16, "gmm_fp8")
    S = int(gs.sum())
    assert (got[S:] == (P[S:] if acc else 0)).all()
    assert host(err)[0] == 0


FP8_VALID = {
    "small": ([300, 0, 257, 128], [299, 0, 1, 0]),
    "big": ([1024, 1024], [1000, 3]),
    # valid rows ending at and around the waves' 32-row fragment boundaries
    "frag": ([128] * 10 + [384], [1, 31, 32, 33, 63, 64, 65, 96, 97, 128, 300]),
}


@pytest.mark.parametrize("trans", [True, False], ids=["nk", "kn"])
@pytest.mark.parametrize("case", list(FP8_VALID))
def test_gmm_fp8_valid_rows(gpu_lib, case, trans):
    """FP8 gmm skips lhs rows past valid_rows (garbage codes here)."""
    gs = np.array(FP8_VALID[case][0], dtype=np.int32)
    valid = np.array(FP8_VALID[case][1], dtype=np.int32)
    big = case == "big"
    G, M, K, N = len(gs), int(gs.sum()), 256, 264
    g = np.random.default_rng(4 + big)
    qa = _codes(g, (M, K), "e4m3")
    qb = _codes(g, (G, N, K), "e4m3")
    qa0 = qa.copy()
    off = np.concatenate([[0], np.cumsum(gs)])
    for e in range(G):
        qa0[off[e] + valid[e]:off[e + 1]] = 0
    sa, sb = np.float32([0.03]), np.full(G, 0.5, np.float32)
    out = gpu_lib.moe_gmm_fp8(_u8(qa), "e4m3", dev(sa), _u8(qb) if trans else _kn(qb), "e4m3",
                              dev(sb), dev_i32(gs), out_dtype=torch.float32,
                              valid_rows=dev_i32(valid), trans_rhs=trans)
    want = oracle.gmm(F8.dequantize(qa0, "e4m3", sa[0]), F8.dequantize(qb, "e4m3", sb), gs,
                      trans_rhs=True)
    assert_close(host(out), want, TOL_F32, "gmm_fp8 valid_rows")


TGMM8_CASES = [
    # group sizes, valid rows, Kd, N, formats, out, accumulate
    ([130, 0, 257, 1, 64, 0, 300], None, 136, 264, "e4m3", "e5m2", "f32", False),
    ([130, 0, 257, 1, 64, 0, 300], [100, 0, 257, 0, 64, 0, 1], 264, 136, "e4m3", "e5m2", "bf16", True),
    ([1000, 24], None, 128, 256, "e4m3", "e4m3", "f32", False),
    ([0, 0, 0], None, 64, 64, "e4m3", "e5m2", "f32", True),
]


@pytest.mark.parametrize("case", TGMM8_CASES, ids=[f"G{len(c[0])}-{c[2]}x{c[3]}-v{int(c[1] is not None)}-{c[6]}-a{int(c[7])}" for c in TGMM8_CASES])
def test_tgmm_fp8(gpu_lib, case):
    gs, valid, Kd, N, fa, fb, ot, acc = case
    gs = np.array(gs, dtype=np.int32)
    G = len(gs)
    g = np.random.default_rng(Kd * 3 + N + G)
    M = int(gs.sum()) + 7
    qa = _codes(g, (M, Kd), fa)
    qb = _codes(g, (M, N), fb)
    off = np.concatenate([[0], np.cumsum(gs)])
    if valid is not None:
        valid = np.array(valid, dtype=np.int32)
        for e in range(G):
            qb[off[e] + valid[e]:off[e + 1]] = 0     # rows past valid_rows are zero
    P = gpu_lib.moe_fp8_padded_rows(M, G)
    at = _padded_t(qa[:off[-1]], gs, P)
    bt = _padded_t(qb[:off[-1]], gs, P)
    sa, sb = np.float32([0.25]), np.float32([0.0078125 * 3])
    part = g.standard_normal((G, Kd, N)).astype(np.float32) if acc else None
    if part is not None and ot == "bf16":
        part = ms.bf16_round(part)
    out = dev(part, TD[ot]) if acc else poison(torch.empty((G, Kd, N), dtype=TD[ot], device="cuda"))
    gpu_lib.moe_tgmm_fp8(_u8(at), fa, dev(sa), _u8(bt), fb, dev(sb), dev_i32(gs), M, out=out,
                         accumulate=acc, valid_rows=None if valid is None else dev_i32(valid))
    A = F8.dequantize(qa, fa, sa[0])
    B = F8.dequantize(qb, fb, sb[0])
    want = oracle.tgmm(A, B, gs, partial=part)
    got = host(out)
    assert_close(got, want, TOL_F32 if ot == "f32" else TOL_BF16, "tgmm_fp8")
    for e in np.where(gs == 0)[0]:
        assert (got[e] == (part[e] if acc else 0)).all()


def test_fp8_quantize_then_tgmm(gpu_lib):
    """The GPU's own transposed copies feed the FP8 tgmm: equal to the
    oracle's quantization and tgmm of the same bf16 inputs."""
    g = np.random.default_rng(9)
    gs = np.array([300, 0, 129, 64, 1], dtype=np.int32)
    G, M, Kd, N = len(gs), int(gs.sum()), 136, 264
    x = _draw(g, (M, Kd), "bf16", 1.0)
    d = _draw(g, (M, N), "bf16", 1.0)
    P = gpu_lib.moe_fp8_padded_rows(M, G)
    xd, dd, gsd = dev(x, torch.bfloat16), dev(d, torch.bfloat16), dev_i32(gs)
    sx = gpu_lib.moe_fp8_amax_scale(xd, "e4m3")
    sd = gpu_lib.moe_fp8_amax_scale(dd, "e5m2")
    xt = torch.empty((Kd, P), dtype=torch.uint8, device="cuda")
    dt_ = torch.empty((N, P), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_fp8_quantize(xd, gsd, sx[1], "e4m3", qt=xt)
    gpu_lib.moe_fp8_quantize(dd, gsd, sd[1], "e5m2", qt=dt_)
    out = gpu_lib.moe_tgmm_fp8(xt, "e4m3", sx[2], dt_, "e5m2", sd[2], gsd, M, out_dtype=torch.float32)
    _, _, xq = F8.quantize_tensor(x, "e4m3")
    _, _, dq = F8.quantize_tensor(d, "e5m2")
    assert_close(host(out), oracle.tgmm(xq, dq, gs), TOL_F32, "quantize + tgmm_fp8")
