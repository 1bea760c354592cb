"""The C ABI without a GPU: the library loads, exports every entry point
declared in include/moe.h with the binding's signature, and its host-side
logic (row bounds, workspace size, argument checks that return before any
launch) behaves as documented."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_grouped_top_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declarations():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = {}
    for m in re.finditer(r"^\s*([A-Za-z_][\w\s\*]*?)\b(moe_\w+)\s*\(([^;]*?)\)\s*;", src, flags=re.M | re.S):
        params = [p.strip() for p in m.group(3).split(",") if p.strip() and p.strip() != "void"]
        decls[m.group(2)] = params
    return decls


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m mixture_experts_grouped_top_amd.build)")
    return moe.load()


def test_header_declares_the_abi():
    d = _declarations()
    for name in ["moe_route", "moe_route_bwd", "moe_permute", "moe_permute_bwd", "moe_gmm",
                 "moe_tgmm", "moe_swiglu", "moe_swiglu_bwd", "moe_combine", "moe_combine_bwd",
                 "moe_rows_bound", "moe_permute_workspace", "moe_status_string",
                 "moe_abi_version", "moe_aux_loss_workspace", "moe_aux_loss",
                 "moe_aux_loss_bwd", "moe_group_sum_workspace", "moe_group_sum",
                 "moe_fp8_scale_workspace", "moe_fp8_amax_scale", "moe_fp8_padded_rows",
                 "moe_fp8_quantize", "moe_gmm_fp8", "moe_tgmm_fp8", "moe_gmm_swiglu",
                 "moe_gmm_swiglu_bwd", "moe_router_bwd", "moe_router_bwd_workspace",
                 "moe_permute_noalloc"]:
        assert name in d, name


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declarations():
        assert name in exported, f"{name} declared in moe.h but not exported"
        assert getattr(lib, name) is not None


def test_binding_signatures_match_header():
    d = _declarations()
    assert set(moe.SIGNATURES) == set(d)
    for name, (_, args) in moe.SIGNATURES.items():
        assert len(args) == len(d[name]), (name, len(args), len(d[name]))


def test_rows_bound_matches_oracle(lib):
    for (T, K, E, a, C, lay) in [(512, 2, 8, 0, 0, 0), (4096, 8, 256, 128, 0, 0),
                                 (8192, 1, 256, 0, 32, 1), (8192, 1, 256, 0, 32, 0),
                                 (333, 4, 16, 8, 0, 0), (0, 1, 1, 0, 0, 0)]:
        assert moe.moe_rows_bound(T, K, E, a, C, lay) == oracle.rows_bound(T, K, E, a, C, bool(lay))
    assert lib.moe_rows_bound(10, 0, 4, 0, 0, 0) == -1
    assert lib.moe_rows_bound(10, 1, 4, 0, 0, 1) == -1   # capacity layout needs C > 0


def test_workspace_and_status(lib):
    assert moe.moe_permute_workspace(4096, 8, 256) >= 32 * 256 * 4
    assert moe.moe_permute_workspace(4096, 8, 256) % 256 == 0
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.moe_status_string(code)
    assert lib.moe_abi_version() == moe.ABI_VERSION
    # group-sum partial rows: (ceil(M / 256) + G) * N float32
    assert moe.moe_group_sum_workspace(1000, 8, 64) == (4 + 8) * 64 * 4
    assert moe.moe_group_sum_workspace(0, 3, 16) == 3 * 16 * 4


def test_argument_checks_return_before_launch(lib):
    """Invalid arguments are rejected on the host (no device pointer is touched)."""
    P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    # K > E
    assert lib.moe_route(P, None, 0, 0, 0, 8, 4, 5, 0, 1, P, P, None) == -1
    # unknown score, unknown bias mode
    assert lib.moe_route(P, None, 0, 0, 0, 8, 4, 2, 7, 1, P, P, None) == -1
    assert lib.moe_route(P, None, 5, 0, 0, 8, 4, 2, 0, 1, P, P, None) == -1
    # groups: E not divisible, too few candidates, topk_groups out of range
    assert lib.moe_route(P, None, 0, 3, 1, 8, 16, 2, 0, 1, P, P, None) == -1
    assert lib.moe_route(P, None, 1, 8, 1, 8, 16, 3, 1, 1, P, P, None) == -1
    assert lib.moe_route(P, None, 1, 4, 5, 8, 16, 2, 1, 1, P, P, None) == -1
    # E too large
    assert lib.moe_route_bwd(P, None, 0, P, P, 8, 2048, 2, 0, 1, P, 0, None) == -1
    # aux loss: no tokens, missing workspace
    assert lib.moe_aux_loss(P, P, 0, 8, 2, 0, 0.1, P, None, None, P, 1 << 20, None) == -1
    assert lib.moe_aux_loss(P, P, 16, 8, 2, 0, 0.1, P, None, None, None, 0, None) == -5
    # bad d_logits dtype is caught after the size checks
    # gmm: G = 0, M_out > M_lhs, K not a multiple of 8, bad dtype, ld < K
    args = lambda **kw: dict(dict(lhs=P, M_lhs=64, ld=64, rhs=P, ldr=64, gst=64 * 64, tr=0, gs=P,
                                  G=2, Kd=64, N=64, it=1, out=P, M_out=64, ldo=64, ot=1, acc=0),
                             **kw)

    def gmm(**kw):
        a = args(**kw)
        return lib.moe_gmm(a["lhs"], a["M_lhs"], a["ld"], a["rhs"], a["ldr"], a["gst"], a["tr"],
                           a["gs"], None, a["G"], a["Kd"], a["N"], a["it"], a.get("bias"),
                           a["out"], a["M_out"], a["ldo"], a["ot"], a["acc"], None, None)
    assert gmm(G=0) == -1
    assert gmm(M_out=65) == -1
    assert gmm(Kd=60, ld=60) == -1
    assert gmm(it=5) == -2
    assert gmm(ot=9) == -2
    assert gmm(ld=32) == -1
    assert gmm(G=5000) == -1
    assert gmm(bias=ctypes.c_void_p(18)) == -1      # misaligned bias
    # gmm_swiglu: F not a multiple of 128, float32 inputs, weight row stride below 2F,
    # act row stride below F, misaligned act
    def swi(F=128, it=1, ldr=256, lda=128, act=P):
        return lib.moe_gmm_swiglu(P, 64, 64, P, ldr, 64 * ldr, P, None, 2, 64, F, it, None, None,
                                  0, act, lda, 64, None, None)
    assert swi(F=64, ldr=128, lda=64) == -1
    assert swi(it=0) == -2
    assert swi(ldr=248) == -1
    assert swi(lda=120) == -1
    assert swi(act=ctypes.c_void_p(24)) == -1
    # gmm_swiglu_bwd: narrow F, short contraction, float32, h row stride below F
    def swb(F=256, K=64, it=1, ldh=256):
        return lib.moe_gmm_swiglu_bwd(P, 64, 64, P, 64, 64 * F, P, None, 2, K, F, it, P, P, ldh,
                                      P, P, F, 64, None, None)
    assert swb(F=128, ldh=128) == -1
    assert swb(K=32) == -1
    assert swb(it=0) == -2
    assert swb(ldh=248) == -1
    # group sum: N not a multiple of 8, G too large, missing or short workspace, bad dtype
    W = ctypes.c_void_p(256)
    assert lib.moe_group_sum(P, 12, 1, P, None, 2, 10, 12, P, 0, 0, W, 1 << 20, None, None) == -1
    assert lib.moe_group_sum(P, 64, 1, P, None, 1025, 10, 64, P, 0, 0, W, 1 << 20, None, None) == -1
    assert lib.moe_group_sum(P, 64, 1, P, None, 2, 10, 64, P, 0, 0, None, 0, None, None) == -5
    assert lib.moe_group_sum(P, 64, 1, P, None, 2, 10, 64, P, 0, 0, W, 64, None, None) == -5
    assert lib.moe_group_sum(P, 64, 4, P, None, 2, 10, 64, P, 0, 0, W, 1 << 20, None, None) == -2
    # fp8: unknown format, rows not divisible by G, K not a multiple of 16, G > 1000,
    # transposed copy narrower than the padded layout
    assert lib.moe_fp8_amax_scale(P, 64, 1, 64, 64, 1, 7, P, W, 1 << 20, None) == -1
    assert lib.moe_fp8_amax_scale(P, 64, 1, 65, 64, 2, 0, P, W, 1 << 20, None) == -1
    assert lib.moe_fp8_amax_scale(P, 64, 1, 64, 64, 1, 0, P, None, 0, None) == -5
    assert lib.moe_gmm_fp8(P, 64, 64, 0, P, P, 40, 40 * 64, 1, 0, P, P, None, 2, 40, 64, None, P,
                           64, 64, 1, 0, None, None) == -1
    assert lib.moe_gmm_fp8(P, 64, 64, 0, P, P, 64, 64 * 64, 1, 0, P, P, None, 1001, 64, 64, None,
                           P, 64, 64, 1, 0, None, None) == -1
    # [K, N] weight (trans_rhs = 0): its row stride must cover N
    assert lib.moe_gmm_fp8(P, 64, 64, 0, P, P, 64, 64 * 96, 0, 0, P, P, None, 2, 64, 96, None, P,
                           64, 96, 1, 0, None, None) == -1
    assert lib.moe_fp8_padded_rows(100, 3) == 64 * (2 + 2)
    assert lib.moe_fp8_quantize(P, 64, 1, 100, 64, P, 3, P, 0, 0, None, 0, P, 128, 0, None,
                                None) == -1
    assert lib.moe_tgmm_fp8(P, 128, 0, P, P, 256, 1, P, P, None, 3, 100, 64, 64, P, 64, 64 * 64,
                            1, 0, None, None) == -1
    # tgmm: output group stride too small
    assert lib.moe_tgmm(P, 64, P, 64, P, None, 2, 10, 64, 64, 1, P, 64, 64, 1, 0, None, None) == -1
    # permute: rows below the static bound, missing workspace
    assert lib.moe_permute(P, 1, 16, 64, P, 2, 4, 0, 0, 0, P, 31, P, P, P, P, P, P, 1 << 20,
                           None, None) == -3
    assert lib.moe_permute(P, 1, 16, 64, P, 2, 4, 0, 0, 0, P, 32, P, P, P, P, P, None, 0,
                           None, None) == -5
    # router backward: D not a multiple of 8, E too large, bad dx dtype, short workspace
    W2 = ctypes.c_void_p(1 << 20)
    ws = moe.moe_router_bwd_workspace(64, 64, 8)
    assert ws >= 256 + 64 * 24 * 2 * 2
    assert lib.moe_router_bwd(P, P, P, 64, 60, 8, P, P, 1, 1, W2, ws, None, None) == -1
    assert lib.moe_router_bwd(P, P, P, 64, 64, 1025, P, P, 1, 1, W2, 1 << 30, None, None) == -1
    assert lib.moe_router_bwd(P, P, P, 64, 64, 8, P, P, 7, 1, W2, ws, None, None) == -2
    assert lib.moe_router_bwd(P, P, P, 64, 64, 8, P, P, 1, 1, W2, ws - 1, None, None) == -5
    assert lib.moe_router_bwd(P, P, P, 64, 64, 8, P, P, 1, 1, ctypes.c_void_p(16), ws, None,
                              None) == -5
    # permute without a workspace: past its static scratch (ceil(T K / 1024) E > 262144 words)
    assert lib.moe_permute_noalloc(P, 1, 131073, 64, P, 8, 256, 0, 0, 0, P, 131073 * 8, P, P, P,
                                   P, P, None, None) == -5
    assert lib.moe_permute_noalloc(P, 1, 16, 64, P, 2, 4, 0, 0, 0, P, 31, P, P, P, P, P, None,
                                   None) == -3
    # combine: D not a multiple of 8
    assert lib.moe_combine(P, 1, 4, 12, 2, 8, P, P, P, None) == -1
    assert lib.moe_swiglu(P, P, 3, 4, 8, 8, P, 1, None) == -2
    assert lib.moe_swiglu(P, P, 1, 4, 16, 8, P, 1, None) == -1      # row stride below F


def test_binding_rejects_bad_shapes_and_index_dtypes(lib):
    """The binding checks shapes and index vectors before any pointer is
    taken (CPU tensors: a check that passed would fail later on the device
    check, with another message)."""
    import torch
    bf = torch.bfloat16
    lhs = torch.zeros((64, 32), dtype=bf)
    rhs = torch.zeros((2, 32, 48), dtype=bf)
    gs = torch.tensor([30, 34], dtype=torch.int32)

    def raises(match, fn, *a, **kw):
        with pytest.raises(moe.MoeError, match=match):
            fn(*a, **kw)

    raises("group_sizes must be a contiguous int32", moe.moe_gmm, lhs, rhs, gs.long())
    raises("group_sizes must be a contiguous int32", moe.moe_gmm, lhs, rhs, gs[:1])
    raises("valid_rows must be a contiguous int32", moe.moe_gmm, lhs, rhs, gs,
           valid_rows=torch.tensor([1, 2, 3], dtype=torch.int32))
    raises("out must be", moe.moe_gmm, lhs, rhs, gs, out=torch.zeros((64, 40), dtype=bf))
    raises("out must be", moe.moe_gmm, lhs, rhs, gs, out=torch.zeros((64, 48, 1), dtype=bf))
    raises("out does not have out_dtype", moe.moe_gmm, lhs, rhs, gs,
           out=torch.zeros((64, 48), dtype=bf), out_dtype=torch.float32)
    x2 = torch.zeros((64, 48), dtype=bf)
    raises("out must be", moe.moe_tgmm, lhs, x2, gs, out=torch.zeros((2, 32, 40), dtype=bf))
    raises("out must be", moe.moe_tgmm, lhs, x2, gs, out=torch.zeros((3, 32, 48), dtype=bf))
    raises("group_sizes must be a contiguous int32", moe.moe_tgmm, lhs, x2, gs.long())
    raises("valid_rows must be a contiguous int32", moe.moe_tgmm, lhs, x2, gs,
           valid_rows=gs.long())
    raises("dtypes differ", moe.moe_tgmm, lhs, x2.float(), gs)
    raises("group_sizes must be a contiguous int32", moe.moe_group_sum, x2, gs.long())
    wi = torch.zeros((2, 32, 256), dtype=bf)
    raises("act must be", moe.moe_gmm_swiglu, lhs, wi, gs, act=torch.zeros((64, 64), dtype=bf))
    raises("h must be", moe.moe_gmm_swiglu, lhs, wi, gs, h=torch.zeros((64, 128), dtype=bf))
    raises("group_sizes must be a contiguous int32", moe.moe_gmm_swiglu, lhs, wi, gs.long())


def test_header_serves_plain_c_callers(tmp_path, lib):
    """include/moe.h compiles as strict C99 and C++17 with every warning an
    error, and a C program linked against libmoe.so through it calls the
    library (host-side entry points only: no GPU is touched)."""
    src = tmp_path / "caller.c"
    src.write_text(
        '#include "moe.h"\n'
        "#include <stdio.h>\n"
        "int main(void) {\n"
        "  const int64_t rows = moe_rows_bound(4096, 8, 256, 128, 0, 0);\n"
        "  printf(\"%d %lld %s\\n\", moe_abi_version(), (long long)rows, moe_status_string(MOE_ERR_ARG));\n"
        "  return 0;\n"
        "}\n")
    inc = os.path.join(ROOT, "include")
    libdir = os.path.dirname(moe.LIB_PATH)
    exe = tmp_path / "caller"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc,
                    str(src), "-o", str(exe), os.path.join(libdir, "libmoe.so"),
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True)
    cpp = tmp_path / "caller.cpp"
    cpp.write_text('#include "moe.h"\nint main() { return moe_abi_version() > 0 ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc,
                    "-fsyntax-only", str(cpp)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    ver, rows, msg = r.stdout.split(" ", 2)
    assert int(ver) == lib.moe_abi_version()
    assert int(rows) == lib.moe_rows_bound(4096, 8, 256, 128, 0, 0)
    assert msg.strip().startswith("invalid argument")
