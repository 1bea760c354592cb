"""moe_permute_noalloc (static device scratch, no workspace argument) against
moe_permute (caller workspace) through the C ABI: index maps, counts and
x_sorted bit for bit, on consecutive calls whose sizes shrink, so that a
later call runs over the scratch an earlier, larger call left behind."""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev_i32, poison

pytestmark = pytest.mark.gpu

KEYS = ("counts", "group_sizes", "group_offsets", "row_of_slot", "slot_of_row")


def _ids(g, T, K, E):
    """K distinct experts per token, Zipf-skewed (some experts empty)."""
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    logp = np.log(p / p.sum())
    return np.argsort(-(logp[None, :] + g.gumbel(size=(T, E))), axis=1)[:, :K].astype(np.int32)


# T, K, E, align, capacity, capacity_layout, D (0 = index maps only); each
# sequence runs its calls in this order, largest first
SEQUENCES = {
    # the largest supported size (ceil(T K / 1024) * E = 262144 words), then smaller ones
    "max_then_smaller": [(131072, 8, 256, 0, 0, 0, 0), (4096, 8, 256, 128, 0, 0, 7168),
                         (300, 2, 8, 0, 0, 0, 64)],
    "dropping_then_smaller": [(8192, 1, 256, 0, 32, 0, 512), (700, 1, 32, 0, 22, 1, 192)],
    "aligned_then_no_tokens": [(2000, 4, 64, 16, 0, 0, 256), (0, 2, 8, 0, 0, 0, 64)],
}


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_matches_permute(gpu_lib, name):
    g = np.random.default_rng(len(name))
    for (T, K, E, align, cap, lay, D) in SEQUENCES[name]:
        print(f"[noalloc] {name}: T={T} K={K} E={E} align={align} C={cap} layout={lay} D={D}",
              flush=True)
        ids = dev_i32(_ids(g, T, K, E) if T else np.zeros((0, K), np.int32))
        x = None
        if D:
            x = torch.from_numpy(g.standard_normal((T, D)).astype(np.float32)).cuda()
            x = x.to(torch.bfloat16)
        kw = dict(E=E, align=align, capacity=cap, capacity_layout=bool(lay))
        ref = gpu_lib.moe_permute(x, ids, with_rows=x is not None, **kw)
        rows = gpu_lib.moe_rows_bound(T, K, E, align, cap, bool(lay))
        out = {k: poison(torch.empty_like(ref[k])) for k in KEYS}
        xs = poison(torch.empty_like(ref["x_sorted"])) if x is not None else None
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = gpu_lib.moe_permute(x, ids, rows=rows, x_sorted=xs, with_rows=x is not None,
                                  out=out, err=err, noalloc=True, **kw)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (name, T, k)
        if x is not None:
            assert torch.equal(got["x_sorted"].view(torch.int16),
                               ref["x_sorted"].view(torch.int16)), (name, T, "x_sorted")
        assert int(err.item()) == 0


def test_noalloc_rejects_sizes_past_its_scratch(gpu_lib):
    T, K, E = 131073, 8, 256     # ceil(T K / 1024) * E = 262400 words > 262144
    ids = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.MoeError, match="workspace"):
        gpu_lib.moe_permute(None, ids, E, with_rows=False, noalloc=True)
