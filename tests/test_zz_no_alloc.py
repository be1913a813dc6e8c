"""The allocation-free AdamW entry point, adamw_clip_step_noalloc, against
adamw_clip_step, whose kernels it shares: two calls in a row on one GPU, the
second over fewer and smaller items than the first (the fixed scratch keeps
the first call's table and partial sums beyond what the second writes), two
steps each with a skipped gradient, an active clip, both weight dtypes.  The
two entry points build the same segment table and partial layout, so
weights, moments and the reported norm must agree bit for bit."""

import pytest
import torch

from adamw_optimizer_step_amd import api

from gpu_common import require_gpu, storage_draw, to_dev

pytestmark = pytest.mark.gpu

CALLS = [[3 * 2048 + 5, 100, 70000, 8, 2048 * 4 * 3 + 1, 4096], [1000, 17]]


def _state(sizes, dtype, seed):
    p = [to_dev(storage_draw(seed, 0, i, (n,), 0.02, dtype), dtype) for i, n in enumerate(sizes)]
    m = [torch.zeros(n, device="cuda") for n in sizes]
    v = [torch.zeros(n, device="cuda") for n in sizes]
    return p, m, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    require_gpu()
    for c, sizes in enumerate(CALLS):
        pa, ma, va = _state(sizes, dtype, 90 + c)
        pb, mb, vb = [t.clone() for t in pa], [t.clone() for t in ma], [t.clone() for t in va]
        for t in (1, 2):
            g = [to_dev(storage_draw(90 + c, t, i, (n,), 1.0, dtype), dtype)
                 for i, n in enumerate(sizes)]
            if t == 2:
                g[1] = None                       # a skipped gradient
            steps = [t] * len(sizes)
            wd = [0.1 if i % 2 else 0.0 for i in range(len(sizes))]
            na = torch.zeros(1, dtype=torch.float64, device="cuda")
            nb = torch.zeros(1, dtype=torch.float64, device="cuda")
            api.adamw_clip_step(pa, g, ma, va, steps, lr=3e-4, weight_decay=wd, max_norm=1.0,
                                norm_out=na)
            api.adamw_clip_step_noalloc(pb, g, mb, vb, steps, lr=3e-4, weight_decay=wd,
                                        max_norm=1.0, norm_out=nb)
            torch.cuda.synchronize()
            print(f"[noalloc] {dtype} call {c} step {t}: T = {na.item():.6f}", flush=True)
            assert na.item() > 1.0                 # the clip is active
            assert torch.equal(na, nb)
            for x, y in zip(pa + ma + va, pb + mb + vb):
                assert torch.equal(x, y)
