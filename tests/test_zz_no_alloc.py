"""moe_route_qb_noalloc (routing on the library's per-device scratch array,
for callers that cannot allocate) against moe_route_qb on a workspace:
bit-identical results on two calls in a row, the second one smaller, so
that the second call runs on scratch the first one left behind."""
import numpy as np
import pytest
import torch

import workloads
from oracle import layer as olayer

pytestmark = pytest.mark.gpu


def scores(T, n, std, seed):
    return torch.from_numpy(olayer.sigmoid(workloads.qb_logits(T, n, std, seed))
                            .astype(np.float32)).cuda()


def same(a, b):
    for key in ("idx", "w", "loads", "bias", "info"):
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8)), key


def test_noalloc_matches_workspace_entry_point_twice():
    import sparse_moe_ffn_sigmoid_amd as moe
    print("\n[gpu case] no-alloc routing T=4096 n=896 k=16, then T=300 n=64 k=6", flush=True)
    cases = [(scores(4096, 896, 0.5, 21), 16, None, moe.MOE_QB_BATCH),
             (scores(300, 64, 1.0, 22), 6, None, moe.MOE_QB_BATCH)]
    for s, k, bias, mode in cases:
        got = moe.route_qb_noalloc(s, k, bias, mode)
        ref = moe.route_qb(s, k, bias, mode)
        torch.cuda.synchronize()
        same(got, ref)
        assert int(got["info"][1]) == 0
    # frozen bias on the same scratch, after both batch calls
    s, k = cases[1][0], 6
    b = torch.linspace(-0.05, 0.05, 64, dtype=torch.float64, device="cuda")
    same(moe.route_qb_noalloc(s, k, b, moe.MOE_QB_FROZEN), moe.route_qb(s, k, b, moe.MOE_QB_FROZEN))


def test_noalloc_rejects_batches_beyond_the_scratch():
    import sparse_moe_ffn_sigmoid_amd as moe
    s = torch.zeros((8192, 896), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.route_qb_noalloc(s, 16)
