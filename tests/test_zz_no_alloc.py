"""The allocation-free selection entry point (tg_select_topk_noalloc, for callers that cannot
allocate device memory) against tg_select_topk with a caller workspace: two calls in a row on
one GPU, the second with a smaller input; bit-exact indices and counts.  Also the host-side
refusal of a problem larger than its scratch (no device work)."""
import numpy as np
import pytest

from tests._gpu import device, say, to_np

pytestmark = pytest.mark.gpu


def _pair(tg, dev, scores, forced, K, nF):
    import torch

    B, N = scores.shape
    M = tg.tg_kept_count(N, nF, K)
    s = torch.from_numpy(scores).to(dev)
    f = None if forced is None else torch.from_numpy(forced).to(dev)
    ref = torch.full((B, M), -7, dtype=torch.int32, device=dev)
    rc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    tg.tg_select_topk(s, f, K, nF, ref, rc, ws=tg.select_workspace(B, N, dev))
    got = torch.full((B, M), -9, dtype=torch.int32, device=dev)
    gc = torch.full((B,), -9, dtype=torch.int32, device=dev)
    say("select noalloc", B, N, K, nF)
    tg.tg_select_topk_noalloc(s, f, K, nF, got, gc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(got), to_np(ref))
    np.testing.assert_array_equal(to_np(gc), to_np(rc))


def test_noalloc_matches_workspace_call_twice():
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    rng = np.random.default_rng(2024)
    # first call: two rows of 70000 tokens, tie-rich bf16-grid scores, different forced counts
    B, N = 2, 70000
    s = (rng.standard_normal((B, N)).astype(np.float32) * 64).round() / 64
    f = np.zeros((B, N), np.uint8)
    f[0, rng.choice(N, 300, replace=False)] = 1
    f[1, rng.choice(N, 180, replace=False)] = 1
    _pair(tg, dev, s, f, 5000, 300)
    # second call, smaller: one row of 40000 tokens (still more than one work-group's 32768, so the
    # scratch is used again), no mask, a budget inside a large tie class
    s2 = np.where(rng.random((1, 40000)) < 0.5, np.float32(0.25), rng.standard_normal((1, 40000)).astype(np.float32))
    _pair(tg, dev, s2.astype(np.float32), None, 9000, 0)


def test_noalloc_refuses_beyond_its_scratch():
    import ctypes

    import learned_token_pruning_gatescore_amd as tg

    lib = tg.load()
    fake = ctypes.c_void_p(0x10000)
    # 64 rows of 2^20 tokens need far more than the scratch: refused on the host, nothing launched
    assert lib.tg_select_topk_noalloc(fake, None, 64, 1 << 20, 10, 0, fake, None, None) == 2
    assert b"scratch" in lib.tg_last_error()
