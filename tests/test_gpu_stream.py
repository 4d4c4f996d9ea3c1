"""The binding's stream argument: work issued on a side stream (a torch Stream object or its raw
handle) gives the same bytes as on the current stream.  Selection and compaction bit-exact,
scores bit-identical (same kernel, same inputs)."""
import numpy as np
import pytest

from learned_token_pruning_gatescore_amd import workloads as wl
from tests._gpu import dev_tensor, device, say, to_np

pytestmark = pytest.mark.gpu


def test_side_stream_matches_current_stream():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    w = wl.WORKLOADS["qwen3_8k"]
    gi = wl.gate_inputs(w)
    h = dev_tensor(gi["hidden"], w.dtype, dev)
    w1 = dev_tensor(gi["w1"], w.dtype, dev)
    w2 = dev_tensor(gi["w2"], w.dtype, dev)
    forced = torch.from_numpy(gi["forced"]).to(dev)
    K = w.Ks[0]
    M = tg.tg_kept_count(w.N, w.n_forced, K)

    def path(stream):
        scores = torch.full((w.B, w.N), float("nan"), device=dev)
        gates = torch.full_like(scores, float("nan"))
        kept = torch.full((w.B, M), -7, dtype=torch.int32, device=dev)
        hk = torch.zeros((w.B, M, w.d), dtype=h.dtype, device=dev)
        pk = torch.zeros((w.B, M), dtype=torch.int32, device=dev)
        gk = torch.zeros((w.B, M), device=dev)
        torch.cuda.synchronize()  # the buffers are filled on the current stream first
        tg.tg_gate_score(h, w1, w2, forced, scores, gates, stream=stream)
        tg.tg_select_topk(scores, forced, K, w.n_forced, kept, stream=stream)
        tg.tg_compact(h, None, gates, kept, hk, pk, gk, stream=stream)
        torch.cuda.synchronize()
        return [to_np(x) for x in (scores, gates, kept, hk, pk, gk)]

    say("stream", w.name)
    ref = path(None)
    side = torch.cuda.Stream()
    for s in (side, side.cuda_stream):
        got = path(s)
        for a, b in zip(got, ref):
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))
