"""The decode step captured into a HIP graph replays to the eager result."""
import numpy as np
import pytest

from flint_cases import CacheDecodeCase, dev, up

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import full_gqa_decode_amd as fl
    case = CacheDecodeCase(8, [5000], window=0)
    q, kc, vc = up(case.q), up(case.kc), up(case.vc)
    bt, sl, sk = up(case.bt), up(case.seq_lens), up(case.sinks)
    ws = torch.zeros(fl.flint_attn_decode_workspace_size(case.FL, 1, 5000), dtype=torch.uint8,
                     device=dev())
    eager = torch.empty((1, 32, 128), dtype=torch.float32, device=dev())
    fl.flint_attn_decode(case.FL, q, kc, vc, bt, sl, 5000, sk, eager, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fl.flint_attn_decode(case.FL, q, kc, vc, bt, sl, 5000, sk, out, workspace=ws)
    ref = eager.cpu().numpy()
    for _ in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)
        # eager work between replays
        fl.flint_attn_decode(case.FL, q, kc, vc, bt, sl, 5000, sk, eager, workspace=ws)
        torch.cuda.synchronize()
