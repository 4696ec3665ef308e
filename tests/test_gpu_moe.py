"""GPU parity of the MoE sublayer (router, sigmoid top-k, routed and shared
SwiGLU experts) against the fp64 oracle (O9, O10), through the C ABI.

Weights are N(0, 1/fan_in) bf16 drawn on the GPU by a seeded torch generator
and copied to the host for the oracle; x ~ N(0,1) from synth.  The expert
selection is an integer decided by floating point: every case checks first
that the oracle's logits leave a gap of at least 1e-3 at the top-k boundary,
far above fp32 rounding, so both sides must pick the same experts."""
import numpy as np
import pytest

import oracle
import synth
from flint_cases import TOL, assert_parity, check_err, dev, up

pytestmark = pytest.mark.gpu

FLINT = dict(hidden=2048, experts=256, top_k=6, inter=512, shared=1)


class MoeCase:
    def __init__(self, seed, T, shape=FLINT, x=None):
        import torch
        import full_gqa_decode_amd as fl
        self.M = oracle.moe(**shape)
        self.FM = fl.moe_layer(shape["hidden"], shape["experts"], shape["top_k"], shape["inter"],
                               shape["shared"])
        H, E, I, S = shape["hidden"], shape["experts"], shape["inter"], shape["shared"]
        tag = (seed, 60)
        self.wr = synth.normal_bf16_bits_torch(0, tag + (1,), (E, H), dev(), std=H ** -0.5)
        self.wgu = synth.normal_bf16_bits_torch(0, tag + (2,), (E + S, 2, I, H), dev(),
                                                std=H ** -0.5)
        self.wd = synth.normal_bf16_bits_torch(0, tag + (3,), (E + S, H, I), dev(), std=I ** -0.5)
        torch.cuda.synchronize()
        self.x = synth.normal(seed, (61,), (T, H)) if x is None else np.asarray(x, np.float32)
        self.T = T

    def host(self, t):
        return t.cpu().numpy().view(np.uint16)

    def topk_gap(self):
        """Smallest distance, over the tokens, between the k-th and (k+1)-th
        largest exact router logit (inf when every expert is selected)."""
        if self.M.top_k >= self.M.experts:
            return np.inf
        wr = self.host(self.wr)
        z = synth.bf16_bits_to_f32(wr).astype(np.float64) @ self.x.T.astype(np.float64)
        zs = -np.sort(-z, axis=0)
        return float((zs[self.M.top_k - 1] - zs[self.M.top_k]).min())

    def expected(self):
        gap = self.topk_gap()
        assert gap > 1e-3, f"top-k boundary too close for a parity case ({gap:.2e})"
        wr = self.host(self.wr)
        return oracle.moe_forward(self.M, self.x, wr, self.host(self.wgu), self.host(self.wd))

    def run_gpu(self):
        import torch
        import full_gqa_decode_amd as fl
        out, ids, w = fl.flint_moe_forward(self.FM, up(self.x), self.wr, self.wgu, self.wd)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check(case):
    ids_ref, w_ref, y_ref = case.expected()
    y, ids, w = case.run_gpu()
    assert np.array_equal(ids, ids_ref)
    assert np.abs(w - w_ref).max() <= 1e-5
    err = float(np.abs(y.astype(np.float64) - y_ref).max())
    print(f"moe T={case.T}: max err {err:.3e} (|y| max {np.abs(y_ref).max():.2f})", flush=True)
    check_err(err, y_ref)
    return y


@pytest.mark.parametrize("T", [1, 2, 8])
def test_moe_flint_shape(T):
    check(MoeCase(1, T))


def test_moe_other_shape_two_shared_experts_top8():
    check(MoeCase(2, 3, dict(hidden=1024, experts=64, top_k=8, inter=512, shared=2)))


@pytest.mark.parametrize("T,shape", [
    (5, dict(hidden=1536, experts=100, top_k=4, inter=512, shared=1)),
    (3, dict(hidden=4096, experts=256, top_k=6, inter=512, shared=1)),
    (7, dict(hidden=3584, experts=37, top_k=2, inter=512, shared=2)),
    (4, dict(hidden=2560, experts=9, top_k=8, inter=512, shared=0)),
])
def test_moe_other_hidden_sizes_and_expert_counts(T, shape):
    # hidden/512 = 3, 8, 7, 5 (the kernels are specialised on it), expert
    # counts that are not a multiple of the 64-lane selection width
    check(MoeCase(7, T, shape))


@pytest.mark.parametrize("T,top_k,shared", [
    (6, 1, 1), (1, 2, 1), (2, 5, 1), (3, 7, 2), (4, 8, 1), (8, 3, 0), (7, 6, 0), (5, 4, 2),
])
def test_moe_every_token_and_slot_count(T, top_k, shared):
    # with the other tests, every token count 1..8 (the router's 1-, 2-, 4- and
    # 8-token forms with clamped indices) and every slot count top_k + shared
    # from 1 to 10 (one down-kernel form each) is run.  The first seed whose
    # exact logits leave a clear top-k boundary is taken.
    shape = dict(hidden=512, experts=24, top_k=top_k, inter=512, shared=shared)
    for seed in range(100 + 10 * T + top_k, 140 + 10 * T + top_k):
        case = MoeCase(seed, T, shape)
        if case.topk_gap() > 1e-3:
            break
    check(case)


def test_moe_without_shared_expert():
    check(MoeCase(3, 2, dict(hidden=512, experts=256, top_k=1, inter=512, shared=0)))


def test_moe_tokens_that_share_experts():
    x = synth.normal(4, (61,), (3, 2048))
    x = np.stack([x[0], x[1], x[0], x[2], x[1]])
    y = check(MoeCase(4, 5, x=x))
    assert np.array_equal(y[0], y[2]) and np.array_equal(y[1], y[4])


def test_moe_rank_one_closed_form_at_flint_shape():
    # router row e = c_e e_0, gate/up rows a_j e_0 / b_j e_0, down rows c_r v:
    # with x[0] = 1 every product is exact and the output has a closed form
    import torch
    import full_gqa_decode_amd as fl
    rng = synth.rng(5, 1)
    H, E, I, S, K = 2048, 256, 512, 1, 6
    q8 = lambda a: np.round(a * 8) / 8
    z = rng.permutation(E) / 8.0 - 16.0
    a = q8(rng.uniform(-2, 2, (E + S, I)))
    b = q8(rng.uniform(-2, 2, (E + S, I)))
    c = q8(rng.uniform(-1, 1, (E + S, H)))
    v = q8(rng.uniform(-1, 1, (E + S, I)))
    bits = lambda arr: (np.asarray(arr, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wr = np.zeros((E, H), np.uint16)
    wr[:, 0] = bits(z)
    wgu = torch.zeros((E + S, 2, I, H), dtype=torch.int16, device=dev())
    wgu[:, 0, :, 0] = up(bits(a))
    wgu[:, 1, :, 0] = up(bits(b))
    wd = up(bits(np.einsum("er,ej->erj", c.astype(np.float32), v.astype(np.float32))))
    x = synth.normal(5, (2,), (1, H))
    x[0, 0] = 1.0
    out, ids, w = fl.flint_moe_forward(fl.moe_layer(), up(x), up(wr), wgu, wd)
    torch.cuda.synchronize()
    top = np.argsort(-z, kind="stable")[:K]
    s = 1.0 / (1.0 + np.exp(-z[top]))
    silu = lambda g: g / (1.0 + np.exp(-g))
    expert = np.array([c[e] * float(np.sum(v[e] * silu(a[e]) * b[e])) for e in range(E + S)])
    ref = (s / s.sum()) @ expert[top] + expert[E]
    assert ids.cpu().numpy()[0].tolist() == top.tolist()
    assert np.abs(w.cpu().numpy()[0] - s / s.sum()).max() <= 1e-6
    assert np.abs(out.cpu().numpy()[0] - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())


def test_moe_nan_token_stays_in_its_row():
    import torch
    import full_gqa_decode_amd as fl
    case = MoeCase(6, 2)
    x = case.x.copy()
    x[1, 100] = np.nan
    out, ids, _ = fl.flint_moe_forward(case.FM, up(x), case.wr, case.wgu, case.wd)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isnan(o[1]).all() and np.isfinite(o[0]).all()
    ids = ids.cpu().numpy()
    assert ((ids >= 0) & (ids < 256)).all()
    one = MoeCase(6, 1, x=case.x[:1])
    _, _, y_ref = one.expected()
    assert_parity(o[0], y_ref[0])


def test_moe_graph_replays_match_eager():
    import torch
    import full_gqa_decode_amd as fl
    case = MoeCase(7, 4)
    xd = up(case.x)
    ws = torch.empty(fl.flint_moe_workspace_size(case.FM, 4), dtype=torch.uint8, device=dev())
    out = torch.empty((4, 2048), dtype=torch.float32, device=dev())
    ids = torch.empty((4, 6), dtype=torch.int32, device=dev())
    w = torch.empty((4, 6), dtype=torch.float32, device=dev())
    run = lambda: fl.flint_moe_forward(case.FM, xd, case.wr, case.wgu, case.wd, out=out,
                                       topk_ids=ids, topk_weights=w, workspace=ws)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
