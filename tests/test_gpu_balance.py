"""GPU parity of the auxiliary-loss-free bias update against the oracle.

The update is integer comparisons plus one fp32 addition per expert, so the
bias after moe_bias_update must equal the oracle's bit for bit; the loads it
uses (the permute's counts) must equal the oracle's count of the batch's pairs.
"""
import numpy as np
import pytest
import torch

from oracle import balance
from parity import say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import configs, synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu

SMALL_BIASED = LayerShape(
    name="balance_groups", T=777, dim=384, n_routed=32, n_groups=4, topk_groups=2, top_k=4,
    n_shared=1, inter_dim=320, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
    seed=11, bias_range=0.1)
SHAPES = [configs.TINY_F32, SMALL_BIASED, configs.V3_DECODE_FP8, configs.V3_PREFILL_BF16]


def _gate_and_route(cfg, T, x, w_gate, bias):
    E, K = cfg.n_routed, cfg.top_k
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    B.moe_gate(cfg, T, x, w_gate, bias, logits, idx, w)
    r = B.make_routing(cfg, T)
    B.moe_permute(cfg, T, idx, r)
    return idx, r


def _bits(t):
    return t.detach().cpu().numpy().astype(np.float32).view(np.uint32)


@pytest.mark.parametrize("shape", SHAPES, ids=[s.name for s in SHAPES])
@pytest.mark.parametrize("gamma", [1e-3, 2.0 ** -10])
def test_bias_update_matches_oracle(shape, gamma):
    say(f"[moe_bias_update] {shape.name} gamma={gamma}")
    x, w_gate, bias0 = synth.make_gate_inputs(shape, device="cuda")
    cfg = B.config_of(shape)
    T, E, K = shape.T, shape.n_routed, shape.top_k
    idx, r = _gate_and_route(cfg, T, x, w_gate, bias0)
    bias = bias0.clone()
    before = bias.cpu().numpy()
    B.moe_bias_update(cfg, T, r, gamma, bias)
    torch.cuda.synchronize()
    loads = balance.expert_loads(idx.cpu().numpy(), E)
    assert np.array_equal(r.counts.cpu().numpy(), loads)
    want = balance.bias_update(before, loads, T, K, gamma)
    assert np.array_equal(_bits(bias), want.view(np.uint32))


def test_bias_update_noop_cases():
    shape = configs.TINY_F32
    cfg = B.config_of(shape)
    E, K, T = shape.n_routed, shape.top_k, 64          # 256 pairs over 16 experts: 16 each
    say("[moe_bias_update] balanced loads and gamma = 0")
    idx = ((torch.arange(T * K, dtype=torch.int32) % E).reshape(T, K)).cuda()
    r = B.make_routing(cfg, T)
    B.moe_permute(cfg, T, idx, r)
    bias = torch.linspace(-0.1, 0.1, E, dtype=torch.float32, device="cuda")
    bias[3] = -0.0                                     # a negative zero must survive untouched
    before = _bits(bias)
    B.moe_bias_update(cfg, T, r, 0.25, bias)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(bias), before)
    # gamma = 0 on skewed loads: every value stays, and the bits are the oracle's
    # (one fp32 addition: an underloaded -0.0 becomes +0.0, as -0 + 0 = +0)
    skew = torch.zeros(T, K, dtype=torch.int32, device="cuda")
    skew[:, 1] = 1
    B.moe_permute(cfg, T, skew, r)
    start = bias.cpu().numpy()
    B.moe_bias_update(cfg, T, r, 0.0, bias)
    torch.cuda.synchronize()
    want = balance.bias_update(start, balance.expert_loads(skew.cpu().numpy(), E), T, K, 0.0)
    assert np.array_equal(_bits(bias), want.view(np.uint32))
    assert np.array_equal(bias.cpu().numpy(), start)


def test_bias_update_fractional_mean():
    # 5 tokens x 4 slots over 24 experts: mean 20/24 < 1, so every used expert is
    # overloaded and every unused one underloaded
    shape = LayerShape(name="frac", T=5, dim=64, n_routed=24, n_groups=1, topk_groups=1, top_k=4,
                       n_shared=0, inter_dim=64, score="sigmoid", route_scale=1.0, act="f32",
                       weight="f32", seed=3)
    cfg = B.config_of(shape)
    say("[moe_bias_update] fractional mean")
    g = torch.Generator().manual_seed(9)
    idx = torch.stack([torch.randperm(24, generator=g)[:4] for _ in range(5)]).to(torch.int32)
    r = B.make_routing(cfg, 5)
    B.moe_permute(cfg, 5, idx.cuda(), r)
    bias = torch.zeros(24, dtype=torch.float32, device="cuda")
    B.moe_bias_update(cfg, 5, r, 0.5, bias)
    torch.cuda.synchronize()
    loads = balance.expert_loads(idx.numpy(), 24)
    want = balance.bias_update(np.zeros(24, np.float32), loads, 5, 4, 0.5)
    assert np.array_equal(_bits(bias), want.view(np.uint32))
    assert set(np.unique(want)) <= {-0.5, 0.5}


def test_repeated_balancing_steps():
    """Gate -> permute -> update, 25 times on the GPU (the gate sees each new bias);
    the oracle replays every step from the GPU's routing and must agree bit for bit."""
    shape = SMALL_BIASED
    x, w_gate, bias0 = synth.make_gate_inputs(shape, device="cuda")
    cfg = B.config_of(shape)
    T, E, K = shape.T, shape.n_routed, shape.top_k
    bias = bias0.clone()
    ref = bias.cpu().numpy().astype(np.float32)
    say("[moe_bias_update] 25 chained steps")
    spread = []
    for _ in range(25):
        idx, r = _gate_and_route(cfg, T, x, w_gate, bias)
        B.moe_bias_update(cfg, T, r, 2e-3, bias)
        torch.cuda.synchronize()
        loads = balance.expert_loads(idx.cpu().numpy(), E)
        ref = balance.bias_update(ref, loads, T, K, 2e-3)
        assert np.array_equal(_bits(bias), ref.view(np.uint32))
        spread.append(loads.max() - loads.min())
    assert spread[-1] < spread[0]


@pytest.mark.parametrize("E,K,T,seq_len,score", [
    (16, 4, 64, 64, "sigmoid"), (16, 2, 300, 100, "softmax"), (256, 8, 8192, 4096, "sigmoid"),
    (160, 6, 4096, 1, "softmax"), (512, 32, 96, 32, "sigmoid"), (37, 3, 50, 25, "sigmoid"),
    (100, 6, 66, 33, "softmax")])
def test_balance_loss_matches_oracle(E, K, T, seq_len, score):
    """Seeded logits and routings given to both sides."""
    say(f"[moe_balance_loss] E={E} K={K} T={T} seq_len={seq_len} {score}")
    g = torch.Generator().manual_seed(E * 1000 + T)
    logits = torch.randn(T, E, generator=g) * 2.0
    idx = torch.stack([torch.randperm(E, generator=g)[:K] for _ in range(T)]).to(torch.int32)
    shape = LayerShape(name="bl", T=T, dim=128, n_routed=E, n_groups=1, topk_groups=1, top_k=K,
                       n_shared=0, inter_dim=128, score=score, route_scale=1.0, act="f32", weight="f32")
    cfg = B.config_of(shape)
    loss = torch.empty(T // seq_len, dtype=torch.float32, device="cuda")
    B.moe_balance_loss(cfg, T, seq_len, logits.cuda(), idx.cuda(), 1e-3, loss)
    torch.cuda.synchronize()
    want = balance.sequence_balance_loss(logits.numpy().astype(np.float64), idx.numpy(), score, 1e-3, seq_len)
    got = loss.cpu().numpy().astype(np.float64)
    assert np.allclose(got, want, rtol=2e-6, atol=0)
    # a second call on a workspace full of NaN bytes: the partials are fully rewritten
    ws = torch.full((B.moe_balance_loss_workspace_size(cfg, T, seq_len),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    loss2 = torch.empty_like(loss)
    B.moe_balance_loss(cfg, T, seq_len, logits.cuda(), idx.cuda(), 1e-3, loss2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)


def test_balance_loss_on_the_v3_gate():
    """The V3 prefill batch: the oracle forms its own float64 logits from x and W_g and
    uses the GPU's (certified) routing for the indicator."""
    import oracle
    from oracle_bridge import to_f64
    shape = configs.V3_PREFILL_BF16
    say("[moe_balance_loss] v3 prefill gate")
    x, w_gate, bias = synth.make_gate_inputs(shape, device="cuda")
    cfg = B.config_of(shape)
    T, E, K = shape.T, shape.n_routed, shape.top_k
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    B.moe_gate(cfg, T, x, w_gate, bias, logits, idx, w)
    loss = torch.empty(2, dtype=torch.float32, device="cuda")
    B.moe_balance_loss(cfg, T, T // 2, logits, idx, 1e-4, loss)
    torch.cuda.synchronize()
    l64 = oracle.gate_logits(to_f64(x), to_f64(w_gate))
    want = balance.sequence_balance_loss(l64, idx.cpu().numpy(), "sigmoid", 1e-4, T // 2)
    assert np.allclose(loss.cpu().numpy().astype(np.float64), want, rtol=1e-5, atol=0)
