"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every case compares every output element: the reduced-size cases and the
full-size workloads alike (all tokens, a global and a per-row bound).  Each
full-size workload also runs twice and must give bit-identical outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from mixture_experts_layer_38_amd import datagen
from mixture_experts_layer_38_amd.configs import CONFIGS, MoEConfig, scaled
from tests.gpu_harness import (TOL_AUX, check_dispatch, check_logits, check_output,
                               check_routing, load_summary, run_forward, say)

pytestmark = pytest.mark.gpu

C = CONFIGS
REDUCED = {
    "tiny_fp32": C["tiny_fp32"],
    "decode_d512": scaled(C["mixtral_decode"], d=512, F=1536),
    "prefill_t600_ragged": scaled(C["mixtral_prefill"], T=600, d=264, F=200),
    "prefill_t2048": scaled(C["mixtral_prefill"], T=2048, d=512, F=1024),
    "prefill_t700_ntail": scaled(C["mixtral_prefill"], T=700, d=384, F=640),
    "dsv3_t256": scaled(C["dsv3_routed"], T=256, d=256, F=256),
    "capacity_t2048": scaled(C["capacity_top2"], T=2048, d=256, F=1408),
    "fp32_ragged": scaled(C["tiny_fp32"], T=77, d=40, E=5, K=3, F=24),
    "decode_t64_e4": scaled(C["mixtral_decode"], T=64, d=256, E=4, F=520),
    "one_token": scaled(C["mixtral_prefill"], T=1, d=256, F=512),
    "k_equals_e": scaled(C["mixtral_decode"], T=40, d=128, E=4, K=4, F=256),
    "top1_decode": scaled(C["mixtral_decode"], T=48, d=512, K=1, F=768),
    "top1_prefill": scaled(C["mixtral_prefill"], T=900, d=320, K=1, F=384),
    # decode-sized batches that take the one-launch router + dispatch path
    "small_e16_ragged_d": scaled(C["dsv3_routed"], T=37, d=584, E=16, K=4, F=256),
    "small_t64_e16": scaled(C["capacity_top2"], T=64, d=256, E=16, F=128),
    # the largest sizes the boundary accepts: E = 1024 with K = 32 (one-stage
    # reductions, every expert on the weight-streaming kernel), d = 65536 on
    # the decode path, F = 65536 on the prefill path
    "max_e1024_k32": scaled(C["dsv3_routed"], T=96, d=64, E=1024, K=32, F=64),
    "max_d65536_decode": scaled(C["mixtral_decode"], T=40, d=65536, E=2, K=1, F=64),
    "max_f65536_prefill": scaled(C["mixtral_prefill"], T=100, d=128, E=2, K=2, F=65536),
}


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _case(orc, cfg: MoEConfig, logit_bias=None, flags: int = 0, repeat: int = 1):
    say(f"[case] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} K={cfg.K} F={cfg.F} {cfg.dtype} "
        f"C={cfg.capacity} flags={flags}")
    inp = datagen.make_inputs(cfg)
    bias = inp["logit_bias"] if logit_bias is None else logit_bias
    outs, _ = run_forward(cfg, inp, bias, flags=flags, repeat=repeat)
    out = outs[0] if repeat > 1 else outs
    if repeat > 1:
        for i, o in enumerate(outs[1:], 1):
            for k in out:
                assert np.array_equal(out[k], o[k]), f"run {i} differs from run 0 in {k}"
        say(f"    {repeat} runs bit-identical in all {len(out)} outputs")
    say("   ", load_summary(cfg, out))
    check_logits(orc, inp, out["logits"])
    ids, w, probs = check_routing(orc, cfg, out, bias, flags)
    ref = check_dispatch(orc, cfg, ids, out, cfg.capacity)
    err, worst, row = check_output(orc, cfg, inp, ids, w, ref["assign_row"], out["y"])
    say(f"    output error {err:.3e}, worst row {row}: {worst:.3e}")
    return inp, out, ids, w, probs


@pytest.mark.parametrize("name", list(REDUCED))
def test_forward_reduced(orc, name):
    _case(orc, REDUCED[name])


def test_forward_determinism():
    cfg = REDUCED["capacity_t2048"]
    inp = datagen.make_inputs(cfg)
    outs, _ = run_forward(cfg, inp, repeat=2)
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_all_tokens_to_one_expert(orc):
    cfg = scaled(C["mixtral_prefill"], T=300, d=256, F=512, skew="none")
    bias = np.zeros(cfg.E, np.float32)
    bias[3] = 100.0
    inp, out, ids, _, _ = _case(orc, cfg, logit_bias=bias)
    assert np.all(ids[:, 0] == 3) and out["counts"][3] == cfg.T


def test_capacity_zero_one_and_unlimited(orc):
    base = scaled(C["capacity_top2"], T=512, d=128, F=256)
    for cf in (0.0, 1.0 / 16, 1.0, 64.0):
        cfg = scaled(base, capacity_factor=cf)
        inp, out, *_ = _case(orc, cfg)
        if cfg.capacity == 0:
            assert out["offsets"][-1] == 0 and np.all(out["y"] == 0)


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_decode", "mixtral_prefill", "capacity_top2",
                                  "dsv3_routed"])
@pytest.mark.timeout(900)
def test_forward_full_size(orc, name):
    """Each workload at its full size: every token against the oracle, and two
    runs bit-identical."""
    cfg = C[name]
    inp, out, ids, w, probs = _case(orc, cfg, repeat=2)
    if cfg.alpha is not None:
        _check_aux_and_bias(orc, cfg, out, probs)


def _check_aux_and_bias(orc, cfg, out, probs):
    import torch
    from mixture_experts_layer_38_amd import moe_aux_loss, moe_bias_update, problem_of
    p = problem_of(cfg)
    counts = torch.from_numpy(out["counts"]).cuda()
    psum = torch.from_numpy(out["prob_sum"]).cuda()
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    moe_aux_loss(p, counts, psum, aux)
    beta = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    moe_bias_update(p, counts, cfg.alpha, beta)
    torch.cuda.synchronize()
    aux_ref = orc.aux_loss(out["counts"], probs, cfg.K)
    assert abs(float(aux.item()) - aux_ref) <= TOL_AUX * abs(aux_ref), (aux.item(), aux_ref)
    psum_ref = probs.sum(0)
    assert np.abs(out["prob_sum"] - psum_ref).max() <= 1e-5 * cfg.T / cfg.E + 1e-6
    beta_ref = orc.bias_update(out["counts"], cfg.T, cfg.K, cfg.alpha, np.zeros(cfg.E, np.float32))
    assert np.array_equal(beta.cpu().numpy(), beta_ref)
    say(f"    aux {aux.item():.6f} (oracle {aux_ref:.6f}, E*aux {cfg.E * aux_ref:.3f}); "
        f"bias +{int((beta_ref > 0).sum())} -{int((beta_ref < 0).sum())}")


@pytest.mark.parametrize("name", ["capacity_t2048", "small_t64_e16"])
def test_aux_and_bias_reduced(orc, name):
    cfg = REDUCED[name]
    inp, out, ids, w, probs = _case(orc, cfg)
    _check_aux_and_bias(orc, cfg, out, probs)


def test_small_batch_capacity(orc):
    """A per-expert cap on a decode-sized batch (the one-launch router path)."""
    base = scaled(C["capacity_top2"], T=48, d=128, E=16, F=128)
    for cf in (0.0, 0.25, 1.0):
        cfg = scaled(base, capacity_factor=cf)
        inp, out, *_ = _case(orc, cfg)
        if cfg.capacity == 0:
            assert out["offsets"][-1] == 0 and np.all(out["y"] == 0)


@pytest.mark.parametrize("name,flags", [("dsv3_t256", 1), ("capacity_t2048", 2), ("prefill_t600_ragged", 3),
                                        ("tiny_fp32", 1), ("decode_d512", 2), ("decode_d512", 1),
                                        ("small_e16_ragged_d", 3)])
def test_forward_routing_variants(orc, name, flags):
    """Bias for selection only (flag 1), unweighted mean combine (flag 2), both."""
    _case(orc, REDUCED[name], flags=flags)
