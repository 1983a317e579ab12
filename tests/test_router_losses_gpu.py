"""Router regularisers against the oracle: the z-loss of the router scores and
the top-K-only aux loss, on the GPU's own scores and routing (the oracle
recomputes the routing probabilities from those scores).  Two paths: the
standalone moe_router_losses over stored scores, and the same values gathered
by the routing kernel inside moe_forward (optional outputs z_loss and
aux_topk), on both router paths (decode-sized one-block routing and the
batched route kernel) and with the bias used for selection only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mixture_experts_layer_38_amd as moe
from mixture_experts_layer_38_amd import datagen
from mixture_experts_layer_38_amd.configs import CONFIGS, scaled
from tests.gpu_harness import run_forward, say

pytestmark = pytest.mark.gpu

TOL_REL = 1e-5


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _losses(cfg, logits, bias, ids, counts):
    import torch
    p = moe.problem_of(cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    z = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    a = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_router_losses_workspace_size(p), dtype=torch.uint8, device="cuda")
    moe.moe_router_losses(p, dev(logits), None if bias is None else dev(bias.astype(np.float32)),
                          dev(ids), dev(counts), z, a, ws)
    torch.cuda.synchronize()
    return float(z.item()), float(a.item())


def _check(orc, cfg, logits, bias, ids, counts, got=None):
    z, a = _losses(cfg, logits, bias, ids, counts) if got is None else got
    _, _, probs = orc.route(logits, cfg.K, bias)
    z_ref = orc.z_loss(logits)
    a_ref = orc.aux_topk(counts, ids, probs)
    say(f"    z_loss {z:.6f} (oracle {z_ref:.6f})  aux_topk {a:.6f} (oracle {a_ref:.6f}, "
        f"full aux {orc.aux_loss(counts, probs, cfg.K):.6f})")
    assert abs(z - z_ref) <= TOL_REL * abs(z_ref), (z, z_ref)
    assert abs(a - a_ref) <= TOL_REL * abs(a_ref), (a, a_ref)


@pytest.mark.parametrize("name,cfg", [
    ("capacity_full", CONFIGS["capacity_top2"]),
    ("dsv3_t512", scaled(CONFIGS["dsv3_routed"], T=512, d=256, F=256)),
    ("decode", scaled(CONFIGS["mixtral_decode"], d=512, F=1024)),
    ("prefill_t1000", scaled(CONFIGS["mixtral_prefill"], T=1000, d=256, F=512)),
])
def test_router_losses_after_forward(orc, name, cfg):
    say(f"[case] router losses {name} T={cfg.T} E={cfg.E} K={cfg.K}")
    inp = datagen.make_inputs(cfg)
    out, _ = run_forward(cfg, inp)
    _check(orc, cfg, out["logits"], inp["logit_bias"], out["topk_ids"], out["counts"])


def test_router_losses_many_experts(orc):
    """E = 1000, K = 7 (sixteen experts per lane), scores of large magnitude."""
    cfg = scaled(CONFIGS["dsv3_routed"], T=300, d=64, E=1000, K=7, F=64)
    say(f"[case] router losses E={cfg.E} K={cfg.K}")
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((cfg.T, cfg.E)) * 8).astype(np.float32)
    bias = rng.uniform(-1, 1, cfg.E).astype(np.float32)
    ids, _, _ = orc.route(logits, cfg.K, bias)
    counts = np.bincount(ids.ravel(), minlength=cfg.E).astype(np.int32)
    _check(orc, cfg, logits, bias, ids, counts)


@pytest.mark.parametrize("name,cfg,flags", [
    ("capacity_full", CONFIGS["capacity_top2"], 0),
    ("dsv3_t512", scaled(CONFIGS["dsv3_routed"], T=512, d=256, F=256), 0),
    ("dsv3_t512_select_only", scaled(CONFIGS["dsv3_routed"], T=512, d=256, F=256), 1),
    ("decode_small_path", scaled(CONFIGS["mixtral_decode"], d=512, F=1024), 0),
    ("small_path_biased_select_only", scaled(CONFIGS["capacity_top2"], T=48, d=256, E=16, F=128), 1),
    ("small_path_biased", scaled(CONFIGS["capacity_top2"], T=64, d=256, E=16, F=128), 0),
    ("prefill_t1000", scaled(CONFIGS["mixtral_prefill"], T=1000, d=256, F=512), 0),
    ("e1000_k7", scaled(CONFIGS["dsv3_routed"], T=300, d=64, E=1000, K=7, F=64), 0),
])
def test_router_losses_inside_forward(orc, name, cfg, flags):
    say(f"[case] router losses inside the layer {name} T={cfg.T} E={cfg.E} K={cfg.K} flags={flags}")
    inp = datagen.make_inputs(cfg)
    out, _ = run_forward(cfg, inp, flags=flags, losses=True)
    got = (float(out["z_loss"][0]), float(out["aux_topk"][0]))
    _check(orc, cfg, out["logits"], inp["logit_bias"], out["topk_ids"], out["counts"], got=got)
