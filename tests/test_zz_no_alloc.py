"""The allocation-free layer (moe_forward_noalloc) against moe_forward, through
the C ABI: the same kernels on the library's static per-GPU workspace must give
bit-identical results to the caller-workspace entry point, on two calls in a
row (the second on a smaller problem, so stale contents of the static array
from the first call are present) and again after that."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_38_amd as moe
from mixture_experts_layer_38_amd import datagen
from mixture_experts_layer_38_amd.configs import CONFIGS, scaled
from mixture_experts_layer_38_amd.layer import MoELayer, to_device, to_host
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu


def _host(dbg: dict, y, dtype: str) -> dict:
    out = {k: v.cpu().numpy() for k, v in dbg.items()}
    out["y"] = to_host(y, dtype)
    return out


def _both(cfg):
    say(f"[noalloc] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} K={cfg.K} F={cfg.F} C={cfg.capacity}")
    inp = datagen.make_inputs(cfg)
    layer = MoELayer.from_host(cfg, inp)
    assert moe.moe_workspace_size(layer.p) <= moe.MOE_NOALLOC_WS_BYTES
    x = to_device(inp["x"], cfg.dtype)
    bias = None if inp["logit_bias"] is None else torch.from_numpy(inp["logit_bias"]).cuda()
    dbg_a = layer.alloc_debug()
    y_a = layer.forward(x, bias, dbg=dbg_a)
    dbg_b = layer.alloc_debug()
    y_b = torch.full_like(y_a, float("nan"))
    moe.moe_forward_noalloc(layer.p, x, layer.w_router, layer.w1, layer.w3, layer.w2, bias, y_b, dbg_b)
    torch.cuda.synchronize()
    a, b = _host(dbg_a, y_a, cfg.dtype), _host(dbg_b, y_b, cfg.dtype)
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{k} differs between moe_forward and moe_forward_noalloc"
    say(f"    identical in all {len(a)} outputs (S={int(a['offsets'][-1])})")


def test_noalloc_matches_forward_twice():
    # first a prefill-sized batch (tile plan, tiled GEMMs, split partial tiles
    # in the static array), then a smaller decode-sized one on top of its contents
    _both(scaled(CONFIGS["mixtral_prefill"], T=300, d=256, F=512))
    _both(scaled(CONFIGS["mixtral_decode"], T=24, d=512, F=1024))


def test_noalloc_capacity_and_many_experts():
    _both(scaled(CONFIGS["capacity_top2"], T=640, d=256, E=8, F=384))
    _both(scaled(CONFIGS["dsv3_routed"], T=48, d=512, F=256))


def test_noalloc_rejects_a_problem_over_the_limit():
    p = moe.problem_of(CONFIGS["mixtral_prefill"])
    assert moe.moe_workspace_size(p) > moe.MOE_NOALLOC_WS_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as ex:
        moe.moe_forward_noalloc(p, t, t, t, t, t, None, t)
    assert ex.value.status == 4  # MOE_ERR_WORKSPACE, refused before any launch
