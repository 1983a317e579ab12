"""MoE-layer forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 20] [--only WORKLOAD]

One step is one pass of the whole hot path (router, dispatch, grouped SwiGLU
FFN, combine; for the capacity-limited layer also the aux loss and one bias
update) over one batch of seeded synthetic tokens whose inputs and weights are
already resident in HBM.  The headline line is the Mixtral-8x7B-shaped decode
step (T=32, d=4096, E=8, K=2, F=14336, bf16).  The prefill step (T=8192,
Zipf(1.2) routing skew) runs on the same resident weights and is reported in
the "prefill" object; the DeepSeek-V3-shaped layer (T=4096, d=7168, E=256,
K=8, F=2048) and the capacity-limited layer (T=16384, d=2048, E=64, K=2,
F=1408, C=512) in "dsv3_routed" and "capacity_top2".  Each carries the
roofline of its dominant kernel and of the whole layer, against the datasheet
peaks and against the achievable peaks that two microbenchmarks measure on the
same GPU ("peaks").  The CPU oracle is timed on a bounded sample of the decode
workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec, Mixtral shape decode+prefill; % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA


# Source files whose text fixes each timed kernel (a change invalidates its counters).
KERNEL_SOURCES = {
    "decode": ["mixture_experts_layer_38_amd/csrc/kernels/ffn_decode.hip",
               "mixture_experts_layer_38_amd/csrc/device_common.h"],
    "prefill": ["mixture_experts_layer_38_amd/csrc/kernels/ffn_prefill.hip",
                "mixture_experts_layer_38_amd/csrc/kernels/ffn_tiles.h",
                "mixture_experts_layer_38_amd/csrc/device_common.h"],
    # the whole expert FFN of a large batch: the tiled GEMMs and the
    # small-expert launches (decode kernel file)
    "ffn": ["mixture_experts_layer_38_amd/csrc/kernels/ffn_prefill.hip",
            "mixture_experts_layer_38_amd/csrc/kernels/ffn_tiles.h",
            "mixture_experts_layer_38_amd/csrc/kernels/ffn_decode.hip",
            "mixture_experts_layer_38_amd/csrc/kernels/ffn.hip",
            "mixture_experts_layer_38_amd/csrc/device_common.h"],
}


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, family: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the same counters on a
    plain copy of known size; None when the summary is missing or was taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash(family):
        return None
    return rec.get("hbm_bytes_per_launch")


def gate_up_algorithmic(cfg, counts_kept: np.ndarray):
    """Algorithmic bytes and flops of one gate/up GEMM step: the W1 and W3 rows
    of every expert with at least one kept row, each read once, plus the
    grouped token rows read and the activation rows written.  The step's time
    covers every launch it takes (tiled GEMM and small-expert launch)."""
    S = int(counts_kept.sum())
    active = int((counts_kept > 0).sum())
    b = cfg.elem_bytes
    bytes_ = active * 2 * cfg.F * cfg.d * b + S * cfg.d * b + S * cfg.F * b
    flops = 2.0 * S * 2 * cfg.d * cfg.F
    return bytes_, flops


def ffn_algorithmic(cfg, counts_kept: np.ndarray):
    """Algorithmic bytes and flops of the whole expert FFN (both GEMMs, every
    launch): W1, W3 and W2 of every expert with at least one kept row, each
    read once, plus the grouped token rows read and the expert output rows
    written (the activation rows between the GEMMs are an intermediate)."""
    S = int(counts_kept.sum())
    active = int((counts_kept > 0).sum())
    b = cfg.elem_bytes
    bytes_ = active * 3 * cfg.F * cfg.d * b + 2 * S * cfg.d * b
    flops = 2.0 * S * 3 * cfg.d * cfg.F
    return bytes_, flops


def layer_algorithmic(cfg, counts_kept: np.ndarray):
    """Algorithmic bytes and flops of the whole layer (router + experts)."""
    S = int(counts_kept.sum())
    active = int((counts_kept > 0).sum())
    b = cfg.elem_bytes
    bytes_ = active * 3 * cfg.F * cfg.d * b + 2 * cfg.T * cfg.d * b + cfg.d * cfg.E * b
    flops = 2.0 * cfg.T * cfg.d * cfg.E + 2.0 * S * 3 * cfg.d * cfg.F
    return bytes_, flops


def make_pass(cfg, layer, x, bias, y):
    """One pass of the whole hot path over the resident batch: the layer, and
    for a workload with a bias-update step also the aux loss and one update of
    the balancing bias (from the pass's counts and probability sums)."""
    import torch
    if cfg.alpha is None:
        return lambda: layer.forward(x, bias, y=y)
    extra = {"counts": torch.empty(cfg.E, dtype=torch.int32, device="cuda"),
             "prob_sum": torch.empty(cfg.E, dtype=torch.float32, device="cuda")}
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    beta = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")

    def run():
        layer.forward(x, bias, y=y, dbg=extra)
        layer.aux_loss(extra["counts"], extra["prob_sum"], out=aux)
        layer.bias_update(extra["counts"], cfg.alpha, beta)
    return run


def time_workload(cfg, layer, x, bias, steps: int, warmup: int, kernel: str, use_graph: bool = False):
    """Time `steps` passes of the whole hot path (after `warmup` untimed ones),
    each over the resident batch.  With use_graph the pass is captured once in
    a HIP graph and replayed (the library's launches are capture-safe: no
    allocation, no memset, no host synchronisation).  The dominant kernel's
    launch time is then measured over `steps` eager passes with HIP events
    recorded on the kernel's own stream (outside the timed region); the same
    eager passes give the spread of the per-pass device time (HIP events
    around each pass: p10, median, p90)."""
    import torch
    import mixture_experts_layer_38_amd as moe
    y = torch.empty((cfg.T, cfg.d), dtype=layer.torch_dtype, device="cuda")
    dbg = layer.alloc_debug()
    layer.forward(x, bias, y=y, dbg=dbg)
    torch.cuda.synchronize()
    kept = dbg["kept"].cpu().numpy()
    counts = dbg["counts"].cpu().numpy()
    del dbg
    one_pass = make_pass(cfg, layer, x, bias, y)
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_pass()  # first launches set kernel attributes
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        run = graph.replay
    else:
        run = one_pass
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # dominant kernel: eager passes with the library's timing hook
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in starts + stops:  # materialise the underlying hipEvent_t
        e.record()
    torch.cuda.synchronize()
    step_a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    step_b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    keep = moe.moe_set_kernel_timer(kernel, starts, stops)
    for i in range(steps):
        step_a[i].record()
        one_pass()
        step_b[i].record()
    torch.cuda.synchronize()
    n_rec = moe.moe_kernel_timer_count(kernel)
    moe.moe_set_kernel_timer(kernel, [], [])
    del keep
    kern_ms = [starts[i].elapsed_time(stops[i]) for i in range(n_rec)]
    step_ms = np.array([step_a[i].elapsed_time(step_b[i]) for i in range(steps)])
    spread = {"p10": float(np.percentile(step_ms, 10)), "median": float(np.median(step_ms)),
              "p90": float(np.percentile(step_ms, 90)), "passes": int(steps)}
    return wall, float(np.mean(kern_ms)) if kern_ms else float("nan"), counts, kept, spread


def workload_record(cfg, layer, x, bias, steps: int, warmup: int, use_graph: bool, peaks: dict,
                    kernel: str = "ffn_gate_up"):
    """Throughput of one workload with the roofline of its dominant kernel and
    of the whole layer.  The dominant kernel is the gate/up GEMM (kernel
    "ffn_gate_up"), or the whole expert FFN ("ffn": both GEMMs with every
    launch, the small-expert launches included).  The
    bound is the MFMA peak when its arithmetic intensity is above the ridge
    point of the two peaks, else HBM."""
    wall, k_ms, counts, kept, spread = time_workload(cfg, layer, x, bias, steps, warmup, kernel, use_graph)
    ms = wall / steps * 1e3
    gb, gf = (ffn_algorithmic if kernel == "ffn" else gate_up_algorithmic)(cfg, kept)
    lb, lf = layer_algorithmic(cfg, kept)
    family = "decode" if cfg.T <= 64 else ("ffn" if kernel == "ffn" else "prefill")
    traffic = load_traffic(cfg.name, kernel, family)
    if gf / gb > MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = gf / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kernel, "achieved": ach, "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFS, "traffic": traffic, "kernel_ms": k_ms,
                "algorithmic_flops": gf}
        if peaks.get("mfma_bf16_TFs"):
            roof["frac_of_achievable"] = ach / peaks["mfma_bf16_TFs"]
        lay = {"mfma_frac": lf / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS}
    else:
        ach = gb / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kernel, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic, "kernel_ms": k_ms,
                "algorithmic_bytes": gb}
        if peaks.get("hbm_read_GBs"):
            roof["frac_of_achievable"] = ach / peaks["hbm_read_GBs"]
        lay = {"hbm_frac": lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if peaks.get("hbm_read_GBs"):
            lay["hbm_frac_of_achievable"] = lb / (ms * 1e-3) / 1e9 / peaks["hbm_read_GBs"]
    avg = cfg.T * cfg.K / cfg.E
    lay.update(algorithmic_bytes=lb, algorithmic_flops=lf)
    rec = {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} K={cfg.K} F={cfg.F} {cfg.dtype}"
                       + (f" C={cfg.capacity}" if cfg.capacity >= 0 else ""),
           "value": cfg.T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": steps,
           "roofline": roof, "step_ms": spread, "layer": lay,
           "routing": {"counts_max_over_avg": float(counts.max() / avg), "counts_min": int(counts.min()),
                       "counts_max": int(counts.max()), "kept_rows": int(kept.sum()),
                       "dropped_rows": int(counts.sum() - kept.sum()),
                       "active_experts": int((kept > 0).sum())}}
    if cfg.E <= 16:
        rec["routing"]["counts"] = counts.tolist()
    return rec


def time_chunked(cfg, layer, x, bias, chunk: int, steps: int):
    """The same prefill batch through moe_forward_chunked (chunks of `chunk`
    tokens, one workspace of one chunk's size): step time and workspace bytes
    against the unchunked layer."""
    import torch
    import mixture_experts_layer_38_amd as moe
    p = layer.p
    ws_bytes = moe.moe_forward_chunked_workspace_size(p, chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.T, cfg.d), dtype=layer.torch_dtype, device="cuda")

    def run():
        moe.moe_forward_chunked(p, chunk, x, layer.w_router, layer.w1, layer.w3, layer.w2, bias, y, ws)
    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    return {"chunk_tokens": chunk, "ms_per_step": ms, "value": cfg.T / (ms * 1e-3), "unit": "tokens/s",
            "workspace_bytes": ws_bytes, "workspace_bytes_unchunked": moe.moe_workspace_size(p)}


def _event_ms(fn, reps: int) -> float:
    """Mean milliseconds of fn() over reps back-to-back calls (HIP events on the current stream)."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _kernel_ms(kernel: str, fn, reps: int) -> float:
    """Mean milliseconds of the library kernel `kernel` over reps calls of fn()
    (HIP events recorded by the library's timing hook); NaN if it never ran."""
    import torch
    import mixture_experts_layer_38_amd as moe
    fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for e in starts + stops:
        e.record()
    torch.cuda.synchronize()
    keep = moe.moe_set_kernel_timer(kernel, starts, stops)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    n = moe.moe_kernel_timer_count(kernel)
    moe.moe_set_kernel_timer(kernel, [], [])
    del keep
    return float(np.mean([starts[i].elapsed_time(stops[i]) for i in range(n)])) if n else float("nan")


def time_variants(cfg, layer, x, bias, steps: int, concat: bool = True):
    """The layer's other forms on the same resident batch: the routing
    variants (bias for selection only, unweighted mean), the router
    regularisers, and the concatenation combine (K outputs concatenated, one
    linear layer [d, K*d]) with its roofline."""
    import torch
    import mixture_experts_layer_38_amd as moe
    from mixture_experts_layer_38_amd.layer import MoELayer
    out = {}
    y = torch.empty((cfg.T, cfg.d), dtype=layer.torch_dtype, device="cuda")
    for name, flags in (("bias_select_only", moe.MOE_FLAG_BIAS_SELECT_ONLY), ("mean_combine", moe.MOE_FLAG_COMBINE_MEAN)):
        v = MoELayer(cfg.T, cfg.d, cfg.E, cfg.K, cfg.F, cfg.dtype, layer.w_router, layer.w1, layer.w3, layer.w2,
                     cfg.capacity, flags=flags)
        ms = _event_ms(lambda: v.forward(x, bias, y=y), steps)
        out[name] = {"ms_per_step": ms, "value": cfg.T / (ms * 1e-3), "unit": "tokens/s"}
    dbg = layer.alloc_debug()
    layer.forward(x, bias, y=y, dbg=dbg)
    p = layer.p
    ws = torch.empty(moe.moe_router_losses_workspace_size(p), dtype=torch.uint8, device="cuda")
    z = torch.empty(1, dtype=torch.float32, device="cuda")
    a = torch.empty(1, dtype=torch.float32, device="cuda")
    ms = _event_ms(lambda: moe.moe_router_losses(p, dbg["logits"], bias, dbg["topk_ids"], dbg["counts"], z, a, ws),
                   steps)
    # Inside the layer the routing kernel gathers both regularisers from its
    # own softmax; what they add is the routing kernel's extra time plus (on
    # the batched path) one small reduce kernel, both timed with HIP events.
    with_l = {"z_loss": z, "aux_topk": a}
    r0 = _kernel_ms("router", lambda: layer.forward(x, bias, y=y), steps)
    r1 = _kernel_ms("router", lambda: layer.forward(x, bias, y=y, dbg=with_l), steps)
    red = _kernel_ms("router_losses", lambda: layer.forward(x, bias, y=y, dbg=with_l), steps)
    out["router_losses"] = {"us_per_call": (r1 - r0 + (red if red == red else 0.0)) * 1e3,
                            "inside_layer": {"route_kernel_us": r0 * 1e3, "route_kernel_with_losses_us": r1 * 1e3,
                                             "reduce_us": red * 1e3 if red == red else 0.0},
                            "standalone_us_per_call": ms * 1e3}
    if concat:
        g = torch.Generator(device="cuda").manual_seed(11)
        S, dk = cfg.T * cfg.K, cfg.K * cfg.d
        h = torch.randn(S, cfg.d, device="cuda", generator=g).to(layer.torch_dtype)
        w_cat = (torch.randn(cfg.d, dk, device="cuda", generator=g) / dk ** 0.5).to(layer.torch_dtype)
        cws = torch.empty(moe.moe_combine_concat_workspace_size(p), dtype=torch.uint8, device="cuda")
        ms = _event_ms(lambda: moe.moe_combine_concat(p, h, dbg["assign_row"], w_cat, y, cws), steps)
        es = h.element_size()
        nbytes = (cfg.d * dk + S * cfg.d + cfg.T * cfg.d) * es
        flops = 2.0 * cfg.T * dk * cfg.d
        rec = {"us_per_call": ms * 1e3, "algorithmic_bytes": nbytes, "algorithmic_flops": flops}
        if cfg.T <= 64:
            rec["roofline"] = {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        else:
            rec["roofline"] = {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFS,
                               "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS}
        out["concat_combine"] = rec
    if cfg.T <= 64:
        out["skewed_routing"] = time_skewed_decode(cfg, layer, steps)
    return out


def time_skewed_decode(cfg, layer, steps: int):
    """The decode step on the same weights under a skewed routing: a Zipf(1.2)
    per-expert logit offset (the prefill batch's skew) at T = 32 and T = 64
    tokens, with fresh N(0, 1) token rows.  Experts then hold up to 64 rows,
    which the decode kernels take in passes of 16, 32 or 64 token rows."""
    import torch
    from mixture_experts_layer_38_amd.layer import MoELayer
    from mixture_experts_layer_38_amd.configs import scaled
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    pz = r ** -1.2
    bias = torch.from_numpy(np.log(pz / pz.sum()).astype(np.float32)).cuda()
    g = torch.Generator(device="cuda").manual_seed(12)
    out = {}
    for T in (32, 64):
        scfg = scaled(cfg, T=T, skew="zipf", zipf_s=1.2)
        x = torch.randn(T, cfg.d, device="cuda", generator=g).to(layer.torch_dtype)
        v = MoELayer(T, cfg.d, cfg.E, cfg.K, cfg.F, cfg.dtype, layer.w_router, layer.w1, layer.w3, layer.w2,
                     cfg.capacity)
        y = torch.empty((T, cfg.d), dtype=layer.torch_dtype, device="cuda")
        dbg = v.alloc_debug()
        v.forward(x, bias, y=y, dbg=dbg)
        torch.cuda.synchronize()
        kept = dbg["kept"].cpu().numpy()
        ms = _event_ms(lambda: v.forward(x, bias, y=y), steps)
        lb, _ = layer_algorithmic(scfg, kept)
        out[f"zipf1.2_t{T}"] = {"ms_per_step": ms, "value": T / (ms * 1e-3), "unit": "tokens/s",
                                "counts": dbg["counts"].cpu().numpy().tolist(),
                                "layer_hbm_frac": lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, min_seconds: float = 10.0, max_reps: int = 200):
    """The CPU oracle (fp64, OpenMP on this host's cores) on the same workload:
    whole forward passes of the first min(T, 32) tokens (routing, grouping,
    SwiGLU experts and combine), repeated until at least `min_seconds` of CPU
    work have been timed."""
    import oracle
    orc = oracle.get()
    n_tokens = min(cfg.T, 32)
    toks = np.arange(n_tokens, dtype=np.int64)
    x = np.ascontiguousarray(inp["x"][:n_tokens])
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.forward(x, inp["w_router"], inp["w1"], inp["w3"], inp["w2"], cfg.K,
                    inp["logit_bias"], cfg.capacity, toks)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    return {"value": reps * n_tokens / dt, "unit": "tokens/s", "cores": orc.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": dt,
            "sample": f"{reps} full forward passes of {n_tokens} tokens of {cfg.name} "
                      f"(router, routing, grouping, fp64 SwiGLU experts and combine)"}


def measure_peaks() -> dict:
    """Achievable HBM read rate and dense bf16 MFMA rate on this GPU
    (libmoepeaks.so microbenchmarks), beside the datasheet peaks."""
    from mixture_experts_layer_38_amd import peaks
    gbs, blocks = peaks.hbm_read_gbs()
    return {"hbm_read_GBs": gbs, "mfma_bf16_TFs": peaks.mfma_bf16_tfs(),
            "datasheet": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFs": MFMA_BF16_PEAK_TFS},
            "probes": f"stream read of 4 GiB (plain 16-byte loads, 8 in flight per thread, contiguous "
                      f"32 KB pieces per workgroup; best of 256-4096 workgroups: {blocks}); "
                      "100000 rounds of 8 independent 32x32x16 bf16 MFMAs per wave on random "
                      "register operands, 4 waves per SIMD"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None, choices=[None, "mixtral_decode", "mixtral_prefill", "dsv3_routed",
                                                     "capacity_top2"],
                    help="time one workload only (its object becomes the line's headline fields)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--other-steps", type=int, default=20, help="steps of the DeepSeek-V3-shaped and capacity layers")
    ap.add_argument("--prefill-chunk", type=int, default=2048)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the routing/combine variants and router losses")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per pass instead of launching eagerly "
                         "(measured about 1%% slower on the decode step)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_38_amd as moe
    from mixture_experts_layer_38_amd import datagen
    from mixture_experts_layer_38_amd.configs import CONFIGS
    from mixture_experts_layer_38_amd.layer import MoELayer, to_device

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    moe.load()
    want = (lambda n: args.only is None or args.only == n)
    peaks_rec = {}
    if not args.no_peaks:
        log("measuring the achievable HBM read and bf16 MFMA rates")
        peaks_rec = measure_peaks()
    records = {}
    cfg = CONFIGS["mixtral_decode"]
    inp = None
    if want("mixtral_decode") or want("mixtral_prefill"):
        log("generating the Mixtral-shaped inputs")
        inp = datagen.make_inputs(cfg)
        layer = MoELayer.from_host(cfg, inp)
        x = to_device(inp["x"], cfg.dtype)
        if want("mixtral_decode"):
            log("timing mixtral_decode")
            records["mixtral_decode"] = workload_record(cfg, layer, x, None, args.steps, args.warmup, args.graph,
                                                        peaks_rec)
            if not args.no_variants:
                log("timing the decode variants")
                records["mixtral_decode"]["variants"] = time_variants(cfg, layer, x, None, 20, concat=True)
        if want("mixtral_prefill"):
            pcfg = CONFIGS["mixtral_prefill"]
            pin = datagen.make_inputs(pcfg, with_experts=False)
            player = MoELayer(pcfg.T, pcfg.d, pcfg.E, pcfg.K, pcfg.F, pcfg.dtype, layer.w_router,
                              layer.w1, layer.w3, layer.w2, pcfg.capacity)
            px = to_device(pin["x"], pcfg.dtype)
            pb = torch.from_numpy(pin["logit_bias"]).cuda()
            log("timing mixtral_prefill")
            rec = workload_record(pcfg, player, px, pb, args.prefill_steps, 5, args.graph, peaks_rec)
            rec["chunked"] = time_chunked(pcfg, player, px, pb, args.prefill_chunk, args.prefill_steps)
            rec["chunked_4096"] = time_chunked(pcfg, player, px, pb, 4096, args.prefill_steps)
            if not args.no_variants:
                rec["variants"] = time_variants(pcfg, player, px, pb, 3)
            records["mixtral_prefill"] = rec
            del player, px
        del layer, x
        torch.cuda.empty_cache()
    for name in ("dsv3_routed", "capacity_top2"):
        if not want(name):
            continue
        ocfg = CONFIGS[name]
        log(f"generating the {name} inputs")
        oin = datagen.make_inputs(ocfg)
        olayer = MoELayer.from_host(ocfg, oin)
        ox = to_device(oin["x"], ocfg.dtype)
        ob = None if oin["logit_bias"] is None else torch.from_numpy(oin["logit_bias"]).cuda()
        del oin
        log(f"timing {name}")
        records[name] = workload_record(ocfg, olayer, ox, ob, args.other_steps, 5, args.graph, peaks_rec,
                                        kernel="ffn")
        del olayer, ox, ob
        torch.cuda.empty_cache()

    head_name = args.only or "mixtral_decode"
    head = records[head_name]
    hcfg = CONFIGS[head_name]
    steps = args.steps if head_name == "mixtral_decode" else (
        args.prefill_steps if head_name == "mixtral_prefill" else args.other_steps)
    result = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": hcfg.dtype, "data": "synthetic",
        "config": {"workload": head["workload"], "T": hcfg.T, "d_model": hcfg.d, "experts": hcfg.E,
                   "top_k": hcfg.K, "d_ff": hcfg.F, "capacity": hcfg.capacity,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "roofline": head["roofline"],
        "step_ms": head["step_ms"],
        "layer": head["layer"],
        "routing": head["routing"],
    }
    for k in ("variants", "chunked", "chunked_4096"):
        if k in head:
            result[k] = head[k]
    for name in ("mixtral_prefill", "dsv3_routed", "capacity_top2"):
        if name in records and name != head_name:
            key = "prefill" if name == "mixtral_prefill" else name
            result[key] = records[name]
    if peaks_rec:
        result["peaks"] = peaks_rec
    if not args.no_cpu and head_name == "mixtral_decode" and inp is not None:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
