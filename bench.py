"""Throughput of one tensor-parallel rank's shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra]

Headline: the LLaMA-7B MLP shard at TP=4 (X[4096,4096] bf16, gate/up [4096,2752],
down [2752,4096], fp32 partial out) — one step = one tp_mlp_shard call (fused
SiLU(gate)*up GEMM + down GEMM). `value` is shard TFLOP/s (2*M*K*N per GEMM, 277.03
GFLOP per step). Alongside: the 7B TP=2 decode step (attention shard over a 1024-token
KV cache + MLP shard at 32 tokens + vocabulary-split LM head) in GB/s of compulsory HBM
bytes, and the same MLP shard on OCP E4M3 operands (tp_mlp_shard_fp8) against the fp8
MFMA peak, and the step after the merge (tp_merge_rmsnorm: 4 fp32 partials of [8192, 4096]
summed into the bf16 residual stream, then RMSNorm) against the HBM bandwidth, and the
backward of the MLP down shard (tp_linear_backward), and a top-2 MoE MLP over 8 local
experts (tp_moe_mlp_shard, 2048 tokens; TFLOP/s of the expert MLPs). Inputs are
seeded synthetic tensors already resident in HBM. With --extra the attention shard (B=4,
S=2048) and the 70B GQA layer shard are timed too.

Prints ONE JSON line. Per-kernel durations come from HIP events that libtpshard records
around each launch on the launch stream during every 10th timed step (the events cost a few
microseconds per kernel, so they are not recorded on the other steps).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense MFMA)
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 2.4 GHz x 8192 flop/clk/CU (dense MFMA)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--extra", action="store_true", help="also time the attention and 70B layer shards")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle sample")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 2.5 s clock/power reading (for profiled runs)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (3 times): the reference that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiled run")
    return ap.parse_args()


STEP_STATS = {}


def _stats(name: str, per_step_ms):
    xs = sorted(per_step_ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    STEP_STATS[name] = {"median_ms": med, "min_ms": xs[0], "max_ms": xs[-1]}


def timed(step, warmup: int, steps: int, name: str = None, sample_every: int = 10):
    """Run warmup untimed steps, then time exactly `steps` steps; returns ms per step.

    Only two events bracket the timed steps. libtpshard's per-kernel HIP events (which add a
    few microseconds per kernel) are switched on for every `sample_every`-th timed step only,
    so the kernel averages come from inside the timed region at a cost of ~1% of it. If
    `name` is given, a second pass of `steps` steps with one event per step gives the per-step
    median / min / max (STEP_STATS[name])."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tp.profile_reset()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        sampled = i % sample_every == 0
        if sampled:
            tp.profile_enable(True)
        step()
        if sampled:
            tp.profile_enable(False)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if name:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(s)
        for i in range(steps):
            step()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        _stats(name, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return ms


def clock_power(step, seconds: float = 2.5):
    """GPU clock (MHz) and socket power (W) while `step` runs back to back for `seconds`.
    The amdgpu kernel driver refreshes its metrics table about once a second, so only readings taken after
    a refresh (a new system-clock stamp) while the load runs are kept. None if the amdsmi
    library is missing."""
    try:
        import amdsmi
    except Exception:   # noqa: BLE001
        return None
    import torch
    try:
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
        stamp0 = amdsmi.amdsmi_get_gpu_metrics_info(h).get("system_clock_counter")
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        step()
        e1.record(s)
        torch.cuda.synchronize()
        n = max(1, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
        seen, fresh = {stamp0}, []
        t0 = tlast = time.perf_counter()
        for _ in range(n):   # launches block once the queue is full, so the reads interleave
            step()
            now = time.perf_counter()
            if now - tlast > 0.05:
                tlast = now
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                st = m.get("system_clock_counter")
                if st not in seen and now - t0 > 0.5:
                    fresh.append((m.get("current_gfxclk"), m.get("current_socket_power")))
                seen.add(st)
        torch.cuda.synchronize()
        amdsmi.amdsmi_shut_down()
    except Exception as e:   # noqa: BLE001
        return {"error": str(e)}
    if not fresh:
        return {"error": "no metrics refresh during the load"}
    clk = [c for c, _ in fresh if isinstance(c, (int, float))]
    pw = [p for _, p in fresh if isinstance(p, (int, float))]
    return {"gfx_clk_mhz": (sum(clk) / len(clk)) if clk else None,
            "socket_power_w": (sum(pw) / len(pw)) if pw else None,
            "readings": len(fresh), "seconds": seconds,
            "source": "amdsmi gpu metrics (refreshed ~1/s), during back-to-back steps"}


def kernel_avg(prefix: str):
    import tensor_transformer_layer_rank_amd as tp
    ms, n = tp.profile_read(prefix)
    return (ms / n if n else None), n


def mlp_bench(args):
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.mlp7b_tp4()
    T, H, I = inp.T, inp.H, inp.I
    X, Wg, Wu, Wd = dev(inp.X), dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down)
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.mlp_workspace_size(T, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16), dtype=torch.uint8, device="cuda")

    def step():
        tp.mlp_shard(X, Wg, Wu, Wd, Y=Y, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "mlp")
    gu_ms, gu_n = kernel_avg("gemm_bf16_swiglu")
    fx_ms, fx_n = kernel_avg("fixup_swiglu")
    dn_ms, dn_n = kernel_avg("gemm_bf16_f32out")
    # the tail-split fix-up pass belongs to the gate/up GEMM: count its time per launch
    gu_main_ms = gu_ms
    if fx_n:
        gu_ms = gu_ms + fx_ms * fx_n / gu_n
    flops_gu = 2.0 * T * H * I * 2
    flops_dn = 2.0 * T * I * H
    flops = flops_gu + flops_dn
    res = {
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "flops_per_step": flops,
        "kernels": {
            "gemm_bf16_swiglu": {"avg_us": gu_ms * 1e3, "launches": gu_n,
                                 "main_avg_us": gu_main_ms * 1e3,
                                 "fixup_avg_us": (fx_ms * 1e3) if fx_n else 0.0,
                                 "tflops": flops_gu / (gu_ms * 1e-3) / 1e12},
            "gemm_bf16_f32out(down)": {"avg_us": dn_ms * 1e3, "launches": dn_n,
                                       "tflops": flops_dn / (dn_ms * 1e-3) / 1e12},
        },
        "step_stats": STEP_STATS.get("mlp"),
        "clock_power": None if args.no_clock else clock_power(step),
        "roofline": {
            "bound": "mfma", "kernel": "gemm_bf16_swiglu",
            "achieved": flops_gu / (gu_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": flops_gu / (gu_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": recorded_traffic("gemm_bf16_swiglu"),
        },
    }
    return res, inp


def fp8_mlp_bench(args):
    """The same MLP shard on OCP E4M3 codes with per-tensor scales (tp_mlp_shard_fp8)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev_codes
    inp = wl.mlp7b_tp4_fp8()
    T, H, I = inp.T, inp.H, inp.I
    X, Wg, Wu, Wd = (dev_codes(a) for a in (inp.X, inp.W_gate, inp.W_up, inp.W_down))
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.mlp_fp8_workspace_size(T, H, I, tp.TP_MLP_SWIGLU), dtype=torch.uint8, device="cuda")
    scales = (inp.x_scale, inp.wg_scale, inp.wu_scale, inp.wd_scale, inp.h_scale)

    def step():
        tp.mlp_shard_fp8(X, Wg, Wu, Wd, scales, Y=Y, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "fp8_mlp")
    gu_ms, gu_n = kernel_avg("gemm_f8_swiglu")
    fx_ms, fx_n = kernel_avg("fixup_swiglu")
    dn_ms, _ = kernel_avg("gemm_f8_f32out")
    if fx_n:
        gu_ms = gu_ms + fx_ms * fx_n / gu_n
    flops_gu = 2.0 * T * H * I * 2
    flops_dn = 2.0 * T * I * H
    tf = (flops_gu + flops_dn) / (ms * 1e-3) / 1e12
    return {
        "workload": "mlp7b_tp4_fp8: the mlp7b_tp4 shapes as OCP E4M3 codes, per-tensor fp32 scales, "
                    "h re-encoded to E4M3 with a static scale",
        "ms_per_step": ms,
        "tflops": tf,
        "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
        "step_stats": STEP_STATS.get("fp8_mlp"),
        "kernels": {"gemm_f8_swiglu(+fixup)": {"avg_us": gu_ms * 1e3, "tflops": flops_gu / (gu_ms * 1e-3) / 1e12},
                    "gemm_f8_f32out(down)": {"avg_us": dn_ms * 1e3, "tflops": flops_dn / (dn_ms * 1e-3) / 1e12}},
        "roofline": {"bound": "mfma", "kernel": "gemm_f8_swiglu", "achieved": flops_gu / (gu_ms * 1e-3) / 1e12,
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops_gu / (gu_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                     "traffic": recorded_traffic("gemm_f8_swiglu")},
    }


def merge_bench(args):
    """The step after the merge (tp_merge_rmsnorm): 4 fp32 partials of [8192, 4096] summed
    into the bf16 residual stream, then RMSNorm; HBM-bound."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.merge7b_tp4()
    T, H, k = inp.T, inp.H, len(inp.partials)
    parts = [dev(p, "f32") for p in inp.partials]
    res, gamma = dev(inp.residual), dev(inp.gamma)
    R = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    N = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        tp.merge_rmsnorm(parts, res, gamma, inp.eps, residual_out=R, normed=N)

    ms = timed(step, args.warmup, args.steps, "merge")
    k_ms, _ = kernel_avg("merge_rmsnorm")
    nbytes = float(T * H * (4 * k + 2 + 2 + 2) + 2 * H)   # partials, residual, 2 outputs, gain
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    return {
        "workload": "merge7b_tp4: 4 fp32 partials [8192,4096] + bf16 residual -> bf16 residual, bf16 RMSNorm(eps 1e-5)",
        "ms_per_step": ms,
        "gbs": nbytes / (ms * 1e-3) / 1e9,
        "step_stats": STEP_STATS.get("merge"),
        "roofline": {"bound": "hbm", "kernel": "merge_rmsnorm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": recorded_traffic("merge_rmsnorm"),
                     "bytes_per_launch": nbytes},
    }


def backward_bench(args):
    """Backward of the 7B TP=4 MLP down shard (tp_linear_backward: dX = dY.W^T, dW = X^T.dY
    after the bf16 transposes of W and X)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.backward7b_tp4()
    T, K = inp.X.shape
    N = inp.W.shape[1]
    X, W, dY = dev(inp.X), dev(inp.W), dev(inp.dY)
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dW = torch.empty((K, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.linear_backward_workspace_size(T, K, N), dtype=torch.uint8, device="cuda")

    def step():
        tp.linear_backward(X, W, dY, dX=dX, dW=dW, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "backward")
    flops = 4.0 * T * K * N
    g_ms, g_n = kernel_avg("gemm_bf16_f32out")
    t_ms, t_n = kernel_avg("transpose_bf16")
    fx_ms, fx_n = kernel_avg("fixup_gemm")
    g_ms, t_ms, fx_ms = g_ms or 0.0, t_ms or 0.0, fx_ms or 0.0
    sampled = len(range(0, args.steps, 10))
    gemm_ms = (g_ms * g_n + fx_ms * fx_n) / sampled       # both products (one paired launch when N == T)
    gemm_tf = flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    return {
        "workload": "backward7b_tp4: X = h [4096,2752], W_down shard [2752,4096], dY [4096,4096] bf16 -> dX, dW fp32",
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "step_stats": STEP_STATS.get("backward"),
        "kernels": {"gemm (dX and dW per step, incl. tail fix-up)": {"us_per_step": gemm_ms * 1e3,
                                                                    "launches_per_step": g_n / sampled,
                                                                    "tflops": gemm_tf},
                    "transpose_bf16 (W, X)": {"avg_us": t_ms * 1e3, "launches_per_step": t_n / sampled}},
    }


def moe_bench(args):
    """Top-2 MoE MLP on one rank (tp_moe_mlp_shard): 2048 tokens, 8 local experts whose SwiGLU
    MLPs are TP=4 shards (H 4096, I 3584); gather, per-expert gate/up + down, gated combine."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.moe8x7b_tp4()
    T, H = inp.X.shape
    I = inp.W_gate.shape[2]
    R = int(inp.expert_offsets[-1])
    X, Wg, Wu, Wd = dev(inp.X), dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down)
    rt = torch.from_numpy(inp.row_token.copy()).cuda()
    tr = torch.from_numpy(inp.token_rows.copy()).cuda()
    gates = dev(inp.gates, "f32")
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tp.moe_workspace_size(T, H, I, inp.expert_offsets), 1), dtype=torch.uint8, device="cuda")

    def step():
        tp.moe_mlp_shard(X, Wg, Wu, Wd, inp.expert_offsets, rt, tr, gates, Y=Y, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "moe")
    flops = 6.0 * R * H * I
    kern = {}
    for name in ("moe_gather", "gemm_bf16_swiglu", "fixup_swiglu", "gemm_bf16_f32out", "fixup_gemm",
                 "skinny", "moe_combine"):
        k_ms, k_n = kernel_avg(name)
        if k_n:
            kern[name] = {"avg_us": k_ms * 1e3, "launches_per_step": k_n / len(range(0, args.steps, 10))}
    return {
        "workload": f"moe8x7b_tp4: T={T} tokens, top-2 of 8 experts ({R} dispatched rows), "
                    f"expert shards gate/up [{H},{I}], down [{I},{H}] bf16 -> fp32 partial",
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "flops_per_step": flops,
        "step_stats": STEP_STATS.get("moe"),
        "kernels": kern,
    }


def graph_timed(step, warmup: int, steps: int, name: str = None):
    """Capture one step into a HIP graph (torch.cuda.CUDAGraph) and time `steps` replays
    between two events; a second pass with one event per replay gives the per-replay median
    and minimum (STEP_STATS[name])."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if name:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        _stats(name, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return ms


def decode_bench(args):
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.decode7b_tp2()
    B, H, hq, hkv, L = inp.B, inp.H, inp.hq, inp.hkv, inp.cache_len + 1
    X = dev(inp.X)
    Wqkv, Wo, Wg, Wu, Wd, Wlm = (dev(w) for w in (inp.W_qkv, inp.W_o, inp.W_gate, inp.W_up, inp.W_down, inp.W_lm))
    kc, vc = dev(inp.k_cache), dev(inp.v_cache)
    I, V = inp.W_gate.shape[1], inp.W_lm.shape[1]
    Ya = torch.empty((B, H), dtype=torch.float32, device="cuda")
    Ym = torch.empty((B, H), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, V), dtype=torch.float32, device="cuda")
    ws_a = torch.empty(tp.attn_workspace_size(B, 1, H, hq, hkv, inp.theta, kc, vc, inp.cache_len),
                       dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(tp.mlp_workspace_size(B, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16), dtype=torch.uint8, device="cuda")
    ws_l = torch.empty(tp.linear_workspace_size(B, H, V, tp.TP_BF16), dtype=torch.uint8, device="cuda")

    def step():
        tp.attn_shard(X, Wqkv, Wo, B, 1, hq, hkv, inp.theta, k_cache=kc, v_cache=vc,
                      cache_len=inp.cache_len, Y=Ya, workspace=ws_a)
        tp.mlp_shard(X, Wg, Wu, Wd, Y=Ym, workspace=ws_m)
        tp.column_linear(X, Wlm, Y=logits, workspace=ws_l)

    # the three parts are independent: in the graph they are branches on their own streams
    # (default priority), joined at the end of the step
    s_attn, s_mlp = torch.cuda.Stream(), torch.cuda.Stream()

    def step_branches():
        cur = torch.cuda.current_stream()
        s_attn.wait_stream(cur)
        s_mlp.wait_stream(cur)
        with torch.cuda.stream(s_attn):
            tp.attn_shard(X, Wqkv, Wo, B, 1, hq, hkv, inp.theta, k_cache=kc, v_cache=vc,
                          cache_len=inp.cache_len, Y=Ya, workspace=ws_a)
        with torch.cuda.stream(s_mlp):
            tp.mlp_shard(X, Wg, Wu, Wd, Y=Ym, workspace=ws_m)
        tp.column_linear(X, Wlm, Y=logits, workspace=ws_l)
        cur.wait_stream(s_attn)
        cur.wait_stream(s_mlp)

    ms_eager = timed(step, args.warmup, args.steps)       # per-kernel HIP-event timing
    ms_serial = graph_timed(step, args.warmup, args.steps)
    ms = graph_timed(step_branches, args.warmup, args.steps, "decode")   # the step as one HIP graph
    d = 128
    w_bytes = 2 * (H * (hq + 2 * hkv) * d + hq * d * H + 2 * H * I + I * H + H * V)
    kv_bytes = 2 * 2 * B * hkv * (L - 1) * d          # cached keys and values read once
    new_kv = 2 * 2 * B * hkv * d                       # the new key/value written (and read back)
    act = 2 * B * H + 4 * (2 * B * H + B * V)          # X in; two fp32 partials and the logits out
    total = w_bytes + kv_bytes + 2 * new_kv + act
    att_ms, att_n = kernel_avg("decode_attn")
    sk_ms, sk_n = kernel_avg("skinny_gemm")
    return {
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "ms_per_step_graph_serial": ms_serial,
        "step_stats": STEP_STATS.get("decode"),
        "graph": "one HIP graph per step: attention, MLP and LM-head branches on separate streams",
        "bytes_per_step": total,
        "gbs": total / (ms * 1e-3) / 1e9,
        "frac_hbm": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels": {"decode_attn(avg_us)": att_ms * 1e3 if att_ms else None,
                    "skinny_gemm*(avg_us)": sk_ms * 1e3 if sk_ms else None,
                    "skinny_gemm*(launches/step)": sk_n / max(-(-args.steps // 10), 1)},
        "workload": "decode7b_tp2: B=32 one token each, 16 local heads (MHA), KV cache 1024 tokens, "
                    "H=4096, I_shard=5504, LM head [4096,16000]",
    }


def attn_bench(args, name):
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from tests._util import dev
    inp = wl.WORKLOADS[name]()
    B, S, H, hq, hkv = inp.B, inp.S, inp.H, inp.hq, inp.hkv
    X, Wqkv, Wo = dev(inp.X), dev(inp.W_qkv), dev(inp.W_o)
    T = B * S
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.attn_workspace_size(B, S, H, hq, hkv, inp.theta), dtype=torch.uint8, device="cuda")
    mlp = None
    if inp.mlp is not None:
        m = inp.mlp
        I = m.W_gate.shape[1]
        mlp = (dev(m.W_gate), dev(m.W_up), dev(m.W_down),
               torch.empty((T, H), dtype=torch.float32, device="cuda"),
               torch.empty(tp.mlp_workspace_size(T, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16), dtype=torch.uint8, device="cuda"))

    def step():
        tp.attn_shard(X, Wqkv, Wo, B, S, hq, hkv, inp.theta, Y=Y, workspace=ws)
        if mlp:
            tp.mlp_shard(X, mlp[0], mlp[1], mlp[2], Y=mlp[3], workspace=mlp[4])

    ms = timed(step, max(2, args.warmup // 2), max(5, args.steps // 2))
    d = 128
    f_qkv = 2.0 * T * H * (hq + 2 * hkv) * d
    f_att = 2.0 * 2 * d * B * hq * S * (S + 1) / 2      # causal triangle only: QK^T and PV
    f_o = 2.0 * T * hq * d * H
    f_mlp = 0.0
    if inp.mlp is not None:
        I = inp.mlp.W_gate.shape[1]
        f_mlp = 2.0 * T * H * I * 3
    flops = f_qkv + f_att + f_o + f_mlp
    fa_ms, _ = kernel_avg("flash_attn_fwd")
    q_ms, _ = kernel_avg("gemm_bf16_qkv_rope")
    return {"ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "flash_attn_tflops": f_att / (fa_ms * 1e-3) / 1e12 if fa_ms else None,
            "qkv_rope_tflops": f_qkv / (q_ms * 1e-3) / 1e12 if q_ms else None}


def traffic_probe():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    import torch
    a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was taken on
    the current kernel source (profiles/traffic.json records the source file's hash)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[kernel]
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
            return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(inp, target_s: float):
    """The fp64 oracle on a row sample of the same MLP shard, on this host's cores."""
    import numpy as np
    import oracle as O
    rows0 = 32
    t0 = time.perf_counter()
    O.mlp_swiglu_shard(inp.X[:rows0], inp.W_gate, inp.W_up, inp.W_down)
    t_small = time.perf_counter() - t0
    rows = int(min(inp.T, max(rows0, rows0 * target_s / max(t_small, 1e-3))))
    rows = max(rows0, rows - rows % 32)
    # the whole shard may take less than the target: repeat it (same rows) to about target_s
    t0 = time.perf_counter()
    O.mlp_swiglu_shard(inp.X[:rows], inp.W_gate, inp.W_up, inp.W_down)
    first = time.perf_counter() - t0
    reps = max(1, min(60, int(target_s / max(first, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        O.mlp_swiglu_shard(inp.X[:rows], inp.W_gate, inp.W_up, inp.W_down)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * inp.H * inp.I * 3 * reps
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    cores = threads or len(os.sched_getaffinity(0))
    cpu_model, blas = None, None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version', '')}".strip()
    except Exception:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model, "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas,
            "sample": f"fp64 NumPy oracle on rows 0..{rows - 1} of the 4096-row MLP shard, {reps} run(s) "
                      f"({flops / 1e9:.1f} GFLOP in {dt:.2f} s)",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU: one rank's shard; "
                                   "run with --gpus 1 (multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    import tensor_transformer_layer_rank_amd as tp
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    tp.load()
    mlp, inp = mlp_bench(args)
    dec = decode_bench(args)
    fp8 = fp8_mlp_bench(args)
    merge = merge_bench(args)
    bwd = backward_bench(args)
    moe = moe_bench(args)
    extra = {}
    if args.extra:
        extra["attn7b_tp4"] = attn_bench(args, "attn7b_tp4")
        extra["layer70b_tp8"] = attn_bench(args, "layer70b_tp8")
    if args.traffic_probe:
        traffic_probe()
    cpu = None if args.no_cpu else cpu_baseline(inp, args.cpu_seconds)
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": "shard TFLOP/s (+% bf16 MFMA peak) for 7B TP=4 MLP; decode GB/s (%HBM)",
        "value": round(mlp["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mlp["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, bf16-rounded)",
        "config": {"workload": "mlp7b_tp4: LLaMA-7B MLP shard at TP=4, X[4096,4096] (B=8,S=512), "
                               "gate/up [4096,2752], down [2752,4096], fp32 partial out",
                   "frac_bf16_peak": round(mlp["tflops"] / PEAK_BF16_TFLOPS, 4),
                   "decode_gbs": round(dec["gbs"], 1),
                   "decode_frac_hbm": round(dec["frac_hbm"], 4),
                   "decode_ms_per_step": round(dec["ms_per_step"], 5)},
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in mlp["roofline"].items()},
        "cpu_baseline": cpu and {k: v for k, v in cpu.items() if k != "seconds"},
        "step_stats": mlp["step_stats"],
        "clock_power": mlp["clock_power"],
        "kernels": mlp["kernels"],
        "decode": dec,
        "fp8_mlp": fp8,
        "merge_rmsnorm": merge,
        "backward": bwd,
        "moe": moe,
        "extra": extra or None,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", None)},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
