"""Throughput of one tensor-parallel rank's shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline: the LLaMA-7B MLP shard at TP=4 (X[4096,4096] bf16, gate/up [4096,2752],
down [2752,4096], fp32 partial out) — one step = one tp_mlp_shard call (fused
SiLU(gate)*up GEMM + down GEMM). `value` is shard TFLOP/s (2*M*K*N per GEMM, 277.03
GFLOP per step). Every workload of the shard is timed in the same run, each checked
element by element against the fp64 oracle afterwards, with the oracle's own time on
this host's cores:
  c0 the integer fp32 TP=2 MLP, both ranks in turn plus the partial sum (latency, bit-exact);
  c1 the 7B TP=4 MLP shard (headline);
  c2 the 7B TP=4 attention shard (B=4, S=2048, 8 heads: QKV + RoPE, flash attention, O);
  c3 the 70B TP=8 GQA layer shard (attention with 8 q heads / 1 kv head, plus the MLP shard);
  c4 the 7B TP=2 decode step (attention over a 1024-token KV cache + MLP at 32 tokens +
     vocabulary-split LM head, one HIP graph) in GB/s of compulsory HBM bytes, with the
     weights packed once into 128-column strips (tp_pack_strips, outside the timed region);
     the step on the weights in place is timed beside it.
Beside them: the MLP shard on OCP E4M3 operands (tp_mlp_shard_fp8), the step after the
merge (tp_merge_rmsnorm), the backward of the MLP down shard (tp_linear_backward) and a
top-2 MoE MLP over 8 local experts (tp_moe_mlp_shard); and two ceilings measured on the box:
the matrix pipes' rate under the power limit (tp_mfma_rate_probe) and the HBM read rate of
the decode GEMMs' access pattern (tp_hbm_read_probe). Inputs are seeded synthetic tensors
already resident in HBM when timing starts.

Prints ONE JSON line. Each leg's timed steps are bracketed by events recorded after every
step (per-step times come from the timed pass). Per-kernel durations come from HIP events
that libtpshard records around each launch on the launch stream during every 10th timed
step (they cost a few microseconds per kernel, so the other steps run without them).
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
    ap.add_argument("--prewarm", type=float, default=1.5,
                    help="seconds of untimed back-to-back headline steps before the first leg (clock settling)")
    ap.add_argument("--no-parity", action="store_true", help="skip the element-wise oracle comparison")
    ap.add_argument("--legs", default="all",
                    help="comma-separated subset of c0,c1,c2,c3,c4,fp8,merge,backward,moe,ceiling,hbm (profiling runs); "
                         "the headline needs c1")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle sample")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 2.5 s clock/power reading (for profiled runs)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (3 times): the reference that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiled run")
    return ap.parse_args()


STEP_STATS = {}
PREWARM = {}


def _stats(name: str, per_step_ms):
    xs = sorted(per_step_ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    STEP_STATS[name] = {"median_ms": med, "min_ms": xs[0], "max_ms": xs[-1],
                        "first_ms": per_step_ms[0], "last_ms": per_step_ms[-1]}


def prewarm(step, seconds: float):
    """Run `step` back to back for about `seconds` before anything is timed. From an idle GPU the
    clock takes far longer than a few short steps to settle (it ramps under load and then falls
    to what the board's power limit allows), so without this the first timed steps of the first
    leg run at a different clock than the rest. Untimed; its length is reported."""
    import torch
    if seconds <= 0:
        return 0
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()
    return n


class TimingEvent:
    """A HIP event for timing only, recorded on a torch stream (the current one by default).
    Created with hipEventDisableSystemFence: recording it does not write back and invalidate the
    caches at system scope, which a default event does (torch.cuda.Event), costing microseconds
    per record and slowing the kernels after it. Same interface as torch.cuda.Event for timing."""
    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            import torch  # noqa: F401  (loads the HIP runtime that torch and libtpshard share)
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = h
        self._ct = ctypes
        self.e = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.e), 0x20000000)   # hipEventDisableSystemFence
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = TimingEvent._hip.hipEventRecord(self.e, self._ct.c_void_p(s.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, other) -> float:
        ms = self._ct.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.e, other.e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if TimingEvent._hip is not None and self.e:
            TimingEvent._hip.hipEventDestroy(self.e)


def timed(step, warmup: int, steps: int, name: str = None, sample_every: int = 10, keep_steps: bool = False):
    """Run `warmup` untimed steps, then time exactly `steps` steps; returns ms per step.

    The timed region is bracketed by the first and last of steps+1 events, one recorded after
    each step, so the per-step times come from the timed pass itself (STEP_STATS[name]; the whole
    list when keep_steps). libtpshard's per-kernel HIP events (a few microseconds per kernel) are
    switched on for every `sample_every`-th timed step only, starting with the step after the
    first, so the kernel averages come from inside the timed region (sample_every = 0: never)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tp.profile_reset()
    s = torch.cuda.current_stream()
    ev = [TimingEvent() for _ in range(steps + 1)]
    ev[0].record(s)
    for i in range(steps):
        sampled = sample_every > 0 and (i % sample_every == sample_every - 1 or
                                        (steps < sample_every and i == steps - 1))
        if sampled:
            tp.profile_enable(True)
        step()
        if sampled:
            tp.profile_enable(False)
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    if name:
        _stats(name, per)
        if keep_steps:
            STEP_STATS[name]["per_step_ms"] = [round(x, 5) for x in per]
    return ms


def sampled_steps(steps: int, sample_every: int = 10) -> int:
    n = sum(1 for i in range(steps) if i % sample_every == sample_every - 1)
    return n if n else 1


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
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(s)
        step()
        e1.record(s)
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1)
        n = max(1, int(seconds * 1e3 / max(step_ms, 1e-3)))
        seen, fresh = {stamp0}, []
        t0 = tlast = time.perf_counter()
        for i in range(n):   # launches block once the queue is full, so the reads interleave
            step()
            if step_ms > 2.0 and i % max(1, int(20.0 / step_ms)) == 0:
                torch.cuda.synchronize()   # long steps: keep the host in step with the GPU
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


def _dev(a, dtype="bf16"):
    from workloads.device import to_device
    return to_device(a, dtype)


def _host(t):
    from workloads.device import to_host
    return to_host(t)


# ---------------------------------------------------------------------------- c0

def int_mlp_bench(args):
    """c0: the integer fp32 TP=2 MLP, both ranks in turn (column + ReLU, row partial), then the
    partial sum; latency-bound, reported in microseconds per step."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.mlp_relu_tp2()
    X = _dev(inp.X, "f32")
    # rank r holds columns r*128.. of W1 and rows r*128.. of W2
    W1 = [_dev(inp.W_gate[:, r * 128:(r + 1) * 128], "f32") for r in range(2)]
    W2 = [_dev(inp.W_down[r * 128:(r + 1) * 128, :], "f32") for r in range(2)]
    H = [torch.empty((16, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    P = [torch.empty((16, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
    Y = torch.empty((16, 64), dtype=torch.float32, device="cuda")

    def step():
        for r in range(2):
            tp.column_linear(X, W1[r], Y=H[r], act=tp.TP_ACT_RELU)
            tp.row_linear_partial(H[r], W2[r], Y=P[r])
        tp.partial_sum(P, out=Y)

    ms = timed(step, args.warmup, args.steps, "c0")
    # the same five calls captured as one HIP graph: the GPU-side latency without the per-call
    # host cost (Python, ctypes, argument checks, launch)
    g_ms, _ = graph_timed(step, args.warmup, args.steps, "c0_graph")
    return {"workload": "mlp_relu_tp2: integer fp32 MLP, X[16,64], W1[64,256] column-split into 2x[64,128] + ReLU, "
                        "W2[256,64] row-split into 2x[128,64]; both ranks in turn, then tp_partial_sum (5 launches)",
            "us_per_step": ms * 1e3, "us_per_step_graph": g_ms * 1e3, "flops_per_step": 2.0 * 16 * 64 * 256 * 2,
            "step_stats": STEP_STATS.get("c0"), "step_stats_graph": STEP_STATS.get("c0_graph"),
            "graph": "the five calls of a step captured as one HIP graph (torch.cuda.CUDAGraph), replays timed"}, \
        {"inp": inp, "Y": Y}


# ---------------------------------------------------------------------------- c1

def mlp_bench(args):
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.mlp7b_tp4()
    T, H, I = inp.T, inp.H, inp.I
    X, Wg, Wu, Wd = _dev(inp.X), _dev(inp.W_gate), _dev(inp.W_up), _dev(inp.W_down)
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.mlp_workspace_size(T, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16), dtype=torch.uint8, device="cuda")

    def step():
        tp.mlp_shard(X, Wg, Wu, Wd, Y=Y, workspace=ws)

    t0 = time.perf_counter()
    n_pre = prewarm(step, args.prewarm)
    PREWARM.update({"seconds": round(time.perf_counter() - t0, 3), "steps": n_pre,
                    "what": "untimed back-to-back headline steps before any timing (clock settling)"})
    ms = timed(step, args.warmup, args.steps, "mlp", keep_steps=True)
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
    return res, {"inp": inp, "Y": Y}


# ---------------------------------------------------------------------------- c2, c3

def attn_bench(args, name):
    """c2 (attn7b_tp4) or c3 (layer70b_tp8: the attention shard and the MLP shard on the same X,
    two fp32 partials)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.WORKLOADS[name]()
    B, S, H, hq, hkv = inp.B, inp.S, inp.H, inp.hq, inp.hkv
    X, Wqkv, Wo = _dev(inp.X), _dev(inp.W_qkv), _dev(inp.W_o)
    T = B * S
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.attn_workspace_size(B, S, H, hq, hkv, inp.theta), dtype=torch.uint8, device="cuda")
    mlp = None
    if inp.mlp is not None:
        m = inp.mlp
        I = m.W_gate.shape[1]
        mlp = (_dev(m.W_gate), _dev(m.W_up), _dev(m.W_down),
               torch.empty((T, H), dtype=torch.float32, device="cuda"),
               # the 70B shard keeps h in fp16 (with bf16 h its worst element is 2.8e-2 of the 3e-2 bar)
               torch.empty(tp.mlp_workspace_size(T, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_F16),
                           dtype=torch.uint8, device="cuda"))

    def step():
        tp.attn_shard(X, Wqkv, Wo, B, S, hq, hkv, inp.theta, Y=Y, workspace=ws)
        if mlp:
            tp.mlp_shard(X, mlp[0], mlp[1], mlp[2], Y=mlp[3], workspace=mlp[4], h_dtype=tp.TP_F16)

    ms = timed(step, args.warmup, args.steps, name)
    d = 128
    f_qkv = 2.0 * T * H * (hq + 2 * hkv) * d
    f_att = 2.0 * 2 * d * B * hq * S * (S + 1) / 2      # causal triangle only: QK^T and PV
    f_o = 2.0 * T * hq * d * H
    f_mlp = 0.0
    if inp.mlp is not None:
        f_mlp = 2.0 * T * H * inp.mlp.W_gate.shape[1] * 3
    flops = f_qkv + f_att + f_o + f_mlp
    nsamp = sampled_steps(args.steps)
    kern = {}
    for kname, f in (("gemm_bf16_qkv_rope", f_qkv), ("flash_attn_fwd", f_att), ("gemm_bf16_swiglu", None),
                     ("gemm_bf16_f32out", None), ("gemm_f16_f32out", None), ("bf16_to_f16", None),
                     ("fixup_gemm", None), ("fixup_swiglu", None), ("rope_table", None)):
        k_ms, k_n = kernel_avg(kname)
        if k_n:
            kern[kname] = {"avg_us": k_ms * 1e3, "launches_per_step": k_n / nsamp}
            if f:
                kern[kname]["tflops"] = f / (k_ms * 1e-3) / 1e12
    out = {"workload": inp.name, "ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
           "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flops_per_step": flops,
           "flops": {"qkv": f_qkv, "attention_causal": f_att, "o": f_o, "mlp": f_mlp},
           "step_stats": STEP_STATS.get(name), "kernels": kern}
    return out, {"inp": inp, "Y": Y, "Ym": mlp[3] if mlp else None}


# ---------------------------------------------------------------------------- c4

def graph_timed(step, warmup: int, steps: int, name: str = None):
    """Capture one step into a HIP graph (torch.cuda.CUDAGraph) and time `steps` replays, one event
    after each replay (per-replay times: STEP_STATS[name]). Returns (ms per replay, graph)."""
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
    ev = [TimingEvent() for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    if name:
        _stats(name, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return ms, g


def decode_bench(args):
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.decode7b_tp2()
    B, H, hq, hkv, L = inp.B, inp.H, inp.hq, inp.hkv, inp.cache_len + 1
    X = _dev(inp.X)
    Wqkv, Wo, Wg, Wu, Wd, Wlm = (_dev(w) for w in (inp.W_qkv, inp.W_o, inp.W_gate, inp.W_up, inp.W_down, inp.W_lm))
    kc, vc = _dev(inp.k_cache), _dev(inp.v_cache)
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

    ws_f = torch.empty(tp.decode_step_workspace_size(B, H, hq, hkv, inp.theta, kc, vc, inp.cache_len, I, V),
                       dtype=torch.uint8, device="cuda")

    def step_fused():   # tp_decode_step: the same three parts in four launches on one stream
        tp.decode_step(X, Wqkv, Wo, hq, hkv, inp.theta, kc, vc, inp.cache_len, Wg, Wu, Wd, Wlm,
                       Y_attn=Ya, Y_mlp=Ym, logits=logits, workspace=ws_f)

    # the same weights packed once into 128-column strips (load-time layout, not timed): every
    # workgroup of the step's GEMM launches then streams one contiguous block per K chunk
    packed = [tp.pack_strips(w) for w in (Wqkv, Wo, Wg, Wu, Wd, Wlm)]

    def step_packed():   # tp_decode_step_packed: the same step on the packed weights
        tp.decode_step(X, packed[0], packed[1], hq, hkv, inp.theta, kc, vc, inp.cache_len, packed[2], packed[3],
                       packed[4], packed[5], Y_attn=Ya, Y_mlp=Ym, logits=logits, workspace=ws_f, packed=True,
                       I=I, V=V)

    outs = (Ya, Ym, logits)
    ms_sep_eager = timed(step, args.warmup, args.steps)
    ms_sep_graph, _ = graph_timed(step_branches, args.warmup, args.steps)
    ms_inplace_eager = timed(step_fused, args.warmup, args.steps, "decode_inplace", sample_every=0)
    eager = [_host(t) for t in outs] + [_host(kc[:, :, inp.cache_len])]
    ms_inplace_graph, _ = graph_timed(step_fused, args.warmup, args.steps)
    timed(step_packed, args.warmup, args.steps)                 # per-kernel HIP-event timing
    att_ms, att_n = kernel_avg("decode_attn")
    sk_ms, sk_n = kernel_avg("skinny_gemm")
    rd_ms, rd_n = kernel_avg("skinny_reduce")
    x_ms, _ = kernel_avg("skinny_gemm_x")
    out_ms, _ = kernel_avg("skinny_gemm_out")
    for t in outs:
        t.fill_(float("nan"))
    # the headline: the packed step issued on one stream, no per-kernel events
    ms = timed(step_packed, args.warmup, args.steps, "decode", sample_every=0)
    torch.cuda.synchronize()
    # its outputs must equal the eager in-place step's, bit for bit (the packed step runs the same
    # kernels and sums; only the weight addresses differ)
    packed_out = [_host(t) for t in outs] + [_host(kc[:, :, inp.cache_len])]
    same_packed = all(a.tobytes() == b.tobytes() for a, b in zip(eager, packed_out))
    for t in outs:
        t.fill_(float("nan"))
    ms_graph, g = graph_timed(step_packed, args.warmup, args.steps, "decode_graph")   # as one HIP graph
    torch.cuda.synchronize()
    # the outputs left by the last timed replay must equal the eager step's, bit for bit
    replay = [_host(t) for t in outs] + [_host(kc[:, :, inp.cache_len])]
    same = all(a.tobytes() == b.tobytes() for a, b in zip(eager, replay))
    # The same steps with the 256 MB Infinity Cache flushed first: a 512 MiB buffer is read and
    # rewritten before each one (outside its events), so no step finds weights or cache rows that
    # the previous step left in the cache. Back-to-back steps re-read a 606 MB working set.
    flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    n_cold = min(args.steps, 20)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(n_cold)]
    for e0, e1 in ev:
        flush.add_(1.0)
        e0.record()
        step_packed()
        e1.record()
    torch.cuda.synchronize()
    cold = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    ms_cold = sum(cold) / len(cold)
    del flush
    d = 128
    w_bytes = 2 * (H * (hq + 2 * hkv) * d + hq * d * H + 2 * H * I + I * H + H * V)
    kv_bytes = 2 * 2 * B * hkv * (L - 1) * d          # cached keys and values read once
    new_kv = 2 * 2 * B * hkv * d                       # the new key/value written (and read back)
    act = 2 * B * H + 4 * (2 * B * H + B * V)          # X in; two fp32 partials and the logits out
    total = w_bytes + kv_bytes + 2 * new_kv + act
    nsamp = sampled_steps(args.steps)
    return {
        "ms_per_step": ms,
        "ms_per_step_graph": ms_graph,
        "step_stats_graph": STEP_STATS.get("decode_graph"),
        "ms_per_step_weights_in_place": ms_inplace_eager,
        "ms_per_step_weights_in_place_graph": ms_inplace_graph,
        "gbs_weights_in_place": total / (ms_inplace_eager * 1e-3) / 1e9,
        "step_stats_weights_in_place": STEP_STATS.get("decode_inplace"),
        "ms_per_step_cache_flushed": ms_cold,
        "median_ms_cache_flushed": cold[len(cold) // 2],
        "ms_per_step_separate_calls_eager": ms_sep_eager,
        "ms_per_step_separate_calls_graph": ms_sep_graph,
        "step_stats": STEP_STATS.get("decode"),
        "step": "tp_decode_step_packed (4 launches on one stream; the weights packed once into 128-column "
                "strips by tp_pack_strips, outside the timed region), no per-kernel events; graph: the same "
                "step captured as one HIP graph and replayed; weights_in_place: tp_decode_step on the [K, N] "
                "weights; separate_calls: tp_attn_shard, tp_mlp_shard, tp_column_linear as three graph "
                "branches on their own streams; kernels: per-kernel events on every 10th step of another pass",
        "packed_outputs_equal_in_place": same_packed,
        "graph_outputs_equal_eager": same,
        "bytes_per_step": total,
        "gbs": total / (ms * 1e-3) / 1e9,
        "gbs_cache_flushed": total / (ms_cold * 1e-3) / 1e9,
        "frac_hbm": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels": {"decode_attn(avg_us)": att_ms * 1e3 if att_ms else None,
                    "skinny_gemm_x: QKV + gate/up (avg_us)": x_ms * 1e3 if x_ms else None,
                    "skinny_gemm_out: O + down + head (avg_us)": out_ms * 1e3 if out_ms else None,
                    "skinny_gemm*(launches/step)": sk_n / nsamp,
                    "skinny_reduce*(avg_us)": rd_ms * 1e3 if rd_ms else None,
                    "skinny_reduce*(launches/step)": rd_n / nsamp},
        "workload": "decode7b_tp2: B=32 one token each, 16 local heads (MHA), KV cache 1024 tokens, "
                    "H=4096, I_shard=5504, LM head [4096,16000]",
    }, {"inp": inp, "eager": eager}


# ---------------------------------------------------------------------------- other legs

def fp8_mlp_bench(args):
    """The same MLP shard on OCP E4M3 codes with per-tensor scales (tp_mlp_shard_fp8)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    from workloads.device import codes_to_device
    inp = wl.mlp7b_tp4_fp8()
    T, H, I = inp.T, inp.H, inp.I
    X, Wg, Wu, Wd = (codes_to_device(a) for a in (inp.X, inp.W_gate, inp.W_up, inp.W_down))
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
    inp = wl.merge7b_tp4()
    T, H, k = inp.T, inp.H, len(inp.partials)
    parts = [_dev(p, "f32") for p in inp.partials]
    res, gamma = _dev(inp.residual), _dev(inp.gamma)
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
    """Backward of the 7B TP=4 MLP down shard (tp_linear_backward: dX = dY.W^T, dW = X^T.dY)."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.backward7b_tp4()
    T, K = inp.X.shape
    N = inp.W.shape[1]
    X, W, dY = _dev(inp.X), _dev(inp.W), _dev(inp.dY)
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    dW = torch.empty((K, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.linear_backward_workspace_size(T, K, N), dtype=torch.uint8, device="cuda")

    def step():
        tp.linear_backward(X, W, dY, dX=dX, dW=dW, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "backward")
    flops = 4.0 * T * K * N
    nsamp = sampled_steps(args.steps)
    kern = {}
    gemm_ms = 0.0
    for name in ("gemm_bf16_f32out", "fixup_gemm", "transpose_bf16"):
        k_ms, k_n = kernel_avg(name)
        if k_n:
            kern[name] = {"avg_us": k_ms * 1e3, "launches_per_step": k_n / nsamp}
            if name != "transpose_bf16":
                gemm_ms += k_ms * k_n / nsamp
    return {
        "workload": "backward7b_tp4: X = h [4096,2752], W_down shard [2752,4096], dY [4096,4096] bf16 -> dX, dW fp32",
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "step_stats": STEP_STATS.get("backward"),
        "gemm_tflops": flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
        "kernels": kern,
    }


def moe_bench(args):
    """Top-2 MoE MLP on one rank (tp_moe_mlp_shard): 2048 tokens, 8 local experts whose SwiGLU
    MLPs are TP=4 shards (H 4096, I 3584); gather, grouped gate/up + down, gated combine."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    import workloads as wl
    inp = wl.moe8x7b_tp4()
    T, H = inp.X.shape
    I = inp.W_gate.shape[2]
    R = int(inp.expert_offsets[-1])
    X, Wg, Wu, Wd = _dev(inp.X), _dev(inp.W_gate), _dev(inp.W_up), _dev(inp.W_down)
    rt = torch.from_numpy(inp.row_token.copy()).cuda()
    tr = torch.from_numpy(inp.token_rows.copy()).cuda()
    gates = _dev(inp.gates, "f32")
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tp.moe_workspace_size(T, H, I, inp.expert_offsets), 1), dtype=torch.uint8, device="cuda")

    def step():
        tp.moe_mlp_shard(X, Wg, Wu, Wd, inp.expert_offsets, rt, tr, gates, Y=Y, workspace=ws)

    ms = timed(step, args.warmup, args.steps, "moe")
    flops = 6.0 * R * H * I
    nsamp = sampled_steps(args.steps)
    kern = {}
    for name in ("moe_gather", "gemm_bf16_swiglu", "fixup_swiglu", "gemm_bf16_f32out", "fixup_gemm",
                 "skinny", "moe_combine"):
        k_ms, k_n = kernel_avg(name)
        if k_n:
            kern[name] = {"avg_us": k_ms * 1e3, "launches_per_step": k_n / nsamp}
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


def ceiling_bench(args):
    """The matrix pipe's sustained bf16 rate with operands in registers (tp_mfma_rate_probe), for
    random N(0,1) operands and for low-entropy ones, with the clock and socket power meanwhile:
    the power-limited roof that any bf16 GEMM on real data sits under."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(9)
    pats = {"random_normal": torch.randn(8 * 256 * 8, device="cuda", generator=g).to(torch.bfloat16),
            "ones": torch.ones(8 * 256 * 8, device="cuda", dtype=torch.bfloat16),
            "zeros": torch.zeros(8 * 256 * 8, device="cuda", dtype=torch.bfloat16)}
    res = {}
    for name, ops in pats.items():
        def run(iters):
            tp.mfma_rate_probe(ops, out, n_wg, iters)
        e0, e1 = TimingEvent(), TimingEvent()
        run(2000)
        torch.cuda.synchronize()
        e0.record()
        run(2000)
        e1.record()
        torch.cuda.synchronize()
        iters = max(1000, int(2000 * 20.0 / max(e0.elapsed_time(e1), 1e-3)))   # ~20 ms per launch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.5:   # settle the clock at the power limit first
            run(iters)
            torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            run(iters)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        flops = n_wg * 4 * 16 * iters * 32768.0
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, "ms_per_launch": ms,
                     "clock_power": None if args.no_clock else clock_power(lambda: run(iters), 2.0)}
    # The headline MLP step itself (same shapes, same kernels and instruction stream) on operands that
    # draw little power: zero activations with the random weights, and everything zero. Its rate
    # then shows what the kernels' schedule reaches when the board's power limit does not set the
    # clock (the outputs are zero; nothing here is a parity case).
    import workloads as wl
    inp = wl.mlp7b_tp4()
    T, H, I = inp.T, inp.H, inp.I
    Wg, Wu, Wd = _dev(inp.W_gate), _dev(inp.W_up), _dev(inp.W_down)
    X0 = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(tp.mlp_workspace_size(T, H, I, tp.TP_MLP_SWIGLU, tp.TP_BF16), dtype=torch.uint8, device="cuda")
    flops = 2.0 * T * H * 2 * I + 2.0 * T * I * H
    mlp = {}
    for name, (x, wg, wu, wd) in {"zero_activations": (X0, Wg, Wu, Wd),
                                  "all_zero": (X0, torch.zeros_like(Wg), torch.zeros_like(Wu), torch.zeros_like(Wd))}.items():
        def step():
            tp.mlp_shard(x, wg, wu, wd, Y=Y, workspace=ws)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.5:   # let the clock settle on this load
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        for _ in range(50):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 50
        mlp[name] = {"ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                     "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "clock_power": None if args.no_clock else clock_power(step, 2.0)}
    return {"what": "v_mfma_f32_32x32x16_bf16 back to back, operands in registers, 16 accumulators per wave, "
                    "one 4-wave workgroup per compute unit (tp_mfma_rate_probe)", "patterns": res,
            "mlp7b_tp4_low_power_operands": mlp}


def hbm_read_bench(args):
    """The HBM read rate the decode GEMMs' access pattern can reach without their arithmetic
    (tp_hbm_read_probe): the grids of the decode step's two weight-streaming launches, each
    workgroup reading a contiguous run in 8 KB blocks. Five buffers of the launch's size are read
    in turn, so no launch finds its bytes in the 256 MB Infinity Cache; back-to-back launches."""
    import torch
    import tensor_transformer_layer_rank_amd as tp
    res = {}
    out = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")
    for name, n_wg, nbytes in (("decode_K1_grid", 402, 140509184), ("decode_K3_grid", 378, 192937984),
                               ("512_workgroups", 512, 140509184)):
        per = nbytes // n_wg // 8192 * 8192
        stride = (per * n_wg + (1 << 20)) // 256 * 256
        buf = torch.ones(stride * 5, dtype=torch.uint8, device="cuda")
        for i in range(10):
            tp.hbm_read_probe(buf[(i % 5) * stride:], per, n_wg, out)
        torch.cuda.synchronize()
        reps = 100
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        for i in range(reps):
            tp.hbm_read_probe(buf[(i % 5) * stride:], per, n_wg, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"workgroups": n_wg, "bytes": per * n_wg, "us_per_launch": ms * 1e3,
                     "gbs": per * n_wg / (ms * 1e-3) / 1e9, "frac_hbm": per * n_wg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del buf
    return {"what": "contiguous run per workgroup, 4 waves, 16-byte nontemporal loads in 8 KB blocks, one block "
                    "ahead, two workgroups per compute unit; five buffers read in turn (tp_hbm_read_probe)",
            "grids": res}


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


# ---------------------------------------------------------------------------- parity + CPU oracle

def _cmp(got, ref, out="f32"):
    """relF, max-abs, and max-abs past half an ulp of the stored value (bf16 outputs)."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    half_ulp = {"f32": 0.0, "bf16": 2.0 ** -8}[out]
    rf = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return {"relF": rf, "max_abs": float(diff.max()),
            "max_abs_past_storage_rounding": float((diff - half_ulp * np.abs(ref)).max()),
            "elements": int(got.size), "finite": bool(np.all(np.isfinite(got))),
            "pass": bool(np.all(np.isfinite(got)) and rf <= 5e-3 and float((diff - half_ulp * np.abs(ref)).max()) <= 3e-2)}


def cpu_oracle_leg(keep):
    """The CPU baseline leg, per workload: the fp64 oracle computes each workload's whole output
    on this host's cores (its wall time is reported as that workload's CPU baseline), and every
    element of the GPU's output (as left by its timed steps) is compared with it. Runs after all
    GPU timing."""
    import numpy as np
    import oracle as O
    res = {}
    if "c0" in keep:
        k = keep["c0"]
        inp = k["inp"]
        t0 = time.perf_counter()
        refs = [O.mlp_relu_shard(inp.X, O.column_shard(inp.W_gate, r, 2), O.row_shard(inp.W_down, r, 2))
                for r in range(2)]
        ref = O.partial_sum(refs)
        dt = time.perf_counter() - t0
        got = _host(k["Y"])
        res["c0"] = {"bit_exact": bool(np.array_equal(got, ref)), "oracle_s": dt, "elements": int(got.size)}
    if "c1" in keep:
        k = keep["c1"]
        inp = k["inp"]
        t0 = time.perf_counter()
        ref = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
        dt = time.perf_counter() - t0
        res["c1"] = {**_cmp(_host(k["Y"]), ref), "oracle_s": dt}
    for c in ("c2", "c3"):
        if c not in keep:
            continue
        k = keep[c]
        inp = k["inp"]
        t0 = time.perf_counter()
        ref = O.attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.B, inp.S, inp.hq, inp.hkv, inp.d, inp.theta)
        dt = time.perf_counter() - t0
        r = {"attention": {**_cmp(_host(k["Y"]), ref), "oracle_s": dt}}
        del ref
        if k["Ym"] is not None:
            m = inp.mlp
            t0 = time.perf_counter()
            ref = O.mlp_swiglu_shard(m.X, m.W_gate, m.W_up, m.W_down)
            dt = time.perf_counter() - t0
            r["mlp"] = {**_cmp(_host(k["Ym"]), ref), "oracle_s": dt}
            del ref
        res[c] = r
    if "c4" in keep:
        k = keep["c4"]
        inp = k["inp"]
        ya, ym, lg, kn = k["eager"]
        t0 = time.perf_counter()
        att, knew, _ = O.decode_attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.k_cache, inp.v_cache, inp.cache_len,
                                           inp.hq, inp.hkv, inp.d, inp.theta)
        mlp = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
        lm = O.lm_head_shard(inp.X, inp.W_lm)
        dt = time.perf_counter() - t0
        res["c4"] = {"attention": _cmp(ya, att), "mlp": _cmp(ym, mlp), "logits": _cmp(lg, lm),
                     "appended_keys": _cmp(kn, knew, "bf16"), "oracle_s": dt}
    return res


def cpu_baseline(inp, target_s: float):
    """The fp64 oracle on the same MLP shard (c1), on this host's cores, repeated to about target_s."""
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


def _round(x, nd=5):
    """nd decimals, or 4 significant digits for magnitudes below 1e-3 (error norms stay readable)."""
    if isinstance(x, float):
        return float(f"{x:.4g}") if x != 0.0 and abs(x) < 1e-3 else round(x, nd)
    if isinstance(x, dict):
        return {k: _round(v, nd) for k, v in x.items()}
    if isinstance(x, list):
        return [_round(v, nd) for v in x]
    return x


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: one rank's shard; "
                                   "run with --gpus 1 (multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    import tensor_transformer_layer_rank_amd as tp
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    tp.load()
    legs = set(args.legs.split(",")) if args.legs != "all" else \
        {"c0", "c1", "c2", "c3", "c4", "fp8", "merge", "backward", "moe", "ceiling", "hbm"}
    keep = {}
    mlp = c0 = c2 = c3 = dec = fp8 = merge = bwd = moe = None
    t_start = time.perf_counter()

    def done(leg):   # one progress line per finished leg, on stderr (stdout carries the JSON line)
        print(f"bench: {leg} done at {time.perf_counter() - t_start:.1f} s", file=sys.stderr, flush=True)

    if "c1" in legs:
        mlp, keep["c1"] = mlp_bench(args)        # headline first, after the clock-settling prewarm
        done("c1")
    if "c0" in legs:
        c0, keep["c0"] = int_mlp_bench(args)
        done("c0")
    if "c2" in legs:
        c2, keep["c2"] = attn_bench(args, "attn7b_tp4")
        done("c2")
    if "c3" in legs:
        c3, keep["c3"] = attn_bench(args, "layer70b_tp8")
        done("c3")
    if "c4" in legs:
        dec, keep["c4"] = decode_bench(args)
        done("c4")
    if "fp8" in legs:
        fp8 = fp8_mlp_bench(args)
        done("fp8")
    if "merge" in legs:
        merge = merge_bench(args)
        done("merge")
    if "backward" in legs:
        bwd = backward_bench(args)
        done("backward")
    if "moe" in legs:
        moe = moe_bench(args)
        done("moe")
    ceiling = None
    if "ceiling" in legs:
        ceiling = ceiling_bench(args)
        done("ceiling")
    hbm = None
    if "hbm" in legs:
        hbm = hbm_read_bench(args)
        done("hbm read ceiling")
    if args.traffic_probe:
        traffic_probe()
    torch.cuda.synchronize()
    par = None if args.no_parity else cpu_oracle_leg(keep)
    if par is not None:
        done("parity (fp64 oracle over every output element)")
    if mlp is None:
        print(json.dumps({"legs": sorted(legs), "c0": c0, "c2": c2, "c3": c3, "decode": dec, "fp8_mlp": fp8,
                          "merge_rmsnorm": merge, "backward": bwd, "moe": moe, "mfma_ceiling": ceiling, "hbm_read_ceiling": hbm,
                          "parity": par}))
        return
    cpu = None if args.no_cpu else cpu_baseline(keep["c1"]["inp"], args.cpu_seconds)
    if cpu is not None:
        done("cpu baseline")
    props = torch.cuda.get_device_properties(0)
    c1 = {"workload": "mlp7b_tp4", "ms_per_step": mlp["ms_per_step"], "tflops": mlp["tflops"],
          "frac_bf16_peak": mlp["tflops"] / PEAK_BF16_TFLOPS}
    configs = {"c0_mlp_relu_tp2": c0, "c1_mlp7b_tp4": c1, "c2_attn7b_tp4": c2, "c3_layer70b_tp8": c3,
               "c4_decode7b_tp2": dec and {k: dec[k] for k in ("ms_per_step", "gbs", "frac_hbm",
                                                              "ms_per_step_graph", "ms_per_step_weights_in_place",
                                                              "gbs_weights_in_place", "packed_outputs_equal_in_place",
                                                              "graph_outputs_equal_eager")}}
    if par:
        for key, c in (("c0_mlp_relu_tp2", "c0"), ("c1_mlp7b_tp4", "c1"), ("c2_attn7b_tp4", "c2"),
                       ("c3_layer70b_tp8", "c3"), ("c4_decode7b_tp2", "c4")):
            if c in par and configs[key] is not None:
                configs[key]["parity"] = par[c]
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
                   "decode_gbs": dec and round(dec["gbs"], 1),
                   "decode_frac_hbm": dec and round(dec["frac_hbm"], 4),
                   "decode_ms_per_step": dec and round(dec["ms_per_step"], 5)},
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in mlp["roofline"].items()},
        "cpu_baseline": cpu and {k: v for k, v in cpu.items() if k != "seconds"},
        "prewarm": PREWARM,
        "step_stats": mlp["step_stats"],
        "clock_power": mlp["clock_power"],
        "kernels": mlp["kernels"],
        "configs": configs,
        "decode": dec,
        "fp8_mlp": fp8,
        "merge_rmsnorm": merge,
        "backward": bwd,
        "moe": moe,
        "mfma_ceiling": ceiling,
        "hbm_read_ceiling": hbm,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", None)},
    }
    print(json.dumps(_round(out)))


if __name__ == "__main__":
    main()
