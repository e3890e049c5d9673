"""Benchmark of the fused GEMM + epilogue path on one MI355X.

A step is one execute of the fused RELU_BIAS kernel on the 7B-FFN workload
(fp16, m=4096, n=11008, k=4096, fp32 accumulation), inputs resident in HBM. The
metric is 2mnk / time in TFLOP/s and its fraction of the dense fp16 MFMA peak.

Also measured (reported under "variants", not in "value"): the unfused three-kernel
chain on the same inputs, bf16 GELU_BIAS, RELU_AUX_BIAS, the bf16 8192^3
RELU_AUX_BIAS + DRELU_BGRAD pair, the rest of that layer's backward with transposed
operands, a whole two-layer training step at 8192, the square 4096^3 fused/unfused
pair, and the large (65536,16384)x(16384,8192) fp16 shape with and without the mask. The CPU oracle is timed on the headline workload on the
host cores, in whole passes for a bounded time (about 12 s).

Prints one JSON line (the last line of stdout).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6        # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_ffn_f16_4096x11008x4096.txt")
COPY_PROBE_BYTES = 1 << 30


# Other measurements, reported under "variants": name -> (workload, epilogue, dtype,
# inputs drawn on the device[, operand storage "TN" | "NT": A passed as its (k, m)
# transpose | B passed as its (n, k) transpose]). None stands for the headline workload.
VARIANTS = {
    # the headline kernel timed like every variant, beside its unfused chain
    "ffn_relu_bias_f16": (None, "RELU_BIAS", "f16", False),
    "ffn_unfused_f16": (None, "RELU_BIAS_UNFUSED", "f16", False),
    "ffn_aux_f16": (None, "RELU_AUX_BIAS", "f16", False),
    # the same product with the identity epilogue and with no epilogue: what bias + ReLU
    # cost inside the fused kernel
    "ffn_bias_f16": (None, "BIAS", "f16", False),
    "ffn_none_f16": (None, "NONE", "f16", False),
    "ffn_gelu_bf16": ("ffn_gelu_bf16_4096x11008x4096", "GELU_BIAS", "bf16", False),
    # the same fused product with B held as its (n, k) transpose (a linear layer's weight
    # as stored, out x in): every B fragment is then one ds_read_b128
    "ffn_relu_bias_f16_bt": (None, "RELU_BIAS", "f16", False, "NT"),
    "mlp8192_fwd_aux_bf16": ("mlp_bf16_8192", "RELU_AUX_BIAS", "bf16", True),
    "mlp8192_bwd_drelu_bgrad_bf16": ("mlp_bf16_8192", "DRELU_BGRAD", "bf16", True),
    # its unfused baseline: GEMM -> T1, ReLU backward against the forward activation,
    # row sums for bgrad, each a kernel of its own
    "mlp8192_bwd_unfused_bf16": ("mlp_bf16_8192", "DRELU_BGRAD_UNFUSED", "bf16", True),
    "large_relu_bias_f16": ("large_f16_65536x8192x16384", "RELU_BIAS", "f16", True),
    "large_aux_f16": ("large_f16_65536x8192x16384", "RELU_AUX_BIAS", "f16", True),
    "small_relu_bias_f16": ("relu_bias_f16_1024x512x2048", "RELU_BIAS", "f16", False),
    # the rest of the 8192 MLP layer's backward with the weights as stored: dX = W^T . dY
    # (DRELU_BGRAD on the W^T of the (k, m) weight) and dW = dZ . X^T (B as stored X)
    "mlp8192_bwd_wt_drelu_bgrad_bf16": ("mlp_bf16_8192", "DRELU_BGRAD", "bf16", True, "TN"),
    "mlp8192_dw_bf16": ("mlp_bf16_8192", "NONE", "bf16", True, "NT"),
    # one GPU's share of an 8-way split along n (no exchange in the forward; the backward
    # leaves a partial bgrad of m values for one all-reduce)
    "ffn_shard8_relu_bias_f16": ("ffn_shard8_f16_4096x1376x4096", "RELU_BIAS", "f16", False),
    "ffn_shard4_relu_bias_f16": ("ffn_shard4_f16_4096x2752x4096", "RELU_BIAS", "f16", False),
    "mlp8192_shard8_bwd_drelu_bgrad_bf16": ("mlp_shard8_bf16_8192x1024x8192", "DRELU_BGRAD", "bf16", True),
    # the square size the epilog-configuration page recommends for comparing fused and
    # unfused latency
    "square4096_relu_bias_f16": ("square_f16_4096", "RELU_BIAS", "f16", False),
    "square4096_unfused_f16": ("square_f16_4096", "RELU_BIAS_UNFUSED", "f16", False),
}
LAYOUTS = {"NN": (False, False), "TN": (True, False), "NT": (False, True)}
# The HBM-bound rows timed cold as well: each execute follows a 1 GiB scratch write, which
# evicts the 256 MB MALL and the L2s, so the operands come from HBM, and a read of the same
# bytes, which leaves clean lines behind.
COLD_VARIANTS = {"small_relu_bias_f16_cold": "small_relu_bias_f16", "ffn_unfused_f16_cold": "ffn_unfused_f16",
                 "mlp8192_bwd_drelu_bgrad_bf16_cold": "mlp8192_bwd_drelu_bgrad_bf16"}
FLUSH_BYTES = 1 << 30


# The sources that define the headline kernel's device code: the kernel headers and the
# fp16 instantiation unit (the host runtime in api.hip only picks the configuration,
# which the counter summary's `kernel` line pins separately).
KERNEL_SOURCES = ("gemm_dtl.hpp", "gemm_generic.hpp", "kernels.hpp", "launch.hpp", "tiles.hpp", "inst_f16.hip")


def kernel_source_hash() -> str:
    """SHA-256 over the headline kernel's sources: HBM-traffic counters taken for one
    version of the kernel are reported only while those sources are unchanged."""
    import hashlib
    csrc = os.path.join(ROOT, "gemm_epilogues_epilog_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel_desc: str):
    """HBM bytes per launch of the headline kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by the copy-kernel calibration), or None when the
    summary is missing or was taken on other kernel sources or another configuration."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith(("#", " ", "|")):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash() or kv.get("kernel") != kernel_desc:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe(repeats: int = 5):
    """A plain device-to-device copy of COPY_PROBE_BYTES, run `repeats` times: the
    calibration kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(repeats):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-16:], src[-16:])
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written": COPY_PROBE_BYTES,
                      "repeats": repeats}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(W, device_rng: bool):
    """Inputs of workload W on the GPU. The headline workload uses the seeded CPU
    generator shared with the tests; the large variants draw on the device (seeded)."""
    import torch
    from gemm_epilogues_epilog_amd import inputs
    if not device_rng:
        return W.a().cuda(), W.b().cuda(), W.bias().cuda()
    g = torch.Generator(device="cuda").manual_seed(W.seed)
    dt = inputs.TORCH_DT[W.dtype]
    A = (torch.randn(W.m, W.k, device="cuda", generator=g) * W.std_a).to(dt)
    B = (torch.randn(W.k, W.n, device="cuda", generator=g) * W.std_b).to(dt)
    bias = (torch.randn(W.m, device="cuda", generator=g) * W.std_bias).to(inputs.TORCH_DT[W.vec_dtype])
    return A, B, bias


WARM_S = 0.5          # every timing starts after at least this much untimed work: the clock settles
VARIANT_STEPS = 50    # timed executes per variant (after VARIANT_WARMUP and WARM_S of warm-up)
VARIANT_WARMUP = 10
HEADLINE_EVENTS = 200  # event-timed executes of the headline kernel (roofline.achieved)


def time_execute(ge, handle, args, steps, warmup, warm_s=WARM_S, event_steps=None):
    """Warm up (`warmup` executes, continued until `warm_s` seconds have passed), then
    time `steps` executes back to back under the host wall clock, bracketed by
    synchronisations (the throughput) and by one HIP event pair on the launch stream
    (the average launch duration: the kernels' own time plus the short gaps between
    back-to-back launches), and then `event_steps` (default `steps`) executes with one
    HIP event pair each (the spread of single launches; each pair also times its own
    event packet, a few microseconds, so these run a little long)."""
    import torch
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_warm < warm_s:
        ge.gemm_epilog_execute(handle, *args, stream=sptr)
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(steps):
        ge.gemm_epilog_execute(handle, *args, stream=sptr)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(event_steps or steps)]
    for e0, e1 in ev:
        e0.record(stream)
        ge.gemm_epilog_execute(handle, *args, stream=sptr)
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)   # ms
    return {"wall_ms_per_step": wall * 1e3 / steps, "region_ms_per_launch": r0.elapsed_time(r1) / steps,
            "event_ms_mean": sum(per) / len(per),
            "event_ms_median": per[len(per) // 2], "event_ms_p10": per[len(per) // 10],
            "event_ms_p90": per[min(len(per) - 1, (len(per) * 9) // 10)], "timed": len(per),
            "warmup_executes": done}


def time_execute_cold(ge, handle, args, steps):
    """`steps` executes, each after a FLUSH_BYTES scratch write that is then read back,
    timed alone with a HIP event pair on the launch stream (the flush is outside the
    pair). The write evicts the operands from the L2s and the MALL; the read-back
    replaces the dirty lines it leaves with clean ones, so the timed execute does not pay
    for writing the flush's own data back (a fill alone put 7% on the unfused chain and
    4% on the DRELU_BGRAD product at 8192)."""
    import torch
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(VARIANT_WARMUP):
        ge.gemm_epilog_execute(handle, *args, stream=sptr)
    for i, (e0, e1) in enumerate(ev):
        flush.fill_(i)
        flush.sum()
        e0.record(stream)
        ge.gemm_epilog_execute(handle, *args, stream=sptr)
        e1.record(stream)
    torch.cuda.synchronize()
    del flush
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return {"wall_ms_per_step": None, "event_ms_mean": sum(per) / len(per), "event_ms_median": per[len(per) // 2],
            "event_ms_p10": per[len(per) // 10], "event_ms_p90": per[min(len(per) - 1, (len(per) * 9) // 10)],
            "timed": len(per), "warmup_executes": VARIANT_WARMUP}


def run_variant(ge, W, epilog, dtype, steps, warmup, device_rng, layout="NN", cold=False):
    import torch
    A, B, bias = device_inputs(W, device_rng)
    m, n, k = W.m, W.n, W.k
    ta, tb = LAYOUTS[layout]
    t0 = time.perf_counter()
    if ta or tb:
        h = ge.gemm_epilog_plan_ex(m, n, k, (dtype, dtype, dtype), epilog, int(ta), int(tb))
    else:
        h = ge.gemm_epilog_plan(m, n, k, (dtype, dtype, dtype), epilog)
    plan_ms = (time.perf_counter() - t0) * 1e3
    D = torch.empty(m, n, dtype=A.dtype, device="cuda")
    aux = bg = None
    if epilog in ("RELU_AUX_BIAS", "DRELU_BGRAD"):
        aux = torch.zeros((m + 31) // 32, n, dtype=torch.int32, device="cuda")
    if epilog == "DRELU_BGRAD":
        bg = torch.empty(m, dtype=A.dtype, device="cuda")
        # a realistic mask: the forward pass of the same inputs
        hf = ge.gemm_epilog_plan(m, n, k, (dtype, dtype, dtype), "RELU_AUX_BIAS")
        ge.gemm_epilog_execute(hf, A, B, bias, D, aux, None)
        torch.cuda.synchronize()
        ge.gemm_epilog_free(hf)
        bias = None
    if epilog == "DRELU_BGRAD_UNFUSED":
        bg = torch.empty(m, dtype=A.dtype, device="cuda")
        # a realistic activation: the unfused forward pass of the same inputs
        aux = torch.empty(m, n, dtype=A.dtype, device="cuda")
        hf = ge.gemm_epilog_plan(m, n, k, (dtype, dtype, dtype), "RELU_BIAS_UNFUSED")
        ge.gemm_epilog_execute(hf, A, B, bias, aux, None, None)
        torch.cuda.synchronize()
        ge.gemm_epilog_free(hf)
        bias = None
    if ta:   # the same operands in the storage order the plan takes
        A = A.t().contiguous()
    if tb:
        B = B.t().contiguous()
    if cold:
        r = time_execute_cold(ge, h, (A, B, bias, D, aux, bg), steps)
    else:
        r = time_execute(ge, h, (A, B, bias, D, aux, bg), steps, warmup)
    desc = ge.gemm_epilog_describe(h)
    ge.gemm_epilog_free(h)
    t = r["event_ms_median"] * 1e-3
    byts = algorithmic_bytes(m, n, k, dtype, epilog)
    out = {"epilog": epilog, "dtype": dtype, "m": m, "n": n, "k": k, "layout": layout, "plan_ms": round(plan_ms, 3),
           "kernel": desc, "median_ms": round(r["event_ms_median"], 4), "p10_ms": round(r["event_ms_p10"], 4),
           "p90_ms": round(r["event_ms_p90"], 4), "timed": r["timed"], "warmup_executes": r["warmup_executes"],
           "tflops": round(2 * m * n * k / t / 1e12, 1), "algorithmic_bytes": byts,
           "gbs": round(byts / t / 1e9, 1), "frac_of_hbm": round(byts / t / 1e9 / PEAK_HBM_GBS, 4)}
    if cold:
        out["cold"] = f"each execute after a {FLUSH_BYTES >> 20} MiB scratch write and read-back"
    del A, B, D, aux, bg
    torch.cuda.empty_cache()
    return out


def algorithmic_bytes(m, n, k, dtype, epilog):
    """HBM bytes one execute must move at least: A, B and D once, the bias (or, for
    DRELU_BGRAD, the mask read and bgrad written), the mask written by RELU_AUX_BIAS, for
    the unfused chain its two elementwise kernels' reads and writes of T1 and T2, and for
    the unfused backward T1 written and read, the activation read and D read again."""
    es = 2 if dtype in ("f16", "bf16") else 4
    mask = 4 * ((m + 31) // 32) * n
    byts = es * (m * k + k * n + m * n + m)
    if epilog in ("RELU_AUX_BIAS", "DRELU_BGRAD"):
        byts += mask
    if epilog in ("RELU_BIAS_UNFUSED", "DRELU_BGRAD_UNFUSED"):
        byts += 4 * m * n * es
    return byts


def launch_floor(steps: int = 1000):
    """What any kernel costs on this machine, for scale beside the latency-bound small
    problems: a 4-byte fill (torch) timed with HIP event pairs and back to back."""
    import torch
    x = torch.empty(1, device="cuda")
    for _ in range(200):
        x.fill_(1.0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        x.fill_(1.0)
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t0) * 1e6 / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(200)]
    for e0, e1 in ev:
        e0.record()
        x.fill_(1.0)
        e1.record()
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    return {"what": "torch fill_ of 4 bytes", "event_median_us": round(per[len(per) // 2], 2),
            "back_to_back_us": round(b2b, 2)}


PROBE_HEADLINE_CASE = "f16 N(0,1/64) (the FFN workload's operands)"


def mfma_probe(ge, iters: int = 20000, workgroups: int = 512, only=None):
    """The MFMA-only probe (gemm_epilog_mfma_probe) on the value distributions of the
    workloads and on constant values: what the matrix cores sustain on those values
    under the power limit. Each case: one warm-up launch, then 5 timed with HIP events.
    `only`: names of the cases to run (all by default)."""
    import torch
    from gemm_epilogues_epilog_amd import probe as gprobe
    g = torch.Generator(device="cuda").manual_seed(0)
    n = 1 << 19   # 1 MiB of fp16/bf16 values
    makers = {
        PROBE_HEADLINE_CASE: ("f16", lambda: torch.randn(n, device="cuda", generator=g) / 64),
        "f16 N(0,1)": ("f16", lambda: torch.randn(n, device="cuda", generator=g)),
        "bf16 N(0,1/64)": ("bf16", lambda: torch.randn(n, device="cuda", generator=g) / 64),
        "f16 constant 1/64": ("f16", lambda: torch.full((n,), 1.0 / 64, device="cuda")),
        "f16 zeros": ("f16", lambda: torch.zeros(n, device="cuda")),
    }
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    flop = workgroups * 16 * iters * 32768
    res = {}
    for name, (dt, make) in makers.items():
        if only is not None and name not in only:
            continue
        ops = make().to(torch.float16 if dt == "f16" else torch.bfloat16)
        gprobe.gemm_epilog_mfma_probe(ops, dt, iters, workgroups, out)
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gprobe.gemm_epilog_mfma_probe(ops, dt, iters, workgroups, out)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        t = sorted(times)[2]
        res[name] = {"ms": round(t, 3), "tflops": round(flop / (t * 1e-3) / 1e12, 1),
                     "frac_of_peak": round(flop / (t * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
    return {"probe": "back-to-back v_mfma_f32_32x32x16 alternating two operand pairs, 4 chains per wave, "
                     "no memory traffic", "workgroups": workgroups, "iters": iters, "flop_per_launch": flop,
            "cases": res}


def run_autotune(ge, W, steps: int, warmup: int, repeats: int = 20):
    """The plan's table choice against gemm_epilog_autotune's measured choice on the
    same inputs: both timed like a variant, plus the wall time of the search."""
    import torch
    A, B, bias = device_inputs(W, device_rng=False)
    D = torch.empty(W.m, W.n, dtype=A.dtype, device="cuda")
    h = ge.gemm_epilog_plan(W.m, W.n, W.k, (W.dtype, W.dtype, W.dtype), W.epilog)
    args = (A, B, bias, D, None, None)
    before = ge.gemm_epilog_describe(h)
    r0 = time_execute(ge, h, args, steps, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    best = ge.gemm_epilog_autotune(h, *args, repeats=repeats)
    search_ms = (time.perf_counter() - t0) * 1e3
    after = ge.gemm_epilog_describe(h)
    r1 = time_execute(ge, h, args, steps, warmup)
    ge.gemm_epilog_free(h)
    del A, B, D
    torch.cuda.empty_cache()
    return {"workload": W.name, "epilog": W.epilog, "table_kernel": before, "table_median_ms": round(r0["event_ms_median"], 4),
            "tuned_kernel": after, "tuned_median_ms": round(r1["event_ms_median"], 4),
            "search_best_ms": round(best, 4), "search_wall_ms": round(search_ms, 1), "repeats": repeats}


def run_mlp_step(steps: int, warmup: int, size: int = 8192, dtype: str = "bf16", fused: bool = True):
    """One training step of the two-layer perceptron (batch, input, hidden and output
    all `size`): RELU_AUX_BIAS and NONE forward, then dW2 = dY H^T, the DRELU_BGRAD
    product W2^T dY with db1, and dW1 = dZ1 X^T, five executes per step. Inputs drawn
    on the device with the distributions of gemm_epilogues_epilog_amd.inputs.mlp_case.
    fused=False runs the unfused baselines in place of RELU_AUX_BIAS and DRELU_BGRAD."""
    import torch
    from gemm_epilogues_epilog_amd import inputs
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    t = inputs.TORCH_DT[dtype]
    g = torch.Generator(device="cuda").manual_seed(0)
    n = size
    X = torch.randn(n, n, device="cuda", generator=g).to(t)
    W1 = (torch.randn(n, n, device="cuda", generator=g) * n ** -0.5).to(t)
    b1 = (torch.randn(n, device="cuda", generator=g) * 0.02).to(t)
    W2 = (torch.randn(n, n, device="cuda", generator=g) * n ** -0.5).to(t)
    dY = torch.randn(n, n, device="cuda", generator=g).to(t)
    t0 = time.perf_counter()
    st = MLP2Step(n, n, n, n, dtype, fused=fused)
    plan_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(warmup):
        st.step(X, W1, b1, W2, dY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step(X, W1, b1, W2, dY)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        st.step(X, W1, b1, W2, dY)
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    kernels = [p.describe() for p in st.plans]
    flops = st.flops()
    st.free()
    del X, W1, b1, W2, dY, st
    torch.cuda.empty_cache()
    med = per[len(per) // 2]
    fwd, bwd = ("RELU_AUX_BIAS", "DRELU_BGRAD") if fused else ("RELU_BIAS_UNFUSED", "DRELU_BGRAD_UNFUSED")
    return {"what": f"2-layer MLP training step, batch = input = hidden = output = {n}, {dtype}: "
                    f"{fwd}, NONE; dW2 (B^T), {bwd} + db1 (A^T), dW1 (B^T)",
            "plan_ms": round(plan_ms, 3), "wall_ms_per_step": round(wall_ms, 4), "median_ms": round(med, 4),
            "p10_ms": round(per[len(per) // 10], 4), "p90_ms": round(per[(len(per) * 9) // 10], 4),
            "tflops": round(flops / (wall_ms * 1e-3) / 1e12, 1), "kernels": kernels}


def cpu_threads():
    """Threads for the oracle: every CPU this process may run on, capped at the CPU share
    the environment grants (OMP_NUM_THREADS, where set). Returns (threads, facts)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(usable, int(share)) if share.isdigit() and int(share) > 0 else usable
    return threads, {"host_cpus": os.cpu_count(), "usable_cpus": usable,
                     "cpu_share": int(share) if share.isdigit() else None}


def cpu_baseline(W, budget_s: float):
    """The CPU oracle on the whole headline workload, repeated until about budget_s
    seconds have passed (at least one full pass); inputs are drawn before timing.
    Returns (the cpu_baseline object, the oracle's D of the last pass)."""
    import numpy as np
    import torch
    import oracle

    def to_np(t):
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    a, b, bias = to_np(W.a()), to_np(W.b()), to_np(W.bias())
    threads, facts = cpu_threads()
    threads = min(threads, (W.m + 31) // 32)   # the oracle splits 32-row groups
    passes = 0
    out = None
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < budget_s:
        out = oracle.gemm_epilog(a, b, W.epilog, bias=bias, ab=W.dtype, nthreads=threads)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(passes * W.flops() / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "threads": threads, **facts, "kind": "oracle",
            "sample": f"{passes} full pass(es) of {W.name} {W.epilog} ({W.flops() / 1e9:.1f} GFLOP each) "
                      f"in {dt:.1f} s on {threads} threads (every usable CPU, within the CPU share), "
                      "inputs drawn before timing"}, out["D"]


def parity_stats(D_gpu, D_ref, dtype: str):
    """The GPU's full headline output against the oracle's (from the cpu_baseline pass),
    in the tolerance of the fused path: |y - y_ref| <= tol max(1, |y_ref|)."""
    import numpy as np
    import oracle
    tol = {"f16": 2e-2, "bf16": 2e-2, "f32": 1e-4}[dtype]
    y = oracle.to_f32(D_gpu, dtype).astype(np.float64)
    r = oracle.to_f32(D_ref, dtype).astype(np.float64)
    err = np.abs(y - r)
    ratio = err / (tol * np.maximum(1.0, np.abs(r)))
    bad = ~(ratio <= 1.0)
    return {"checked": "every element of the headline D against the oracle's", "elements": int(y.size),
            "outside_tolerance": int(bad.sum()), "non_finite": int((~np.isfinite(y)).sum()),
            "max_abs_err": float(err.max()), "max_err_over_tol": round(float(ratio.max()), 5),
            "bitwise_equal_frac": round(float((y == r).mean()), 5), "tolerance": f"{tol} * max(1, |ref|)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed executes first (continued until 0.5 s of warm-up: the clock settles under load)")
    ap.add_argument("--no-variants", action="store_true", help="time only the headline kernel")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--skip-cpu", action="store_true", help="leave out the cpu_baseline leg (profiling runs)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the MFMA-rate probe on the workloads' value distributions and print its line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 1 GiB copy that calibrates the HBM byte counters")
    ap.add_argument("--only", choices=sorted(VARIANTS) + sorted(COLD_VARIANTS) +
                    ["mlp8192_train_step_bf16", "mlp8192_train_step_bf16_unfused", "autotune_small",
                     "autotune_headline", "launch_floor"],
                    help="time one variant alone (--steps executes after --warmup) and print its line; "
                         "for profiling runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the fused epilogue shards by output tiles; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_epilogues_epilog_amd as ge
    from gemm_epilogues_epilog_amd import inputs

    ge.load()
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.mfma_probe:
        print(json.dumps(mfma_probe(ge)), flush=True)
        return
    if args.only in ("autotune_small", "autotune_headline"):
        wname = "relu_bias_f16_1024x512x2048" if args.only == "autotune_small" else inputs.HEADLINE
        print(json.dumps({"variant": args.only, **run_autotune(ge, inputs.WORKLOADS[wname], args.steps, args.warmup)}),
              flush=True)
        return
    if args.only == "launch_floor":
        print(json.dumps({"variant": args.only, **launch_floor()}), flush=True)
        return
    if args.only in ("mlp8192_train_step_bf16", "mlp8192_train_step_bf16_unfused"):
        r = run_mlp_step(args.steps, args.warmup, fused=not args.only.endswith("_unfused"))
        print(json.dumps({"variant": args.only, **r}), flush=True)
        return
    if args.only:
        cold = args.only in COLD_VARIANTS
        wname, ep, dt, dev_rng, *lay = VARIANTS[COLD_VARIANTS.get(args.only, args.only)]
        Wv = inputs.WORKLOADS[inputs.HEADLINE if wname is None else wname]
        r = run_variant(ge, Wv, ep, dt, args.steps, args.warmup, dev_rng, *lay, cold=cold)
        print(json.dumps({"variant": args.only, **r}), flush=True)
        return
    prop = torch.cuda.get_device_properties(0)
    W = inputs.WORKLOADS[inputs.HEADLINE]
    from gemm_epilogues_epilog_amd import probe as gprobe
    dev_cus, dev_mhz = gprobe.gemm_epilog_device_info()
    log(f"[bench] device {prop.name} {getattr(prop, 'gcnArchName', '')} CUs {prop.multi_processor_count} "
        f"(runtime: {dev_cus} CUs, peak clock {dev_mhz} MHz)")
    log(f"[bench] headline {W.name}: generating inputs")
    A, B, bias = device_inputs(W, device_rng=False)
    D = torch.empty(W.m, W.n, dtype=A.dtype, device="cuda")
    t0 = time.perf_counter()
    h = ge.gemm_epilog_plan(W.m, W.n, W.k, (W.dtype, W.dtype, W.dtype), W.epilog)
    plan_ms = (time.perf_counter() - t0) * 1e3
    log(f"[bench] plan {plan_ms:.3f} ms: {ge.gemm_epilog_describe(h)}")
    r = time_execute(ge, h, (A, B, bias, D, None, None), args.steps, args.warmup,
                     event_steps=max(args.steps, HEADLINE_EVENTS))
    kernel_desc = ge.gemm_epilog_describe(h)
    ge.gemm_epilog_free(h)
    torch.cuda.synchronize()
    D_host = D.cpu().numpy() if not args.skip_cpu else None
    flops = W.flops()
    value = flops / (r["wall_ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (r["region_ms_per_launch"] * 1e-3) / 1e12
    log(f"[bench] headline: {r}")

    traffic = read_traffic(kernel_desc)
    # what the matrix cores alone sustain on the headline's operand values (the MFMA-only
    # probe): the practical ceiling under the power limit, next to the spec peak
    probe_tflops = mfma_probe(ge, only=(PROBE_HEADLINE_CASE,))["cases"][PROBE_HEADLINE_CASE]["tflops"]
    log(f"[bench] mfma probe on the headline's value distribution: {probe_tflops} TFLOP/s")

    variants = {}
    if not args.no_variants:
        vsteps, vwarm = VARIANT_STEPS, VARIANT_WARMUP
        for name, (wname, ep, dt, dev_rng, *lay) in VARIANTS.items():
            Wv = inputs.WORKLOADS[inputs.HEADLINE if wname is None else wname]
            log(f"[bench] variant {name}")
            variants[name] = run_variant(ge, Wv, ep, dt, vsteps, vwarm, dev_rng, *lay)
            log(f"[bench]   {variants[name]}")
        # fused and unfused both timed as variants: same warm-up, same number of executes
        fused_ms = variants["ffn_relu_bias_f16"]["median_ms"]
        unf = variants["ffn_unfused_f16"]["median_ms"]
        variants["ffn_fusion_saving"] = {"fused_ms": fused_ms, "unfused_ms": unf,
                                         "saving_frac": round(1 - fused_ms / unf, 4),
                                         "timing": "both as variants: event medians of 50 executes after "
                                                   "10 + 0.5 s of warm-up"}
        sq_f, sq_u = variants["square4096_relu_bias_f16"]["median_ms"], variants["square4096_unfused_f16"]["median_ms"]
        variants["square4096_fusion_saving"] = {"fused_ms": sq_f, "unfused_ms": sq_u,
                                                "saving_frac": round(1 - sq_f / sq_u, 4)}
        bw_f = variants["mlp8192_bwd_drelu_bgrad_bf16"]["median_ms"]
        bw_u = variants["mlp8192_bwd_unfused_bf16"]["median_ms"]
        variants["mlp8192_bwd_fusion_saving"] = {"fused_ms": bw_f, "unfused_ms": bw_u,
                                                 "saving_frac": round(1 - bw_f / bw_u, 4)}
        for name, base in COLD_VARIANTS.items():
            wname, ep, dt, dev_rng, *lay = VARIANTS[base]
            Wv = inputs.WORKLOADS[inputs.HEADLINE if wname is None else wname]
            log(f"[bench] variant {name}")
            variants[name] = run_variant(ge, Wv, ep, dt, vsteps, vwarm, dev_rng, *lay, cold=True)
            log(f"[bench]   {variants[name]}")
        for wname in ("relu_bias_f16_1024x512x2048", inputs.HEADLINE):
            log(f"[bench] autotune {wname}")
            variants[f"autotune_{wname}"] = run_autotune(ge, inputs.WORKLOADS[wname], vsteps, vwarm)
            log(f"[bench]   {variants[f'autotune_{wname}']}")
        variants["launch_floor"] = launch_floor()
        log(f"[bench] launch floor {variants['launch_floor']}")
        for name, fused in (("mlp8192_train_step_bf16", True), ("mlp8192_train_step_bf16_unfused", False)):
            log(f"[bench] variant {name}")
            variants[name] = run_mlp_step(vsteps, vwarm, fused=fused)
            log(f"[bench]   {variants[name]}")
        st_f = variants["mlp8192_train_step_bf16"]["median_ms"]
        st_u = variants["mlp8192_train_step_bf16_unfused"]["median_ms"]
        variants["mlp8192_step_fusion_saving"] = {"fused_ms": st_f, "unfused_ms": st_u,
                                                  "saving_frac": round(1 - st_f / st_u, 4)}

    del A, B, D
    torch.cuda.empty_cache()
    log("[bench] cpu baseline (oracle)")
    cpu, parity = None, None
    if not args.skip_cpu:
        cpu, D_ref = cpu_baseline(W, args.cpu_budget)
        parity = parity_stats(D_host, D_ref, W.dtype)
    log(f"[bench] cpu: {cpu}")
    log(f"[bench] parity: {parity}")

    out = {
        "metric": "fused GEMM+bias+ReLU TFLOP/s & % fp16 MFMA peak (4096x11008x4096)",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": W.name, "m": W.m, "n": W.n, "k": W.k, "epilog": W.epilog,
                   "accumulate": "f32", "kernel": kernel_desc, "plan_ms": round(plan_ms, 3),
                   "cus": prop.multi_processor_count, "device_cus": dev_cus, "device_peak_clock_mhz": dev_mhz,
                   "peak_derivation": "256 CUs x 2.4 GHz x 4096 flop/clk (dense fp16/bf16 MFMA)",
                   "frac_of_peak": round(value / PEAK_F16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                     "kernel_ms_mean": round(r["region_ms_per_launch"], 4), "kernel_launches_timed": args.steps,
                     "kernel_timing": "one HIP event pair on the launch stream around the timed back-to-back executes",
                     "event_pair_ms_median": round(r["event_ms_median"], 4),
                     "event_pair_ms_p10": round(r["event_ms_p10"], 4), "event_pair_ms_p90": round(r["event_ms_p90"], 4),
                     "event_pairs": r["timed"], "warmup_executes": r["warmup_executes"],
                     "mfma_only_on_same_values": probe_tflops,
                     "frac_of_mfma_only": round(achieved / probe_tflops, 4)},
        "cpu_baseline": cpu,
        "parity": parity,
        "variants": variants,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
