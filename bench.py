"""Benchmark of the hot path on one MI355X.

One step = one fused attention forward on the causal bf16 workload
(B=2, H=16 -> B*H = 32, N=4096, d=128, every 64th query row x8) followed by
one stable row softmax over fp32 [32768, 8192].  Inputs are seeded synthetic
tensors already resident in HBM.  W untimed warm-up steps, then K timed steps
between device synchronisations; HIP events recorded on the launch stream
(torch's current stream) around each launch give each kernel's mean launch
duration (timing-only events, without the system-scope fence a default
event performs).  The defaults (50 warm-up, 100 timed steps, about 80 ms of GPU
work) measure the sustained state: once the softmax starts alternating with
the attention, the GPU's clock management lowers the attention kernel's
clock for roughly the first 30 steps (its launches run up to 15% longer)
before it settles.

Prints one JSON line:
  value             attention TFLOPS, counted FLOPs 4*B*H*N^2*d / 2 (causal)
                    over the mean attention launch time (median and fastest
                    launch beside it)
  roofline          attention kernel against the bf16 matrix-core peak
  softmax           row-softmax GB/s (8 algorithmic bytes per element)
  roofline_softmax  softmax kernel against the HBM peak
  cpu_baseline      the fp64 oracle on the host cores, on a bounded sample
                    of the same workload (and its parity on that sample)
  device            GPU name, architecture, compute units, peak engine clock
  supplementary     measured before the warm-up (see main): every other attention
                    workload (fp32 [1,1,128,64], bf16 [2,8,1024,64],
                    [4,16,2048,128], causal [1,32,8192,128]) with mean,
                    median and fastest launch, the fp32 kernel on the headline
                    shape (both masks), the headline shape without
                    the mask, a plain device copy of the softmax input as the
                    practical HBM ceiling, the split-KV forward beside the
                    single pass on long rows / few heads, packed
                    variable-length sequences beside padding, and the
                    backward pass of the headline workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOPS & % bf16 MFMA peak (B·H=32,N=4096,d=128); softmax GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


ATTN_SOURCES = ["online_softmax_08_amd/csrc/attn_fwd_bf16.hip",
                "online_softmax_08_amd/csrc/device_common.h"]
SOFTMAX_SOURCES = ["online_softmax_08_amd/csrc/row_softmax.hip",
                   "online_softmax_08_amd/csrc/device_common.h"]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def hip_runtime():
    """The HIP runtime this process already has loaded (torch's), never a
    second copy of it."""
    import ctypes
    for name in ("libamdhip64.so.7", "libamdhip64.so"):
        try:
            return ctypes.CDLL(name, mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        except OSError:
            continue
    raise RuntimeError("the HIP runtime is not loaded in this process")


def device_info(torch) -> dict:
    """Name, architecture, compute-unit count and peak engine clock of the GPU
    the run used, from the HIP device attributes."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "max_sclk_mhz": None}
    val = ctypes.c_int(0)
    # hipDeviceAttributeClockRate (peak clock in kHz) is entry 5 of
    # hipDeviceAttribute_t in hip_runtime_api.h.
    if hip_runtime().hipDeviceGetAttribute(ctypes.byref(val), 5, torch.cuda.current_device()) == 0:
        info["max_sclk_mhz"] = val.value // 1000
    return info


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventCreateWithFlags flag (hip_runtime_api.h)
TIMER = "HIP events on the launch stream, created with hipEventDisableSystemFence"


class KernelTimer:
    """Timing-only HIP events recorded on torch's current stream (the stream
    the kernels are launched on).

    They are created with hipEventDisableSystemFence, the flag HIP documents
    for events that only measure time: recording a default event performs a
    system-scope release, which writes back and invalidates the L2 inside the
    interval the event closes and leaves the next launch a cold cache.  The
    host orders itself with torch.cuda.synchronize(), not through these
    events."""

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        hip = hip_runtime()
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.hip = hip
        self.stream = vp(torch.cuda.current_stream().cuda_stream)
        self.events = []

    def _check(self, st, what):
        if st != 0:
            raise RuntimeError(f"{what} returned HIP error {st}")

    def event(self):
        e = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(e)
        return e

    def record(self, e):
        self._check(self.hip.hipEventRecord(e, self.stream), "hipEventRecord")

    def ms(self, a, b):
        """Milliseconds between two recorded events (both complete: call after
        a device synchronisation)."""
        f = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(f), a, b), "hipEventElapsedTime")
        return f.value

    def free(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def measured_traffic(tag: str, sources) -> float | None:
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{tag}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(sources):
        return None
    return float(rec["hbm_bytes_per_dispatch"])


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing leg (profiling runs)")
    ap.add_argument("--supplementary", choices=("before", "after", "none"), default="before",
                    help="when to run the supplementary measurements: before the warm-up and "
                         "timed steps (default), after them, or not at all (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy per step (outside the timed "
                         "region) to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels shard by batch*head with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import torch

    import online_softmax_08_amd as osm
    from online_softmax_08_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wa = inputs.ATTN[inputs.HEADLINE_ATTN]
    ws = inputs.SOFTMAX[inputs.HEADLINE_SOFTMAX]
    print(f"# {wa.describe()}", file=sys.stderr, flush=True)
    print(f"# {ws.describe()}", file=sys.stderr, flush=True)
    q_cpu, k_cpu, v_cpu = inputs.attn_inputs(wa)
    x_cpu = inputs.softmax_inputs(ws)
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    x = x_cpu.to(dev)
    O = torch.empty_like(q)
    lse = torch.empty((wa.B, wa.H, wa.N), dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    if args.copy_probe:
        csrc = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        cdst = torch.empty_like(csrc)

    def step():
        osm.attention(q, k, v, causal=wa.causal, out=O, lse=lse)
        osm.softmax(x, out=y)

    # The supplementary figures are measured first: besides being figures
    # of their own, their second or so of GPU work takes the clocks out of
    # the idle state the GPU sits in while the inputs are drawn, so that the
    # timed steps see the sustained state even after a short warm-up (from
    # idle, the first ~10 ms of alternating steps run up to 10% slower).
    # The backward figure takes O and lse from one forward call.
    supp = None
    if args.supplementary == "before":
        step()
        supp = supplementary(osm, wa, ws, q, k, v, x, O, lse)
    for _ in range(args.warmup):
        step()
        if args.copy_probe:
            cdst.copy_(csrc)
    torch.cuda.synchronize()

    # Timed region: K steps, each one attention launch followed by one row
    # softmax launch, between two device synchronisations (wall clock per
    # step).  HIP events recorded on the launch stream (torch's current
    # stream) before the attention, between the two launches and after the
    # softmax give each kernel's launch duration; their means over the K
    # steps are the per-kernel figures.
    K = args.steps
    timer = KernelTimer(torch)
    ev = [[timer.event() for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        timer.record(e[0])
        osm.attention(q, k, v, causal=wa.causal, out=O, lse=lse)
        timer.record(e[1])
        osm.softmax(x, out=y)
        timer.record(e[2])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe:
        for _ in range(K):
            cdst.copy_(csrc)
        torch.cuda.synchronize()

    attn_t = [timer.ms(e[0], e[1]) for e in ev]
    sm_t = [timer.ms(e[1], e[2]) for e in ev]
    timer.free()
    attn_ms, sm_ms = sum(attn_t) / K, sum(sm_t) / K
    attn_tflops = wa.flops / (attn_ms * 1e-3) / 1e12
    sm_gbs = ws.bytes / (sm_ms * 1e-3) / 1e9
    # Algorithmic HBM bytes of the attention kernel: Q, K, V read once, O and
    # lse written once.
    attn_bytes = 4 * wa.B * wa.H * wa.N * wa.d * 2 + wa.B * wa.H * wa.N * 4
    traffic_attn = measured_traffic("attn_fwd_bf16_B2H16N4096d128_causal", ATTN_SOURCES)
    traffic_sm = measured_traffic("row_softmax_32768x8192", SOFTMAX_SOURCES)

    out = {
        "metric": METRIC,
        "value": round(attn_tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn, resident in HBM)",
        "config": {"workload": f"{wa.name} + {ws.name}", "B": wa.B, "H": wa.H, "N": wa.N,
                   "d": wa.d, "causal": wa.causal, "softmax_shape": [ws.B, ws.N],
                   "seeds": [wa.seed, ws.seed]},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_attn,
                     "kernel": "attn_fwd_bf16_pp_kernel", "kernel_ms": round(attn_ms, 4),
                     "kernel_ms_median": round(median(attn_t), 4),
                     "kernel_ms_min": round(min(attn_t), 4),
                     "flops_per_launch": wa.flops, "algorithmic_bytes": attn_bytes,
                     "timer": TIMER},
        "softmax": {"value": round(sm_gbs, 1), "unit": "GB/s", "kernel_ms": round(sm_ms, 4),
                    "kernel_ms_median": round(median(sm_t), 4),
                    "kernel_ms_min": round(min(sm_t), 4)},
        "device": device_info(torch),
        "roofline_softmax": {"bound": "hbm", "achieved": round(sm_gbs, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(sm_gbs / PEAK_HBM_GBS, 4),
                             "traffic": traffic_sm, "kernel": "softmax_block_vec4",
                             "algorithmic_bytes": ws.bytes},
        "cpu_baseline": None,
    }
    # The CPU baseline (seconds of host work, GPU idle) comes last.
    if args.supplementary == "after":
        supp = supplementary(osm, wa, ws, q, k, v, x, O, lse)
    out["supplementary"] = supp
    out["supplementary_order"] = args.supplementary
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wa, ws, q_cpu, k_cpu, v_cpu, x_cpu, O, lse, y)
    print(json.dumps(out), flush=True)
    return 0


def supplementary(osm, wa, ws, q, k, v, x, O, lse, reps=30, warm=10, warm_ms=15.0):
    """Figures measured outside the timed region, not part of a step: the same
    attention shape without the causal mask, a plain device copy of the
    softmax input (the practical ceiling for a read-once / write-once
    kernel on this GPU), the split-KV forward on long rows, the backward pass
    of the headline workload (its FLOPs counted as 2.5 times the forward's,
    the five products of the gradient; the kernels compute seven), the
    split backward on the long-row input, and the fp8 forward on the headline
    shape with per-tensor and with block scales (and the block quantizers)."""
    import torch

    from online_softmax_08_amd import inputs

    def launch_times(fn):
        # at least `warm` launches and warm_ms of back-to-back launches, so
        # that each figure is taken at the clocks that workload settles at
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + warm_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
        timer = KernelTimer(torch)
        ev = [(timer.event(), timer.event()) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            timer.record(a)
            fn()
            timer.record(b)
        torch.cuda.synchronize()
        t = [timer.ms(a, b) for a, b in ev]
        timer.free()
        return t

    def per_launch_ms(fn):
        t = launch_times(fn)
        return sum(t) / len(t)

    # Every attention workload of the parity suite at its own size (the
    # causal N = 4096 one is the timed headline above), each as its own
    # sequence of launches: counted FLOPs over the mean, median and fastest
    # launch, against the matrix-core peak of its arithmetic type.
    configs = {}
    for name, w in inputs.ATTN.items():
        if name == wa.name:
            continue
        qc, kc, vc = (t.to(q.device) for t in inputs.attn_inputs(w))
        Oc = torch.empty_like(qc)
        lc = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
        t = launch_times(lambda: osm.attention(qc, kc, vc, causal=w.causal, out=Oc, lse=lc))
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
        tf = w.flops / (median(t) * 1e-3) / 1e12
        configs[name] = {"shape": [w.B, w.H, w.N, w.d], "causal": w.causal, "dtype": w.dtype,
                         "tflops_median": round(tf, 2),
                         "tflops_mean": round(w.flops / (sum(t) / len(t) * 1e-3) / 1e12, 2),
                         "frac_median": round(tf / peak, 4), "peak_tflops": peak,
                         "ms_median": round(median(t), 4), "ms_min": round(min(t), 4),
                         "ms_mean": round(sum(t) / len(t), 4)}
        del qc, kc, vc, Oc, lc

    # The fp32 kernel on an input large enough to fill the chip (the fp32
    # workload above is one workgroup and launch-bound): the headline shape's
    # fp32 draws, both masks.
    wf = inputs.ATTN[inputs.HEADLINE_ATTN]
    qf, kf, vf = (t.float().to(q.device) for t in inputs.attn_inputs(wf))
    Of = torch.empty_like(qf)
    lf = torch.empty((wf.B, wf.H, wf.N), dtype=torch.float32, device=q.device)
    f32_large = {"workload": f"fp32 B={wf.B} H={wf.H} N={wf.N} d={wf.d} (the headline draws in fp32)",
                 "peak_tflops": PEAK_FP32_MFMA_TFLOPS}
    for causal in (False, True):
        t = launch_times(lambda: osm.attention(qf, kf, vf, causal=causal, out=Of, lse=lf))
        flops = 4.0 * wf.B * wf.H * wf.N * wf.N * wf.d / (2 if causal else 1)
        tf = flops / (median(t) * 1e-3) / 1e12
        f32_large["causal" if causal else "noncausal"] = {
            "tflops_median": round(tf, 1), "frac_median": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
            "ms_median": round(median(t), 4), "ms_min": round(min(t), 4)}
    del qf, kf, vf, Of, lf

    O2 = torch.empty_like(q)
    lse2 = torch.empty((wa.B, wa.H, wa.N), dtype=torch.float32, device=q.device)
    nc_ms = per_launch_ms(lambda: osm.attention(q, k, v, causal=False, out=O2, lse=lse2))
    nc_flops = 4.0 * wa.B * wa.H * wa.N * wa.N * wa.d
    dst = torch.empty_like(x)
    cp_ms = per_launch_ms(lambda: dst.copy_(x))
    # Split-KV on long rows and few heads (256-row query blocks alone would
    # cover an eighth of the CUs), next to the single pass on the same input.
    B, H, N, d = 1, 2, 8192, 128
    g = torch.Generator().manual_seed(5)
    qs, ks, vs = (torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).to(q.device)
                  for _ in range(3))
    split = {"workload": f"bf16 B={B} H={H} N={N} d={d}"}
    for causal in (False, True):
        ns, ws_bytes = osm.attn_fwd_splitkv_plan(B, H, N, d, causal, 0)
        wsp = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        flops = 4.0 * B * H * N * N * d / (2 if causal else 1)
        t_split = per_launch_ms(lambda: osm.attention_splitkv(qs, ks, vs, causal=causal,
                                                              nsplit=ns, workspace=wsp))
        t_one = per_launch_ms(lambda: osm.attention(qs, ks, vs, causal=causal))
        split["causal" if causal else "noncausal"] = {
            "nsplit": ns, "split_tflops": round(flops / (t_split * 1e-3) / 1e12, 1),
            "single_pass_tflops": round(flops / (t_one * 1e-3) / 1e12, 1),
            "split_ms": round(t_split, 4), "single_pass_ms": round(t_one, 4)}
    # Packed variable-length sequences (8 lengths from 387 to 7007, 16 heads,
    # d = 128) beside the same sequences padded to the longest.
    lengths = [7007, 5311, 4312, 2397, 2699, 581, 853, 387]
    Hv, dv, Lmax, tot = 16, 128, max(lengths), sum(lengths)
    g = torch.Generator().manual_seed(11)
    qv, kv_, vv = (torch.randn((Hv, tot, dv), generator=g).to(torch.bfloat16).to(q.device)
                   for _ in range(3))
    qp, kp, vp = (torch.randn((len(lengths), Hv, Lmax, dv), generator=g).to(torch.bfloat16)
                  .to(q.device) for _ in range(3))
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lengths)), dtype=torch.int32,
                      device=q.device)
    varlen = {"workload": f"bf16 H={Hv} d={dv}, sequence lengths {lengths}"}
    for causal in (False, True):
        useful = sum(4.0 * Hv * n * n * dv / (2 if causal else 1) for n in lengths)
        t_packed = per_launch_ms(lambda: osm.attention_varlen(qv, kv_, vv, cu, Lmax, causal=causal))
        t_padded = per_launch_ms(lambda: osm.attention(qp, kp, vp, causal=causal))
        varlen["causal" if causal else "noncausal"] = {
            "packed_tflops_useful": round(useful / (t_packed * 1e-3) / 1e12, 1),
            "packed_ms": round(t_packed, 4), "padded_ms": round(t_padded, 4)}
    # Backward of the headline workload, from the timed forward's O and lse.
    go = inputs.grad_output(q.shape, wa.seed + 1).to(q.device)
    wsb = torch.empty(osm.attn_bwd_workspace_bytes(wa.B, wa.H, wa.N), dtype=torch.uint8,
                      device=q.device)
    bwd_ms = per_launch_ms(lambda: osm.attention_backward(q, k, v, O, lse, go, causal=wa.causal,
                                                          workspace=wsb))
    bwd_flops = 2.5 * 4.0 * wa.B * wa.H * wa.N * wa.N * wa.d / (2 if wa.causal else 1)
    # Backward on few heads (the split-KV input above): the split backward at
    # the library's range count beside the unsplit call.
    gs = inputs.grad_output(qs.shape, 6).to(q.device)
    bsplit = {"workload": f"bf16 B={B} H={H} N={N} d={d} backward"}
    for causal in (False, True):
        Os, ls = osm.attention(qs, ks, vs, causal=causal)
        ns, ws_bytes = osm.attn_bwd_split_plan(B, H, H, N, d, causal, 0)
        wsp = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        ws1 = torch.empty(osm.attn_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=q.device)
        flops = 2.5 * 4.0 * B * H * N * N * d / (2 if causal else 1)
        t_split = per_launch_ms(lambda: osm.attention_backward_split(
            qs, ks, vs, Os, ls, gs, causal=causal, nsplit=ns, workspace=wsp))
        t_one = per_launch_ms(lambda: osm.attention_backward(qs, ks, vs, Os, ls, gs, causal=causal,
                                                             workspace=ws1))
        bsplit["causal" if causal else "noncausal"] = {
            "nsplit": ns, "split_tflops": round(flops / (t_split * 1e-3) / 1e12, 1),
            "unsplit_tflops": round(flops / (t_one * 1e-3) / 1e12, 1),
            "split_ms": round(t_split, 4), "unsplit_ms": round(t_one, 4)}
    # The fp8 forward on the headline workload's shape and recipe (every
    # 64th query row x8), each tensor stored as E4M3 with its own scale,
    # with and without the mask; FLOPs as for bf16, against the fp8 peak.
    (q8, k8, v8), sc8 = inputs.attn_inputs_fp8(wa)
    q8, k8, v8 = q8.to(q.device), k8.to(q.device), v8.to(q.device)
    fp8 = {"workload": f"fp8 (E4M3, per-tensor scales) B={wa.B} H={wa.H} N={wa.N} d={wa.d}, "
                       f"every {wa.boost_every}th query row x{wa.boost:g}",
           "peak_tflops": PEAK_FP8_TFLOPS}
    for causal in (False, True):
        t = launch_times(lambda: osm.attention_fp8(q8, k8, v8, *sc8, causal=causal))
        flops = 4.0 * wa.B * wa.H * wa.N * wa.N * wa.d / (2 if causal else 1)
        tf = flops / (median(t) * 1e-3) / 1e12
        fp8["causal" if causal else "noncausal"] = {
            "tflops_median": round(tf, 1), "frac_median": round(tf / PEAK_FP8_TFLOPS, 4),
            "ms_median": round(median(t), 4), "ms_min": round(min(t), 4)}
    # The block-quantized fp8 forward on the same inputs: Q and K rotated
    # (random signs, Hadamard) and quantized with a power-of-two scale per 32
    # head columns, V per 32 keys of a column, by the library's quantizers
    # (timed on their own, HBM bytes: 2 read + 1 + 1/32 written per element);
    # the attention against the fp8 peak.
    signs = inputs.hadamard_signs(wa.d, seed=wa.seed + 1)
    qm, qsm = osm.quantize_fp8_rows(q, signs)
    km, ksm = osm.quantize_fp8_rows(k, signs)
    vm, vsm = osm.quantize_fp8_cols(v)
    # The quantizers take ~10 us at this size, less than the host needs to
    # issue a call, so they are timed on the batch repeated 4 times, 20
    # launches back to back between two events (the launches queue up and
    # the figure is the kernels' own rate).
    q4, v4 = q.repeat(4, 1, 1, 1), v.repeat(4, 1, 1, 1)
    qbytes = q4.numel() * (3 + 1 / 32)

    def back_to_back_ms(fn, n=20):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        timer = KernelTimer(torch)
        e0, e1 = timer.event(), timer.event()
        timer.record(e0)
        for _ in range(n):
            fn()
        timer.record(e1)
        torch.cuda.synchronize()
        t = timer.ms(e0, e1) / n
        timer.free()
        return t
    t_rows = back_to_back_ms(lambda: osm.quantize_fp8_rows(q4, signs))
    t_cols = back_to_back_ms(lambda: osm.quantize_fp8_cols(v4))
    del q4, v4
    fp8mx = {"workload": f"fp8 (E4M3, block scales per 32 elements, Q and K rotated) "
                         f"B={wa.B} H={wa.H} N={wa.N} d={wa.d}, inputs of the headline recipe; "
                         f"quantizers on B={4 * wa.B}",
             "peak_tflops": PEAK_FP8_TFLOPS,
             "quantize_rows_rotated_gbs": round(qbytes / (t_rows * 1e-3) / 1e9, 1),
             "quantize_cols_gbs": round(qbytes / (t_cols * 1e-3) / 1e9, 1),
             "quantize_rows_ms": round(t_rows, 4), "quantize_cols_ms": round(t_cols, 4)}
    for causal in (False, True):
        t = launch_times(lambda: osm.attention_fp8_mx(qm, qsm, km, ksm, vm, vsm, causal=causal))
        flops = 4.0 * wa.B * wa.H * wa.N * wa.N * wa.d / (2 if causal else 1)
        tf = flops / (median(t) * 1e-3) / 1e12
        fp8mx["causal" if causal else "noncausal"] = {
            "tflops_median": round(tf, 1), "frac_median": round(tf / PEAK_FP8_TFLOPS, 4),
            "ms_median": round(median(t), 4), "ms_min": round(min(t), 4)}
    return {
        "attn_fp8": fp8,
        "attn_fp8_block": fp8mx,
        "attn_backward": {"workload": f"{wa.name} backward (dQ, dK, dV)",
                          "value": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1), "unit": "TFLOPS",
                          "flops_per_call": bwd_flops, "call_ms": round(bwd_ms, 4)},
        "attn_noncausal": {"workload": f"bf16 B={wa.B} H={wa.H} N={wa.N} d={wa.d}, no mask",
                           "value": round(nc_flops / (nc_ms * 1e-3) / 1e12, 2), "unit": "TFLOPS",
                           "kernel_ms": round(nc_ms, 4)},
        "hbm_copy": {"workload": f"device copy of the fp32 [{ws.B}, {ws.N}] softmax input",
                     "value": round(ws.bytes / (cp_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                     "kernel_ms": round(cp_ms, 4)},
        "attn_splitkv": split,
        "attn_backward_split": bsplit,
        "attn_varlen": varlen,
        "attn_configs": configs,
        "attn_f32_large": f32_large,
    }


def cpu_baseline(wa, ws, q_cpu, k_cpu, v_cpu, x_cpu, O, lse, y):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload, on this host's cores; also report the GPU's max-abs error on
    that sample."""
    import numpy as np
    import torch

    import oracle

    n_slices = wa.B * wa.H  # every (batch, head) slice, every query row of each
    bh = np.repeat(np.arange(n_slices), wa.N)
    qi = np.tile(np.arange(wa.N), n_slices)
    Q = q_cpu.reshape(wa.B * wa.H, 1, wa.N, wa.d)[:n_slices].reshape(1, n_slices, wa.N, wa.d)
    Kc = k_cpu.reshape(wa.B * wa.H, 1, wa.N, wa.d)[:n_slices].reshape(1, n_slices, wa.N, wa.d)
    Vc = v_cpu.reshape(wa.B * wa.H, 1, wa.N, wa.d)[:n_slices].reshape(1, n_slices, wa.N, wa.d)
    Qd, Kd, Vd = (t.to(torch.float64).numpy() for t in (Q, Kc, Vc))
    t0 = time.perf_counter()
    Oref, lref = oracle.attn_rows(Qd, Kd, Vd, wa.scale, wa.causal, bh, qi)
    dt = time.perf_counter() - t0
    flops = n_slices * 4.0 * wa.d * (wa.N * (wa.N + 1) / 2 if wa.causal else wa.N * wa.N)
    Og = O.reshape(wa.B * wa.H, wa.N, wa.d)[:n_slices].reshape(-1, wa.d).double().cpu().numpy()
    lg = lse.reshape(wa.B * wa.H, wa.N)[:n_slices].reshape(-1).double().cpu().numpy()

    rows = 4096
    xs = x_cpu[:rows].to(torch.float64).numpy()
    t1 = time.perf_counter()
    yref = oracle.row_softmax(xs)
    dts = time.perf_counter() - t1
    ys = y[:rows].double().cpu().numpy()
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"attention: all {n_slices} (batch, head) slices x all {wa.N} query rows, "
                  f"fp64 three-pass ({dt:.2f} s); softmax: {rows} of {ws.B} rows ({dts:.2f} s)",
        "seconds": round(dt, 3),
        "softmax_gbs": round(rows * ws.N * 8 / dts / 1e9, 4),
        "max_abs_err_O": float(np.max(np.abs(Og - Oref))),
        "max_abs_err_lse": float(np.max(np.abs(lg - lref))),
        "max_abs_err_softmax": float(np.max(np.abs(ys - yref))),
    }


if __name__ == "__main__":
    sys.exit(main())
