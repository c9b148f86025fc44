#!/usr/bin/env python
"""Absorbed-MLA decode benchmark on one MI355X.

One step = the whole hot path for one batch: W^UK absorption into the query
with the split planner in the same launch -> paged split-KV attention over
the latent cache -> partition merge fused with the W^UV up-projection, issued
as three mla_decode_step_stages calls with HIP events recorded by this script
on the launch stream around the attention launch of every 4th step, so the
step time and the attention kernel's own time come from the same timed steps
(a pair of events adds ~4 us to its step; sampling keeps that under 1 us per
step on average).  Inputs are
seeded synthetic tensors already resident in HBM; the timed region rotates
through several physically distinct copies of the latent cache so repeated
steps cannot be served from the 256 MB last-level cache.

Before the W warm-up steps the device is settled: started from idle, MI355X
runs this step 10-20 % slower for its first ~100-200 executions (20-40 ms;
GEMM or copy loads do not bring it there), so a few-millisecond run would
time that ramp instead of the serving state.  The step runs untimed until
the time per 10 steps is stable (at most --settle-ms); the JSON line reports
the settle (steps, ms) beside the W warm-up and K timed steps.

After the timed steps: the same steps as one mla_decode_step call each (for
comparison), a per-stage breakdown, the separate entry points (mla_absorb_q,
mla_decode_absorbed, mla_up_proj_v), the secondary paths (cache producer,
MHA-mode prefill, GQA-path decode; each settled on itself the same way before
it is timed), an HBM copy probe and the float64 oracle on a bounded sample of
the workload on the host cores.

Prints one JSON line.  Metric: latent-cache bytes read per second (TB/s) of
the whole step, with decode tokens/s and the roofline fractions alongside.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-KV TB/s + decode tok/s, absorbed MLA n_h=128 B=64 ctx 8K, % roofline"
HEADLINE = "v3_bf16_B64_ctx8192"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
CSRC = os.path.join(ROOT, "mla_latent_kv_05_amd", "csrc")
# sources of the bf16-cache attention kernel (the traffic counters are tied to them)
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("decode_mfma.hip", "mfma_common.h", "device_util.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_pipe_kernel_bf16_B64_ctx8192_traffic.md")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    if workload != HEADLINE or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("traffic:"):
            for kv in line.split()[1:]:
                k, _, v = kv.partition("=")
                fields[k] = v
    if fields.get("kernel_sha256_16") != kernel_hash():
        return None
    try:
        return int(fields["bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _oracle_rate(case, P, seconds: float, start: int = 0):
    """The float64 oracle on whole sequences of the workload (gather pages,
    absorb, decode, up-project) in batch order from `start` until `seconds`
    have passed; returns (latent bytes/s, tokens/s, sequences, seconds)."""
    import oracle
    qc = oracle.bf16_to_f64(P["q_c"]).reshape(case.B, case.s_q, case.n_h, case.d_h)
    wuk = oracle.bf16_to_f64(P["w_uk"])
    wuv = oracle.bf16_to_f64(P["w_uv"])
    done, nbytes, t0 = 0, 0, time.perf_counter()
    while True:
        b = (start + done) % case.B
        _, qr, c, kr = oracle.decode_case_rows(case, b)
        ql = oracle.absorb_q(qc[b], wuk, case.n_h, case.d_h)
        o_lat, _ = oracle.mqa_decode_rows(ql, qr, c, kr, case.softmax_scale)
        oracle.up_proj_v(o_lat, wuv, case.n_h, case.d_h)
        done += 1
        nbytes += int(case.seq_lens[b]) * case.row_bytes
        el = time.perf_counter() - t0
        if el >= seconds:
            return nbytes / el, done * case.s_q / el, done, el


def cpu_baseline(case, P, seconds: float) -> dict:
    """The float64 oracle on a bounded sample of the same workload, reported
    in the GPU's unit: three runs with the BLAS thread pool as numpy has it
    (median reported) and one run limited to a single thread (the per-core
    figure), each taking a quarter of `seconds`."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        pools = threadpool_info()
    except Exception:  # noqa: BLE001
        threadpool_info, threadpool_limits, pools = None, None, []
    blas = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "architecture", "threading_layer")}
            for p in pools if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in pools] or [os.cpu_count() or 1])
    part = seconds / 4
    runs = [_oracle_rate(case, P, part, start=r * 7) for r in range(3)]
    rates = sorted(r[0] for r in runs)
    med = rates[1]
    med_run = next(r for r in runs if r[0] == med)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1 = _oracle_rate(case, P, part, start=21)
        single = {"value": r1[0] / 1e12, "unit": "TB/s", "cores": 1, "tok_s": r1[1], "sequences": r1[2],
                  "seconds": r1[3]}
    return {"value": med / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole sequences of the workload in batch order ({case.B} in the batch; page gather, "
                      f"W^UK absorb, decode, W^UV in float64 numpy), {part:.1f} s per run; median of 3 runs "
                      f"({', '.join(str(r[2]) for r in runs)} sequences); rate = latent bytes of those "
                      f"sequences / time",
            "runs_TBps": [r / 1e12 for r in rates], "tok_s": med_run[1], "seconds": sum(r[3] for r in runs),
            "per_core": single, "blas": blas}


def stream_probe(dev, mib: int = 2048, reps: int = 10) -> dict:
    """Achievable HBM stream rate on this device: a plain device-to-device
    copy of `mib` MiB (read + write bytes per second), timed with events."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(3)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"kind": "device copy", "bytes_moved": 2 * n, "ms": ms, "GBps": 2 * n / (ms * 1e-3) / 1e9,
            "frac_of_peak": 2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def settle_device(run_step, max_ms: float, min_ms: float = 50.0, window: int = 10, tol: float = 0.02) -> dict:
    """Bring the device from idle to the state it holds while serving before
    the warm-up steps.  Started from idle, MI355X runs this step 10-20 %
    slower for its first ~100-200 executions (~20-40 ms); GEMM or copy loads of
    any length do not reach that state, the step itself does.  So the step
    runs untimed in windows of `window` until two consecutive windows agree
    within `tol` (at least `min_ms`, at most `max_ms`); the JSON line reports
    how many steps and milliseconds that took."""
    import torch
    if max_ms <= 0:
        return {"kind": None, "steps": 0, "ms": 0.0}
    t0 = time.perf_counter()
    prev, n, stable = None, 0, False
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(window):
            run_step(n)
            n += 1
        e1.record()
        torch.cuda.synchronize()
        cur = e0.elapsed_time(e1) / window
        el = (time.perf_counter() - t0) * 1e3
        stable = prev is not None and abs(cur - prev) <= tol * prev
        if (stable and el >= min_ms) or el >= max_ms:
            break
        prev = cur
    return {"kind": "the measured step, untimed, until two consecutive windows of "
                    f"{window} steps agree within {tol:.0%}", "steps": n, "ms": el, "stable": stable,
            "last_window_ms_per_step": cur}


def device_info(dev) -> dict:
    """Software versions and the device's compute clock as the amdgpu kernel
    module lists it (the sclk levels of the card in sysfs, where readable)."""
    import glob

    import torch
    p = torch.cuda.get_device_properties(dev)
    info = {"torch": torch.__version__, "hip": torch.version.hip, "device": p.name,
            "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1)}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    sclk = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            lines = [ln.strip() for ln in open(f) if ln.strip()]
        except OSError:
            continue
        if lines:
            sclk.append({"card": f.split("/")[4], "levels": lines})
    info["sclk"] = sclk or None
    return info


def copy_probe(mib: int) -> int:
    """A plain copy of known size: HBM counters (FETCH_SIZE / WRITE_SIZE) read
    on it give the bytes-per-count scale used for the decode kernel."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
    return 0


def bench_append(case, steps: int, dev) -> dict:
    """The cache producer for the step's new tokens (T = B * s_q, V3 hidden
    size 7168): projection through [W^DKV; W^KR], RoPE, storage in the cache's
    format.  Weight-bound: algorithmic bytes = the stacked weight + the hidden
    states read once + the rows written."""
    import torch
    from mla_latent_kv_05_amd import binding, inputs
    T, d, d_c, d_r = case.B * case.s_q, 7168, case.d_c, case.d_r
    inp = inputs.append_inputs(7, T, d=d, d_c=d_c, d_r=d_r, num_blocks=max(2, (T + 63) // 64 + 1))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    h, w = bf(inp["h"]), bf(inp["w"])
    pos, slots = torch.from_numpy(inp["pos"]).to(dev), torch.from_numpy(inp["slots"]).to(dev)
    if case.kv_dtype == "bf16":
        cache = torch.zeros((inp["num_blocks"], 64, d_c + d_r), dtype=torch.bfloat16, device=dev)
        kdt, row_b = binding.MLA_BF16, (d_c + d_r) * 2
    else:
        cache = torch.zeros((inp["num_blocks"], 64 * (d_c + 2 * d_r + 4)), dtype=torch.uint8, device=dev)
        kdt, row_b = binding.MLA_FP8_E4M3, d_c + 2 * d_r + 4
    ws = binding.cache_append_workspace(T, d, d_c, d_r, device=dev)

    def run():
        binding.cache_append(h, w, pos, slots, cache, d_c, d_r, 64, kv_dtype=kdt, workspace=ws)
    settle = settle_device(lambda i: run(), 300.0)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(20, steps)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    algo = (d_c + d_r) * d * 2 + T * d * 2 + T * row_b
    gbs = algo / (us * 1e-6) / 1e9
    return {"tokens": T, "d": d, "kv_dtype": case.kv_dtype, "us_per_call": us, "algorithmic_bytes": algo,
            "achieved_GBps": gbs, "bound": "hbm", "peak_GBps": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
            "settle_ms": round(settle["ms"], 1)}


PREFILL_T = 4096
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(steps: int, dev, T: int = PREFILL_T) -> dict:
    """MHA-mode prefill of one T-token sequence at V3 heads (128 heads, d_h 128,
    d_r 64, d_c 512, bf16): the key/value expansion from the latent and the
    causal attention.  MFMA-bound: algorithmic flops of the attention =
    2 * (d_h + d_r + d_h) * n_h * T(T+1)/2 (QK^T and PV over the causal
    triangle); of the expansion 2 * 2 * T * d_c * n_h * d_h."""
    import torch
    from mla_latent_kv_05_amd import binding
    n_h, d_h, d_r, d_c = 128, 128, 64, 512
    g = torch.Generator(device=dev)
    g.manual_seed(17)

    def rn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)
    c_kv = rn(T, d_c)
    w_uk, w_uv = rn(n_h * d_h, d_c, std=d_c ** -0.5), rn(n_h * d_h, d_c, std=d_c ** -0.5)
    q, k_r = rn(T, n_h, d_h + d_r), rn(T, d_r)
    scale = (d_h + d_r) ** -0.5

    def timed(fn, n):
        settle_device(lambda i: fn(), 300.0)  # the op itself, untimed, until its rate is stable
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3
    k_c, v_c = binding.expand_kv(c_kv, w_uk, w_uv, d_h)
    n = max(10, min(steps, 50))
    us_exp = timed(lambda: binding.expand_kv(c_kv, w_uk, w_uv, d_h), n)
    us_att = timed(lambda: binding.prefill_mha(q, k_c, k_r, v_c, scale), n)
    # the same two products through torch's vendor GEMM, for context
    w_uk_t, w_uv_t = w_uk.t().contiguous(), w_uv.t().contiguous()
    us_vendor = timed(lambda: (torch.mm(c_kv, w_uk_t), torch.mm(c_kv, w_uv_t)), n)
    fl_att = 2.0 * (d_h + d_r + d_h) * n_h * T * (T + 1) / 2
    fl_exp = 2.0 * 2 * T * d_c * n_h * d_h
    tf_att = fl_att / (us_att * 1e-6) / 1e12
    tf_exp = fl_exp / (us_exp * 1e-6) / 1e12
    return {"tokens": T, "n_h": n_h, "d_qk": d_h + d_r, "d_v": d_h, "dtype": "bf16",
            "attention": {"us_per_call": us_att, "algorithmic_flops": fl_att, "achieved_TFLOPs": tf_att,
                          "bound": "mfma", "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                          "frac": tf_att / MFMA_BF16_PEAK_TFLOPS},
            "expand_kv": {"us_per_call": us_exp, "algorithmic_flops": fl_exp, "achieved_TFLOPs": tf_exp,
                          "bound": "mfma", "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                          "frac": tf_exp / MFMA_BF16_PEAK_TFLOPS,
                          "torch_mm_same_products_us": us_vendor},
            "timing": "each op runs untimed until two 10-call windows agree within 2 % (at most 300 ms), "
                      "then 3 untimed calls and the timed ones"}


def bench_gqa(steps: int, dev, B: int = 64, L: int = 8192) -> dict:
    """GQLA's GQA decode path on the same context: B sequences of L tokens,
    8 groups of 16 heads, two new tokens per step (MTP), bf16 per-group
    expanded cache.  HBM-bound: algorithmic bytes = every cached token's
    (2 * 8 * 128 + 64) * 2 = 4224 bytes read once."""
    import torch
    from mla_latent_kv_05_amd import binding
    n_h, n_g, d_h, d_r, s_q, bs = 128, 8, 128, 64, 2, 64
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    nb = B * ((L + bs - 1) // bs)
    row = 2 * n_g * d_h + d_r
    cache = torch.randn(nb, bs * row, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    perm = torch.randperm(nb, generator=g, device=dev).to(torch.int32)
    table = perm.view(B, -1).contiguous()
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_c = torch.randn(B, s_q, n_h, d_h, generator=g, device=dev).to(torch.bfloat16)
    q_r = torch.randn(B, s_q, n_h, d_r, generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty(B, s_q, n_h, d_h, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, s_q, n_h, dtype=torch.float32, device=dev)
    scale = (d_h + d_r) ** -0.5

    def run():
        binding.gqa_decode(q_c, q_r, cache, table, lens, n_g, scale, out=o, lse=lse)
    settle = settle_device(lambda i: run(), 300.0)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(10, min(steps, 50))
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    algo = B * L * row * 2
    gbs = algo / (us * 1e-6) / 1e9
    return {"B": B, "ctx": L, "s_q": s_q, "n_g": n_g, "bytes_per_token": row * 2, "us_per_call": us,
            "algorithmic_bytes": algo, "achieved_GBps": gbs, "bound": "hbm", "peak_GBps": HBM_PEAK_GBS,
            "frac": gbs / HBM_PEAK_GBS, "decode_tok_s": B * s_q / (us * 1e-6), "settle_ms": round(settle["ms"], 1)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--copies", type=int, default=4, help="physically distinct cache copies rotated per step")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic split planning")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="timed steps launched eagerly from Python, or replayed from captured HIP graphs "
                         "(one per cache copy; on this stack a replay costs more than the eager launches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-producer measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the MHA-mode prefill measurement")
    ap.add_argument("--no-gqa", action="store_true", help="skip the GQA-path decode measurement")
    ap.add_argument("--no-stream-probe", action="store_true", help="skip the device-copy bandwidth probe")
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the kernel's events around the attention launch of every N-th timed step "
                         "(each pair adds ~4 us to its step)")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="at most this many milliseconds of untimed steps before the warm-up steps, ending once the "
                         "per-step time is stable, to bring the device from idle to its serving state (0 = none)")
    ap.add_argument("--step-api", choices=("staged", "fused", "separate"), default="staged",
                    help="time the step as three mla_decode_step_stages calls with events around the attention "
                         "launch (default: step and kernel times from the same steps), as one mla_decode_step "
                         "call, or as mla_absorb_q + mla_decode_absorbed + mla_up_proj_v")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the reference kernel "
                         "for scaling HBM traffic counters) and exit")
    args = ap.parse_args()
    if args.event_every < 1:
        ap.error("--event-every must be at least 1")
    if args.copy_probe:
        return copy_probe(args.copy_probe)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    import torch

    from mla_latent_kv_05_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()

    w = inputs.WORKLOADS[args.workload]
    assert w["kind"] == "decode", "bench.py times the decode workloads"
    case = inputs.workload_case(args.workload)
    B, s_q, n_h, d_c, d_r, d_h = case.B, case.s_q, case.n_h, case.d_c, case.d_r, case.d_h
    T_q = B * s_q
    P = inputs.projection_weights(w["seed"] + 100, T_q=T_q, n_h=n_h, d_h=d_h, d_c=d_c)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if case.kv_dtype == "bf16":
        base = bf(case.cache)
    else:
        base = torch.from_numpy(np.ascontiguousarray(case.cache)).to(dev)
    kv_dtype = {"bf16": binding.MLA_BF16, "fp8": binding.MLA_FP8_E4M3, "int4": binding.MLA_INT4,
                "int2": binding.MLA_INT2}[case.kv_dtype]
    fmt = {"bf16": 0, "fp8": 1, "int4": 2, "int2": 3}[case.kv_dtype]  # the kernel's template argument
    caches = [base] + [base.clone() for _ in range(max(0, args.copies - 1))]
    table = torch.from_numpy(np.maximum(case.block_table, 0).astype(np.int32)).to(dev)
    lens = torch.from_numpy(case.seq_lens.astype(np.int32)).to(dev)
    q_c, w_uk, w_uv = bf(P["q_c"]), bf(P["w_uk"]), bf(P["w_uv"])
    q_rope = bf(case.q_rope)
    q_lat = torch.empty((T_q, n_h, d_c), dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty((B, s_q, n_h, d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, n_h), dtype=torch.float32, device=dev)
    o = torch.empty((T_q, n_h, d_h), dtype=torch.bfloat16, device=dev)
    ws = binding.alloc_workspace(B, s_q, n_h, d_c, table.shape[1], args.splits, device=dev)
    scale = 1.0 / math.sqrt(d_h + d_r)

    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
          for k in ("a", "b", "c", "d", "k0", "k1")}

    qn4 = q_c.view(B, s_q, n_h, d_h)
    ws_step = binding.decode_step_workspace(B, s_q, n_h, d_c, table.shape[1], args.splits, device=dev)
    step_args = lambda i: (qn4, w_uk, q_rope, caches[i % len(caches)], table, lens, w_uv, scale)  # noqa: E731
    step_kw = dict(kv_dtype=kv_dtype, num_splits=args.splits, workspace=ws_step, out=o.view(B, s_q, n_h, d_h),
                   lse=lse)

    def fused_step(i):
        """absorb + attention + merge fused with W^UV: one library call, three launches"""
        binding.decode_step(*step_args(i), **step_kw)

    def staged_step(i, tag=("k0", "k1"), only_kernel=True):
        """the same three launches as three calls of mla_decode_step_stages,
        with this script's own events on the launch stream around the
        attention stage of every --event-every'th step (a pair of events
        costs ~4 us of step time) and, for the breakdown, around every stage
        of every step"""
        sample = not only_kernel or i % args.event_every == 0
        i %= args.steps + 1
        if not only_kernel:
            ev["a"][i].record()
        binding.decode_step_stages(binding.MLA_STAGE_ABSORB, *step_args(i), **step_kw)
        if sample:
            ev[tag[0]][i].record()
        binding.decode_step_stages(binding.MLA_STAGE_ATTEND, *step_args(i), **step_kw)
        if sample:
            ev[tag[1]][i].record()
        binding.decode_step_stages(binding.MLA_STAGE_MERGE, *step_args(i), **step_kw)
        if not only_kernel:
            ev["d"][i].record()

    def separate_step(i, timed=False):
        if timed:
            ev["a"][i].record()
        binding.absorb_q(q_c, w_uk, out=q_lat)
        if timed:
            ev["b"][i].record()
        binding.decode(q_lat.view(B, s_q, n_h, d_c), q_rope, caches[i % len(caches)], table, lens, scale,
                       kv_dtype=kv_dtype, d_r=d_r, out=o_lat, lse=lse, workspace=ws, num_splits=args.splits)
        if timed:
            ev["c"][i].record()
        binding.up_proj_v(o_lat.view(T_q, n_h, d_c), w_uv, d_h, out=o)
        if timed:
            ev["d"][i].record()

    # the timed step: by default the three stage calls with events around the
    # attention launch, so the step time and the kernel's own time come from
    # the same timed steps (HIP graphs replay the single call instead)
    api = "fused" if (args.launch == "graph" and args.step_api == "staged") else args.step_api
    step = {"staged": staged_step, "fused": fused_step, "separate": separate_step}[api]
    settle = settle_device(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed_loop(run_steps, n):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        run_steps(n)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n, time.perf_counter() - t0

    def eager_steps(n):
        for i in range(n):
            step(i)

    # one captured HIP graph per cache copy, each holding one whole step
    # (absorb, decode call, up-projection); replays launch the same kernels
    # with no host work between them
    graph_ms = None
    if args.launch == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            eager_steps(len(caches))  # warm the side stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for c in range(len(caches)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

        def graph_steps(n):
            for i in range(n):
                graphs[i % len(graphs)].replay()
        graph_ms, t_wall = timed_loop(graph_steps, args.steps)
    eager_ms, t_eager = timed_loop(eager_steps, args.steps)
    if graph_ms is None:
        t_wall = t_eager
    ms_step = graph_ms if graph_ms is not None else eager_ms

    # The attention kernel's own time: the events this script recorded on the
    # launch stream around every attention launch of the timed steps (the
    # library records nothing).  When the timed step was not the staged one,
    # a second back-to-back loop of staged steps supplies them.
    def kernel_steps(n):
        for i in range(n):
            staged_step(i)

    def fused_steps(n):
        for i in range(n):
            fused_step(i)
    if api == "staged":
        staged_ms = ms_step
        fused_ms, _ = timed_loop(fused_steps, args.steps)  # the single-call API, for comparison
    else:
        staged_ms, _ = timed_loop(kernel_steps, args.steps)
        fused_ms = ms_step if api == "fused" else None
    kernel_all = [ev["k0"][i].elapsed_time(ev["k1"][i]) for i in range(0, args.steps, args.event_every)]
    kernel_ms = float(np.mean(kernel_all))
    kernel_med = float(np.median(kernel_all))
    # per-stage breakdown (events around every stage; not a timed loop)
    for i in range(args.steps):
        staged_step(i, only_kernel=False)
    torch.cuda.synchronize()
    absorb_ms = float(np.mean([ev["a"][i].elapsed_time(ev["k0"][i]) for i in range(args.steps)]))
    merge_ms = float(np.mean([ev["k1"][i].elapsed_time(ev["d"][i]) for i in range(args.steps)]))
    kernel_bd_ms = float(np.mean([ev["k0"][i].elapsed_time(ev["k1"][i]) for i in range(args.steps)]))
    # the separate entry points (absorb, decode call with planner + merge, up-projection)
    for i in range(args.steps):
        separate_step(i, timed=True)
    torch.cuda.synchronize()
    decode_ms = float(np.mean([ev["b"][i].elapsed_time(ev["c"][i]) for i in range(args.steps)]))
    sep_absorb_ms = float(np.mean([ev["a"][i].elapsed_time(ev["b"][i]) for i in range(args.steps)]))
    up_ms = float(np.mean([ev["c"][i].elapsed_time(ev["d"][i]) for i in range(args.steps)]))

    latent_bytes = case.latent_bytes
    value = latent_bytes / (ms_step * 1e-3) / 1e12
    tok_s = T_q / (ms_step * 1e-3)
    flops = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        for i in range(s_q):
            vis = L - s_q + i + 1
            flops += vis * (2 * n_h * (d_c + d_r) + 2 * n_h * d_c)
    # roofline of the dominant kernel: the attention kernel alone, from the
    # events this script records around its launch in the back-to-back loop
    if case.kv_dtype == "bf16":
        achieved = latent_bytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_MFMA_PEAK_TFLOPS}
    kname = f"decode_pipe_kernel<{fmt}>"
    roof["traffic"] = measured_traffic(args.workload)
    roof["kernel"] = kname
    roof["kernel_ms"] = kernel_ms
    roof["kernel_ms_median"] = kernel_med
    roof["timing"] = (f"HIP events recorded by bench.py on the launch stream around the attention launch of every "
                      f"{args.event_every}th step ({len(kernel_all)} launches) of the "
                      + ("timed steps" if api == "staged" else "a second back-to-back loop of whole steps")
                      + " (mla_decode_step_stages, one stage per call)")
    roof["units_per_launch"] = {"tokens": int(case.seq_lens.sum()), "bytes_per_token": case.row_bytes,
                                "flops": flops}
    step_frac = value * 1e3 / HBM_PEAK_GBS

    rec = {
        "metric": METRIC, "value": value, "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"bf16": "bf16", "fp8": "fp8e4m3+bf16", "int4": "int4+bf16", "int2": "int2/int4+bf16"}[case.kv_dtype],
        "data": "synthetic: seeded PCG64 N(0,1) latent cache rounded to bf16 (fp8: per-token amax/448 e4m3fn; "
                "int4/int2: groups of 32 with fp16 scale and min), "
                "q_lat N(0,1/512) from W^UK absorption, shuffled 64-token pages",
        "config": {"workload": args.workload, "n_h": n_h, "d_c": d_c, "d_r": d_r, "d_h": d_h, "B": B,
                   "s_q": s_q, "ctx": int(case.seq_lens.max()) if w["lens"][0] == "fixed" else "log-uniform",
                   "page_tokens": case.block_size, "kv_dtype": case.kv_dtype, "splits": args.splits or "auto",
                   "cache_copies": len(caches), "launch": args.launch, "step_api": api},
        "decode_tok_s": tok_s, "latent_bytes": latent_bytes,
        "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
        # call-level fraction: latent bytes over the whole step (planner,
        # absorption, attention, merge, W^UV); roofline.frac is the kernel's
        "roofline_frac_step": step_frac if case.kv_dtype == "bf16" else None,
        "staged_ms_per_step": staged_ms, "fused_call_ms_per_step": fused_ms,
        "stages_ms_events_between": {"absorb_plan": absorb_ms, "attention": kernel_bd_ms, "merge_up": merge_ms},
        "separate_calls_ms": {"absorb_q": sep_absorb_ms, "decode_absorbed": decode_ms, "up_proj_v": up_ms,
                              "decode_absorbed_TBps": latent_bytes / (decode_ms * 1e-3) / 1e12},
        "wall_s": t_wall,
        "settle": settle,
        "roofline": roof,
        "env": device_info(dev),
    }
    if not args.no_stream_probe:
        rec["stream_probe"] = stream_probe(dev)
    if case.kv_dtype in ("bf16", "fp8") and not args.no_append:
        rec["cache_append"] = bench_append(case, args.steps, dev)
    if not args.no_prefill:
        rec["prefill_mha"] = bench_prefill(args.steps, dev)
    if not args.no_gqa:
        rec["gqa_decode"] = bench_gqa(args.steps, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, P, args.cpu_seconds)
        rec["cpu_baseline"]["cpu_model"] = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                                                 if l.startswith("model name")), platform.processor())
        rec["cpu_baseline"]["affinity_cores"] = len(os.sched_getaffinity(0))
        rec["cpu_baseline"]["numpy"] = np.__version__
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
