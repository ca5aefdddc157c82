"""Benchmark of the BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one prefill pass of a BitNet b1.58 2B4T MLP over M = 4096 tokens, all
on the GPU through the C ABI:
    per-token int8 quantization of x [4096][2560]
    gate|up contraction 2560 -> 2 x 6912 (one weight scale per matrix) + rescale,
        with the ReLU^2 gating in the same kernel: writes [4096][6912]
    ffn_sub_norm folded into the quantization of [4096][6912]
    down contraction 6912 -> 2560 + rescale
Weights are packed once before timing (the packed-checkpoint mode). ``value``
is int8 TOPS of the whole step: 2 M N K of both contractions / step time, the
step time being the time of exactly K steps between two events after the
untimed settling run and the W warmup steps.
``roofline`` is the gated gate|up contraction kernel against dense int8 MFMA peak,
its mean duration over back-to-back launches between two HIP events on the
stream it runs on; its ``traffic`` comes from the
committed counter profile when the kernel source is unchanged since. ``decode``
reports the weight-streaming kernel (M = 1, 4, 16) in packed-weight GB/s against
HBM peak: the mean time per launch over back-to-back launches, each reading a
different copy of the weights from a ring larger than the 256 MB last-level
cache; and the same projection at M = 1 and 4 from the weights stored five
codes per byte (base 3), in GB/s of those stored bytes. ``head`` times the final
norm + bfloat16 lm_head (128256 x 2560) at 1 and 4 tokens in GB/s of the head.
``stack`` times the 30-layer projection stack at M = 1 and 64, and
``stack.token_step`` a whole-model decode step (embedding, 30 layers with RoPE,
KV cache and attention over 4096 positions, final norm, head) for 1 and 4
sequences. ``online`` times the online mode from fp32 and bfloat16 masters;
``kernels`` the step's kernels one by one and the plain (ungated) gate|up
contraction; ``small_configs`` the single-layer and small-FFN workloads;
``peaks_measured`` the HBM read rate and int8 MFMA rate this GPU reaches with the
library's probes (the MFMA rate on fixed operands and on operands that vary like
the GEMMs' do: the second draws more power and runs at a lower clock). ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same step's tokens, on one thread and on the usable host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BitLinear prefill int8 TOPS & decode packed-weight GB/s, % of roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
M, H, I = 4096, 2560, 6912
VOCAB = 128256
ROPE_THETA = 5e5  # rope_theta 500,000 over 4096 positions ([nnterp] "Loading")
ROPE_POSITIONS = 4096
BASE_SEED = 1234
RING_BYTES = 600 * 2 ** 20  # > 2 x the 256 MB last-level cache
TOKEN_STEP_BATCHES = (1, 4)  # sequences per whole-model decode step
SETTLE_S = 0.2  # untimed run of the prefill step before its warmup steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-reps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--stack-only", action="store_true", help="run only the 30-layer stack leg (no JSON line)")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy (outside the timed region) whose known size scales "
                         "the HBM byte counters of a profiler run")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the data-parallel path shards tokens "
                                   "with no exchange, so per-GPU throughput is the single-GPU figure",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from ternary_weight_bitlinear_w1_amd import bitlinear as bl
    from ternary_weight_bitlinear_w1_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bl.lib()  # fails loudly if the HIP library is missing
    if args.stack_only:
        log(json.dumps(bench_stack(torch, bl, synth, dev, args.stack_steps, max(2, args.warmup // 2),
                                   head_table(torch, synth, dev))))
        return

    def seed(layer, tensor):
        return synth.stream_seed(BASE_SEED, 4, layer, tensor)

    # ---------------------------------------------------------------- weights (offline)
    log("generating weights")
    w_gate = synth.weights(seed(0, 1), I, H)
    w_up = synth.weights(seed(0, 2), I, H)
    w_down = synth.weights(seed(0, 3), H, I)
    packed_gu = torch.empty((2 * I, H // 4), dtype=torch.uint8, device=dev)
    g_gate = bl.quantize_weights(torch.from_numpy(w_gate).to(dev))
    g_up = bl.quantize_weights(torch.from_numpy(w_up).to(dev))
    packed_gu[:I].copy_(g_gate[0])
    packed_gu[I:].copy_(g_up[0])
    packed_d, g_d = bl.quantize_weights(torch.from_numpy(w_down).to(dev))
    gam_gu = [float(np.float32(g_gate[1].item())), float(np.float32(g_up[1].item()))]
    gam_d = [float(np.float32(g_d.item()))]
    x = torch.from_numpy(synth.activations(seed(0, 5), M, H)).to(dev)

    # buffers of the step
    codes1 = torch.empty((M, H), dtype=torch.int8, device=dev)
    codes2 = torch.empty((M, I), dtype=torch.int8, device=dev)
    deq1 = torch.empty(M, dtype=torch.float32, device=dev)
    deq2 = torch.empty(M, dtype=torch.float32, device=dev)
    rs1 = torch.empty(M, dtype=torch.int32, device=dev)
    rs2 = torch.empty(M, dtype=torch.int32, device=dev)
    mi = torch.empty((M, I), dtype=torch.float32, device=dev)
    y = torch.empty((M, H), dtype=torch.float32, device=dev)
    L = bl.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    c_float = bl.ctypes.c_float
    g_gu_c = (c_float * 2)(*gam_gu)
    se_gu = (bl.ctypes.c_int64 * 2)(I, 2 * I)
    g_d_c = (c_float * 1)(*gam_d)
    se_d = (bl.ctypes.c_int64 * 1)(H)
    ws_n = max(L.bitlinear_forward_workspace_bytes(M, H, I, 0),
               L.bitlinear_forward_relu2_glu_workspace_bytes(M, I, H, 0, bl.PATH_PREFILL))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)

    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {bl.status_name(st)} {L.bitlinear_last_error().decode()}")

    def q1():
        ok(L.bitlinear_quantize_acts(x.data_ptr(), M, H, bl.ACT_ABSMAX, None, c_float(1e-5), codes1.data_ptr(),
                                     deq1.data_ptr(), rs1.data_ptr(), sp), "quantize x")

    def f_gu():
        ok(L.bitlinear_forward_relu2_glu(None, codes1.data_ptr(), deq1.data_ptr(), rs1.data_ptr(), M, H,
                                         packed_gu.data_ptr(), I, g_gu_c, mi.data_ptr(), bl.PATH_PREFILL,
                                         ws.data_ptr(), ws_n, sp),
           "gate|up + relu2")

    def q2():
        ok(L.bitlinear_quantize_acts(mi.data_ptr(), M, I, bl.ACT_RMSNORM, None, c_float(1e-5),
                                     codes2.data_ptr(), deq2.data_ptr(), rs2.data_ptr(), sp), "sub-norm")

    def f_d():
        ok(L.bitlinear_forward(None, codes2.data_ptr(), deq2.data_ptr(), rs2.data_ptr(), M, I, packed_d.data_ptr(),
                               H, g_d_c, se_d, 1, y.data_ptr(), None, bl.PATH_PREFILL, ws.data_ptr(), ws_n, sp),
           "down")

    ops = [("quant_x", q1), ("gemm_gate_up_relu2", f_gu), ("quant_subnorm", q2), ("gemm_down", f_d)]

    if args.calibrate_copy:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 1.0, out=dst)  # one elementwise kernel: reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
        log("calibration kernel: 268435456 bytes read, 268435456 bytes written")

    # ---------------------------------------------------------------- prefill step
    def step():
        for _, f in ops:
            f()

    # the GPU leaves its idle clocks: the step runs untimed for at least
    # SETTLE_S seconds before the warmup steps (weight packing alone is too
    # short a load for that)
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n_settle += 20
    log(f"prefill: {n_settle} untimed settling steps, then warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly K steps between two events, nothing else
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_a.record(stream)
    for _ in range(args.steps):
        step()
    t_b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = t_a.elapsed_time(t_b) / args.steps
    # each operation's share, from a second pass with an event between operations
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        for j, (_, f) in enumerate(ops):
            f()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    per_op = {name: float(np.mean([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(args.steps)]))
              for j, (name, _) in enumerate(ops)}
    ops_gu = 2.0 * M * (2 * I) * H
    ops_d = 2.0 * M * H * I
    tops = (ops_gu + ops_d) / (step_ms * 1e-3) / 1e12
    # each contraction alone, launched back to back between two events on the
    # stream it runs on: its mean duration per launch
    def back_to_back(f, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f()
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    gu_ms = back_to_back(f_gu, args.steps)
    d_ms = back_to_back(f_d, args.steps)
    # the plain gate|up GEMM of the prefill workload (two weight scales, fp32
    # [4096][13824] output: the ungated form, twice the output bytes)
    y_gu = torch.empty((M, 2 * I), dtype=torch.float32, device=dev)

    def f_gu_plain():
        ok(L.bitlinear_forward(None, codes1.data_ptr(), deq1.data_ptr(), rs1.data_ptr(), M, H, packed_gu.data_ptr(),
                               2 * I, g_gu_c, se_gu, 2, y_gu.data_ptr(), None, bl.PATH_PREFILL, ws.data_ptr(), ws_n,
                               sp), "gate|up plain")

    f_gu_plain()
    gu_plain_ms = back_to_back(f_gu_plain, args.steps)
    del y_gu
    gu_plain_tops = ops_gu / (gu_plain_ms * 1e-3) / 1e12
    log(f"plain gate|up (fp32 [4096][13824] out) alone {gu_plain_ms * 1e3:.1f} us ({gu_plain_tops:.0f} TOPS)")
    gu_tops = ops_gu / (gu_ms * 1e-3) / 1e12
    d_tops = ops_d / (d_ms * 1e-3) / 1e12
    log(f"gated gate|up alone {gu_ms * 1e3:.1f} us ({gu_tops:.0f} TOPS), down alone {d_ms * 1e3:.1f} us "
        f"({d_tops:.0f} TOPS)")
    log(f"step {step_ms:.3f} ms ({tops:.0f} TOPS); per op ms {per_op}; wall/step {wall / args.steps * 1e3:.3f} ms")

    # quantization kernels against HBM: bytes read + written per launch
    q1_bytes = M * H * 4 + M * H + M * 12
    q2_bytes = M * I * 4 + M * I + M * 12
    kernels = {
        "gemm_gate_up_relu2": {"ms": gu_ms, "ms_in_step": per_op["gemm_gate_up_relu2"], "tops": gu_tops,
                               "frac_mfma": gu_tops / PEAK_INT8_TOPS},
        "gemm_down": {"ms": d_ms, "ms_in_step": per_op["gemm_down"], "tops": d_tops,
                      "frac_mfma": d_tops / PEAK_INT8_TOPS},
        "gemm_gate_up_plain": {"ms": gu_plain_ms, "tops": gu_plain_tops, "frac_mfma": gu_plain_tops / PEAK_INT8_TOPS,
                               "what": "gate|up 2560 -> 2 x 6912, fp32 [4096][13824] output, no gating"},
        "quant_x": {"ms": per_op["quant_x"], "gbs": q1_bytes / (per_op["quant_x"] * 1e-3) / 1e9},
        "quant_subnorm": {"ms": per_op["quant_subnorm"], "gbs": q2_bytes / (per_op["quant_subnorm"] * 1e-3) / 1e9},
    }
    for kq in ("quant_x", "quant_subnorm"):
        kernels[kq]["frac_hbm"] = kernels[kq]["gbs"] / PEAK_HBM_GBS

    # ---------------------------------------------------------------- measured peaks, small workloads
    peaks = bench_peaks(torch, bl, dev)
    small = bench_small_configs(torch, bl, synth, dev, max(20, args.steps))

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        decode = bench_decode(torch, bl, synth, dev, args.decode_reps, packed_gu, gam_gu, packed_d, gam_d)

    # ---------------------------------------------------------------- online mode
    online = None
    if not args.no_decode:
        online = bench_online(torch, bl, synth, dev, args.decode_reps // 4, w_gate, w_up)

    # ---------------------------------------------------------------- head
    head = None
    table = None
    if not args.no_decode or not args.no_stack:
        table = head_table(torch, synth, dev)
    if not args.no_decode:
        head = bench_head(torch, bl, synth, dev, args.decode_reps // 4, table)

    # ---------------------------------------------------------------- 30-layer stack, token step
    stack = None
    if not args.no_stack:
        stack = bench_stack(torch, bl, synth, dev, args.stack_steps, max(2, args.warmup // 2), table)
    del table

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w_gate, w_up, w_down, x.cpu().numpy(), args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "prefill of one BitNet b1.58 2B4T MLP: M=4096 tokens, quantize -> gate|up "
                               "2560->2x6912 with ReLU^2 gating -> ffn_sub_norm quantize -> down 6912->2560",
                   "tokens": M, "hidden": H, "intermediate": I, "ops_per_step": ops_gu + ops_d},
        "roofline": {"bound": "mfma", "kernel": "gemm_prefill gated (gate|up + ReLU^2, M=4096 N=2x6912 K=2560)",
                     "achieved": round(gu_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tops / PEAK_INT8_TOPS, 4), "traffic": measured_traffic(),
                     "peak_measured": peaks["mfma_int8_tops"],
                     "frac_of_measured": round(gu_tops / peaks["mfma_int8_tops"], 4),
                     "peak_measured_varied": peaks["mfma_int8_tops_varied"],
                     "frac_of_measured_varied": round(gu_tops / peaks["mfma_int8_tops_varied"], 4),
                     "algorithmic_ops_per_launch": ops_gu,
                     "algorithmic_bytes_per_launch": M * H + 2 * I * H // 4 + 4 * M * I + 8 * M},
        "kernels": kernels,
        "peaks_measured": peaks,
        "small_configs": small,
        "decode_roofline": decode_roofline(decode),
        "decode": decode,
        "online": online,
        "head": head,
        "stack": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_peaks(torch, bl, dev):
    """What this GPU reaches on its two bounds, measured here with the library's
    probes: a read stream over 2 GiB (larger than the last-level cache) and
    independent int8 MFMA chains on every SIMD (two waves per SIMD)."""
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.ones(2 ** 29, dtype=torch.float32, device=dev)  # 2 GiB
    nb = buf.numel() * 4

    def timed(f, reps):
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    t_read = timed(lambda: bl.probe_read(buf, sink=sink), 10)
    del buf
    torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters, wgs = 4000, 2 * cus
    t_mfma = timed(lambda: bl.probe_mfma(iters, wgs, sink), 5)
    t_varied = timed(lambda: bl.probe_mfma(iters, wgs, sink, varied=True), 5)
    mfma_ops = wgs * 4 * iters * 8 * 65536.0
    res = {"hbm_read_gbs": round(nb / t_read / 1e9, 1), "mfma_int8_tops": round(mfma_ops / t_mfma / 1e12, 1),
           "mfma_int8_tops_varied": round(mfma_ops / t_varied / 1e12, 1),
           "compute_units": cus,
           "what": "read probe over 2 GiB; int8 MFMA probe: 2 workgroups x 4 waves per CU, 8 independent "
                   "v_mfma_i32_32x32x32_i8 chains per wave, on fixed operands and (varied) on operands that "
                   "change from one MFMA to the next (A in {0,1,2}, B any int8: the GEMMs' value ranges)"}
    log(f"measured peaks: HBM read {res['hbm_read_gbs']:.0f} GB/s (spec {PEAK_HBM_GBS:.0f}), int8 MFMA "
        f"{res['mfma_int8_tops']:.0f} TOPS on fixed operands, {res['mfma_int8_tops_varied']:.0f} TOPS on varied "
        f"operands (spec {PEAK_INT8_TOPS:.0f})")
    return res


def bench_small_configs(torch, bl, synth, dev, reps):
    """The two small workloads, each a chain of a few launches: the single layer
    (M=128, K=256 -> N=512, quantization inside bitlinear_forward) and the FFN
    block (M=1024, hidden 512, intermediate 2048, bitlinear_block_forward).
    ``us``: mean GPU time per call, 20 calls captured back to back in one HIP
    graph and replayed; ``eager_us``: mean time per call of back-to-back calls
    from Python, which the host's cost per call can pace. Int8 TOPS from ``us``."""
    stream = torch.cuda.current_stream(dev)
    res = {}
    # single layer
    m, k, n = 128, 256, 512
    w = torch.from_numpy(synth.weights(synth.stream_seed(BASE_SEED, 1, 0, 1), n, k)).to(dev)
    packed, g = bl.quantize_weights(w)
    gam = [float(np.float32(g.item()))]
    x = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 1, 0, 5), m, k, 4)).to(dev)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)

    def timed(f):
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    def graphed(f):
        return graph_per_launch_us(torch, lambda i, sp: f(), 20)

    f1 = lambda: bl.forward(packed, k, gam, x=x, out=y)  # noqa: E731
    eager = timed(f1)
    us = graphed(f1)
    res["single_layer"] = {"us": round(us, 2), "eager_us": round(eager, 2),
                           "tops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 3),
                           "launches": 2, "workload": "M=128, K=256 -> N=512, fp32 in and out"}
    # FFN block
    m, hd, it = 1024, 512, 2048
    mats = [synth.weights(synth.stream_seed(BASE_SEED, 2, 0, t), n_, k_) for t, (n_, k_) in
            enumerate(((it, hd), (it, hd), (hd, it)))]
    pk, gm = [], []
    for wm in mats:
        p_, g_ = bl.quantize_weights(torch.from_numpy(wm).to(dev))
        pk.append(p_)
        gm.append(float(np.float32(g_.item())))
    lw = bl.LayerWeights(gate_up=torch.cat(pk[:2]), gate_up_gamma=gm[:2], down=pk[2], down_gamma=gm[2])
    spec = bl.BlockSpec(bl.BLOCK_FFN, hd, it, [lw])
    xb = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 2, 0, 5), m, hd)).to(dev)
    yb = torch.empty_like(xb)
    ws = torch.empty(max(1, bl.block_workspace_bytes(spec, m)), dtype=torch.uint8, device=dev)
    f2 = lambda: bl.block_forward(spec, xb, out=yb, workspace=ws)  # noqa: E731
    eager = timed(f2)
    us = graphed(f2)
    res["ffn_block"] = {"us": round(us, 2), "eager_us": round(eager, 2),
                        "tops": round(2.0 * m * 3 * it * hd / (us * 1e-6) / 1e12, 2),
                        "workload": "M=1024, hidden 512, intermediate 2048: quantize, gate|up + ReLU^2, "
                                    "ffn_sub_norm quantize, down"}
    log(f"single layer {res['single_layer']['us']:.1f} us; FFN block {res['ffn_block']['us']:.1f} us "
        f"({res['ffn_block']['tops']:.0f} TOPS)")
    return res


def decode_roofline(decode):
    """The decode GEMV at the decode-sweep shapes (gate|up 2560 -> 2 x 6912 and
    down 6912 -> 2560, M = 1, 4, 16), one projection per launch, in packed-weight
    GB/s against 8 TB/s, with the read probe's time over the same bytes (the
    per-launch floor) beside each. The launch over the whole 628 MB ring is a
    probe of the kernel's streaming rate without that floor, not a workload."""
    if not decode or "gate_up_m1" not in decode:
        return None
    shapes = {}
    for name in ("gate_up", "down"):
        floor = decode.get(f"{name}_read_floor")
        for m in (1, 4, 16):
            r = decode.get(f"{name}_m{m}")
            if r:
                shapes[f"{name}_m{m}"] = {"achieved": r["gbs_packed"], "frac": r["frac_hbm"], "us": r["us"],
                                          "read_floor_us": floor["us"] if floor else None,
                                          "us_vs_read_floor": r.get("us_vs_read_floor")}
    one = decode["gate_up_m1"]
    ring = decode.get("gate_up_m1_probe_whole_ring")
    return {"bound": "hbm", "kernel": "decode GEMV (gemv_dot4 at m=1, gemv_decode at m=4 and 16), packed 2-bit",
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "achieved": one["gbs_packed"], "frac": one["frac_hbm"], "shape": "gate|up m=1",
            "config_shapes": shapes,
            "probe_whole_ring": ({"achieved": ring["gbs_packed"], "frac": ring["frac_hbm"], "us": ring["us"],
                                  "bytes": ring["packed_bytes"],
                                  "what": "one launch over every ring copy stacked (not a workload shape)"}
                                 if ring else None)}


def measured_traffic():
    """HBM-side bytes per gate|up GEMM launch from the committed counter profile
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a known-size kernel); None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "counters_gemm_prefill_m4096.md")
    src = os.path.join(ROOT, "ternary_weight_bitlinear_w1_amd", "csrc", "gemm_prefill.hip")
    try:
        fields = dict(line.strip().split(": ", 1) for line in open(prof) if ": " in line and line.startswith("    "))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if fields.get("gemm_source_sha256_16") == digest:
            return int(fields["traffic_bytes_gate_up"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def graph_per_launch_us(torch, launch, reps, replays=4):
    """Mean GPU time per launch of reps launches captured back to back in one HIP
    graph (launch(i, stream) enqueues launch i on the given stream), so the host's
    cost per call does not pace the GPU."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for i in range(reps):
            launch(i, sp)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (replays * reps) * 1e3


def bench_decode(torch, bl, synth, dev, reps, packed_gu, gam_gu, packed_d, gam_d):
    """Weight-streaming kernel at M = 1, 4, 16; each launch reads another copy of the
    packed weights from a ring larger than the last-level cache. Back-to-back
    launches are captured in a HIP graph and replayed."""
    res = {}
    L = bl.lib()
    stream = torch.cuda.current_stream(dev)
    sp0 = stream.cuda_stream
    for name, packed, k, gam, seg in (("gate_up", packed_gu, H, gam_gu, [I, 2 * I]),
                                      ("down", packed_d, I, gam_d, [H])):
        n = packed.shape[0]
        nbytes = packed.numel()
        copies = max(2, RING_BYTES // nbytes)
        ring = packed.unsqueeze(0).repeat(copies, 1, 1)
        ptrs = [ring[i].data_ptr() for i in range(copies)]
        g_c = (bl.ctypes.c_float * len(gam))(*gam)
        se_c = (bl.ctypes.c_int64 * len(seg))(*seg)
        for m in (1, 4, 16):
            xm = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 3, m, 5), m, k,
                                                    synth.outlier_count(k))).to(dev)
            codes, deq, rs = bl.quantize_acts(xm)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            ws_n = L.bitlinear_forward_workspace_bytes(m, n, k, 0)
            ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
            cp, dp, rp, yp, wp = codes.data_ptr(), deq.data_ptr(), rs.data_ptr(), y.data_ptr(), ws.data_ptr()

            def launch(i, sp):
                st = L.bitlinear_forward(None, cp, dp, rp, m, k, ptrs[i % copies], n, g_c, se_c, len(gam), yp, None,
                                         bl.PATH_DECODE, wp, ws_n, sp)
                if st != 0:
                    raise RuntimeError(L.bitlinear_last_error().decode())

            for i in range(20):
                launch(i, sp0)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i in range(reps):
                evs[i][0].record(stream)
                launch(i, sp0)
                evs[i][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
            b2b_us = graph_per_launch_us(torch, launch, reps)
            gbs = nbytes / (b2b_us * 1e-6) / 1e9
            res[f"{name}_m{m}"] = {"us": round(b2b_us, 3), "gbs_packed": round(gbs, 1),
                                   "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "single_launch_event_us": round(us, 3),
                                   "packed_bytes": nbytes, "ring_copies": copies}
            log(f"decode {name} m={m}: {b2b_us:.2f} us/launch back-to-back (graph), {gbs:.0f} GB/s "
                f"(one launch between events: {us:.2f} us)")
            if m in (1, 4, 16):
                res[f"{name}_m{m}_probe_whole_ring"] = bench_decode_tall(torch, L, bl, ring, k, gam[0], seg[0], codes,
                                                                         deq, rs, y, reps, name, m, sp0, stream)
        # reference: a device copy of the same bytes (one ring copy per launch,
        # back to back; it reads them once and writes them once) -- the cost of
        # one launch that moves these bytes on this GPU
        dst = torch.empty_like(ring[0])
        views = [ring[i] for i in range(copies)]
        floor_us = graph_per_launch_us(torch, lambda i, sp: dst.copy_(views[i % copies]), reps)
        res[f"{name}_copy_reference"] = {"us": round(floor_us, 3),
                                         "gbs_read": round(nbytes / (floor_us * 1e-6) / 1e9, 1),
                                         "what": "device copy of the same packed bytes, one ring copy per launch"}
        log(f"decode {name}: a device copy of the same {nbytes} bytes takes {floor_us:.2f} us/launch "
            f"({nbytes / (floor_us * 1e-6) / 1e9:.0f} GB/s read)")
        # the read floor: the library's read probe over the same bytes (one ring
        # copy per launch, back to back), the least time one launch that reads
        # them takes on this GPU (the best of four launch shapes: 8, 4, 2 or 1
        # loads of 16 bytes per thread)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        shapes = {}
        for per_thread in (8, 4, 2, 1):
            grid = -(-nbytes // (16 * 256 * per_thread))

            def probe(i, sp, grid=grid):
                st = L.bitlinear_probe_read(ptrs[i % copies], nbytes, grid, sink.data_ptr(), sp)
                if st != 0:
                    raise RuntimeError(L.bitlinear_last_error().decode())

            shapes[per_thread] = graph_per_launch_us(torch, probe, reps)
        best = min(shapes, key=shapes.get)
        read_us = shapes[best]
        res[f"{name}_read_floor"] = {"us": round(read_us, 3),
                                     "gbs_read": round(nbytes / (read_us * 1e-6) / 1e9, 1),
                                     "loads_per_thread": best,
                                     "us_by_loads_per_thread": {str(k_): round(v, 3) for k_, v in shapes.items()},
                                     "what": "read probe over the same packed bytes, one ring copy per launch, "
                                             "the fastest of four launch shapes"}
        for m in (1, 4, 16):
            res[f"{name}_m{m}"]["us_vs_read_floor"] = round(res[f"{name}_m{m}"]["us"] / read_us, 3)
        log(f"decode {name}: the read probe over the same {nbytes} bytes takes {read_us:.2f} us/launch "
            f"({nbytes / (read_us * 1e-6) / 1e9:.0f} GB/s)")
        del ring, dst, views
        torch.cuda.empty_cache()
        # the same projection from the base-3 storage (five codes per byte), m = 1 and 4
        w3 = bl.pack_base3(packed, k)
        nb3 = w3.numel()
        copies = max(2, RING_BYTES // nb3)
        ring = w3.unsqueeze(0).repeat(copies, 1, 1)
        ptrs3 = [ring[i].data_ptr() for i in range(copies)]
        for m in (1, 4):
            xm = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 3, m, 5), m, k,
                                                    synth.outlier_count(k))).to(dev)
            codes, deq, _ = bl.quantize_acts(xm)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            cp, dp, yp = codes.data_ptr(), deq.data_ptr(), y.data_ptr()

            def launch3(i, sp):
                st = L.bitlinear_forward_base3(None, cp, dp, m, k, ptrs3[i % copies], n, g_c, se_c, len(gam), yp,
                                               None, None, 0, sp)
                if st != 0:
                    raise RuntimeError(L.bitlinear_last_error().decode())

            for i in range(20):
                launch3(i, sp0)
            torch.cuda.synchronize()
            b2b_us = graph_per_launch_us(torch, launch3, reps)
            gbs = nb3 / (b2b_us * 1e-6) / 1e9
            res[f"{name}_base3_m{m}"] = {"us": round(b2b_us, 3), "gbs_stored": round(gbs, 1),
                                         "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "stored_bytes": nb3,
                                         "us_vs_two_bit": round(b2b_us / res[f"{name}_m{m}"]["us"], 3)}
            log(f"decode {name} base-3 m={m}: {b2b_us:.2f} us/launch back-to-back, {gbs:.0f} GB/s of "
                f"{nb3} stored bytes ({b2b_us / res[f'{name}_m{m}']['us']:.3f} x the two-bit time)")
        del ring, w3
        torch.cuda.empty_cache()
    return res


def bench_decode_tall(torch, L, bl, ring, k, gamma, seg0, codes, deq, rs, y_ref, reps, name, m, sp, stream):
    """The same decode kernel in one launch over every copy of the ring at once
    (copies x n rows, one gamma): a launch that streams more than twice the
    last-level cache, so its fixed cost no longer sets the time. The first
    seg0 outputs must equal those of the ordinary launch bit for bit."""
    copies, n = ring.shape[0], ring.shape[1]
    tall = ring.view(copies * n, ring.shape[2])
    nt = tall.shape[0]
    g_c = (bl.ctypes.c_float * 1)(gamma)
    se_c = (bl.ctypes.c_int64 * 1)(nt)
    y = torch.empty((m, nt), dtype=torch.float32, device=y_ref.device)
    ws_n = L.bitlinear_forward_workspace_bytes(m, nt, k, 0)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=y_ref.device)

    def launch():
        st = L.bitlinear_forward(None, codes.data_ptr(), deq.data_ptr(), rs.data_ptr(), m, k, tall.data_ptr(), nt,
                                 g_c, se_c, 1, y.data_ptr(), None, bl.PATH_DECODE, ws.data_ptr(), ws_n, sp)
        if st != 0:
            raise RuntimeError(L.bitlinear_last_error().decode())

    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    if not torch.equal(y[:, :seg0], y_ref[:, :seg0]):
        raise RuntimeError(f"decode {name} m={m}: the whole-ring launch differs from the ordinary one")
    n_rep = max(5, reps // 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_rep):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n_rep * 1e3
    nbytes = tall.numel()
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"decode {name} m={m}, one launch over the whole ring ({nt} rows, {nbytes / 1e6:.0f} MB): {us:.1f} us, "
        f"{gbs:.0f} GB/s packed ({gbs / PEAK_HBM_GBS:.2f} of HBM)")
    del y, ws
    return {"us": round(us, 2), "rows": nt, "packed_bytes": nbytes, "gbs_packed": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def head_table(torch, synth, dev):
    """The tied embedding / head table, 128256 x 2560 bfloat16 (as uint16 bits),
    N(0, 0.02) rounded to bfloat16."""
    log("head: generating the 128256 x 2560 table")
    table = torch.empty((VOCAB, H), dtype=torch.uint16, device=dev)
    rows = 16032
    for r0 in range(0, VOCAB, rows):
        n = min(rows, VOCAB - r0)
        w = torch.from_numpy(synth.weights(synth.stream_seed(BASE_SEED, 6, r0, 1), n, H)).to(dev)
        table[r0:r0 + n] = w.to(torch.bfloat16).view(torch.uint16)
        del w
    return table


def bench_head(torch, bl, synth, dev, reps, table):
    """The model's head at decode: final norm + the bfloat16 lm_head (128256 x 2560,
    656.7 MB, larger than the last-level cache, so every launch streams it from
    HBM), for 1 and 4 tokens: mean time per call over back-to-back calls."""
    V, K = VOCAB, H
    L = bl.lib()
    sp = torch.cuda.current_stream(dev).cuda_stream
    stream = torch.cuda.current_stream(dev)
    gain = torch.full((K,), 0.1, dtype=torch.float32, device=dev)
    nbytes = V * K * 2
    res = {}
    for m in (1, 4):
        x = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 6, m, 5), m, K)).to(dev)
        y = torch.empty((m, V), dtype=torch.float32, device=dev)
        wsn = L.bitlinear_lm_head_workspace_bytes(m, K)
        ws = torch.empty(max(wsn, 1), dtype=torch.uint8, device=dev)

        def call():
            st = L.bitlinear_lm_head(x.data_ptr(), m, K, gain.data_ptr(), 1e-5, table.data_ptr(), V, y.data_ptr(),
                                     None, ws.data_ptr(), wsn, sp)
            if st != 0:
                raise RuntimeError(L.bitlinear_last_error().decode())

        for _ in range(5):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"m{m}"] = {"us": round(us, 2), "gbs_head": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                        "head_bytes": nbytes}
        log(f"head m={m}: {us:.1f} us per call (final norm + lm_head), {gbs:.0f} GB/s of the 656.7 MB table")
    return res


def bench_online(torch, bl, synth, dev, reps, w_gate, w_up):
    """The online checkpoint mode at one decode token: the gate and up masters
    (2 x 6912 x 2560) are ternarized inside every forward (a mean|W| pass and a
    ternarize pass per matrix, each reading the masters), then projected. Both
    master storages: fp32, and bfloat16 (the bf16 checkpoint: the fp32 masters
    rounded to bfloat16, half the bytes)."""
    w32 = torch.from_numpy(np.concatenate([w_gate, w_up])).to(dev)
    n, k = w32.shape
    x = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 3, 1, 5), 1, k, synth.outlier_count(k))).to(dev)
    seg = (bl.ctypes.c_int64 * 2)(n // 2, n)
    L = bl.lib()
    nb = int(L.bitlinear_forward_online_workspace_bytes(1, n, k, 1, seg, 2))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {"workload": "online mode, gate|up 2560 -> 2 x 6912 masters, one token"}
    for name, w, dt, esize in (("f32", w32, bl.MASTER_F32, 4),
                               ("bf16", w32.to(torch.bfloat16).view(torch.uint16), bl.MASTER_BF16, 2)):
        def run():
            st = L.bitlinear_forward_online(x.data_ptr(), None, None, None, 1, k, w.data_ptr(), dt, n, seg, 2, None,
                                            y.data_ptr(), None, bl.PATH_AUTO, ws.data_ptr(), nb, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"online forward: {bl.status_name(st)} {L.bitlinear_last_error().decode()}")

        for _ in range(3):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        master = esize * n * k
        read = 2 * master  # the mean|W| pass and the ternarize pass each read the masters
        gbs = read / (us * 1e-6) / 1e9
        log(f"online gate|up m=1, {name} masters: {us:.1f} us per forward, {master / 1e6:.1f} MB read twice: "
            f"{gbs:.0f} GB/s")
        res[name] = {"us": round(us, 2), "master_bytes": master, "master_bytes_read": read,
                     "gbs_masters_read": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        del w
    del w32, ws
    return res


STACK_LAYERS, STACK_HEADS, STACK_KV_HEADS, STACK_HEAD_DIM = 30, 20, 5, 128


def bench_stack(torch, bl, synth, dev, steps, warmup, table):
    """One step of the 30-layer decoder projection stack of the 2B4T shapes
    (q|k|v, self-only attention, o, gate|up, ReLU^2, down, residuals; gains 1)
    through bitlinear_block_forward at M = 1 and M = 64. Reports the step time
    and the packed-weight bytes of the step per second."""
    kvd = STACK_KV_HEADS * STACK_HEAD_DIM
    shapes = [(H, H), (kvd, H), (kvd, H), (H, H), (I, H), (I, H), (H, I)]
    log(f"stack: packing {STACK_LAYERS} layers")
    layers, packed_bytes, weights = [], 0, 0
    for l in range(STACK_LAYERS):
        p, g = [], []
        for t, (n, k) in enumerate(shapes):
            w = torch.from_numpy(synth.weights(synth.stream_seed(BASE_SEED, 5, l, 10 + t), n, k)).to(dev)
            pk, gm = bl.quantize_weights(w)
            p.append(pk)
            g.append(float(np.float32(gm.item())))
            packed_bytes += pk.numel()
            weights += n * k
            del w
        layers.append(bl.LayerWeights(qkv=torch.cat(p[0:3]), qkv_gamma=g[0:3], o=p[3], o_gamma=g[3],
                                      gate_up=torch.cat(p[4:6]), gate_up_gamma=g[4:6], down=p[6], down_gamma=g[6]))
        del p
    spec = bl.BlockSpec(bl.BLOCK_DECODER, H, I, layers, STACK_HEADS, STACK_KV_HEADS, STACK_HEAD_DIM, 1e-5)
    blk, keep = spec.to_c()
    L = bl.lib()
    stream = torch.cuda.current_stream(dev)
    res = {"layers": STACK_LAYERS, "weights": weights, "packed_bytes": packed_bytes}
    for m in (1, 64):
        x = torch.from_numpy(synth.activations(synth.stream_seed(BASE_SEED, 5, m, 5), m, H)).to(dev)
        y = torch.empty_like(x)
        nb = int(L.bitlinear_block_workspace_bytes(bl.ctypes.byref(blk), m))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

        def step():
            st = L.bitlinear_block_forward(bl.ctypes.byref(blk), x.data_ptr(), m, y.data_ptr(), None, ws.data_ptr(),
                                           nb, torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError(f"block forward: {bl.status_name(st)} {L.bitlinear_last_error().decode()}")

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        eager = y.clone()

        def timed(run):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            t0 = time.perf_counter()
            for a, b in ev:
                a.record(stream)
                run()
                b.record(stream)
            torch.cuda.synchronize()
            host_ms = (time.perf_counter() - t0) * 1e3 / steps
            return sorted(a.elapsed_time(b) for a, b in ev), host_ms

        t_eager, host_eager = timed(step)
        # the same step captured once into a HIP graph and replayed: one host
        # call per step instead of one per kernel
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, eager):
            raise RuntimeError(f"stack m={m}: graph replay differs from the eager step")
        t_graph, host_graph = timed(graph.replay)
        if not torch.equal(y, eager):
            raise RuntimeError(f"stack m={m}: graph replay differs from the eager step")
        t = t_graph
        ms = float(np.median(t))
        gbs = packed_bytes / (ms * 1e-3) / 1e9
        ops = 2.0 * m * weights
        res[f"m{m}"] = {"ms_per_step": round(ms, 4), "p10_ms": round(t[len(t) // 10], 4),
                        "p90_ms": round(t[(9 * len(t)) // 10], 4), "gbs_packed": round(gbs, 1),
                        "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "tops": round(ops / (ms * 1e-3) / 1e12, 2),
                        "eager_ms_per_step": round(float(np.median(t_eager)), 4),
                        "eager_host_ms_per_step": round(host_eager, 4)}
        log(f"stack m={m}: graph {ms:.3f} ms/step, {gbs:.0f} GB/s packed, {ops / (ms * 1e-3) / 1e12:.1f} TOPS; "
            f"eager {np.median(t_eager):.3f} ms/step (host {host_eager:.3f} ms/step)")
        del graph, x, y, ws
    res["token_step"] = bench_token_step(torch, bl, dev, layers, table, steps, warmup)
    del keep, layers
    return res


def bench_token_step(torch, bl, dev, layers, table, steps, warmup):
    """One decode step of the whole model for B sequences (B = 1 and 4) at position
    4095 of a 4096-position context: embedding gather, 30 decoder layers with RoPE,
    bfloat16 KV cache append and causal attention over 4096 positions, final norm
    and the bfloat16 head. Caches hold seeded N(0, 1) values; the step is captured
    into a HIP graph and replayed. Reports ms per step, tokens/s, and the bytes a
    step must read (packed weights, head, the sequences' caches) per second."""
    T = 4096
    kvd = STACK_KV_HEADS * STACK_HEAD_DIM
    L = bl.lib()
    stream = torch.cuda.current_stream(dev)
    res = {}
    packed = sum(l.qkv.numel() + l.o.numel() + l.gate_up.numel() + l.down.numel() for l in layers)
    rope_tab = bl.rope_table(ROPE_THETA, STACK_HEAD_DIM, ROPE_POSITIONS, dev)
    for B in TOKEN_STEP_BATCHES:
        gen = torch.Generator(device=dev)
        gen.manual_seed(BASE_SEED + B)
        caches = []
        for _ in layers:
            kc = torch.randn((B, STACK_KV_HEADS, T, STACK_HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
            vc = torch.randn((B, STACK_KV_HEADS, T, STACK_HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
            caches.append((kc.view(torch.uint16), vc.view(torch.uint16)))
        cl = [bl.LayerWeights(qkv=l.qkv, qkv_gamma=l.qkv_gamma, o=l.o, o_gamma=l.o_gamma, gate_up=l.gate_up,
                              gate_up_gamma=l.gate_up_gamma, down=l.down, down_gamma=l.down_gamma, k_cache=kc,
                              v_cache=vc) for l, (kc, vc) in zip(layers, caches)]
        slot = torch.arange(B, dtype=torch.int64, device=dev)
        pos = torch.full((B,), T - 1, dtype=torch.int64, device=dev)
        spec = bl.BlockSpec(bl.BLOCK_DECODER_CACHED, H, I, cl, STACK_HEADS, STACK_KV_HEADS, STACK_HEAD_DIM, 1e-5,
                            slot=slot, pos=pos, rope_table=rope_tab)
        blk, keep = spec.to_c()
        ids = torch.arange(B, dtype=torch.int64, device=dev) * 7919 + 11
        x = torch.empty((B, H), dtype=torch.float32, device=dev)
        h = torch.empty_like(x)
        logits = torch.empty((B, VOCAB), dtype=torch.float32, device=dev)
        gain = torch.full((H,), 0.1, dtype=torch.float32, device=dev)
        nb = int(L.bitlinear_block_workspace_bytes(bl.ctypes.byref(blk), B))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        nh = int(L.bitlinear_lm_head_workspace_bytes(B, H))
        wsh = torch.empty(max(nh, 1), dtype=torch.uint8, device=dev)

        def step():
            sp = torch.cuda.current_stream(dev).cuda_stream
            for name, st in (("embed", L.bitlinear_embed(ids.data_ptr(), B, table.data_ptr(), VOCAB, H, x.data_ptr(),
                                                          sp)),
                             ("block", L.bitlinear_block_forward(bl.ctypes.byref(blk), x.data_ptr(), B, h.data_ptr(),
                                                                 None, ws.data_ptr(), nb, sp)),
                             ("head", L.bitlinear_lm_head(h.data_ptr(), B, H, gain.data_ptr(), 1e-5, table.data_ptr(),
                                                          VOCAB, logits.data_ptr(), None, wsh.data_ptr(), nh, sp))):
                if st != 0:
                    raise RuntimeError(f"token step {name}: {bl.status_name(st)} {L.bitlinear_last_error().decode()}")

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        eager = logits.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(logits, eager):
            raise RuntimeError(f"token step B={B}: graph replay differs from the eager step")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        ms = float(np.median(t))
        kv_bytes = B * len(layers) * T * 2 * kvd * 2
        step_bytes = packed + VOCAB * H * 2 + kv_bytes
        gbs = step_bytes / (ms * 1e-3) / 1e9
        res[f"b{B}"] = {"ms_per_step": round(ms, 4), "p10_ms": round(t[len(t) // 10], 4),
                        "p90_ms": round(t[(9 * len(t)) // 10], 4), "tokens_per_s": round(B / (ms * 1e-3), 1),
                        "bytes_per_step": step_bytes, "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                        "context": T}
        log(f"token step B={B} (position {T - 1}): {ms:.3f} ms/step, {B / (ms * 1e-3):.0f} tokens/s, "
            f"{step_bytes / 1e6:.0f} MB read per step = {gbs:.0f} GB/s")
        del graph, keep, caches, cl, ws, wsh
        torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Host cores this process may use, at most 16 (one GPU's share of the box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w_gate, w_up, w_down, x, seconds):
    """The CPU oracle, as it stands (plain C, one call per step), on a bounded
    sample of the step's tokens: once on one thread, once on the host cores
    this process may use (up to 16; one thread per contiguous block of tokens,
    each running the oracle on its block: tokens are independent, the per-token
    arithmetic is the same, so is every result). TOPS scale with the sample.
    Also times the oracle, on one thread, on the single layer and on one decode
    projection of each shape."""
    import threading

    import oracle
    from ternary_weight_bitlinear_w1_amd import synth
    log("cpu baseline: oracle weights")
    gams = [oracle.absmean(w) for w in (w_gate, w_up, w_down)]
    c_gu = np.concatenate([oracle.ternarize(w_gate, gams[0]), oracle.ternarize(w_up, gams[1])])
    c_d = oracle.ternarize(w_down, gams[2])
    ops_per_token = 2.0 * (2 * I * H + H * I)

    def step(rows):
        oracle.ffn_block(rows, c_gu, gams[:2], c_d, gams[2], None, 1e-5)

    t = time.perf_counter()
    step(x[:2])
    per_tok = (time.perf_counter() - t) / 2
    # single thread: about half the CPU budget
    n1 = int(max(2, min(M, 0.5 * seconds / max(per_tok, 1e-6))))
    t = time.perf_counter()
    step(x[:n1])
    dt1 = time.perf_counter() - t
    single = {"value": round(ops_per_token * n1 / dt1 / 1e12, 6), "cores": 1, "tokens": n1, "seconds": round(dt1, 2)}
    # every usable core: about the same wall time again
    threads = cpu_threads()
    nt = int(max(threads, min(M, threads * 0.5 * seconds / max(per_tok, 1e-6))))
    bounds = np.linspace(0, nt, threads + 1).astype(int)
    errs = []

    def work(a, b):
        try:
            step(x[a:b])
        except Exception as e:  # noqa: BLE001 (reported below)
            errs.append(e)

    th = [threading.Thread(target=work, args=(int(bounds[i]), int(bounds[i + 1]))) for i in range(threads)]
    t = time.perf_counter()
    for h in th:
        h.start()
    for h in th:
        h.join()
    dtn = time.perf_counter() - t
    if errs:
        raise errs[0]
    log(f"cpu baseline: {n1} tokens on 1 thread in {dt1:.1f} s; {nt} tokens on {threads} threads in {dtn:.1f} s")

    # the other workloads, on one thread (small) or all threads (the FFN block)
    other = {}
    xs = synth.activations(synth.stream_seed(BASE_SEED, 1, 0, 5), 128, 256, 4)
    ws_ = synth.weights(synth.stream_seed(BASE_SEED, 1, 0, 1), 512, 256)
    g1 = oracle.absmean(ws_)
    c1 = oracle.ternarize(ws_, g1)
    t = time.perf_counter()
    oracle.forward(xs, c1, [g1])
    other["single_layer_ms"] = round((time.perf_counter() - t) * 1e3, 2)
    for name, c, k, seg in (("decode_gate_up_m1_ms", c_gu, H, [I, 2 * I]), ("decode_down_m1_ms", c_d, I, [H])):
        xm = synth.activations(synth.stream_seed(BASE_SEED, 3, 1, 5), 1, k, synth.outlier_count(k))
        t = time.perf_counter()
        oracle.forward(xm, c, [gams[0], gams[1]] if len(seg) == 2 else [gams[2]], seg)
        other[name] = round((time.perf_counter() - t) * 1e3, 2)
    return {"value": round(ops_per_token * nt / dtn / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"first {nt} of the {M} tokens of the prefill MLP step (same weights and inputs), "
                      f"{threads} threads on contiguous token blocks, {dtn:.1f} s",
            "seconds": round(dtn, 2), "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": single, "other_workloads": other}


if __name__ == "__main__":
    main()
