"""Benchmark: W4A16 decode projections on one MI355X.

A step is one decode token through the projections of a 42-layer,
2560-hidden transformer (the Gemma-4 E4B shapes of the decode workload):
per layer q, k, v, o (2560/512/512/2560 <- 2560), fused gate+up
(20480 <- 2560) and down (2560 <- 10240) at M = 1, every layer with its own
weights (2.2 GB in total, far beyond the 256 MB last-level cache, so each
call streams its weights from HBM).  q, k and v read the same activations and
are launched together (w4a16_matmul_grouped: separate matrices and outputs,
bitwise the same results as separate calls); o, gate+up and down are single
w4a16_matmul calls, as the data dependences of a decoder layer require.  The
step is captured once in a HIP graph and replayed.  The same step at
M = k+1 in {2, 3, 5} (speculative-verify batches) and the step with six
separate launches per layer are reported alongside.

Prints ONE JSON line.  The value is whole-step throughput in algorithmic
GB/s: packed codes + bf16 scales/biases + bf16 x + bf16 y per call.
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

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

METRIC = "achieved HBM GB/s (% of MI355X peak) for W4A16 qmv M=1 and qmm M=k+1"
PEAK_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
# MI355X fp32 vector peak (256 CUs x 4 SIMDs x 32 lanes x 2 flops x 2.4 GHz):
# a wave64 v_fmac_f32 with register operands issues in two cycles per SIMD
# (measured: 2.3), without the packed instructions the build does not use.
PEAK_FP32_FMA_TFLOPS = 157.3
# Issue cycles per wave64 instruction per SIMD by class, at the rate the SIMD
# executes it: fp32 fma and simple integer ops 2 (32 lanes per cycle), the
# mixed-precision v_fma_mix_f32 that dequantizes each weight 4 (16 lanes per
# cycle; measured 2.3 and 4.2 with two or more waves per SIMD).  A packed word
# (eight weights) costs 8 v_fma_mix_f32, 5 mask/shift ops and 8 M fmas.
CUS, SIMDS, CLOCK_GHZ = 256, 4, 2.4   # compute units, SIMDs per CU, shader clock
WORD_ISSUE_CYCLES = (8 * 4 + 5 * 2, 8 * 2)    # (per word, per word and activation row)
PREFILL_M = (16, 64, 512, 4096)
LAYERS = 42
# untimed replay time before each measurement (beyond the warm-up count): the
# first measurement runs the step for a second so the clocks have settled
FIRST_WARM_S = 1.0
WARM_S = 0.25


def call_bytes(M: int, N: int, K: int, group: int = 64) -> int:
    """Algorithmic bytes of one product: codes + scales + biases + x + y (bf16)."""
    return N * K // 2 + N * (K // group) * 4 + 2 * M * K + 2 * M * N


def step_bytes(M: int, layers: int) -> int:
    return layers * sum(call_bytes(M, *synthetic.PROJECTIONS[p]) for p in synthetic.LAYER_ORDER)


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "qmm_dense_decode_step_traffic.json")


def launch_grid(kernel: str, Ns) -> int:
    """Work-items launched by the dense kernel named `kernel` for matrices of
    Ns rows sharing one launch: a grid of (blocks of the tallest matrix) x
    (matrices) blocks; a block is 4 waves holding 16 row groups of R rows, or,
    with a K-split of S, RS row sets of S waves sharing 4 row groups of R rows.
    One matrix at two rows per lane and one row set whose blocks are not a
    whole number of rounds over the CUs ends in one-row-per-lane blocks (16
    rows, or 4 with a K-split) after the last whole round, if those fit one
    per CU."""
    M, R, CPL, KS, PRE, DEPTH, RS = (int(v) for v in kernel[kernel.index("<") + 1:kernel.index(">")].split(",")[:7])
    rows = (16 if KS == 1 else 4 * RS) * R
    threads = 64 * (4 if KS == 1 else KS * RS)
    blocks = -(-max(Ns) // rows)
    if R == 2 and RS == 1 and len(Ns) == 1 and blocks > CUS and blocks % CUS:
        big = blocks // CUS * CUS
        tail_rows = 16 if KS == 1 else 4
        small = -(-(Ns[0] - big * rows) // tail_rows)
        if small <= CUS:
            blocks = big + small
    return blocks * len(Ns) * threads


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_stack(torch, layers: int):
    """Per projection: seeded layer-0 weights uploaded, other layers' codes xor-ed on device."""
    from decode_w4a16_affine_amd import GROUP

    stack = {}
    host0 = {}
    for i, p in enumerate(synthetic.LAYER_ORDER):
        N, K = synthetic.PROJECTIONS[p]
        w = synthetic.quantized_weights(N, K, seed=0, tag=(i,))
        host0[p] = w
        qw0 = torch.from_numpy(w.qw.view(np.int32)).cuda()
        s0 = torch.from_numpy(w.scales.view(np.int16)).view(torch.bfloat16).cuda()
        b0 = torch.from_numpy(w.biases.view(np.int16)).view(torch.bfloat16).cuda()
        qw = torch.empty((layers, N, K // 8), dtype=torch.int32, device="cuda")
        s = torch.empty((layers, N, K // GROUP), dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(s)
        for l in range(layers):
            key = np.array([(0x9E3779B9 * l) & 0xFFFFFFFF], dtype=np.uint32).view(np.int32)[0]
            qw[l] = qw0 ^ int(key)
            s[l] = s0
            b[l] = b0
        x = synthetic.activations(8, K, seed=0, tag=(100 + i,))
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty((8, N), dtype=torch.bfloat16, device="cuda")
        stack[p] = dict(qw=qw, s=s, b=b, x=xd, y=y, N=N, K=K)
    torch.cuda.synchronize()
    return stack, host0


# Launch units of one layer: the projections in a unit share their activations
# and go out in one call.
UNITS_GROUPED = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate_up",)), ("down", ("down",)))
UNITS_SEPARATE = tuple((p, (p,)) for p in synthetic.LAYER_ORDER)


def make_step(w4, stack, M: int, layers: int, units=UNITS_GROUPED, only=None):
    units = [u for u in units if only is None or u[0] in only]
    xs = {u: stack[ps[0]]["x"][:M] for u, ps in units}
    ys = {p: stack[p]["y"][:M] for _, ps in units for p in ps}

    def step():
        for l in range(layers):
            for u, ps in units:
                if len(ps) == 1:
                    d = stack[ps[0]]
                    w4.w4a16_matmul(xs[u], d["qw"][l], d["s"][l], d["b"][l], ys[ps[0]])
                else:
                    w4.w4a16_matmul_grouped(xs[u], [(stack[p]["qw"][l], stack[p]["s"][l], stack[p]["b"][l], ys[p])
                                                   for p in ps])

    return step


def unit_bytes(M: int, ps) -> int:
    return sum(call_bytes(M, *synthetic.PROJECTIONS[p]) for p in ps)


def unit_flops(M: int, ps) -> int:
    # per weight: the dequantizing fma, then one fma per activation row
    return sum(2 * (M + 1) * synthetic.PROJECTIONS[p][0] * synthetic.PROJECTIONS[p][1] for p in ps)


def step_fp32_floor_ms(M: int, layers: int) -> float:
    """The step's fp32 fmas at PEAK_FP32_FMA_TFLOPS (no launch or memory time)."""
    return layers * sum(unit_flops(M, ps) for _, ps in UNITS_GROUPED) / (PEAK_FP32_FMA_TFLOPS * 1e12) * 1e3


def prefill_matrix_factor(M: int, N: int):
    """Matrix-core work of w4a16_matmul_prefill over its algorithmic 2 M N K
    flops, by the form the entry point picks: 128-row LDS tiles 1.25 (a pass
    over the codes and a quarter-size pass for the activation sums), 64-row
    tiles 1.5 (that pass is half the size), the per-wave form 2 (hi and lo
    weight parts); None up to 16 rows (decode kernels, no matrix cores)."""
    if M <= 16:
        return None
    t128 = -(-M // 128) * -(-N // 128)
    t64 = -(-M // 64) * -(-N // 128)
    if M > 40 and t128 < 256 and 160 <= t64 < 256:
        return 1.5
    if M > 64 and t128 >= 96:
        return 1.25
    return 2.0


def unit_issue_floor_us(M: int, ps) -> float:
    """VALU issue time of the literal arithmetic of one launch spread evenly
    over every SIMD (WORD_ISSUE_CYCLES per packed word; no launch, memory,
    LDS or reduction time)."""
    words = sum(synthetic.PROJECTIONS[p][0] * synthetic.PROJECTIONS[p][1] for p in ps) / 8
    cycles = words / 64 / (CUS * SIMDS) * (WORD_ISSUE_CYCLES[0] + WORD_ISSUE_CYCLES[1] * M)
    return cycles / (CLOCK_GHZ * 1e3)


def step_issue_floor_ms(M: int, layers: int) -> float:
    return layers * sum(unit_issue_floor_us(M, ps) for _, ps in UNITS_GROUPED) * 1e-3


def capture(torch, fn):
    fn()  # eager warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps: int, warmup: int, min_warm_s: float = 0.0, per_step: bool = False):
    """Replay `warmup` times, and further until `min_warm_s` seconds of replays
    have run (the GPU's clocks settle only after some tenths of a second of
    load), then time `steps` replays between two events: the mean ms per
    replay.  per_step: also an event between consecutive replays, and return
    (mean, [ms of each replay])."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    # graph replays run on the current stream, where the events are recorded
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step else 2)]
    ev[0].record()
    for i in range(steps):
        g.replay()
        if per_step:
            ev[i + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / steps
    if not per_step:
        return mean
    return mean, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def percentiles(ms):
    """p10, median and p90 of per-step times (ms)."""
    q = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return dict(p10=round(float(q[0]), 5), p50=round(float(q[1]), 5), p90=round(float(q[2]), 5))


def kernel_durations(torch, w4, stack, layers: int, M: int = 1, reps: int = 10):
    """Average duration of one launch of each unit of the grouped step at M
    activation rows: a graph holding that unit's launch for every layer (cold
    weights) is replayed `reps` times between two events on the replay stream,
    and the elapsed time is divided by the number of launches.  Graph replays
    leave no measurable gap between consecutive kernels beyond the launch
    floor, so this is the kernel duration as the step sees it."""
    out = {}
    for u, ps in UNITS_GROUPED + tuple(x for x in UNITS_SEPARATE if x[0] in ("q", "k", "v")):
        units = UNITS_GROUPED if u in dict(UNITS_GROUPED) else UNITS_SEPARATE
        g = capture(torch, make_step(w4, stack, M, layers, units=units, only=(u,)))
        out[u] = time_graph(torch, g, reps, 2, WARM_S) * 1e3 / layers
        del g
    return out


def read_ceiling(torch, nbytes: int = 1 << 30, reps: int = 20):
    """GB/s of the plain 128-bit streaming-read kernel (libw4a16_probe.so) over
    `nbytes` of device memory (four times the 256 MB last-level cache), timed
    launch by launch between events after a second of warm-up; the best of a
    few launch shapes and both cache policies (median over the launches of
    each) is the ceiling."""
    from decode_w4a16_affine_amd import profiling

    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    src.fill_(0x01234567)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < FIRST_WARM_S or time.perf_counter() - t0 < 0.2:
        for _ in range(4):
            profiling.stream_read(torch, src, sink, 3 * cus, True)
        torch.cuda.synchronize()
    tried = {}
    for nt in (True, False):
        for per_cu in (2, 3, 4):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record()
            for i in range(reps):
                profiling.stream_read(torch, src, sink, per_cu * cus, nt)
                ev[i + 1].record()
            torch.cuda.synchronize()
            ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
            tried[f"{'nt' if nt else 'plain'}_{per_cu}_per_cu"] = nbytes / (ms * 1e-3) / 1e9
    del src, sink
    best = max(tried, key=lambda k: float(np.median(tried[k])))
    gbs = tried[best]
    return dict(gbs=round(float(np.median(gbs)), 1), gbs_best=round(float(gbs.max()), 1),
                gbs_p10=round(float(np.percentile(gbs, 10)), 1), gbs_p90=round(float(np.percentile(gbs, 90)), 1),
                frac_of_peak=round(float(np.median(gbs)) / PEAK_GBS, 4), bytes=nbytes, launches=reps,
                kernel=f"stream_read_kernel (16-byte loads, 2 in flight per thread), best shape {best}",
                medians={k: round(float(np.median(v)), 1) for k, v in tried.items()})


def host_cpu():
    """CPU model and counts of the host the CPU baseline runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), cpus_usable=affinity)


def config_timings(torch, w4, reps: int = 5):
    """Per-call time of the tiny, LM-head, square and routed configurations,
    cold: C copies of each matrix (codes xor-ed per copy on device, scales and
    biases copied) are rotated so that consecutive calls never share weights and
    one pass over the copies exceeds the 256 MB last-level cache.  Each call
    sequence is one HIP graph replayed between two events."""
    out = {}

    def upload(w, copies, shape=None):
        qw0 = torch.from_numpy(w.qw.view(np.int32)).cuda()
        s0 = torch.from_numpy(w.scales.view(np.int16)).view(torch.bfloat16).cuda()
        b0 = torch.from_numpy(w.biases.view(np.int16)).view(torch.bfloat16).cuda()
        if shape is not None:
            qw0, s0, b0 = qw0.view(shape[0]), s0.view(shape[1]), b0.view(shape[1])
        qw = torch.empty((copies,) + tuple(qw0.shape), dtype=torch.int32, device="cuda")
        sc = torch.empty((copies,) + tuple(s0.shape), dtype=torch.bfloat16, device="cuda")
        bi = torch.empty_like(sc)
        for c in range(copies):
            key = np.array([(0x9E3779B9 * c) & 0xFFFFFFFF], dtype=np.uint32).view(np.int32)[0]
            qw[c] = qw0 ^ int(key)
            sc[c] = s0
            bi[c] = b0
        del qw0, s0, b0
        torch.cuda.synchronize()
        return qw, sc, bi

    def timed(calls, nbytes):
        # one graph of len(calls) calls over rotated weight copies; every
        # replay is timed between events, and its mean per call is one sample:
        # at least 100 calls for calls under 100 MB, at least 20 above
        g = capture(torch, lambda: [c() for c in calls])
        need = 100 if nbytes < 100e6 else 20
        nrep = max(reps, -(-need // len(calls)))
        _, each = time_graph(torch, g, nrep, 2, WARM_S, per_step=True)
        del g
        per_call = np.array(each) * 1e3 / len(calls)
        p10, us, p90 = (float(v) for v in np.percentile(per_call, [10, 50, 90]))
        gbs = nbytes / (us * 1e-6) / 1e9
        return dict(us=round(us, 3), p10_us=round(p10, 3), p90_us=round(p90, 3),
                    mean_us=round(float(per_call.mean()), 3), calls=nrep * len(calls),
                    gbs=round(gbs, 1), frac_of_peak=round(gbs / PEAK_GBS, 4))

    # tiny qmv (latency-bound; reported for completeness)
    t = synthetic.TINY
    w = synthetic.quantized_weights(t["N"], t["K"], seed=0)
    qw, sc, bi = upload(w, 8)
    x = torch.from_numpy(synthetic.activations(1, t["K"], seed=0).view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.empty((1, t["N"]), dtype=torch.bfloat16, device="cuda")
    calls = [lambda c=c: w4.w4a16_matmul(x, qw[c], sc[c], bi[c], y) for c in range(8)]
    out["tiny"] = {"1": timed(calls, call_bytes(1, t["N"], t["K"]))}
    del qw, sc, bi
    log(f"tiny: {out['tiny']}")

    # tied LM head with fused argmax (bf16 logits and int32 argmax written)
    t = synthetic.LM_HEAD
    N, K = t["N"], t["K"]
    w = synthetic.quantized_weights(N, K, seed=0, tag=(N,), bias="exact")
    qw, sc, bi = upload(w, 3)
    del w
    out["lm_head"] = {}
    for M in t["M"]:
        x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N,)).view(np.int16)).view(torch.bfloat16).cuda()
        logits = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        am = torch.empty((M,), dtype=torch.int32, device="cuda")
        ws = torch.empty((w4.w4a16_lmhead_argmax_workspace_bytes(M, N, K),), dtype=torch.uint8, device="cuda")
        calls = [lambda c=c: w4.w4a16_lmhead_argmax(x, qw[c], sc[c], bi[c], logits, am, ws)
                 for c in (0, 1, 2, 0, 1, 2)]
        out["lm_head"][str(M)] = timed(calls, call_bytes(M, N, K) + 4 * M)
    log(f"lm_head: {out['lm_head']}")

    # quantized row gather from the same (tied embedding) table to bf16: a
    # decode step's tokens and a prefill-sized batch of seeded random rows
    out["gather"] = {}
    for R in (8, 4096):
        rows = torch.from_numpy(np.random.default_rng(R).integers(0, N, size=R).astype(np.int32)).cuda()
        emb = torch.empty((R, K), dtype=torch.bfloat16, device="cuda")
        calls = [lambda c=c: w4.w4a16_gather_rows(qw[c], sc[c], bi[c], rows, emb) for c in (0, 1, 2, 0, 1, 2)]
        out["gather"][str(R)] = timed(calls, R * (K // 2 + (K // 64) * 4 + 2 * K + 4))
    del qw, sc, bi
    log(f"gather: {out['gather']}")

    # group 128 (scales and biases per 128 codes): the largest decode
    # projections and the square matrix at M = 1 and a verify batch
    out["group128"] = {}
    for name, (N, K) in (("gate_up", synthetic.PROJECTIONS["gate_up"]), ("down", synthetic.PROJECTIONS["down"]),
                         ("square", (synthetic.SQUARE["N"], synthetic.SQUARE["K"]))):
        w = synthetic.quantized_weights(N, K, group=128, seed=0, tag=(N, 128))
        copies = max(3, -(-(512 << 20) // w.nbytes))   # one pass over the copies: > 2x the 256 MB cache
        qw, sc, bi = upload(w, copies)
        del w
        out["group128"][name] = {}
        for M in (1, 5):
            x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N, 128)).view(np.int16)).view(torch.bfloat16).cuda()
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            calls = [lambda c=c: w4.w4a16_matmul(x, qw[c], sc[c], bi[c], y, group=128) for c in range(copies)]
            out["group128"][name][str(M)] = timed(calls, call_bytes(M, N, K, 128))
        del qw, sc, bi
    log(f"group128: {out['group128']}")

    # GeGLU on the fused gate+up matrix (w4a16_matmul_geglu: h = GELU(gate) * up,
    # [M, I] written) beside the plain product of the same matrix ([M, 2I]
    # written, no activation): the epilogue's cost over the stream it rides on
    N, K = synthetic.PROJECTIONS["gate_up"]
    w = synthetic.quantized_weights(N, K, seed=0, tag=(N, 11))
    copies = max(3, -(-(512 << 20) // w.nbytes))
    qw, sc, bi = upload(w, copies)
    del w
    out["geglu"] = {}
    for M in (1, 5):
        x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N, 11)).view(np.int16)).view(torch.bfloat16).cuda()
        h = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        calls = [lambda c=c: w4.w4a16_matmul_geglu(x, qw[c], sc[c], bi[c], h) for c in range(copies)]
        fused = timed(calls, call_bytes(M, N, K) - M * N)
        calls = [lambda c=c: w4.w4a16_matmul(x, qw[c], sc[c], bi[c], y) for c in range(copies)]
        out["geglu"][str(M)] = dict(fused, plain_product_us=timed(calls, call_bytes(M, N, K))["us"])
    del qw, sc, bi
    log(f"geglu: {out['geglu']}")

    # square qmv / qmm
    t = synthetic.SQUARE
    N, K = t["N"], t["K"]
    w = synthetic.quantized_weights(N, K, seed=0, tag=(N,))
    qw, sc, bi = upload(w, 8)
    del w
    out["square"] = {}
    for M in t["M"]:
        x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N,)).view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        calls = [lambda c=c: w4.w4a16_matmul(x, qw[c], sc[c], bi[c], y) for c in range(8)]
        out["square"][str(M)] = timed(calls, call_bytes(M, N, K))
    del qw, sc, bi
    log(f"square: {out['square']}")

    # prefill-sized products (w4a16_matmul_prefill, matrix cores) on the decode
    # stack's gate+up and down shapes: flop-bound, so priced against the dense
    # bf16 matrix-core peak.  Algorithmic flops are 2*M*N*K; the matrix cores
    # execute prefill_matrix_factor(M, N) times that (mfma_tflops).
    out["prefill"] = {}
    for name in ("gate_up", "down"):
        N, K = synthetic.PROJECTIONS[name]
        w = synthetic.quantized_weights(N, K, seed=0, tag=(N, 7))
        copies = max(2, -(-(512 << 20) // w.nbytes))   # cold weights for the memory-bound small M
        qw, sc, bi = upload(w, copies)
        del w
        out["prefill"][name] = {}
        for M in PREFILL_M:
            x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N, 7)).view(np.int16)).view(torch.bfloat16).cuda()
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            calls = [lambda c=c: w4.w4a16_matmul_prefill(x, qw[c], sc[c], bi[c], y) for c in range(copies)]
            r = timed(calls, call_bytes(M, N, K))
            tflops = 2.0 * M * N * K / (r["us"] * 1e-6) / 1e12
            r.update(tflops=round(tflops, 1), frac_of_bf16_peak=round(tflops / PEAK_BF16_TFLOPS, 4))
            factor = prefill_matrix_factor(M, N)
            if factor is not None:
                r.update(mfma_tflops=round(factor * tflops, 1))
            out["prefill"][name][str(M)] = r
            del x, y
        del qw, sc, bi
    log(f"prefill: {out['prefill']}")

    # routed MoE stack: 64 experts, top-8 of 64 per token
    t = synthetic.MOE
    E, N, K, top_k = t["E"], t["N"], t["K"], t["top_k"]
    w = synthetic.quantized_weights(E * N, K, seed=0, tag=(E,))
    qw, sc, bi = upload(w, 3, shape=((E, N, K // 8), (E, N, K // 64)))
    del w
    out["moe"] = {}
    for M in t["M"]:
        ids_h = synthetic.expert_ids(M, top_k, E, seed=0)
        ids = torch.from_numpy(ids_h).cuda()
        x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(E,)).view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty((M, top_k, N), dtype=torch.bfloat16, device="cuda")
        calls = [lambda c=c: w4.w4a16_matmul_id(x, qw[c], sc[c], bi[c], ids, y) for c in (0, 1, 2, 0, 1, 2)]
        U = len(np.unique(ids_h))
        nbytes = U * (N * K // 2 + N * (K // 64) * 4) + 2 * M * K + 2 * M * top_k * N + 4 * M * top_k
        out["moe"][str(M)] = dict(timed(calls, nbytes), experts=U)
    del qw, sc, bi
    log(f"moe: {out['moe']}")
    torch.cuda.empty_cache()
    return out


def cpu_baseline(host0, seconds: float = 10.0):
    """The oracle, as it stands, on one host core over layer 0's projections."""
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    xs = {p: synthetic.activations(1, host0[p].K, seed=0, tag=(100 + i,))
          for i, p in enumerate(synthetic.LAYER_ORDER)}
    done_bytes = 0
    calls = 0
    t0 = time.perf_counter()
    while True:
        for p in synthetic.LAYER_ORDER:
            w = host0[p]
            oracle.qmm(xs[p], w.qw, w.scales, w.biases)
            done_bytes += call_bytes(1, w.N, w.K)
            calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(done_bytes / dt / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{calls} single-row products over one layer's q,k,v,o,gate_up,down weights "
                       f"({calls // 6} layer passes, {dt:.1f} s, 1 thread, fp64 accumulation)")


def cpu_baseline_threads(host0, threads: int, seconds: float = 10.0):
    """The same oracle function over row slices of each projection on `threads`
    host threads (the C call releases the GIL; row results are unchanged)."""
    import concurrent.futures as cf

    import oracle

    xs = {p: synthetic.activations(1, host0[p].K, seed=0, tag=(100 + i,))
          for i, p in enumerate(synthetic.LAYER_ORDER)}
    slices = {p: np.array_split(np.arange(host0[p].N, dtype=np.int32), threads) for p in synthetic.LAYER_ORDER}
    done_bytes = 0
    passes = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while True:
            for p in synthetic.LAYER_ORDER:
                w = host0[p]
                list(ex.map(lambda r: oracle.qmm(xs[p], w.qw, w.scales, w.biases, rows=r), slices[p]))
                done_bytes += call_bytes(1, w.N, w.K)
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return dict(value=round(done_bytes / dt / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{passes} passes over one layer's q,k,v,o,gate_up,down weights at M=1, rows split "
                       f"over {threads} threads ({dt:.1f} s, fp64 accumulation)")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--warm-seconds", type=float, default=None,
                    help="untimed replay time before each measurement (default: 1 s before the first, "
                         "0.25 s before the others; profiler runs use 0)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-call timings of the tiny, LM-head, row-gather, group-128, square and routed configurations")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device-to-device copy (a known-size reference for "
                         "memory-traffic counters)")
    args = ap.parse_args()
    global FIRST_WARM_S, WARM_S
    if args.warm_seconds is not None:
        FIRST_WARM_S = WARM_S = max(0.0, args.warm_seconds)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(a multi-GPU deployment would shard output rows or experts; this benchmark runs on one)", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_w4a16_affine_amd as w4

    w4.lib()  # fails loudly when the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    L = args.layers
    log(f"building {L}-layer weight stack")
    stack, host0 = build_stack(torch, L)

    results = {}
    Ms = [1] if args.no_verify else [1] + list(synthetic.VERIFY_M)
    for M in Ms:
        g = capture(torch, make_step(w4, stack, M, L))
        steps = args.steps if M == 1 else max(10, args.steps // 2)
        warm = args.warmup if M == 1 else max(3, args.warmup // 2)
        ms, each = time_graph(torch, g, steps, warm, FIRST_WARM_S if M == 1 else WARM_S, per_step=True)
        nb = step_bytes(M, L)
        results[M] = dict(ms=ms, gbs=nb / (ms * 1e-3) / 1e9, bytes=nb, steps=steps, warmup=warm,
                          pct=percentiles(each))
        log(f"M={M}: {ms:.4f} ms/step, {results[M]['gbs']:.1f} GB/s")
        del g
    g = capture(torch, make_step(w4, stack, 1, L, units=UNITS_SEPARATE))
    ms_sep = time_graph(torch, g, args.steps, args.warmup, WARM_S)
    del g
    log(f"M=1, six launches per layer: {ms_sep:.4f} ms/step")

    # Dominant kernel (largest share of the M=1 step): one kernel symbol per
    # schedule, so launch units are grouped by the kernel that serves them.
    dur = kernel_durations(torch, w4, stack, L)
    per_group = {}
    for u, ps in UNITS_GROUPED:
        N, K = synthetic.PROJECTIONS[ps[0]]
        kern = w4.w4a16_schedule_name(1, N, K)
        e = per_group.setdefault(kern, dict(us_total=0.0, bytes_total=0, launches=0, units=[], grids=[]))
        e["us_total"] += dur[u]
        e["bytes_total"] += unit_bytes(1, ps)
        e["launches"] += 1
        e["units"].append(u)
        e["grids"].append(launch_grid(kern, [synthetic.PROJECTIONS[p][0] for p in ps]))
    dom = max(per_group, key=lambda k: per_group[k]["us_total"])
    pg = per_group[dom]
    avg_us = pg["us_total"] / pg["launches"]
    avg_bytes = pg["bytes_total"] / pg["launches"]
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9
    # HBM bytes per launch from the committed counter record (null when the
    # kernels changed after the counters were taken)
    from decode_w4a16_affine_amd import profiling

    weights = {}
    for grid in pg["grids"]:
        weights[grid] = weights.get(grid, 0) + 1
    traffic = profiling.traffic_per_launch(TRAFFIC_RECORD, dom, weights)
    unit_ps = dict(UNITS_GROUPED + UNITS_SEPARATE)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_GBS, 4),
                    traffic=None if traffic is None else int(traffic),
                    kernel=dom, serves=pg["units"], avg_launch_us=round(avg_us, 3),
                    avg_launch_bytes=int(avg_bytes),
                    per_launch_us={u: round(v, 3) for u, v in dur.items()},
                    per_launch_gbs={u: round(unit_bytes(1, unit_ps[u]) / (v * 1e-6) / 1e9, 1)
                                    for u, v in dur.items()},
                    per_launch_frac={u: round(unit_bytes(1, unit_ps[u]) / (v * 1e-6) / 1e9 / PEAK_GBS, 4)
                                     for u, v in dur.items()})

    # the verify steps' launches, unit by unit, with the kernel each one runs
    verify_units = {}
    for M in results:
        if M == 1:
            continue
        d = kernel_durations(torch, w4, stack, L, M=M)
        verify_units[M] = {u: dict(us=round(v, 3), gbs=round(unit_bytes(M, unit_ps[u]) / (v * 1e-6) / 1e9, 1),
                                   frac_of_peak=round(unit_bytes(M, unit_ps[u]) / (v * 1e-6) / 1e9 / PEAK_GBS, 4),
                                   fp32_tflops=round(unit_flops(M, unit_ps[u]) / (v * 1e-6) / 1e12, 2),
                                   frac_of_fp32_fma_peak=round(unit_flops(M, unit_ps[u]) / (v * 1e-6) / 1e12
                                                               / PEAK_FP32_FMA_TFLOPS, 4),
                                   issue_floor_us=round(unit_issue_floor_us(M, unit_ps[u]), 3),
                                   kernel=w4.w4a16_schedule_name(M, *synthetic.PROJECTIONS[unit_ps[u][0]]))
                           for u, v in d.items()}
        log(f"M={M} launches (us): " + ", ".join(f"{u} {v['us']}" for u, v in verify_units[M].items()))

    log("read ceiling (1 GiB, 16-byte streaming read)")
    ceiling = read_ceiling(torch)
    log(f"read ceiling: {ceiling['gbs']} GB/s")
    roofline.update(read_ceiling_gbs=ceiling["gbs"], frac_of_read_ceiling=round(achieved / ceiling["gbs"], 4))

    configs = None if args.no_configs else config_timings(torch, w4)

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    host = host_cpu()
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, 1 core)")
        cpu = cpu_baseline(host0, args.cpu_seconds)
        # at most 16 threads: the CPU share of one GPU on the benchmark hosts,
        # whatever the host reports (the host's counts are recorded beside it)
        threads = max(1, min(16, host["cpus_usable"] or 1))
        log(f"cpu baseline (oracle, {threads} threads)")
        cpu_all = cpu_baseline_threads(host0, threads, args.cpu_seconds)
        for c in (cpu, cpu_all):
            c.update(host)

    r1 = results[1]
    line = {
        "metric": METRIC,
        "value": round(r1["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r1["steps"],
        "warmup": r1["warmup"],
        "ms_per_step": round(r1["ms"], 5),
        "ms_per_step_pct": r1["pct"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode step, M=1: {L} layers x (q,k,v,o 2560/512/512/2560<-2560, "
                               "gate_up 20480<-2560, down 2560<-10240), W4 group 64, bf16 x/y; "
                               "q/k/v in one grouped launch, one HIP graph per step",
                   "layers": L, "bytes_per_step": r1["bytes"], "frac_of_peak": round(r1["gbs"] / PEAK_GBS, 4),
                   "six_launches_per_layer": dict(ms_per_step=round(ms_sep, 5),
                                                  gbs=round(r1["bytes"] / (ms_sep * 1e-3) / 1e9, 2))},
        "verify": {str(M): dict(gbs=round(r["gbs"], 2), ms_per_step=round(r["ms"], 5),
                                frac_of_peak=round(r["gbs"] / PEAK_GBS, 4),
                                cost_vs_m1=round(r["ms"] / r1["ms"], 4), ms_per_step_pct=r["pct"],
                                fp32_fma_floor_ms=round(step_fp32_floor_ms(M, L), 5),
                                hbm_floor_ms=round(r["bytes"] / (PEAK_GBS * 1e9) * 1e3, 5),
                                frac_of_fp32_fma_peak=round(step_fp32_floor_ms(M, L) / r["ms"], 4),
                                issue_floor_ms=round(step_issue_floor_ms(M, L), 5),
                                per_launch=verify_units.get(M))
                   for M, r in results.items() if M != 1},
        "roofline": roofline,
        "read_ceiling": ceiling,
        "read_ceiling_gbs": ceiling["gbs"],
        "cpu_model": host["cpu_model"],
        "host_cpus": host,
        "configs": configs,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_all,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
