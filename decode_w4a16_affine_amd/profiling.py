"""Summaries of rocprofv3 output for the W4A16 kernels.

Turns the CSV files of ``rocprofv3 --kernel-trace --stats`` and of two
``rocprofv3 --pmc`` passes (FETCH_SIZE, then WRITE_SIZE) into short text
summaries and a per-kernel traffic record.  Counter readings are converted to
HBM bytes with the factor that a device-to-device copy of known size reads on
the same counter (the benchmark's ``--calibrate-copy`` phase runs one).

    python -m decode_w4a16_affine_amd.profiling stats  <kernel_stats.csv> <out.md> "<command>"
    python -m decode_w4a16_affine_amd.profiling trace  <kernel_trace.csv> <out.md> "<command>" [kernel]
    python -m decode_w4a16_affine_amd.profiling traffic <fetch.csv> <write.csv> <out.json> "<fetch cmd>" "<write cmd>"
    python -m decode_w4a16_affine_amd.profiling traffic-md <traffic.json> <out.md>
    python -m decode_w4a16_affine_amd.profiling sq <counter_collection.csv>[,<more.csv>] <out.md> "<command>"
    python -m decode_w4a16_affine_amd.profiling prefill-workload [M]
    python -m decode_w4a16_affine_amd.profiling configs-workload

``configs-workload`` runs every configuration's decode kernels a few times on
cold weights, then the calibration copy (the program for the counter passes of
the configuration kernels).  ``prefill-workload`` runs the prefill products of the decode stack's gate+up
and down shapes at M rows (default 4096; four eager calls each, seeded
synthetic inputs): the program to run under ``rocprofv3 --pmc`` for the
matrix-core kernels.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# the device code's sources and the script that holds its compile flags
KERNEL_SOURCES = [os.path.join(HERE, "csrc", f) for f in
                  ("qmm_device.hpp", "qmm_prefill.hpp", "sched.hpp", "kernels.hpp", "ops.hpp", "inst.hip",
                   "prefill.hip", "w4a16.hip")] + [os.path.join(HERE, "build.py")]
PROBE_LIB = os.path.join(HERE, "libw4a16_probe.so")


PROBE_EXPORTS = ("w4a16_probe_stream_read", "w4a16_probe_bf16_round_check")


def probe_lib():
    """libw4a16_probe.so (include/w4a16_probe.h), loaded once."""
    import ctypes

    global _probe
    try:
        return _probe
    except NameError:
        pass
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.w4a16_probe_stream_read.restype = ctypes.c_int
    lib.w4a16_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p]
    lib.w4a16_probe_bf16_round_check.restype = ctypes.c_int
    lib.w4a16_probe_bf16_round_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    _probe = lib
    return lib


def bf16_round_check(torch):
    """(patterns where the hardware bf16 conversion and the rounding helper
    differ, the smallest such fp32 pattern or 0xFFFFFFFF): one launch over all
    2^32 fp32 bit patterns (include/w4a16_probe.h)."""
    import ctypes

    lib = probe_lib()
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.w4a16_probe_bf16_round_check(ctypes.c_void_p(mism.data_ptr()), ctypes.c_void_p(first.data_ptr()),
                                          ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"w4a16_probe_bf16_round_check failed: hipError {rc}")
    torch.cuda.synchronize()
    return int(mism.item()), int(first.item()) & 0xFFFFFFFF


def stream_read(torch, src, sink, blocks: int = 0, nontemporal: bool = True, stream=None) -> None:
    """One launch of the 128-bit streaming-read kernel (include/w4a16_probe.h) over
    the bytes of the contiguous device tensor `src`; `sink` a 4-byte device tensor."""
    import ctypes

    lib = probe_lib()
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda):
        raise ValueError("stream_read takes contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    st = (stream or torch.cuda.current_stream()).cuda_stream
    rc = lib.w4a16_probe_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                     blocks, int(bool(nontemporal)), ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"w4a16_probe_stream_read failed: hipError {rc}")
COPY_BYTES = 256 << 20


def kernel_source_sha() -> str:
    """Hash of the device code and its build flags; counters taken on other code are stale."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    m = re.search(r"(qmm_\w+_kernel<[^>]*>|argmax_finalize_kernel|dequant_rows_kernel|gather_rows_kernel|pack_kernel|"
                  r"stream_read_kernel|bf16_round_check_kernel)", name)
    return m.group(1) if m else name.split("(")[0][:80]


def _ours(name: str) -> bool:
    """A kernel of this library (not a runtime copy or a torch kernel)."""
    return short_name(name) != name.split("(")[0][:80] or "qmm_" in name


def traffic_markdown(record_json: str, out_md: str) -> None:
    """The traffic record as a table: HBM bytes per launch by kernel and grid."""
    rec = json.load(open(record_json))
    lines = ["# HBM traffic per launch (rocprofv3 counters)", "",
             f"FETCH_SIZE: `{rec['fetch_command']}`", "", f"WRITE_SIZE: `{rec['write_command']}`", "",
             f"Counter bytes are scaled by the reading of a {rec['copy_bytes'] >> 20} MiB device copy in the same run: "
             f"fetch x{rec['fetch_factor']}, write x{rec['write_factor']}.  Kernel sources: sha256 "
             f"{rec['source_sha256'][:16]}.", "",
             "| kernel | grid (work-items) | fetched bytes | written bytes | HBM bytes |", "|---|---|---|---|---|"]
    for k, d in rec["kernels"].items():
        for g, v in d.items():
            lines.append(f"| `{k}` | {g} | {v['fetch_bytes']:,} | {v['write_bytes']:,} | {v['hbm_bytes']:,} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace(trace_csv: str, out_md: str, command: str, focus: str = "") -> dict:
    """Per-kernel distribution of the dispatch durations in a rocprofv3 kernel
    trace, and for each kernel the launch period of back-to-back dispatches
    of that kernel (start to next start when no other kernel ran between: the
    duration plus the gap a graph leaves before the next launch, which is what
    events around a graph of consecutive launches measure)."""
    import numpy as np

    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Name") or ""
            st = int(r.get("Start_Timestamp") or r.get("Begin_Ns") or 0)
            en = int(r.get("End_Timestamp") or r.get("End_Ns") or 0)
            rows.append((st, en, short_name(name)))
    rows.sort()
    dur, period = {}, {}
    for i, (st, en, k) in enumerate(rows):
        dur.setdefault(k, []).append((en - st) / 1e3)
        if i + 1 < len(rows) and rows[i + 1][2] == k:
            period.setdefault(k, []).append((rows[i + 1][0] - st) / 1e3)
    total = sum(sum(v) for v in dur.values()) or 1.0
    order = sorted(dur, key=lambda k: -sum(dur[k]))
    lines = ["# rocprofv3 kernel trace: dispatch durations", "", f"Command: `{command}`", "",
             "Durations are end minus start of each dispatch (us).  The launch period is start to next start",
             "over pairs of consecutive dispatches of the same kernel (graph replays of one projection's",
             "launches), i.e. the duration plus the gap before the next launch.", "",
             "| kernel | calls | mean | p10 | median | p90 | share | back-to-back pairs | median launch period |",
             "|---|---|---|---|---|---|---|---|---|"]
    summary = {}
    for k in order:
        d = np.array(dur[k])
        pr = np.array(period.get(k, []))
        q = np.percentile(d, [10, 50, 90])
        summary[k] = dict(calls=int(d.size), mean_us=float(d.mean()), p10_us=float(q[0]), median_us=float(q[1]),
                          p90_us=float(q[2]), pairs=int(pr.size),
                          period_median_us=float(np.median(pr)) if pr.size else None)
        per = f"{np.median(pr):.3f}" if pr.size else "-"
        lines.append(f"| `{k}` | {d.size} | {d.mean():.3f} | {q[0]:.3f} | {q[1]:.3f} | {q[2]:.3f} | "
                     f"{100 * d.sum() / total:.2f}% | {pr.size} | {per} |")
        if len(lines) > 60:
            break
    if focus:
        for k, v in summary.items():
            if k == focus:
                lines += ["", f"Focus `{k}`: mean {v['mean_us']:.3f} us, median {v['median_us']:.3f} us, "
                              f"median launch period {v['period_median_us']} us over {v['pairs']} pairs."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return summary


def _per_dispatch(path: str, counter: str):
    out = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") == counter:
            out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]) * 1024.0))
    return out


def _copy_factor(rows) -> float:
    """Known bytes / counter bytes for the 256 MiB copy (the largest copy dispatch)."""
    copies = [v for n, g, v in rows if "copyBuffer" in n]
    big = sorted(copies, reverse=True)[:3]
    if not big:
        raise ValueError("no copy dispatch found for calibration")
    return COPY_BYTES / statistics.median(big)


def summarize_traffic(fetch_csv: str, write_csv: str, out_json: str, fetch_cmd: str, write_cmd: str) -> dict:
    fr = _per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = _per_dispatch(write_csv, "WRITE_SIZE")
    ff, wf = _copy_factor(fr), _copy_factor(wr)
    kernels = {}
    for rows, key, fac in ((fr, "fetch_bytes", ff), (wr, "write_bytes", wf)):
        groups = {}
        for n, g, v in rows:
            if not _ours(n):
                continue
            groups.setdefault((short_name(n), g), []).append(v * fac)
        for (k, g), vals in groups.items():
            kernels.setdefault(k, {}).setdefault(str(g), {})[key] = statistics.median(vals)
    rec = dict(source_sha256=kernel_source_sha(), copy_bytes=COPY_BYTES,
               fetch_factor=round(ff, 5), write_factor=round(wf, 5),
               fetch_command=fetch_cmd, write_command=write_cmd,
               kernels={k: {g: dict(fetch_bytes=round(v.get("fetch_bytes", 0.0)),
                                    write_bytes=round(v.get("write_bytes", 0.0)),
                                    hbm_bytes=round(v.get("fetch_bytes", 0.0) + v.get("write_bytes", 0.0)))
                            for g, v in sorted(d.items(), key=lambda kv: int(kv[0]))}
                        for k, d in sorted(kernels.items())})
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def traffic_per_launch(record_path: str, kernel: str, grid_sizes_weights: dict):
    """Average HBM bytes per launch of `kernel` over launches with the given grid
    sizes (grid size -> launches per step), or None when the record is stale."""
    if not os.path.exists(record_path):
        return None
    rec = json.load(open(record_path))
    if rec.get("source_sha256") != kernel_source_sha():
        return None
    d = rec.get("kernels", {}).get(kernel)
    if not d:
        return None
    tot = n = 0
    for g, w in grid_sizes_weights.items():
        if str(g) not in d:
            return None
        tot += d[str(g)]["hbm_bytes"] * w
        n += w
    return tot / n if n else None


# VALU issue time of a launch if every SIMD issued one wave64 instruction per
# 4 cycles at 2.4 GHz: total VALU instructions / (256 CUs x 4 SIMDs) x 4
# cycles.  4 cycles is the rate of the dequantizing v_fma_mix_f32; fp32 fmas
# and simple integer ops issue in about 2.3 (two or more waves per SIMD), so
# for the decode kernels' mix (about 8 of every 53 instructions at M = 5, 8 of
# 21 at M = 1) this is an upper estimate, roughly 1.3-1.6 times the issue time.
VALU_US_PER_INSTR = 4.0 / (256 * 4) / 2400.0


def summarize_sq(csv_path: str, out_md: str, command: str) -> None:
    """Per kernel and grid size: median shader-sequencer counts per launch and
    per wave (VALU and LDS instructions, LDS bank-conflict cycles per LDS
    instruction, wave cycles), and the launch's VALU issue time at one wave
    instruction per SIMD per 4 cycles (an upper estimate, see VALU_US_PER_INSTR)."""
    groups = {}
    for path in csv_path.split(","):   # several counter passes of the same program
        for r in csv.DictReader(open(path)):
            if "qmm_" not in r["Kernel_Name"]:
                continue
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            groups.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    matrix = any("SQ_INSTS_MFMA" in d for d in groups.values())
    lines = ["# Shader-sequencer counters per launch", "", f"Command: `{command}`", "",
             "| kernel | grid | waves | VALU instr / wave | VALU issue (us, all SIMDs) | LDS instr / wave | "
             "LDS conflict cycles / LDS instr | "
             "wave cycles / wave |" + (" MFMA instr / wave | MFMA busy / CU busy (per SIMD) | SQ_WAIT_INST_ANY "
                                       "/ wave cycles | SQ_WAIT_INST_LDS / wave cycles |" if matrix else ""),
             "|---|---|---|---|---|---|---|---|" + ("---|---|---|---|" if matrix else "")]
    for (k, g), d in sorted(groups.items()):
        med = {c: statistics.median(v) for c, v in d.items()}
        waves = med.get("SQ_WAVES", 0.0) or 1.0
        lds = med.get("SQ_INSTS_LDS", 0.0)
        line = (f"| `{k}` | {g} | {int(waves)} | {med.get('SQ_INSTS_VALU', 0.0) / waves:.0f} | "
                f"{med.get('SQ_INSTS_VALU', 0.0) * VALU_US_PER_INSTR:.2f} | {lds / waves:.0f} | "
                f"{med.get('SQ_LDS_BANK_CONFLICT', 0.0) / max(lds, 1.0):.2f} | "
                f"{med.get('SQ_WAVE_CYCLES', 0.0) / waves:.0f} |")
        if matrix:
            wc = max(med.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            line += (f" {med.get('SQ_INSTS_MFMA', 0.0) / waves:.0f} | "
                     f"{med.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / 4 / max(med.get('SQ_BUSY_CU_CYCLES', 0.0), 1.0):.2f} | "
                     f"{med.get('SQ_WAIT_INST_ANY', 0.0) / wc:.2f} | {med.get('SQ_WAIT_INST_LDS', 0.0) / wc:.2f} |")
        lines.append(line)
    # memory waiting and vector-memory instructions in flight, where a pass
    # collected them (SQ_INST_LEVEL_VMEM accumulates the outstanding count
    # every cycle, so divided by the wave cycles it is the average in flight)
    extra = [(k, g, d) for (k, g), d in sorted(groups.items()) if "SQ_WAIT_ANY" in d and "SQ_INST_LEVEL_VMEM" in d]
    if extra:
        lines += ["", "| kernel | grid | SQ_WAIT_ANY / wave cycles | vector-memory reads / wave | "
                      "vector-memory instructions in flight (average) |", "|---|---|---|---|---|"]
        for k, g, d in extra:
            med = {c: statistics.median(v) for c, v in d.items()}
            wc = max(med.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            waves = med.get("SQ_WAVES", 0.0) or 1.0
            lines.append(f"| `{k}` | {g} | {med['SQ_WAIT_ANY'] / wc:.2f} | "
                         f"{med.get('SQ_INSTS_VMEM_RD', 0.0) / waves:.0f} | {med['SQ_INST_LEVEL_VMEM'] / wc:.2f} |")
    # wave states, where a pass collected them: SQ_WAIT_ANY (wave-cycles spent
    # waiting for anything), SQ_WAIT_INST_ANY (waiting for any instruction
    # issue) and SQ_ACTIVE_INST_ANY (working on instructions), each over the
    # wave cycles; the three add up to about one
    states = [(k, g, d) for (k, g), d in sorted(groups.items())
              if all(c in d for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY"))]
    if states:
        lines += ["", "Wave states, fractions of SQ_WAVE_CYCLES:", "",
                  "| kernel | grid | waves | SQ_WAIT_ANY | SQ_WAIT_INST_ANY | SQ_ACTIVE_INST_ANY | "
                  "SQ_ACTIVE_INST_VALU | SQ_ACTIVE_INST_LDS | vector-memory instructions in flight (average) |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for k, g, d in states:
            med = {c: statistics.median(v) for c, v in d.items()}
            wc = max(med.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            cell = lambda c: f"{med[c] / wc:.2f}" if c in med else "-"   # noqa: E731
            lines.append(f"| `{k}` | {g} | {int(med.get('SQ_WAVES', 0.0))} | {cell('SQ_WAIT_ANY')} | "
                         f"{cell('SQ_WAIT_INST_ANY')} | {cell('SQ_ACTIVE_INST_ANY')} | {cell('SQ_ACTIVE_INST_VALU')} | "
                         f"{cell('SQ_ACTIVE_INST_LDS')} | {cell('SQ_INST_LEVEL_VMEM')} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def configs_workload(calls: int = 3) -> None:
    """The configurations' kernels, a few eager calls each on rotated weight
    copies (cold weights), then a 256 MiB device copy (the counters' byte
    calibration): the program to run under ``rocprofv3 --pmc``.  Covers the
    decode projections at M = 1, 2, 3, 5, the tied LM head (argmax) at M = 1
    and 3, the square matrix at M = 1, 4, 8, the routed stack at M = 1 and 8,
    GeGLU on the gate+up matrix at M = 1 and 5 and the row gather."""
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import torch

    import decode_w4a16_affine_amd as w4
    import synthetic

    def dev(w, copies, shape=None):
        qw0 = torch.from_numpy(w.qw.view(np.int32)).cuda()
        s0 = torch.from_numpy(w.scales.view(np.int16)).view(torch.bfloat16).cuda()
        b0 = torch.from_numpy(w.biases.view(np.int16)).view(torch.bfloat16).cuda()
        if shape is not None:
            qw0, s0, b0 = qw0.view(shape[0]), s0.view(shape[1]), b0.view(shape[1])
        out = []
        for c in range(copies):
            key = int(np.array([(0x9E3779B9 * c) & 0xFFFFFFFF], dtype=np.uint32).view(np.int32)[0])
            out.append((qw0 ^ key, s0.clone(), b0.clone()))
        return out

    def xs(M, K, tag):
        return torch.from_numpy(synthetic.activations(M, K, seed=0, tag=tag).view(np.int16)).view(torch.bfloat16).cuda()

    for name in synthetic.LAYER_ORDER:
        N, K = synthetic.PROJECTIONS[name]
        mats = dev(synthetic.quantized_weights(N, K, seed=0, tag=(N, 21)), 24)
        for M in (1, 2, 3, 5):
            x = xs(M, K, (N, 21))
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            for i in range(calls * 8):
                q, sc, bi = mats[i % len(mats)]
                w4.w4a16_matmul(x, q, sc, bi, y)
        torch.cuda.synchronize()
        print(f"{name}: done", flush=True)
        del mats
    t = synthetic.LM_HEAD
    N, K = t["N"], t["K"]
    mats = dev(synthetic.quantized_weights(N, K, seed=0, tag=(N,), bias="exact"), 3)
    for M in t["M"]:
        x = xs(M, K, (N,))
        for i in range(calls):
            q, sc, bi = mats[i % 3]
            w4.lmhead_argmax(x, q, sc, bi)
        rows = torch.arange(0, N, N // 4096, dtype=torch.int32, device="cuda")
        w4.gather_rows(q, sc, bi, rows)
    torch.cuda.synchronize()
    print("lm head: done", flush=True)
    del mats
    t = synthetic.SQUARE
    mats = dev(synthetic.quantized_weights(t["N"], t["K"], seed=0, tag=(t["N"],)), 4)
    for M in t["M"]:
        x = xs(M, t["K"], (t["N"],))
        for i in range(calls):
            q, sc, bi = mats[i % 4]
            w4.matmul(x, q, sc, bi)
    torch.cuda.synchronize()
    print("square: done", flush=True)
    del mats
    t = synthetic.MOE
    E, N, K, top_k = t["E"], t["N"], t["K"], t["top_k"]
    mats = dev(synthetic.quantized_weights(E * N, K, seed=0, tag=(E,)), 3, shape=((E, N, K // 8), (E, N, K // 64)))
    for M in t["M"]:
        ids = torch.from_numpy(synthetic.expert_ids(M, top_k, E, seed=0)).cuda()
        x = xs(M, K, (E,))
        for i in range(calls):
            q, sc, bi = mats[i % 3]
            w4.matmul_id(x, q, sc, bi, ids)
    torch.cuda.synchronize()
    print("routed: done", flush=True)
    del mats
    N, K = synthetic.PROJECTIONS["gate_up"]
    mats = dev(synthetic.quantized_weights(N, K, seed=0, tag=(N, 11)), 12)
    for M in (1, 5):
        x = xs(M, K, (N, 11))
        h = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
        for i in range(calls * 4):
            q, sc, bi = mats[i % len(mats)]
            w4.w4a16_matmul_geglu(x, q, sc, bi, h)
    torch.cuda.synchronize()
    print("geglu: done", flush=True)
    del mats
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("calibration copy: done", flush=True)


def prefill_workload(M: int = 4096) -> None:
    """Four eager prefill calls on each of the gate+up and down shapes at M rows."""
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import torch

    import decode_w4a16_affine_amd as w4
    import synthetic

    for name in ("gate_up", "down"):
        N, K = synthetic.PROJECTIONS[name]
        w = synthetic.quantized_weights(N, K, seed=0, tag=(N, 7))
        qw = torch.from_numpy(w.qw.view(np.int32)).cuda()
        s = torch.from_numpy(w.scales.view(np.int16)).view(torch.bfloat16).cuda()
        b = torch.from_numpy(w.biases.view(np.int16)).view(torch.bfloat16).cuda()
        x = torch.from_numpy(synthetic.activations(M, K, seed=0, tag=(N, 7)).view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(4):
            w4.w4a16_matmul_prefill(x, qw, s, b, y)
        torch.cuda.synchronize()
        print(f"prefill {name} M={M}: 4 calls", flush=True)


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "configs-workload":
        configs_workload()
    elif len(sys.argv) >= 2 and sys.argv[1] == "prefill-workload":
        prefill_workload(int(sys.argv[2]) if len(sys.argv) >= 3 else 4096)
    elif len(sys.argv) >= 2 and sys.argv[1] == "stats":
        summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 2 and sys.argv[1] == "trace":
        summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) >= 6 else "")
    elif len(sys.argv) >= 2 and sys.argv[1] == "sq":
        summarize_sq(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 2 and sys.argv[1] == "traffic":
        print(json.dumps(summarize_traffic(*sys.argv[2:7]), indent=1))
    elif len(sys.argv) >= 2 and sys.argv[1] == "traffic-md":
        traffic_markdown(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
