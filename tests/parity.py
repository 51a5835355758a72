"""Helpers for the GPU parity tests: device transfer and the acceptance checks.

Acceptance (element by element, against the CPU oracle):
  (i)   dequantized weights: bit-exact;
  (ii)  fp32 output: |y32 - y64| <= 1e-3 * sum_k |w x|;
  (iii) bf16 output: within 1 ulp of round-to-nearest-even(y64), for every
        element whose value is large enough that an fp32 sum can resolve it
        (|y64| >= (K/16 + 8) * 2^-16 * sum_k |w x|, the worst-case error of a
        chain of K/16 fp32 fmas plus an 8-level tree, set against half a bf16
        ulp); elements below that are judged by (ii) alone and counted;
  (iv)  argmax: equal wherever the oracle's top-2 gap exceeds the two bounds.
"""
from __future__ import annotations

import concurrent.futures as cf
import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_qw(qw: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(qw).view(np.int32)).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().astype(np.float32)


class DevWeights:
    def __init__(self, w):
        self.qw = dev_qw(w.qw)
        self.s = dev_bf16(w.scales)
        self.b = dev_bf16(w.biases)


def oracle_qmm(orc, x, w, rows=None, workers=8):
    """orc.qmm over row slices in threads (the C call releases the GIL)."""
    N = w.qw.shape[0]
    idx = np.arange(N, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
    parts = np.array_split(idx, min(workers, max(1, len(idx))))
    with cf.ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda r: orc.qmm(x, w.qw, w.scales, w.biases, group=w.group, rows=r), parts))
    y = np.concatenate([r[0] for r in res], axis=1)
    a = np.concatenate([r[1] for r in res], axis=1)
    return y, a


def check_f32(y32, y64, absy, what=""):
    y32 = np.asarray(y32, dtype=np.float64)
    err = np.abs(y32 - y64)
    bad = ~(err <= 1e-3 * absy)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} fp32 outputs outside 1e-3*sum|wx|; first {tuple(i)}: "
                             f"gpu {y32[tuple(i)]!r} oracle {y64[tuple(i)]!r} bound {1e-3 * absy[tuple(i)]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(absy > 0, err / absy, 0.0)
    return float(r.max()) if r.size else 0.0


def ordered(bits):
    b = np.asarray(bits).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits, b_bits):
    return np.abs(ordered(a_bits) - ordered(b_bits))


def check_bf16(orc, ybits, y64, absy, K, what=""):
    ref = orc.f64_to_bf16(y64)
    d = ulp_distance(ybits, ref)
    exempt = np.abs(y64) < (K / 16 + 8) * 2.0 ** -16 * absy
    bad = (d > 1) & ~exempt
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} bf16 outputs beyond 1 ulp; first {tuple(i)}: gpu "
                             f"{int(np.asarray(ybits)[tuple(i)]):#06x} oracle {int(ref[tuple(i)]):#06x}")
    return int(exempt.sum())


def check_argmax(orc, am, y64, absy, what=""):
    """(iv): compare where the oracle's top-2 gap exceeds the bounds of both."""
    checked = 0
    for m in range(y64.shape[0]):
        best, gap = orc.argmax(y64[m])
        order = np.argsort(-y64[m], kind="stable")
        second = order[1] if order[0] == best else order[0]
        if gap > 1e-3 * (absy[m, best] + absy[m, second]):
            assert int(am[m]) == best, f"{what}: row {m}: gpu argmax {int(am[m])} oracle {best} gap {gap}"
            checked += 1
    return checked
