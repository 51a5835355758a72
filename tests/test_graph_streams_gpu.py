"""Replays of captured HIP graphs and concurrent streams give the eager results.

The benchmark measures every product through graph replays, and the C ABI is
stateless (all state lives in caller-owned buffers), so:
  * a graph holding the dense, grouped, LM-head (logits and argmax), routed,
    GeGLU and prefill calls reproduces the eager outputs bit for bit on every replay,
    with eager work (clearing the outputs) and synchronizations between the
    replays;
  * the same calls issued on two streams at once, each with its own outputs
    and workspace, give the single-stream results bit for bit.
All inputs are the seeded synthetic workloads at small sizes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_w4a16_affine_amd as w4
import synthetic
from parity import DevWeights, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


class Calls:
    """One of each product on its own seeded inputs; run() enqueues them all
    on the current stream, writing this instance's output buffers."""

    def __init__(self, seed: int):
        K = 2560
        self.dense = {}
        for i, (N, M) in enumerate(((2560, 1), (2560, 3), (20480, 5), (5000, 8))):
            w = synthetic.quantized_weights(N, K, seed=seed + i)
            x = dev_bf16(synthetic.activations(M, K, seed=seed + i))
            self.dense[(N, M)] = (DevWeights(w), x, torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
        self.grouped = []
        for i, N in enumerate((2560, 512, 512)):
            w = DevWeights(synthetic.quantized_weights(N, K, seed=seed + 10 + i))
            self.grouped.append((w, torch.empty((2, N), dtype=torch.float32, device="cuda")))
        self.gx = dev_bf16(synthetic.activations(2, K, seed=seed + 10))
        Nh = 70000
        self.head = DevWeights(synthetic.quantized_weights(Nh, K, seed=seed + 20, bias="exact"))
        self.hx = dev_bf16(synthetic.activations(3, K, seed=seed + 20))
        self.logits = torch.empty((3, Nh), dtype=torch.bfloat16, device="cuda")
        self.argmax = torch.empty((3,), dtype=torch.int32, device="cuda")
        self.ws = torch.empty((w4.w4a16_lmhead_argmax_workspace_bytes(3, Nh, K),), dtype=torch.uint8, device="cuda")
        E, Ne, Ke, top_k = 16, 1024, 2048, 4
        we = synthetic.quantized_weights(Ne, Ke, seed=seed + 30, lead=(E,))
        self.eq = torch.from_numpy(np.ascontiguousarray(we.qw).view(np.int32)).cuda()
        self.es = dev_bf16(we.scales)
        self.eb = dev_bf16(we.biases)
        self.ex = dev_bf16(synthetic.activations(4, Ke, seed=seed + 30))
        self.ids = dev_i32(synthetic.expert_ids(4, top_k, E, seed=seed + 30))
        self.ey = torch.empty((4, top_k, Ne), dtype=torch.bfloat16, device="cuda")
        wp = synthetic.quantized_weights(4096, K, seed=seed + 40)
        self.pw = DevWeights(wp)
        self.px = dev_bf16(synthetic.activations(300, K, seed=seed + 40))
        self.py = torch.empty((300, 4096), dtype=torch.bfloat16, device="cuda")
        wg = synthetic.quantized_weights(2 * 2200, K, seed=seed + 50)
        self.gw = DevWeights(wg)
        self.ggx = dev_bf16(synthetic.activations(5, K, seed=seed + 50))
        self.gh = torch.empty((5, 2200), dtype=torch.bfloat16, device="cuda")

    def outputs(self):
        return ([y for (_, _, y) in self.dense.values()] + [y for (_, y) in self.grouped]
                + [self.logits, self.argmax, self.ey, self.py, self.gh])

    def run(self, stream=None):
        for (w, x, y) in self.dense.values():
            w4.w4a16_matmul(x, w.qw, w.s, w.b, y, stream=stream)
        w4.w4a16_matmul_grouped(self.gx, [(w.qw, w.s, w.b, y) for (w, y) in self.grouped], stream=stream)
        w4.w4a16_lmhead_argmax(self.hx, self.head.qw, self.head.s, self.head.b, self.logits, self.argmax, self.ws,
                               stream=stream)
        w4.w4a16_matmul_id(self.ex, self.eq, self.es, self.eb, self.ids, self.ey, stream=stream)
        w4.w4a16_matmul_prefill(self.px, self.pw.qw, self.pw.s, self.pw.b, self.py, stream=stream)
        w4.w4a16_matmul_geglu(self.ggx, self.gw.qw, self.gw.s, self.gw.b, self.gh, stream=stream)

    def snapshot(self):
        torch.cuda.synchronize()
        return [t.detach().clone() for t in self.outputs()]


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                       b.view(torch.uint8) if b.dtype != torch.int32 else b)


def test_graph_replays_match_eager():
    c = Calls(seed=300)
    c.run()
    ref = c.snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in c.outputs():
            t.zero_()          # eager work between replays; the replay must rewrite everything
        torch.cuda.synchronize()
        g.replay()
        got = c.snapshot()
        say(f"graph replay {rep}")
        for i, (a, b) in enumerate(zip(got, ref)):
            assert same_bits(a, b), f"replay {rep}: output {i} differs from the eager result"
    del g


def test_two_streams_match_one():
    a, b = Calls(seed=400), Calls(seed=500)
    a.run()
    b.run()
    ref_a, ref_b = a.snapshot(), b.snapshot()
    for t in a.outputs() + b.outputs():
        t.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for rep in range(3):
        with torch.cuda.stream(s1):
            a.run()
        with torch.cuda.stream(s2):
            b.run()
        torch.cuda.synchronize()
        say(f"two streams, pass {rep}")
        for i, (x, y) in enumerate(zip(a.snapshot(), ref_a)):
            assert same_bits(x, y), f"stream 1 output {i}"
        for i, (x, y) in enumerate(zip(b.snapshot(), ref_b)):
            assert same_bits(x, y), f"stream 2 output {i}"
