"""The hot path under HIP graph capture (through the C ABI): block statistics,
routing, the fused forward and the backward, captured once into one graph and
replayed. None of the entry points allocates, clears memory with a memset or
synchronises with the host when the caller passes the outputs and the
workspaces, so the captured graph is the whole step. Every replay (with eager
work and host synchronisations between replays) must equal the eager result
bit for bit: the kernels are deterministic (fixed reduction orders, no
atomics on floating point), and a replay after the inputs are rewritten in
place must follow the new inputs."""

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from block_sparse_taylor_amd import inputs as I

from gpu_common import say, to_device

pytestmark = pytest.mark.gpu


class Step:
    """Static buffers of one step and the calls that fill them."""

    def __init__(self, q, k, v, do, topk, second_order):
        self.q, self.k, self.v, self.do = q, k, v, do
        self.topk, self.so = topk, second_order
        B, H, T, D = q.shape
        N = P.num_blocks(T)
        self.st = P.alloc_stats(k, second_order)
        self.ws = P.stats_workspace(k)
        self.idx = torch.empty(B, H, N, topk, dtype=torch.int32, device=q.device)
        self.wg = torch.empty(B, H, N, N, dtype=torch.float32, device=q.device) if second_order else None
        self.o = torch.empty_like(q)
        self.grads = tuple(torch.empty_like(q) for _ in range(3))
        self.bws = P.attn_bwd_workspace(q)

    def __call__(self):
        P.pisa_block_stats(self.q, self.k, self.v, second_order=self.so, out=self.st, workspace=self.ws)
        P.pisa_route_topk(self.q, self.st, self.topk, band=1, second_order=self.so, idx=self.idx, wgate=self.wg)
        P.pisa_attn_fwd(self.q, self.k, self.v, self.st, self.idx, self.wg, band=1, second_order=self.so,
                        out=self.o)
        P.pisa_attn_bwd(self.q, self.k, self.v, self.o, self.do, self.st, self.idx, self.wg, band=1,
                        second_order=self.so, workspace=self.bws, out=self.grads)

    def results(self):
        out = [self.idx, self.o, *self.grads]
        if self.wg is not None:
            out.append(self.wg)
        return [t.clone() for t in out]


def eager_busywork():
    a = torch.randn(2048, 2048, device="cuda")
    torch.cuda.synchronize()
    return float((a @ a).sum())


@pytest.mark.parametrize("name,heads,second_order", [("wan14", [0, 1, 2, 3], False), ("hunyuan", [0, 1], True)])
def test_step_replays_in_a_graph(name, heads, second_order):
    w = I.WORKLOADS[name]
    say(f"[gpu] graph capture {name} heads={heads} second_order={second_order}")
    arrs = I.make_inputs(w, heads=heads)
    q, k, v = (to_device(a, w.dtype) for a in arrs)
    r = np.random.default_rng(21)
    do = to_device(I.bf16_bits(r.standard_normal(arrs[0].shape).astype(np.float32)), "bf16")
    topk = P.topk_for_density(w.density, P.num_blocks(w.seq_len))

    eager = Step(q, k, v, do, topk, second_order)
    eager()
    torch.cuda.synchronize()
    want = eager.results()

    static = Step(q.clone(), k.clone(), v.clone(), do.clone(), topk, second_order)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        static()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static()
    torch.cuda.synchronize()

    for rep in range(3):
        eager_busywork()
        g.replay()
        torch.cuda.synchronize()
        got = static.results()
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep
        say(f"[gpu]   replay {rep}: equal to the eager step")

    # new inputs written in place: the replay follows them
    q2 = torch.flip(q, dims=[2]).contiguous()
    eager2 = Step(q2, k, v, do, topk, second_order)
    eager2()
    static.q.copy_(q2)
    torch.cuda.synchronize()
    eager_busywork()
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(static.results(), eager2.results()):
        assert torch.equal(a, b)
    say("[gpu]   replay on rewritten inputs: equal to the eager step")
