"""isa_forward and isa_backward captured into one HIP graph (through
torch.cuda.CUDAGraph, i.e. hipStreamBeginCapture on the current stream).

The library enqueues only kernels on the caller's stream: no allocation,
no memset, no host synchronisation. So the pair can be captured once and
replayed on new contents of the same buffers. The kernels are deterministic,
so every replay must reproduce the eager calls on the same inputs bit for
bit. The replays alternate two input sets and run eager library calls in
between, and the outputs are filled with NaN bits before each replay, so a
replay that skipped a write or read stale state would show."""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import isa_inputs
from parity_util import bf16_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
isa = pytest.importorskip("block_sparse_attention_blockwise_amd")


def log(msg):
    print(f"[gpu-graph {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    isa.lib()
    return torch.device("cuda:0")


def _inputs(p, stream, dev):
    inp = isa_inputs.make_inputs(stream, p.B, p.H, p.L_src, p.L_ctx, p.D)
    rng = np.random.default_rng([7, stream])
    dO = isa_inputs.round_to_bf16(
        rng.standard_normal((p.B, p.H, p.L_src + p.L_ctx, p.D)).astype(np.float32))[0]
    return [bf16_tensor(inp[n][0], dev) for n in "QKV"] + [bf16_tensor(dO, dev)]


def _eager(p, Q, K, V, dO, dev):
    ws = isa.workspace(p, dev)
    O = isa.forward(Q, K, V, p, workspace=ws)
    return [O] + list(isa.backward(Q, K, V, O, dO, p, ws))


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("gamma,rope", [(0.0, 0.0), (0.5, 10000.0)])
def test_forward_backward_graph_replays_match_eager(dev, gamma, rope):
    # ragged segments (partial last blocks in both), D = 128, b = 64
    p = isa.Params(1, 4, 1000, 1100, 128, 64, 0.125, 0.5, 0.0625, gamma, rope)
    log(f"graph capture: H=4 L_src=1000 L_ctx=1100 D=128 b=64 gamma={gamma} rope={rope}")
    sets = [_inputs(p, 40 + k, dev) for k in range(2)]
    refs = [_eager(p, *s, dev) for s in sets]
    torch.cuda.synchronize()

    # static buffers the graph reads and writes
    Qs, Ks, Vs, dOs = (torch.empty_like(t) for t in sets[0])
    Os, dQs, dKs, dVs = (torch.empty_like(t) for t in sets[0])
    ws = isa.workspace(p, dev)

    def step():
        isa.forward(Qs, Ks, Vs, p, out=Os, workspace=ws)
        isa.backward(Qs, Ks, Vs, Os, dOs, p, ws, out=(dQs, dKs, dVs))

    for dst, src in zip((Qs, Ks, Vs, dOs), sets[0]):
        dst.copy_(src)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    nan_bits = torch.full_like(Os.view(torch.int16), -1)   # 0xffff: a bf16 NaN
    for r in range(4):
        k = r % 2
        for dst, src in zip((Qs, Ks, Vs, dOs), sets[k]):
            dst.copy_(src)
        for t in (Os, dQs, dKs, dVs):
            t.view(torch.int16).copy_(nan_bits)
        # eager library work between replays (its own workspace and outputs)
        other = _eager(p, *sets[1 - k], dev)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (Os, dQs, dKs, dVs)
        for name, g, ref in zip(("O", "dQ", "dK", "dV"), got, refs[k]):
            assert _same_bits(g, ref), f"replay {r}: {name} differs from the eager call"
        for name, g, ref in zip(("O", "dQ", "dK", "dV"), other, refs[1 - k]):
            assert _same_bits(g, ref), f"eager call between replays: {name} not reproducible"
        log(f"replay {r} (input set {k}): O, dQ, dK, dV identical to eager")
