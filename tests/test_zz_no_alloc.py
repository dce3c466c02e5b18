"""GPU check of isa_forward_noalloc (the forward whose workspace is the
library's static device scratch) through the C ABI: its output must be
bit-identical to isa_forward's on the same inputs, on consecutive calls that
share the scratch (the second with a smaller input, so stale contents of the
first call would show), and requests beyond the scratch are refused."""
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
    print(f"[gpu-noalloc {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def _qkv(p, stream, dev):
    inp = isa_inputs.make_inputs(stream, p.B, p.H, p.L_src, p.L_ctx, p.D)
    return [bf16_tensor(inp[n][0], dev) for n in "QKV"]


def _same(a, b):
    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


def test_noalloc_forward_matches_forward():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    isa.init()
    cases = [
        # a large call first, then smaller ones that reuse the same scratch;
        # the first has N_kv = 656 > 640, so its exact sets go through the
        # exact-set selection's row scratch in the static array as well
        isa.Params(1, 1, 40960, 8192, 128, 64),
        isa.Params(1, 8, 8192, 8192, 128, 64),
        isa.Params(1, 2, 700, 451, 64, 32, 0.25, 0.5, 0.125, gamma=0.5),
        isa.Params(2, 3, 333, 290, 128, 64, 0.5, 0.25, 0.25, rope_base=10000.0),
    ]
    for k, p in enumerate(cases):
        pl = isa.plan(p)
        log(f"case {k}: {p} noalloc_bytes {pl['noalloc_bytes']}")
        assert pl["noalloc_bytes"] <= isa.NOALLOC_SCRATCH_BYTES
        Q, K, V = _qkv(p, 200 + k, dev)
        ref = isa.forward(Q, K, V, p)
        O = torch.full_like(Q, float("nan"))
        for rep in range(2):
            isa.forward_noalloc(Q, K, V, p, out=O)
            torch.cuda.synchronize()
            assert torch.isfinite(O.float()).all()
            assert _same(O, ref), f"case {k} call {rep}: output differs from isa_forward"
        log(f"  case {k}: bit-identical to isa_forward on two calls")


def test_noalloc_refuses_requests_beyond_the_scratch():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    p = isa.Params(1, 40, 32768, 32768, 128, 64)
    assert isa.plan(p)["noalloc_bytes"] > isa.NOALLOC_SCRATCH_BYTES
    L = 65536
    Q = torch.zeros(1, 40, L, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(isa.IsaError) as e:
        isa.forward_noalloc(Q, Q, Q, p)
    assert e.value.code == isa.ISA_ERR_SCRATCH
