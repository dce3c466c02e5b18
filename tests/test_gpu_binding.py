"""The Python binding refuses malformed arguments before anything is
enqueued: the C entry points receive bare pointers, so a wrong-sized output,
index list or workspace has to be caught here. A workspace of any dtype is
sized in bytes."""
from __future__ import annotations

import pytest

import isa_inputs
from parity_util import bf16_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
isa = pytest.importorskip("block_sparse_attention_blockwise_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    isa.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def case(dev):
    p = isa.Params(1, 2, 300, 200, 64, 64)
    inp = isa_inputs.make_inputs(61, p.B, p.H, p.L_src, p.L_ctx, p.D)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    return p, Q, K, V


def test_forward_rejects_bad_out_and_workspace(dev, case):
    p, Q, K, V = case
    need = isa.plan(p)["workspace_bytes"]
    bad_out = [torch.empty(1, 2, 499, 64, dtype=torch.bfloat16, device=dev),
               torch.empty(1, 2, 500, 64, dtype=torch.float16, device=dev),
               torch.empty(1, 2, 64, 500, dtype=torch.bfloat16, device=dev).transpose(2, 3)]
    for o in bad_out:
        with pytest.raises(ValueError):
            isa.forward(Q, K, V, p, out=o)
    with pytest.raises(ValueError, match="bytes"):
        isa.forward(Q, K, V, p, workspace=torch.empty(need - 16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="shape"):
        isa.forward(Q, K[:, :, :-1].contiguous(), V, p)
    # a float32 workspace is measured in bytes and gives the same result
    ref = isa.forward(Q, K, V, p)
    ws32 = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    got = isa.forward(Q, K, V, p, workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_backward_rejects_bad_buffers(dev, case):
    p, Q, K, V = case
    ws = isa.workspace(p, dev)
    O = isa.forward(Q, K, V, p, workspace=ws)
    dO = torch.ones_like(O)
    with pytest.raises(ValueError, match="bytes"):
        isa.backward(Q, K, V, O, dO, p, ws[:-16])
    with pytest.raises(ValueError, match="triple"):
        isa.backward(Q, K, V, O, dO, p, ws, out=(torch.empty_like(Q),) * 2)
    with pytest.raises(ValueError, match="dK"):
        isa.backward(Q, K, V, O, dO, p, ws,
                     out=(torch.empty_like(Q), torch.empty_like(Q)[:, :1].contiguous(), torch.empty_like(Q)))
    with pytest.raises(ValueError, match="dO"):
        isa.backward(Q, K, V, O, dO.float(), p, ws)


def test_step_entry_points_reject_bad_index_lists(dev, case):
    p, Q, K, V = case
    qc, kc, kcb, vcb = isa.pool_coarse(Q, K, V, p)
    ctx, _ = isa.ctx_topk(qc, kc, p)
    _, si, fi, ei = isa.sharpness_split(qc, kc, ctx, p)
    with pytest.raises(ValueError, match="ctx_idx"):
        isa.sharpness_split(qc, kc, ctx.long(), p)
    with pytest.raises(ValueError, match="qc"):
        isa.ctx_topk(qc.float(), kc, p)
    with pytest.raises(ValueError, match="sharp_idx"):
        isa.sharp_attn(Q, K, V, ctx, si[..., :-1].contiguous(), p)
    with pytest.raises(ValueError, match="flat_exact_idx"):
        isa.flat_taylor_attn(Q, K, V, kcb, vcb, ctx, fi, ei[..., :-1].contiguous(), p)
    with pytest.raises(ValueError, match="vc_bf16"):
        isa.flat_taylor_attn(Q, K, V, kcb, vcb.float(), ctx, fi, ei, p)
    with pytest.raises(ValueError, match="O"):
        isa.coarse_residual(qc, kc, vcb, ctx, torch.empty(3, device=dev, dtype=torch.bfloat16), p)
    with pytest.raises(ValueError, match="out"):
        isa.dense_attn(Q, K, V, out=torch.empty_like(Q)[..., :32].contiguous())
