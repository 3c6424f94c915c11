"""The allocation-free attention backward (mt_op_attn_bwd_noalloc, the
entry point for callers that cannot allocate device memory) against
mt_op_attn_bwd with a caller workspace: the same kernels on the same
inputs, so the same bits.  Two calls in a row, the second with a smaller
input (the static scratch still holds the first call's rows), then a
third at the first size again; sizes beyond the static scratch are
refused before anything is launched."""
import pytest

pytestmark = pytest.mark.gpu


def _env():
    import torch
    from layer_streamed_amd import mt
    assert torch.cuda.is_available()
    return torch, mt


def _case(B, T, Hq, Hkv, d, seed):
    torch, mt = _env()
    g = torch.Generator(device="cuda").manual_seed(seed)
    ld = (Hq + 2 * Hkv) * d
    QKV = torch.randn((B * T, ld), device="cuda", generator=g).to(torch.bfloat16)
    DO = torch.randn((B * T, Hq * d), device="cuda", generator=g).to(torch.bfloat16)
    O = torch.empty((B * T, Hq * d), device="cuda", dtype=torch.bfloat16)
    LSE = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    mt.attn_fwd(QKV, O, LSE, B, T, Hq, Hkv, d)
    delta = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    ref = torch.full((B * T, ld), float("nan"), device="cuda", dtype=torch.bfloat16)
    mt.attn_bwd(QKV, O, LSE, DO, delta, ref, B, T, Hq, Hkv, d)
    out = torch.full((B * T, ld), float("nan"), device="cuda", dtype=torch.bfloat16)
    mt.attn_bwd_noalloc(QKV, O, LSE, DO, out, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (B, T, Hq, Hkv, d)


def test_noalloc_attention_backward_equals_workspace_form():
    _case(2, 1024, 28, 4, 128, 1)   # the 7B heads
    _case(1, 300, 8, 2, 64, 2)      # smaller, ragged T, head_dim 64
    _case(3, 77, 10, 2, 128, 3)     # smaller still, group 5
    _case(2, 1024, 28, 4, 128, 4)   # the first size again, new inputs


def test_noalloc_refuses_sizes_beyond_the_static_scratch():
    torch, mt = _env()
    dummy = torch.zeros(64, device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(64, device="cuda", dtype=torch.float32)
    T = mt.ATTN_NOALLOC_MAX_ROWS // 32 + 1  # 32 heads x T rows: one row too many
    with pytest.raises(mt.MTError) as e:
        mt.attn_bwd_noalloc(dummy, dummy, lse, dummy, dummy, 1, T, 32, 8, 128)
    assert e.value.status == mt.MT_E_SHAPE
    with pytest.raises(mt.MTError) as e:
        mt.attn_bwd_noalloc(None, dummy, lse, dummy, dummy, 1, 8, 4, 2, 64)
    assert e.value.status == mt.MT_E_INVALID
    torch.cuda.synchronize()
