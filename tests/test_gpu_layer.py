"""Layer-template parity on the GPU: mt_layer_fwd and mt_layer_recompute_bwd
against the oracle's layer_forward / layer_backward on the same seeded
weights and inputs (bf16 on the GPU, fp32 in the oracle)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import decoder as D

pytestmark = pytest.mark.gpu

TOL = 2e-2  # relative Frobenius, bf16 storage with fp32 accumulation


def _env():
    import torch
    from layer_streamed_amd import mt
    assert torch.cuda.is_available()
    return torch, mt


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-30))


def _layer_case(shape, B, T, seed, mlp_chunk=0, x_scale=1.0, fp32=False):
    """fp32=True runs the fp32 debug precision: the GPU holds the fp32
    values unrounded and the oracle runs in float64."""
    torch, mt = _env()
    rnd = (lambda a: a.astype(np.float64)) if fp32 else oracle.bf16_round
    names = synth.layer_param_names(0)
    w = synth.make_weights(shape, seed=seed, names=names)
    w = {n.split(".")[-1]: v for n, v in w.items()}
    rng = np.random.default_rng(seed + 1)
    # gains away from 1 so their gradients are exercised
    w["attn_norm"] = (1 + 0.1 * rng.standard_normal(shape.hidden)).astype(np.float32)
    w["mlp_norm"] = (1 + 0.1 * rng.standard_normal(shape.hidden)).astype(np.float32)
    wb = {k: rnd(v) for k, v in w.items()}  # the values the GPU holds
    x = rnd((rng.standard_normal((B, T, shape.hidden)) * x_scale).astype(np.float32))
    dy = rnd((rng.standard_normal((B, T, shape.hidden)) * 1e-2).astype(np.float32))

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        return t if fp32 else t.to(torch.bfloat16)

    W = {
        "attn_norm": dev(wb["attn_norm"]),
        "w_qkv": dev(np.concatenate([wb["w_q"], wb["w_k"], wb["w_v"]])),
        "w_o": dev(wb["w_o"]),
        "mlp_norm": dev(wb["mlp_norm"]),
        "w_gate_up": dev(np.concatenate([wb["w_gate"], wb["w_up"]])),
        "w_down": dev(wb["w_down"]),
    }
    view = mt.LayerView(*[W[k].data_ptr() for k, _ in mt.LayerView._fields_])
    G = {k: torch.full_like(v, float("nan")) for k, v in W.items()}
    gview = mt.GradView(*[G[k].data_ptr() for k, _ in mt.GradView._fields_])
    mcfg = mt.model_cfg(shape)
    rcfg = mt.run_cfg(mlp_chunk_tokens=mlp_chunk,
                      precision=mt.PREC_FP32_DEBUG if fp32 else mt.PREC_BF16)
    X = dev(x.reshape(B * T, -1))
    Y = torch.empty_like(X)
    ws = torch.empty(mt.layer_workspace_bytes(mcfg, rcfg, B, T, 1), dtype=torch.uint8, device="cuda")
    mt.layer_fwd(mcfg, rcfg, view, X, Y, B, T, ws)
    DX = dev(dy.reshape(B * T, -1))  # dy in, dx out (aliasing allowed)
    mt.layer_recompute_bwd(mcfg, rcfg, view, X, DX, DX, gview, B, T, ws)
    torch.cuda.synchronize()
    cos, sin = D.rope_cos_sin(T, shape.head_dim, shape.rope_theta, np.float32)
    y_ref, saved = D.layer_forward(wb, x, shape, cos, sin)
    dx_ref, g_ref = D.layer_backward(wb, saved, dy, shape, cos, sin)
    out = {
        "y": (Y.float().cpu().numpy(), y_ref.reshape(B * T, -1)),
        "dx": (DX.float().cpu().numpy(), dx_ref.reshape(B * T, -1)),
        "attn_norm": (G["attn_norm"].float().cpu().numpy(), g_ref["attn_norm"]),
        "w_qkv": (G["w_qkv"].float().cpu().numpy(),
                  np.concatenate([g_ref["w_q"], g_ref["w_k"], g_ref["w_v"]])),
        "w_o": (G["w_o"].float().cpu().numpy(), g_ref["w_o"]),
        "mlp_norm": (G["mlp_norm"].float().cpu().numpy(), g_ref["mlp_norm"]),
        "w_gate_up": (G["w_gate_up"].float().cpu().numpy(),
                      np.concatenate([g_ref["w_gate"], g_ref["w_up"]])),
        "w_down": (G["w_down"].float().cpu().numpy(), g_ref["w_down"]),
    }
    return out


CASES = [
    ("tiny", synth.CONFIGS["tiny-2l-h256"], 2, 128, 0),
    ("tiny-ragged-T", synth.CONFIGS["tiny-2l-h256"], 3, 77, 0),
    ("tiny-chunked-mlp", synth.CONFIGS["tiny-2l-h256"], 2, 100, 64),
    ("gqa5-d128", synth.ModelShape(name="gqa5", n_layers=1, hidden=640, n_heads=10,
                                   n_kv_heads=2, head_dim=128, ffn=1536, vocab=1024), 2, 192, 0),
]


@pytest.mark.parametrize("name,shape,B,T,chunk", CASES, ids=[c[0] for c in CASES])
def test_layer_forward_and_recompute_backward(name, shape, B, T, chunk):
    out = _layer_case(shape, B, T, seed=11, mlp_chunk=chunk)
    for k, (gpu, ref) in out.items():
        assert np.isfinite(gpu).all(), k
        assert rel(gpu, ref) < TOL, (k, rel(gpu, ref))


def test_layer_7b_shape_one_sequence():
    """One Qwen2.5-7B-shaped layer (H 3584, 28/4 heads, F 18944) on one
    sequence of 256 tokens against the oracle."""
    shape = synth.CONFIGS["qwen2.5-7b-b16-t1024"]
    out = _layer_case(shape, 1, 256, seed=3)
    for k, (gpu, ref) in out.items():
        assert rel(gpu, ref) < TOL, (k, rel(gpu, ref))


@pytest.mark.parametrize("cfg", ["qwen2.5-14b-b8-t2048", "width2x-8l-b8-t1024",
                                 "qwen2.5-72b-l4-b8-t1024", "width3.5x-2l-b8-t1024"],
                         ids=["14b-h5120-gqa5", "width2x-h7168-gqa7", "72b-h8192-gqa8",
                              "width3.5x-h12544-gqa7"])
def test_layer_wide_shapes_one_sequence(cfg):
    """One layer at the other workloads' widths against the oracle: the
    14B shape (H 5120, 40/8 heads, F 13824), the 2.0x width point (H 7168,
    56/8 heads, F 37888), the 72B shape (H 8192, 64/8 heads, F 29568) and
    the widest point of the width study (H 12544, 98/14 heads, F 66304,
    whose RMSNorm backward takes the wide-row kernel), on one sequence of
    384 tokens."""
    shape = synth.CONFIGS[cfg]
    out = _layer_case(shape, 1, 384, seed=5)
    for k, (gpu, ref) in out.items():
        assert np.isfinite(gpu).all(), k
        assert rel(gpu, ref) < TOL, (k, rel(gpu, ref))


def test_layer_7b_full_batch_one_sequence_checked():
    """One Qwen2.5-7B-shaped layer at the benchmark's launch configuration
    (B 16 x T 1024: the 256 x 256 GEMM tiles with split tail tiles, the
    full attention grids) through the calls the engine makes for it
    (mt_layer_fwd_keep, then mt_layer_bwd_saved).  The upstream gradient is
    zero outside one sequence, so that sequence's output and input
    gradient and every weight gradient (a sum over all tokens) are what the
    oracle computes for that sequence alone, and the other sequences' input
    gradients are exactly zero."""
    torch, mt = _env()
    shape = synth.CONFIGS["qwen2.5-7b-b16-t1024"]
    B, T, H, bc = 16, 1024, shape.hidden, 5
    names = synth.layer_param_names(0)
    w = {n.split(".")[-1]: v for n, v in synth.make_weights(shape, seed=31, names=names).items()}
    rng = np.random.default_rng(32)
    w["attn_norm"] = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    w["mlp_norm"] = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    wb = {k: oracle.bf16_round(v) for k, v in w.items()}
    x = oracle.bf16_round(rng.standard_normal((B, T, H)).astype(np.float32))
    dy = np.zeros((B, T, H), np.float32)
    dy[bc] = oracle.bf16_round((rng.standard_normal((T, H)) * 1e-2).astype(np.float32))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(torch.bfloat16)

    W = {"attn_norm": dev(wb["attn_norm"]),
         "w_qkv": dev(np.concatenate([wb["w_q"], wb["w_k"], wb["w_v"]])), "w_o": dev(wb["w_o"]),
         "mlp_norm": dev(wb["mlp_norm"]),
         "w_gate_up": dev(np.concatenate([wb["w_gate"], wb["w_up"]])), "w_down": dev(wb["w_down"])}
    view = mt.LayerView(*[W[k].data_ptr() for k, _ in mt.LayerView._fields_])
    G = {k: torch.full_like(v, float("nan")) for k, v in W.items()}
    gview = mt.GradView(*[G[k].data_ptr() for k, _ in mt.GradView._fields_])
    mcfg, rcfg = mt.model_cfg(shape), mt.run_cfg()
    X = dev(x.reshape(B * T, H))
    Y = torch.empty_like(X)
    DX = dev(dy.reshape(B * T, H))
    internals = torch.empty(mt.layer_internals_bytes(mcfg, rcfg, B, T), dtype=torch.uint8,
                            device="cuda")
    ws = torch.empty(mt.layer_workspace_bytes(mcfg, rcfg, B, T, 2), dtype=torch.uint8,
                     device="cuda")
    mt.layer_fwd_keep(mcfg, rcfg, view, X, Y, B, T, internals)
    mt.layer_bwd_saved(mcfg, rcfg, view, X, DX, DX, gview, B, T, internals, ws)
    torch.cuda.synchronize()
    cos, sin = D.rope_cos_sin(T, shape.head_dim, shape.rope_theta, np.float32)
    y_ref, saved = D.layer_forward(wb, x[bc:bc + 1], shape, cos, sin)
    dx_ref, g_ref = D.layer_backward(wb, saved, dy[bc:bc + 1], shape, cos, sin)
    rows = slice(bc * T, (bc + 1) * T)
    dxg = DX.float().cpu().numpy()
    checks = {
        "y": (Y[rows].float().cpu().numpy(), y_ref.reshape(T, H)),
        "dx": (dxg[rows], dx_ref.reshape(T, H)),
        "attn_norm": (G["attn_norm"].float().cpu().numpy(), g_ref["attn_norm"]),
        "w_qkv": (G["w_qkv"].float().cpu().numpy(),
                  np.concatenate([g_ref["w_q"], g_ref["w_k"], g_ref["w_v"]])),
        "w_o": (G["w_o"].float().cpu().numpy(), g_ref["w_o"]),
        "mlp_norm": (G["mlp_norm"].float().cpu().numpy(), g_ref["mlp_norm"]),
        "w_gate_up": (G["w_gate_up"].float().cpu().numpy(),
                      np.concatenate([g_ref["w_gate"], g_ref["w_up"]])),
        "w_down": (G["w_down"].float().cpu().numpy(), g_ref["w_down"]),
    }
    for k, (gpu, ref) in checks.items():
        assert np.isfinite(gpu).all(), k
        assert rel(gpu, ref) < TOL, (k, rel(gpu, ref))
    other = np.delete(dxg.reshape(B, T, H), bc, axis=0)
    assert not other.any(), "input gradient of a sequence with zero upstream gradient"
    assert np.isfinite(Y.float().cpu().numpy()).all()


# fp32 debug precision: every buffer fp32, fp32 FMA kernels; the oracle in
# float64.  The bar is 1e-4 relative (the fp32 error of the longest
# reductions here is ~1e-6).
F32_TOL = 1e-4

F32_CASES = [
    ("tiny", synth.CONFIGS["tiny-2l-h256"], 2, 128, 0),
    ("tiny-ragged-chunked", synth.CONFIGS["tiny-2l-h256"], 3, 45, 64),
    ("gqa5-d128", synth.ModelShape(name="gqa5", n_layers=1, hidden=640, n_heads=10,
                                   n_kv_heads=2, head_dim=128, ffn=1536, vocab=1024), 1, 96, 0),
]


@pytest.mark.parametrize("name,shape,B,T,chunk", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_layer_fp32_debug_precision(name, shape, B, T, chunk):
    out = _layer_case(shape, B, T, seed=12, mlp_chunk=chunk, fp32=True)
    for k, (gpu, ref) in out.items():
        assert np.isfinite(gpu).all(), k
        assert rel(gpu, ref) < F32_TOL, (k, rel(gpu, ref))


@pytest.mark.parametrize("chunk", [0, 64], ids=["whole-mlp", "chunked-mlp"])
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_kept_internals_backward_is_bitwise_the_recompute(fp32, chunk):
    """mt_layer_fwd_keep + mt_layer_bwd_saved (no recompute of the attention
    half; with a chunked MLP each chunk's gate/up is recomputed from the kept
    normed input) against mt_layer_fwd + mt_layer_recompute_bwd on the same
    weights and input: same kernels on the same inputs, so every output is
    bitwise equal."""
    torch, mt = _env()
    shape = synth.ModelShape(name="gqa5", n_layers=1, hidden=640, n_heads=10, n_kv_heads=2,
                             head_dim=128, ffn=1536, vocab=1024)
    B, T = 2, 96
    names = synth.layer_param_names(0)
    w = {n.split(".")[-1]: v for n, v in synth.make_weights(shape, seed=21, names=names).items()}
    rng = np.random.default_rng(22)
    dt = torch.float32 if fp32 else torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)

    W = {"attn_norm": dev(1 + 0.1 * rng.standard_normal(shape.hidden)),
         "w_qkv": dev(np.concatenate([w["w_q"], w["w_k"], w["w_v"]])), "w_o": dev(w["w_o"]),
         "mlp_norm": dev(1 + 0.1 * rng.standard_normal(shape.hidden)),
         "w_gate_up": dev(np.concatenate([w["w_gate"], w["w_up"]])), "w_down": dev(w["w_down"])}
    view = mt.LayerView(*[W[k].data_ptr() for k, _ in mt.LayerView._fields_])
    mcfg = mt.model_cfg(shape)
    rcfg = mt.run_cfg(precision=mt.PREC_FP32_DEBUG if fp32 else mt.PREC_BF16,
                      mlp_chunk_tokens=chunk)
    X = dev(rng.standard_normal((B * T, shape.hidden)))
    DY = dev(rng.standard_normal((B * T, shape.hidden)) * 1e-2)
    outs = []
    for keep in (False, True):
        G = {k: torch.full_like(v, float("nan")) for k, v in W.items()}
        gview = mt.GradView(*[G[k].data_ptr() for k, _ in mt.GradView._fields_])
        Y = torch.empty_like(X)
        DX = DY.clone()
        if keep:
            nb = mt.layer_internals_bytes(mcfg, rcfg, B, T)
            assert nb > 0
            internals = torch.empty(nb, dtype=torch.uint8, device="cuda")
            ws = torch.empty(mt.layer_workspace_bytes(mcfg, rcfg, B, T, 2), dtype=torch.uint8,
                             device="cuda")
            assert ws.numel() < mt.layer_workspace_bytes(mcfg, rcfg, B, T, 1)
            mt.layer_fwd_keep(mcfg, rcfg, view, X, Y, B, T, internals)
            mt.layer_bwd_saved(mcfg, rcfg, view, X, DX, DX, gview, B, T, internals, ws)
        else:
            ws = torch.empty(mt.layer_workspace_bytes(mcfg, rcfg, B, T, 1), dtype=torch.uint8,
                             device="cuda")
            mt.layer_fwd(mcfg, rcfg, view, X, Y, B, T, ws)
            mt.layer_recompute_bwd(mcfg, rcfg, view, X, DX, DX, gview, B, T, ws)
        torch.cuda.synchronize()
        outs.append({"y": Y.clone(), "dx": DX.clone(), **{k: v.clone() for k, v in G.items()}})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k
        assert torch.isfinite(outs[1][k].float()).all(), k
    # a chunked MLP keeps no gate/up: less to keep than a whole one
    whole = mt.layer_internals_bytes(mcfg, mt.run_cfg(), B, T)
    assert 0 < mt.layer_internals_bytes(mcfg, mt.run_cfg(mlp_chunk_tokens=64), B, T) < whole
