"""Host-side pieces of libmt that run without a GPU: the library loads and
exports every entry point its headers declare, the CPU Adam matches the
oracle's Adam bit for bit, and argument validation rejects bad calls
without touching state."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import decoder as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mt():
    from layer_streamed_amd import mt
    return mt


def _declared():
    names = set()
    for h in ("mt.h", "mt_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(mt_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    mt = _mt()
    lib = C.CDLL(mt.LIB_PATH)
    missing = [n for n in sorted(_declared()) if not hasattr(lib, n)]
    assert not missing, missing
    assert _declared() <= set(mt.EXPORTED)


def _adam(p, m, v, g, step, dtype, shadow=True, shadow_offset=0, **hp):
    mt = _mt()
    cfg = mt.run_cfg(**hp)
    # shadow_offset shifts the bf16 copy off 16-byte alignment (the
    # vectorized path streams 16-byte stores after a scalar prologue)
    sh = np.zeros(p.size + shadow_offset, np.uint16)[shadow_offset:] if shadow else None
    gbuf = D.bf16_bits(g) if dtype == mt.DT_BF16 else np.ascontiguousarray(g, np.float32)
    st = mt.call("mt_host_adam", mt.ptr(p), mt.ptr(m), mt.ptr(v), mt.ptr(gbuf), dtype,
                 mt.ptr(sh), p.size, step, C.byref(cfg))
    return st, sh


@pytest.mark.parametrize("dtype", [0, 1], ids=["bf16_grad", "f32_grad"])
@pytest.mark.parametrize("threads", [1, 7])
@pytest.mark.parametrize("offset", [0, 3])
def test_host_adam_bitwise_equals_oracle(dtype, threads, offset):
    rng = np.random.default_rng(1 + dtype)
    n = 100_003
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g[:50] = 0
    if dtype == 0:
        g = D.bf16_round(g)
    for step in (1, 3):
        rp, rm, rv = D.adam_update(p.copy(), m.copy(), v.copy(), g, step, 1e-4, 0.9, 0.999, 1e-8)
        pp, mm, vv = p.copy(), m.copy(), v.copy()
        st, sh = _adam(pp, mm, vv, g, step, dtype, shadow_offset=offset, host_threads=threads)
        assert st == 0
        np.testing.assert_array_equal(mm, rm)
        np.testing.assert_array_equal(vv, rv)
        np.testing.assert_array_equal(pp, rp)
        np.testing.assert_array_equal(sh, D.bf16_bits(rp))


def test_host_adam_refuses_nonfinite_and_leaves_state():
    mt = _mt()
    n = 9000
    p = np.ones(n, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    g = np.full(n, 0.5, np.float32)
    g[4321] = np.nan
    st, sh = _adam(p, m, v, g, 1, mt.DT_F32, check_finite=1)
    assert st == mt.MT_E_NONFINITE
    assert "NaN" in mt.last_error()
    assert (p == 1).all() and not m.any() and not v.any() and not sh.any()


def test_host_adam_validates_arguments():
    mt = _mt()
    p = np.ones(8, np.float32)
    m = np.zeros(8, np.float32)
    v = np.zeros(8, np.float32)
    g = np.ones(8, np.float32)
    st, _ = _adam(p, m, v, g, 0, mt.DT_F32)
    assert st == mt.MT_E_INVALID
    st, _ = _adam(p, m, v, g, 1, 7)
    assert st == mt.MT_E_INVALID
    cfg = mt.run_cfg()
    assert mt.call("mt_host_adam", None, None, None, None, 1, None, 8, 1, C.byref(cfg)) == mt.MT_E_INVALID
    assert (p == 1).all()


def test_run_cfg_defaults():
    r = _mt().run_cfg()
    assert r.ckpt_interval == 4 and r.prefetch_depth == 2 and r.use_slab_pool == 1
    assert r.lr == 1e-4 and r.beta1 == 0.9 and r.beta2 == 0.999 and r.eps == 1e-8


@pytest.mark.parametrize("prec", [0, 1], ids=["bf16", "fp32_debug"])
def test_host_store_roundtrip_and_streamed_copy(prec):
    """A model in pageable host memory (no GPU): parameters round-trip, and
    the streamed copy is the bf16 rounding of the master (bf16 precision)
    or the master itself (fp32 debug precision)."""
    import synth
    mt = _mt()
    s = synth.CONFIGS["tiny-2l-h256"]
    m = mt.Model(s, host_alloc=mt.HOST_PAGEABLE, precision=prec)
    w = synth.make_weights(s, seed=9)
    m.set_params(w)
    for n in ("embed", "layers.1.w_k", "lm_head", "final_norm"):
        np.testing.assert_array_equal(m.get(n), w[n])
        sh = m.get(n, mt.GET_SHADOW)
        np.testing.assert_array_equal(sh, D.bf16_round(w[n]) if prec == 0 else w[n])
    m.close()


def test_workspace_grows_with_fp32_and_rejects_unknown_precision():
    import synth
    mt = _mt()
    s = synth.CONFIGS["tiny-2l-h256"]
    mc = mt.model_cfg(s)
    b = mt.layer_workspace_bytes(mc, mt.run_cfg(precision=0), 2, 128, 1)
    f = mt.layer_workspace_bytes(mc, mt.run_cfg(precision=1), 2, 128, 1)
    assert 0 < b < f
    assert mt.layer_workspace_bytes(mc, mt.run_cfg(precision=2), 2, 128, 1) == 0


def test_arena_query_without_model_matches_model_and_depth_study():
    """The model-free arena query equals the model's own (pageable host
    store, no GPU), for several schedules; over the depth study's layer
    counts (listing page, Table 5) the arena grows only by the checkpoint
    slots (one activation per K layers), not by any per-layer weight or
    gradient storage."""
    import synth
    mt = _mt()
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=5, ckpt_interval=2)
    for kw in (dict(), dict(keep_internals=0), dict(resident_layers=2), dict(prefetch_depth=3),
               dict(precision=1), dict(mlp_chunk_tokens=64, head_chunk_tokens=100)):
        m = mt.Model(s, host_alloc=mt.HOST_PAGEABLE, **kw)
        assert m.arena_bytes(2, 128) == mt.arena_bytes_for(s, 2, 128, **kw) > 0, kw
        m.close()
    q7 = synth.CONFIGS["qwen2.5-7b-b16-t1024"]
    act = q7.tokens * q7.hidden * 2
    base = mt.arena_bytes_for(q7)
    for L in (42, 56, 84, 132, 180):
        got = mt.arena_bytes_for(q7.with_(n_layers=L))
        slots = (L // q7.ckpt_interval) - (q7.n_layers // q7.ckpt_interval)
        assert got - base == slots * act, (L, got - base, slots * act)
    assert mt.arena_bytes_for(q7, prefetch_depth=4) == 0


def test_set_schedule_validates_and_keeps_fixed_knobs():
    import synth
    mt = _mt()
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=5, ckpt_interval=2)
    m = mt.Model(s, host_alloc=mt.HOST_PAGEABLE)
    a0 = m.arena_bytes(2, 128)
    m.set_schedule(keep_internals=0, ckpt_interval=1, resident_layers=2, prefetch_depth=3)
    assert m.arena_bytes(2, 128) == mt.arena_bytes_for(
        s, 2, 128, keep_internals=0, ckpt_interval=1, resident_layers=2, prefetch_depth=3) != a0
    for bad in (dict(precision=1), dict(host_threads=3), dict(prefetch_depth=0),
                dict(resident_layers=6), dict(n_slabs=3)):
        with pytest.raises(mt.MTError) as e:
            m.set_schedule(**bad)
        assert e.value.status == mt.MT_E_INVALID, bad
    m.set_schedule(use_slab_pool=0)
    m.set_schedule(use_slab_pool=1)  # the pool allocated at creation
    m.close()
    m = mt.Model(s, host_alloc=mt.HOST_PAGEABLE, use_slab_pool=0)
    with pytest.raises(mt.MTError):
        m.set_schedule(use_slab_pool=1)
    m.close()


def test_opt_8bit_host_store_and_validation():
    """A pageable model with 8-bit states: parameters round-trip, the moments
    read back as zero after a set, the knob is fixed at creation, and
    clipping refuses a slab pool too small to hold every gradient."""
    import synth
    mt = _mt()
    s = synth.CONFIGS["tiny-2l-h256"]
    m = mt.Model(s, host_alloc=mt.HOST_PAGEABLE, opt_8bit=1)
    w = synth.make_weights(s, seed=9)
    m.set_params(w)
    for n in ("embed", "layers.1.w_k", "lm_head", "final_norm"):
        np.testing.assert_array_equal(m.get(n), w[n])
        assert not m.get(n, mt.GET_M).any() and not m.get(n, mt.GET_V).any()
    with pytest.raises(mt.MTError):
        m.set_schedule(opt_8bit=0)
    m.set_schedule(clip_norm=1.0)  # 8 slabs >= 2 layers + head
    m.close()
    with pytest.raises(mt.MTError) as e:
        mt.Model(s.with_(n_layers=9), host_alloc=mt.HOST_PAGEABLE, clip_norm=1.0)
    assert e.value.status == mt.MT_E_INVALID
    mt.Model(s.with_(n_layers=9), host_alloc=mt.HOST_PAGEABLE, clip_norm=1.0, n_slabs=10).close()
    with pytest.raises(mt.MTError):  # hidden not a multiple of 128
        mt.Model(s.with_(hidden=192, n_heads=3, n_kv_heads=1), host_alloc=mt.HOST_PAGEABLE,
                 opt_8bit=1)
