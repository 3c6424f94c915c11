"""The whole streamed training step on the GPU (mt_stream_step) against the
oracle's train_step, and the schedule invariances the method implies: the
result does not depend on how work is spread over streams, on the
checkpoint interval, on the prefetch depth or on the slab pool."""
import numpy as np
import pytest

import synth
from oracle import decoder as D

pytestmark = pytest.mark.gpu

LOSS_TOL = 1e-2
REL_TOL = 2e-2


def _env():
    import torch
    from layer_streamed_amd import mt
    assert torch.cuda.is_available()
    return torch, mt


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-30))


def _run(shape, weights, ids, steps=1, **run_kw):
    torch, mt = _env()
    m = mt.Model(shape, keep_grads=1, **run_kw)
    m.set_params(weights)
    B, T = ids.shape
    arena = torch.empty(m.arena_bytes(B, T), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    losses, stats = [], None
    for _ in range(steps):
        loss, stats = m.step(ids, arena, streams)
        losses.append(loss)
    names = synth.param_names(shape)
    out = {
        "loss": losses,
        "grad": {n: m.get(n, mt.GET_GRAD) for n in names},
        "master": {n: m.get(n, mt.GET_MASTER) for n in names},
        "shadow": {n: m.get(n, mt.GET_SHADOW) for n in names},
        "m": {n: m.get(n, mt.GET_M) for n in names},
        "stats": stats,
        "steps": m.step_count,
    }
    m.close()
    return out


@pytest.fixture(scope="module")
def tiny():
    s = synth.CONFIGS["tiny-2l-h256"]
    return s, synth.make_weights(s), synth.make_tokens(s)


def test_step_matches_oracle(tiny):
    s, w, ids = tiny
    g = _run(s, w, ids)
    loss, grads, newp, state = D.train_step(w, ids, s)
    assert abs(g["loss"][0] - loss) < LOSS_TOL, (g["loss"][0], loss)
    for n in synth.param_names(s):
        assert rel(g["grad"][n], grads[n]) < REL_TOL, (n, rel(g["grad"][n], grads[n]))
        assert rel(g["master"][n], newp[n]) < REL_TOL, n
        # first moment after one step is (1 - beta1) g: a second check on g
        assert rel(g["m"][n], state[n][0]) < REL_TOL, n
    # the streamed copy is the RNE bf16 of the updated master
    for n in synth.param_names(s):
        np.testing.assert_array_equal(g["shadow"][n], D.bf16_round(g["master"][n]))
    assert g["steps"] == 1
    st = g["stats"]
    assert st["units_updated"] == s.n_layers + 2
    assert st["h2d_bytes"] > 0 and st["d2h_bytes"] > 0


def test_two_steps_match_oracle(tiny):
    s, w, ids = tiny
    g = _run(s, w, ids, steps=2)
    loss1, _, p1, st1 = D.train_step(w, ids, s)
    loss2, grads2, p2, _ = D.train_step(p1, ids, s, state=st1, step=2)
    assert abs(g["loss"][0] - loss1) < LOSS_TOL
    assert abs(g["loss"][1] - loss2) < LOSS_TOL
    for n in synth.param_names(s):
        assert rel(g["grad"][n], grads2[n]) < REL_TOL, n
        assert rel(g["master"][n], p2[n]) < REL_TOL, n


@pytest.mark.parametrize("defer", [1, 0], ids=["deferred", "in-step"])
def test_two_steps_different_batches_match_oracle(tiny, defer):
    """Step 2 runs a different batch whose tokens overlap step 1's only in
    part: the embedding rows of step 2's batch get their deferred step-1
    update before the gather, rows only step 1 touched get Adam with a zero
    gradient in step 2 (their moments still move them), and the loss of
    step 2 is that of a new batch.  Against two oracle train_step calls,
    with the deferred head / embedding updates on and off."""
    torch, mt = _env()
    s, w, ids1 = tiny
    ids2 = synth.make_tokens(s, seed=77)
    r1, r2 = set(ids1.ravel().tolist()), set(ids2.ravel().tolist())
    only1 = np.array(sorted(r1 - r2))
    assert r1 & r2 and len(only1) > 0 and r2 - r1
    m = mt.Model(s, keep_grads=1, defer_updates=defer)
    m.set_params(w)
    B, T = ids1.shape
    arena = torch.empty(m.arena_bytes(B, T), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    l1, _ = m.step(ids1, arena, streams)
    l2, _ = m.step(ids2, arena, streams)
    names = synth.param_names(s)
    grad = {n: m.get(n, mt.GET_GRAD) for n in names}
    master = {n: m.get(n, mt.GET_MASTER) for n in names}
    m.close()
    ref1, g1, p1, st1 = D.train_step(w, ids1, s)
    ref2, g2, p2, _ = D.train_step(p1, ids2, s, state=st1, step=2)
    assert abs(l1 - ref1) < LOSS_TOL and abs(l2 - ref2) < LOSS_TOL, (l1, ref1, l2, ref2)
    for n in names:
        assert rel(grad[n], g2[n]) < REL_TOL, (n, rel(grad[n], g2[n]))
        assert rel(master[n], p2[n]) < REL_TOL, (n, rel(master[n], p2[n]))
    # rows touched only in step 1: no gradient in step 2, moved by Adam
    # anyway.  Adam's first steps move a weight by about lr * sign(g), so
    # compare the movement where step 1's gradient is clearly away from 0
    # (bf16 rounding may flip the sign of a gradient element near zero).
    assert not grad["embed"][only1].any()
    gr = g1["embed"][only1]
    sure = np.abs(gr) > 0.1 * np.sqrt(np.mean(gr * gr))
    moved = (master["embed"] - w["embed"])[only1][sure]
    assert rel(moved, (p2["embed"] - w["embed"])[only1][sure]) < REL_TOL
    assert np.abs(master["embed"][only1] - p1["embed"][only1]).min() > 0


@pytest.mark.parametrize("kw", [dict(serialize=1), dict(ckpt_interval=2), dict(prefetch_depth=1),
                                dict(prefetch_depth=3), dict(use_slab_pool=0),
                                dict(n_slabs=1), dict(host_threads=3), dict(keep_internals=0),
                                dict(keep_internals=0, ckpt_interval=1), dict(defer_updates=0),
                                dict(resident_layers=1), dict(resident_layers=2)],
                         ids=["serialized", "K2", "depth1", "depth3", "no-pool", "one-slab",
                              "3-threads", "recompute", "recompute-K1", "no-defer", "resident1",
                              "resident2"])
def test_schedule_invariance_bitwise(tiny, kw):
    s, w, ids = tiny
    base = _run(s, w, ids)
    other = _run(s, w, ids, **kw)
    assert base["loss"] == other["loss"]
    for n in synth.param_names(s):
        np.testing.assert_array_equal(base["grad"][n], other["grad"][n], err_msg=n)
        np.testing.assert_array_equal(base["master"][n], other["master"][n], err_msg=n)


def test_streamed_deeper_model_matches_oracle():
    """5 layers with K = 2 (segments of 2, 2 and 1 layers), ragged T.

    Weights are drawn bf16-representable so the comparison measures the
    GPU's bf16 activations and gradients, not the rounding of the inputs
    (which alone moves the attention-projection gradients of this model by
    about 1% in the oracle itself)."""
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=5, ckpt_interval=2, seq=60, batch=3)
    w = synth.make_weights(s, seed=4, bf16_exact=True)
    ids = synth.make_tokens(s, seed=5)
    g = _run(s, w, ids)
    loss, grads, newp, _ = D.train_step(w, ids, s)
    assert abs(g["loss"][0] - loss) < LOSS_TOL
    for n in synth.param_names(s):
        assert rel(g["grad"][n], grads[n]) < REL_TOL, (n, rel(g["grad"][n], grads[n]))


def test_bad_tokens_rejected_without_update(tiny):
    torch, mt = _env()
    s, w, ids = tiny
    m = mt.Model(s)
    m.set_params(w)
    arena = torch.empty(m.arena_bytes(*ids.shape), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    bad = ids.copy()
    bad[1, 5] = s.vocab
    with pytest.raises(mt.MTError) as e:
        m.step(bad, arena, streams)
    assert e.value.status == mt.MT_E_INVALID
    assert m.step_count == 0
    np.testing.assert_array_equal(m.get("lm_head"), w["lm_head"])
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mt.MTError) as e:
        m.step(ids, small, streams)
    assert e.value.status == mt.MT_E_OOM_DEVICE
    m.close()


def test_chunked_mlp_and_head_long_sequence_matches_oracle():
    """Long sequence with both chunked paths on: MLP over 512-token chunks,
    LM head over 768-token chunks (ragged last chunk of each), K = 2."""
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=3, ckpt_interval=2, batch=1, seq=2000,
                                             mlp_chunk_tokens=512)
    w = synth.make_weights(s, seed=8, bf16_exact=True)
    ids = synth.make_tokens(s, seed=9)
    g = _run(s, w, ids, head_chunk_tokens=768)
    loss, grads, newp, _ = D.train_step(w, ids, s)
    assert abs(g["loss"][0] - loss) < LOSS_TOL, (g["loss"][0], loss)
    for n in synth.param_names(s):
        assert rel(g["grad"][n], grads[n]) < REL_TOL, (n, rel(g["grad"][n], grads[n]))


# fp32 debug precision: streamed copy, activations, gradients and slabs all
# fp32; the oracle in float64.  Bar: 1e-4 relative (loss: absolute).
F32_TOL = 1e-4


@pytest.mark.parametrize("kw", [dict(), dict(mlp_chunk_tokens=64, head_chunk_tokens=100)],
                         ids=["whole", "chunked"])
def test_step_fp32_debug_precision_matches_oracle(tiny, kw):
    torch, mt = _env()
    s, w, ids = tiny
    g = _run(s, w, ids, precision=mt.PREC_FP32_DEBUG, **kw)
    w64 = {k: v.astype(np.float64) for k, v in w.items()}
    loss, grads, newp, state = D.train_step(w64, ids, s)
    assert abs(g["loss"][0] - loss) < F32_TOL, (g["loss"][0], loss)
    for n in synth.param_names(s):
        assert rel(g["grad"][n], grads[n]) < F32_TOL, (n, rel(g["grad"][n], grads[n]))
        assert rel(g["m"][n], state[n][0]) < F32_TOL, n
        assert rel(g["master"][n], newp[n]) < F32_TOL, n
        # the streamed copy is the updated master itself
        np.testing.assert_array_equal(g["shadow"][n], g["master"][n])
    # the update itself: away from gradients within fp32 noise of zero,
    # Adam's first step moves each weight by lr * sign(g)
    for n in synth.param_names(s):
        dp, dref = g["master"][n] - w[n], newp[n] - w64[n]
        sure = np.abs(grads[n]) > 1e-3 * np.abs(grads[n]).max()
        assert rel(dp[sure], dref[sure]) < 1e-3, (n, rel(dp[sure], dref[sure]))


def test_step_fp32_schedule_invariance_bitwise(tiny):
    torch, mt = _env()
    s, w, ids = tiny
    base = _run(s, w, ids, precision=mt.PREC_FP32_DEBUG)
    other = _run(s, w, ids, precision=mt.PREC_FP32_DEBUG, serialize=1, ckpt_interval=2)
    assert base["loss"] == other["loss"]
    for n in synth.param_names(s):
        np.testing.assert_array_equal(base["grad"][n], other["grad"][n], err_msg=n)
        np.testing.assert_array_equal(base["master"][n], other["master"][n], err_msg=n)


def test_deferred_updates_apply_before_reads_and_never_after_a_set(tiny):
    """With deferred head / embedding updates: two steps equal two steps
    without deferral bitwise (the second step applies the first's pending
    updates while it streams), and a parameter set after a step keeps the
    set value (the pending update lands before the set, not after)."""
    torch, mt = _env()
    s, w, ids = tiny
    a = _run(s, w, ids, steps=2)
    b = _run(s, w, ids, steps=2, defer_updates=0)
    assert a["loss"] == b["loss"]
    for n in synth.param_names(s):
        np.testing.assert_array_equal(a["master"][n], b["master"][n], err_msg=n)
        np.testing.assert_array_equal(a["shadow"][n], b["shadow"][n], err_msg=n)
    m = mt.Model(s)
    m.set_params(w)
    arena = torch.empty(m.arena_bytes(*ids.shape), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    m.step(ids, arena, streams)
    new = np.full(w["lm_head"].shape, 0.125, np.float32)
    m.set_param("lm_head", new)
    np.testing.assert_array_equal(m.get("lm_head"), new)
    m.step(ids, arena, streams)  # uses the set head (no stale pending update)
    assert m.step_count == 2
    m.close()


def _steps(shape, weights, ids, n, arenas=None, set_between=None, **run_kw):
    """n steps; arenas[i] picks the arena of step i (0 or 1, two arenas of
    the same size); set_between = (step, name, value) sets a parameter
    before that step."""
    torch, mt = _env()
    m = mt.Model(shape, **run_kw)
    m.set_params(weights)
    B, T = ids.shape
    ar = [torch.empty(m.arena_bytes(B, T), dtype=torch.uint8, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    losses, h2d = [], []
    for i in range(n):
        if set_between and set_between[0] == i:
            m.set_param(set_between[1], set_between[2])
        loss, st = m.step(ids, ar[arenas[i] if arenas else 0], streams)
        losses.append(loss)
        h2d.append(st["h2d_bytes"])
    names = synth.param_names(shape)
    out = {"loss": losses, "h2d": h2d,
           "master": {n_: m.get(n_, mt.GET_MASTER) for n_ in names},
           "shadow": {n_: m.get(n_, mt.GET_SHADOW) for n_ in names}}
    m.close()
    return out


def _same(a, b, names):
    assert a["loss"] == b["loss"]
    for n in names:
        np.testing.assert_array_equal(a["master"][n], b["master"][n], err_msg=n)
        np.testing.assert_array_equal(a["shadow"][n], b["shadow"][n], err_msg=n)


@pytest.mark.parametrize("R", [1, 3, 5])
def test_resident_layers_bitwise_over_steps(R):
    """Resident layers (kept on the device between steps, refilled after
    each update): three steps equal three steps without them bitwise, and
    from the second step on the forward streams R layers fewer; a set
    parameter or a different arena makes the next step load them again,
    still with the same results."""
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=5, ckpt_interval=2, seq=60, batch=3)
    w = synth.make_weights(s, seed=4)
    ids = synth.make_tokens(s, seed=5)
    names = synth.param_names(s)
    base = _steps(s, w, ids, 3)
    res = _steps(s, w, ids, 3, resident_layers=R)
    _same(base, res, names)
    # step 1 loads the resident layers (and uploads their update); steps 2
    # and 3 skip those loads but still upload the updates: the same bytes
    # per step as step 1 minus R layer loads
    assert res["h2d"][1] == res["h2d"][2] < res["h2d"][0]
    # another arena in step 2, a set parameter before step 3
    new = (w["layers.4.w_down"] * 0.5).astype(np.float32)
    base2 = _steps(s, w, ids, 3, set_between=(2, "layers.4.w_down", new))
    res2 = _steps(s, w, ids, 3, arenas=[0, 1, 1], set_between=(2, "layers.4.w_down", new),
                  resident_layers=R)
    _same(base2, res2, names)
    assert res2["h2d"][1] == res2["h2d"][0]  # new arena: loaded again
    assert res2["h2d"][2] == res2["h2d"][0]  # after a set: loaded again


@pytest.mark.parametrize("kw", [dict(precision=1), dict(mlp_chunk_tokens=64, head_chunk_tokens=100),
                                dict(serialize=1), dict(keep_internals=0, ckpt_interval=1)],
                         ids=["fp32", "chunked", "serialized", "recompute-K1"])
def test_resident_layers_bitwise_in_every_mode(kw):
    """Resident layers in the fp32 debug precision, with the chunked MLP and
    head (recompute schedule), on one stream and with K = 1: two steps equal
    two steps without resident layers, bitwise."""
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=4, ckpt_interval=2, seq=96, batch=2)
    if "ckpt_interval" in kw:
        s = s.with_(ckpt_interval=kw["ckpt_interval"])
    w = synth.make_weights(s, seed=6)
    ids = synth.make_tokens(s, seed=7)
    names = synth.param_names(s)
    run_kw = {k: v for k, v in kw.items() if k != "ckpt_interval"}
    base = _steps(s, w, ids, 2, **run_kw)
    res = _steps(s, w, ids, 2, resident_layers=2, **run_kw)
    _same(base, res, names)
    assert res["h2d"][1] < res["h2d"][0]


def test_chunked_mlp_kept_attention_internals_bitwise():
    """With a chunked MLP, keeping the attention half's internals (and
    recomputing each chunk's gate/up in the backward) equals the full
    recompute schedule bitwise over two steps."""
    s = synth.CONFIGS["tiny-2l-h256"].with_(n_layers=4, ckpt_interval=2, seq=96, batch=2)
    w = synth.make_weights(s, seed=8)
    ids = synth.make_tokens(s, seed=9)
    kw = dict(mlp_chunk_tokens=64, head_chunk_tokens=100)
    base = _steps(s, w, ids, 2, keep_internals=0, **kw)
    kept = _steps(s, w, ids, 2, keep_internals=1, **kw)
    _same(base, kept, synth.param_names(s))


# Hybrid 8-bit optimizer states and global-norm clipping (LazyTrain
# abstract): the streamed step against the oracle's train_step_adam8.


def _run8(shape, weights, batches, **run_kw):
    torch, mt = _env()
    m = mt.Model(shape, keep_grads=1, opt_8bit=1, **run_kw)
    m.set_params(weights)
    B, T = batches[0].shape
    arena = torch.empty(m.arena_bytes(B, T), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    losses, stats = [], []
    for ids in batches:
        loss, st = m.step(ids, arena, streams)
        losses.append(loss)
        stats.append(st)
    names = synth.param_names(shape)
    out = {"loss": losses, "stats": stats,
           "grad": {n: m.get(n, mt.GET_GRAD) for n in names},
           "master": {n: m.get(n, mt.GET_MASTER) for n in names},
           "m": {n: m.get(n, mt.GET_M) for n in names},
           "v": {n: m.get(n, mt.GET_V) for n in names}}
    m.close()
    return out


@pytest.mark.parametrize("clip", [0.0, 0.05], ids=["no-clip", "clip"])
def test_step_adam8_two_batches_match_oracle(tiny, clip):
    """Two steps on different batches with the hybrid 8-bit states (and,
    in the second case, a clipping norm below the gradient's norm, so every
    gradient is scaled): loss, gradients, updated masters and the moments
    the 8-bit states hold against the oracle; the clipping factor the step
    reports against the oracle's."""
    from oracle import adam8 as A8
    s, w, ids1 = tiny
    ids2 = synth.make_tokens(s, seed=77)
    g = _run8(s, w, [ids1, ids2], clip_norm=clip)
    l1, _, c1, p1, st1 = A8.train_step_adam8(w, ids1, s, max_norm=clip)
    l2, g2, c2, p2, st2 = A8.train_step_adam8(p1, ids2, s, state=st1, step=2, max_norm=clip)
    assert abs(g["loss"][0] - l1) < LOSS_TOL and abs(g["loss"][1] - l2) < LOSS_TOL
    if clip:
        assert c1 < 1 and c2 < 1  # clipping is active in both steps
        for st, c in zip(g["stats"], (c1, c2)):
            assert abs(st["clip_factor"] - c) / c < REL_TOL, (st["clip_factor"], c)
    else:
        assert all(st["clip_factor"] == 1.0 for st in g["stats"])
    for n in synth.param_names(s):
        assert rel(g["grad"][n], g2[n]) < REL_TOL, (n, rel(g["grad"][n], g2[n]))
        assert rel(g["master"][n], p2[n]) < REL_TOL, n
        m_ref = A8.dequantize(st2[n][0], st2[n][1]).reshape(w[n].shape)
        r_ref = A8.dequantize(st2[n][2], st2[n][3]).reshape(w[n].shape)
        assert rel(g["m"][n], m_ref) < 3 * REL_TOL, (n, rel(g["m"][n], m_ref))
        assert rel(g["v"][n], r_ref * r_ref) < 3 * REL_TOL, (n, rel(g["v"][n], r_ref * r_ref))


@pytest.mark.parametrize("kw", [dict(defer_updates=0), dict(serialize=1, ckpt_interval=2),
                                dict(resident_layers=1), dict(use_slab_pool=0)],
                         ids=["no-defer", "serialized-K2", "resident1", "no-pool"])
def test_step_adam8_clip_schedule_invariance_bitwise(tiny, kw):
    """The 8-bit states with clipping do not depend on the schedule: three
    steps give bitwise the same losses, masters and moments."""
    s, w, ids1 = tiny
    batches = [ids1, synth.make_tokens(s, seed=78), synth.make_tokens(s, seed=79)]
    run_kw = {k: v for k, v in kw.items() if k != "ckpt_interval"}
    sh = s.with_(ckpt_interval=kw.get("ckpt_interval", s.ckpt_interval))
    base = _run8(s, w, batches, clip_norm=0.05)
    other = _run8(sh, w, batches, clip_norm=0.05, **run_kw)
    assert base["loss"] == other["loss"]
    assert [x["clip_factor"] for x in base["stats"]] == [x["clip_factor"] for x in other["stats"]]
    for n in synth.param_names(s):
        np.testing.assert_array_equal(base["master"][n], other["master"][n], err_msg=n)
        np.testing.assert_array_equal(base["m"][n], other["m"][n], err_msg=n)
        np.testing.assert_array_equal(base["v"][n], other["v"][n], err_msg=n)


# Global-norm clipping with fp32 moments, and the layers' clipped updates
# the next step applies while it streams (defer_updates).


def _run_clip(shape, weights, batches, get_between=False, **run_kw):
    """Steps over `batches` with fp32 moments; get_between reads every
    master after each step (which applies the pending updates early)."""
    torch, mt = _env()
    m = mt.Model(shape, keep_grads=1, **run_kw)
    m.set_params(weights)
    B, T = batches[0].shape
    arena = torch.empty(m.arena_bytes(B, T), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    names = synth.param_names(shape)
    losses, stats, grads = [], [], []
    for ids in batches:
        loss, st = m.step(ids, arena, streams)
        losses.append(loss)
        stats.append(st)
        grads.append({n: m.get(n, mt.GET_GRAD) for n in names})
        if get_between:
            for n in names:
                m.get(n, mt.GET_MASTER)
    out = {"loss": losses, "stats": stats, "grads": grads,
           "master": {n: m.get(n, mt.GET_MASTER) for n in names},
           "shadow": {n: m.get(n, mt.GET_SHADOW) for n in names},
           "m": {n: m.get(n, mt.GET_M) for n in names},
           "v": {n: m.get(n, mt.GET_V) for n in names}}
    m.close()
    return out


def _oracle_clip_fp32(params, ids, shape, state, step, max_norm):
    """Forward, backward, global-norm clipping (the oracle's coefficient)
    and the fp32 Adam of the oracle on the clipped gradient."""
    from oracle import adam8 as A8
    loss, grads = D.loss_and_grads(params, ids, shape, "resident", None)
    c = A8.clip_coefficient(grads, max_norm)
    new_p, new_s = {}, {}
    for n, p in params.items():
        m, v = state[n] if state else (np.zeros_like(p), np.zeros_like(p))
        g = (np.asarray(grads[n], np.float32) * np.float32(c)).astype(np.float32)
        new_p[n], m2, v2 = D.adam_update(p, m, v, g, step, shape.lr, shape.beta1, shape.beta2,
                                         shape.adam_eps)
        new_s[n] = (m2, v2)
    return loss, grads, c, new_p, new_s


def test_step_clip_fp32_two_batches_match_oracle(tiny):
    """Two steps on different batches with fp32 moments and a clipping norm
    below the gradient's (every gradient scaled): loss, gradients, clip
    factor, masters and moments against the oracle."""
    s, w, ids1 = tiny
    ids2 = synth.make_tokens(s, seed=81)
    g = _run_clip(s, w, [ids1, ids2], clip_norm=0.05)
    l1, g1, c1, p1, st1 = _oracle_clip_fp32(w, ids1, s, None, 1, 0.05)
    l2, g2, c2, p2, st2 = _oracle_clip_fp32(p1, ids2, s, st1, 2, 0.05)
    assert c1 < 1 and c2 < 1
    assert abs(g["loss"][0] - l1) < LOSS_TOL and abs(g["loss"][1] - l2) < LOSS_TOL
    for st, c in zip(g["stats"], (c1, c2)):
        assert abs(st["clip_factor"] - c) / c < REL_TOL, (st["clip_factor"], c)
    for n in synth.param_names(s):
        assert rel(g["grads"][0][n], g1[n]) < REL_TOL, n
        assert rel(g["grads"][1][n], g2[n]) < REL_TOL, n
        assert rel(g["master"][n], p2[n]) < REL_TOL, n
        assert rel(g["m"][n], st2[n][0]) < REL_TOL, n
        assert rel(g["v"][n], st2[n][1]) < 2 * REL_TOL, n


@pytest.mark.parametrize("kw", [dict(), dict(resident_layers=1), dict(use_slab_pool=0),
                                dict(get_between=True), dict(opt_8bit=1, get_between=True)],
                         ids=["deferred", "resident1", "no-pool", "read-between",
                              "8bit-read-between"])
def test_step_clip_deferred_layer_updates_bitwise(tiny, kw):
    """With clipping, the layers' updates run at the start of the next step
    (before each layer's first load); three steps on different batches give
    bitwise the losses, kept gradients, masters, streamed copies and moments
    of the in-step updates, also when the model is read between steps (the
    read applies the pending updates) and with a resident layer (its
    device copy is refreshed from the updated streamed copy)."""
    s, w, ids1 = tiny
    batches = [ids1, synth.make_tokens(s, seed=82), synth.make_tokens(s, seed=83)]
    kw = dict(kw)
    base_kw = {"opt_8bit": kw.get("opt_8bit", 0)}
    base = _run_clip(s, w, batches, clip_norm=0.05, defer_updates=0, **base_kw)
    other = _run_clip(s, w, batches, clip_norm=0.05, **kw)
    assert base["loss"] == other["loss"]
    assert [x["clip_factor"] for x in base["stats"]] == [x["clip_factor"] for x in other["stats"]]
    for n in synth.param_names(s):
        for i in range(3):
            np.testing.assert_array_equal(base["grads"][i][n], other["grads"][i][n], err_msg=n)
        for k in ("master", "shadow", "m", "v"):
            np.testing.assert_array_equal(base[k][n], other[k][n], err_msg=f"{k} {n}")
