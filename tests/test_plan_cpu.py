"""The engine's stream schedule, checked on the CPU for hazards.

The schedule (mt_debug_plan) is what mt_stream_step replays with HIP
events.  These tests walk it as a discrete-event system: every layer runs
forward once and backward once, every compute op finds its weights loaded,
no weight slot is overwritten while an earlier occupant still has a reader,
loads never wait on compute that comes after their own first use (no
deadlock), and no load runs more than `depth` ops ahead.
"""
import pytest

FWD, HEAD, REFWD, BWD, FWDK = 0, 1, 2, 3, 4


def _plan(L, K, depth, keep=1, resident=0):
    from layer_streamed_amd import mt
    return mt.debug_plan(L, K, depth, keep, resident)


@pytest.mark.parametrize("L", [1, 2, 5, 28])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 7, 28])
@pytest.mark.parametrize("depth", [1, 2, 3])
@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("resident", [0, 1, 5, 12, 28])
def test_plan_is_hazard_free(L, K, depth, keep, resident):
    if K > L:
        K = L
    R = min(resident, L)
    st, ops, loads, n_slots = _plan(L, K, depth, keep, R)
    assert st == 0
    kinds = ops[:, 0].tolist()
    a_last = ((L - 1) // K) * K
    # forward of every layer in order (the last segment keeping its
    # internals when internals are kept), then the head
    assert kinds[:L] == [FWDK if keep and l >= a_last else FWD for l in range(L)]
    assert ops[:L, 1].tolist() == list(range(L))
    assert kinds[L] == HEAD
    # backward: segments from the last, each re-forwarding from the
    # checkpoint (every layer when internals are kept, else all but the
    # last; nothing for the last segment when it kept them in the forward),
    # then backward in reverse
    rest = ops[L + 1:]
    expect = []
    for a in reversed(range(0, L, K)):
        e = min(a + K, L)
        if not (keep and a == a_last):
            expect += [(REFWD, l) for l in range(a, e if keep else e - 1)]
        expect += [(BWD, l) for l in reversed(range(a, e))]
    assert [(int(k), int(l)) for k, l, _ in rest] == expect
    if keep:  # the last segment's backward reads the forward's loads
        for k, l, ld in ops[L + 1:]:
            if k == BWD and l >= a_last:
                assert ld == ops[l][2]
    # every op reads a load of its own unit, inside that load's live range
    for i, (kind, layer, load) in enumerate(ops):
        unit, slot, first, last, wait, gate = loads[load]
        assert unit == (L if kind == HEAD else layer)
        assert first <= i <= last
    # a resident layer (1 .. R, or all) has one load, in slot -3 - c,
    # serving every op of it
    rs = 1 if R < L else 0
    for l in range(L):
        used = {int(ld) for k, lay, ld in ops if k != HEAD and lay == l}
        if rs <= l < rs + R:
            assert len(used) == 1
            assert loads[used.pop()][1] == -3 - (l - rs)
    assert sum(1 for ld in loads if ld[1] <= -3) == R
    # loads are issued in order of first use; dependencies precede the use
    firsts = loads[:, 2].tolist()
    assert firsts == sorted(firsts)
    for j, (unit, slot, first, last, wait, gate) in enumerate(loads):
        assert wait < first and gate < first
        # forward loads look further ahead when resident layers leave the
        # link idle; the head then follows the last layer's forward load
        ahead = max(depth, n_slots) if (R > 0 and first < L) else depth
        base = first - ahead if first - ahead >= 0 else -1
        if unit == L and R > 0 and j > 0:
            assert gate == min(base, loads[j - 1][5])
        else:
            assert gate == base
    # slot reuse: the next occupant waits for the last reader of the previous
    by_slot = {}
    for j, (unit, slot, first, last, wait, gate) in enumerate(loads):
        if slot == -2:
            assert unit == L
            continue
        if slot <= -3:
            assert unit == rs + (-3 - slot) and wait == -1
            continue
        assert 0 <= slot < n_slots
        if slot in by_slot:
            prev = loads[by_slot[slot]]
            assert wait >= prev[3], (j, slot)
            assert first > prev[3]
        by_slot[slot] = j


@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("resident", [0, 6])
def test_plan_single_stream_replay_never_reads_stale_weights(keep, resident):
    """Replay the plan as the executor does on one in-order stream and track
    which unit each slot holds at every compute op."""
    L, K, depth = 28, 4, 2
    st, ops, loads, n_slots = _plan(L, K, depth, keep, resident)
    assert st == 0
    holds = {}
    nxt = 0
    for i, (kind, layer, load) in enumerate(ops):
        while nxt < len(loads) and max(loads[nxt][4], loads[nxt][5]) < i:
            unit, slot = loads[nxt][0], loads[nxt][1]
            holds[slot] = (unit, nxt)
            nxt += 1
        unit, slot = loads[load][0], loads[load][1]
        assert holds[slot] == (unit, load), (i, kind, layer)


def test_plan_resident_layers_skip_their_loads():
    """With the last R layers resident, those layers have one load each (in
    the first step the only copy of them; later steps skip it), and the
    backward reloads only the streamed layers' segments."""
    L, K = 28, 4
    for R in (0, 4, 8, 12, 27, 28):
        st, ops, loads, _ = _plan(L, K, 2, 1, R)
        assert st == 0
        rs = 1 if R < L else 0
        # forward: one load per layer + head; backward: re-forward loads of
        # the streamed layers outside the last segment
        refwd_loaded = sum(1 for l in range(L - K) if not rs <= l < rs + R)
        assert len(loads) == L + 1 + refwd_loaded
        assert (ops[:, 0] == BWD).sum() == L


def test_plan_counts_match_the_method():
    """Per step: L forward loads + head + backward loads; the forward uses
    each layer once, backward once.  Without kept internals the re-forward
    covers (K-1)/K of the layers (each backward then recomputes its layer)
    and every backward loads its weights again; with them, the re-forward
    covers every layer but the last segment's, which kept its internals in
    the forward and whose backward reuses the forward's weight loads."""
    L, K = 28, 4
    for keep, refwd, n_loads in ((0, L - L // K, 2 * L + 1), (1, L - K, 2 * L + 1 - K)):
        st, ops, loads, _ = _plan(L, K, 2, keep)
        assert len(loads) == n_loads
        assert (ops[:, 0] == REFWD).sum() == refwd
        assert (ops[:, 0] == BWD).sum() == L
        assert (ops[:, 0] == FWDK).sum() == (K if keep else 0)
