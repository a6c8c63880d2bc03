"""Pins for slot positions and the additive mask.

Layouts (pytorch/executorch PR 24473, Summary): a sink cache pins a prefix of
sink_size slots and runs the rest as a ring; a ring cache is a sink cache with
sink_size 0; a full-context cache uses the position as the slot and rejects a
write past its slot count.  The oracle's closed form is checked against a
step-by-step eviction simulator (fill free slots in order, then evict the
oldest non-sink entry), against hand-computed slots, and the mask against
hand-built examples and the plain causal mask it must reduce to.
"""
import numpy as np
import pytest


def _simulate(sink, window, last_pos):
    """Eviction simulator: returns the slot chosen for every position."""
    S = sink + window
    held = [None] * S
    out = []
    for p in range(last_pos + 1):
        if p < sink:
            slot = p
        elif None in held[sink:]:
            slot = sink + held[sink:].index(None)
        else:
            ages = [(held[s], s) for s in range(sink, S)]
            slot = min(ages)[1]                    # oldest non-sink position
        held[slot] = p
        out.append(slot)
    return np.array(out, np.int32)


def _sequential(slots):
    """One call writes its tokens one after another: a token whose slot a
    later token of the same call takes again is not written (-1)."""
    out = slots.copy()
    for t in range(len(slots)):
        if np.any(slots[t + 1:] == slots[t]):
            out[t] = -1
    return out


@pytest.mark.parametrize("sink,window", [(4, 2044), (0, 1024), (2, 3), (1, 1), (0, 7)])
def test_positions_match_eviction_simulation(orc, sink, window):
    last = 6000
    want = _simulate(sink, window, last)
    cp = np.full(sink + window, -1, np.int32)
    got = orc.positions_sink(0, last + 1, sink, window, cp)
    assert np.array_equal(got, _sequential(want))
    # chunked calls: the same slots per chunk (minus in-chunk overwrites) and
    # the same final positions
    cp2 = np.full(sink + window, -1, np.int32)
    p = 0
    sizes = [1, 5, 17, 300, 1]
    while p + sum(sizes) <= last:
        sizes.append(min(999, last + 1 - p - sum(sizes)))
    sizes = [s for s in sizes if s > 0]
    for T in sizes:
        assert np.array_equal(orc.positions_sink(p, T, sink, window, cp2), _sequential(want[p:p + T]))
        p += T
    assert p == last + 1
    assert np.array_equal(cp, cp2)
    # every slot's position is the simulator's last occupant
    for s in range(sink + window):
        held = np.nonzero(want == s)[0]
        assert cp[s] == (held.max() if held.size else -1)


def test_positions_hand_values(orc):
    one = lambda p, sink, window: int(orc.positions_sink(p, 1, sink, window)[0])
    assert [one(p, 4, 2044) for p in (0, 3, 4, 2047, 2048, 2049)] == [0, 3, 4, 2047, 4, 5]
    assert one(6000, 4, 2044) == 4 + (5996 % 2044) == 1912
    assert [one(p, 0, 1024) for p in (1023, 1024, 6000)] == [1023, 0, 880]
    # one call longer than the window: the early tokens of a reused slot are dropped
    s = orc.positions_sink(0, 10, 2, 3)
    assert list(s) == [0, 1, -1, -1, -1, -1, -1, 4, 2, 3]     # slots of 7, 8, 9: 2 + (p - 2) % 3


def test_positions_full_rejects_past_capacity(orc):
    sm, flags = orc.positions_full(250, 10, 256)
    assert list(sm) == [250, 251, 252, 253, 254, 255, -1, -1, -1, -1]
    assert flags == orc.FLAG_POS_CAPACITY
    sm, flags = orc.positions_full(0, 64, 256)
    assert list(sm) == list(range(64)) and flags == 0


def test_mask_hand_example(orc):
    # sink 2, window 3: positions 0..6 land in slots 0,1,2,3,4,2,3
    cp = np.full(5, -1, np.int32)
    orc.positions_sink(0, 7, 2, 3, cp)
    assert list(cp) == [0, 1, 5, 6, 4]
    m = orc.build_mask(cp, 4, 3, 2, 3)            # query positions 4, 5, 6
    inf = -np.inf
    assert m.tolist() == [[0, 0, inf, inf, 0],
                          [0, 0, 0, inf, 0],
                          [0, 0, 0, 0, 0]]
    # empty slots (-1) are never visible
    cp = np.array([0, 1, 2, -1, -1], np.int32)
    assert orc.build_mask(cp, 2, 1, 2, 3).tolist() == [[0, 0, 0, inf, inf]]


def test_mask_full_context_is_causal(orc):
    S, kv_len, Lq = 64, 40, 8
    cp = np.full(S, -1, np.int32)
    cp[:kv_len] = np.arange(kv_len)
    m = orc.build_mask(cp, kv_len - Lq, Lq, 0, S)
    j = np.arange(S)[None, :]
    qp = (kv_len - Lq + np.arange(Lq))[:, None]
    want = np.where((j <= qp), 0.0, -np.inf)
    assert np.array_equal(m, want)


@pytest.mark.parametrize("sink,window", [(4, 2044), (0, 1024)])
def test_decode_mask_all_visible_after_write(orc, sink, window):
    """Write-before-attend single-token decode sees every filled slot."""
    S = sink + window
    cp = np.full(S, -1, np.int32)
    for p in range(0, 6001):
        orc.positions_sink(p, 1, sink, window, cp)
        if p in (0, 3, 4, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 6000):
            m = orc.build_mask(cp, p, 1, sink, window)
            kv_len = min(p + 1, S)
            assert np.all(m[0, :kv_len] == 0) and np.all(np.isneginf(m[0, kv_len:]))
