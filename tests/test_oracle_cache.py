"""Pins for the oracle's rolling-cache simulation (hand-worked sequences and invariants)."""
import pytest

from oracle.cache import RollingCacheModel


def _run(Lc, sink, window, n):
    m = RollingCacheModel(Lc, sink, window)
    out = []
    for c in range(n):
        slot = m.write(c)
        out.append((slot, m.visible_chunks(), m.visible_len()))
    return out


def test_window_only_fill_then_evict():
    # 4-chunk window, no sink (the streaming configuration: current chunk + 3 previous)
    got = _run(10, 0, 40, 9)
    expect = [
        (0, [0], 10), (10, [0, 1], 20), (20, [0, 1, 2], 30), (30, [0, 1, 2, 3], 40),
        (0, [1, 2, 3, 4], 40), (10, [2, 3, 4, 5], 40), (20, [3, 4, 5, 6], 40), (30, [4, 5, 6, 7], 40),
        (0, [5, 6, 7, 8], 40),
    ]
    assert got == expect


def test_one_sink_three_window():
    got = _run(10, 10, 30, 8)
    expect = [
        (0, [0], 10), (10, [0, 1], 20), (20, [0, 1, 2], 30), (30, [0, 1, 2, 3], 40),
        (10, [0, 2, 3, 4], 40), (20, [0, 3, 4, 5], 40), (30, [0, 4, 5, 6], 40), (10, [0, 5, 6, 7], 40),
    ]
    assert got == expect


def test_two_sinks_one_window():
    got = _run(10, 20, 10, 5)
    expect = [(0, [0], 10), (10, [0, 1], 20), (20, [0, 1, 2], 30), (20, [0, 1, 3], 30), (20, [0, 1, 4], 30)]
    assert got == expect


@pytest.mark.parametrize("Lc,sink,window", [(3, 0, 3), (5, 10, 20), (7, 7, 49), (2, 6, 4)])
def test_invariants(Lc, sink, window):
    m = RollingCacheModel(Lc, sink, window)
    n_sink, n_win = sink // Lc, window // Lc
    for c in range(3 * (n_sink + n_win) + 5):
        slot = m.write(c)
        assert 0 <= slot < sink + window and slot % Lc == 0
        vis = m.visible_chunks()
        # sinks first, then the most recent window chunks, chunk c always visible and last
        assert vis[-1] == c
        assert vis[:min(c + 1, n_sink)] == list(range(min(c + 1, n_sink)))
        recent = [x for x in range(n_sink, c + 1)][-n_win:]
        assert vis[min(c + 1, n_sink):] == recent
        # visible chunks occupy distinct slots; sinks never move
        slots = [m.slot_of(x) for x in vis]
        assert len(set(slots)) == len(slots)
        for s in range(min(c + 1, n_sink)):
            assert m.slot_of(s) == s * Lc


def test_rejects_bad_geometry():
    with pytest.raises(ValueError):
        RollingCacheModel(10, 5, 40)
    with pytest.raises(ValueError):
        RollingCacheModel(10, 0, 0)
    m = RollingCacheModel(10, 0, 20)
    with pytest.raises(ValueError):
        m.write(1)
