"""Delta cache policy: the oracle pinned by a hand-derived trace and by invariants over random
traces, then the library's C++ manager against the oracle, decision by decision."""
import numpy as np
import pytest

import oracle.residency_oracle as R


def test_oracle_hand_trace():
    # 4 variants of 10 bytes, room for 3, the top 1 pinned
    c = R.ResidencyRef([10, 10, 10, 10], 30, num_pinned=1)
    assert c.request(0) == (R.LOAD, [])           # cold start
    assert c.request(0) == (R.QUEUED, [])         # waits for the load in flight
    c.load_done(0)
    assert c.request(0) == (R.HIT, [])            # variant 0: 3 requests, pinned
    assert c.request(1) == (R.LOAD, [])
    c.load_done(1)
    assert c.request(2) == (R.LOAD, [])
    c.load_done(2)
    assert c.request(1) == (R.HIT, [])            # 1 is now more recent than 2
    assert c.request(3) == (R.LOAD, [2])          # full: the least recent unpinned goes
    assert c.state == [R.RESIDENT, R.RESIDENT, R.ABSENT, R.LOADING]
    assert c.request(2) == (R.LOAD, [1])          # 3 is loading, 0 pinned: only 1 can go
    assert c.request(1) == (R.NO_ROOM, [])        # 0 pinned, 2 and 3 loading: nothing to evict
    assert c.state == [R.RESIDENT, R.ABSENT, R.LOADING, R.LOADING]
    c.load_done(3)
    c.load_done(2)
    # counts now 0:3, 1:3, 2:2, 3:1: the pinned one is 0 (tie with 1 goes to the smaller id)
    assert c.pinned() == {0}
    # this request makes 1 the most requested (4 against 3): 1 is pinned now, and 0, the least
    # recent of the others (time 3, against 7 for 3 and 8 for 2), is evicted
    assert c.request(1) == (R.LOAD, [0])
    assert c.pinned() == {1}
    with pytest.raises(ValueError):
        c.load_done(0)


def test_oracle_hand_trace_holds():
    # 3 variants of 10 bytes, room for 2, nothing pinned
    c = R.ResidencyRef([10, 10, 10], 20, num_pinned=0)
    assert c.request(0, hold=True) == (R.LOAD, [])  # a batch needs 0, then 1
    c.load_done(0)
    assert c.request(1, hold=True) == (R.LOAD, [])
    c.load_done(1)
    # 0 is the least recent, but held: without the hold it would go; now 1 is held too
    assert c.request(2) == (R.NO_ROOM, [])
    c.release(1)
    assert c.request(2) == (R.LOAD, [1])            # the only unheld resident one goes
    c.load_done(2)
    assert c.request(2, hold=True) == (R.HIT, [])   # a hit holds too
    assert c.request(1) == (R.NO_ROOM, [])          # 0 and 2 are both held
    assert c.holds == [1, 0, 1]
    c.release(0)
    assert c.request(1) == (R.LOAD, [0])            # 0 released: the least recent unheld goes
    assert c.holds == [0, 0, 1]
    assert c.request(1, hold=True) == (R.QUEUED, [])  # queued behind the load, and held
    assert c.holds == [0, 1, 1]
    with pytest.raises(ValueError):
        c.release(0)


def test_oracle_pins_follow_traffic():
    c = R.ResidencyRef([5] * 6, 10, num_pinned=2)
    for v in (4, 4, 4, 2, 2, 5):
        c.request(v)
        if c.state[v] == R.LOADING:
            c.load_done(v)
    assert c.pinned() == {4, 2}
    # 4 and 2 are resident and pinned, so 5 cannot be loaded and any other request finds no room
    assert c.state[4] == R.RESIDENT and c.state[2] == R.RESIDENT and c.state[5] == R.ABSENT
    assert c.request(0) == (R.NO_ROOM, [])


def _random_trace(seed, n, steps):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, n + 1) ** 1.1
    return rng.choice(n, size=steps, p=p / p.sum()), rng.random(steps)


@pytest.mark.parametrize("seed", range(6))
def test_oracle_invariants(seed):
    n = 14
    sizes = np.random.default_rng(100 + seed).integers(1, 9, size=n) * 1000
    cap = int(sizes.sum() * 0.6)
    c = R.ResidencyRef(sizes, cap, num_pinned=6)
    trace, coin = _random_trace(seed, n, 3000)
    for v, u in zip(trace, coin):
        state_before = list(c.state)
        act, ev = c.request(int(v))
        pins = c.pinned()  # the pinned set counts the request itself
        assert c.used() <= cap
        for e in ev:  # only resident, unpinned, other variants are evicted
            assert state_before[e] == R.RESIDENT and e not in pins and e != v
        if act == R.NO_ROOM:
            assert c.state == state_before
        if u < 0.7:  # loads finish at random later points
            for w in range(n):
                if c.state[w] == R.LOADING:
                    c.load_done(w)
    # with room for the pinned set, the top variants by traffic end up resident
    top = sorted(range(n), key=lambda v: (-c.count[v], v))[:6]
    for v in top:
        if c.state[v] == R.ABSENT:
            c.request(v)
            c.load_done(v)
        assert c.state[v] != R.ABSENT


bd = pytest.importorskip("tenant_serving_bitdelta_amd")


@pytest.mark.parametrize("seed,n,pinned,frac,hold", [(0, 14, 6, 0.6, 0), (1, 14, 6, 0.45, 0),
                                                     (2, 5, 1, 0.5, 0), (3, 64, 6, 0.3, 0),
                                                     (4, 14, 0, 0.5, 0), (5, 3, 6, 0.9, 0),
                                                     (6, 14, 6, 0.6, 1), (7, 14, 0, 0.45, 1),
                                                     (8, 64, 6, 0.3, 1)])
def test_manager_matches_oracle(seed, n, pinned, frac, hold):
    rng = np.random.default_rng(200 + seed)
    sizes = [int(s) for s in rng.integers(1, 9, size=n) * 1_000_000_007]  # > 2^32 in total
    cap = max(int(sum(sizes) * frac), max(sizes))
    ref = R.ResidencyRef(sizes, cap, num_pinned=pinned)
    lib = bd.Residency(sizes, cap, num_pinned=pinned)
    trace, coin = _random_trace(seed, n, 4000)
    for step, (v, u) in enumerate(zip(trace, coin)):
        h = bool(hold) and rng.random() < 0.5
        got, want = lib.request(int(v), hold=h), ref.request(int(v), hold=h)
        assert got == (want[0], want[1]), (step, got, want)
        # held requests finish (release) at random later points
        for w in range(n):
            while ref.holds[w] and rng.random() < 0.3:
                ref.release(w)
                lib.release(w)
        assert [lib.holds(w) for w in range(n)] == ref.holds, step
        # a random subset of the loads in flight finishes
        for w in range(n):
            if ref.state[w] == R.LOADING and rng.random() < u:
                ref.load_done(w)
                lib.load_done(w)
        assert [lib.state(w) for w in range(n)] == ref.state, step
        assert lib.used_bytes() == ref.used()


def test_manager_holds_errors():
    r = bd.Residency([10, 10, 10], 20, num_pinned=0)
    with pytest.raises(bd.BitDeltaError):
        r.release(0)                                     # no holder
    assert r.request(0, hold=True) == (bd.Residency.LOAD, [])
    r.load_done(0)
    assert r.request(1, hold=True) == (bd.Residency.LOAD, [])
    r.load_done(1)
    assert r.request(2) == (bd.Residency.NO_ROOM, [])    # both residents held
    r.release(0)
    assert r.holds(0) == 0 and r.holds(1) == 1
    assert r.request(2) == (bd.Residency.LOAD, [0])
    assert r.holds(7) == -1


def test_manager_argument_errors():
    with pytest.raises(bd.BitDeltaError):
        bd.Residency([], 10)
    with pytest.raises(bd.BitDeltaError):
        bd.Residency([10, 0], 10)
    with pytest.raises(bd.BitDeltaError):
        bd.Residency([10], 0)
    with pytest.raises(bd.BitDeltaError):
        bd.Residency([10], 10, num_pinned=-1)
    r = bd.Residency([10, 10], 10)
    with pytest.raises(bd.BitDeltaError):
        r.request(2)
    with pytest.raises(bd.BitDeltaError):
        r.load_done(0)  # not loading
    assert r.state(5) == -1
    assert r.request(0) == (bd.Residency.LOAD, [])
    assert r.request(1) == (bd.Residency.NO_ROOM, [])  # 0 is loading and cannot be evicted
    r.load_done(0)
    assert r.request(1) == (bd.Residency.NO_ROOM, [])  # 0 pinned (num_pinned 6)


def test_manager_concurrent_requests():
    """Eight threads request and finish loads at once: every load is started exactly once per
    absence (no double loads), the bytes held never exceed the capacity, and the final states
    agree with the loads still open."""
    import threading
    n, cap = 14, 40
    sizes = [5] * n
    r = bd.Residency(sizes, cap, num_pinned=6)
    lock = threading.Lock()
    loading = set()
    errors = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        p = 1.0 / np.arange(1, n + 1) ** 1.1
        for v in rng.choice(n, size=2000, p=p / p.sum()):
            act, _ = r.request(int(v))
            if act == bd.Residency.LOAD:
                with lock:
                    if int(v) in loading:
                        errors.append(("double load", int(v)))
                    loading.add(int(v))
            if r.used_bytes() > cap:
                errors.append(("over capacity", r.used_bytes()))
            if rng.random() < 0.5:
                with lock:
                    done = list(loading)
                    loading.clear()
                for w in done:
                    r.load_done(w)

    threads = [threading.Thread(target=worker, args=(300 + i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]
    for w in range(n):
        assert (r.state(w) == bd.Residency.LOADING) == (w in loading)
