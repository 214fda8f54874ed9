"""The expert pool's slot policy (host code, no device work) against a plain
Python model of its rules, on random traces and on scenarios the rules fix."""
import numpy as np
import pytest

import quantized_moe_expert_route_amd as M
from tests.pool_ref import PoolModel


def cfg(L, E, slots, trans):
    return M.MoePoolConfig(L, E, 4096, 1024, 2048, slots, trans)


def run_both(L, E, slots, trans, ops):
    got, gst = M.moe_pool_policy_trace(cfg(L, E, slots, trans), ops)
    ref = PoolModel(L, E, slots, trans)
    want = [ref.resolve(l, ids) if k == 0 else ref.prefetch(l, ids) for k, l, ids in ops]
    return got, gst, want, ref.st


@pytest.mark.parametrize("seed", range(12))
def test_policy_matches_model_random_traces(seed):
    rng = np.random.default_rng(seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(4, 40))
    slots = int(rng.integers(3, 24))
    trans = int(rng.integers(1, slots + 1))
    zipf = rng.zipf(1.3, 4000) - 1
    ops = []
    for _ in range(300):
        n = int(rng.integers(0, 7))
        ids = [int(v) % (E + 3) - (1 if rng.random() < 0.05 else 0) for v in zipf[:n]]
        zipf = np.roll(zipf, -n - 1)
        kind = 1 if rng.random() < 0.25 else 0
        ops.append((kind, int(rng.integers(0, L + (1 if rng.random() < 0.03 else 0))), ids))
    got, gst, want, wst = run_both(L, E, slots, trans, ops)
    for i, (g, w) in enumerate(zip(got, want)):
        assert (g is None and w is None) or [tuple(x) for x in g] == w, (i, ops[i], g, w)
    assert gst == wst


def test_hot_set_needs_more_touches_than_coldest():
    """Two hot-set slots: experts 0 and 1 fill them; expert 2 (one touch) is
    loaded transient; only when its touches exceed those of the coldest
    resident does it replace it (promotion without a copy when it is held)."""
    ops = [(0, 0, [0]), (0, 0, [1]), (0, 0, [1]), (0, 0, [2]), (0, 0, [3]), (0, 0, [2]),
           (0, 0, [2])]
    got, st = M.moe_pool_policy_trace(cfg(1, 8, 3, 1), ops)
    assert got[0] == [(0, 0, 1)] and got[1] == [(1, 1, 1)] and got[2] == [(1, 1, 0)]
    assert got[3] == [(2, 2, 1)]                    # transient: 1 touch, not > expert 0's 1
    assert got[4] == [(3, 2, 1)]                    # expert 3 reuses the transient slot
    assert got[5] == [(2, 0, 1)]                    # 2 touches > expert 0's 1: takes its slot
    assert got[6] == [(2, 0, 0)]                    # now a resident hit
    assert st["admitted"] == 3 and st["transient_loads"] == 2 and st["evictions"] == 2


def test_admission_replaces_coldest_and_keeps_hot_set_stable():
    """Zipf-like traffic: the hottest experts end up resident and stay there;
    a stream of one-off experts only ever takes the transient slot."""
    ops = [(0, 0, [0, 1])] * 5 + [(0, 0, [0, 1, 10 + i]) for i in range(20)]
    got, st = M.moe_pool_policy_trace(cfg(1, 40, 3, 1), ops)
    for i in range(5, 25):
        g = dict((k, (s, c)) for k, s, c in got[i])
        assert g[0][1] == 0 and g[1][1] == 0       # hot experts hit every step
        assert g[10 + i - 5][0] == 2               # one-offs cycle through the transient slot
    assert st["hits_resident"] == 2 * 24 and st["transient_loads"] == 20


def test_slots_in_use_this_epoch_are_protected():
    """Four unique experts with three slots cannot be placed in one epoch: the
    resolve fails and leaves the policy unchanged; the next one succeeds."""
    ops = [(0, 0, [0, 1, 2, 3]), (0, 0, [0, 1, 2])]
    got, st = M.moe_pool_policy_trace(cfg(1, 8, 3, 1), ops)
    assert got[0] is None and got[1] is not None
    assert st["epochs"] == 1 and st["requests"] == 3


def test_prefetch_loads_without_touching_and_hits_later():
    ops = [(1, 1, [5, 6]), (0, 1, [5, 6, 7]), (1, 0, [2]), (0, 0, [2, 2, 9])]
    got, st = M.moe_pool_policy_trace(cfg(2, 10, 5, 2), ops)
    assert [c for _, _, c in got[1]] == [0, 0, 1]
    assert got[3] == [(2, got[2][0][1], 0), (9, got[3][1][1], 1)]
    assert st["prefetch_loads"] == 3 and st["prefetch_hits"] == 3
    assert st["requests"] == 5


def test_pool_config_validation():
    bad = [cfg(0, 8, 3, 1), cfg(1, 0, 3, 1), cfg(1, 8, 0, 0), cfg(1, 8, 3, 0), cfg(1, 8, 3, 4),
           M.MoePoolConfig(1, 8, 4096, 8, 2048, 3, 1), M.MoePoolConfig(1, 8, 4096, 1024, 4096, 3, 1)]
    for c in bad:
        with pytest.raises(M.MoeError):
            M.moe_pool_policy_trace(c, [(0, 0, [1])])
