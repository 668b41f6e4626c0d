"""Expert-cache policy (host logic, no GPU): the library's simulator against
a plain Python model of the pages' cache (a per-layer LRU cache plus a
pinned hot store filled from recorded usage), and closed-form cases."""
import numpy as np
import pytest

import int4_routed_expert_moe_amd as moe


def model(E, S, P, max_promote, idx_steps, usage=None, pred_steps=None):
    """Slots [0, P) pinned with the most used experts; on each step the
    distinct routed experts hit if resident when the step starts (and are
    marked used); then up to max_promote misses (ascending) take an unpinned
    slot: an empty one (lowest), else the one used or filled longest ago
    (lowest on ties).  With predictions, before step t the distinct
    predicted experts are handled the same way, stamped with the previous
    step (resident ones refreshed first and kept, then up to max_promote
    others placed in slots neither kept nor filled by this prefetch), their
    copies landed before the step."""
    occupant = [None] * S
    stamp = [0] * S
    if usage is not None:
        ranked = sorted((e for e in range(E) if usage[e] > 0), key=lambda e: (-int(usage[e]), e))
        for s, e in enumerate(ranked[:P]):
            occupant[s] = e
    hits, misses = [], []

    def place(wanted, t_stamp):
        resident = {occupant[s]: s for s in range(S) if occupant[s] is not None}
        for e in wanted:  # every resident expert of the step is fresh first
            if e in resident:
                stamp[resident[e]] = t_stamp
        promoted = 0
        # slots of predicted experts, and those filled by this batch (their
        # copies are in flight), are no victims
        busy = {resident[e] for e in wanted if e in resident}
        for e in wanted:
            if e in resident or promoted == max_promote:
                continue
            free = [s for s in range(P, S) if occupant[s] is None and s not in busy]
            cand = [k for k in range(P, S) if k not in busy]
            if free:
                s = free[0]
            elif cand:
                s = min(cand, key=lambda k: (stamp[k], k))
            else:
                continue
            busy.add(s)
            occupant[s] = e
            stamp[s] = t_stamp
            promoted += 1

    for t, row in enumerate(idx_steps, start=1):
        if pred_steps is not None:
            place(sorted({int(e) for e in pred_steps[t - 1] if e >= 0}), t - 1)
        routed = sorted({int(e) for e in row if e >= 0})
        resident = {occupant[s]: s for s in range(S) if occupant[s] is not None}
        h = sum(e in resident for e in routed)
        m = len(routed) - h
        for e in routed:  # every resident expert of the step is fresh first
            if e in resident:
                stamp[resident[e]] = t
        promoted = 0
        for e in routed:
            if e in resident or promoted == max_promote:
                continue
            free = [s for s in range(P, S) if occupant[s] is None]
            if free:
                s = free[0]
            elif S > P:
                s = min(range(P, S), key=lambda k: (stamp[k], k))
            else:
                continue
            occupant[s] = e
            stamp[s] = t
            promoted += 1
        hits.append(h)
        misses.append(m)
    slot_of = np.full(E, -1, np.int32)
    for s in range(S):
        if occupant[s] is not None:
            slot_of[occupant[s]] = s
    return np.array(hits), np.array(misses), slot_of


def zipf_steps(rng, E, K, n_steps, a=1.1):
    p = 1.0 / np.arange(1, E + 1) ** a
    p /= p.sum()
    perm = rng.permutation(E)
    return np.stack([perm[rng.choice(E, K, replace=False, p=p)] for _ in range(n_steps)])


@pytest.mark.parametrize("E,S,P,K,mp", [(8, 3, 1, 2, 2), (64, 16, 4, 8, 2), (256, 64, 16, 8, 1),
                                        (256, 128, 0, 8, 8), (32, 32, 8, 4, 4)])
def test_simulator_matches_model(E, S, P, K, mp):
    rng = np.random.default_rng(E + S + P)
    steps = zipf_steps(rng, E, K, 300)
    steps[rng.random(steps.shape) < 0.1] = -1  # top-p drops
    usage = np.bincount(zipf_steps(rng, E, K, 50).ravel(), minlength=E).astype(np.uint64)
    for u in (None, usage):
        got = moe.cache_simulate(E, S, P, mp, steps, usage=u)
        want = model(E, S, P, mp, steps, usage=u)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_cyclic_pattern_defeats_lru():
    """One more expert than LRU slots, visited in a cycle: every access
    misses (the LRU victim is always the next one needed)."""
    E, S = 16, 5
    steps = np.array([[e % (S + 1)] for e in range(60)], np.int32)
    hits, misses, _ = moe.cache_simulate(E, S, 0, 1, steps)
    assert hits.sum() == 0 and misses.sum() == 60


def test_large_cache_misses_each_expert_once():
    rng = np.random.default_rng(3)
    steps = zipf_steps(rng, 64, 8, 200)
    hits, misses, slot_of = moe.cache_simulate(64, 64, 0, 8, steps)
    assert misses.sum() == np.unique(steps).size
    assert np.array_equal(np.sort(slot_of[slot_of >= 0]), np.arange(np.unique(steps).size))


def test_no_slots_all_misses_and_counts_add_up():
    rng = np.random.default_rng(4)
    steps = zipf_steps(rng, 32, 4, 50)
    hits, misses, slot_of = moe.cache_simulate(32, 0, 0, 2, steps)
    assert hits.sum() == 0 and np.all(slot_of == -1)
    assert np.array_equal(misses, [np.unique(r).size for r in steps])


def test_pinned_experts_stay_and_always_hit():
    rng = np.random.default_rng(5)
    E, S, P = 64, 12, 6
    usage = np.zeros(E, np.uint64)
    hot = [3, 9, 17, 22, 40, 41]
    usage[hot] = [50, 40, 30, 20, 10, 5]
    steps = zipf_steps(rng, E, 6, 200)
    steps[:, 0] = np.array(hot)[np.arange(200) % 6]
    hits, misses, slot_of = moe.cache_simulate(E, S, P, 3, steps, usage=usage)
    assert [slot_of[e] for e in hot] == list(range(6))
    total = np.array([np.unique(r).size for r in steps])
    assert np.all(hits >= 1) and np.array_equal(hits + misses, total)


def predictions(rng, steps, E, right=0.7):
    """Each entry of the true routing kept with probability `right`, else a
    random expert (or -1)."""
    pred = steps.copy()
    wrong = rng.random(steps.shape) >= right
    pred[wrong] = rng.integers(-1, E, size=int(wrong.sum()))
    return pred


@pytest.mark.parametrize("E,S,P,K,mp", [(8, 3, 1, 2, 2), (64, 16, 4, 8, 2), (256, 64, 16, 8, 1),
                                        (256, 128, 0, 8, 8), (32, 32, 8, 4, 4)])
def test_simulator_with_prefetch_matches_model(E, S, P, K, mp):
    rng = np.random.default_rng(7 * E + S + P)
    steps = zipf_steps(rng, E, K, 300)
    steps[rng.random(steps.shape) < 0.1] = -1
    pred = predictions(rng, steps, E)
    usage = np.bincount(zipf_steps(rng, E, K, 50).ravel(), minlength=E).astype(np.uint64)
    for u in (None, usage):
        got = moe.cache_simulate(E, S, P, mp, steps, usage=u, pred=pred)
        want = model(E, S, P, mp, steps, usage=u, pred_steps=pred)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_exact_prediction_never_misses():
    """Predictions equal to the routing, room for a step's experts and a
    promotion budget that covers them: every routed expert is resident when
    its step runs, however the routing moves."""
    rng = np.random.default_rng(3)
    E, K = 64, 8
    steps = np.stack([rng.choice(E, K, replace=False) for _ in range(100)]).astype(np.int32)
    hits, misses, _ = moe.cache_simulate(E, K, 0, K, steps, pred=steps)
    assert misses.sum() == 0 and hits.sum() == steps.size
    # without the prediction the same cache misses nearly every time
    hits0, misses0, _ = moe.cache_simulate(E, K, 0, K, steps)
    assert misses0.sum() > steps.size // 2


def test_prefetch_keeps_predicted_residents():
    """Two LRU slots hold experts 1 and 2; a prediction of {1, 3} brings 3
    into the slot of 2 (the only one not predicted), never into 1's, even
    though both slots were last used at the same step."""
    steps = np.array([[1, 2], [1, 3]], np.int32)
    pred = np.array([[1, 2], [1, 3]], np.int32)
    hits, misses, slot_of = moe.cache_simulate(8, 2, 0, 2, steps, pred=pred)
    assert hits.tolist() == [2, 2] and misses.tolist() == [0, 0]
    assert slot_of[1] == 0 and slot_of[3] == 1 and slot_of[2] == -1


def test_wrong_prediction_changes_only_residency():
    """Predictions of experts never routed: they take LRU slots (so later
    steps can lose hits) but hits + misses still count each routed expert
    once per step."""
    rng = np.random.default_rng(4)
    E, K = 32, 4
    steps = zipf_steps(rng, E, K, 200)
    pred = (steps + 16) % E  # a different expert for every entry
    hits, misses, _ = moe.cache_simulate(E, 12, 2, 2, steps, pred=pred)
    routed = np.array([len(set(r.tolist())) for r in steps])
    assert np.array_equal(hits + misses, routed)


def test_prefetch_helps_a_near_prediction():
    """A prediction right most of the time (70 %, as the pages report for
    routing one layer ahead) raises the hit count of the same cache."""
    rng = np.random.default_rng(5)
    E, K, S = 256, 8, 64
    steps = zipf_steps(rng, E, K, 400)
    pred = predictions(rng, steps, E, right=0.7)
    h0, _, _ = moe.cache_simulate(E, S, 0, 2, steps)
    h1, _, _ = moe.cache_simulate(E, S, 0, 2, steps, pred=pred)
    assert h1.sum() > h0.sum()
