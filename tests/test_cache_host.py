"""CPU checks of the expert cache's slot assignment (moe_lru_simulate runs the
library's own LRU on the host) against a textbook least-recently-used model
written here: within a batch the keys already resident are touched first,
then each missing key takes the least recently used slot not used by the
batch (lowest index among equals, never-used slots first)."""
import numpy as np
import pytest

import routing_quant_expert_amd as R


def textbook_lru(n_slots, batches):
    slot_of, key_of = {}, [None] * n_slots
    last, epoch = [0] * n_slots, [0] * n_slots
    clock = 0
    out = []
    for b, keys in enumerate(batches, 1):
        res = [None] * len(keys)
        for i, k in enumerate(keys):
            if k in slot_of:
                clock += 1
                s = slot_of[k]
                last[s], epoch[s] = clock, b
                res[i] = (s, 0)
        for i, k in enumerate(keys):
            if res[i] is not None:
                continue
            if k in slot_of:            # a repeat of a key placed earlier in this batch
                clock += 1
                s = slot_of[k]
                last[s], epoch[s] = clock, b
                res[i] = (s, 0)
                continue
            free = [s for s in range(n_slots) if epoch[s] != b]
            if not free:
                res[i] = (-1, 1)
                continue
            s = min(free, key=lambda j: (last[j], j))
            if key_of[s] is not None:
                del slot_of[key_of[s]]
            key_of[s], slot_of[k] = k, s
            clock += 1
            last[s], epoch[s] = clock, b
            res[i] = (s, 1)
        out += res
    return [r[0] for r in out], [r[1] for r in out]


@pytest.mark.parametrize("n_slots", [1, 3, 8, 20])
def test_lru_matches_textbook_model(n_slots):
    rng = np.random.default_rng(n_slots)
    n_keys = 40
    batches = []
    for _ in range(300):
        size = int(rng.integers(1, n_slots + 3))
        keys = rng.choice(n_keys, size=min(size, n_keys), replace=False).tolist()
        if rng.random() < 0.2 and keys:
            keys.append(keys[0])         # a repeated key inside a batch
        batches.append(keys)
    slots, miss = R.lru_simulate(n_slots, n_keys, batches)
    ws, wm = textbook_lru(n_slots, batches)
    assert list(slots) == ws and list(miss) == wm
    # every key of a batch that found a slot holds it at the batch's end, no two keys share one
    q = 0
    for keys in batches:
        got = {}
        for k in keys:
            if slots[q] >= 0:
                assert got.get(k, slots[q]) == slots[q]
                got[k] = slots[q]
            q += 1
        assert len(set(got.values())) == len(got)


def test_lru_hits_after_warm_batch_and_capacity():
    slots, miss = R.lru_simulate(4, 10, [[1, 2, 3, 4], [4, 3, 2, 1], [5, 6, 7, 8, 9]])
    assert list(miss[:4]) == [1, 1, 1, 1] and list(miss[4:8]) == [0, 0, 0, 0]
    assert list(slots[4:8]) == [3, 2, 1, 0]
    # a batch of five distinct keys does not fit four slots: the fifth gets none
    assert list(slots[8:12]) != [-1] * 4 and slots[12] == -1


def test_lru_rejects_bad_arguments():
    with pytest.raises(R.MoeError):
        R.lru_simulate(0, 10, [[1]])
    with pytest.raises(R.MoeError):
        R.lru_simulate(2, 10, [[11]])
