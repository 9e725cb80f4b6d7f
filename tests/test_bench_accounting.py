"""The benchmark's algorithmic-work accounting, against brute force on tiny cases (CPU).

The roofline fractions the benchmark reports divide these counts by measured times,
so they are checked here by enumerating the key sets position by position.
"""
import random

import torch

import bench


def _local_keys(i, window, n_sink):
    # keys of row i of a local head: the last `window` causal positions and the sinks
    return set(range(max(0, i - window + 1), i + 1)) | set(range(min(n_sink, i + 1)))


def test_local_key_total_matches_enumeration():
    for L, window, n_sink in [(1, 4, 2), (3, 4, 2), (4, 4, 2), (5, 4, 2), (37, 8, 3), (100, 16, 4), (10, 16, 4),
                              (50, 1, 0), (50, 1, 5), (64, 64, 4), (65, 64, 4), (200, 7, 100)]:
        want = sum(len(_local_keys(i, window, n_sink)) for i in range(L))
        assert bench.local_key_total(L, window, n_sink) == want, (L, window, n_sink)


def test_decode_union_rows_matches_enumeration():
    rng = random.Random(1234)
    for trial in range(20):
        batch = rng.randint(1, 4)
        lens = [rng.randint(1, 60) for _ in range(batch)]
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        n_slots = rng.randint(1, 3)
        window, n_sink = rng.randint(1, 20), rng.randint(0, 5)
        idx = torch.full((n_slots, cu[-1]), -1, dtype=torch.int32)
        counts = torch.zeros((n_slots, batch), dtype=torch.int64)
        members = {}
        for r in range(n_slots):
            for b, L in enumerate(lens):
                m = sorted(rng.sample(range(L), rng.randint(0, L)))
                members[r, b] = set(m)
                counts[r, b] = len(m)
                idx[r, cu[b]:cu[b] + len(m)] = torch.tensor(m, dtype=torch.int32)
        # KV groups: some with local heads, retrieval slots dealt over them (a group may have none)
        n_groups = rng.randint(1, 3)
        groups = [(rng.random() < 0.5, []) for _ in range(n_groups)]
        for r in range(n_slots):
            groups[rng.randrange(n_groups)][1].append(r)
        want = 0
        for has_local, slots in groups:
            for b, L in enumerate(lens):
                rows = set()
                if has_local:
                    rows |= set(range(max(0, L - window), L)) | set(range(min(n_sink, L)))
                for r in slots:
                    rows |= members[r, b]
                want += len(rows)
        got = bench.decode_union_rows(torch, lens, cu, counts, idx, window, n_sink, groups)
        assert got == want, trial
