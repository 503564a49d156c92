"""Host logic of a decode step (CPU only, no device call): the merge of the
selection's per-head promotion runs into one set of copies per KV-head group.

Each query head of a group lists its own top-K* blocks as runs; the group's
blocks to copy are the union (U_g).  The merged entries must cover exactly
the union of every (kind, group)'s runs, as maximal disjoint runs (adjacent
runs joined, so no block is copied twice and no copy is split needlessly),
in (kind, group, start) order."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def kvq():
    import certified_quantized_kv_amd as m
    return m


def enc(kind, group, start, length):
    return length | (start << 16) | (group << 32) | (kind << 48)


def reference(entries):
    cover = {}
    for e in entries:
        length, start = e & 0xFFFF, (e >> 16) & 0xFFFF
        key = (e >> 48, (e >> 32) & 0xFFFF)
        cover.setdefault(key, set()).update(range(start, start + length))
    out = []
    for key in sorted(cover):
        blocks = sorted(cover[key])
        s = p = blocks[0]
        for b in blocks[1:] + [None]:
            if b is not None and b == p + 1:
                p = b
                continue
            out.append(enc(key[0], key[1], s, p + 1 - s))
            if b is not None:
                s = p = b
    return out


def test_merge_cases(kvq):
    cases = [
        [],
        [enc(0, 3, 10, 5)],
        [enc(0, 0, 0, 4), enc(0, 0, 4, 4)],                       # adjacent -> one run
        [enc(0, 1, 5, 10), enc(0, 1, 0, 20), enc(0, 1, 7, 1)],      # nested
        [enc(0, 2, 0, 3), enc(0, 2, 5, 3)],                       # gap of two blocks stays
        [enc(1, 0, 0, 8), enc(0, 0, 0, 8)],                       # kinds stay apart
        [enc(0, 7, 2048, 1), enc(0, 6, 0, 2049)],                 # groups stay apart
    ]
    for c in cases:
        got = [int(x) for x in kvq.merge_runs(c)]
        assert got == reference(c), c


def test_merge_random_selections(kvq):
    """Four heads per group, each selecting most blocks of a 2049-block
    sequence (as top-K* does on near-uniform attention), runs listed per head
    and shuffled across heads and groups, as the atomics leave them."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        nb = int(rng.integers(1, 2050))
        ents = []
        for g in range(int(rng.integers(1, 9))):
            for h in range(4):
                sel = rng.random(nb) < rng.choice([0.3, 0.9, 0.995, 1.0])
                b = 0
                while b < nb:
                    if not sel[b]:
                        b += 1
                        continue
                    e = b
                    while e < nb and sel[e]:
                        e += 1
                    ents.append(enc(0, g, b, e - b))
                    b = e
            if rng.random() < 0.3:
                ents.append(enc(1, g, int(rng.integers(0, nb)), 1))
        rng.shuffle(ents)
        got = [int(x) for x in kvq.merge_runs(ents)]
        ref = reference(ents)
        assert got == ref, trial
        # every block of the union once: lengths add up to the union's size
        total = sum(e & 0xFFFF for e in ents if not (e >> 48))
        assert sum(e & 0xFFFF for e in got if not (e >> 48)) <= total


def test_merge_rejects_malformed(kvq):
    for bad in ([enc(0, 0, 3, 0)], [enc(0, 0, 0xFFF0, 0x20)], [enc(2, 0, 0, 1)]):
        with pytest.raises(kvq.KvqError):
            kvq.merge_runs(bad)
