"""Host model of the decode work split (no GPU): the 32-token steps of all (sequence, KV head)
segments form one line cut into equal worker ranges; a worker's first piece writes slot 2w,
its last piece (if different) slot 2w+1, whole segments write no partial. This checks that the
merge rule -- visit the non-empty workers from worker_of(first step) to worker_of(last step),
taking slot 2w+1 for the first one unless the segment starts its range -- finds exactly the
slots that were written, for many segment-length mixes and worker counts (including more
workers than steps)."""
import random


def range_begin(N, n, w):
    return N * w // n


def worker_of(N, n, r):
    return ((r + 1) * n - 1) // N


def pieces_written(ns, Hkv, n):
    P = [0]
    for x in ns:
        P.append(P[-1] + x)
    N = Hkv * P[-1]
    written, whole = {}, set()
    for w in range(n):
        R0, R1 = range_begin(N, n, w), range_begin(N, n, w + 1)
        r = R0
        while r < R1:
            s = max(i for i in range(len(ns)) if Hkv * P[i] <= r and P[i + 1] > P[i])
            g, k = divmod(r - Hkv * P[s], ns[s])
            seg_end = Hkv * P[s] + (g + 1) * ns[s]
            end = min(R1, seg_end)
            if k == 0 and end == seg_end:
                whole.add((s, g))
            else:
                written.setdefault((s, g), []).append(2 * w + (0 if r == R0 else 1))
            r = end
    return P, N, written, whole


def merge_visits(P, N, n, Hkv, ns, s, g):
    G0 = Hkv * P[s] + g * ns[s]
    wf, wl = worker_of(N, n, G0), worker_of(N, n, G0 + ns[s] - 1)
    if wf == wl:
        return None
    first = 2 * wf + (1 if G0 != range_begin(N, n, wf) else 0)
    return [first if w == wf else 2 * w for w in range(wf, wl + 1)
            if range_begin(N, n, w + 1) != range_begin(N, n, w)]


def test_merge_visits_exactly_the_written_slots():
    rnd = random.Random(0)
    for _ in range(2000):
        S, Hkv = rnd.randint(1, 8), rnd.randint(1, 4)
        ns = [rnd.choice([0, 1, 2, 3, 5, 17, 64]) for _ in range(S)]
        if sum(ns) == 0:
            continue
        n = rnd.choice([1, 2, 3, 7, 31, 50, 1000])
        P, N, written, whole = pieces_written(ns, Hkv, n)
        for s in range(S):
            for g in range(Hkv):
                if ns[s] == 0:
                    continue
                v = merge_visits(P, N, n, Hkv, ns, s, g)
                if v is None:
                    assert (s, g) in whole and (s, g) not in written
                else:
                    assert (s, g) not in whole
                    assert sorted(v) == sorted(written[(s, g)])
        # every slot is written at most once, and only slots 2w / 2w+1 of real workers
        slots = [x for v in written.values() for x in v]
        assert len(slots) == len(set(slots)) and all(0 <= x < 2 * n for x in slots)


def test_ranges_are_balanced():
    for N, n in ((59000, 1024), (7, 3), (186, 2048), (10 ** 9, 2048)):
        sizes = [range_begin(N, n, w + 1) - range_begin(N, n, w) for w in range(n)]
        assert sum(sizes) == N and max(sizes) - min(sizes) <= 1
