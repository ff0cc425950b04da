"""Host model of the decode work split (no GPU).

The 32-token steps of all (sequence, KV head) segments form one line. Each step weighs 4 and
each segment start weighs piece_weight more (a mark before its first step); worker w owns the
steps whose weighted start lies in [Nw * w / n, Nw * (w + 1) / n). The first piece of a range
writes slot 2w, its last piece (if different) slot 2w+1, whole segments write no partial.

This checks, for many length mixes, worker counts (including more workers than steps) and
piece weights, that the ranges tile the line, that the merge rule finds exactly the slots that
were written, and that the weighted cut balances steps + pieces. It also models the
wave-parallel sequence search (two ballot rounds of 64 candidates)."""
import bisect
import random

STEP_W = 4


def ceil_div(a, b):
    return -(-a // b)


class Line:
    def __init__(self, ns, Hkv, pw, n):
        self.ns, self.Hkv, self.pw, self.n = ns, Hkv, pw, n
        self.P, self.Wp = [0], [0]
        for x in ns:
            self.P.append(self.P[-1] + x)
            self.Wp.append(self.Wp[-1] + STEP_W * x + (pw if x > 0 else 0))
        self.N, self.Nw = Hkv * self.P[-1], Hkv * self.Wp[-1]

    def wbegin(self, w):
        return self.Nw * w // self.n

    def owner(self, x):
        return ((x + 1) * self.n - 1) // self.Nw

    def in_segment_before(self, x, ws0, ns):
        off = x - ws0 - self.pw
        return 0 if off <= 0 else min(ns, ceil_div(off, STEP_W))

    def steps_before(self, x):
        if x >= self.Nw:
            return self.N
        s = max(i for i in range(len(self.ns)) if self.Hkv * self.Wp[i] <= x)
        ns = self.ns[s]
        seg_w = STEP_W * ns + self.pw
        g = (x - self.Hkv * self.Wp[s]) // seg_w
        return self.Hkv * self.P[s] + g * ns + \
            self.in_segment_before(x, self.Hkv * self.Wp[s] + g * seg_w, ns)


def segments(line):
    """(s, g, first step index, ns) in line order."""
    out = []
    for s, ns in enumerate(line.ns):
        for g in range(line.Hkv):
            if ns:
                out.append((s, g, line.Hkv * line.P[s] + g * ns, ns))
    return out


def decode_writes(line):
    written, whole, cover = {}, set(), []
    segs = segments(line)
    for w in range(line.n):
        b0, end = line.steps_before(line.wbegin(w)), line.steps_before(line.wbegin(w + 1))
        cover.append((b0, end))
        x = b0
        while x < end:
            s, g, G0, ns = next(t for t in segs if t[2] <= x < t[2] + t[3])
            e = min(end, G0 + ns)
            if x == G0 and e == G0 + ns:
                whole.add((s, g))
            else:
                written.setdefault((s, g), []).append(2 * w + (0 if x == b0 else 1))
            x = e
    return written, whole, cover


def merge_reads(line, s, g):
    ns = line.ns[s]
    seg_w = STEP_W * ns + line.pw
    ws0 = line.Hkv * line.Wp[s] + g * seg_w
    first = ws0 + line.pw
    rf, rl = line.owner(first), line.owner(first + STEP_W * (ns - 1))
    if rf == rl:
        return None
    reads = [2 * rf + (0 if line.wbegin(rf) > ws0 - STEP_W else 1)]
    before = line.in_segment_before(line.wbegin(rf + 1), ws0, ns)
    for r in range(rf + 1, rl + 1):
        after = ns if r == rl else line.in_segment_before(line.wbegin(r + 1), ws0, ns)
        if after > before:
            reads.append(2 * r)
        before = after
    return reads


def test_merge_reads_exactly_the_written_slots():
    rnd = random.Random(0)
    for _ in range(1500):
        S, Hkv = rnd.randint(1, 8), rnd.randint(1, 4)
        ns = [rnd.choice([0, 1, 2, 3, 5, 17, 64]) for _ in range(S)]
        if sum(ns) == 0:
            continue
        line = Line(ns, Hkv, rnd.choice([0, 1, 4, 7, 64]), rnd.choice([1, 2, 3, 7, 31, 50, 1000]))
        written, whole, cover = decode_writes(line)
        assert cover[0][0] == 0 and cover[-1][1] == line.N       # ranges tile the line
        assert all(cover[i][1] == cover[i + 1][0] for i in range(line.n - 1))
        for s in range(S):
            for g in range(Hkv):
                if ns[s] == 0:
                    continue
                reads = merge_reads(line, s, g)
                if reads is None:
                    assert (s, g) in whole and (s, g) not in written
                else:
                    assert (s, g) not in whole
                    assert sorted(reads) == sorted(written[(s, g)])
        slots = [x for v in written.values() for x in v]
        assert len(slots) == len(set(slots)) and all(0 <= x < 2 * line.n for x in slots)


def test_weighted_cut_balances_steps_and_pieces():
    """Short and long sequences mixed: with piece weight 4 the per-worker cost steps + pieces
    (the model the weight encodes) varies by about one step at most, while a plain step cut
    lets it vary by the number of short sequences a range happens to hold."""
    rnd = random.Random(1)
    ns = [rnd.choice([1, 2, 3, 128]) for _ in range(200)]
    n = 64

    def spread(pw):
        line = Line(ns, 8, pw, n)
        written, whole, cover = decode_writes(line)
        segs = segments(line)
        costs = []
        for b0, end in cover:
            pieces = sum(1 for (_, _, G0, k) in segs if G0 < end and G0 + k > b0)
            costs.append((end - b0) + pieces)
        return max(costs) - min(costs)

    assert spread(4) <= 3
    assert spread(0) > 3 * spread(4)


def test_zero_piece_weight_is_an_equal_step_cut():
    """Piece weight 0: the ranges hold equal step counts, up to one step."""
    for ns, n in (([5, 7, 0, 9], 3), ([64] * 10, 7), ([1] * 50, 200), ([3, 0, 0, 1000], 64)):
        line = Line(ns, 2, 0, n)
        sizes = [line.steps_before(line.wbegin(w + 1)) - line.steps_before(line.wbegin(w))
                 for w in range(n)]
        assert sum(sizes) == line.N and max(sizes) - min(sizes) <= 1


def find_seq_ballot(prefix, S, Hkv, r):
    """The wave-parallel search: 64 candidates per round, the answer is (passing lanes) - 1."""
    stride = (S + 63) >> 6
    base, cnt = 0, S
    if stride > 1:
        ok = [stride * l < S and Hkv * prefix[stride * l] <= r for l in range(64)]
        base = stride * (sum(ok) - 1)
        cnt = min(S - base, stride)
    ok = [l < cnt and Hkv * prefix[base + l] <= r for l in range(64)]
    return base + sum(ok) - 1


def test_ballot_search_matches_bisection():
    rnd = random.Random(3)
    for S in (1, 2, 5, 63, 64, 65, 127, 128, 129, 255, 256, 1000, 4095, 4096):
        ns = [rnd.choice([0, 0, 1, 3, 40]) for _ in range(S)]
        ns[rnd.randrange(S)] += 1
        prefix = [0]
        for x in ns:
            prefix.append(prefix[-1] + x)
        Hkv = rnd.choice([1, 8])
        for r in list(range(0, min(Hkv * prefix[S], 300))) + \
                [rnd.randrange(Hkv * prefix[S]) for _ in range(300)]:
            want = bisect.bisect_right([Hkv * p for p in prefix[:S]], r) - 1
            assert find_seq_ballot(prefix, S, Hkv, r) == want
            assert ns[want] > 0          # the largest such s is a sequence with work
