"""The rule by which the merge launch picks its threads when some pattern
has dilation 1 (every position is then gathered): patterns are ranked by
dilation, a row with two or more covering patterns is merged by the thread
that enumerates it as a gathered row of its second covering pattern, and a
pattern is not enumerated when two patterns ranked before it gather all of
its rows (r_i | r_j, r_j | w'_j, r_i | w'_i). Checked here by brute force
over small geometries: every row that needs a merge is claimed exactly
once and no other row is claimed. Gathering follows the segment / dilation
/ head-offset construction of the LongNet blog ("LongNet's attention
allocation principle" and the multi-head paragraph after it)."""
import random

import pytest


def enumeration(N, patterns):
    P = [(min(w, N), r) for (w, r) in patterns]
    order = sorted(range(len(P)), key=lambda i: (P[i][1], i))
    rank = {i: k for k, i in enumerate(order)}

    def covers(i, j):
        return P[j][1] % P[i][1] == 0 and P[j][0] % P[j][1] == 0 and P[i][0] % P[i][1] == 0

    enum = [order[k] for k in range(1, len(P))
            if sum(covers(order[q], order[k]) for q in range(k)) < 2]
    return P, rank, enum


def claimed_rows(N, H, patterns):
    P, rank, enum = enumeration(N, patterns)
    claimed = {}
    for h in range(H):
        for j in enum:
            wp, r = P[j]
            off = h % r
            for s in range(N // wp):
                for m in range(-(-wp // r)):
                    if off + m * r >= wp:
                        continue
                    t = s * wp + off + m * r
                    cover = [i for i, (w2, r2) in enumerate(P) if (t % w2) % r2 == h % r2]
                    assert j in cover
                    if sum(rank[i] < rank[j] for i in cover) == 1:
                        assert (t, h) not in claimed
                        claimed[(t, h)] = j
    return claimed


def needs_merge(N, H, patterns):
    rows = set()
    for h in range(H):
        for t in range(N):
            c = sum(((t % min(w, N)) % r) == h % r for (w, r) in patterns)
            if c >= 2:
                rows.add((t, h))
    return rows


def cases():
    out = [
        (600, 3, [(600, 1), (200, 3), (300, 2)]),
        (256, 5, [(64, 1), (64, 1), (256, 4)]),
        (1020, 4, [(1020, 3), (510, 1), (204, 5)]),
        (512, 3, [(512, 1), (256, 2), (128, 4), (64, 8), (512, 8), (256, 1), (128, 2), (64, 1)]),
        (96, 4, [(1000, 7), (8, 1), (96, 96)]),
        (480, 6, [(480, 6), (160, 1), (96, 2)]),
        (2048, 16, [(256, 1), (512, 2), (1024, 4), (2048, 8), (2048, 16)]),
    ]
    rng = random.Random(7)
    for _ in range(150):
        N = rng.choice([24, 36, 48, 60, 72, 96, 120])
        divs = [d for d in range(1, N + 1) if N % d == 0]
        n = rng.randint(2, 5)
        pats = [(rng.choice(divs + [2 * N]), rng.randint(1, 9)) for _ in range(n)]
        pats[rng.randrange(n)] = (rng.choice(divs), 1)
        out.append((N, rng.randint(1, 6), pats))
    return out


@pytest.mark.parametrize("N,H,patterns", cases())
def test_every_row_needing_a_merge_is_claimed_once(N, H, patterns):
    assert set(claimed_rows(N, H, patterns)) == needs_merge(N, H, patterns)


def test_nested_dilations_enumerate_one_pattern():
    # dilations 1, 2, 4, ... with segment lengths they divide: only the r = 2
    # pattern can be a second cover
    _, _, enum = enumeration(32768, [(2048, 1), (4096, 2), (8192, 4), (16384, 8), (32768, 16)])
    assert enum == [1]
