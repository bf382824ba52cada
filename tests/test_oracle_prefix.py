"""Pins for oracle/prefix.py (shared-prefix grouping) by brute force over all
pairs of sequences, plus one hand-worked case."""
import numpy as np
import pytest

from oracle import prefix as P


def _cases():
    for seed in range(40):
        r = np.random.default_rng(seed)
        vocab = int(r.integers(2, 5))
        seqs = []
        for _ in range(int(r.integers(0, 25))):
            if seqs and r.random() < 0.5:      # plant a family member: copy a prefix of an earlier one
                src = seqs[int(r.integers(len(seqs)))]
                k = int(r.integers(0, len(src) + 1))
                tail = r.integers(0, vocab, int(r.integers(0, 6))).tolist()
                s = src[:k] + tail
                if not s:
                    s = [0]
            else:
                s = r.integers(0, vocab, int(r.integers(1, 9))).tolist()
            seqs.append(s)
        keys = None if seed % 4 == 0 else r.integers(-1, 3, len(seqs)).tolist()
        yield seqs, keys, int(r.choice([1, 2, 3, 5]))


def test_hand_worked_case():
    seqs = [[1, 2, 3, 4], [1, 2, 3, 5], [1, 2, 9], [7, 7], [1, 2, 3, 4, 6]]
    # one key: 0, 1, 2, 4 share [1, 2] (LCP 2); [7, 7] stands alone
    g, f, ln = P.prefix_groups_reference(seqs, None, 2)
    assert g.tolist() == [0, 0, 0, -1, 0] and f.tolist() == [0] and ln.tolist() == [2]
    # sequence 2 under another key: 0, 1, 4 share [1, 2, 3]; its shortest member
    # has 4 tokens, so the node keeps 3 and every member keeps >= 1
    g, f, ln = P.prefix_groups_reference(seqs, [0, 0, 1, 0, 0], 2)
    assert g.tolist() == [0, 0, -1, -1, 0] and f.tolist() == [0] and ln.tolist() == [3]
    # identical sequences: the node stops one token short of their end
    g, f, ln = P.prefix_groups_reference([[5, 6, 7], [5, 6, 7]], None, 1)
    assert g.tolist() == [0, 0] and ln.tolist() == [2]
    # min_len equal to a member's length: that member cannot keep a token
    g, _, _ = P.prefix_groups_reference([[5, 6], [5, 6, 7], [5, 6, 8]], None, 2)
    assert g.tolist() == [-1, 0, 0]


@pytest.mark.parametrize("case", list(_cases()))
def test_grouping_by_brute_force(case):
    seqs, keys, m = case
    g, first, ln = P.prefix_groups_reference(seqs, keys, m)
    n = len(seqs)
    key = [0 if keys is None else keys[i] for i in range(n)]
    cand = [key[i] >= 0 and len(seqs[i]) > m for i in range(n)]
    # exactly: same group <=> both candidates, same key, same first m tokens
    for i in range(n):
        if not cand[i]:
            assert g[i] == -1
        for j in range(i + 1, n):
            same = cand[i] and cand[j] and key[i] == key[j] and seqs[i][:m] == seqs[j][:m]
            assert (g[i] >= 0 and g[i] == g[j]) == same, (i, j)
    # a candidate with no partner stays alone
    for i in range(n):
        if cand[i] and g[i] < 0:
            assert not any(cand[j] and j != i and key[j] == key[i] and seqs[j][:m] == seqs[i][:m]
                           for j in range(n))
    # numbering and node contents
    assert list(first) == sorted(first)
    for k in range(len(first)):
        mem = [i for i in range(n) if g[i] == k]
        assert len(mem) >= 2 and first[k] == min(mem)
        L = int(ln[k])
        assert L >= m
        head = seqs[first[k]][:L]
        assert all(seqs[i][:L] == head and len(seqs[i]) > L for i in mem)
        # maximal: one more token would either leave a member empty or not be shared
        longer_ok = all(len(seqs[i]) > L + 1 for i in mem) and \
            len({seqs[i][L] for i in mem}) == 1
        assert not longer_ok


def test_tree_hand_worked_case():
    seqs = [[1, 2, 3, 4, 5, 6, 7], [1, 2, 3, 4, 5, 6, 8], [1, 2, 3, 9, 9, 9, 9], [1, 2, 3, 9, 9, 9, 1],
            [1, 2, 3, 7], [5, 5]]
    g, nodes = P.prefix_tree_reference(seqs, None, 2)
    # [1 2 3] for the first five; [4 5 6] and [9 9 9] below it; [1 2 3 7] stays at the top node
    assert nodes == [(-1, 0, 0, 3), (0, 0, 3, 6), (0, 2, 3, 6)]
    assert g.tolist() == [1, 1, 2, 2, 0, -1]
    # with min_len 4 the top-level cut already separates the two families
    g, nodes = P.prefix_tree_reference(seqs, None, 4)
    assert nodes == [(-1, 0, 0, 6), (-1, 2, 0, 6)] and g.tolist() == [0, 0, 1, 1, -1, -1]
    # a part whose extra shared run is shorter than min_len stays with its parent
    abc = [[1, 2, 3, 4, 5, 7], [1, 2, 3, 4, 5, 8], [1, 2, 3, 9, 0]]
    g, nodes = P.prefix_tree_reference(abc, None, 3)
    assert nodes == [(-1, 0, 0, 3)] and g.tolist() == [0, 0, 0]
    g, nodes = P.prefix_tree_reference(abc, None, 2)
    assert nodes == [(-1, 0, 0, 3), (0, 0, 3, 5)] and g.tolist() == [1, 1, 0]


@pytest.mark.parametrize("case", list(_cases()))
@pytest.mark.parametrize("m", [1, 2])
def test_tree_by_brute_force(case, m):
    seqs, keys, _ = case
    g, nodes = P.prefix_tree_reference(seqs, keys, m)
    n = len(seqs)
    g1, f1, l1 = P.prefix_groups_reference(seqs, keys, m)
    roots = [k for k, x in enumerate(nodes) if x[0] < 0]
    assert [nodes[k][1] for k in roots] == list(f1) and [nodes[k][3] for k in roots] == list(l1)

    def subtree(k):
        out = {i for i in range(n) if g[i] == k}
        for c, x in enumerate(nodes):
            if x[0] == k:
                out |= subtree(c)
        return out

    for k, (par, first, start, end) in enumerate(nodes):
        assert par < k                                              # parents first
        mem = sorted(subtree(k))
        assert len(mem) >= 2 and first == mem[0]
        assert start == (nodes[par][3] if par >= 0 else 0)
        assert end >= start + m
        head = seqs[first][:end]
        assert all(seqs[i][:end] == head and len(seqs[i]) > end for i in mem)
        longer = all(len(seqs[i]) > end + 1 for i in mem) and len({seqs[i][end] for i in mem}) == 1
        assert not longer                                           # end is the cut common prefix
        # each next-token part is a child exactly when it qualifies
        parts = {}
        for i in mem:
            parts.setdefault(seqs[i][end], []).append(i)
        kids = {nodes[c][1]: c for c, x in enumerate(nodes) if x[0] == k}
        for part in parts.values():
            cut = min(min(len(seqs[i]) for i in part) - 1,
                      next((t for t in range(len(seqs[part[0]]))
                            if any(t >= len(seqs[i]) or seqs[i][t] != seqs[part[0]][t] for i in part)),
                           len(seqs[part[0]])))
            qualifies = len(part) >= 2 and cut >= end + m
            assert qualifies == (min(part) in kids and sorted(subtree(kids[min(part)])) == sorted(part))
