"""Shared suffix prefixes: which suffixes share a prefix node -- the reference
semantics. TEST INFRASTRUCTURE ONLY (see the package header).

[pt] "Futuro e método" lists a radix index for prefix sharing among the
authors' future work; [fa] (body) names the one workload where the engine
loses to vLLM: agent traces, whose documents share prefixes the current model
cannot exploit. Neither page says how sharing is to be chosen.

Reading taken (the plainest one-level rule): among the suffixes of one anchor,
those whose first ``min_len`` tokens are equal form a group when there are at
least two of them and each is longer than ``min_len``. A group's node is the
members' longest common prefix, shortened where needed so that every member
keeps at least one token of its own (the head reads a suffix's last
position). Groups are numbered by their smallest member. A suffix with no
anchor (a filter row) is never grouped: a node continues an anchor.

Computed here by hashing the first ``min_len`` tokens and comparing members
token by token -- a different route from the library's sorted radix order.

Pins (tests/test_oracle_prefix.py): on random cases with planted families,
brute force over all pairs checks that grouping is exactly "same key and same
first min_len tokens", that each node's tokens are a prefix of every member,
that the node length is maximal under the one-token rule, and the numbering.
The two-level attention identity is pinned in tests/test_oracle_attention.py.
"""
from __future__ import annotations

import numpy as np


def prefix_groups_reference(seqs, keys, min_len):
    """seqs: list of 1-D int sequences; keys: per-sequence key (negative = not
    grouped) or None (one key). Returns (group_of [n], node_first, node_len)."""
    n = len(seqs)
    classes = {}
    for i, s in enumerate(seqs):
        k = 0 if keys is None else int(keys[i])
        if k < 0 or len(s) <= min_len:
            continue
        classes.setdefault((k, tuple(int(x) for x in s[:min_len])), []).append(i)
    nodes = []
    for members in classes.values():
        if len(members) < 2:
            continue
        first = min(members)
        ref = [int(x) for x in seqs[first]]
        common = len(ref)
        for m in members:
            s = [int(x) for x in seqs[m]]
            k = 0
            while k < min(common, len(s)) and s[k] == ref[k]:
                k += 1
            common = k
        shortest = min(len(seqs[m]) for m in members)
        nodes.append((first, min(common, shortest - 1), sorted(members)))
    nodes.sort()
    group_of = np.full(n, -1, np.int32)
    for g, (_, _, members) in enumerate(nodes):
        group_of[members] = g
    return (group_of, np.array([x[0] for x in nodes], np.int32),
            np.array([x[1] for x in nodes], np.int32))


def prefix_tree_reference(seqs, keys, min_len):
    """Nested shared prefixes (reading): the groups of ``prefix_groups_reference``
    are the top level; inside a node that covers tokens [.., l) its members are
    split by their token at position l, and a part of two or more whose own
    common prefix (cut to leave each member a token) reaches l + min_len
    becomes a child node covering [l, l'), recursively; everyone else stays a
    direct member of the node.

    Returns (group_of [n] = deepest node of each sequence or -1, nodes = list
    of (parent node or -1, smallest member, start, end)) with nodes numbered
    parents first: top-level nodes by smallest member, each followed by its
    subtree, children by smallest member."""
    n = len(seqs)
    group_of = np.full(n, -1, np.int32)
    nodes = []

    def lcp_cut(members):
        ref = [int(x) for x in seqs[members[0]]]
        common = len(ref)
        for m in members[1:]:
            s = [int(x) for x in seqs[m]]
            k = 0
            while k < min(common, len(s)) and s[k] == ref[k]:
                k += 1
            common = k
        return min(common, min(len(seqs[m]) for m in members) - 1)

    def build(members, parent, start):
        end = lcp_cut(members)
        me = len(nodes)
        nodes.append((parent, min(members), start, end))
        for m in members:
            group_of[m] = me
        parts = {}
        for m in members:
            parts.setdefault(int(seqs[m][end]), []).append(m)
        for part in sorted(parts.values(), key=min):
            if len(part) >= 2 and lcp_cut(part) >= end + min_len:
                build(part, me, end)

    g1, firsts, _ = prefix_groups_reference(seqs, keys, min_len)
    for k in range(len(firsts)):
        build(sorted(np.flatnonzero(g1 == k).tolist()), -1, 0)
    return group_of, nodes
