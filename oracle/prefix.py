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
