"""Checks that pin the block-manager model to facts other than itself.

Each ``check_*`` takes a module exposing ``BlockManager`` and ``NoBlocks``
(the real ``oracle.block_manager`` or a mutant). The facts: a hand-worked
scenario (``tests/golden/block_manager_hand_worked.json``), invariants that
any correct pool must keep after every operation (reference counts equal the
number of tables holding a block; the free list holds exactly the unreferenced
blocks; a table covers its sequence; a block shared by two sequences sits under
identical token prefixes), maximal prefix reuse, re-admission after
preemption, and failures that leave the state untouched.
"""

from __future__ import annotations

import copy
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def replay_golden(make, check_refs=None):
    """Run the golden scenario on managers built by make(num_blocks, block_size)."""
    with open(os.path.join(GOLDEN, "block_manager_hand_worked.json"), encoding="utf-8") as f:
        g = json.load(f)
    bm = make(g["num_blocks"], g["block_size"])
    for i, s in enumerate(g["steps"]):
        op = s["op"]
        if op == "reset":
            bm = make(g["num_blocks"], g["block_size"])
            continue
        if op == "allocate":
            assert bm.allocate(s["seq"], s["tokens"]) == s["cached"], f"step {i}"
        elif op == "append":
            assert bm.append(s["seq"], s["token"]) == (not s.get("fails")), f"step {i}"
        elif op == "free":
            bm.free_seq(s["seq"])
        assert bm.tables() == s["tables"], f"step {i}: {bm.tables()}"
        assert bm.free_list() == s["free"], f"step {i}: {bm.free_list()}"
        if i == 9 and check_refs is not None:
            assert check_refs(bm) == g["final_refs_after_step_10"]


class _Model:
    """Uniform face over the oracle model (append returns success instead of raising)."""

    def __init__(self, orc, num_blocks, block_size, order=None):
        self.orc = orc
        self.m = orc.BlockManager(num_blocks, block_size, order)

    def allocate(self, seq, tokens):
        try:
            return self.m.allocate(seq, tokens)
        except self.orc.NoBlocks:
            return None

    def append(self, seq, token):
        try:
            self.m.append(seq, token)
            return True
        except self.orc.NoBlocks:
            return False

    def free_seq(self, seq):
        self.m.free_seq(seq)

    def tables(self):
        return {k: self.m.table(k) for k in self.m.seqs}

    def free_list(self):
        return list(self.m.free)


def check_golden(orc):
    replay_golden(lambda n, b: _Model(orc, n, b), check_refs=lambda bm: list(bm.m.ref))


def random_ops(rng, n_ops, prefixes, bs, apply):
    """Drive n_ops operations: allocations drawn from a few shared prefixes (with random
    tails), appends and frees. apply(op, seq, arg) returns False when the operation
    failed for lack of blocks; failed allocations leave no sequence behind."""
    live, nxt = [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.4 or not live:
            p = prefixes[rng.integers(len(prefixes))]
            cut = int(rng.integers(1, len(p) + 1))
            tail = rng.integers(0, 50, int(rng.integers(0, 3 * bs))).tolist()
            if apply("allocate", nxt, p[:cut] + tail):
                live.append(nxt)
            nxt += 1
        elif r < 0.85:
            apply("append", live[rng.integers(len(live))], int(rng.integers(0, 50)))
        else:
            apply("free", live.pop(int(rng.integers(len(live)))), None)


def _check_state(m, tokens, bs):
    ref = [0] * len(m.ref)
    for s in m.seqs:
        t = m.table(s)
        assert len(t) == -(-m.length(s) // bs)
        for b in t:
            ref[b] += 1
    assert ref == m.ref
    assert sorted(m.free) == sorted(b for b, r in enumerate(m.ref) if r == 0)
    assert len(set(m.free)) == len(m.free)
    seqs = list(m.seqs)
    for i, a in enumerate(seqs):
        ta = m.table(a)
        for c in seqs[i + 1:]:
            tc = m.table(c)
            for j, (x, y) in enumerate(zip(ta, tc)):
                if x == y:  # a shared block: both sequences hold the same tokens up to its end
                    end = (j + 1) * bs
                    assert tokens[a][:end] == tokens[c][:end]
                    assert len(tokens[a]) >= end and len(tokens[c]) >= end


def check_invariants_random(orc, seed=0, n_ops=400):
    rng = np.random.default_rng(seed)
    bs = 4
    prefixes = [rng.integers(0, 50, 40).tolist() for _ in range(3)]
    m = orc.BlockManager(48, bs, rng.permutation(48))
    tokens = {}

    def apply(op, s, arg):
        before = copy.deepcopy(m.__dict__)
        try:
            if op == "allocate":
                m.allocate(s, arg)
                tokens[s] = list(arg)
            elif op == "append":
                m.append(s, arg)
                tokens[s].append(arg)
            else:
                m.free_seq(s)
                del tokens[s]
        except orc.NoBlocks:
            assert m.__dict__ == before  # a failure changes nothing
            return False
        _check_state(m, tokens, bs)
        return True

    random_ops(rng, n_ops, prefixes, bs, apply)


def check_maximal_reuse(orc):
    bs = 4
    rng = np.random.default_rng(1)
    p = rng.integers(0, 1000, 10 * bs + 3).tolist()
    for k in (0, 1, 5, 10):
        m = orc.BlockManager(64, bs)
        m.allocate("s1", p)
        q = p[:k * bs] + [1001, 1002, 1003, 1004, 1005]
        cached = m.allocate("s2", q)
        assert cached == min(k, (len(q) - 1) // bs) * bs
        assert m.table("s2")[:k] == m.table("s1")[:k]
    # a prompt equal to a cached one still computes its last block
    m = orc.BlockManager(64, bs)
    m.allocate("a", p[:8 * bs])
    assert m.allocate("b", p[:8 * bs]) == 7 * bs


def check_preempt_and_readmit(orc):
    bs = 4
    p = list(range(100, 100 + 6 * bs + 1))
    m = orc.BlockManager(20, bs)
    m.allocate("s", p)
    first = m.table("s")
    m.free_seq("s")  # preempted: its blocks go back to the pool, still hashed
    assert m.allocate("s", p) == 6 * bs
    assert m.table("s")[:6] == first[:6]


def check_failures_are_atomic(orc):
    bs = 2
    m = orc.BlockManager(3, bs)
    m.allocate("a", [1, 2, 3, 4, 5])    # blocks 0, 1, 2
    m.free_seq("a")                     # free: 2, 1, 0 (0 and 1 still hashed)
    m.allocate("c", [7])                # takes 2
    before = copy.deepcopy(m.__dict__)
    try:  # hits 0 and 1 (both free) and needs 2 more: 4 > 2 free
        m.allocate("d", [1, 2, 3, 4, 5, 6, 7])
        raise AssertionError("allocation beyond the pool succeeded")
    except orc.NoBlocks:
        pass
    assert m.__dict__ == before
    m2 = orc.BlockManager(1, bs)
    m2.allocate("x", [1, 2])
    before = copy.deepcopy(m2.__dict__)
    try:
        m2.append("x", 3)
        raise AssertionError("append without a free block succeeded")
    except orc.NoBlocks:
        pass
    assert m2.__dict__ == before


ALL_CHECKS = [check_golden, check_invariants_random, check_maximal_reuse, check_preempt_and_readmit,
              check_failures_are_atomic]
