"""The C++ block manager (libpa.so, include/pa_blocks.h) against the Python model: bit-exact.

Host-only: no GPU is needed. Every operation of seeded random workloads is
applied to both and their tables, free lists, reference counts, cached-token
counts and failures must agree exactly; the metadata builders must reproduce
what the model's tables give; XXH64 must equal the xxhash package's.
"""

import numpy as np
import pytest
import xxhash

import oracle.block_manager as orc
from paged_kv_cache_heads_amd import PAError
from paged_kv_cache_heads_amd.blocks import PA_ERR_NO_BLOCKS, PA_ERR_NOT_FOUND, BlockManager, xxh64
from tests import oracle_pins_blocks as pins


class _Native:
    """The C++ manager behind the face the golden replay expects (sequence names -> ids)."""

    def __init__(self, num_blocks, block_size):
        self.bm = BlockManager(num_blocks, block_size)
        self.ids, self.names = {}, {}

    def _id(self, name):
        if name not in self.ids:
            self.ids[name] = len(self.ids)
            self.names[self.ids[name]] = name
        return self.ids[name]

    def allocate(self, seq, tokens):
        try:
            return self.bm.allocate(self._id(seq), tokens)
        except PAError as e:
            assert e.status == PA_ERR_NO_BLOCKS
            return None

    def append(self, seq, token):
        try:
            self.bm.append(self._id(seq), token)
            return True
        except PAError as e:
            assert e.status == PA_ERR_NO_BLOCKS
            return False

    def free_seq(self, seq):
        self.bm.free_seq(self._id(seq))

    def tables(self):
        return {n: self.bm.table(i) for n, i in self.ids.items() if self.bm.length(i) >= 0}

    def free_list(self):
        return self.bm.free_list()


def test_golden_scenario():
    refs = lambda nat: [nat.bm.ref(b) for b in range(nat.bm.num_blocks)]  # noqa: E731
    pins.replay_golden(lambda n, b: _Native(n, b), check_refs=refs)


@pytest.mark.parametrize("n", [0, 1, 3, 4, 7, 8, 31, 32, 33, 63, 64, 100, 1023, 1024, 4096])
def test_xxh64_matches_xxhash(n):
    rng = np.random.default_rng(n)
    data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
    for seed in (0, 1, 0x9E3779B97F4A7C15, 2 ** 64 - 1):
        assert xxh64(data, seed) == xxhash.xxh64_intdigest(data, seed=seed)


def _compare(model, native, live):
    assert native.free_list() == model.free
    assert [native.ref(b) for b in range(len(model.ref))] == model.ref
    for s in live:
        assert native.table(s) == model.table(s)
        assert native.length(s) == model.length(s)


@pytest.mark.parametrize("seed,bs,nblocks", [(0, 1, 40), (1, 2, 24), (2, 4, 48), (3, 16, 32), (4, 256, 12),
                                             (5, 4, 8), (6, 3, 64)])
def test_random_workload_matches_model(seed, bs, nblocks):
    rng = np.random.default_rng(seed)
    order = rng.permutation(nblocks)
    model = orc.BlockManager(nblocks, bs, order)
    native = BlockManager(nblocks, bs, order)
    prefixes = [rng.integers(0, 30, 12 * bs).tolist() for _ in range(3)]
    live = set()

    def apply(op, s, arg):
        try:
            if op == "allocate":
                want = model.allocate(s, arg)
            elif op == "append":
                model.append(s, arg)
            else:
                model.free_seq(s)
            ok_model = True
        except orc.NoBlocks:
            ok_model = False
        try:
            if op == "allocate":
                got = native.allocate(s, arg)
                assert got == want
            elif op == "append":
                native.append(s, arg)
            else:
                native.free_seq(s)
            ok_native = True
        except PAError as e:
            assert e.status == PA_ERR_NO_BLOCKS
            ok_native = False
        assert ok_native == ok_model, (op, s)
        if ok_model and op == "allocate":
            live.add(s)
        if op == "free":
            live.discard(s)
        _compare(model, native, live)
        return ok_model

    pins.random_ops(rng, 600, prefixes, bs, apply)


def test_decode_and_prefill_metadata_match_tables():
    rng = np.random.default_rng(7)
    bs = 16
    model = orc.BlockManager(64, bs)
    native = BlockManager(64, bs)
    shared = rng.integers(0, 100, 3 * bs).tolist()
    cached = []
    lens = [1, 15, 16, 17, 40, 48, 49]
    for i, n in enumerate(lens):
        toks = shared[:min(n, len(shared))] + rng.integers(100, 200, max(0, n - len(shared))).tolist()
        c = native.allocate(i, toks)
        assert c == model.allocate(i, toks)
        cached.append(c)
    ids = list(range(len(lens)))
    width = 5
    bt, cq, ck, sm = native.prefill_metadata(ids, cached, width)
    want_sm = [model.slot(i, p) for i in ids for p in range(cached[i], model.length(i))]
    assert sm.tolist() == want_sm
    assert cq.tolist() == np.concatenate([[0], np.cumsum([model.length(i) - cached[i] for i in ids])]).tolist()
    assert ck.tolist() == np.concatenate([[0], np.cumsum([model.length(i) for i in ids])]).tolist()
    for i in ids:
        t = model.table(i)
        assert bt[i].tolist() == t + [-1] * (width - len(t))
    for i in ids:  # one decode step each
        native.append(i, 7)
        model.append(i, 7)
    bt, cl, sm = native.decode_metadata(ids, width)
    assert cl.tolist() == [model.length(i) for i in ids]
    assert sm.tolist() == [model.slot(i, model.length(i) - 1) for i in ids]
    for i in ids:
        t = model.table(i)
        assert bt[i].tolist() == t + [-1] * (width - len(t))


def test_errors():
    bm = BlockManager(4, 4)
    bm.allocate(1, [1, 2, 3])
    with pytest.raises(PAError) as e:
        bm.allocate(1, [4])
    assert e.value.status == 2  # already live
    with pytest.raises(PAError) as e:
        bm.append(9, 1)
    assert e.value.status == PA_ERR_NOT_FOUND
    with pytest.raises(PAError) as e:
        bm.free_seq(9)
    assert e.value.status == PA_ERR_NOT_FOUND
    with pytest.raises(PAError) as e:
        bm.allocate(2, list(range(20)))  # 5 blocks > 3 free
    assert e.value.status == PA_ERR_NO_BLOCKS
    assert bm.num_free() == 3 and bm.length(2) == -1
    with pytest.raises(PAError) as e:
        BlockManager(3, 4, order=[0, 0, 1])
    assert e.value.status == 2
    with pytest.raises(PAError) as e:
        BlockManager(0, 4)
    assert e.value.status == 2
    with pytest.raises(PAError) as e:
        bm.decode_metadata([1], 0)
    assert e.value.status == 2
    with pytest.raises(PAError) as e:
        bm.prefill_metadata([1], [4], 2)  # num_cached past the length
    assert e.value.status == 2


def test_engine_sized_workload_matches_model():
    # 256 sequences of 100..2048 prompt tokens over 256-token blocks, half sharing a
    # 1024-token system prompt, then 64 decode steps each, with preemption when full
    rng = np.random.default_rng(11)
    bs, nb = 256, 4096
    order = rng.permutation(nb)
    model, native = orc.BlockManager(nb, bs, order), BlockManager(nb, bs, order)
    system = rng.integers(0, 32000, 1024).tolist()
    live = []
    for s in range(256):
        n = int(rng.integers(100, 2049))
        toks = (system + rng.integers(0, 32000, n).tolist()) if s % 2 else rng.integers(0, 32000, n).tolist()
        assert native.allocate(s, toks) == model.allocate(s, toks)
        live.append(s)
    for _ in range(64):
        for s in list(live):
            t = int(rng.integers(0, 32000))
            try:
                model.append(s, t)
                ok = True
            except orc.NoBlocks:
                ok = False
            if ok:
                native.append(s, t)
            else:  # preempt the newest sequence, as a scheduler would
                with pytest.raises(PAError):
                    native.append(s, t)
                victim = live.pop()
                model.free_seq(victim)
                native.free_seq(victim)
    _compare(model, native, live)


def test_append_batch_matches_single_appends():
    rng = np.random.default_rng(12)
    bs = 4
    model, native = orc.BlockManager(10, bs), BlockManager(10, bs)
    for i in range(3):
        toks = rng.integers(0, 9, 5).tolist()
        native.allocate(i, toks)
        model.allocate(i, toks)
    ids = [0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2]
    toks = rng.integers(0, 9, len(ids)).tolist()
    done_model = 0
    for i, t in zip(ids, toks):
        try:
            model.append(i, t)
            done_model += 1
        except orc.NoBlocks:
            break
    with pytest.raises(PAError) as e:  # the pool runs out part way
        native.append_batch(ids, toks)
    assert e.value.status == PA_ERR_NO_BLOCKS
    assert done_model < len(ids)
    _compare(model, native, [0, 1, 2])
