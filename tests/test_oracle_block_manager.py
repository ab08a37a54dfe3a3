"""Pins of the oracle's block-manager model (oracle/block_manager.py).

Pinned by a hand-worked example that applies the pages' rules step by step,
and by the property the bookkeeping exists for: after any sequence of
allocate / fork / append / free operations, reading a sequence's tokens
through its block table (with every copy-on-write copy applied to a simulated
cache) gives back exactly that sequence's own token history -- shared
prefixes included, and no sequence ever seeing another's appended tokens."""
import numpy as np
import pytest

from oracle.block_manager import BlockManagerError, BlockManagerRef


def test_worked_example():
    bm = BlockManagerRef(num_blocks=4, block_size=2)
    bm.add_sequence(0, 3)                       # blocks 0, 1 (token 2 at block 1 offset 0)
    assert bm.table(0) == ([0, 1], 3)
    bm.fork(0, 1)                               # child shares both, counts 2
    assert bm.ref == {0: 2, 1: 2}
    assert bm.append(1) == (2 * 2 + 1, (1, 2))  # offset 1 of a shared block: copy into 2
    assert bm.table(1) == ([0, 2], 4)
    assert bm.ref == {0: 2, 1: 1, 2: 1}
    assert bm.append(0) == (1 * 2 + 1, None)    # block 1 is now the parent's alone
    assert bm.append(0) == (3 * 2 + 0, None)    # full: fresh block 3
    with pytest.raises(BlockManagerError) as e:
        bm.append(1)                            # full again, pool empty
    assert e.value.kind == "no_blocks"
    assert bm.table(1) == ([0, 2], 4)           # unchanged by the failure
    bm.free_sequence(0)                         # 0: count 2 -> 1; 1 and 3 freed
    assert bm.free == [1, 3] and bm.ref == {0: 1, 2: 1}
    assert bm.append(1) == (1 * 2 + 0, None)    # lowest free id first
    assert bm.token_slots(1, 0, 5) == [0, 1, 4, 5, 2]
    bm.check()


def test_errors_leave_state_unchanged():
    bm = BlockManagerRef(3, 4)
    bm.add_sequence(7, 9)                       # 3 blocks
    with pytest.raises(BlockManagerError) as e:
        bm.add_sequence(8, 1)
    assert e.value.kind == "no_blocks"
    with pytest.raises(BlockManagerError) as e:
        bm.add_sequence(7, 1)
    assert e.value.kind == "sequence"
    with pytest.raises(BlockManagerError) as e:
        bm.fork(9, 10)
    assert e.value.kind == "sequence"
    with pytest.raises(BlockManagerError) as e:
        bm.free_sequence(9)
    assert e.value.kind == "sequence"
    bm.fork(7, 8)
    with pytest.raises(BlockManagerError) as e:
        bm.append_batch([7, 8, 7])              # 7 copies (needs a block): none free
    assert e.value.kind == "no_blocks" and e.value.done == 0
    assert bm.table(7) == ([0, 1, 2], 9) and bm.table(8) == ([0, 1, 2], 9)
    bm.check()


def _simulate(seed, num_blocks, block_size, steps):
    """Random operations on the model, with a simulated cache (slot -> token)
    that receives every write and every copy-on-write copy."""
    rng = np.random.default_rng(seed)
    bm = BlockManagerRef(num_blocks, block_size)
    cache = {}
    history = {}                                  # seq -> list of token values
    next_id, next_tok = 0, 1

    def write(slot, tok):
        cache[slot] = tok

    def copy(src, dst):
        for o in range(block_size):
            if src * block_size + o in cache:
                cache[dst * block_size + o] = cache[src * block_size + o]
            else:
                cache.pop(dst * block_size + o, None)

    for _ in range(steps):
        op = rng.choice(["add", "fork", "append", "append", "append", "free"])
        live = sorted(history)
        try:
            if op == "add" or not live:
                n = int(rng.integers(0, 3 * block_size))
                bm.add_sequence(next_id, n)
                toks = list(range(next_tok, next_tok + n))
                next_tok += n
                for slot, t in zip(bm.token_slots(next_id, 0, n), toks):
                    write(slot, t)
                history[next_id] = toks
                next_id += 1
            elif op == "fork":
                p = int(rng.choice(live))
                bm.fork(p, next_id)
                history[next_id] = list(history[p])
                next_id += 1
            elif op == "append":
                batch = [int(x) for x in rng.choice(live, size=min(len(live), 4), replace=False)]
                try:
                    slots, pairs, done = bm.append_batch(batch)
                except BlockManagerError as e:
                    slots, pairs, done = e.slots, e.pairs, e.done
                for src, dst in pairs:                # copies before the writes
                    copy(src, dst)
                for sid, slot in zip(batch[:done], slots):
                    write(slot, next_tok)
                    history[sid].append(next_tok)
                    next_tok += 1
            else:
                sid = int(rng.choice(live))
                bm.free_sequence(sid)
                del history[sid]
        except BlockManagerError:
            pass
        bm.check()
        for sid, toks in history.items():
            blocks, n = bm.table(sid)
            assert n == len(toks)
            got = [cache.get(s) for s in bm.token_slots(sid, 0, n)]
            assert got == toks, f"sequence {sid} reads {got}, wrote {toks}"
    return bm


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("num_blocks,block_size", [(12, 2), (40, 4), (64, 16), (7, 1)])
def test_every_sequence_reads_back_its_own_tokens(seed, num_blocks, block_size):
    _simulate(seed, num_blocks, block_size, 300)
