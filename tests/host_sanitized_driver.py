"""Runs the library's host code (block pool, prefix cache, H2O rule, table
checks) built with the address and undefined-behaviour sanitizers against
the oracle, in a process of its own (started by test_host_sanitized.py with
the sanitizer runtime preloaded).  Exits non-zero on any mismatch; the
sanitizers abort the process on any error they find.

Usage: python host_sanitized_driver.py <path of the sanitized library>
"""

import ctypes
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import oracle  # noqa: E402

L = ctypes.CDLL(sys.argv[1])
_p, _i, _i32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32
_i32p = ctypes.POINTER(_i32)
for name, args, res in (
        ("pkv_last_error", [], ctypes.c_char_p),
        ("pkv_pool_create", [_i, _p], _p), ("pkv_pool_destroy", [_p], None),
        ("pkv_pool_alloc", [_p, _i32p], _i), ("pkv_pool_incref", [_p, _i32], _i),
        ("pkv_pool_decref", [_p, _i32], _i), ("pkv_pool_refcount", [_p, _i32], _i32),
        ("pkv_pool_append", [_p, _p, _i32, _i32p, _i32, _i, _i32p, _i32p, _i32p], _i),
        ("pkv_pool_free_list", [_p, _p, _i32, _i32p], _i),
        ("pkv_pool_allocate_sequence", [_p, _i32, _i, _p, _i32, _i32p], _i),
        ("pkv_pool_fork", [_p, _p, _i32], _i), ("pkv_pool_release", [_p, _p, _i32], _i),
        ("pkv_prefix_cache_create", [_p, _i], _p), ("pkv_prefix_cache_destroy", [_p], None),
        ("pkv_prefix_cache_match", [_p, _p, _i, _p, _i, _p], _i),
        ("pkv_prefix_cache_insert", [_p, _p, _i, _p, _i, _p], _i),
        ("pkv_prefix_cache_evict", [_p, _i, _p], _i), ("pkv_prefix_cache_size", [_p], _i),
        ("pkv_h2o_retain", [_p, _i, _i, _i, _p, _p], _i),
        ("pkv_validate_tables", [_p, _i, _p, _i, _i, _i, _p, _i], _i),
        ("pkv_validate_shared_prefix", [_p, _i, _p, _i, _i, _i], _i)):
    f = getattr(L, name)
    f.argtypes, f.restype = args, res


def arr(vals, n=None):
    vals = [int(v) for v in vals]
    return (_i32 * max(1, n if n is not None else len(vals)))(*vals)


class Pool:
    def __init__(self, nb, order):
        self.h = L.pkv_pool_create(nb, ctypes.cast(arr(order), _p))
        self.nb = nb

    def ok(self, st):
        if st != 0:
            raise RuntimeError(L.pkv_last_error().decode())

    def allocate_sequence(self, length, bs=16):
        out, n = arr([], self.nb), _i32()
        self.ok(L.pkv_pool_allocate_sequence(self.h, length, bs, ctypes.cast(out, _p), self.nb, ctypes.byref(n)))
        return list(out[: n.value])

    def fork(self, t):
        self.ok(L.pkv_pool_fork(self.h, ctypes.cast(arr(t), _p), len(t)))
        return list(t)

    def release(self, t):
        self.ok(L.pkv_pool_release(self.h, ctypes.cast(arr(t), _p), len(t)))

    def append(self, table, length, bs, cap):
        a = arr(table, cap)
        n, slot, src, dst = _i32(len(table)), _i32(), _i32(), _i32()
        self.ok(L.pkv_pool_append(self.h, ctypes.cast(a, _p), cap, ctypes.byref(n), length, bs, ctypes.byref(slot),
                                  ctypes.byref(src), ctypes.byref(dst)))
        table[:] = list(a[: n.value])
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def free_list(self):
        out, n = arr([], self.nb), _i32()
        self.ok(L.pkv_pool_free_list(self.h, ctypes.cast(out, _p), self.nb, ctypes.byref(n)))
        return list(out[: n.value])


def check_pool():
    rng = random.Random(11)
    for trial in range(40):
        nb = rng.randint(4, 60)
        order = list(range(nb))
        rng.shuffle(order)
        lp, op = Pool(nb, order), oracle.pool.BlockPool(nb, order)
        seqs = []
        for _ in range(300):
            r = rng.random()
            if r < 0.3 or not seqs:
                n = rng.randint(0, 40)
                if -(-n // 16) > len(op.free_list):
                    # too few free blocks: the library refuses and changes nothing
                    before = lp.free_list()
                    try:
                        lp.allocate_sequence(n)
                    except RuntimeError:
                        assert lp.free_list() == before
                        continue
                    raise AssertionError("library allocated past an empty pool")
                seqs.append([lp.allocate_sequence(n), op.allocate_sequence(n, 16), n])
            elif r < 0.45:
                i = rng.randrange(len(seqs))
                seqs.append([lp.fork(seqs[i][0]), op.fork(seqs[i][1]), seqs[i][2]])
            elif r < 0.85:
                s = seqs[rng.randrange(len(seqs))]
                try:
                    oslot, ocow = op.append(s[1], s[2], 16)
                except oracle.pool.PoolExhausted:
                    continue
                lslot, lcow = lp.append(s[0], s[2], 16, len(s[0]) + 1)
                assert (lslot, lcow) == (oslot, ocow) and s[0] == s[1]
                s[2] += 1
            else:
                s = seqs.pop(rng.randrange(len(seqs)))
                lp.release(s[0])
                op.release(s[1])
            assert lp.free_list() == list(op.free_list)
            for b in range(nb):
                assert L.pkv_pool_refcount(lp.h, b) == op.refcount[b]
        # error paths leave the pool unchanged
        before = lp.free_list()
        assert L.pkv_pool_release(lp.h, ctypes.cast(arr([nb + 5]), _p), 1) != 0
        assert L.pkv_pool_fork(lp.h, ctypes.cast(arr([-1]), _p), 1) != 0
        assert L.pkv_pool_allocate_sequence(lp.h, 16 * (nb + 1), 16, ctypes.cast(arr([], nb + 1), _p), nb + 1,
                                            ctypes.byref(_i32())) != 0
        assert lp.free_list() == before
        L.pkv_pool_destroy(lp.h)


def check_prefix_cache():
    rng = random.Random(9)
    bs = 4
    pool = Pool(4000, list(range(4000)))
    c = L.pkv_prefix_cache_create(pool.h, bs)
    o = oracle.reuse.PrefixCache(bs)
    for _ in range(400):
        toks = [1, 2, 3, 4, 5, 6, 7, 8][: rng.randint(0, 8)] + [rng.randint(0, 3) for _ in range(rng.randint(0, 30))]
        cap = len(toks) // bs
        out, got = arr([], cap), _i()
        assert L.pkv_prefix_cache_match(c, ctypes.cast(arr(toks), _p), len(toks), ctypes.cast(out, _p), cap,
                                        ctypes.byref(got)) == 0
        hits = list(out[: got.value])
        assert hits == o.match(toks)
        blocks = hits + [pool.allocate_sequence(1, 1)[0] for _ in range(-(-len(toks) // bs) - len(hits))]
        added = _i()
        assert L.pkv_prefix_cache_insert(c, ctypes.cast(arr(toks), _p), len(toks), ctypes.cast(arr(blocks), _p),
                                         len(blocks), ctypes.byref(added)) == 0
        assert added.value == o.insert(toks, blocks)
        pool.release(blocks)
    assert L.pkv_prefix_cache_size(c) == len(o.blocks)
    ev = _i()
    assert L.pkv_prefix_cache_evict(c, 10 ** 6, ctypes.byref(ev)) == 0 and ev.value == len(o.blocks)
    assert len(pool.free_list()) == 4000
    L.pkv_prefix_cache_destroy(c)
    L.pkv_pool_destroy(pool.h)


def check_h2o():
    rng = random.Random(4)
    for _ in range(500):
        n = rng.randint(0, 60)
        scores = [rng.choice([0.0, 0.25, 1.0, 3.5]) for _ in range(n)]
        budget, recent = rng.randint(0, n + 2), 0
        recent = rng.randint(0, budget + 1)
        buf = (ctypes.c_float * max(1, n))(*scores)
        out, k = arr([], n), _i()
        assert L.pkv_h2o_retain(ctypes.cast(buf, _p), n, budget, recent, ctypes.cast(out, _p), ctypes.byref(k)) == 0
        assert list(out[: k.value]) == oracle.reuse.h2o_retain(scores, budget, recent)


def check_tables():
    rng = random.Random(3)
    for _ in range(300):
        S, mbs, nb = rng.randint(0, 6), rng.randint(0, 9), rng.randint(1, 40)
        lens = [rng.randint(0, mbs * 16 + 3) for _ in range(S)]
        bt = [rng.randint(-1, nb) for _ in range(S * mbs)]
        slots = [rng.randint(-2, nb * 16) for _ in range(rng.randint(0, 12))]
        st = L.pkv_validate_tables(ctypes.cast(arr(bt), _p), mbs, ctypes.cast(arr(lens), _p), S, 16, nb,
                                   ctypes.cast(arr(slots), _p), len(slots))
        ok = all(L_ <= mbs * 16 for L_ in lens) and all(
            0 <= bt[s * mbs + i] < nb for s in range(S) for i in range(-(-lens[s] // 16)))
        pos = [x for x in slots if x >= 0]
        ok = ok and all(x < nb * 16 for x in pos) and len(set(pos)) == len(pos)
        assert (st == 0) == ok, (S, mbs, nb, lens, bt, slots)
        P = rng.randint(0, mbs)
        st = L.pkv_validate_shared_prefix(ctypes.cast(arr(bt), _p), mbs, ctypes.cast(arr(lens), _p), S, 16, P)
        want = all(L_ >= 16 * P for L_ in lens) and all(bt[s * mbs + i] == bt[i] for s in range(S) for i in range(P))
        assert (st == 0) == want


if __name__ == "__main__":
    check_pool()
    check_prefix_cache()
    check_h2o()
    check_tables()
    print("host code under ASan/UBSan: pool, prefix cache, H2O, table checks all match the oracle")
