"""CPU check of the write order the short-conv compaction uses inside one
thread (one 16-byte column piece of one row), against the oracle's
token-by-token decode of the conv state.

The kernel moves row n + i of [source rows, inputs] to row i of the final
slot and row bnd_len + i to row i of the boundary slot, in ascending i, all in
one thread: a later read sees that thread's earlier writes. The model below
replays exactly that sequence of reads and writes on a small pool, for every
relation the C ABI accepts between the source, final and boundary slots
(vLLM RecoverSSM PR, Commits item 6: a fold must not read a source another
fold has already overwritten). It also shows that the plain final-then-
boundary order fails when the final state is written in place and the
boundary goes elsewhere -- the input the library orders differently.
"""
import itertools

import numpy as np
import pytest

import oracle


def kernel_order(pool, x, src, dst, n, bl, bs, final_first_always=False):
    """The compaction's reads and writes of one row, in the kernel's order."""
    Ls = pool.shape[1]

    def row(r):
        return pool[src, r].copy() if r < Ls else x[r - Ls].copy()

    def write_final():
        for i in range(Ls):
            pool[dst, i] = row(n + i)

    def write_bnd():
        for i in range(Ls):
            pool[bs, i] = row(bl + i)

    if bl > 0 and bs != dst:
        if dst == src and not final_first_always:
            write_bnd()
            write_final()
        else:
            write_final()
            write_bnd()
    else:
        write_final()


@pytest.mark.parametrize("Ls", [1, 3, 6])
def test_kernel_order_matches_token_walk(oracle_mod, Ls):
    rng = np.random.default_rng(400 + Ls)
    T, C = 4, 3
    for n in range(1, T + 1):
        for bl in range(0, n):
            # slots 0 = source; final and boundary slots drawn from {0, 1, 2}
            for dst, bs in itertools.product(range(3), range(3)):
                if bl == 0 and bs != 2:
                    continue
                pool = rng.standard_normal((3, Ls, C)).astype(np.float32)
                x = rng.standard_normal((n, C)).astype(np.float32)
                fin, bnd = oracle.conv_commit(pool[0].copy(), x, n, bl)
                got = pool.copy()
                kernel_order(got, x, 0, dst, n, bl if bl else 0, bs if bl else -1)
                np.testing.assert_array_equal(got[dst], fin, err_msg=f"{n} {bl} {dst} {bs}")
                if bnd is not None and bs != dst:
                    np.testing.assert_array_equal(got[bs], bnd, err_msg=f"{n} {bl} {dst} {bs}")


def test_final_first_fails_for_in_place_final_with_outside_boundary(oracle_mod):
    """The order the library uses elsewhere (final rows, then boundary rows)
    reads already-shifted source rows when dst == src and the boundary goes to
    another slot: the boundary state comes out wrong."""
    rng = np.random.default_rng(409)
    Ls, C, n, bl = 3, 4, 3, 1
    pool = rng.standard_normal((2, Ls, C)).astype(np.float32)
    x = rng.standard_normal((n, C)).astype(np.float32)
    fin, bnd = oracle.conv_commit(pool[0].copy(), x, n, bl)
    got = pool.copy()
    kernel_order(got, x, 0, 0, n, bl, 1, final_first_always=True)
    np.testing.assert_array_equal(got[0], fin)
    assert not np.array_equal(got[1], bnd)
