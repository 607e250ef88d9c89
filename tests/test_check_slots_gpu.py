"""GPU checks of gdn_check_slots, the debug check of a commit's slot
preconditions (rows of one commit run concurrently, so a slot one row writes
must not be written or read by another: vLLM RecoverSSM PR, Commits item 6,
is that race between programs). Each alias kind is planted in an otherwise
clean set of rows and must set GDN_ROW_ALIAS; clean sets, in-place commits,
boundary states written into the row's own source slot and dead rows must
not. The align plans of random block tables (the oracle's planner) pass."""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_speculative_gdn_amd as G
from gpu_harness import dev_i32

pytestmark = pytest.mark.gpu


def check(src, dst, n, rec=None, bl=None, bs=None) -> int:
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.gdn_check_slots(dev_i32(src), dev_i32(dst), dev_i32(n),
                      rec_slot=None if rec is None else dev_i32(rec),
                      bnd_len=None if bl is None else dev_i32(bl),
                      bnd_slot=None if bs is None else dev_i32(bs), err_flags=err)
    torch.cuda.synchronize()
    return int(err.item())


def test_each_alias_kind_is_flagged(gdn):
    src = np.arange(6)
    dst = np.arange(10, 16)
    n = np.array([2, 1, 3, 4, 2, 1])
    rec = np.arange(20, 26)
    none_b = np.zeros(6, np.int32), np.full(6, -1)
    assert check(src, dst, n, rec, *none_b) == 0
    assert check(src, src, n, rec) == 0                      # in place
    d = dst.copy(); d[3] = d[1]
    assert check(src, d, n) == G.ROW_ALIAS                   # two rows, one destination
    d = dst.copy(); d[2] = src[4]
    assert check(src, d, n) == G.ROW_ALIAS                   # writes another row's source
    bl, bs = none_b[0].copy(), none_b[1].copy()
    bl[0], bs[0] = 1, src[0]
    assert check(src, dst, n, rec, bl, bs) == 0              # boundary into its own source
    bs[0] = dst[5]
    assert check(src, dst, n, rec, bl, bs) == G.ROW_ALIAS    # boundary into another destination
    bs[0] = src[3]
    assert check(src, dst, n, rec, bl, bs) == G.ROW_ALIAS    # boundary into another source
    r = rec.copy(); r[4] = r[2]
    assert check(src, dst, n, r) == G.ROW_ALIAS              # shared record slot
    d = dst.copy(); d[1] = d[0]
    m = n.copy(); m[1] = 0
    assert check(src, d, m) == 0                             # a row with n = 0 is dead
    s = src.copy(); s[1] = -1
    assert check(s, d, n) == 0                               # a row with a null source is dead


def test_align_plans_are_alias_free(gdn):
    rng = np.random.default_rng(101)
    rows, blk, max_n, cols = 64, 16, 16, 40
    p0 = rng.integers(1, blk * (cols - 2), rows).astype(np.int32)
    n = rng.integers(0, max_n + 1, rows).astype(np.int32)
    table = rng.permutation(rows * cols).reshape(rows, cols).astype(np.int32)
    src, dst, bl, bs, perr = oracle.align_plan(p0, n, table, blk, max_n)
    assert (perr == 0).all() and (bl > 0).any()
    assert check(src, dst, n, None, bl, bs) == 0
    # two rows sharing a block-table column for their final state
    live = np.flatnonzero(n > 0)
    a, b = live[0], live[1]
    table2 = table.copy()
    table2[b, (p0[b] + n[b] - 1) // blk] = table[a, (p0[a] + n[a] - 1) // blk]
    src2, dst2, bl2, bs2, perr2 = oracle.align_plan(p0, n, table2, blk, max_n)
    assert (perr2 == 0).all()
    assert check(src2, dst2, n, None, bl2, bs2) == G.ROW_ALIAS
