"""Pins of the oracle's KV commit after a verify ([lanes] "헤드냐, LoRA냐": one shared KV line, the
AR verifies and appends; [alphalab] walkthrough step 4: keep the accepted prefix, discard the rest).

  - a hand-worked example (two requests, a tree path and a prefix with a gap);
  - the linear case (kept rows = the accepted prefix) moves nothing and only advances the length;
  - random paths against numpy's gather of the old block rows (the definition is a gather), with
    every row outside the kept range untouched;
  - invalid requests (count, order, range, length) are flagged and left unchanged, valid ones in the
    same call still commit;
  - the accepted node lists of the oracle's tree verify always satisfy the commit's precondition
    (strictly increasing: a parent's index is below its child's), so they can be passed as is.
"""
import numpy as np
import pytest

from lossless_draft_verification_spec_amd import workloads


def test_hand_example(orc):
    kv = np.arange(2 * 10 * 4, dtype=np.int32).reshape(2, 10, 4).copy()
    length = np.array([2, 3], np.int32)
    keep = np.array([[1, 3, -1], [0, 2, 3]], np.int32)
    st = orc.kv_commit(kv, 4, np.array([2, 3], np.int32), length, keep=keep)
    assert st.tolist() == [0, 0] and length.tolist() == [4, 6]
    r0 = np.arange(40).reshape(10, 4)
    want0 = r0.copy()
    want0[2], want0[3] = r0[3], r0[5]
    assert (kv[0] == want0).all()
    r1 = np.arange(40, 80).reshape(10, 4)
    want1 = r1.copy()
    want1[3], want1[4], want1[5] = r1[3], r1[5], r1[6]
    assert (kv[1] == want1).all()


def test_prefix_keeps_data_in_place(orc):
    rng = np.random.default_rng(1)
    kv = rng.integers(0, 2**16, size=(5, 40, 24), dtype=np.uint16)
    before = kv.copy()
    length = rng.integers(0, 30, size=5).astype(np.int32)
    n = rng.integers(0, 9, size=5).astype(np.int32)
    start = length.copy()
    st = orc.kv_commit(kv, 9, n, length)
    assert (st == 0).all() and (length == start + n).all()
    assert (kv == before).all()


@pytest.mark.parametrize("seed", range(5))
def test_random_paths_match_gather(orc, seed):
    rng = np.random.default_rng(seed)
    batch, Lmax, row, blk = 6, 80, 37, 32
    kv = rng.standard_normal((batch, Lmax, row)).astype(np.float32)
    old = kv.copy()
    length = rng.integers(0, Lmax - blk + 1, size=batch).astype(np.int32)
    start = length.copy()
    n = rng.integers(0, 9, size=batch).astype(np.int32)
    keep = np.full((batch, 8), -1, np.int32)
    for r in range(batch):
        keep[r, :n[r]] = np.sort(rng.choice(blk, size=n[r], replace=False))
    st = orc.kv_commit(kv, blk, n, length, keep=keep)
    assert (st == 0).all() and (length == start + n).all()
    for r in range(batch):
        L, k = start[r], n[r]
        want = old[r].copy()
        want[L:L + k] = np.take(old[r], L + keep[r, :k], axis=0)
        assert np.array_equal(kv[r], want)


def test_invalid_requests_are_flagged_and_untouched(orc):
    batch, Lmax, row, blk = 6, 20, 8, 6
    kv = np.arange(batch * Lmax * row, dtype=np.int16).reshape(batch, Lmax, row).copy()
    old = kv.copy()
    length = np.array([0, 3, 15, 2, 2, 1], np.int32)
    n = np.array([7, 2, 1, 3, 2, 2], np.int32)
    keep = np.array([[0, 1, 2, 3, 4, 5, 6],   # n > blk
                     [2, 2, -1, -1, -1, -1, -1],  # not strictly increasing
                     [0, -1, -1, -1, -1, -1, -1],  # len + blk > Lmax
                     [1, 3, 6, -1, -1, -1, -1],    # position outside the block
                     [4, 5, -1, -1, -1, -1, -1],   # valid
                     [-1, 3, -1, -1, -1, -1, -1]], np.int32)  # negative position
    start = length.copy()
    st = orc.kv_commit(kv, blk, n, length, keep=keep)
    assert st.tolist() == [orc.ST_BAD_KEEP] * 4 + [0, orc.ST_BAD_KEEP]
    for r in (0, 1, 2, 3, 5):
        assert np.array_equal(kv[r], old[r]) and length[r] == start[r]
    assert length[4] == 4
    assert np.array_equal(kv[4][2:4], old[4][6:8])


def test_tree_accept_nodes_satisfy_the_commit(orc):
    tin = workloads.make_tree("c4b", device="cpu", batch=3, V=2000)
    p = tin.p.numpy()
    par, tok = tin.parent.numpy(), tin.node_tokens.numpy()
    N, D = par.shape[1], tin.preset.depth
    for step in range(20):
        o = orc.verify_tree(p, par, tok, D, seed=3, step=step)
        for r in range(3):
            k = o["accept_len"][r]
            nodes = o["accept_nodes"][r, :k]
            assert (np.diff(nodes) > 0).all() and (nodes >= 0).all() and (nodes < N).all()
        kv = np.zeros((3, N + 4, 2), np.float32)
        kv[:, :, 0] = np.arange(N + 4)
        length = np.zeros(3, np.int32)
        st = orc.kv_commit(kv, N, o["accept_len"].astype(np.int32), length,
                           keep=o["accept_nodes"].astype(np.int32))
        assert (st == 0).all()
        for r in range(3):
            k = o["accept_len"][r]
            assert (kv[r, :k, 0] == o["accept_nodes"][r, :k]).all()
