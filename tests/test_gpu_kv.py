"""Parity of the KV commit of the HIP library (through its C ABI) with the CPU oracle: bit-exact
lines and lengths, for random kept paths, the prefix case, invalid requests, the tree verify's
accepted nodes fed in as they are, and a full-size batch of 114,688-byte rows."""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import (ST_BAD_KEEP, psispec_kv_commit,
                                                  psispec_verify_tree, workloads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _random_case(batch, Lmax, row_words, blk, maxk, seed, prefix=False):
    rng = np.random.default_rng(seed)
    kv = rng.integers(-2**31, 2**31 - 1, size=(batch, Lmax, row_words), dtype=np.int64)
    kv = kv.astype(np.int32)
    length = rng.integers(0, Lmax - blk + 1, size=batch).astype(np.int32)
    n = rng.integers(0, min(maxk, blk) + 1, size=batch).astype(np.int32)
    keep = np.full((batch, maxk), -1, np.int32)
    for r in range(batch):
        keep[r, :n[r]] = np.arange(n[r]) if prefix else np.sort(
            rng.choice(blk, size=n[r], replace=False))
    return kv, length, n, keep


def _run_both(kv, length, n, keep, blk, use_keep=True):
    kv_g = torch.from_numpy(kv).to(DEV)
    len_g = torch.from_numpy(length).to(DEV)
    st_g = torch.empty(kv.shape[0], dtype=torch.int32, device=DEV)
    psispec_kv_commit(kv_g, blk, torch.from_numpy(n).to(DEV), len_g,
                      keep=torch.from_numpy(keep).to(DEV) if use_keep else None, status=st_g)
    torch.cuda.synchronize()
    kv_o, len_o = kv.copy(), length.copy()
    st_o = oracle.kv_commit(kv_o, blk, n, len_o, keep=keep if use_keep else None)
    assert np.array_equal(st_g.cpu().numpy(), st_o)
    assert np.array_equal(len_g.cpu().numpy(), len_o)
    assert np.array_equal(kv_g.cpu().numpy(), kv_o)
    return st_o


@pytest.mark.parametrize("batch,Lmax,row_words,blk,maxk", [
    (1, 40, 4, 8, 8), (5, 64, 12, 32, 8), (7, 70, 1024, 32, 9), (3, 50, 1028, 16, 16),
    (2, 1100, 8, 1024, 64), (64, 48, 256, 17, 8)])
def test_random_paths(batch, Lmax, row_words, blk, maxk):
    for seed in range(3):
        kv, length, n, keep = _random_case(batch, Lmax, row_words, blk, maxk, seed)
        st = _run_both(kv, length, n, keep, blk)
        assert (st == 0).all()


def test_prefix_and_empty_commits():
    kv, length, n, keep = _random_case(6, 40, 20, 9, 9, 11, prefix=True)
    n[0] = 0
    _run_both(kv, length, n, keep, 9, use_keep=False)
    _run_both(kv, length, n, keep, 9, use_keep=True)


def test_invalid_requests_are_flagged():
    kv, length, n, keep = _random_case(6, 30, 8, 6, 7, 5)
    n[0] = 7                              # more than the block
    keep[1, :2] = [3, 3]; n[1] = 2        # not strictly increasing
    length[2] = 25                        # len + blk > Lmax
    keep[3, :1] = [6]; n[3] = 1           # outside the block
    keep[4, :2] = [1, 4]; n[4] = 2        # valid
    keep[5, :2] = [-1, 2]; n[5] = 2       # negative
    st = _run_both(kv, length, n, keep, 6)
    assert st.tolist() == [ST_BAD_KEEP] * 4 + [0, ST_BAD_KEEP]


def test_tree_verify_outputs_feed_the_commit():
    """The tree verify's accept_len and accept_nodes go straight into the commit on the device."""
    from dataclasses import replace
    pt = replace(workloads.PRESETS["sweep_tree"], boost=2.0)
    tin = workloads.make_tree(pt, device=DEV, batch=16, V=20000)
    N, D = tin.preset.N, tin.preset.depth
    row_words, Lmax = 64, 96
    rng = np.random.default_rng(2)
    for step in range(4):
        o = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, D, seed=tin.seed, step=step)
        torch.cuda.synchronize()
        n = o["accept_len"].cpu().numpy().astype(np.int32)
        keep = o["accept_nodes"].cpu().numpy().astype(np.int32)
        kv = rng.integers(0, 2**31 - 1, size=(16, Lmax, row_words), dtype=np.int64).astype(np.int32)
        length = rng.integers(0, Lmax - N + 1, size=16).astype(np.int32)
        st = _run_both(kv, length, n, keep, N)
        assert (st == 0).all()


def test_full_size_rows():
    """batch 256, 114,688-byte rows (28 layers x K and V x 8 heads x 128 dims, bf16), 32-position
    blocks: compared on sampled lines."""
    batch, Lmax, blk, maxk = 256, 128, 32, 8
    row_words = 114688 // 4
    g = torch.Generator(device=DEV).manual_seed(3)
    kv = torch.randint(-2**31, 2**31 - 1, (batch, Lmax, row_words), generator=g, device=DEV,
                       dtype=torch.int32)
    rng = np.random.default_rng(4)
    length = rng.integers(0, Lmax - blk + 1, size=batch).astype(np.int32)
    n = rng.integers(0, maxk + 1, size=batch).astype(np.int32)
    keep = np.full((batch, maxk), -1, np.int32)
    for r in range(batch):
        keep[r, :n[r]] = np.sort(rng.choice(blk, size=n[r], replace=False))
    sample = [0, 1, 97, 200, 255]
    before = {r: kv[r].cpu().numpy() for r in sample}
    len_g = torch.from_numpy(length).to(DEV)
    st = torch.empty(batch, dtype=torch.int32, device=DEV)
    psispec_kv_commit(kv, blk, torch.from_numpy(n).to(DEV), len_g, keep=torch.from_numpy(keep).to(DEV),
                      status=st)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all()
    assert np.array_equal(len_g.cpu().numpy(), length + n)
    for r in sample:
        line = before[r][None].copy()
        ln = length[r:r + 1].copy()
        oracle.kv_commit(line, blk, n[r:r + 1], ln, keep=keep[r:r + 1])
        assert np.array_equal(kv[r].cpu().numpy(), line[0]), r
