"""The C-ABI library loads and exports every function that include/*.h declares (no GPU needed:
nothing is called but the host-only argument checks and the workspace queries)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"\b(psispec_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def libpsispec():
    import lossless_draft_verification_spec_amd as pkg
    return pkg.lib()


def test_every_declared_symbol_is_exported(libpsispec):
    names = _declared()
    assert {"psispec_verify_linear", "psispec_verify_tree", "psispec_strerror"} <= names
    for n in sorted(names):
        assert hasattr(libpsispec, n), n


def test_workspace_queries_and_host_checks(libpsispec):
    import lossless_draft_verification_spec_amd as pkg
    assert pkg.linear_workspace_bytes(64, 8, 151936, pkg.PSISPEC_BF16) > 0
    assert pkg.linear_workspace_bytes(64, 65, 151936, pkg.PSISPEC_BF16) == 0  # B > 64
    assert pkg.linear_workspace_bytes(64, 8, 151936, 7) == 0                  # bad dtype
    assert pkg.tree_workspace_bytes(8, 32, 151936, pkg.PSISPEC_F32) > 0
    assert pkg.tree_workspace_bytes(8, 2000, 151936, pkg.PSISPEC_F32) == 0
    # argument errors are caught on the host before anything is launched
    L = libpsispec
    s = pkg.psispec_sampling(0.0, 1.0, 0, 0, 0, 0, 0)  # temperature 0
    rc = L.psispec_verify_linear(None, None, 1, None, 1, 4, 10, ctypes.byref(s), None, None, None,
                                 None, None, None, 0, None)
    assert rc == -1
    s = pkg.psispec_sampling(1.0, 1.5, 0, 0, 0, 0, 0)  # top_p > 1
    rc = L.psispec_verify_linear(None, None, 1, None, 1, 4, 10, ctypes.byref(s), None, None, None,
                                 None, None, None, 0, None)
    assert rc == -1
    s = pkg.psispec_sampling(1.0, 1.0, 0, 0, 0, 0, 0)
    rc = L.psispec_verify_linear(None, None, 5, None, 1, 4, 10, ctypes.byref(s), None, None, None,
                                 None, None, None, 0, None)
    assert rc == -2  # dtype
    rc = L.psispec_verify_linear(ctypes.c_void_p(16), ctypes.c_void_p(16), 1, ctypes.c_void_p(16),
                                 1, 4, 10, ctypes.byref(s), ctypes.c_void_p(16),
                                 ctypes.c_void_p(16), None, None, None, None, 0, None)
    assert rc == -3  # no workspace
    rc = L.psispec_verify_tree(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, None, None, 1, 4, 10, 4,
                               ctypes.byref(s), None, None, None, None, None, None, 0, None)
    assert rc == -1  # sampled-candidate tree without parent / node tokens / outputs
    fake = ctypes.c_void_p(256)
    rc = L.psispec_verify_tree(fake, fake, 0, fake, fake, 1, 4, 10, 4, ctypes.byref(s), fake, fake,
                               fake, None, None, None, 0, None)
    assert rc == -3  # sampled-candidate tree without a workspace
    assert L.psispec_strerror(-3).decode().startswith("workspace")
    # batch 0 is a no-op that succeeds without touching anything
    rc = L.psispec_verify_linear(None, None, 1, None, 0, 4, 10, ctypes.byref(s), None, None, None,
                                 None, None, None, 0, None)
    assert rc == 0


def test_sample_drafts_host_checks(libpsispec):
    import lossless_draft_verification_spec_amd as pkg
    L = libpsispec
    assert pkg.drafts_workspace_bytes(64, 8, 151936, pkg.PSISPEC_BF16) > 0
    assert pkg.drafts_workspace_bytes(64, 0, 151936, pkg.PSISPEC_BF16) == 0
    assert pkg.drafts_workspace_bytes(64, 65, 151936, pkg.PSISPEC_BF16) == 0
    fake = ctypes.c_void_p(256)
    out = ctypes.c_void_p(512)
    s = pkg.psispec_sampling(1.0, 1.0, 0, 0, 0, 0, 0)
    # no q rows without the Uno layout
    assert L.psispec_sample_drafts(None, 0, None, 1, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   1 << 30, None) == -1
    # Uno layout: the AR rows are required and their stride must cover a row
    s.flags = pkg.PSISPEC_FIRST_FROM_TARGET
    assert L.psispec_sample_drafts(None, 100, fake, 1, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   1 << 30, None) == -1
    assert L.psispec_sample_drafts(fake, 99, fake, 1, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   1 << 30, None) == -1
    # missing output, bad dtype, small workspace
    assert L.psispec_sample_drafts(fake, 100, fake, 1, 2, 4, 100, ctypes.byref(s), None, None, fake,
                                   1 << 30, None) == -1
    assert L.psispec_sample_drafts(fake, 100, fake, 9, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   1 << 30, None) == -2
    assert L.psispec_sample_drafts(fake, 100, fake, 1, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   16, None) == -3
    s.temperature = float("nan")
    assert L.psispec_sample_drafts(fake, 100, fake, 1, 2, 4, 100, ctypes.byref(s), out, None, fake,
                                   1 << 30, None) == -1


def test_max_children_flag_host_checks(libpsispec):
    """The bound on children per node is taken by the tree verify with q rows only, for 1..8; every
    other call, and a bound outside that range, is refused before anything is launched."""
    import lossless_draft_verification_spec_amd as pkg
    L = libpsispec
    fake = ctypes.c_void_p(256)
    s = pkg.psispec_sampling(1.0, 1.0, 0, 0, 0, 0, 0)

    def tree(q, flags, batch=0):
        s.flags = flags
        return L.psispec_verify_tree(fake, q, 0, fake, fake, batch, 4, 10, 4, ctypes.byref(s),
                                     fake, fake, fake, None, None, None, 0, None)

    for k in range(1, 9):
        assert tree(fake, k << pkg.PSISPEC_MAX_CHILDREN_SHIFT) == 0  # batch 0: accepted, a no-op
    assert tree(fake, 9 << pkg.PSISPEC_MAX_CHILDREN_SHIFT) == -1
    assert tree(fake, 15 << pkg.PSISPEC_MAX_CHILDREN_SHIFT) == -1
    assert tree(None, 4 << pkg.PSISPEC_MAX_CHILDREN_SHIFT) == -1  # chosen candidates: not taken
    assert tree(fake, 1 << 8) == -1  # bits above the field stay reserved
    assert tree(fake, 4 << pkg.PSISPEC_MAX_CHILDREN_SHIFT, batch=1) == -3  # checked, then no workspace
    s.flags = 4 << pkg.PSISPEC_MAX_CHILDREN_SHIFT
    assert L.psispec_verify_linear(None, None, 1, None, 0, 4, 10, ctypes.byref(s), None, None,
                                   None, None, None, None, 0, None) == -1
    assert L.psispec_sample_drafts(fake, 100, fake, 1, 2, 4, 100, ctypes.byref(s), fake, None,
                                   fake, 1 << 30, None) == -1


def test_kv_commit_host_checks(libpsispec):
    L = libpsispec
    fake = ctypes.c_void_p(256)
    # row bytes not a multiple of 16, line stride too small, block beyond the line or 1024
    assert L.psispec_kv_commit(fake, 1000, 24, 10, 4, None, 0, fake, fake, None, 2, None) == -1
    assert L.psispec_kv_commit(fake, 128, 32, 10, 4, None, 0, fake, fake, None, 2, None) == -1
    assert L.psispec_kv_commit(fake, 320, 32, 10, 11, None, 0, fake, fake, None, 2, None) == -1
    assert L.psispec_kv_commit(fake, 2048 * 32, 32, 2048, 1025, None, 0, fake, fake, None, 2,
                               None) == -1
    # missing lengths, misaligned lines, keep without a stride
    assert L.psispec_kv_commit(fake, 320, 32, 10, 4, None, 0, fake, None, None, 2, None) == -1
    assert L.psispec_kv_commit(ctypes.c_void_p(8), 320, 32, 10, 4, None, 0, fake, fake, None, 2,
                               None) == -1
    assert L.psispec_kv_commit(fake, 320, 32, 10, 4, fake, 0, fake, fake, None, 2, None) == -1
    # an empty batch launches nothing
    assert L.psispec_kv_commit(None, 320, 32, 10, 4, None, 0, None, None, None, 0, None) == 0


def test_lmhead_host_checks(libpsispec):
    """The LM-head call's shape rules and its top-p / debug-buffer rules are checked on the host,
    before anything is launched (pointers here are never dereferenced)."""
    import lossless_draft_verification_spec_amd as pkg
    L = libpsispec
    assert pkg.lmhead_workspace_bytes(128, 8, 4096, 151936, 16) > 0
    assert pkg.lmhead_workspace_bytes(128, 8, 4096, 151937, 16) == 0  # V not a multiple of 8
    assert pkg.lmhead_workspace_bytes(128, 8, 4000, 151936, 16) == 0  # H not a multiple of 64
    assert pkg.lmhead_workspace_bytes(128, 8, 4096, 151936, 65) == 0  # r > 64
    P = ctypes.c_void_p(256)
    big = ctypes.c_size_t(1 << 40)

    def call(top_p, pdbg, qdbg):
        s = pkg.psispec_sampling(1.0, top_p, 0, 0, 0, 0, 0)
        return L.psispec_lmhead_verify(P, P, P, None, None, 1.0, 2, 2, 64, 256, 0, P,
                                       ctypes.byref(s), P, P, None, None, None, pdbg, qdbg, P,
                                       big, None)

    assert call(0.9, None, None) == -5  # top-p needs the logits in memory: unsupported
    assert call(1.0, P, None) == -1     # debug buffers go together
    assert call(1.0, None, ctypes.c_void_p(8)) == -1
