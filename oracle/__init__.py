"""CPU oracle of the Psi-Spec verify step -- TEST INFRASTRUCTURE ONLY.

A plain single-threaded fp64 C implementation (``psispec_oracle.c``) and this ctypes binding.  Only
the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.
The GPU library never calls it and shares no code with it.

Arrays are numpy arrays on the host.  Logits may be float32, bfloat16 bit patterns (uint16) or
float64 (oracle-only, for the fp64 LM-head logits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "psispec_oracle.c")
_LIB = os.path.join(_HERE, "libpsispec_oracle.so")

F32, BF16, F64 = 0, 1, 2
FIRST_FROM_TARGET = 1
PURPOSE_ACCEPT, PURPOSE_RESAMPLE, PURPOSE_DRAFT = 0, 1, 2
ST_NONFINITE, ST_BAD_TOKEN, ST_Q_ZERO, ST_RESID_ZERO, ST_BAD_PARENT = 1, 2, 4, 8, 16
ST_BAD_KEEP = 32


# A test may point the binding at another build of the same source (the sanitizer build).
_ALT = os.environ.get("PSISPEC_ORACLE_LIB")


def build(force: bool = True, out: str | None = None, checks: tuple = ()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction) into an in-tree .so, or into
    `out` with extra instrumentation flags `checks` (e.g. address and undefined-behaviour
    sanitizers for the host-only test build)."""
    target = out or _LIB
    if force or not os.path.exists(target) or os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra", *checks, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, target)
    return target


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _ALT:
            L = ctypes.CDLL(_ALT)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, u32, u64, dbl = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double
        L.psispec_oracle_philox.argtypes = [u64, P, P]
        L.psispec_oracle_philox.restype = None
        L.psispec_oracle_uniform.argtypes = [u64, u32, u32, u32, u32]
        L.psispec_oracle_uniform.restype = dbl
        L.psispec_oracle_row_probs.argtypes = [P, i32, i32, dbl, dbl, P, P]
        L.psispec_oracle_row_probs.restype = i32
        L.psispec_oracle_verify_linear.argtypes = (
            [P, P, i32, P, i32, i32, i32, dbl, dbl, u64, u32, u32, u32, P, P] + [P] * 10)
        L.psispec_oracle_verify_linear.restype = i32
        L.psispec_oracle_verify_tree.argtypes = (
            [P, i32, P, P, i32, i32, i32, i32, dbl, dbl, u64, u32, u32, P, P] + [P] * 10)
        L.psispec_oracle_verify_tree.restype = i32
        L.psispec_oracle_verify_tree_sampled.argtypes = (
            [P, P, i32, P, P, i32, i32, i32, i32, dbl, dbl, u64, u32, u32, P, P] + [P] * 10)
        L.psispec_oracle_verify_tree_sampled.restype = i32
        L.psispec_oracle_sample_drafts.argtypes = (
            [P, ctypes.c_int64, P, i32, i32, i32, i32, dbl, dbl, u64, u32, u32, u32] + [P] * 5)
        L.psispec_oracle_sample_drafts.restype = i32
        L.psispec_oracle_kv_commit.argtypes = [P, ctypes.c_int64, ctypes.c_int64, i32, i32, P, i32, P,
                                               P, P, i32]
        L.psispec_oracle_kv_commit.restype = i32
        L.psispec_oracle_lmhead_logits.argtypes = [P, P, P, P, dbl, i32, i32, i32, i32, P]
        L.psispec_oracle_lmhead_logits.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported logits dtype {a.dtype} (float32, bf16 bits as uint16, float64)")


def philox(seed: int, ctr) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().psispec_oracle_philox(seed & (2**64 - 1), _ptr(c), _ptr(out))
    return out


def uniform(seed: int, request: int, position: int, purpose: int, step: int) -> float:
    return lib().psispec_oracle_uniform(seed & (2**64 - 1), request, position, purpose, step)


def row_probs(row: np.ndarray, T: float = 1.0, top_p: float = 1.0):
    row = np.ascontiguousarray(row)
    V = row.shape[-1]
    pi = np.zeros(V, dtype=np.float64)
    margin = ctypes.c_double(0.0)
    st = lib().psispec_oracle_row_probs(_ptr(row), _dtype_code(row), V, T, top_p, _ptr(pi),
                                        ctypes.byref(margin))
    return pi, int(st), margin.value


def verify_linear(p, q, draft, T=1.0, top_p=1.0, seed=0, step=0, request_base=0, flags=0,
                  u_accept=None, u_resample=None, want_resid=False):
    """p[batch][B+1][V], q[batch][B][V] (or None with FIRST_FROM_TARGET and B == 1), draft[batch][B]."""
    p = np.ascontiguousarray(p)
    q = None if q is None else np.ascontiguousarray(q)
    draft = np.ascontiguousarray(draft, dtype=np.int32)
    batch, B1, V = p.shape
    B = B1 - 1
    if q is not None and (q.shape != (batch, B, V) or q.dtype != p.dtype):
        raise ValueError("q must be [batch][B][V] with the dtype of p")
    if draft.shape != (batch, B):
        raise ValueError("draft must be [batch][B]")
    ua = None if u_accept is None else np.ascontiguousarray(u_accept, dtype=np.float64)
    ur = None if u_resample is None else np.ascontiguousarray(u_resample, dtype=np.float64)
    out = dict(
        accept_len=np.zeros(batch, np.int32), out_tokens=np.zeros((batch, B + 1), np.int32),
        ratios=np.zeros((batch, B), np.float64), accept_mask=np.zeros(batch, np.uint64),
        status=np.zeros(batch, np.int32), margin_accept=np.zeros((batch, B), np.float64),
        margin_sample=np.zeros(batch, np.float64),
        margin_topp=np.zeros((batch, 2 * B + 1), np.float64))
    if want_resid:
        out["resid_w"] = np.zeros((batch, V), np.float64)
        out["resid_S"] = np.zeros(batch, np.float64)
    rc = lib().psispec_oracle_verify_linear(
        _ptr(p), _ptr(q), _dtype_code(p), _ptr(draft), batch, B, V, float(T), float(top_p),
        seed & (2**64 - 1), step, request_base, flags, _ptr(ua), _ptr(ur),
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out["ratios"]),
        _ptr(out["accept_mask"]), _ptr(out["status"]), _ptr(out["margin_accept"]),
        _ptr(out["margin_sample"]), _ptr(out["margin_topp"]), _ptr(out.get("resid_w")),
        _ptr(out.get("resid_S")))
    if rc != 0:
        raise ValueError(f"oracle verify_linear rejected its arguments (code {rc})")
    return out


def sample_drafts(ar, q, B=None, T=1.0, top_p=1.0, seed=0, step=0, request_base=0, flags=0,
                  u_draw=None):
    """Drafted tokens [batch][B].  q[batch][B][V] (row 0 unread with FIRST_FROM_TARGET; None allowed
    then when B == 1); ar (read only with FIRST_FROM_TARGET): [batch][V] or [batch][k][V], whose
    request r starts its first row at element r * (k V)."""
    q = None if q is None else np.ascontiguousarray(q)
    ar = None if ar is None else np.ascontiguousarray(ar)
    if q is not None:
        batch, B, V = q.shape
        code = _dtype_code(q)
    else:
        batch, V = ar.shape[0], ar.shape[-1]
        B = 1 if B is None else B
        code = _dtype_code(ar)
    stride = 0
    if ar is not None:
        if ar.shape[0] != batch or ar.shape[-1] != V or (q is not None and ar.dtype != q.dtype):
            raise ValueError("ar must be [batch][...][V] with the dtype of q")
        stride = ar.size // max(batch, 1)
    ud = None if u_draw is None else np.ascontiguousarray(u_draw, dtype=np.float64)
    out = dict(tokens=np.zeros((batch, B), np.int32), status=np.zeros((batch, B), np.int32),
               margin_sample=np.zeros((batch, B), np.float64),
               margin_topp=np.zeros((batch, B), np.float64))
    rc = lib().psispec_oracle_sample_drafts(
        _ptr(ar), stride, _ptr(q), code, batch, B, V, float(T), float(top_p), seed & (2**64 - 1),
        step, request_base, flags, _ptr(ud), _ptr(out["tokens"]), _ptr(out["status"]),
        _ptr(out["margin_sample"]), _ptr(out["margin_topp"]))
    if rc != 0:
        raise ValueError(f"oracle sample_drafts rejected its arguments (code {rc})")
    return out


def verify_tree(p, parent, node_tokens, max_depth, T=1.0, top_p=1.0, seed=0, step=0,
                request_base=0, u_accept=None, u_resample=None, want_resid=False):
    """p[batch][N+1][V] (row 0 = root, row j+1 = node j), parent/node_tokens [batch][N]."""
    p = np.ascontiguousarray(p)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    node_tokens = np.ascontiguousarray(node_tokens, dtype=np.int32)
    batch, N1, V = p.shape
    N = N1 - 1
    if parent.shape != (batch, N) or node_tokens.shape != (batch, N):
        raise ValueError("parent and node_tokens must be [batch][N]")
    ua = None if u_accept is None else np.ascontiguousarray(u_accept, dtype=np.float64)
    ur = None if u_resample is None else np.ascontiguousarray(u_resample, dtype=np.float64)
    out = dict(
        accept_len=np.zeros(batch, np.int32), accept_nodes=np.zeros((batch, max_depth), np.int32),
        out_tokens=np.zeros((batch, max_depth + 1), np.int32),
        node_ratios=np.zeros((batch, N), np.float64), status=np.zeros(batch, np.int32),
        margin_accept=np.zeros((batch, N), np.float64), margin_sample=np.zeros(batch, np.float64),
        margin_topp=np.zeros((batch, N + 1), np.float64))
    if want_resid:
        out["resid_w"] = np.zeros((batch, V), np.float64)
        out["resid_S"] = np.zeros(batch, np.float64)
    rc = lib().psispec_oracle_verify_tree(
        _ptr(p), _dtype_code(p), _ptr(parent), _ptr(node_tokens), batch, N, V, max_depth, float(T),
        float(top_p), seed & (2**64 - 1), step, request_base, _ptr(ua), _ptr(ur),
        _ptr(out["accept_len"]), _ptr(out["accept_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out["node_ratios"]), _ptr(out["status"]), _ptr(out["margin_accept"]),
        _ptr(out["margin_sample"]), _ptr(out["margin_topp"]), _ptr(out.get("resid_w")),
        _ptr(out.get("resid_S")))
    if rc != 0:
        raise ValueError(f"oracle verify_tree rejected its arguments (code {rc})")
    return out


def kv_commit(kv, blk, n_keep, length, keep=None):
    """KV commit on host arrays.  kv: [batch][Lmax][row] array of any dtype (rows are opaque bytes),
    changed in place; keep [batch][k] int32 or None (the prefix); n_keep, length [batch] int32
    (length changed in place).  Returns the status array."""
    assert kv.flags.c_contiguous
    batch, Lmax = kv.shape[0], kv.shape[1]
    row_bytes = kv.strides[1]
    keep_a = None if keep is None else np.ascontiguousarray(keep, dtype=np.int32)
    nk = np.ascontiguousarray(n_keep, dtype=np.int32)
    assert length.dtype == np.int32 and length.flags.c_contiguous
    st = np.zeros(batch, np.int32)
    rc = lib().psispec_oracle_kv_commit(
        _ptr(kv), kv.strides[0], row_bytes, Lmax, blk, _ptr(keep_a),
        0 if keep_a is None else keep_a.shape[1], _ptr(nk), _ptr(length), _ptr(st), batch)
    if rc != 0:
        raise ValueError(f"oracle kv_commit rejected its arguments (code {rc})")
    return st


def verify_tree_sampled(p, q, parent, node_tokens, max_depth, T=1.0, top_p=1.0, seed=0, step=0,
                        request_base=0, u_accept=None, u_resample=None, want_resid=False):
    """Tree verify with candidates drawn from q: p, q [batch][N+1][V] (row 0 = root, row j+1 =
    node j; q row v+1 is the distribution node v's children were drawn from)."""
    p = np.ascontiguousarray(p)
    q = np.ascontiguousarray(q)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    node_tokens = np.ascontiguousarray(node_tokens, dtype=np.int32)
    batch, N1, V = p.shape
    N = N1 - 1
    if q.shape != p.shape or q.dtype != p.dtype:
        raise ValueError("q must match p")
    if parent.shape != (batch, N) or node_tokens.shape != (batch, N):
        raise ValueError("parent and node_tokens must be [batch][N]")
    ua = None if u_accept is None else np.ascontiguousarray(u_accept, dtype=np.float64)
    ur = None if u_resample is None else np.ascontiguousarray(u_resample, dtype=np.float64)
    out = dict(
        accept_len=np.zeros(batch, np.int32), accept_nodes=np.zeros((batch, max_depth), np.int32),
        out_tokens=np.zeros((batch, max_depth + 1), np.int32),
        node_ratios=np.zeros((batch, N), np.float64), status=np.zeros(batch, np.int32),
        margin_accept=np.zeros((batch, N), np.float64), margin_sample=np.zeros(batch, np.float64),
        margin_topp=np.zeros((batch, 2 * (N + 1)), np.float64))
    if want_resid:
        out["resid_w"] = np.zeros((batch, V), np.float64)
        out["resid_S"] = np.zeros(batch, np.float64)
    rc = lib().psispec_oracle_verify_tree_sampled(
        _ptr(p), _ptr(q), _dtype_code(p), _ptr(parent), _ptr(node_tokens), batch, N, V, max_depth,
        float(T), float(top_p), seed & (2**64 - 1), step, request_base, _ptr(ua), _ptr(ur),
        _ptr(out["accept_len"]), _ptr(out["accept_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out["node_ratios"]), _ptr(out["status"]), _ptr(out["margin_accept"]),
        _ptr(out["margin_sample"]), _ptr(out["margin_topp"]), _ptr(out.get("resid_w")),
        _ptr(out.get("resid_S")))
    if rc != 0:
        raise ValueError(f"oracle verify_tree_sampled rejected its arguments (code {rc})")
    return out


def lmhead_logits(h, W, A=None, Bl=None, scale=1.0):
    """fp64 logits of bf16 (uint16 bit pattern) hidden states h[M][H] times W[H][V] (+ LoRA)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    M, H = h.shape
    V = W.shape[1]
    r = 0
    if A is not None:
        A = np.ascontiguousarray(A, dtype=np.uint16)
        Bl = np.ascontiguousarray(Bl, dtype=np.uint16)
        r = A.shape[1]
    out = np.zeros((M, V), dtype=np.float64)
    rc = lib().psispec_oracle_lmhead_logits(_ptr(h), _ptr(W), _ptr(A), _ptr(Bl), float(scale), M, H,
                                            V, r, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle lmhead_logits rejected its arguments (code {rc})")
    return out


def lmhead_logits_rows(h, W, A=None, Bl=None, scale=1.0):
    """fp64 logits of bf16 hidden rows h[M][H] (uint16 bit patterns) times W[H][V] (+ the LoRA
    delta scale (h A) Bl, A[H][r], Bl[r][V]): the arithmetic of lmhead_logits with numpy's fp64
    matmul as the product, for full-size rows where the plain loops would take minutes.  W (and
    A, Bl) may also be given already widened to float64."""
    def val(x):
        x = np.asarray(x)
        if x.dtype == np.float64:
            return x
        x = np.ascontiguousarray(x, dtype=np.uint16)
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    hv = val(h)
    out = hv @ val(W)
    if A is not None and np.asarray(A).size:
        out += scale * ((hv @ val(A)) @ val(Bl))
    return out


def widen_bf16(x):
    """float64 values of bf16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
