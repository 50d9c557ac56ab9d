"""Psi-Spec verify step on MI355X: Python binding of libpsispec (HIP, gfx950).

The functions below only marshal arguments: they check shapes, allocate outputs and the workspace
with torch on the tensors' device, and call the C ABI declared in include/psispec.h on torch's
current stream.  Every step of the verify runs in the library's HIP kernels; there is no fallback:
if libpsispec.so is missing or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpsispec.so")

PSISPEC_F32, PSISPEC_BF16 = 0, 1
PSISPEC_FIRST_FROM_TARGET = 1
PSISPEC_MAX_CHILDREN_SHIFT = 4  # flags bits 4..7: bound on children per node (sampled tree)
ST_NONFINITE, ST_BAD_TOKEN, ST_Q_ZERO, ST_RESID_ZERO, ST_BAD_PARENT = 1, 2, 4, 8, 16
ST_BAD_KEEP = 32

EXPORTS = ("psispec_verify_linear_workspace", "psispec_verify_linear",
           "psispec_verify_linear_noalloc",
           "psispec_verify_tree_workspace", "psispec_verify_tree", "psispec_lmhead_verify_workspace",
           "psispec_lmhead_verify", "psispec_sample_drafts_workspace", "psispec_sample_drafts",
           "psispec_kv_commit", "psispec_strerror", "psispec_timing_enable",
           "psispec_timing_read", "psispec_peak_read", "psispec_peak_mfma")


class PsispecError(RuntimeError):
    pass


class psispec_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_double), ("top_p", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32),
                ("request_base", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


_lib = None


def lib():
    """Load libpsispec.so (built in-tree by `python -m lossless_draft_verification_spec_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PsispecError(f"{LIB_PATH} is missing: build it with "
                               "`python -m lossless_draft_verification_spec_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.psispec_verify_linear_workspace.argtypes = [i32, i32, i32, i32]
        L.psispec_verify_linear_workspace.restype = sz
        L.psispec_verify_linear.argtypes = [P, P, i32, P, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
        L.psispec_verify_linear.restype = i32
        L.psispec_verify_linear_noalloc.argtypes = [P, P, i32, P, i32, i32, i32, P, P, P, P, P, P,
                                                    P]
        L.psispec_verify_linear_noalloc.restype = i32
        L.psispec_verify_tree_workspace.argtypes = [i32, i32, i32, i32]
        L.psispec_verify_tree_workspace.restype = sz
        L.psispec_verify_tree.argtypes = [P, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                          sz, P]
        L.psispec_verify_tree.restype = i32
        L.psispec_lmhead_verify_workspace.argtypes = [i32, i32, i32, i32, i32]
        L.psispec_lmhead_verify_workspace.restype = sz
        L.psispec_lmhead_verify.argtypes = ([P, P, P, P, P, ctypes.c_float, i32, i32, i32, i32, i32,
                                             P, P, P, P, P, P, P, P, P, P, sz, P])
        L.psispec_lmhead_verify.restype = i32
        L.psispec_sample_drafts_workspace.argtypes = [i32, i32, i32, i32]
        L.psispec_sample_drafts_workspace.restype = sz
        L.psispec_sample_drafts.argtypes = [P, ctypes.c_int64, P, i32, i32, i32, i32, P, P, P, P, sz,
                                            P]
        L.psispec_sample_drafts.restype = i32
        L.psispec_kv_commit.argtypes = [P, ctypes.c_int64, ctypes.c_int64, i32, i32, P, i32, P, P, P,
                                        i32, P]
        L.psispec_kv_commit.restype = i32
        L.psispec_strerror.argtypes = [i32]
        L.psispec_strerror.restype = ctypes.c_char_p
        L.psispec_timing_enable.argtypes = [i32]
        L.psispec_timing_enable.restype = i32
        L.psispec_peak_read.argtypes = [P, sz, P, i32, P]
        L.psispec_peak_read.restype = i32
        L.psispec_peak_mfma.argtypes = [ctypes.c_int64, P, i32, P]
        L.psispec_peak_mfma.restype = i32
        L.psispec_timing_read.argtypes = [P, P, P, i32]
        L.psispec_timing_read.restype = i32
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise PsispecError(f"{what}: {lib().psispec_strerror(rc).decode()} (code {rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PSISPEC_BF16
    if t.dtype == torch.float32:
        return PSISPEC_F32
    raise PsispecError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise PsispecError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise PsispecError(f"{name} must be contiguous")
    return t.data_ptr()


def _same_dev(t: torch.Tensor, dev, name: str):
    if t.device != dev:
        raise PsispecError(f"{name} is on {t.device}, expected {dev}")


def _out_check(t: torch.Tensor | None, shape, dtype, dev, name: str, exact: bool = True):
    """A caller-supplied output: a contiguous GPU tensor on `dev` of `dtype` holding `shape`
    (exactly, or at least that many elements): the library writes through its raw pointer."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.get_device() != dev.index:
        raise PsispecError(f"{name} must be a GPU tensor on {dev}")
    if not t.is_contiguous():
        raise PsispecError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise PsispecError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape == shape:  # the common case: exactly the shape asked for
        return
    need = 1
    for n in shape:
        need *= int(n)
    if exact or t.numel() < need:
        raise PsispecError(f"{name} must hold {tuple(shape)} elements, got {tuple(t.shape)}")


def _check_out(out: dict, spec: dict, dev):
    """spec: name -> (shape, dtype, required)."""
    for name, (shape, dtype, required) in spec.items():
        t = out.get(name)
        if t is None:
            if required:
                raise PsispecError(f"out[{name!r}] is required")
            continue
        _out_check(t, shape, dtype, dev, f"out[{name!r}]", exact=False)


def _check_linear_out(out: dict, batch: int, B: int, dev):
    _check_out(out, {"accept_len": ((batch,), torch.int32, True),
                     "out_tokens": ((batch, B + 1), torch.int32, True),
                     "ratios": ((batch, B), torch.float32, False),
                     "accept_mask": ((batch,), torch.int64, False),
                     "status": ((batch,), torch.int32, False)}, dev)


def _ptr(t):
    return None if t is None else t.data_ptr()  # an int: ctypes passes it as the void* argument


def _sampling(temperature, top_p, seed, step, request_base, flags):
    return psispec_sampling(float(temperature), float(top_p), int(seed) & (2**64 - 1),
                            int(step) & 0xFFFFFFFF, int(request_base) & 0xFFFFFFFF, int(flags), 0)


# the current device's current stream as a raw pointer (torch's own accessor when it has one:
# torch.cuda.current_stream() builds a Stream object, a few microseconds per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def linear_workspace_bytes(batch, B, V, dtype) -> int:
    return int(lib().psispec_verify_linear_workspace(batch, B, V, dtype))


def tree_workspace_bytes(batch, N, V, dtype) -> int:
    return int(lib().psispec_verify_tree_workspace(batch, N, V, dtype))


def psispec_verify_linear(p_logits: torch.Tensor, q_logits: torch.Tensor, draft_tokens: torch.Tensor,
                          temperature: float = 1.0, top_p: float = 1.0, seed: int = 0, step: int = 0,
                          request_base: int = 0, flags: int = 0, workspace: torch.Tensor | None = None,
                          out: dict | None = None, stream=None) -> dict:
    """Linear verify.  p_logits [batch][B+1][V], q_logits [batch][B][V] (bf16 or fp32, same dtype),
    draft_tokens [batch][B] int32, all on one GPU.  Returns accept_len [batch], out_tokens
    [batch][B+1], ratios [batch][B] (fp32), accept_mask [batch] (int64 bit pattern), status [batch].
    Asynchronous on the current stream."""
    if p_logits.dim() != 3 or q_logits.dim() != 3:
        raise PsispecError("p_logits must be [batch][B+1][V] and q_logits [batch][B][V]")
    batch, Bp1, V = p_logits.shape
    B = Bp1 - 1
    if tuple(q_logits.shape) != (batch, B, V) or q_logits.dtype != p_logits.dtype:
        raise PsispecError("q_logits must be [batch][B][V] with the dtype of p_logits")
    if tuple(draft_tokens.shape) != (batch, B) or draft_tokens.dtype != torch.int32:
        raise PsispecError("draft_tokens must be int32 [batch][B]")
    dt = _dtype_code(p_logits)
    dev = p_logits.device
    for name, t in (("p_logits", p_logits), ("q_logits", q_logits), ("draft_tokens", draft_tokens)):
        _dev(t, name)
        if t.device != dev:
            raise PsispecError(f"{name} is on {t.device}, expected {dev}")
    if out is None:
        out = dict(accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(batch, B + 1, dtype=torch.int32, device=dev),
                   ratios=torch.empty(batch, B, dtype=torch.float32, device=dev),
                   accept_mask=torch.empty(batch, dtype=torch.int64, device=dev),
                   status=torch.empty(batch, dtype=torch.int32, device=dev))
    else:
        _check_linear_out(out, batch, B, dev)
    need = linear_workspace_bytes(batch, B, V, dt)
    if need == 0:
        raise PsispecError("unsupported sizes (B must be 1..64)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    s = _sampling(temperature, top_p, seed, step, request_base, flags)
    rc = lib().psispec_verify_linear(
        _ptr(p_logits), _ptr(q_logits), dt, _ptr(draft_tokens), batch, B, V, ctypes.byref(s),
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("ratios")),
        _ptr(out.get("accept_mask")), _ptr(out.get("status")), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check(rc, "psispec_verify_linear")
    return out


def psispec_verify_linear_noalloc(p_logits: torch.Tensor, q_logits: torch.Tensor,
                                  draft_tokens: torch.Tensor, out: dict, temperature: float = 1.0,
                                  top_p: float = 1.0, seed: int = 0, step: int = 0,
                                  request_base: int = 0, flags: int = 0, stream=None) -> dict:
    """psispec_verify_linear through the entry point that allocates nothing (its scratch is the
    library's fixed 64 MiB device array): the caller passes the output tensors in `out`
    (accept_len, out_tokens required; ratios, accept_mask, status optional)."""
    if p_logits.dim() != 3 or q_logits.dim() != 3:
        raise PsispecError("p_logits must be [batch][B+1][V] and q_logits [batch][B][V]")
    batch, Bp1, V = p_logits.shape
    B = Bp1 - 1
    if tuple(q_logits.shape) != (batch, B, V) or q_logits.dtype != p_logits.dtype:
        raise PsispecError("q_logits must be [batch][B][V] with the dtype of p_logits")
    if tuple(draft_tokens.shape) != (batch, B) or draft_tokens.dtype != torch.int32:
        raise PsispecError("draft_tokens must be int32 [batch][B]")
    dt = _dtype_code(p_logits)
    dev = p_logits.device
    for name, t in (("p_logits", p_logits), ("q_logits", q_logits), ("draft_tokens", draft_tokens)):
        _dev(t, name)
        _same_dev(t, dev, name)
    _check_linear_out(out, batch, B, dev)
    s = _sampling(temperature, top_p, seed, step, request_base, flags)
    rc = lib().psispec_verify_linear_noalloc(
        _ptr(p_logits), _ptr(q_logits), dt, _ptr(draft_tokens), batch, B, V, ctypes.byref(s),
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("ratios")),
        _ptr(out.get("accept_mask")), _ptr(out.get("status")), _stream(stream))
    _check(rc, "psispec_verify_linear_noalloc")
    return out


def psispec_verify_tree(p_logits: torch.Tensor, parent: torch.Tensor, node_tokens: torch.Tensor,
                        max_depth: int, temperature: float = 1.0, top_p: float = 1.0, seed: int = 0,
                        step: int = 0, request_base: int = 0, q_logits: torch.Tensor | None = None,
                        max_children: int = 0, workspace: torch.Tensor | None = None,
                        out: dict | None = None, stream=None) -> dict:
    """Tree verify.  p_logits [batch][N+1][V] (row 0 = root, row j+1 = node j), parent and
    node_tokens int32 [batch][N].  With q_logits ([batch][N+1][V], p's dtype: row v+1 is the
    distribution node v's children were drawn from) the candidates are taken as drawn from the
    draft and verified by recursive rejection; without it, as chosen (e.g. top-k).  Returns
    accept_len, accept_nodes [batch][max_depth], out_tokens [batch][max_depth+1], node_ratios
    [batch][N], status.  max_children (with q_logits only, 1..8; 0 = not given): no node has more
    children than this, so the verify skips the residual passes for more; a node with more is
    reported as ST_BAD_PARENT."""
    if p_logits.dim() != 3:
        raise PsispecError("p_logits must be [batch][N+1][V]")
    batch, Np1, V = p_logits.shape
    N = Np1 - 1
    dt = _dtype_code(p_logits)
    dev = p_logits.device
    _dev(p_logits, "p_logits")
    for name, t in (("parent", parent), ("node_tokens", node_tokens)):
        if tuple(t.shape) != (batch, N) or t.dtype != torch.int32:
            raise PsispecError(f"{name} must be int32 [batch][N]")
        _dev(t, name)
        _same_dev(t, dev, name)
    if q_logits is not None:
        if tuple(q_logits.shape) != tuple(p_logits.shape) or q_logits.dtype != p_logits.dtype:
            raise PsispecError("q_logits must be [batch][N+1][V] with the dtype of p_logits")
        _dev(q_logits, "q_logits")
        _same_dev(q_logits, dev, "q_logits")
    if out is None:
        out = dict(accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                   accept_nodes=torch.empty(batch, max_depth, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(batch, max_depth + 1, dtype=torch.int32, device=dev),
                   node_ratios=torch.empty(batch, N, dtype=torch.float32, device=dev),
                   status=torch.empty(batch, dtype=torch.int32, device=dev))
    else:
        _check_out(out, {"accept_len": ((batch,), torch.int32, True),
                         "accept_nodes": ((batch, max_depth), torch.int32, True),
                         "out_tokens": ((batch, max_depth + 1), torch.int32, True),
                         "node_ratios": ((batch, N), torch.float32, False),
                         "status": ((batch,), torch.int32, False)}, dev)
    need = tree_workspace_bytes(batch, N, V, dt)
    if need == 0:
        raise PsispecError("unsupported sizes (N must be 1..1024)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if not 0 <= int(max_children) <= 8:
        raise PsispecError("max_children must be 0..8")
    if max_children and q_logits is None:
        raise PsispecError("max_children applies to trees drawn from the draft (q_logits)")
    s = _sampling(temperature, top_p, seed, step, request_base,
                  int(max_children) << PSISPEC_MAX_CHILDREN_SHIFT)
    rc = lib().psispec_verify_tree(
        _ptr(p_logits), _ptr(q_logits), dt, _ptr(parent), _ptr(node_tokens), batch, N, V,
        int(max_depth), ctypes.byref(s), _ptr(out["accept_len"]), _ptr(out["accept_nodes"]),
        _ptr(out["out_tokens"]), _ptr(out.get("node_ratios")), _ptr(out.get("status")),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "psispec_verify_tree")
    return out


def lmhead_workspace_bytes(batch, B, H, V, r) -> int:
    return int(lib().psispec_lmhead_verify_workspace(batch, B, H, V, r))


def psispec_lmhead_verify(h_ar: torch.Tensor, h_draft: torch.Tensor, W: torch.Tensor,
                          draft_tokens: torch.Tensor, lora_A: torch.Tensor | None = None,
                          lora_B: torch.Tensor | None = None, lora_scale: float = 1.0,
                          temperature: float = 1.0, top_p: float = 1.0, seed: int = 0,
                          step: int = 0, request_base: int = 0, flags: int = 0,
                          p_logits_dbg: torch.Tensor | None = None,
                          q_logits_dbg: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, out: dict | None = None,
                          stream=None) -> dict:
    """LM head + linear verify.  h_ar bf16 [batch][B+1][H], h_draft bf16 [batch][B][H], W bf16
    [H][V], LoRA lora_A bf16 [H][r] and lora_B bf16 [r][V] (or None), draft_tokens int32
    [batch][B].  The logits are never materialised unless p_logits_dbg [batch][B+1][V] and
    q_logits_dbg [batch][B][V] (fp32) are given (required with top_p < 1).  Returns the outputs of
    psispec_verify_linear."""
    if h_ar.dim() != 3 or h_draft.dim() != 3 or W.dim() != 2:
        raise PsispecError("h_ar must be [batch][B+1][H], h_draft [batch][B][H] and W [H][V]")
    batch, Bp1, H = h_ar.shape
    B = Bp1 - 1
    V = W.shape[1]
    if tuple(h_draft.shape) != (batch, B, H) or W.shape[0] != H:
        raise PsispecError("h_draft must be [batch][B][H] and W [H][V]")
    dev = h_ar.device
    for name, t in (("h_ar", h_ar), ("h_draft", h_draft), ("W", W)):
        if t.dtype != torch.bfloat16:
            raise PsispecError(f"{name} must be bfloat16")
        _dev(t, name)
        _same_dev(t, dev, name)
    r = 0
    if lora_A is not None and lora_A.numel():
        r = lora_A.shape[1]
        if (lora_A.dim() != 2 or lora_A.shape[0] != H or lora_B is None
                or tuple(lora_B.shape) != (r, V)):
            raise PsispecError("lora_A must be [H][r] and lora_B [r][V]")
        for name, t in (("lora_A", lora_A), ("lora_B", lora_B)):
            if t.dtype != torch.bfloat16:
                raise PsispecError(f"{name} must be bfloat16")
            _dev(t, name)
            _same_dev(t, dev, name)
    else:
        lora_A = lora_B = None
    if tuple(draft_tokens.shape) != (batch, B) or draft_tokens.dtype != torch.int32:
        raise PsispecError("draft_tokens must be int32 [batch][B]")
    _dev(draft_tokens, "draft_tokens")
    _same_dev(draft_tokens, dev, "draft_tokens")
    if (p_logits_dbg is None) != (q_logits_dbg is None):
        raise PsispecError("p_logits_dbg and q_logits_dbg go together")
    if p_logits_dbg is not None:
        _out_check(p_logits_dbg, (batch, B + 1, V), torch.float32, dev, "p_logits_dbg")
        _out_check(q_logits_dbg, (batch, B, V), torch.float32, dev, "q_logits_dbg")
    if out is None:
        out = dict(accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(batch, B + 1, dtype=torch.int32, device=dev),
                   ratios=torch.empty(batch, B, dtype=torch.float32, device=dev),
                   accept_mask=torch.empty(batch, dtype=torch.int64, device=dev),
                   status=torch.empty(batch, dtype=torch.int32, device=dev))
    else:
        _check_linear_out(out, batch, B, dev)
    need = lmhead_workspace_bytes(batch, B, H, V, r)
    if need == 0:
        raise PsispecError("unsupported sizes (H a multiple of 64, V a multiple of 8, r <= 64, "
                           "B 1..64)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    s = _sampling(temperature, top_p, seed, step, request_base, flags)
    rc = lib().psispec_lmhead_verify(
        _ptr(h_ar), _ptr(h_draft), _ptr(W), _ptr(lora_A), _ptr(lora_B), float(lora_scale),
        batch, B, H, V, r, _ptr(draft_tokens), ctypes.byref(s), _ptr(out["accept_len"]),
        _ptr(out["out_tokens"]), _ptr(out.get("ratios")), _ptr(out.get("accept_mask")),
        _ptr(out.get("status")), _ptr(p_logits_dbg), _ptr(q_logits_dbg), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check(rc, "psispec_lmhead_verify")
    return out


def drafts_workspace_bytes(batch, B, V, dtype) -> int:
    return int(lib().psispec_sample_drafts_workspace(batch, B, V, dtype))


def psispec_sample_drafts(q_logits: torch.Tensor | None, ar_logits: torch.Tensor | None = None,
                          B: int | None = None, temperature: float = 1.0, top_p: float = 1.0,
                          seed: int = 0, step: int = 0, request_base: int = 0, flags: int = 0,
                          workspace: torch.Tensor | None = None, out: dict | None = None,
                          stream=None) -> dict:
    """Drafting step.  q_logits [batch][B][V] (bf16 or fp32); with FIRST_FROM_TARGET, d_0 comes from
    ar_logits: a [batch][V] tensor whose rows are contiguous (any row stride, e.g. p[:, 0, :]) or a
    contiguous [batch][k][V] tensor (row 0 of each request is read).  q_logits may be None with
    FIRST_FROM_TARGET when B == 1.  Returns draft_tokens [batch][B] int32 and status [batch][B]."""
    fft = (flags & PSISPEC_FIRST_FROM_TARGET) != 0
    ref = q_logits if q_logits is not None else ar_logits
    if ref is None:
        raise PsispecError("q_logits is required (or ar_logits with FIRST_FROM_TARGET and B == 1)")
    if q_logits is not None:
        if q_logits.dim() != 3:
            raise PsispecError("q_logits must be [batch][B][V]")
        batch, B, V = q_logits.shape
        _dev(q_logits, "q_logits")
    else:
        if not fft or (B not in (None, 1)):
            raise PsispecError("q_logits may be omitted only with FIRST_FROM_TARGET and B == 1")
        batch, V, B = ar_logits.shape[0], ar_logits.shape[-1], 1
    dt = _dtype_code(ref)
    dev = ref.device
    stride = 0
    if fft:
        if ar_logits is None:
            raise PsispecError("FIRST_FROM_TARGET needs ar_logits")
        if ar_logits.dtype != ref.dtype or ar_logits.shape[0] != batch or ar_logits.shape[-1] != V:
            raise PsispecError("ar_logits must hold [batch] rows of V elements of q's dtype")
        if not ar_logits.is_cuda or ar_logits.device != dev:
            raise PsispecError(f"ar_logits must be on {dev}")
        if ar_logits.dim() == 2:
            if ar_logits.stride(1) != 1 or ar_logits.stride(0) < V:
                raise PsispecError("ar_logits rows must be contiguous and not overlap")
            stride = ar_logits.stride(0)
        elif ar_logits.dim() == 3:
            _dev(ar_logits, "ar_logits")
            stride = ar_logits.shape[1] * V
        else:
            raise PsispecError("ar_logits must be [batch][V] or [batch][k][V]")
    if out is None:
        out = dict(draft_tokens=torch.empty(batch, B, dtype=torch.int32, device=dev),
                   status=torch.empty(batch, B, dtype=torch.int32, device=dev))
    else:
        _check_out(out, {"draft_tokens": ((batch, B), torch.int32, True),
                         "status": ((batch, B), torch.int32, False)}, dev)
    need = drafts_workspace_bytes(batch, B, V, dt)
    if need == 0:
        raise PsispecError("unsupported sizes (B must be 1..64)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    s = _sampling(temperature, top_p, seed, step, request_base, flags)
    rc = lib().psispec_sample_drafts(
        _ptr(ar_logits) if fft else None, stride, _ptr(q_logits), dt, batch, B, V, ctypes.byref(s),
        _ptr(out["draft_tokens"]), _ptr(out.get("status")), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _check(rc, "psispec_sample_drafts")
    return out


def psispec_kv_commit(kv: torch.Tensor, blk: int, n_keep: torch.Tensor, length: torch.Tensor,
                      keep: torch.Tensor | None = None, status: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor | None:
    """KV commit after a verify.  kv: contiguous GPU tensor [batch][Lmax][...] (any dtype; a
    position's row is kv[r][t], opaque bytes, a multiple of 16 bytes); the verify forward wrote the
    block's blk rows at positions length[r] .. length[r]+blk-1.  The kept rows keep[r][:n_keep[r]]
    (int32 [batch][k], strictly increasing; None: the first n_keep rows) move to length[r] onwards
    and length (int32 [batch]) grows by n_keep, in place.  Returns `status` (int32 [batch],
    ST_BAD_KEEP for an invalid request) when given."""
    if kv.dim() < 2:
        raise PsispecError("kv must be [batch][Lmax][...]")
    batch, Lmax = kv.shape[0], kv.shape[1]
    _dev(kv, "kv")
    es = kv.element_size()
    row_bytes = (kv.numel() // max(1, batch * Lmax)) * es
    for name, t in (("n_keep", n_keep), ("length", length)):
        if tuple(t.shape) != (batch,) or t.dtype != torch.int32:
            raise PsispecError(f"{name} must be int32 [batch]")
        _dev(t, name)
        _same_dev(t, kv.device, name)
    ks = 0
    if keep is not None:
        if keep.dim() != 2 or keep.shape[0] != batch or keep.dtype != torch.int32:
            raise PsispecError("keep must be int32 [batch][k]")
        _dev(keep, "keep")
        _same_dev(keep, kv.device, "keep")
        ks = keep.shape[1]
    _out_check(status, (batch,), torch.int32, kv.device, "status", exact=False)
    rc = lib().psispec_kv_commit(_ptr(kv), kv.stride(0) * es, row_bytes, Lmax, int(blk), _ptr(keep),
                                 ks, _ptr(n_keep), _ptr(length), _ptr(status), batch,
                                 _stream(stream))
    _check(rc, "psispec_kv_commit")
    return status


def peak_read(buf: torch.Tensor, out: torch.Tensor, blocks: int, stream=None):
    """Read every 16-byte word of `buf` once (measured HBM read ceiling); out: uint32/int32 [blocks]."""
    _dev(buf, "buf")
    _dev(out, "out")
    if out.numel() < blocks or out.element_size() != 4:
        raise PsispecError("out must hold one 32-bit word per block")
    _check(lib().psispec_peak_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                   int(blocks), _stream(stream)), "psispec_peak_read")


def peak_mfma(iters: int, out: torch.Tensor, blocks: int, stream=None):
    """`iters` rounds of 16 bf16 MFMAs per wave in `blocks` four-wave workgroups (measured MFMA
    issue ceiling); out: float32 [blocks * 256]."""
    _dev(out, "out")
    if out.numel() < blocks * 256 or out.dtype != torch.float32:
        raise PsispecError("out must be float32 with blocks * 256 elements")
    _check(lib().psispec_peak_mfma(int(iters), _ptr(out), int(blocks), _stream(stream)),
           "psispec_peak_mfma")


def timing_enable(on: bool = True):
    _check(lib().psispec_timing_enable(1 if on else 0), "psispec_timing_enable")


def timing_read(max_kernels: int = 32) -> dict:
    """{kernel name: (total device ms, launches)} since timing_enable (synchronises)."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    ms = (ctypes.c_float * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = lib().psispec_timing_read(names, ms, cnt, max_kernels)
    res = {}
    for i in range(n):
        nm = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
        res[nm] = (float(ms[i]), int(cnt[i]))
    return res
