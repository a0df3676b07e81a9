"""ctypes binding of libattn.so.

Argument marshalling only: torch tensors supply device memory and the current
stream, every step of the computation runs in the library's HIP kernels.  The
raw entry points keep the C names (``attn_fwd``, ``attn_verify``,
``attn_verify_noalloc``, ``attn_verify_tree``, ``attn_verify_paged``, ``attn_verify_workspace_bytes``,
``attn_spec_accept``, ``attn_spec_accept_workspace_bytes``, ``attn_bwd``,
``attn_bwd_workspace_bytes``, ``attn_strerror``); ``fwd``, ``bwd``,
``verify``, ``verify_tree``, ``verify_paged`` and ``spec_accept`` are
tensor-level conveniences over them.  Importing this module raises if the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4
ATTN_ERR_TOO_LARGE = -5

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_04_amd.build`")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

lib.attn_fwd.restype = _i
lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]
lib.attn_verify_workspace_bytes.restype = _sz
lib.attn_verify_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]  # B, H, Hkv, kq, d
lib.attn_verify.restype = _i
lib.attn_verify.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
lib.attn_verify_noalloc.restype = _i
lib.attn_verify_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
lib.attn_verify_tree.restype = _i
lib.attn_verify_tree.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                                 _vp]
lib.attn_verify_paged.restype = _i
lib.attn_verify_paged.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                  _vp, _sz, _vp]
lib.attn_spec_accept_workspace_bytes.restype = _sz
lib.attn_spec_accept_workspace_bytes.argtypes = [_i, _i]  # B, V
lib.attn_spec_accept.restype = _i
lib.attn_spec_accept.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]
lib.attn_bwd_workspace_bytes.restype = _sz
lib.attn_bwd_workspace_bytes.argtypes = [_i, _i, _i]  # B, H, Sq
lib.attn_bwd.restype = _i
lib.attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
lib.attn_strerror.restype = ctypes.c_char_p
lib.attn_strerror.argtypes = [_i]

EXPORTED = ("attn_fwd", "attn_verify", "attn_verify_noalloc", "attn_verify_tree", "attn_verify_paged",
            "attn_verify_workspace_bytes", "attn_spec_accept", "attn_spec_accept_workspace_bytes", "attn_bwd", "attn_bwd_workspace_bytes",
            "attn_strerror")


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {attn_strerror(code)} (code {code})")
        self.code = code


def attn_strerror(code: int) -> str:
    return lib.attn_strerror(code).decode()


def attn_fwd(q, k, v, o, lse, B, H, Hkv, Sq, Sk, d, causal, scale, dtype, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_fwd(q, k, v, o, lse, B, H, Hkv, Sq, Sk, d, int(causal), float(scale), dtype, stream)


def attn_verify_workspace_bytes(B, H, Hkv, kq, d) -> int:
    return int(lib.attn_verify_workspace_bytes(B, H, Hkv, kq, d))


def attn_verify(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, o, lse, B, H, Hkv, kq, d,
                scale, dtype, workspace, workspace_bytes, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_verify(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, o, lse, B, H, Hkv,
                           kq, d, float(scale), dtype, workspace, workspace_bytes, stream)


def attn_verify_noalloc(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, o, lse, B, H, Hkv, kq, d,
                        scale, dtype, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_verify_noalloc(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, o, lse, B, H, Hkv,
                                   kq, d, float(scale), dtype, stream)


def attn_verify_tree(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, tree_mask, o, lse, B, H, Hkv,
                     kq, d, scale, dtype, workspace, workspace_bytes, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_verify_tree(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, tree_mask, o, lse, B, H,
                                Hkv, kq, d, float(scale), dtype, workspace, workspace_bytes, stream)


def attn_verify_paged(q, k_pages, v_pages, block_table, max_blocks_per_seq, num_pages, page_size, seqlens_k,
                      max_seqlen_k, o, lse, B, H, Hkv, kq, d, scale, dtype, workspace, workspace_bytes,
                      stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_verify_paged(q, k_pages, v_pages, block_table, max_blocks_per_seq, num_pages, page_size,
                                 seqlens_k, max_seqlen_k, o, lse, B, H, Hkv, kq, d, float(scale), dtype,
                                 workspace, workspace_bytes, stream)


def attn_spec_accept_workspace_bytes(B, V) -> int:
    return int(lib.attn_spec_accept_workspace_bytes(B, V))


def attn_spec_accept(draft_tokens, draft_probs, target_probs, u_accept, u_sample, n_accepted, out_tokens, B, k, V,
                     workspace, workspace_bytes, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_spec_accept(draft_tokens, draft_probs, target_probs, u_accept, u_sample, n_accepted, out_tokens,
                                B, k, V, workspace, workspace_bytes, stream)


def attn_bwd_workspace_bytes(B, H, Sq) -> int:
    return int(lib.attn_bwd_workspace_bytes(B, H, Sq))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Sq, Sk, d, causal, scale, dtype, workspace,
             workspace_bytes, stream) -> int:
    """Raw C entry point (device pointers as ints); returns the ATTN_* code."""
    return lib.attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Sq, Sk, d, int(causal), float(scale), dtype,
                        workspace, workspace_bytes, stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O, LSE of attention over q [B,H,Sq,d], k/v [B,Hkv,Sk,d] on the current stream."""
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    rc = attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Sq, Sk, d,
                  causal, scale, _dtype_code(q), _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd")
    return out, lse


def verify(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens_k: torch.Tensor,
           max_seqlen_k: int, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O, LSE of q [B,H,kq,d] against caches [B,Hkv,stride,d] with int32 seqlens_k [B]."""
    B, H, kq, d = q.shape
    Hkv, stride = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, kq), dtype=torch.float32, device=q.device)
    need = attn_verify_workspace_bytes(B, H, Hkv, kq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if seqlens_k.dtype != torch.int32:
        raise TypeError("seqlens_k must be int32")
    rc = attn_verify(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), max_seqlen_k, stride,
                     _ptr(out), _ptr(lse), B, H, Hkv, kq, d, scale, _dtype_code(q),
                     _ptr(workspace), workspace.numel(), _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_verify")
    return out, lse


def verify_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 seqlens_k: torch.Tensor, max_seqlen_k: int, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O, LSE of q [B,H,kq,d] against pages [num_pages,Hkv,page_size,d] through an int32
    block table [B, max_blocks] with int32 seqlens_k [B]."""
    B, H, kq, d = q.shape
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, kq), dtype=torch.float32, device=q.device)
    need = attn_verify_workspace_bytes(B, H, Hkv, kq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if seqlens_k.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise TypeError("seqlens_k and block_table must be int32")
    rc = attn_verify_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), block_table.shape[1],
                           num_pages, page_size, _ptr(seqlens_k), max_seqlen_k, _ptr(out), _ptr(lse),
                           B, H, Hkv, kq, d, scale, _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_verify_paged")
    return out, lse


def verify_tree(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens_k: torch.Tensor,
                max_seqlen_k: int, tree_mask: torch.Tensor, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """verify() with the new tokens forming a draft tree: tree_mask [B, kq] (int32 or uint32 bits;
    bit t of row i set iff node i sees new token t)."""
    B, H, kq, d = q.shape
    Hkv, stride = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, kq), dtype=torch.float32, device=q.device)
    need = attn_verify_workspace_bytes(B, H, Hkv, kq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if seqlens_k.dtype != torch.int32 or tree_mask.dtype not in (torch.int32, torch.uint32):
        raise TypeError("seqlens_k must be int32 and tree_mask 32-bit")
    if tuple(tree_mask.shape) != (B, kq):
        raise ValueError("tree_mask must be [B, kq]")
    rc = attn_verify_tree(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), max_seqlen_k, stride,
                          _ptr(tree_mask), _ptr(out), _ptr(lse), B, H, Hkv, kq, d, scale, _dtype_code(q),
                          _ptr(workspace), workspace.numel(), _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_verify_tree")
    return out, lse


def spec_accept(draft_tokens: torch.Tensor, draft_probs: torch.Tensor, target_probs: torch.Tensor,
                u_accept: torch.Tensor, u_sample: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, n_accepted: Optional[torch.Tensor] = None,
                out_tokens: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(n_accepted [B], out_tokens [B, k+1]) of the acceptance rule; draft_tokens [B, k] int32,
    draft_probs [B, k, V] and target_probs [B, k+1, V] fp32, u_accept [B, k] and u_sample [B] fp32.
    The two outputs (int32) are written into n_accepted / out_tokens when given."""
    B, k1, V = target_probs.shape
    k = k1 - 1
    for t, dt in ((draft_tokens, torch.int32), (draft_probs, torch.float32), (target_probs, torch.float32),
                  (u_accept, torch.float32), (u_sample, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"expected {dt}, got {t.dtype}")
    if tuple(draft_tokens.shape) != (B, k) or tuple(draft_probs.shape) != (B, k, V) or \
            tuple(u_accept.shape) != (B, k) or tuple(u_sample.shape) != (B,):
        raise ValueError("inconsistent shapes")
    dev = target_probs.device
    n_acc = torch.empty(B, dtype=torch.int32, device=dev) if n_accepted is None else n_accepted
    out = torch.empty((B, k + 1), dtype=torch.int32, device=dev) if out_tokens is None else out_tokens
    if n_acc.dtype != torch.int32 or tuple(n_acc.shape) != (B,) or out.dtype != torch.int32 or \
            tuple(out.shape) != (B, k + 1):
        raise ValueError("outputs must be int32 [B] and [B, k+1]")
    need = attn_spec_accept_workspace_bytes(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    rc = attn_spec_accept(_ptr(draft_tokens), _ptr(draft_probs), _ptr(target_probs), _ptr(u_accept), _ptr(u_sample),
                          _ptr(n_acc), _ptr(out), B, k, V, _ptr(workspace), workspace.numel(), _stream(target_probs))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_spec_accept")
    return n_acc, out


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
        workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(dQ, dK, dV) for the forward outputs o, lse of fwd(q, k, v) and the upstream gradient dout."""
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = attn_bwd_workspace_bytes(B, H, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rc = attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                  B, H, Hkv, Sq, Sk, d, causal, scale, _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(q))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd")
    return dq, dk, dv
