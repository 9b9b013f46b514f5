"""ctypes binding of libspecverify.so (include/spec_verify.h, include/spec_measure.h).

Argument marshalling only: every step of verification runs in the library's HIP
kernels.  PyTorch supplies device memory (inputs, outputs, a cached scratch
workspace) and the current HIP stream.  If the library is not built, every call
raises -- there is no fallback path.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import torch

from .build import library_path

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_MAX_K = 64
SPEC_MAX_TREE_NODES = 1024
SPEC_MAX_NGRAM_N = 16
SPEC_KNOB_CHUNK_VECTORS = 0
SPEC_KNOB_POLL_LIMIT = 1
SPEC_KNOB_SINGLE_LAUNCH = 2
SPEC_KNOB_XCD_LOCAL = 3
FLAG_INVALID = -1    # count output of a sequence with invalid device data
FLAG_TIMED_OUT = -2  # count output of a sequence whose hand-over wait gave up


class SpecError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, func: str, status: int, name: str, detail: str):
        super().__init__(f"{func} failed: {name}: {detail}")
        self.status = status
        self.status_name = name
        self.detail = detail


_lib = None
_lib_lock = threading.Lock()

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "spec_status_string": (ctypes.c_char_p, [_i32]),
    "spec_last_error": (ctypes.c_char_p, []),
    "spec_verify_chain_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "spec_verify_chain": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_chain_noalloc": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                         _vp, _vp, _vp, _vp, _vp, _vp]),
    "spec_verify_tree_greedy_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "spec_verify_tree_greedy": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ngram_propose": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "spec_ngram_verify": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_tree_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "spec_verify_tree": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_tree_mask": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "spec_commit_path": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _sz, _sz, _sz,
                                _vp, _vp, _vp]),
    "spec_gate_default_config": (None, [_vp]),
    "spec_gate_create": (_i32, [_vp, _vp]),
    "spec_gate_destroy": (None, [_vp]),
    "spec_gate_decide": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "spec_gate_observe": (_i32, [_vp, _vp, _vp, _vp, _i32]),
    "spec_gate_tenant": (_i32, [_vp, ctypes.c_uint64, _vp]),
    "spec_gate_tenant_count": (ctypes.c_int64, [_vp]),
    "spec_timing_enable": (_i32, [_i32]),
    "spec_timing_reset": (_i32, []),
    "spec_timing_collect": (_i32, []),
    "spec_timing_entry": (_i32, [_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_longlong),
                                 ctypes.POINTER(ctypes.c_double)]),
    "spec_set_knob": (_i32, [_i32, _i32]),
    "spec_chain_phase_stamps": (_i32, [_vp, _sz]),
    "spec_get_knob": (_i32, [_i32]),
    "spec_probe_read": (_i32, [_vp, _sz, _sz, _vp, _vp]),
    "spec_probe_copy": (_i32, [_vp, _vp, _sz, _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                path = library_path()
                if not os.path.exists(path):
                    raise RuntimeError(
                        f"{path} is missing: build it with `python -m draft_token_verification_09_amd.build` "
                        "(or __graft_entry__.build()); there is no CPU fallback")
                handle = ctypes.CDLL(path)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def loaded_library_path() -> Optional[str]:
    return library_path() if _lib is not None else None


def _check(func: str, status: int) -> None:
    if status != 0:
        L = lib()
        name = L.spec_status_string(status).decode()
        detail = L.spec_last_error().decode()
        raise SpecError(func, status, name, detail)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape: Tuple[int, ...], device) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# -------------------------------------------------------------------- workspaces

_ws_cache: Dict[Tuple[int, int, str], torch.Tensor] = {}


def workspace(nbytes: int, device: torch.device, stream_handle: int, tag: str) -> torch.Tensor:
    """A device scratch buffer cached per (device, stream, tag), grown when a call needs more.
    The library needs no particular contents in it."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle, tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _aligned_ptr(buf: torch.Tensor) -> Tuple[int, int]:
    p = buf.data_ptr()
    off = (-p) % 256
    return p + off, buf.numel() - off


# -------------------------------------------------------------------- entry points


@dataclass
class ChainResult:
    tokens: torch.Tensor         # [B, K+1] int32, -1 padded
    num_accepted: torch.Tensor   # [B] int32 (-1 = invalid input)
    probs: Optional[torch.Tensor]    # [B, K, 3] float32
    packed: Optional[torch.Tensor]   # [B*(K+1)] int32
    offsets: Optional[torch.Tensor]  # [B+1] int32


def spec_verify_chain_workspace_size(B: int, K: int, V: int, dtype_code: int) -> int:
    return int(lib().spec_verify_chain_workspace_size(B, K, V, dtype_code))


def _chain_call(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                temperature: torch.Tensor, u_accept: torch.Tensor, u_final: torch.Tensor,
                draft_len: Optional[torch.Tensor], want_probs: bool, want_packed: bool,
                out: Optional[ChainResult], workspace_buf: Optional[torch.Tensor], stream, use_workspace=True):
    """Checks the tensors and returns (argument tuple of spec_verify_chain, result, buffers
    the call uses).  Without use_workspace the tuple has no workspace arguments (the
    allocation-free entry point)."""
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits)
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", target_logits.dtype, (B, K, V), dev)
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(u_accept, "u_accept", torch.float32, (B, K), dev)
    _need(u_final, "u_final", torch.float32, (B,), dev)
    if draft_len is not None:
        _need(draft_len, "draft_len", torch.int32, (B,), dev)
    if out is None:
        out = ChainResult(
            tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            num_accepted=torch.empty((B,), dtype=torch.int32, device=dev),
            probs=torch.empty((B, K, 3), dtype=torch.float32, device=dev) if want_probs else None,
            packed=torch.empty((max(1, B * (K + 1)),), dtype=torch.int32, device=dev) if want_packed else None,
            offsets=torch.empty((B + 1,), dtype=torch.int32, device=dev) if want_packed else None,
        )
    s = _stream(stream, dev)
    args = (_ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(draft_len),
            _ptr(temperature), _ptr(u_accept), _ptr(u_final), B, K, V,
            _ptr(out.tokens), _ptr(out.num_accepted), _ptr(out.probs),
            _ptr(out.packed), _ptr(out.offsets))
    buf = None
    if use_workspace:
        need = int(lib().spec_verify_chain_workspace_size(B, K, V, code)) if B > 0 else 0
        buf = workspace_buf if workspace_buf is not None else workspace(need, dev, s, "chain")
        wp, wbytes = _aligned_ptr(buf)
        args += (wp, wbytes)
    args += (s,)
    keep = (target_logits, draft_logits, draft_tokens, temperature, u_accept, u_final, draft_len, buf)
    return args, out, keep


def spec_verify_chain(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                      draft_tokens: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                      u_final: torch.Tensor, draft_len: Optional[torch.Tensor] = None, *,
                      want_probs: bool = True, want_packed: bool = False,
                      out: Optional[ChainResult] = None, workspace_buf: Optional[torch.Tensor] = None,
                      stream=None) -> ChainResult:
    """Batched chain verification (spec_verify_chain).  Shapes: target [B, K+1, V],
    draft [B, K, V] or None (one-hot draft), draft_tokens [B, K] int32, temperature [B]
    float32, u_accept [B, K] float32, u_final [B] float32, draft_len [B] int32 or None."""
    args, out, _ = _chain_call(target_logits, draft_logits, draft_tokens, temperature, u_accept, u_final,
                               draft_len, want_probs, want_packed, out, workspace_buf, stream)
    _check("spec_verify_chain", lib().spec_verify_chain(*args))
    return out


def spec_verify_chain_noalloc(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                              draft_tokens: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                              u_final: torch.Tensor, draft_len: Optional[torch.Tensor] = None, *,
                              out: ChainResult, stream=None) -> ChainResult:
    """spec_verify_chain_noalloc: as spec_verify_chain, with the library's own device scratch
    instead of a workspace.  `out` is required (the library allocates nothing, and neither
    does this wrapper)."""
    args, out, _ = _chain_call(target_logits, draft_logits, draft_tokens, temperature, u_accept, u_final,
                               draft_len, out.probs is not None, out.packed is not None, out, None, stream,
                               use_workspace=False)
    _check("spec_verify_chain_noalloc", lib().spec_verify_chain_noalloc(*args))
    return out


class PreparedCall:
    """An entry point with its arguments checked and marshalled once.  Calling the object
    issues the same call again (same buffers, same stream) for the cost of one foreign
    call, for loops that refill fixed buffers between calls.  It keeps references to
    every buffer it names; their shapes and addresses must not change."""

    def __init__(self, name: str, fn, argtypes, args, result, keep):
        self._name = name
        self._fn = fn
        self._args = tuple(t(v) if v is not None else t() for t, v in zip(argtypes, args))
        self.result = result
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _check(self._name, st)
        return self.result


def prepare_spec_verify_chain(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                              draft_tokens: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                              u_final: torch.Tensor, draft_len: Optional[torch.Tensor] = None, *,
                              want_probs: bool = True, want_packed: bool = False,
                              out: Optional[ChainResult] = None, workspace_buf: Optional[torch.Tensor] = None,
                              stream=None) -> PreparedCall:
    """spec_verify_chain with every argument fixed: returns a PreparedCall whose result is
    the ChainResult that each call overwrites."""
    args, out, keep = _chain_call(target_logits, draft_logits, draft_tokens, temperature, u_accept, u_final,
                                  draft_len, want_probs, want_packed, out, workspace_buf, stream)
    return PreparedCall("spec_verify_chain", lib().spec_verify_chain, _SIGNATURES["spec_verify_chain"][1],
                        args, out, keep)


@dataclass
class TreeResult:
    accept_len: torch.Tensor   # [B] int32 (-1 = invalid input)
    tokens: torch.Tensor       # [B, max_depth+1] int32
    path_nodes: torch.Tensor   # [B, max_depth+1] int32
    argmax: Optional[torch.Tensor]  # [B, N1] int32


def _tree_call(target_logits, parent, node_token, max_depth, want_argmax, out, workspace_buf, stream):
    """Checks the tensors and returns (argument tuple of spec_verify_tree_greedy, result,
    buffers the call uses)."""
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N1, V]")
    B, N1, V = target_logits.shape
    dev = target_logits.device
    code = _dtype_code(target_logits)
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _need(parent, "parent", torch.int32, (B, N1), dev)
    _need(node_token, "node_token", torch.int32, (B, N1), dev)
    D1 = max_depth + 1
    if out is None:
        out = TreeResult(
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            tokens=torch.empty((B, D1), dtype=torch.int32, device=dev),
            path_nodes=torch.empty((B, D1), dtype=torch.int32, device=dev),
            argmax=torch.empty((B, N1), dtype=torch.int32, device=dev) if want_argmax else None,
        )
    s = _stream(stream, dev)
    need = int(lib().spec_verify_tree_greedy_workspace_size(B, N1, V, code)) if B > 0 else 0
    buf = workspace_buf if workspace_buf is not None else workspace(need, dev, s, "tree")
    wp, wbytes = _aligned_ptr(buf)
    args = (_ptr(target_logits), code, _ptr(parent), _ptr(node_token), B, N1, V, max_depth,
            _ptr(out.accept_len), _ptr(out.tokens), _ptr(out.path_nodes), _ptr(out.argmax), wp, wbytes, s)
    return args, out, (target_logits, parent, node_token, buf)


def spec_verify_tree_greedy(target_logits: torch.Tensor, parent: torch.Tensor, node_token: torch.Tensor,
                            max_depth: int, *, want_argmax: bool = True, out: Optional[TreeResult] = None,
                            workspace_buf: Optional[torch.Tensor] = None, stream=None) -> TreeResult:
    """Batched greedy tree verification (spec_verify_tree_greedy).  target [B, N1, V],
    parent [B, N1] int32, node_token [B, N1] int32."""
    args, out, _ = _tree_call(target_logits, parent, node_token, max_depth, want_argmax, out, workspace_buf, stream)
    _check("spec_verify_tree_greedy", lib().spec_verify_tree_greedy(*args))
    return out


def prepare_spec_verify_tree_greedy(target_logits: torch.Tensor, parent: torch.Tensor, node_token: torch.Tensor,
                                    max_depth: int, *, want_argmax: bool = True, out: Optional[TreeResult] = None,
                                    workspace_buf: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """spec_verify_tree_greedy with every argument fixed (see PreparedCall)."""
    args, out, keep = _tree_call(target_logits, parent, node_token, max_depth, want_argmax, out, workspace_buf,
                                 stream)
    return PreparedCall("spec_verify_tree_greedy", lib().spec_verify_tree_greedy,
                        _SIGNATURES["spec_verify_tree_greedy"][1], args, out, keep)


def _tree_sampled_call(target_logits, draft_logits, parent, node_token, temperature, u_accept, u_final,
                       max_depth, out, workspace_buf, stream):
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N1, V]")
    B, N1, V = target_logits.shape
    dev = target_logits.device
    code = _dtype_code(target_logits)
    for t, name in ((target_logits, "target_logits"), (draft_logits, "draft_logits")):
        if t.dtype != target_logits.dtype or tuple(t.shape) != (B, N1, V) or t.device != dev:
            raise ValueError(f"{name} must be [B, N1, V] of one dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _need(parent, "parent", torch.int32, (B, N1), dev)
    _need(node_token, "node_token", torch.int32, (B, N1), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(u_accept, "u_accept", torch.float32, (B, N1), dev)
    _need(u_final, "u_final", torch.float32, (B,), dev)
    D1 = max_depth + 1
    if out is None:
        out = TreeResult(
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            tokens=torch.empty((B, D1), dtype=torch.int32, device=dev),
            path_nodes=torch.empty((B, D1), dtype=torch.int32, device=dev),
            argmax=None,
        )
    s = _stream(stream, dev)
    need = int(lib().spec_verify_tree_workspace_size(B, N1, V, code)) if B > 0 else 0
    buf = workspace_buf if workspace_buf is not None else workspace(need, dev, s, "tree_sampled")
    wp, wbytes = _aligned_ptr(buf)
    args = (_ptr(target_logits), _ptr(draft_logits), code, _ptr(parent), _ptr(node_token), _ptr(temperature),
            _ptr(u_accept), _ptr(u_final), B, N1, V, max_depth, _ptr(out.accept_len), _ptr(out.tokens),
            _ptr(out.path_nodes), wp, wbytes, s)
    return args, out, (target_logits, draft_logits, parent, node_token, temperature, u_accept, u_final, buf)


def spec_verify_tree(target_logits: torch.Tensor, draft_logits: torch.Tensor, parent: torch.Tensor,
                     node_token: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                     u_final: torch.Tensor, max_depth: int, *, out: Optional[TreeResult] = None,
                     workspace_buf: Optional[torch.Tensor] = None, stream=None) -> TreeResult:
    """Stochastic tree verification (spec_verify_tree).  target and draft [B, N1, V],
    parent and node_token [B, N1] int32, temperature [B], u_accept [B, N1], u_final [B]."""
    args, out, _ = _tree_sampled_call(target_logits, draft_logits, parent, node_token, temperature, u_accept,
                                      u_final, max_depth, out, workspace_buf, stream)
    _check("spec_verify_tree", lib().spec_verify_tree(*args))
    return out


def prepare_spec_verify_tree(target_logits: torch.Tensor, draft_logits: torch.Tensor, parent: torch.Tensor,
                             node_token: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                             u_final: torch.Tensor, max_depth: int, *, out: Optional[TreeResult] = None,
                             workspace_buf: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """spec_verify_tree with every argument fixed (see PreparedCall)."""
    args, out, keep = _tree_sampled_call(target_logits, draft_logits, parent, node_token, temperature, u_accept,
                                         u_final, max_depth, out, workspace_buf, stream)
    return PreparedCall("spec_verify_tree", lib().spec_verify_tree, _SIGNATURES["spec_verify_tree"][1], args,
                        out, keep)


@dataclass
class NgramResult:
    draft_tokens: torch.Tensor  # [B, K] int32, -1 padded
    draft_len: torch.Tensor     # [B] int32
    match_n: Optional[torch.Tensor]  # [B] int32


def _ngram_call(context, context_len, n_min, n_max, K, want_match_n, out, stream):
    if context.dim() != 2:
        raise ValueError("context must be [B, L_max]")
    B, L_max = context.shape
    dev = context.device
    _need(context, "context", torch.int32, (B, L_max), dev)
    _need(context_len, "context_len", torch.int32, (B,), dev)
    if out is None:
        out = NgramResult(
            draft_tokens=torch.empty((B, K), dtype=torch.int32, device=dev),
            draft_len=torch.empty((B,), dtype=torch.int32, device=dev),
            match_n=torch.empty((B,), dtype=torch.int32, device=dev) if want_match_n else None,
        )
    s = _stream(stream, dev)
    args = (_ptr(context), _ptr(context_len), B, L_max, n_min, n_max, K,
            _ptr(out.draft_tokens), _ptr(out.draft_len), _ptr(out.match_n), s)
    return args, out, (context, context_len)


def ngram_propose(context: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int, K: int, *,
                  want_match_n: bool = True, out: Optional[NgramResult] = None, stream=None) -> NgramResult:
    """Batched prompt n-gram lookup (ngram_propose).  context [B, L_max] int32, context_len [B] int32."""
    args, out, _ = _ngram_call(context, context_len, n_min, n_max, K, want_match_n, out, stream)
    _check("ngram_propose", lib().ngram_propose(*args))
    return out


@dataclass
class NgramVerifyResult:
    proposal: NgramResult
    verify: ChainResult


def _ngram_verify_call(context, context_len, n_min, n_max, target_logits, temperature, u_accept, u_final,
                       want_probs, want_packed, out, workspace_buf, stream):
    if context.dim() != 2 or target_logits.dim() != 3:
        raise ValueError("context must be [B, L_max] and target_logits [B, K+1, V]")
    B, L_max = context.shape
    B2, K1, V = target_logits.shape
    if B2 != B:
        raise ValueError("context and target_logits must have the same batch")
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits)
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _need(context, "context", torch.int32, (B, L_max), dev)
    _need(context_len, "context_len", torch.int32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(u_accept, "u_accept", torch.float32, (B, K), dev)
    _need(u_final, "u_final", torch.float32, (B,), dev)
    if out is None:
        out = NgramVerifyResult(
            proposal=NgramResult(draft_tokens=torch.empty((B, K), dtype=torch.int32, device=dev),
                                 draft_len=torch.empty((B,), dtype=torch.int32, device=dev),
                                 match_n=torch.empty((B,), dtype=torch.int32, device=dev)),
            verify=ChainResult(
                tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                num_accepted=torch.empty((B,), dtype=torch.int32, device=dev),
                probs=torch.empty((B, K, 3), dtype=torch.float32, device=dev) if want_probs else None,
                packed=torch.empty((max(1, B * (K + 1)),), dtype=torch.int32, device=dev) if want_packed else None,
                offsets=torch.empty((B + 1,), dtype=torch.int32, device=dev) if want_packed else None))
    s = _stream(stream, dev)
    need = int(lib().spec_verify_chain_workspace_size(B, K, V, code)) if B > 0 else 0
    buf = workspace_buf if workspace_buf is not None else workspace(need, dev, s, "chain")
    wp, wbytes = _aligned_ptr(buf)
    p, v = out.proposal, out.verify
    args = (_ptr(context), _ptr(context_len), L_max, n_min, n_max, _ptr(target_logits), code, _ptr(temperature),
            _ptr(u_accept), _ptr(u_final), B, K, V, _ptr(p.draft_tokens), _ptr(p.draft_len), _ptr(p.match_n),
            _ptr(v.tokens), _ptr(v.num_accepted), _ptr(v.probs), _ptr(v.packed), _ptr(v.offsets), wp, wbytes, s)
    return args, out, (context, context_len, target_logits, temperature, u_accept, u_final, buf)


def spec_ngram_verify(context: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int,
                      target_logits: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                      u_final: torch.Tensor, *, want_probs: bool = True, want_packed: bool = False,
                      out: Optional[NgramVerifyResult] = None, workspace_buf: Optional[torch.Tensor] = None,
                      stream=None) -> NgramVerifyResult:
    """Prompt n-gram lookup and the verification of its drafts in one call (spec_ngram_verify).
    context [B, L_max] int32, context_len [B] int32, target_logits [B, K+1, V], temperature [B],
    u_accept [B, K], u_final [B]."""
    args, out, _ = _ngram_verify_call(context, context_len, n_min, n_max, target_logits, temperature, u_accept,
                                      u_final, want_probs, want_packed, out, workspace_buf, stream)
    _check("spec_ngram_verify", lib().spec_ngram_verify(*args))
    return out


def prepare_spec_ngram_verify(context: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int,
                              target_logits: torch.Tensor, temperature: torch.Tensor, u_accept: torch.Tensor,
                              u_final: torch.Tensor, *, want_probs: bool = True, want_packed: bool = False,
                              out: Optional[NgramVerifyResult] = None, workspace_buf: Optional[torch.Tensor] = None,
                              stream=None) -> PreparedCall:
    """spec_ngram_verify with every argument fixed (see PreparedCall)."""
    args, out, keep = _ngram_verify_call(context, context_len, n_min, n_max, target_logits, temperature, u_accept,
                                         u_final, want_probs, want_packed, out, workspace_buf, stream)
    return PreparedCall("spec_ngram_verify", lib().spec_ngram_verify, _SIGNATURES["spec_ngram_verify"][1], args,
                        out, keep)


def prepare_ngram_propose(context: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int, K: int, *,
                          want_match_n: bool = True, out: Optional[NgramResult] = None, stream=None) -> PreparedCall:
    """ngram_propose with every argument fixed (see PreparedCall)."""
    args, out, keep = _ngram_call(context, context_len, n_min, n_max, K, want_match_n, out, stream)
    return PreparedCall("ngram_propose", lib().ngram_propose, _SIGNATURES["ngram_propose"][1], args, out, keep)


@dataclass
class TreeMaskResult:
    mask: Optional[torch.Tensor]   # [B, N1, N1] uint8
    depth: Optional[torch.Tensor]  # [B, N1] int32


def _tree_mask_call(parent, want_mask, want_depth, out, stream):
    if parent.dim() != 2:
        raise ValueError("parent must be [B, N1]")
    B, N1 = parent.shape
    dev = parent.device
    _need(parent, "parent", torch.int32, (B, N1), dev)
    if out is None:
        out = TreeMaskResult(
            mask=torch.empty((B, N1, N1), dtype=torch.uint8, device=dev) if want_mask else None,
            depth=torch.empty((B, N1), dtype=torch.int32, device=dev) if want_depth else None,
        )
    if out.mask is not None:
        _need(out.mask, "mask", torch.uint8, (B, N1, N1), dev)
    if out.depth is not None:
        _need(out.depth, "depth", torch.int32, (B, N1), dev)
    s = _stream(stream, dev)
    args = (_ptr(parent), B, N1, _ptr(out.mask), _ptr(out.depth), s)
    return args, out, (parent,)


def spec_tree_mask(parent: torch.Tensor, *, want_mask: bool = True, want_depth: bool = True,
                   out: Optional[TreeMaskResult] = None, stream=None) -> TreeMaskResult:
    """Tree-attention mask and node depths (spec_tree_mask).  parent [B, N1] int32."""
    args, out, _ = _tree_mask_call(parent, want_mask, want_depth, out, stream)
    _check("spec_tree_mask", lib().spec_tree_mask(*args))
    return out


def prepare_spec_tree_mask(parent: torch.Tensor, *, want_mask: bool = True, want_depth: bool = True,
                           out: Optional[TreeMaskResult] = None, stream=None) -> PreparedCall:
    """spec_tree_mask with every argument fixed (see PreparedCall)."""
    args, out, keep = _tree_mask_call(parent, want_mask, want_depth, out, stream)
    return PreparedCall("spec_tree_mask", lib().spec_tree_mask, _SIGNATURES["spec_tree_mask"][1], args, out, keep)


def _plane_view(t: torch.Tensor, name: str, B: int, rows: int):
    """(planes, entry_bytes, plane_stride_bytes) of a [planes, B, rows, W] tensor whose
    last three dimensions are dense (the plane dimension may be strided)."""
    if t.dim() != 4 or t.shape[1] != B or t.shape[2] != rows:
        raise ValueError(f"{name} must be [planes, {B}, {rows}, W], got {tuple(t.shape)}")
    P_, _, _, W = t.shape
    es = t.element_size()
    if t.stride(3) != 1 or t.stride(2) != W or t.stride(1) != rows * W:
        raise ValueError(f"{name} must be dense in its last three dimensions")
    return P_, W * es, t.stride(0) * es


def _commit_call(kv_nodes, path_nodes, accept_len, cache_len, kv_cache, out_cache_len, stream):
    if kv_nodes.dim() != 4:
        raise ValueError("kv_nodes must be [planes, B, N1, W]")
    planes, B, N1, W = kv_nodes.shape
    dev = kv_nodes.device
    if kv_cache.device != dev or kv_cache.dtype != kv_nodes.dtype:
        raise ValueError("kv_cache must match kv_nodes in device and dtype")
    L_cap = kv_cache.shape[2] if kv_cache.dim() == 4 else -1
    p1, eb, sstride = _plane_view(kv_nodes, "kv_nodes", B, N1)
    p2, eb2, dstride = _plane_view(kv_cache, "kv_cache", B, L_cap)
    if p1 != p2 or eb != eb2:
        raise ValueError("kv_nodes and kv_cache must have the same planes and entry width")
    _need(accept_len, "accept_len", torch.int32, (B,), dev)
    _need(cache_len, "cache_len", torch.int32, (B,), dev)
    P = 0
    if path_nodes is not None:
        if path_nodes.dim() != 2 or path_nodes.shape[0] != B:
            raise ValueError("path_nodes must be [B, P]")
        P = path_nodes.shape[1]
        _need(path_nodes, "path_nodes", torch.int32, (B, P), dev)
    if out_cache_len is None:
        out_cache_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_cache_len, "out_cache_len", torch.int32, (B,), dev)
    s = _stream(stream, dev)
    args = (_ptr(kv_nodes), _ptr(path_nodes), P, _ptr(accept_len), _ptr(cache_len), B, N1, L_cap, planes, eb,
            sstride, dstride, _ptr(kv_cache), _ptr(out_cache_len), s)
    return args, out_cache_len, (kv_nodes, path_nodes, accept_len, cache_len, kv_cache)


def spec_commit_path(kv_nodes: torch.Tensor, path_nodes: Optional[torch.Tensor], accept_len: torch.Tensor,
                     cache_len: torch.Tensor, kv_cache: torch.Tensor, *,
                     out_cache_len: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Copy the root's and the accepted nodes' entries into the cache (spec_commit_path).
    kv_nodes [planes, B, N1, W], kv_cache [planes, B, L_cap, W] (same dtype; the plane
    dimension may be strided), path_nodes [B, P] int32 or None (chain), accept_len and
    cache_len [B] int32.  Returns the new cache lengths [B] int32 (-1 = invalid)."""
    args, out, _ = _commit_call(kv_nodes, path_nodes, accept_len, cache_len, kv_cache, out_cache_len, stream)
    _check("spec_commit_path", lib().spec_commit_path(*args))
    return out


def prepare_spec_commit_path(kv_nodes: torch.Tensor, path_nodes: Optional[torch.Tensor], accept_len: torch.Tensor,
                             cache_len: torch.Tensor, kv_cache: torch.Tensor, *,
                             out_cache_len: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """spec_commit_path with every argument fixed (see PreparedCall)."""
    args, out, keep = _commit_call(kv_nodes, path_nodes, accept_len, cache_len, kv_cache, out_cache_len, stream)
    return PreparedCall("spec_commit_path", lib().spec_commit_path, _SIGNATURES["spec_commit_path"][1],
                        args, out, keep)


# -------------------------------------------------------------------- adaptive gate


class GateConfig(ctypes.Structure):
    _fields_ = [("temperature_limit", ctypes.c_double), ("acceptance_floor", ctypes.c_double),
                ("ema_weight", ctypes.c_double), ("cooldown", ctypes.c_int32)]


class GateTenantStats(ctypes.Structure):
    _fields_ = [("ema", ctypes.c_double), ("state", ctypes.c_int32), ("cooldown", ctypes.c_int32),
                ("observations", ctypes.c_int64), ("accepted", ctypes.c_int64), ("drafted", ctypes.c_int64),
                ("trips", ctypes.c_int64)]


GATE_CLOSED, GATE_OPEN, GATE_HALF_OPEN = 0, 1, 2


class SpecGate:
    """The library's adaptive speculation gate (include/spec_gate.h): host-side state,
    host arrays.  decide() says per request whether to speculate; observe() feeds
    verification outcomes (num_accepted, draft_len) back per tenant."""

    def __init__(self, temperature_limit: Optional[float] = None, acceptance_floor: Optional[float] = None,
                 ema_weight: Optional[float] = None, cooldown: Optional[int] = None):
        L = lib()
        cfg = GateConfig()
        L.spec_gate_default_config(ctypes.byref(cfg))
        if temperature_limit is not None:
            cfg.temperature_limit = temperature_limit
        if acceptance_floor is not None:
            cfg.acceptance_floor = acceptance_floor
        if ema_weight is not None:
            cfg.ema_weight = ema_weight
        if cooldown is not None:
            cfg.cooldown = cooldown
        handle = ctypes.c_void_p()
        _check("spec_gate_create", L.spec_gate_create(ctypes.byref(cfg), ctypes.byref(handle)))
        self._h = handle
        self.config = cfg

    def close(self) -> None:
        if self._h:
            lib().spec_gate_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _host(x, dtype):
        import numpy as np

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(x), dtype=dtype)

    def decide(self, tenant, temperature):
        """Per request: True to speculate.  tenant [B] (uint64 keys), temperature [B]."""
        import numpy as np

        t = self._host(tenant, np.uint64)
        T = self._host(temperature, np.float32)
        if t.shape != T.shape or t.ndim != 1:
            raise ValueError("tenant and temperature must be 1-D of one length")
        out = np.empty(t.shape, dtype=np.int32)
        _check("spec_gate_decide", lib().spec_gate_decide(self._h, t.ctypes.data, T.ctypes.data, t.size,
                                                           out.ctypes.data))
        return out.astype(bool)

    def observe(self, tenant, num_accepted, draft_len) -> None:
        """Feed verification outcomes: tenant [B], num_accepted [B], draft_len [B] (tensors
        on any device or arrays; device tensors are copied to the host)."""
        import numpy as np

        t = self._host(tenant, np.uint64)
        a = self._host(num_accepted, np.int32)
        d = self._host(draft_len, np.int32)
        if not (t.shape == a.shape == d.shape) or t.ndim != 1:
            raise ValueError("tenant, num_accepted and draft_len must be 1-D of one length")
        _check("spec_gate_observe", lib().spec_gate_observe(self._h, t.ctypes.data, a.ctypes.data, d.ctypes.data,
                                                             t.size))

    def tenant(self, key: int) -> GateTenantStats:
        st = GateTenantStats()
        _check("spec_gate_tenant", lib().spec_gate_tenant(self._h, key, ctypes.byref(st)))
        return st

    def tenant_count(self) -> int:
        return int(lib().spec_gate_tenant_count(self._h))


# -------------------------------------------------------------------- measurement hooks


def spec_timing_enable(enable: bool) -> None:
    _check("spec_timing_enable", lib().spec_timing_enable(1 if enable else 0))


def spec_timing_reset() -> None:
    _check("spec_timing_reset", lib().spec_timing_reset())


def spec_timing_collect() -> List[Tuple[str, int, float]]:
    """[(kernel name, launches, total milliseconds)] since the last reset."""
    L = lib()
    n = int(L.spec_timing_collect())
    out = []
    for i in range(n):
        name = ctypes.c_char_p()
        launches = ctypes.c_longlong()
        ms = ctypes.c_double()
        _check("spec_timing_entry", L.spec_timing_entry(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms)))
        out.append((name.value.decode(), int(launches.value), float(ms.value)))
    return out


def spec_set_knob(knob_id: int, value: int) -> None:
    """Process-wide override of a library choice (include/spec_measure.h); value < 0 restores
    the default."""
    _check("spec_set_knob", lib().spec_set_knob(knob_id, value))


def spec_get_knob(knob_id: int) -> int:
    return int(lib().spec_get_knob(knob_id))


@contextlib.contextmanager
def knob(knob_id: int, value: int):
    """Set a knob for the duration of a block, then restore its previous value."""
    old = spec_get_knob(knob_id)
    spec_set_knob(knob_id, value)
    try:
        yield
    finally:
        spec_set_knob(knob_id, old)


def spec_chain_phase_stamps(buffer: Optional[torch.Tensor]) -> None:
    """Start (a device int64 tensor) or stop (None) the phase timestamps of chain calls."""
    if buffer is None:
        _check("spec_chain_phase_stamps", lib().spec_chain_phase_stamps(None, 0))
    else:
        if buffer.dtype != torch.int64 or not buffer.is_cuda or not buffer.is_contiguous():
            raise ValueError("the stamp buffer must be a contiguous int64 CUDA tensor")
        _check("spec_chain_phase_stamps", lib().spec_chain_phase_stamps(buffer.data_ptr(), buffer.numel()))


def spec_probe_read(src: torch.Tensor, out: torch.Tensor, chunk_bytes: int = 65536, stream=None) -> None:
    s = _stream(stream, src.device)
    _check("spec_probe_read", lib().spec_probe_read(src.data_ptr(), src.numel() * src.element_size(), chunk_bytes,
                                                    out.data_ptr(), s))


def spec_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    s = _stream(stream, src.device)
    _check("spec_probe_copy", lib().spec_probe_copy(src.data_ptr(), dst.data_ptr(),
                                                    src.numel() * src.element_size(), s))
