"""ctypes binding of libq3moe.so (include/q3moe.h).

Argument marshalling only: every function checks the tensors' device,
dtype and layout, passes raw pointers and the current HIP stream to the C
entry point of the same name, and raises ``Q3MoeError`` on a non-zero
status.  All arithmetic runs in the HIP kernels.  There is no CPU fallback:
if the library is missing this module raises on import of a function.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import NamedTuple, Optional

import torch

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libq3moe.so"

Q4_K, Q6_K = 1, 2
EXPORTS = (
    "q3moe_status_string", "q3moe_qtype_block_bytes", "q3moe_expert_matrix_bytes",
    "q3moe_route_workspace_bytes", "q3moe_route", "q3moe_group_by_expert",
    "q3moe_expert_ffn_workspace_bytes", "q3moe_expert_ffn_status_offset", "q3moe_expert_ffn",
    "q3moe_attn_prologue", "q3moe_rmsnorm", "q3moe_bf16_gemv", "q3moe_kv_write",
    "q3moe_gqa_attention_workspace_bytes", "q3moe_gqa_attention",
    "q3moe_moe_ffn_workspace_bytes", "q3moe_moe_ffn", "q3moe_moe_ffn_prenorm", "q3moe_bf16_gemv3",
    "q3moe_attn_prologue_kv", "q3moe_persistent_path", "q3moe_moe_ffn_noalloc", "q3moe_moe_ffn_q8",
    "q3moe_embed", "q3moe_output_head", "q3moe_kv_write_rows", "q3moe_prefill_attention",
    "q3moe_moe_stack_workspace_bytes", "q3moe_moe_stack",
)


class Q3MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class _Experts(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("qtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("expert_stride_bytes", ctypes.c_int64)]


class _MoeLayer(ctypes.Structure):
    _fields_ = [("norm_gain", ctypes.c_void_p), ("router", ctypes.c_void_p), ("gate", _Experts),
                ("up", _Experts), ("down", _Experts)]


_P, _I64, _I32, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "q3moe_status_string": (ctypes.c_char_p, [_I32]),
    "q3moe_qtype_block_bytes": (_I32, [_I32]),
    "q3moe_expert_matrix_bytes": (_I64, [_I32, _I64, _I64]),
    "q3moe_route_workspace_bytes": (ctypes.c_size_t, [_I64, _I32]),
    "q3moe_route": (_I32, [_P, _I64, _I64, _P, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P]),
    "q3moe_group_by_expert": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _P]),
    "q3moe_expert_ffn_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "q3moe_expert_ffn_status_offset": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "q3moe_expert_ffn": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _P, _P, _Experts, _Experts,
                                _Experts, _P, _I32, _P, ctypes.c_size_t, _P]),
    "q3moe_attn_prologue": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _F, _F, _P]),
    "q3moe_rmsnorm": (_I32, [_P, _I64, _I64, _P, _F, _P, _P]),
    "q3moe_bf16_gemv": (_I32, [_P, _I64, _I64, _P, _I64, _P, _I32, _P]),
    "q3moe_bf16_gemv3": (_I32, [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64, _P, _F, _P, _P, _P, _P]),
    "q3moe_kv_write": (_I32, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _I64, _P]),
    "q3moe_attn_prologue_kv": (_I32, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _F, _F, _P, _P,
                                      _I64, _P]),
    "q3moe_gqa_attention_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32, _I64]),
    "q3moe_gqa_attention": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P, _F, _P, _P,
                                   ctypes.c_size_t, _P]),
    "q3moe_moe_ffn_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "q3moe_moe_ffn": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _P, _Experts, _Experts, _Experts,
                             _P, _P, _P, _I32, _P, ctypes.c_size_t, _P]),
    "q3moe_moe_ffn_prenorm": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _P, _F, _P, _Experts,
                                     _Experts, _Experts, _P, _P, _P, _I32, _P, ctypes.c_size_t,
                                     _P]),
    "q3moe_persistent_path": (_I32, [_I64, _I64, _I64, _I32, _I32, _I32, _I32]),
    "q3moe_kv_write_rows": (_I32, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _I64, _P]),
    "q3moe_prefill_attention": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P, _F, _P, _P]),
    "q3moe_embed": (_I32, [_P, _I64, _P, _I32, _I64, _I64, _P, _P]),
    "q3moe_output_head": (_I32, [_P, _I64, _P, _I32, _I64, _I64, _P, _P]),
    "q3moe_moe_ffn_q8": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _P, _Experts, _Experts, _Experts,
                                _P, _P, _P, _I32, _P, ctypes.c_size_t, _P]),
    "q3moe_moe_stack_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I32]),
    "q3moe_moe_stack": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _F, _P, _I32, _P, _P, _P,
                               ctypes.c_size_t, _P]),
    "q3moe_moe_ffn_noalloc": (_I32, [_P, _I64, _I64, _I64, _I32, _I32, _P, _Experts, _Experts,
                                     _Experts, _P, _P, _P, _I32, _P]),
}

_lib = None


def library() -> ctypes.CDLL:
    """Load libq3moe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_moe_decode_q3moe_amd.build`")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(fn: str, st: int):
    if st != 0:
        raise Q3MoeError(fn, st, library().q3moe_status_string(st).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dims}-D tensor")


class Experts(NamedTuple):
    """A 3-D expert tensor: ``data`` uint8 [E, stride_bytes] (row e is expert
    e's matrix, read at base + e*stride) and its k-quant type."""
    data: torch.Tensor
    qtype: int

    def c(self) -> _Experts:
        if self.data.dtype != torch.uint8 or self.data.dim() != 2 or self.data.stride(1) != 1:
            raise ValueError("expert data must be uint8 [E, stride_bytes] with unit inner stride")
        if self.data.device.type != "cuda":
            raise ValueError("expert data must be on a HIP device")
        return _Experts(self.data.data_ptr(), self.qtype, 0, self.data.stride(0))


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]) -> torch.Tensor:
    """A caller-provided workspace, or a fresh zero-filled one."""
    if given is not None:
        return given
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def q3moe_route_workspace_bytes(T: int, E: int) -> int:
    return library().q3moe_route_workspace_bytes(T, E)


def q3moe_route(hidden: torch.Tensor, router: torch.Tensor, top_k: int,
                topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """-> (topk_idx int32 [T, k], topk_w f32 [T, k]) on hidden's device."""
    _need(hidden, "hidden", torch.float32, 2)
    _need(router, "router", torch.float32, 2)
    T, H = hidden.shape
    E = router.shape[0]
    if router.shape[1] != H:
        raise ValueError("router must be [E, H]")
    dev = hidden.device
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    nbytes = q3moe_route_workspace_bytes(T, E)
    ws = _workspace(nbytes, dev, workspace)
    _check("q3moe_route", library().q3moe_route(
        _ptr(hidden), T, H, _ptr(router), E, top_k, _ptr(topk_idx), _ptr(topk_w),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_w


def q3moe_group_by_expert(topk_idx: torch.Tensor, E: int, counts: Optional[torch.Tensor] = None,
                          offsets: Optional[torch.Tensor] = None,
                          pairs: Optional[torch.Tensor] = None, stream=None):
    """-> (counts int32 [E], offsets int32 [E+1], pairs int32 [T*k]) on the
    device; pairs[:offsets[E]] is the grouped list."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    dev = topk_idx.device
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pairs is None:
        pairs = torch.empty(max(1, T * k), dtype=torch.int32, device=dev)
    for t, name in ((counts, "counts"), (offsets, "offsets"), (pairs, "pairs")):
        _need(t, name, torch.int32, 1)
    if counts.numel() < E or offsets.numel() < E + 1 or pairs.numel() < T * k:
        raise ValueError("output tensors too small")
    _check("q3moe_group_by_expert", library().q3moe_group_by_expert(
        _ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(pairs), _stream(stream)))
    return counts, offsets, pairs


def q3moe_expert_ffn_workspace_bytes(T: int, H: int, F: int, E: int, top_k: int) -> int:
    return library().q3moe_expert_ffn_workspace_bytes(T, H, F, E, top_k)


def q3moe_expert_ffn_status_offset(T: int, H: int, F: int, E: int, top_k: int) -> int:
    return library().q3moe_expert_ffn_status_offset(T, H, F, E, top_k)


def expert_ffn_status(workspace: torch.Tensor, T: int, H: int, F: int, E: int, top_k: int) -> int:
    """The status word an expert-FFN call left in its workspace (0 = ok).
    Synchronises with the device."""
    off = q3moe_expert_ffn_status_offset(T, H, F, E, top_k)
    return int(workspace[off:off + 4].view(torch.int32).item())


def q3moe_expert_ffn(hidden: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                     gate: Experts, up: Experts, down: Experts, F: int,
                     out: Optional[torch.Tensor] = None, accumulate: bool = False,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sparse expert FFN; returns ``out`` f32 [T, H] (allocated if None)."""
    _need(hidden, "hidden", torch.float32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    T, H = hidden.shape
    k = topk_idx.shape[1]
    E = gate.data.shape[0]
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((T, H), dtype=torch.float32, device=hidden.device)
    _need(out, "out", torch.float32, 2)
    nbytes = q3moe_expert_ffn_workspace_bytes(T, H, F, E, k)
    ws = _workspace(nbytes, hidden.device, workspace)
    _check("q3moe_expert_ffn", library().q3moe_expert_ffn(
        _ptr(hidden), T, H, F, E, k, _ptr(topk_idx), _ptr(topk_w),
        gate.c(), up.c(), down.c(), _ptr(out), 1 if accumulate else 0,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def q3moe_persistent_path(T: int, H: int, F: int, E: int, top_k: int, down_qtype: int,
                          with_route: bool) -> int:
    """1 when the MoE block (with_route) or the expert FFN of this shape runs
    as the one persistent kernel on the current device, 0 for separate
    kernels, -1 for a shape the calls reject."""
    return library().q3moe_persistent_path(T, H, F, E, top_k, down_qtype, 1 if with_route else 0)


def q3moe_moe_ffn_workspace_bytes(T: int, H: int, F: int, E: int, top_k: int) -> int:
    return library().q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k)


def q3moe_moe_ffn(hidden: torch.Tensor, router: torch.Tensor, top_k: int, gate: Experts,
                  up: Experts, down: Experts, F: int, out: Optional[torch.Tensor] = None,
                  accumulate: bool = False, topk_idx: Optional[torch.Tensor] = None,
                  topk_w: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, int8_activations: bool = False):
    """Route + expert FFN in one call; -> (out f32 [T, H], topk_idx int32
    [T, k], topk_w f32 [T, k]), each allocated if None.  int8_activations
    calls q3moe_moe_ffn_q8 (gate/up on int8 activations) instead."""
    _need(hidden, "hidden", torch.float32, 2)
    _need(router, "router", torch.float32, 2)
    T, H = hidden.shape
    E = router.shape[0]
    if router.shape[1] != H:
        raise ValueError("router must be [E, H]")
    dev = hidden.device
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    nbytes = q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k)
    ws = _workspace(nbytes, dev, workspace)
    name = "q3moe_moe_ffn_q8" if int8_activations else "q3moe_moe_ffn"
    _check(name, getattr(library(), name)(
        _ptr(hidden), T, H, F, E, top_k, _ptr(router), gate.c(), up.c(), down.c(),
        _ptr(topk_idx), _ptr(topk_w), _ptr(out), 1 if accumulate else 0,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, topk_idx, topk_w


def q3moe_moe_ffn_noalloc(hidden: torch.Tensor, router: torch.Tensor, top_k: int, gate: Experts,
                          up: Experts, down: Experts, F: int, out: Optional[torch.Tensor] = None,
                          accumulate: bool = False, topk_idx: Optional[torch.Tensor] = None,
                          topk_w: Optional[torch.Tensor] = None, stream=None):
    """q3moe_moe_ffn with the library's own device scratch as its workspace
    (no workspace argument, nothing allocated by the call beyond the outputs
    created here when None); -> (out, topk_idx, topk_w)."""
    _need(hidden, "hidden", torch.float32, 2)
    _need(router, "router", torch.float32, 2)
    T, H = hidden.shape
    E = router.shape[0]
    if router.shape[1] != H:
        raise ValueError("router must be [E, H]")
    dev = hidden.device
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    _check("q3moe_moe_ffn_noalloc", library().q3moe_moe_ffn_noalloc(
        _ptr(hidden), T, H, F, E, top_k, _ptr(router), gate.c(), up.c(), down.c(),
        _ptr(topk_idx), _ptr(topk_w), _ptr(out), 1 if accumulate else 0, _stream(stream)))
    return out, topk_idx, topk_w


def q3moe_moe_ffn_prenorm(hidden: torch.Tensor, norm_gain: torch.Tensor, eps: float,
                          router: torch.Tensor, top_k: int, gate: Experts, up: Experts,
                          down: Experts, F: int, out: Optional[torch.Tensor] = None,
                          accumulate: bool = False, topk_idx: Optional[torch.Tensor] = None,
                          topk_w: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """RMSNorm of hidden (gain, eps), then the MoE block on it; out may be
    hidden itself (with accumulate: x += MoE(RMSNorm(x))).  -> (out,
    topk_idx, topk_w), each allocated if None."""
    _need(hidden, "hidden", torch.float32, 2)
    _need(norm_gain, "norm_gain", torch.float32, 1)
    _need(router, "router", torch.float32, 2)
    T, H = hidden.shape
    E = router.shape[0]
    if router.shape[1] != H or norm_gain.numel() != H:
        raise ValueError("router must be [E, H] and norm_gain [H]")
    dev = hidden.device
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    nbytes = q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k)
    ws = _workspace(nbytes, dev, workspace)
    _check("q3moe_moe_ffn_prenorm", library().q3moe_moe_ffn_prenorm(
        _ptr(hidden), T, H, F, E, top_k, _ptr(norm_gain), eps, _ptr(router), gate.c(), up.c(),
        down.c(), _ptr(topk_idx), _ptr(topk_w), _ptr(out), 1 if accumulate else 0,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, topk_idx, topk_w


class MoeLayer(NamedTuple):
    """One layer of q3moe_moe_stack: RMSNorm gain [H] f32, router [E, H]
    f32 and the three expert tensors."""
    norm_gain: torch.Tensor
    router: torch.Tensor
    gate: Experts
    up: Experts
    down: Experts


def q3moe_moe_stack_workspace_bytes(T: int, H: int, F: int, E: int, top_k: int) -> int:
    return library().q3moe_moe_stack_workspace_bytes(T, H, F, E, top_k)


def q3moe_moe_stack(x: torch.Tensor, layers, top_k: int, F: int, eps: float,
                    topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """x <- x + MoE_l(RMSNorm_l(x)) for each MoeLayer in ``layers``, in place
    on x [T, H]; -> (x, topk_idx int32 [L, T, k], topk_w f32 [L, T, k])."""
    _need(x, "x", torch.float32, 2)
    layers = list(layers)
    T, H = x.shape
    L = len(layers)
    dev = x.device
    E = layers[0].router.shape[0] if L else 1
    arr = (_MoeLayer * max(L, 1))()
    for i, ly in enumerate(layers):
        _need(ly.norm_gain, "norm_gain", torch.float32, 1)
        _need(ly.router, "router", torch.float32, 2)
        if ly.router.shape != (E, H) or ly.norm_gain.numel() != H:
            raise ValueError("every layer needs router [E, H] and norm_gain [H] of one shape")
        arr[i] = _MoeLayer(ly.norm_gain.data_ptr(), ly.router.data_ptr(), ly.gate.c(), ly.up.c(),
                           ly.down.c())
    if topk_idx is None:
        topk_idx = torch.empty((L, T, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((L, T, top_k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, 3)
    _need(topk_w, "topk_w", torch.float32, 3)
    if tuple(topk_idx.shape) != (L, T, top_k) or tuple(topk_w.shape) != (L, T, top_k):
        raise ValueError("topk_idx / topk_w must be [layers, T, top_k]")
    ws = _workspace(q3moe_moe_stack_workspace_bytes(T, H, F, E, top_k), dev, workspace)
    _check("q3moe_moe_stack", library().q3moe_moe_stack(
        _ptr(x), T, H, F, E, top_k, eps, ctypes.cast(arr, ctypes.c_void_p), L, _ptr(topk_idx),
        _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return x, topk_idx, topk_w


def q3moe_attn_prologue(q: torch.Tensor, k: torch.Tensor, q_norm: torch.Tensor,
                        k_norm: torch.Tensor, positions: torch.Tensor, eps: float,
                        rope_base: float, stream=None) -> None:
    """In place on q [T, n_q, D] and k [T, n_kv, D]."""
    _need(q, "q", torch.float32, 3)
    _need(k, "k", torch.float32, 3)
    _need(q_norm, "q_norm", torch.float32, 1)
    _need(k_norm, "k_norm", torch.float32, 1)
    _need(positions, "positions", torch.int32, 1)
    T, nq, D = q.shape
    if k.shape[0] != T or k.shape[2] != D or q_norm.numel() != D or k_norm.numel() != D \
            or positions.numel() != T:
        raise ValueError("inconsistent prologue shapes")
    _check("q3moe_attn_prologue", library().q3moe_attn_prologue(
        _ptr(q), _ptr(k), T, nq, k.shape[1], D, _ptr(q_norm), _ptr(k_norm), _ptr(positions),
        eps, rope_base, _stream(stream)))


def q3moe_bf16_gemv3(Ws, x: torch.Tensor, norm_gain: Optional[torch.Tensor] = None,
                     eps: float = 0.0, outs=None, stream=None):
    """Up to three bf16 projections of one input in one launch, optionally
    after its RMSNorm: Ws a list of 1-3 bf16 [N_i, K] tensors; -> list of
    f32 [T, N_i] outputs (allocated where outs is None)."""
    Ws = list(Ws)
    if not 1 <= len(Ws) <= 3:
        raise ValueError("one to three matrices")
    _need(x, "x", torch.float32, 2)
    T, K = x.shape
    for i, W in enumerate(Ws):
        _need(W, f"W{i}", torch.bfloat16, 2)
        if W.shape[1] != K:
            raise ValueError("every W must be [N, K] with K = x.shape[1]")
    if norm_gain is not None:
        _need(norm_gain, "norm_gain", torch.float32, 1)
        if norm_gain.numel() != K:
            raise ValueError("norm_gain must have K elements")
    if outs is None:
        outs = [torch.empty((T, W.shape[0]), dtype=torch.float32, device=x.device) for W in Ws]
    outs = list(outs)
    if len(outs) != len(Ws):
        raise ValueError("one output per matrix")
    for i, o in enumerate(outs):
        _need(o, f"y{i}", torch.float32, 2)
        if tuple(o.shape) != (T, Ws[i].shape[0]):
            raise ValueError(f"y{i} must be [T, N{i}]")
    Wp = [_ptr(W) for W in Ws] + [None] * (3 - len(Ws))
    Np = [W.shape[0] for W in Ws] + [0] * (3 - len(Ws))
    yp = [_ptr(o) for o in outs] + [None] * (3 - len(outs))
    _check("q3moe_bf16_gemv3", library().q3moe_bf16_gemv3(
        Wp[0], Np[0], Wp[1], Np[1], Wp[2], Np[2], K, _ptr(x), T, _ptr(norm_gain), eps,
        yp[0], yp[1], yp[2], _stream(stream)))
    return outs


def q3moe_kv_write_rows(k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Rows of k_new / v_new (f32 [T, n_kv, D]) into slots positions[t] of one
    sequence's caches (bfloat16 [n_kv, S_max, D]), in place."""
    _need(k_new, "k_new", torch.float32, 3)
    _need(v_new, "v_new", torch.float32, 3)
    _need(positions, "positions", torch.int32, 1)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    T, nkv, D = k_new.shape
    if v_new.shape != k_new.shape or k_cache.shape != v_cache.shape or k_cache.shape[0] != nkv \
            or k_cache.shape[2] != D or positions.shape[0] != T:
        raise ValueError("shape mismatch")
    _check("q3moe_kv_write_rows", library().q3moe_kv_write_rows(
        _ptr(k_new), _ptr(v_new), T, nkv, D, _ptr(positions), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[1], _stream(stream)))


def q3moe_prefill_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            positions: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Causal attention of q (f32 [T, n_q, D]) over one sequence's caches
    (bfloat16 [n_kv, S_max, D]); query t sees positions 0..positions[t]."""
    _need(q, "q", torch.float32, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(positions, "positions", torch.int32, 1)
    T, nq, D = q.shape
    nkv, S = k_cache.shape[0], k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, 3)
    _check("q3moe_prefill_attention", library().q3moe_prefill_attention(
        _ptr(q), T, nq, nkv, D, _ptr(k_cache), _ptr(v_cache), S, _ptr(positions), scale, _ptr(out),
        _stream(stream)))
    return out


def _table(W: torch.Tensor, name: str):
    if W.dtype != torch.uint8 or not W.is_contiguous() or W.device.type != "cuda":
        raise ValueError(f"{name} must be a contiguous uint8 tensor on a HIP device")


def q3moe_embed(tokens: torch.Tensor, table: torch.Tensor, qtype: int, V: int, H: int,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rows tokens[t] of a k-quant embedding table (V rows of H/256 blocks),
    dequantised; -> out f32 [T, H]."""
    _need(tokens, "tokens", torch.int32, 1)
    _table(table, "table")
    if table.numel() < V * q3moe_expert_matrix_bytes(qtype, 1, H):
        raise ValueError("table is smaller than V rows")
    T = tokens.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=tokens.device)
    _need(out, "out", torch.float32, 2)
    _check("q3moe_embed", library().q3moe_embed(_ptr(tokens), T, _ptr(table), qtype, V, H,
                                                _ptr(out), _stream(stream)))
    return out


def q3moe_output_head(x: torch.Tensor, W: torch.Tensor, V: int, qtype: int = Q6_K,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """logits f32 [T, V] = W x for a k-quant matrix W of V rows."""
    _need(x, "x", torch.float32, 2)
    _table(W, "W")
    T, H = x.shape
    if W.numel() < V * q3moe_expert_matrix_bytes(qtype, 1, H):
        raise ValueError("W is smaller than V rows")
    if out is None:
        out = torch.empty((T, V), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, 2)
    _check("q3moe_output_head", library().q3moe_output_head(_ptr(x), T, _ptr(W), qtype, V, H,
                                                            _ptr(out), _stream(stream)))
    return out


def q3moe_expert_matrix_bytes(qtype: int, rows: int, cols: int) -> int:
    return library().q3moe_expert_matrix_bytes(qtype, rows, cols)


def q3moe_rmsnorm(x: torch.Tensor, gain: torch.Tensor, eps: float,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _need(x, "x", torch.float32, 2)
    _need(gain, "gain", torch.float32, 1)
    T, n = x.shape
    if gain.numel() != n:
        raise ValueError("gain must have x.shape[1] elements")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.float32, 2)
    _check("q3moe_rmsnorm", library().q3moe_rmsnorm(
        _ptr(x), T, n, _ptr(gain), eps, _ptr(out), _stream(stream)))
    return out


def q3moe_bf16_gemv(W: torch.Tensor, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                    accumulate: bool = False, stream=None) -> torch.Tensor:
    """out [T, N] (+)= x [T, K] @ W[N, K]^T with W bfloat16, x and out f32."""
    _need(W, "W", torch.bfloat16, 2)
    _need(x, "x", torch.float32, 2)
    N, K = W.shape
    T = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [T, K] with K = W.shape[1]")
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing out tensor")
        out = torch.empty((T, N), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, 2)
    if tuple(out.shape) != (T, N):
        raise ValueError("out must be [T, N]")
    _check("q3moe_bf16_gemv", library().q3moe_bf16_gemv(
        _ptr(W), N, K, _ptr(x), T, _ptr(out), 1 if accumulate else 0, _stream(stream)))
    return out


def q3moe_kv_write(k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Write k_new / v_new f32 [B, n_kv, D] into the bfloat16 caches
    [B, n_kv, S_max, D] at positions int32 [B]."""
    _need(k_new, "k_new", torch.float32, 3)
    _need(v_new, "v_new", torch.float32, 3)
    _need(positions, "positions", torch.int32, 1)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, nkv, D = k_new.shape
    S_max = k_cache.shape[2]
    if tuple(v_new.shape) != (B, nkv, D) or positions.numel() != B \
            or tuple(k_cache.shape) != (B, nkv, S_max, D) or v_cache.shape != k_cache.shape:
        raise ValueError("inconsistent KV-write shapes")
    _check("q3moe_kv_write", library().q3moe_kv_write(
        _ptr(k_new), _ptr(v_new), B, nkv, D, _ptr(positions), _ptr(k_cache), _ptr(v_cache),
        S_max, _stream(stream)))


def q3moe_attn_prologue_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           q_norm: torch.Tensor, k_norm: torch.Tensor, positions: torch.Tensor,
                           eps: float, rope_base: float, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, stream=None) -> None:
    """q3moe_attn_prologue on q [B, n_q, D] and k [B, n_kv, D] in place, then
    the rotated k and v [B, n_kv, D] into the bfloat16 caches [B, n_kv, S_max,
    D] at positions int32 [B], in one launch."""
    _need(q, "q", torch.float32, 3)
    _need(k, "k", torch.float32, 3)
    _need(v, "v", torch.float32, 3)
    _need(q_norm, "q_norm", torch.float32, 1)
    _need(k_norm, "k_norm", torch.float32, 1)
    _need(positions, "positions", torch.int32, 1)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, nq, D = q.shape
    nkv = k.shape[1]
    S_max = k_cache.shape[2]
    if tuple(k.shape) != (B, nkv, D) or tuple(v.shape) != (B, nkv, D) or positions.numel() != B \
            or q_norm.numel() != D or k_norm.numel() != D \
            or tuple(k_cache.shape) != (B, nkv, S_max, D) or v_cache.shape != k_cache.shape:
        raise ValueError("inconsistent prologue / KV-write shapes")
    _check("q3moe_attn_prologue_kv", library().q3moe_attn_prologue_kv(
        _ptr(q), _ptr(k), _ptr(v), B, nq, nkv, D, _ptr(q_norm), _ptr(k_norm), _ptr(positions),
        eps, rope_base, _ptr(k_cache), _ptr(v_cache), S_max, _stream(stream)))


def q3moe_gqa_attention_workspace_bytes(B: int, n_q: int, n_kv: int, D: int, S_max: int) -> int:
    return library().q3moe_gqa_attention_workspace_bytes(B, n_q, n_kv, D, S_max)


def q3moe_gqa_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        lengths: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of q f32 [B, n_q, D] over the first lengths[b]
    positions of the bfloat16 caches [B, n_kv, S_max, D]; returns out f32
    [B, n_q, D]."""
    _need(q, "q", torch.float32, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(lengths, "lengths", torch.int32, 1)
    B, nq, D = q.shape
    nkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, nkv, S_max, D) or v_cache.shape != k_cache.shape \
            or lengths.numel() != B:
        raise ValueError("inconsistent attention shapes")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float32, 3)
    nbytes = q3moe_gqa_attention_workspace_bytes(B, nq, nkv, D, S_max)
    ws = workspace if workspace is not None else torch.empty(
        max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check("q3moe_gqa_attention", library().q3moe_gqa_attention(
        _ptr(q), B, nq, nkv, D, _ptr(k_cache), _ptr(v_cache), S_max, _ptr(lengths), scale,
        _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out
