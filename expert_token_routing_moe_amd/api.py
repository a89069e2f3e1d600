"""Python binding of the C ABI in ``include/moe.h`` (argument marshalling only).

Every function here has the name of the C entry point it calls and forwards
``torch`` tensor data pointers to it; all computation happens in the gfx950
kernels of ``libmoe_mi355x.so``.  There is no fallback: if the library is not
built, or a call returns an error status, a ``MoEError`` is raised.

bf16 tensors are ``torch.bfloat16``; index tensors ``torch.int32``; gates and
logits ``torch.float32``.  Every tensor must be contiguous and on the GPU
(except for ``moe_query``, which is host-only).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
DISPATCH_SCRATCH_BYTES = 8 << 20  # MOE_DISPATCH_SCRATCH_BYTES

STAT_NAMES = (
    "assignments", "kept", "dropped", "padded", "capacity", "send_rows",
    "dispatch_bytes", "dispatch_wire_bytes", "dispatch_remote_bytes",
    "combine_bytes", "max_expert_count", "invalid_index",
)


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
        ("k", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("my_rank", ctypes.c_int32), ("drop_policy", ctypes.c_int32),
        ("min_capacity", ctypes.c_int32), ("dispatch_fp8", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("group_limit", ctypes.c_int32),
        ("shared_H", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
    ]


_lib = None


def lib():
    """Load the built library; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoEError("load", MOE_EHIP,
                       f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I, SZ = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_query": [S, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                      ctypes.POINTER(ctypes.c_size_t)],
        "moe_route": [S, P, P, P, P, P, P, P, SZ, P],
        "moe_topk_from_logits": [S, P, P, P, P],
        "moe_dispatch": [S, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_dispatch_noalloc": [S, P, P, P, P, P, P, P, P, P, P, P, P],
        "moe_expert_ffn": [S, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_expert_gate_up": [S, P, P, P, P, P, P, P, P, SZ, P],
        "moe_expert_down": [S, P, P, P, P, P, P],
        "moe_combine": [S, P, P, P, P, P, P],
        "moe_shared_expert": [S, P, P, P, P, P, P, SZ, P],
        "moe_layer_fwd": [S] + [P] * 24 + [SZ, P],
        "moe_fp8_rows_to_bf16": [P, P, ctypes.c_int64, ctypes.c_int32, P, P],
        "moe_stream_read": [P, SZ, P, P],
        "moe_stream_write": [P, SZ, ctypes.c_uint32, P],
        "moe_stream_gather": [P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int64,
                              ctypes.c_int32, P, P],
    }
    for name, argtypes in sig.items():
        f = getattr(L, name)
        f.argtypes = argtypes
        f.restype = I
    L.moe_status_str.argtypes = [I]
    L.moe_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoEError(fn, rc, lib().moe_status_str(rc).decode())


@dataclass(frozen=True)
class Shape:
    """Python mirror of ``moe_shape`` (pages' notation)."""

    T: int
    d: int
    E: int
    k: int
    H: int
    D: int = 1
    my_rank: int = 0
    capacity_factor: float = math.inf
    drop_policy: int = 0
    min_capacity: int = 0
    dispatch_fp8: int = 0
    n_groups: int = 0
    group_limit: int = 0
    shared_H: int = 0

    def c(self) -> moe_shape:
        return moe_shape(self.T, self.d, self.E, self.k, self.H, self.D, self.my_rank,
                         self.drop_policy, self.min_capacity, self.dispatch_fp8,
                         self.n_groups, self.group_limit, self.shared_H,
                         float(self.capacity_factor))

    @classmethod
    def from_config(cls, cfg) -> "Shape":
        return cls(cfg.T, cfg.d, cfg.E, cfg.k, cfg.H, cfg.D, cfg.my_rank, cfg.cf,
                   cfg.drop_policy, cfg.min_capacity, cfg.dispatch_fp8, cfg.n_groups,
                   cfg.group_limit, cfg.shared_H)


def _p(t: torch.Tensor | None, dtype=None):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _need(shape, **tensors):
    """Raise ValueError, before anything reaches the library, if a tensor
    holds fewer elements than the shape makes the call read or write.  Each
    keyword names a tensor (or None) and its required element count as
    (tensor, count); counts come from the shape and moe_query."""
    for name, (t, n) in tensors.items():
        if t is not None and t.numel() < n:
            raise ValueError(f"{name}: {t.numel()} elements, the shape needs {n}")


def _sizes(shape):
    """Element counts of the layer's tensors for this shape."""
    send_rows, _, _ = moe_query(shape)
    T, d, E, k, H, D = shape.T, shape.d, shape.E, shape.k, shape.H, shape.D
    return dict(x=T * d, w_gate=d * E, bias=E, logits=T * E, tk=T * k, send=send_rows * d,
                scale=send_rows, h=send_rows * H, E=E, E1=E + 1, D=D, stats=len(STAT_NAMES),
                w13=E * H * d, w2=E * d * H, y=T * d, ws13=shape.shared_H * d,
                ws2=d * shape.shared_H)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


BF16, I32, F32 = torch.bfloat16, torch.int32, torch.float32


def _send(shape, t):
    """The send buffer: bf16 rows, or E4M3 codes (uint8) under FP8 dispatch."""
    return _p(t, torch.uint8 if shape.dispatch_fp8 else BF16)


def moe_query(shape: Shape):
    """-> (send_rows, capacity, workspace_bytes); host only."""
    sr, cap, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    s = shape.c()
    _check("moe_query", lib().moe_query(ctypes.byref(s), ctypes.byref(sr), ctypes.byref(cap),
                                        ctypes.byref(ws)))
    return sr.value, cap.value, ws.value


def moe_route(shape, x, w_gate, logit_bias, logits_out, topk_idx, topk_w, workspace,
              stream=None):
    z = _sizes(shape)
    _need(shape, x=(x, z["x"]), w_gate=(w_gate, z["w_gate"]), logit_bias=(logit_bias, z["bias"]),
          logits_out=(logits_out, z["logits"]), topk_idx=(topk_idx, z["tk"]),
          topk_w=(topk_w, z["tk"]))
    s = shape.c()
    _check("moe_route", lib().moe_route(
        ctypes.byref(s), _p(x, BF16), _p(w_gate, BF16), _p(logit_bias, F32),
        _p(logits_out, F32), _p(topk_idx, I32), _p(topk_w, F32), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_topk_from_logits(shape, logits, topk_idx, topk_w, stream=None):
    z = _sizes(shape)
    _need(shape, logits=(logits, z["logits"]), topk_idx=(topk_idx, z["tk"]),
          topk_w=(topk_w, z["tk"]))
    s = shape.c()
    _check("moe_topk_from_logits", lib().moe_topk_from_logits(
        ctypes.byref(s), _p(logits, F32), _p(topk_idx, I32), _p(topk_w, F32), _stream(stream)))


def moe_dispatch(shape, x, topk_idx, topk_w, send_buf, send_scale, slot, expert_count,
                 expert_kept, expert_offset, rank_rows, stats, workspace, stream=None):
    """topk_w is read only by drop policy 1 in capacity mode; send_scale only
    under FP8 dispatch; either may be None otherwise."""
    z = _sizes(shape)
    _need(shape, x=(x, z["x"]), topk_idx=(topk_idx, z["tk"]), topk_w=(topk_w, z["tk"]),
          send_buf=(send_buf, z["send"]), send_scale=(send_scale, z["scale"]),
          slot=(slot, z["tk"]), expert_count=(expert_count, z["E"]),
          expert_kept=(expert_kept, z["E"]), expert_offset=(expert_offset, z["E1"]),
          rank_rows=(rank_rows, z["D"]), stats=(stats, z["stats"]))
    s = shape.c()
    _check("moe_dispatch", lib().moe_dispatch(
        ctypes.byref(s), _p(x, BF16), _p(topk_idx, I32), _p(topk_w, F32), _send(shape, send_buf),
        _p(send_scale, F32), _p(slot, I32),
        _p(expert_count, I32), _p(expert_kept, I32), _p(expert_offset, I32),
        _p(rank_rows, I32), _p(stats, torch.int64), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dispatch_noalloc(shape, x, topk_idx, topk_w, send_buf, send_scale, slot, expert_count,
                         expert_kept, expert_offset, rank_rows, stats, stream=None):
    """moe_dispatch without a workspace: the library's static per-GPU scratch
    holds the dispatch's intermediates (no allocation; overlapping calls on
    one GPU race)."""
    z = _sizes(shape)
    _need(shape, x=(x, z["x"]), topk_idx=(topk_idx, z["tk"]), topk_w=(topk_w, z["tk"]),
          send_buf=(send_buf, z["send"]), send_scale=(send_scale, z["scale"]),
          slot=(slot, z["tk"]), expert_count=(expert_count, z["E"]),
          expert_kept=(expert_kept, z["E"]), expert_offset=(expert_offset, z["E1"]),
          rank_rows=(rank_rows, z["D"]), stats=(stats, z["stats"]))
    s = shape.c()
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        ctypes.byref(s), _p(x, BF16), _p(topk_idx, I32), _p(topk_w, F32), _send(shape, send_buf),
        _p(send_scale, F32), _p(slot, I32),
        _p(expert_count, I32), _p(expert_kept, I32), _p(expert_offset, I32),
        _p(rank_rows, I32), _p(stats, torch.int64), _stream(stream)))


def moe_expert_ffn(shape, send_buf, send_scale, expert_offset, expert_kept, w1, w3, w2,
                   expert_out, workspace, stream=None):
    z = _sizes(shape)
    _need(shape, send_buf=(send_buf, z["send"]), send_scale=(send_scale, z["scale"]),
          expert_offset=(expert_offset, z["E1"]), expert_kept=(expert_kept, z["E"]),
          w1=(w1, z["w13"]), w3=(w3, z["w13"]), w2=(w2, z["w2"]),
          expert_out=(expert_out, z["send"]))
    s = shape.c()
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(s), _send(shape, send_buf), _p(send_scale, F32), _p(expert_offset, I32),
        _p(expert_kept, I32),
        _p(w1, BF16), _p(w3, BF16), _p(w2, BF16), _p(expert_out, BF16), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_expert_gate_up(shape, send_buf, send_scale, expert_offset, expert_kept, w1, w3, h,
                       stream=None, workspace=None):
    """workspace (optional, uint8 of moe_query's size): lets E4M3 rows be
    widened to bf16 in one pass before the GEMM on MFMA-bound shapes."""
    z = _sizes(shape)
    _need(shape, send_buf=(send_buf, z["send"]), send_scale=(send_scale, z["scale"]),
          expert_offset=(expert_offset, z["E1"]), expert_kept=(expert_kept, z["E"]),
          w1=(w1, z["w13"]), w3=(w3, z["w13"]), h=(h, z["h"]))
    s = shape.c()
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(
        ctypes.byref(s), _send(shape, send_buf), _p(send_scale, F32), _p(expert_offset, I32),
        _p(expert_kept, I32),
        _p(w1, BF16), _p(w3, BF16), _p(h, BF16), _p(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_expert_down(shape, h, expert_offset, expert_kept, w2, expert_out, stream=None):
    z = _sizes(shape)
    _need(shape, h=(h, z["h"]), expert_offset=(expert_offset, z["E1"]),
          expert_kept=(expert_kept, z["E"]), w2=(w2, z["w2"]),
          expert_out=(expert_out, z["send"]))
    s = shape.c()
    _check("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(s), _p(h, BF16), _p(expert_offset, I32), _p(expert_kept, I32),
        _p(w2, BF16), _p(expert_out, BF16), _stream(stream)))


def moe_combine(shape, expert_out, slot, topk_w, shared_out, y, stream=None):
    """shared_out: the shared expert's [T, d] output, added with weight 1, or None."""
    z = _sizes(shape)
    _need(shape, expert_out=(expert_out, z["send"]), slot=(slot, z["tk"]),
          topk_w=(topk_w, z["tk"]), shared_out=(shared_out, z["y"]), y=(y, z["y"]))
    s = shape.c()
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(s), _p(expert_out, BF16), _p(slot, I32), _p(topk_w, F32),
        _p(shared_out, BF16), _p(y, BF16), _stream(stream)))


def moe_shared_expert(shape, x, w1s, w3s, w2s, shared_out, workspace, stream=None):
    z = _sizes(shape)
    _need(shape, x=(x, z["x"]), w1s=(w1s, z["ws13"]), w3s=(w3s, z["ws13"]),
          w2s=(w2s, z["ws2"]), shared_out=(shared_out, z["y"]))
    s = shape.c()
    _check("moe_shared_expert", lib().moe_shared_expert(
        ctypes.byref(s), _p(x, BF16), _p(w1s, BF16), _p(w3s, BF16), _p(w2s, BF16),
        _p(shared_out, BF16), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_layer_fwd(shape, x, w_gate, logit_bias, w1, w3, w2, buf: "LayerBuffers", stream=None,
                  shared=None):
    """shared: (w1s, w3s, w2s) of the shared expert when shape.shared_H > 0."""
    z = _sizes(shape)
    w1s_, w3s_, w2s_ = shared if shared is not None else (None, None, None)
    _need(shape, x=(x, z["x"]), w_gate=(w_gate, z["w_gate"]), logit_bias=(logit_bias, z["bias"]),
          w1=(w1, z["w13"]), w3=(w3, z["w13"]), w2=(w2, z["w2"]), w1s=(w1s_, z["ws13"]),
          w3s=(w3s_, z["ws13"]), w2s=(w2s_, z["ws2"]), y=(buf.y, z["y"]),
          logits=(buf.logits, z["logits"]), topk_idx=(buf.topk_idx, z["tk"]),
          topk_w=(buf.topk_w, z["tk"]), send_buf=(buf.send_buf, z["send"]),
          send_scale=(buf.send_scale, z["scale"]), slot=(buf.slot, z["tk"]),
          expert_count=(buf.expert_count, z["E"]), expert_kept=(buf.expert_kept, z["E"]),
          expert_offset=(buf.expert_offset, z["E1"]), rank_rows=(buf.rank_rows, z["D"]),
          stats=(buf.stats, z["stats"]), expert_out=(buf.expert_out, z["send"]),
          shared_out=(buf.shared_out, z["y"] if shape.shared_H else 0))
    s = shape.c()
    w1s, w3s, w2s = shared if shared is not None else (None, None, None)
    _check("moe_layer_fwd", lib().moe_layer_fwd(
        ctypes.byref(s), _p(x, BF16), _p(w_gate, BF16), _p(logit_bias, F32), _p(w1, BF16),
        _p(w3, BF16), _p(w2, BF16), _p(w1s, BF16), _p(w3s, BF16), _p(w2s, BF16),
        _p(buf.y, BF16), _p(buf.logits, F32),
        _p(buf.topk_idx, I32), _p(buf.topk_w, F32), _send(shape, buf.send_buf),
        _p(buf.send_scale, F32), _p(buf.slot, I32),
        _p(buf.expert_count, I32), _p(buf.expert_kept, I32), _p(buf.expert_offset, I32),
        _p(buf.rank_rows, I32), _p(buf.stats, torch.int64), _p(buf.expert_out, BF16),
        _p(buf.shared_out, BF16), _p(buf.workspace), buf.workspace.numel(), _stream(stream)))


def moe_fp8_rows_to_bf16(codes, scales, out, stream=None):
    """out = bf16(E4M3 value of codes * row scale), the expert GEMM's decode."""
    rows, d = codes.shape
    if scales.numel() < rows or out.numel() < rows * d:
        raise ValueError(f"scales/out hold {scales.numel()}/{out.numel()} elements, "
                         f"the codes need {rows}/{rows * d}")
    _check("moe_fp8_rows_to_bf16", lib().moe_fp8_rows_to_bf16(
        _p(codes, torch.uint8), _p(scales, F32), rows, d, _p(out, BF16), _stream(stream)))


STREAM_READ_MARK = 0x9E3779B9


def moe_stream_read(src, sink, stream=None):
    """Read src once with the expert GEMMs' non-temporal loads (a probe of the
    device's streaming-read rate).  sink[0] is set to STREAM_READ_MARK only
    by a reading lane whose XOR of the words it read equals the mark."""
    _check("moe_stream_read", lib().moe_stream_read(
        _p(src), src.numel() * src.element_size(), _p(sink, I32), _stream(stream)))


def moe_stream_write(dst, value, stream=None):
    """Fill dst with the 32-bit value, once, with the permute's non-temporal
    16-byte stores (a probe of the device's streaming-store rate)."""
    _check("moe_stream_write", lib().moe_stream_write(
        _p(dst), dst.numel() * dst.element_size(), ctypes.c_uint32(value & 0xFFFFFFFF),
        _stream(stream)))


def moe_stream_gather(rows, slot, out, stream=None):
    """out[t] = XOR over s of rows[slot[t, s]] (16-byte pieces), with the
    combine's access and none of its arithmetic (a probe of that access's
    rate).  rows [nrows, d] bf16; slot [T, k] int32; out [T, d] bf16."""
    nrows, d = rows.shape
    T, k = slot.shape
    if tuple(out.shape) != (T, d):
        raise ValueError(f"moe_stream_gather: out is {tuple(out.shape)}, needs {(T, d)}")
    _check("moe_stream_gather", lib().moe_stream_gather(
        _p(rows, BF16), nrows, d, _p(slot, I32), T, k, _p(out, BF16), _stream(stream)))


@dataclass
class LayerBuffers:
    """Every output and intermediate of one layer call, plus the workspace."""

    y: torch.Tensor
    logits: torch.Tensor | None
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    send_buf: torch.Tensor
    send_scale: torch.Tensor | None
    slot: torch.Tensor
    expert_count: torch.Tensor
    expert_kept: torch.Tensor
    expert_offset: torch.Tensor
    rank_rows: torch.Tensor
    stats: torch.Tensor
    expert_out: torch.Tensor
    shared_out: torch.Tensor | None
    workspace: torch.Tensor

    @classmethod
    def allocate(cls, shape: Shape, device="cuda", keep_logits: bool = True) -> "LayerBuffers":
        send_rows, _, ws = moe_query(shape)
        dev = torch.device(device)
        T, d, E, k, D = shape.T, shape.d, shape.E, shape.k, shape.D
        z = lambda *s, dt: torch.empty(s, dtype=dt, device=dev)
        return cls(
            y=z(T, d, dt=BF16),
            logits=z(T, E, dt=F32) if keep_logits else None,
            topk_idx=z(T, k, dt=I32), topk_w=z(T, k, dt=F32),
            send_buf=z(send_rows, d, dt=torch.uint8 if shape.dispatch_fp8 else BF16),
            send_scale=z(send_rows, dt=F32) if shape.dispatch_fp8 else None,
            slot=z(T, k, dt=I32),
            expert_count=z(E, dt=I32), expert_kept=z(E, dt=I32),
            expert_offset=z(E + 1, dt=I32), rank_rows=z(D, dt=I32),
            stats=z(len(STAT_NAMES), dt=torch.int64),
            expert_out=z(send_rows, d, dt=BF16),
            shared_out=z(T, d, dt=BF16) if shape.shared_H > 0 else None,
            workspace=z(ws, dt=torch.uint8),
        )


def stats_dict(stats: torch.Tensor) -> dict:
    return {n: int(v) for n, v in zip(STAT_NAMES, stats.cpu().tolist())}
