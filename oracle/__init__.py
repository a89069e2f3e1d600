"""CPU oracle for the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it,
and it imports nothing from the product package: the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C loops, IEEE double
accumulation, OpenMP over tokens or rows); this module only marshals numpy
arrays, apart from ``imbalance``, a one-line ratio over loads the C code
returns.  bf16 tensors are passed as ``numpy.uint16`` arrays of raw bits.

Sources, cited by page title and section:
  * "Mixture-of-Experts (MoE) Architecture and Expert Parallelism",
    section 2 "The Gating Network Formulation" -- logits, KeepTopK, softmax,
    and the weighted sum of expert outputs.
  * "EP Math -- Expert Parallelism (MoE)" -- notation (T, d, k, D), dispatch
    and combine volumes, capacity factor, token drop, expert placement.
  * "MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric" -- the
    gated three-matrix expert, drop-before-exchange, per-destination chunks,
    and ("Rank-level skew and the straggler effect") the load imbalance
    ratio.

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, invariants and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

STAT_NAMES = (
    "assignments",
    "kept",
    "dropped",
    "padded",
    "capacity",
    "send_rows",
    "dispatch_bytes",
    "dispatch_wire_bytes",
    "dispatch_remote_bytes",
    "combine_bytes",
    "max_expert_count",
    "invalid_index",
)

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math",
        _SRC, "-o", _SO + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_logits.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_logits.restype = None
    lib.oracle_topk.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk_grouped.argtypes = [i32, i32, i32, i32, i32, P, P, P, P]
    lib.oracle_topk_grouped.restype = ctypes.c_int
    lib.oracle_capacity.argtypes = [i32, i32, i32, ctypes.c_double, i32]
    lib.oracle_capacity.restype = ctypes.c_int64
    lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_double, i32, i32,
                                    i32, P, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_fp8_value.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_value.restype = ctypes.c_double
    lib.oracle_fp8_from_float.argtypes = [ctypes.c_float]
    lib.oracle_fp8_from_float.restype = ctypes.c_uint8
    lib.oracle_fp8_quantize_rows.argtypes = [i32, i32, P, P, P]
    lib.oracle_fp8_quantize_rows.restype = None
    lib.oracle_expert_ffn_fp8.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_expert_ffn_fp8.restype = None
    lib.oracle_dispatch.restype = ctypes.c_int
    lib.oracle_expert_ffn.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_expert_ffn.restype = None
    lib.oracle_expert_gate_up.argtypes = [i32, i32, i32, P, P, P, P, P]
    lib.oracle_expert_gate_up.restype = None
    lib.oracle_expert_gate_up_fp8.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_expert_gate_up_fp8.restype = None
    lib.oracle_expert_down.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_expert_down.restype = None
    lib.oracle_combine.argtypes = [i32, i32, i32, P, P, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_from_double(v: float) -> int:
    """Raw bits of the bf16 nearest to ``v`` (ties to even)."""
    return int(_load().oracle_bf16_from_double(float(v)))


def logits(x: np.ndarray, w_gate: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """H = x W_g (+ b), fp32 [T, E].  x [T, d] bf16 bits, w_gate [d, E] bf16 bits."""
    x = _c(x, np.uint16)
    w_gate = _c(w_gate, np.uint16)
    T, d = x.shape
    d2, E = w_gate.shape
    assert d == d2
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    _load().oracle_logits(T, d, E, _ptr(x), _ptr(w_gate), _ptr(b), _ptr(out))
    return out


def topk(lg: np.ndarray, k: int, groups: int = 1, group_limit: int = 1):
    """KeepTopK + softmax on fp32 logits [T, E] -> (idx int32 [T,k], w fp32 [T,k], gap f64 [T]).

    groups > 1 and group_limit < groups: only the experts of the group_limit
    groups with the largest best logit may be chosen (group-limited routing)."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    idx = np.empty((T, max(k, 0)), np.int32)
    w = np.empty((T, max(k, 0)), np.float32)
    gap = np.empty((T,), np.float64)
    rc = _load().oracle_topk_grouped(T, E, k, groups, group_limit, _ptr(lg), _ptr(idx), _ptr(w),
                                     _ptr(gap))
    if rc != 0:
        raise ValueError(f"oracle top-k: unsupported shape E={E} k={k} groups={groups} "
                         f"limit={group_limit}")
    return idx, w, gap


def capacity(T: int, k: int, E: int, cf: float, min_capacity: int = 0) -> int:
    return int(_load().oracle_capacity(T, k, E, float(cf), int(min_capacity)))


def imbalance(loads) -> float:
    """Load imbalance ratio (max - mean) / mean over per-rank (or per-expert)
    loads, as "MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric"
    defines it in "Rank-level skew and the straggler effect"; 0 when every
    load equals the mean."""
    a = np.asarray(loads, np.float64)
    m = a.mean()
    return float((a.max() - m) / m) if m > 0 else 0.0


def fp8_value(code: int) -> float:
    """Value of an E4M3 code (OCP: bias 7, max 448, 0x7F/0xFF NaN)."""
    return float(_load().oracle_fp8_value(int(code)))


def fp8_from_float(v: float) -> int:
    """E4M3 code nearest to the fp32 value v (ties to even, saturating, sign kept)."""
    return int(_load().oracle_fp8_from_float(float(v)))


def fp8_quantize_rows(x: np.ndarray):
    """bf16 rows [n, d] -> (E4M3 codes uint8 [n, d], fp32 scales [n])."""
    x = _c(x, np.uint16)
    n, d = x.shape
    codes = np.empty((n, d), np.uint8)
    scales = np.empty((n,), np.float32)
    _load().oracle_fp8_quantize_rows(n, d, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def fp8_values(codes: np.ndarray) -> np.ndarray:
    """Vectorised E4M3 decode through the oracle's table of all 256 codes."""
    table = np.array([fp8_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes, np.uint8)]


def dispatch(x: np.ndarray | None, topk_idx: np.ndarray, *, T: int, d: int, E: int,
             D: int, my_rank: int = 0, cf: float = float("inf"),
             with_send_buf: bool = True, drop_policy: int = 0, topk_w=None,
             min_capacity: int = 0, fp8: bool = False) -> dict:
    """Histogram, capacity, positions, slots and the send buffer.

    drop_policy 0 keeps an overflowing expert's first C assignments in token
    order; 1 keeps its C largest gate values (topk_w, fp32 [T, k]).
    fp8: the send buffer holds E4M3 rows (uint8) with per-row fp32 scales
    (out["send_scale"]); otherwise bf16 rows."""
    topk_idx = _c(topk_idx, np.int32)
    k = topk_idx.shape[1]
    assert topk_idx.shape[0] == T
    if topk_w is not None:
        topk_w = _c(topk_w, np.float32)
        assert topk_w.shape == topk_idx.shape
    C = capacity(T, k, E, cf, min_capacity)
    send_rows = T * k if C < 0 else E * C
    send_buf = send_scale = None
    if with_send_buf:
        x = _c(x, np.uint16)
        assert x.shape == (T, d)
        send_buf = np.empty((send_rows, d), np.uint8 if fp8 else np.uint16)
        if fp8:
            send_scale = np.empty((send_rows,), np.float32)
    out = dict(
        slot=np.empty((T, k), np.int32),
        expert_count=np.empty((E,), np.int32),
        expert_kept=np.empty((E,), np.int32),
        expert_offset=np.empty((E + 1,), np.int64),
        rank_rows=np.empty((D,), np.int64),
    )
    stats = np.empty((len(STAT_NAMES),), np.int64)
    rc = _load().oracle_dispatch(
        T, d, E, k, D, my_rank, float(cf), int(min_capacity), int(drop_policy), int(fp8),
        _ptr(x) if with_send_buf else None, _ptr(topk_idx), _ptr(topk_w), _ptr(send_buf),
        _ptr(send_scale), _ptr(out["slot"]), _ptr(out["expert_count"]), _ptr(out["expert_kept"]),
        _ptr(out["expert_offset"]), _ptr(out["rank_rows"]), _ptr(stats))
    if rc != 0:
        raise ValueError(f"oracle_dispatch rejected the shape (rc={rc})")
    out["send_buf"] = send_buf
    out["send_scale"] = send_scale
    out["stats"] = {n: int(v) for n, v in zip(STAT_NAMES, stats)}
    return out


def expert_ffn(rows: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray,
               bound: bool = False):
    """One expert's SwiGLU FFN: rows [n, d], w1/w3 [H, d], w2 [d, H] (bf16 bits) -> [n, d].

    bound=True also returns, per output element, how far the unrounded
    result of an fp32 evaluation of the same expert may lie from the exact
    W2 h (float64 [n, d]; see the C source for the derivation)."""
    rows = _c(rows, np.uint16)
    w1 = _c(w1, np.uint16)
    w3 = _c(w3, np.uint16)
    w2 = _c(w2, np.uint16)
    n, d = rows.shape
    H = w1.shape[0]
    assert w1.shape == (H, d) and w3.shape == (H, d) and w2.shape == (d, H)
    out = np.empty((n, d), np.uint16)
    bnd = np.zeros((n, d), np.float64) if bound else None
    if n:
        _load().oracle_expert_ffn(n, d, H, _ptr(rows), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out),
                                  _ptr(bnd))
    return (out, bnd) if bound else out


def expert_ffn_fp8(codes: np.ndarray, scales: np.ndarray, w1: np.ndarray, w3: np.ndarray,
                   w2: np.ndarray, bound: bool = False):
    """The SwiGLU FFN on E4M3 rows: codes [n, d] uint8, scales [n] fp32 -> bf16 [n, d]
    (and the fp32-evaluation bound with bound=True, as expert_ffn)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    w1 = _c(w1, np.uint16)
    w3 = _c(w3, np.uint16)
    w2 = _c(w2, np.uint16)
    n, d = codes.shape
    H = w1.shape[0]
    assert scales.shape == (n,)
    assert w1.shape == (H, d) and w3.shape == (H, d) and w2.shape == (d, H)
    out = np.empty((n, d), np.uint16)
    bnd = np.zeros((n, d), np.float64) if bound else None
    if n:
        _load().oracle_expert_ffn_fp8(n, d, H, _ptr(codes), _ptr(scales), _ptr(w1), _ptr(w3),
                                      _ptr(w2), _ptr(out), _ptr(bnd))
    return (out, bnd) if bound else out


def expert_gate_up(rows: np.ndarray, w1: np.ndarray, w3: np.ndarray, *, codes=None,
                   scales=None, bound: bool = False):
    """The gate/up half of the expert: h = bf16(SiLU(X W1^T) * (X W3^T)) [n, H].

    rows [n, d] bf16 bits, or codes [n, d] E4M3 + scales [n] (rows=None).
    bound=True also returns, per element of h, the bound on how far an fp32
    evaluation of SiLU(g) u lies from the exact value (float64 [n, H])."""
    w1 = _c(w1, np.uint16)
    w3 = _c(w3, np.uint16)
    H, d = w1.shape
    assert w3.shape == (H, d)
    if codes is not None:
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.float32)
        n = codes.shape[0]
        assert codes.shape == (n, d) and scales.shape == (n,)
    else:
        rows = _c(rows, np.uint16)
        n = rows.shape[0]
        assert rows.shape == (n, d)
    h = np.empty((n, H), np.uint16)
    bnd = np.zeros((n, H), np.float64) if bound else None
    if n:
        if codes is not None:
            _load().oracle_expert_gate_up_fp8(n, d, H, _ptr(codes), _ptr(scales), _ptr(w1),
                                              _ptr(w3), _ptr(h), _ptr(bnd))
        else:
            _load().oracle_expert_gate_up(n, d, H, _ptr(rows), _ptr(w1), _ptr(w3), _ptr(h),
                                          _ptr(bnd))
    return (h, bnd) if bound else h


def expert_down(h: np.ndarray, w2: np.ndarray, bound: bool = False):
    """The down half of the expert: out = bf16(h W2^T) [n, d] from h [n, H] bf16 bits.
    bound=True also returns G(H) sum_j |h_j w2_mj| per element (the fp32
    accumulation bound for the same h)."""
    h = _c(h, np.uint16)
    w2 = _c(w2, np.uint16)
    n, H = h.shape
    d = w2.shape[0]
    assert w2.shape == (d, H)
    out = np.empty((n, d), np.uint16)
    bnd = np.zeros((n, d), np.float64) if bound else None
    if n:
        _load().oracle_expert_down(n, d, H, _ptr(h), _ptr(w2), _ptr(out), _ptr(bnd))
    return (out, bnd) if bound else out


def combine(expert_out: np.ndarray, slot: np.ndarray, topk_w: np.ndarray,
            shared_out: np.ndarray | None = None) -> np.ndarray:
    """y[t] = bf16(sum_s G[t,s] * expert_out[slot[t,s]] + shared_out[t]) over kept s;
    dropped -> 0; shared_out (the shared expert's [T, d] output) is optional."""
    expert_out = _c(expert_out, np.uint16)
    slot = _c(slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = slot.shape
    d = expert_out.shape[1]
    assert topk_w.shape == (T, k)
    assert slot.max(initial=-1) < expert_out.shape[0]
    if shared_out is not None:
        shared_out = _c(shared_out, np.uint16)
        assert shared_out.shape == (T, d)
    y = np.empty((T, d), np.uint16)
    _load().oracle_combine(T, d, k, _ptr(expert_out), _ptr(slot), _ptr(topk_w),
                           _ptr(shared_out), _ptr(y))
    return y


def expert_ffn_all(send_buf: np.ndarray, expert_offset: np.ndarray, expert_kept: np.ndarray,
                   w1: np.ndarray, w3: np.ndarray, w2: np.ndarray,
                   send_scale: np.ndarray | None = None, bound: bool = False):
    """Every expert's FFN on its kept rows; rows that no assignment fills stay
    zero.  With send_scale the rows are E4M3 codes (FP8 dispatch).  bound=True
    also returns the per-element fp32-evaluation bound (0 on unfilled rows)."""
    out = np.zeros(send_buf.shape, np.uint16)
    bnd = np.zeros(send_buf.shape, np.float64) if bound else None
    E = expert_kept.shape[0]
    for e in range(E):
        lo, n = int(expert_offset[e]), int(expert_kept[e])
        if not n:
            continue
        if send_scale is None:
            r = expert_ffn(send_buf[lo:lo + n], w1[e], w3[e], w2[e], bound=bound)
        else:
            r = expert_ffn_fp8(send_buf[lo:lo + n], send_scale[lo:lo + n], w1[e], w3[e], w2[e],
                               bound=bound)
        if bound:
            out[lo:lo + n], bnd[lo:lo + n] = r
        else:
            out[lo:lo + n] = r
    return (out, bnd) if bound else out


def layer_fwd(x, w_gate, w1, w3, w2, *, k: int, D: int, cf: float, my_rank: int = 0,
              bias=None, drop_policy: int = 0, min_capacity: int = 0, fp8: bool = False,
              groups: int = 1, group_limit: int = 1, shared=None) -> dict:
    """The whole forward pass, stage by stage, returning every intermediate.
    shared: (w1s, w3s, w2s) of the shared expert, applied to every token."""
    T, d = x.shape
    E = w_gate.shape[1]
    lg = logits(x, w_gate, bias)
    idx, w, gap = topk(lg, k, groups, group_limit)
    disp = dispatch(x, idx, T=T, d=d, E=E, D=D, my_rank=my_rank, cf=cf,
                    drop_policy=drop_policy, topk_w=w, min_capacity=min_capacity, fp8=fp8)
    eo, eo_bound = expert_ffn_all(disp["send_buf"], disp["expert_offset"], disp["expert_kept"],
                                  w1, w3, w2, send_scale=disp["send_scale"], bound=True)
    so, so_bound = expert_ffn(x, *shared, bound=True) if shared is not None else (None, None)
    y = combine(eo, disp["slot"], w, so)
    return dict(logits=lg, topk_idx=idx, topk_w=w, gap=gap, expert_out=eo, y=y, shared_out=so,
                expert_out_bound=eo_bound, shared_out_bound=so_bound, **disp)
