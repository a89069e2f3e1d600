"""GPU parity: every stage of the HIP path against the CPU oracle, through the
C ABI, on identical seeded inputs.

Acceptance:
  * expert indices bit-exact on identical fp32 logits; on the full path the
    kept set may differ only where the oracle's top-k boundary gap is below
    1e-5, and the order within it only between experts whose oracle logits
    are within 1e-5 of each other;
  * counts, offsets, slots, per-rank rows, counters and the send buffer
    bit-exact (fed the same routing);
  * bf16 outputs within 2e-2 |ref| + F elementwise, F a per-element floor
    derived from the fp32 arithmetic (parity_util), and 5e-3 relative
    Frobenius; each stage is checked on the GPU's own inputs for it, and the
    whole path against the oracle's own intermediate values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from expert_token_routing_moe_amd import api
from expert_token_routing_moe_amd.inputs import CONFIGS, MoEConfig, bf16_bits, make_inputs
from parity_util import (GAP, assert_bf16_close, bits_to_f64, check_expert_rows, combine_floor,
                         expert_dev, gate_rel, logit_tolerance, routing_mismatch, t2f)

pytestmark = pytest.mark.gpu
INF = math.inf

# Oracle-sized cases spanning several tiles and ragged tails.
SMALL = {
    "tiny": CONFIGS["tiny"],
    # T not a multiple of the 256-token chunk, E not a multiple of 8, capacity drops
    "ragged_e6": MoEConfig("ragged_e6", T=300, d=192, E=6, k=3, H=128, cf=1.0, D=3,
                           x_std=1.0, wg_std=0.1, w_std=0.05, seed=11),
    "dropless_e16": MoEConfig("dropless_e16", T=517, d=256, E=16, k=4, H=192, cf=INF, D=4,
                              x_std=1.0, wg_std=0.0625, w_std=0.05, seed=12),
    "e64_skew": MoEConfig("e64_skew", T=700, d=128, E=64, k=2, H=256, cf=1.25, D=8,
                          x_std=1.0, wg_std=1 / math.sqrt(128), w_std=0.05,
                          bias={2: 3.0}, seed=13),
    "e256_k8": MoEConfig("e256_k8", T=130, d=256, E=256, k=8, H=128, cf=INF, D=8,
                         x_std=1.0, wg_std=1 / 16, w_std=0.05, seed=14),
    "k_eq_E": MoEConfig("k_eq_E", T=64, d=64, E=4, k=4, H=64, cf=INF, D=2,
                        x_std=1.0, wg_std=0.125, w_std=0.05, seed=15),
    "one_token": MoEConfig("one_token", T=1, d=128, E=8, k=2, H=128, cf=1.0, D=2,
                           x_std=1.0, wg_std=0.1, w_std=0.05, seed=16),
    # H = 2048: W2 rows 4 KB apart, so the down GEMM takes its rotated K walk
    "h2048": MoEConfig("h2048", T=200, d=128, E=4, k=2, H=2048, cf=INF, D=2,
                       x_std=1.0, wg_std=0.1, w_std=0.03, seed=17),
}

DEV = "cuda"


def _host(inp):
    return {k: (bf16_bits(v) if v is not None and v.dtype == torch.bfloat16 else v)
            for k, v in inp.items()}


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


@pytest.fixture(scope="module", params=list(SMALL))
def case(request):
    cfg = SMALL[request.param]
    print(f"\n[case {cfg.name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} H={cfg.H} "
          f"cf={cfg.cf} D={cfg.D}", flush=True)
    inp = make_inputs(cfg, DEV)
    h = _host(inp)
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    ref = oracle.layer_fwd(h["x"], h["w_gate"], h["w1"], h["w3"], h["w2"], k=cfg.k, D=cfg.D,
                           cf=cfg.cf, my_rank=cfg.my_rank, bias=bias)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    return cfg, inp, h, bias, ref, shape, buf


def test_router_logits_and_selection(case):
    cfg, inp, h, bias, ref, shape, buf = case
    api.moe_route(shape, inp["x"], inp["w_gate"], inp["bias"], buf.logits, buf.topk_idx,
                  buf.topk_w, buf.workspace)
    torch.cuda.synchronize()
    lg = buf.logits.cpu().numpy()
    tol = logit_tolerance(bits_to_f64(h["x"]), bits_to_f64(h["w_gate"]))
    assert np.all(np.abs(lg.astype(np.float64) - ref["logits"]) <= tol)
    # selection on the GPU's own logits is exactly the oracle's KeepTopK
    o_idx, o_w, _ = oracle.topk(lg, cfg.k)
    np.testing.assert_array_equal(buf.topk_idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(buf.topk_w.cpu().numpy(), o_w, rtol=4e-6, atol=1e-7)
    # against the oracle's own routing, differences only at near-ties
    bad = routing_mismatch(buf.topk_idx.cpu().numpy(), ref["topk_idx"], ref["logits"], ref["gap"])
    assert not bad.any(), f"routing differs beyond near-ties for tokens {np.nonzero(bad)[0][:8]}"


# Router launch shapes: several K slices (partial sums, summed and selected
# by the second launch), several expert tiles per token tile (E > 256),
# 256-, 128- and 64-expert tiles, a non-power-of-two slice count, W_g rows
# that are not a multiple of 8 experts (padded copy), a group limit, a bias,
# one token.  (T, d, E, k, G, M, bias)
# (T, d, E, k, G, M, bias): the launch plan each shape gets (expert tile
# width BE, expert tiles, K slices) in the comment
ROUTE_CASES = [
    (200, 1024, 512, 8, 0, 0, False),     # BE 64: 8 expert tiles, 4 slices
    (100, 512, 384, 6, 0, 0, True),       # BE 64: 6 expert tiles, 2 slices
    (333, 2048, 256, 8, 8, 4, True),      # BE 64: 4 expert tiles, 8 slices, group limit
    (70, 768, 64, 2, 0, 0, False),        # BE 64: one expert tile, 3 slices
    (70, 4096, 64, 2, 0, 0, False),       # BE 64: one expert tile, 16 slices
    (129, 512, 12, 3, 0, 0, True),        # E % 8 != 0 (padded W_g copy), 2 slices
    (129, 4096, 12, 3, 0, 0, True),       # E % 8 != 0, 16 slices
    (1, 4096, 256, 8, 0, 0, False),       # one token: BE 64, 4 expert tiles, 16 slices
    (64, 7168, 1024, 16, 0, 0, False),    # BE 64: 16 expert tiles, 28 slices
    (64, 7168, 256, 8, 0, 0, True),       # DeepSeek-V3 decode: BE 64, 4 expert tiles, 28 slices
    (2048, 1024, 512, 8, 0, 0, False),    # BE 256: 2 expert tiles, 4 slices
    (2048, 4096, 128, 4, 0, 0, True),     # BE 128: one expert tile, 16 slices
    (16384, 128, 256, 8, 0, 0, False),    # BE 256, one slice (tiles alone fill the chip)
    (16384, 128, 256, 8, 8, 4, True),     # the same with a group limit and bias
    (32768, 128, 256, 8, 0, 0, False),    # 128-token tiles (twice the tiles needed), BE 256
    (65536, 64, 64, 2, 0, 0, True),       # 128-token tiles, BE 64
    (65536, 64, 256, 8, 8, 4, True),      # 256-token tiles, BE 256, group limit
    (3072, 2048, 256, 8, 0, 0, True),     # BE 256, 5 slices (one round: 240 workgroups)
    (6144, 1024, 256, 8, 8, 4, False),    # BE 256, 2 slices, group limit
    (20480, 128, 256, 8, 0, 0, False),    # 128-token tiles (64-token ones: 320, past one round)
    (40960, 128, 256, 8, 0, 0, True),     # 256-token tiles (128-token ones: 320)
]


@pytest.mark.parametrize("T,d,E,k,G,M,with_bias", ROUTE_CASES)
def test_router_launch_shapes(T, d, E, k, G, M, with_bias):
    print(f"\n[route T={T} d={d} E={E} k={k} G={G} M={M} bias={with_bias}]", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(T * 131 + E)
    x = torch.randn(T, d, generator=g, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(d, E, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    bias = torch.randn(E, generator=g, device=DEV) if with_bias else None
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=1, n_groups=G, group_limit=M)
    _, _, ws_bytes = api.moe_query(shape)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    # a workspace full of arbitrary bytes: nothing in it needs clearing
    ws = torch.randint(0, 256, (ws_bytes,), dtype=torch.uint8, generator=g, device=DEV)
    api.moe_route(shape, x, wg, bias, lg, idx, w, ws)
    torch.cuda.synchronize()
    xh, wh = bf16_bits(x), bf16_bits(wg)
    bh = None if bias is None else bias.cpu().numpy()
    ref = oracle.logits(xh, wh, bh)
    got = lg.cpu().numpy()
    assert np.all(np.abs(got.astype(np.float64) - ref) <= logit_tolerance(bits_to_f64(xh),
                                                                          bits_to_f64(wh)))
    o_idx, o_w, _ = oracle.topk(got, k, G, M)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=4e-6, atol=1e-7)
    r_idx, _, gap = oracle.topk(ref, k, G, M)
    assert not routing_mismatch(idx.cpu().numpy(), r_idx, ref, gap).any()
    # again, without the logits output, on the workspace the first call left:
    # bitwise the same selection
    idx2, w2 = torch.empty_like(idx), torch.empty_like(w)
    api.moe_route(shape, x, wg, bias, None, idx2, w2, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(w2.view(torch.int32), w.view(torch.int32))


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (64, 2), (256, 8), (5, 5), (300, 7),
                                 (200, 70), (1024, 16)])
def test_topk_on_identical_logits_with_ties(E, k):
    rng = np.random.default_rng(E * 7 + k)
    T = 333
    lg = np.concatenate([rng.integers(-3, 4, (T // 2, E)).astype(np.float32),   # many ties
                         rng.standard_normal((T - T // 2, E)).astype(np.float32)])
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0                                                           # signed zeros tie
    shape = api.Shape(T=T, d=64, E=E, k=k, H=64)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    api.moe_topk_from_logits(shape, _f32(lg), idx, w)
    torch.cuda.synchronize()
    o_idx, o_w, _ = oracle.topk(lg, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=4e-6, atol=1e-7)


def _run_dispatch(shape, x, topk_idx, buf, topk_w=None):
    api.moe_dispatch(shape, x, topk_idx, topk_w, buf.send_buf, buf.send_scale, buf.slot,
                     buf.expert_count,
                     buf.expert_kept, buf.expert_offset, buf.rank_rows, buf.stats, buf.workspace)
    torch.cuda.synchronize()


def _assert_dispatch_equal(buf, r, send_rows):
    np.testing.assert_array_equal(buf.expert_count.cpu().numpy(), r["expert_count"])
    np.testing.assert_array_equal(buf.expert_kept.cpu().numpy(), r["expert_kept"])
    np.testing.assert_array_equal(buf.expert_offset.cpu().numpy(), r["expert_offset"])
    np.testing.assert_array_equal(buf.rank_rows.cpu().numpy(), r["rank_rows"])
    np.testing.assert_array_equal(buf.slot.cpu().numpy(), r["slot"])
    assert api.stats_dict(buf.stats) == r["stats"]
    if r["send_buf"] is not None and send_rows:
        np.testing.assert_array_equal(bf16_bits(buf.send_buf[:send_rows]), r["send_buf"])


def _gpu_h(shape, send, scale, off, kept, w1, w3, workspace=None):
    """The GPU's SwiGLU hidden values for a send buffer (the gate/up half)."""
    hg = torch.zeros(send.shape[0], shape.H, dtype=torch.bfloat16, device=DEV)
    api.moe_expert_gate_up(shape, send, scale, off, kept, w1, w3, hg, workspace=workspace)
    torch.cuda.synchronize()
    return bf16_bits(hg)


def _check_layer_y(buf, r, w, h, fp8=False, shared_ref=None, grel=0.0):
    """y of a layer call, on the GPU's routing r/w: the combine stage on the
    GPU's own expert (and shared) outputs, then end to end against the
    oracle's own expert outputs.  shared_ref: (bits, end-to-end bound)."""
    eg = bf16_bits(buf.expert_out)
    sg = bf16_bits(buf.shared_out) if shared_ref is not None else None
    y = t2f(buf.y)
    assert_bf16_close(y, bits_to_f64(oracle.combine(eg, r["slot"], w, sg)), "y (combine)",
                      combine_floor(bits_to_f64(eg), r["slot"], w,
                                    None if sg is None else bits_to_f64(sg)))
    eo, eb = oracle.expert_ffn_all(r["send_buf"], r["expert_offset"], r["expert_kept"], h["w1"],
                                   h["w3"], h["w2"], send_scale=r["send_scale"] if fp8 else None,
                                   bound=True)
    so, sb = shared_ref if shared_ref is not None else (None, None)
    yref = oracle.combine(eo, r["slot"], w, so)
    assert_bf16_close(y, bits_to_f64(yref), "y (end to end)",
                      combine_floor(bits_to_f64(eo), r["slot"], w,
                                    None if so is None else bits_to_f64(so),
                                    o_dev=expert_dev(eo, eb),
                                    shared_dev=None if so is None else expert_dev(so, sb),
                                    gate_rel=grel))


def test_dispatch_bit_exact(case):
    cfg, inp, h, bias, ref, shape, buf = case
    idx = _i32(ref["topk_idx"])
    _run_dispatch(shape, inp["x"], idx, buf)
    r = oracle.dispatch(h["x"], ref["topk_idx"], T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D,
                        my_rank=cfg.my_rank, cf=cfg.cf)
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])


def test_dispatch_invalid_and_repeated_entries(case):
    cfg, inp, h, bias, ref, shape, buf = case
    idx = ref["topk_idx"].copy()
    rng = np.random.default_rng(5)
    n_bad = max(1, cfg.T // 10)
    rows = rng.integers(0, cfg.T, n_bad)
    cols = rng.integers(0, cfg.k, n_bad)
    idx[rows, cols] = rng.choice([-1, cfg.E, cfg.E + 7, -100], n_bad)
    if cfg.k > 1:
        idx[rows[0], 1] = idx[rows[0], 0]   # a repeated expert within one token
    _run_dispatch(shape, inp["x"], _i32(idx), buf)
    r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, my_rank=cfg.my_rank,
                        cf=cfg.cf)
    assert r["stats"]["invalid_index"] > 0
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])


# Shapes past the one-workgroup count-and-scan (more than 32 chunks of 256
# tokens, or chunks x experts beyond its LDS bitmaps): the count kernel per
# chunk, then the scan kernel.  Random distinct experts per token, some
# entries invalid or repeated.
@pytest.mark.parametrize("T,E,k,cf", [(9000, 64, 2, 1.25), (5000, 256, 8, INF),
                                      (8300, 8, 2, 1.0)])
def test_dispatch_count_then_scan_path(T, E, k, cf):
    rng = np.random.default_rng(T + E)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[::97, 0] = -1
    idx[5::101, k - 1] = idx[5::101, 0]
    idx[7::89, 0] = E + 5
    d = 64
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=4, capacity_factor=cf)
    buf = api.LayerBuffers.allocate(shape, DEV)
    _run_dispatch(shape, x, _i32(idx), buf)
    r = oracle.dispatch(bf16_bits(x), idx, T=T, d=d, E=E, D=4, cf=cf)
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    assert r["stats"]["invalid_index"] > 0


@pytest.mark.parametrize("k,cf", [(12, INF), (12, 1.0), (20, INF), (20, 0.75)])
def test_dispatch_and_combine_large_k(k, cf):
    """k above 8 (the count kernel's 16-slot and generic paths, the combine's
    any-k path), with repeated and out-of-range expert ids mixed in:
    dispatch bit-exact, combine within one bf16 ulp of the oracle's."""
    T, d, E = 600, 128, 32
    rng = np.random.default_rng(k * 10 + int(cf == INF))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.integers(0, T, 40)
    idx[bad, rng.integers(0, k, 40)] = rng.choice([-1, E, E + 5], 40)
    idx[bad[:10], 1] = idx[bad[:10], 0]          # repeated experts within a token
    w = rng.random((T, k)).astype(np.float32)
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=4, capacity_factor=cf)
    buf = api.LayerBuffers.allocate(shape, DEV)
    _run_dispatch(shape, x, _i32(idx), buf)
    torch.cuda.synchronize()
    r = oracle.dispatch(bf16_bits(x), idx, T=T, d=d, E=E, D=4, my_rank=0, cf=cf)
    assert r["stats"]["invalid_index"] > 0
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    n = r["stats"]["send_rows"]
    eo_bits = bf16_bits(torch.randn(max(n, 1), d).to(torch.bfloat16))[:n]
    eo = torch.from_numpy(eo_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    api.moe_combine(shape, eo, _i32(r["slot"]), _f32(w), None, y)
    torch.cuda.synchronize()
    want = bits_to_f64(oracle.combine(eo_bits, r["slot"], w))
    got = t2f(y)
    # fp32 accumulation of k terms, then one rounding to bf16: at most one bf16
    # ulp of the result plus k+1 fp32 roundings of the sum of |terms|
    # (cancellation can make the result far smaller than its terms)
    rows = bits_to_f64(eo_bits)
    mag = np.zeros((T, d))
    for s in range(k):
        sl = r["slot"][:, s]
        m = sl >= 0
        mag[m] += np.abs(w[m, s, None].astype(np.float64) * rows[sl[m]])
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    assert np.all(np.abs(got - want) <= np.maximum(ulp, 2.0 ** -133) + (k + 1) * 2.0 ** -24 * mag)


# Token counts below 4096, where the permute gives a token two or four
# wavefronts (an odd T leaves the last workgroup half past T) and the combine
# gives it up to 16 (row shares of 64 pieces or more, ragged against the
# 64 lanes): dispatch bit-exact, combine within the fp32 bound of the
# oracle's, FP8 rows and scales bit-exact too.
@pytest.mark.parametrize("T,d,E,k,cf,fp8", [
    (2049, 128, 16, 2, INF, 0),     # permute: 2 waves, odd T; combine: 1 wave
    (333, 1344, 32, 8, INF, 0),     # permute: 4 waves; combine: 2 waves of 84 pieces
    (64, 7168, 256, 8, 1.0, 0),     # DSV3 decode width, capacity drops; combine: 14 waves
    (1000, 2112, 40, 12, INF, 0),   # k > 8: two slot groups per token, any-k combine, 4 waves
    (777, 1024, 24, 4, 1.25, 1),    # E4M3 rows: every wave takes the whole row's scale
    (3001, 512, 8, 3, 0.8, 0),      # permute: 2 waves, odd T, drops; combine: 1 wave
])
def test_dispatch_and_combine_wave_split(T, d, E, k, cf, fp8):
    rng = np.random.default_rng(T * 7 + d)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[3::53, 0] = -1
    w = rng.random((T, k)).astype(np.float32)
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=4, capacity_factor=cf, dispatch_fp8=fp8)
    buf = api.LayerBuffers.allocate(shape, DEV)
    _run_dispatch(shape, x, _i32(idx), buf)
    r = oracle.dispatch(bf16_bits(x), idx, T=T, d=d, E=E, D=4, cf=cf, fp8=bool(fp8))
    n = r["stats"]["send_rows"]
    if fp8:
        for key in ("expert_count", "expert_kept", "expert_offset", "rank_rows", "slot"):
            np.testing.assert_array_equal(getattr(buf, key).cpu().numpy(), r[key], err_msg=key)
        assert api.stats_dict(buf.stats) == r["stats"]
        np.testing.assert_array_equal(buf.send_buf[:n].cpu().numpy(), r["send_buf"])
        np.testing.assert_array_equal(buf.send_scale[:n].cpu().numpy(), r["send_scale"])
    else:
        _assert_dispatch_equal(buf, r, n)
    eo_bits = bf16_bits(torch.randn(max(n, 1), d).to(torch.bfloat16))[:n]
    eo = torch.from_numpy(eo_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    api.moe_combine(shape, eo, _i32(r["slot"]), _f32(w), None, y)
    torch.cuda.synchronize()
    want = bits_to_f64(oracle.combine(eo_bits, r["slot"], w))
    rows = bits_to_f64(eo_bits)
    mag = np.zeros((T, d))
    for s_ in range(k):
        sl = r["slot"][:, s_]
        m = sl >= 0
        mag[m] += np.abs(w[m, s_, None].astype(np.float64) * rows[sl[m]])
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    got = t2f(y)
    assert np.all(np.abs(got - want) <= np.maximum(ulp, 2.0 ** -133) + (k + 1) * 2.0 ** -24 * mag)


@pytest.mark.parametrize("k", [2, 8, 12])
def test_combine_treats_slots_outside_the_rows_as_dropped(k):
    """A caller's slot array with values at or past send_rows (and -1s): the
    combine reads only rows that exist and counts the others as dropped,
    through the k <= 2, k <= 8 and any-k kernels."""
    T, d, E = 300, 256, 16
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=2)
    n, _, _ = api.moe_query(shape)
    rng = np.random.default_rng(100 + k)
    slot = rng.integers(0, n, (T, k)).astype(np.int32)
    pick = rng.random((T, k))
    slot[pick < 0.1] = -1
    # past the rows, but inside the (padded) buffer: a missing bound would
    # read the padding's large values, not fault
    slot[pick >= 0.8] = n + rng.integers(0, 64, int((pick >= 0.8).sum()))
    w = rng.random((T, k)).astype(np.float32)
    eo_bits = bf16_bits(torch.randn(n, d).to(torch.bfloat16))
    pad = np.full((64, d), np.float32(1e4).view(np.uint32) >> 16, np.uint16)
    eo = torch.from_numpy(np.concatenate([eo_bits, pad]).view(np.int16)).view(
        torch.bfloat16).to(DEV)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    api.moe_combine(shape, eo, _i32(slot), _f32(w), None, y)
    torch.cuda.synchronize()
    kept = np.where((slot >= 0) & (slot < n), slot, -1)
    want = bits_to_f64(oracle.combine(eo_bits, kept, w))
    got = t2f(y)
    rows = bits_to_f64(eo_bits)
    mag = np.zeros((T, d))
    for s in range(k):
        m = kept[:, s] >= 0
        mag[m] += np.abs(w[m, s, None].astype(np.float64) * rows[kept[m, s]])
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    assert np.all(np.abs(got - want) <= np.maximum(ulp, 2.0 ** -133) + (k + 1) * 2.0 ** -24 * mag)


def test_expert_ffn_stage(case):
    cfg, inp, h, bias, ref, shape, buf = case
    # feed the oracle's dispatch so both sides see identical rows
    send = torch.from_numpy(ref["send_buf"].view(np.int16)).view(torch.bfloat16).to(DEV)
    off = _i32(ref["expert_offset"])
    kept = _i32(ref["expert_kept"])
    out = torch.zeros_like(send)
    api.moe_expert_ffn(shape, send, None, off, kept, inp["w1"], inp["w3"], inp["w2"], out,
                       buf.workspace)
    # the two halves apart, so each is checked on its own inputs
    hg = torch.zeros(send.shape[0], cfg.H, dtype=torch.bfloat16, device=DEV)
    out2 = torch.zeros_like(send)
    api.moe_expert_gate_up(shape, send, None, off, kept, inp["w1"], inp["w3"], hg)
    api.moe_expert_down(shape, hg, off, kept, inp["w2"], out2)
    torch.cuda.synchronize()
    got, hb = bf16_bits(out), bf16_bits(hg)
    assert np.array_equal(got, bf16_bits(out2))
    for e in range(cfg.E):
        lo, n = int(ref["expert_offset"][e]), int(ref["expert_kept"][e])
        if n:
            check_expert_rows(f"expert {e}", h["w1"][e], h["w3"][e], h["w2"][e],
                              hb[lo:lo + n], got[lo:lo + n], rows=ref["send_buf"][lo:lo + n])


def test_combine_stage(case):
    cfg, inp, h, bias, ref, shape, buf = case
    eo = torch.from_numpy(ref["expert_out"].view(np.int16)).view(torch.bfloat16).to(DEV)
    y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
    api.moe_combine(shape, eo, _i32(ref["slot"]), _f32(ref["topk_w"]), None, y)
    torch.cuda.synchronize()
    got, want = t2f(y), bits_to_f64(ref["y"])
    res = assert_bf16_close(got, want, "combine",
                            combine_floor(bits_to_f64(ref["expert_out"]), ref["slot"],
                                          ref["topk_w"]))
    # same inputs, fp32 vs double accumulation: at most one bf16 ulp apart
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    assert np.all(np.abs(got - want) <= np.maximum(ulp, 2.0 ** -133))
    assert res is None or res["exact"] > 0.95


def test_layer_fwd_end_to_end(case):
    cfg, inp, h, bias, ref, shape, buf = case
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf)
    torch.cuda.synchronize()
    idx = buf.topk_idx.cpu().numpy()
    flips = np.any(idx != ref["topk_idx"], axis=1)
    assert not routing_mismatch(idx, ref["topk_idx"], ref["logits"], ref["gap"]).any()
    w = buf.topk_w.cpu().numpy()
    if flips.any():
        # a legitimate near-tie flip: check the rest on the GPU's own routing
        r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D,
                            my_rank=cfg.my_rank, cf=cfg.cf)
        eo, eb = oracle.expert_ffn_all(r["send_buf"], r["expert_offset"], r["expert_kept"],
                                       h["w1"], h["w3"], h["w2"], bound=True)
        yref, grel = oracle.combine(eo, r["slot"], w), 0.0
    else:
        r, yref, eo, eb, grel = ref, ref["y"], ref["expert_out"], ref["expert_out_bound"], \
            gate_rel(cfg.k)
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    # the combine on the GPU's own expert outputs and gates
    eg = bf16_bits(buf.expert_out)
    assert_bf16_close(t2f(buf.y), bits_to_f64(oracle.combine(eg, r["slot"], w)), "y (combine)",
                      combine_floor(bits_to_f64(eg), r["slot"], w))
    # end to end, every step by the oracle
    assert_bf16_close(t2f(buf.y), bits_to_f64(yref), "y (end to end)",
                      combine_floor(bits_to_f64(eo), r["slot"], w, o_dev=expert_dev(eo, eb),
                                    gate_rel=grel))
    # determinism: a second run is bitwise identical
    y1 = buf.y.clone()
    eo1 = buf.expert_out.clone()
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf)
    torch.cuda.synchronize()
    assert torch.equal(buf.y.view(torch.int16), y1.view(torch.int16))
    n = r["stats"]["send_rows"]
    kept_rows = np.zeros(n, bool)
    for e in range(cfg.E):
        lo = int(r["expert_offset"][e])
        kept_rows[lo:lo + int(r["expert_kept"][e])] = True
    kr = torch.from_numpy(kept_rows).to(DEV)
    assert torch.equal(buf.expert_out[:n][kr].view(torch.int16), eo1[:n][kr].view(torch.int16))


# ---------------------------------------------------------------------------
# Drop by gate value (drop policy 1) and the minimum capacity.  The oracle is
# fed the GPU's own fp32 gates, so both sides rank on identical values.
# ---------------------------------------------------------------------------

def test_dispatch_by_gate_bit_exact(case):
    cfg, inp, h, bias, ref, shape, buf = case
    sh1 = dataclasses.replace(shape, drop_policy=1)
    b1 = api.LayerBuffers.allocate(sh1, DEV)
    api.moe_route(sh1, inp["x"], inp["w_gate"], inp["bias"], None, b1.topk_idx, b1.topk_w,
                  b1.workspace)
    _run_dispatch(sh1, inp["x"], b1.topk_idx, b1, b1.topk_w)
    idx, w = b1.topk_idx.cpu().numpy(), b1.topk_w.cpu().numpy()
    r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, my_rank=cfg.my_rank,
                        cf=cfg.cf, drop_policy=1, topk_w=w)
    _assert_dispatch_equal(b1, r, r["stats"]["send_rows"])
    r0 = oracle.dispatch(None, idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, my_rank=cfg.my_rank,
                         cf=cfg.cf, with_send_buf=False)
    assert r0["stats"] == r["stats"]
    if r["stats"]["dropped"]:
        print(f"  dropped {r['stats']['dropped']}; slots differing from token order: "
              f"{int((r0['slot'] != r['slot']).sum())}", flush=True)


@pytest.mark.parametrize("T,E,k,cf,levels,seed", [
    (3000, 16, 4, 0.5, 4, 1),      # few gate levels: many exact ties across tokens
    (2500, 8, 2, 0.3, 1, 2),       # one level: probability order is token order
    (1000, 64, 8, 0.25, 1000, 3),  # near-distinct gates, heavy drops
    (300, 6, 3, 1.0, 3, 4),
])
def test_dispatch_by_gate_ties_bit_exact(T, E, k, cf, levels, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = (rng.integers(1, levels + 1, (T, k)) / (levels + 1)).astype(np.float32)
    d = 64
    x = torch.from_numpy(rng.integers(0, 65535, (T, d)).astype(np.uint16).view(np.int16))
    x = x.view(torch.bfloat16).to(DEV)
    shape = api.Shape(T=T, d=d, E=E, k=k, H=64, D=2, capacity_factor=cf, drop_policy=1)
    buf = api.LayerBuffers.allocate(shape, DEV)
    _run_dispatch(shape, x, _i32(idx), buf, _f32(w))
    r = oracle.dispatch(bf16_bits(x), idx, T=T, d=d, E=E, D=2, cf=cf, drop_policy=1, topk_w=w)
    assert r["stats"]["dropped"] > 0
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    if levels == 1:
        r0 = oracle.dispatch(None, idx, T=T, d=d, E=E, D=2, cf=cf, with_send_buf=False)
        np.testing.assert_array_equal(buf.slot.cpu().numpy(), r0["slot"])


@pytest.mark.parametrize("mc", [0, 100, 1000])
def test_dispatch_minimum_capacity(mc):
    cfg = SMALL["e64_skew"]
    inp = make_inputs(cfg, DEV, experts=False)
    for policy in (0, 1):
        shape = dataclasses.replace(api.Shape.from_config(cfg), drop_policy=policy,
                                    min_capacity=mc)
        buf = api.LayerBuffers.allocate(shape, DEV)
        api.moe_route(shape, inp["x"], inp["w_gate"], inp["bias"], None, buf.topk_idx,
                      buf.topk_w, buf.workspace)
        _run_dispatch(shape, inp["x"], buf.topk_idx, buf, buf.topk_w)
        idx, w = buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy()
        r = oracle.dispatch(bf16_bits(inp["x"]), idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D,
                            cf=cfg.cf, drop_policy=policy, topk_w=w, min_capacity=mc)
        assert r["stats"]["capacity"] == max(oracle.capacity(cfg.T, cfg.k, cfg.E, cfg.cf), mc)
        _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
        if mc >= 1000:
            assert r["stats"]["dropped"] == 0


@pytest.mark.parametrize("name", ["tiny", "ragged_e6", "e64_skew", "one_token"])
def test_layer_fwd_by_gate_end_to_end(name):
    cfg = SMALL[name].with_(drop_policy=1)
    inp = make_inputs(cfg, DEV)
    h = _host(inp)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf)
    torch.cuda.synchronize()
    # checked on the GPU's own routing (itself checked against the oracle elsewhere)
    idx, w = buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy()
    r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, cf=cfg.cf,
                        drop_policy=1, topk_w=w)
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    _check_layer_y(buf, r, w, h)


# ---------------------------------------------------------------------------
# FP8 dispatch payload: E4M3 rows with fp32 row scales; combine stays bf16.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 4099 * 16, 3 << 20, 64 << 20])
def test_stream_read_reads_every_word(nbytes):
    """The read-rate probe reads every word once (ragged tails, one to 2048
    workgroups): a zero buffer holding the mark in one word, at the first,
    last, a middle and a tail position, sets the sink; with the mark in two
    words read by one lane the lane's XOR is zero and nothing is stored."""
    mark = np.uint32(api.STREAM_READ_MARK).view(np.int32)
    n = nbytes // 4
    src = torch.zeros(n, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    for p in sorted({0, n - 1, n // 2, max(0, n - 5), 3}):
        if p >= n:
            continue
        src.zero_()
        sink.zero_()
        src[p] = int(mark)
        api.moe_stream_read(src, sink)
        torch.cuda.synchronize()
        assert int(sink[0].item()) == int(mark), f"word {p} of {n} not read"
    src.zero_()
    sink.zero_()
    src[0] = int(mark)
    src[1] = int(mark)  # same 16-byte piece, same lane: XOR 0
    api.moe_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 0


@pytest.mark.parametrize("nbytes", [16, 4099 * 16, 3 << 20, 64 << 20])
def test_stream_write_fills_every_word(nbytes):
    """The store-rate probe writes its value to every word once (ragged
    tails, one to 2048 workgroups) and nothing past the buffer's end."""
    n = nbytes // 4
    pad = 64
    buf = torch.zeros(n + pad, dtype=torch.int32, device=DEV)
    value = 0x5A5A1234
    api.moe_stream_write(buf[:n], value)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[:n] == value).all()
    assert (got[n:] == 0).all()


@pytest.mark.parametrize("k,T,d", [(2, 300, 512), (8, 300, 512), (12, 300, 512),
                                   (8, 64, 7168), (3, 301, 2112), (12, 33, 1536)])
def test_stream_gather_xors_the_slotted_rows(k, T, d):
    """The combine-pattern probe: out[t] is the XOR of the rows its slots
    name, a slot outside [0, nrows) adding nothing (those slots point into
    padding rows, so a missing bound shows as a wrong value).  The wide
    rows at few tokens split a token over 14, 4 and 3 wavefronts."""
    nrows, pad = 700, 64
    rng = np.random.default_rng(7 + k)
    rows = rng.integers(-2 ** 15, 2 ** 15, (nrows + pad, d), dtype=np.int64).astype(np.int16)
    slot = rng.integers(0, nrows, (T, k)).astype(np.int32)
    pick = rng.random((T, k))
    slot[pick < 0.1] = -1
    slot[pick > 0.9] = nrows + rng.integers(0, pad, int((pick > 0.9).sum()))
    want = np.zeros((T, d), np.int16)
    for s in range(k):
        m = (slot[:, s] >= 0) & (slot[:, s] < nrows)
        want[m] ^= rows[slot[m, s]]
    r = torch.from_numpy(rows).to(DEV).view(torch.bfloat16)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    api.moe_stream_gather(r[:nrows], _i32(slot), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy(), want)


def test_fp8_decode_every_code():
    """The expert GEMM's E4M3 -> bf16 decode, through the diagnostic entry
    point: all 256 codes at unit and power-of-two scales, bit-exact."""
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    codes = np.concatenate([codes] * 4)                      # 64 rows
    scales = (2.0 ** np.repeat([0, -3, 4, 0], 16)).astype(np.float32)
    out = torch.empty(64, 16, dtype=torch.bfloat16, device=DEV)
    api.moe_fp8_rows_to_bf16(torch.from_numpy(codes).to(DEV), _f32(scales), out)
    torch.cuda.synchronize()
    got = t2f(out)
    want = oracle.fp8_values(codes) * scales[:, None].astype(np.float64)
    nan = np.isnan(want)
    assert np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], want[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _fp8_shape(shape):
    return dataclasses.replace(shape, dispatch_fp8=1)


def test_dispatch_fp8_bit_exact(case):
    cfg, inp, h, bias, ref, shape, buf = case
    sh8 = _fp8_shape(shape)
    b8 = api.LayerBuffers.allocate(sh8, DEV)
    _run_dispatch(sh8, inp["x"], _i32(ref["topk_idx"]), b8)
    r = oracle.dispatch(h["x"], ref["topk_idx"], T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D,
                        my_rank=cfg.my_rank, cf=cfg.cf, fp8=True)
    n = r["stats"]["send_rows"]
    for key in ("expert_count", "expert_kept", "expert_offset", "rank_rows", "slot"):
        np.testing.assert_array_equal(getattr(b8, key).cpu().numpy(), r[key], err_msg=key)
    assert api.stats_dict(b8.stats) == r["stats"]
    np.testing.assert_array_equal(b8.send_buf[:n].cpu().numpy(), r["send_buf"])
    np.testing.assert_array_equal(b8.send_scale[:n].cpu().numpy(), r["send_scale"])


def test_expert_ffn_fp8_stage(case):
    cfg, inp, h, bias, ref, shape, buf = case
    sh8 = _fp8_shape(shape)
    r = oracle.dispatch(h["x"], ref["topk_idx"], T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D,
                        my_rank=cfg.my_rank, cf=cfg.cf, fp8=True)
    send = torch.from_numpy(r["send_buf"]).to(DEV)
    scale = _f32(r["send_scale"])
    out = torch.zeros(send.shape, dtype=torch.bfloat16, device=DEV)
    ws = api.LayerBuffers.allocate(sh8, DEV).workspace
    off, kept = _i32(r["expert_offset"]), _i32(r["expert_kept"])
    api.moe_expert_ffn(sh8, send, scale, off, kept, inp["w1"], inp["w3"], inp["w2"], out, ws)
    torch.cuda.synchronize()
    got = bf16_bits(out)
    hb = _gpu_h(sh8, send, scale, off, kept, inp["w1"], inp["w3"], ws)
    for e in range(cfg.E):
        lo, n = int(r["expert_offset"][e]), int(r["expert_kept"][e])
        if n:
            check_expert_rows(f"fp8 expert {e}", h["w1"][e], h["w3"][e], h["w2"][e],
                              hb[lo:lo + n], got[lo:lo + n], codes=r["send_buf"][lo:lo + n],
                              scales=r["send_scale"][lo:lo + n])


# Expert row counts that reach every per-wave slice count (0..8) of a 256-row
# tile at each ring depth the GEMM picks (4, 3 and 2 stages; 2 also through its
# compile-time two-stage path, 161..256 rows), experts cut into 2 and 3 equal
# M tiles (257, 384, 400, 513 rows), and empty experts.
TILE_ROWS = [1, 16, 17, 40, 56, 57, 96, 97, 128, 160, 161, 170, 176, 177, 192, 193, 224, 256,
             257, 384, 400, 513, 0, 3]


# (d, H, fp8): the launches estimate 24 M tiles (24 experts, 3,774 rows), so
# d = H = 256 gives both GEMMs fewer tiles than CUs and the 64-column tiles;
# H = 1408 gives the gate/up GEMM 24 x 11 tiles and its 128-column tiles;
# d = 2816 gives the down GEMM 24 x 11 tiles and its 256-column tiles.
TILE_SHAPES = [(256, 256, False), (256, 256, True), (256, 1408, False), (2816, 128, False)]


@pytest.mark.parametrize("d,H,fp8", TILE_SHAPES)
def test_expert_ffn_every_tile_shape(d, H, fp8):
    counts = np.array(TILE_ROWS, np.int32)
    E, n = len(counts), int(counts.sum())
    cfg = MoEConfig("tile_rows", T=n, d=d, E=E, k=1, H=H, cf=INF, D=1, x_std=1.0,
                    wg_std=0.1, w_std=0.05, seed=18, dispatch_fp8=int(fp8))
    print(f"\n[tile rows] d={d} H={H} fp8={fp8} E={E} rows={n}", flush=True)
    inp = make_inputs(cfg, DEV)
    shape = api.Shape.from_config(cfg)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = bf16_bits(inp["x"])  # expert e's rows are x[off[e]:off[e + 1]]
    w1, w3, w2 = (bf16_bits(inp[k]) for k in ("w1", "w3", "w2"))
    if fp8:
        q, sc = oracle.fp8_quantize_rows(x)
        send, scale = torch.from_numpy(q).to(DEV), _f32(sc)
    else:
        send, scale = inp["x"], None
    out = torch.zeros(n, cfg.d, dtype=torch.bfloat16, device=DEV)
    ws = api.LayerBuffers.allocate(shape, DEV).workspace
    api.moe_expert_ffn(shape, send, scale, _i32(off), _i32(counts), inp["w1"], inp["w3"],
                       inp["w2"], out, ws)
    torch.cuda.synchronize()
    got = bf16_bits(out)
    hb = _gpu_h(shape, send, scale, _i32(off), _i32(counts), inp["w1"], inp["w3"], ws)
    for e in range(E):
        lo, m = int(off[e]), int(counts[e])
        if m:
            rows = dict(codes=q[lo:lo + m], scales=sc[lo:lo + m]) if fp8 else \
                dict(rows=x[lo:lo + m])
            check_expert_rows(f"expert {e} ({m} rows)", w1[e], w3[e], w2[e], hb[lo:lo + m],
                              got[lo:lo + m], **rows)


# Expert rows for the two grouped-GEMM kernels: an empty expert; tiles whose
# second 128-row group holds 0..8 non-empty 16-row slices (1, 40, 145, 177,
# 193, 209, 255, 256 rows, and 257 rows cut into two tiles of 129); experts cut
# into 3 and 8 equal M tiles (513, 700 and 2,018 rows); 4,764 rows in all.
PP_ROWS = [0, 1, 40, 145, 177, 193, 209, 255, 256, 257, 513, 700, 2018]


def test_pingpong_gemm_matches_the_ring_kernel():
    """The ping-pong kernel (shapes where an expert is expected to hold >= 512
    rows) and the ring kernel give the same bits on the same rows: a shape of
    6,656 tokens (512 per expert) takes the first, one of 4,764 tokens (367 per
    expert) the second, on the same send buffer, offsets and counts.  The down
    GEMM's K walk is rotated (H = 2048, a 4 KB weight-row pitch).  Three
    experts are also checked against the oracle."""
    counts = np.array(PP_ROWS, np.int32)
    E, n = len(counts), int(counts.sum())
    cfg = MoEConfig("pingpong", T=512 * E, d=4096, E=E, k=1, H=2048, cf=INF, D=1, x_std=1.0,
                    wg_std=0.1, w_std=0.02, seed=29)
    print(f"\n[pingpong] d={cfg.d} H={cfg.H} E={E} rows={n}", flush=True)
    inp = make_inputs(cfg, DEV)
    pp = api.Shape.from_config(cfg)
    ring = api.Shape.from_config(cfg.with_(T=n))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    outs = []
    for shape in (pp, ring):
        h = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device=DEV)
        out = torch.zeros(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
        api.moe_expert_gate_up(shape, inp["x"], None, _i32(off), _i32(counts), inp["w1"],
                               inp["w3"], h)
        api.moe_expert_down(shape, h, _i32(off), _i32(counts), inp["w2"], out)
        torch.cuda.synchronize()
        outs.append((bf16_bits(h[:n]), bf16_bits(out[:n])))
    (hp, op), (hr, orr) = outs
    assert np.array_equal(hp, hr), "h differs between the two kernels"
    assert np.array_equal(op, orr), "expert outputs differ between the two kernels"
    x = bf16_bits(inp["x"])
    w1, w3, w2 = (bf16_bits(inp[k]) for k in ("w1", "w3", "w2"))
    rng = np.random.default_rng(5)
    for e in (1, 5, 12):
        lo, m = int(off[e]), int(counts[e])
        r = np.sort(rng.choice(m, min(m, 24), replace=False)) + lo
        check_expert_rows(f"expert {e} ({m} rows)", w1[e], w3[e], w2[e], hp[r], op[r],
                          rows=x[r])
    del inp
    torch.cuda.empty_cache()


def test_expert_ffn_clips_rows_outside_the_buffers():
    """Caller-given offsets and counts that reach past the send buffer's rows:
    each expert's rows are clipped to [0, send_rows), an expert whose offset
    lies past them has none, and no row past send_rows is read or written.
    The buffers carry 64 padding rows, so a missing clip would show in them
    (never as an access outside an allocation)."""
    counts = np.array([40, 0, 300, 17, 64, 90], np.int32)
    E, n = len(counts), int(counts.sum())
    cfg = MoEConfig("clip_rows", T=n, d=256, E=E, k=1, H=128, cf=INF, D=1, x_std=1.0,
                    wg_std=0.1, w_std=0.05, seed=23)
    inp = make_inputs(cfg, DEV)
    shape = api.Shape.from_config(cfg)
    assert api.moe_query(shape)[0] == n
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    kept = counts.copy()
    kept[5] += 30                       # 30 rows past the end: clipped
    off_in = off.copy()
    off_in[1], kept[1] = n + 5, 10      # starts past the end: no rows
    pad = 64
    x = bf16_bits(inp["x"])
    w1, w3, w2 = (bf16_bits(inp[k]) for k in ("w1", "w3", "w2"))
    big = np.float32(1e4).view(np.uint32) >> 16
    send_np = np.concatenate([x, np.full((pad, cfg.d), big, np.uint16)])
    send = torch.from_numpy(send_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    sentinel = -12345
    h = torch.full((n + pad, cfg.H), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    out = torch.full((n + pad, cfg.d), sentinel, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    api.moe_expert_gate_up(shape, send, None, _i32(off_in), _i32(kept), inp["w1"], inp["w3"], h)
    api.moe_expert_down(shape, h, _i32(off_in), _i32(kept), inp["w2"], out)
    torch.cuda.synchronize()
    hb, ob = bf16_bits(h), bf16_bits(out)
    assert np.all(hb[n:].view(np.int16) == sentinel) and np.all(ob[n:].view(np.int16) == sentinel)
    for e in (0, 2, 3, 4, 5):
        lo, m = int(off[e]), int(counts[e])   # clipped: expert 5 ends at n
        check_expert_rows(f"expert {e} ({m} rows)", w1[e], w3[e], w2[e], hb[lo:lo + m],
                          ob[lo:lo + m], rows=x[lo:lo + m])


def test_fp8_widened_gate_up_matches_register_path():
    """At >= 512 rows per expert (MFMA-bound) the gate/up GEMM, given a
    workspace, widens the E4M3 rows to bf16 in one pass before the bf16 loop;
    without one it widens them in registers.  The two give the same bits on
    every kept row, and the layer (which takes the widened path) matches the
    oracle."""
    cfg = MoEConfig("fp8_widen", T=1536, d=256, E=4, k=2, H=256, cf=INF, D=2, x_std=1.0,
                    wg_std=0.1, w_std=0.05, seed=19, dispatch_fp8=1)  # 768 rows per expert
    print(f"\n[fp8 widen] T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    inp = make_inputs(cfg, DEV)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf)
    torch.cuda.synchronize()
    n = buf.send_buf.shape[0]
    hw = torch.zeros(n, cfg.H, dtype=torch.bfloat16, device=DEV)
    hr = torch.zeros(n, cfg.H, dtype=torch.bfloat16, device=DEV)
    args = (shape, buf.send_buf, buf.send_scale, buf.expert_offset, buf.expert_kept,
            inp["w1"], inp["w3"])
    api.moe_expert_gate_up(*args, hw, workspace=buf.workspace)
    api.moe_expert_gate_up(*args, hr)
    torch.cuda.synchronize()
    off, kept = buf.expert_offset.cpu().numpy(), buf.expert_kept.cpu().numpy()
    assert kept.min() >= 512
    for e in range(cfg.E):
        lo, m = int(off[e]), int(kept[e])
        assert torch.equal(hw[lo:lo + m].view(torch.int16), hr[lo:lo + m].view(torch.int16)), e
    w1, w3, w2 = (bf16_bits(inp[k]) for k in ("w1", "w3", "w2"))
    codes, scales = buf.send_buf.cpu().numpy(), buf.send_scale.cpu().numpy()
    got, hb = bf16_bits(buf.expert_out), bf16_bits(hw)
    for e in range(cfg.E):
        lo, m = int(off[e]), int(kept[e])
        check_expert_rows(f"fp8 widened expert {e}", w1[e], w3[e], w2[e], hb[lo:lo + m],
                          got[lo:lo + m], codes=codes[lo:lo + m], scales=scales[lo:lo + m])


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_fwd_fp8_end_to_end(name):
    cfg = SMALL[name].with_(dispatch_fp8=1)
    inp = make_inputs(cfg, DEV)
    h = _host(inp)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf)
    torch.cuda.synchronize()
    idx, w = buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy()
    r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, cf=cfg.cf, fp8=True)
    n = r["stats"]["send_rows"]
    np.testing.assert_array_equal(buf.send_buf[:n].cpu().numpy(), r["send_buf"])
    _check_layer_y(buf, r, w, h, fp8=True)


# ---------------------------------------------------------------------------
# Group-limited routing and the replicated shared expert.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E,k,G,M,ties", [(256, 8, 8, 4, False), (256, 8, 8, 4, True),
                                          (64, 6, 8, 3, True), (16, 4, 4, 2, True),
                                          (12, 3, 6, 2, False), (1024, 8, 64, 5, False)])
def test_topk_group_limited_on_identical_logits(E, k, G, M, ties):
    T = 777
    rng = np.random.default_rng(E + G + M)
    if ties:
        lg = rng.integers(-3, 4, (T, E)).astype(np.float32)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    shape = api.Shape(T=T, d=64, E=E, k=k, H=64, n_groups=G, group_limit=M)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    api.moe_topk_from_logits(shape, _f32(lg), idx, w)
    torch.cuda.synchronize()
    o_idx, o_w, _ = oracle.topk(lg, k, G, M)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=4e-6, atol=1e-7)


GROUPED = {
    "tiny_g4m2_shared": CONFIGS["tiny"].with_(n_groups=4, group_limit=2, shared_H=256),
    "e256_k8_g8m4_shared": SMALL["e256_k8"].with_(n_groups=8, group_limit=4, shared_H=128),
    "dropless_e16_g8m3": SMALL["dropless_e16"].with_(n_groups=8, group_limit=3),
    "ragged_shared": SMALL["ragged_e6"].with_(shared_H=192),
}


@pytest.mark.parametrize("name", list(GROUPED))
def test_layer_fwd_grouped_and_shared_end_to_end(name):
    cfg = GROUPED[name]
    print(f"\n[grouped {name}] G={cfg.n_groups} M={cfg.group_limit} shared_H={cfg.shared_H}",
          flush=True)
    inp = make_inputs(cfg, DEV)
    h = _host(inp)
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    shared = (inp["w1s"], inp["w3s"], inp["w2s"]) if cfg.shared_H else None
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf, shared=shared)
    torch.cuda.synchronize()
    # routing against the oracle's logits (the gap covers group near-ties too)
    lg_ref = oracle.logits(h["x"], h["w_gate"], bias)
    r_idx, _, gap = oracle.topk(lg_ref, cfg.k, cfg.n_groups, cfg.group_limit)
    idx, w = buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy()
    assert not routing_mismatch(idx, r_idx, lg_ref, gap).any()
    # on identical logits the selection is bit-exact
    o_idx, o_w, _ = oracle.topk(buf.logits.cpu().numpy(), cfg.k, cfg.n_groups, cfg.group_limit)
    np.testing.assert_array_equal(idx, o_idx)
    # downstream on the GPU's own routing
    r = oracle.dispatch(h["x"], idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, cf=cfg.cf)
    _assert_dispatch_equal(buf, r, r["stats"]["send_rows"])
    shared_ref = None
    if cfg.shared_H:
        _check_shared(cfg, inp, h, buf.shared_out)
        shared_ref = oracle.expert_ffn(h["x"], h["w1s"], h["w3s"], h["w2s"], bound=True)
    _check_layer_y(buf, r, w, h, shared_ref=shared_ref)


def _check_shared(cfg, inp, h, shared_out, toks=None):
    """The shared expert's output against the oracle, stage by stage: its
    hidden values come from the gate/up half run as one group of all T
    tokens (the kernels moe_shared_expert uses)."""
    sh = api.Shape(T=cfg.T, d=cfg.d, E=1, k=1, H=cfg.shared_H)
    off, cnt = _i32([0, cfg.T]), _i32([cfg.T])
    hb = _gpu_h(sh, inp["x"], None, off, cnt, inp["w1s"], inp["w3s"])
    so = bf16_bits(shared_out)
    toks = np.arange(cfg.T) if toks is None else toks
    check_expert_rows("shared expert", h["w1s"], h["w3s"], h["w2s"], hb[toks], so[toks],
                      rows=h["x"][toks])


def test_shared_expert_and_combine_stages():
    cfg = CONFIGS["tiny"].with_(shared_H=320, T=300)
    inp = make_inputs(cfg, DEV)
    h = _host(inp)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    api.moe_shared_expert(shape, inp["x"], inp["w1s"], inp["w3s"], inp["w2s"], buf.shared_out,
                          buf.workspace)
    torch.cuda.synchronize()
    _check_shared(cfg, inp, h, buf.shared_out)
    so = oracle.expert_ffn(h["x"], h["w1s"], h["w3s"], h["w2s"])
    # combine on identical inputs: within one bf16 ulp of the oracle
    ref = oracle.layer_fwd(h["x"], h["w_gate"], h["w1"], h["w3"], h["w2"], k=cfg.k, D=cfg.D,
                           cf=cfg.cf)
    eo = torch.from_numpy(ref["expert_out"].view(np.int16)).view(torch.bfloat16).to(DEV)
    sot = torch.from_numpy(so.view(np.int16)).view(torch.bfloat16).to(DEV)
    y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
    api.moe_combine(shape, eo, _i32(ref["slot"]), _f32(ref["topk_w"]), sot, y)
    torch.cuda.synchronize()
    want = bits_to_f64(oracle.combine(ref["expert_out"], ref["slot"], ref["topk_w"], so))
    got = t2f(y)
    # one bf16 ulp of the result, plus the fp32 rounding of k + 1 terms: the
    # shared term can nearly cancel the routed sum
    mag = np.abs(bits_to_f64(so))
    for s_ in range(cfg.k):
        sl = ref["slot"][:, s_]
        rows = np.where(sl[:, None] >= 0, np.abs(bits_to_f64(ref["expert_out"][np.maximum(sl, 0)])), 0)
        mag += ref["topk_w"][:, s_:s_ + 1].astype(np.float64) * rows
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    bound = np.maximum(ulp, 2.0 ** -133) + (cfg.k + 1) * 2.0 ** -24 * mag
    assert np.all(np.abs(got - want) <= bound)
    assert np.mean(got == want) > 0.95


# every output the layer writes in full (expert_out: only its kept rows)
GRAPH_OUTPUTS = ("y", "logits", "topk_idx", "topk_w", "send_buf", "send_scale", "slot",
                 "expert_count", "expert_kept", "expert_offset", "rank_rows", "stats",
                 "shared_out")


# A shape whose grouped GEMMs take the ping-pong kernel (1,024 rows per
# expert, 256 tiles per launch); checked in the graph test only (no oracle).
GRAPH_ONLY = {
    "pingpong": MoEConfig("pingpong_graph", T=2048, d=4096, E=4, k=2, H=2048, cf=INF, D=2,
                          x_std=1.0, wg_std=1 / 64, w_std=0.02, seed=31),
}


@pytest.mark.parametrize("name,fp8", [("tiny", False), ("e64_skew", False), ("ragged_e6", True),
                                      ("pingpong", False)])
def test_layer_fwd_in_hip_graph(name, fp8):
    """The whole layer call is captured in a HIP graph (no allocation, no
    memset, no host synchronisation inside) and every replay reproduces the
    eager outputs bit for bit, also after eager kernels overwrite every
    output between replays."""
    cfg = (SMALL[name] if name in SMALL else GRAPH_ONLY[name]).with_(dispatch_fp8=int(fp8))
    print(f"\n[graph {name} fp8={fp8}]", flush=True)
    inp = make_inputs(cfg, DEV)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    call = lambda: api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"],
                                     inp["w3"], inp["w2"], buf)
    call()
    torch.cuda.synchronize()
    outs = {n: getattr(buf, n) for n in GRAPH_OUTPUTS if getattr(buf, n) is not None}
    ref = {n: t.clone() for n, t in outs.items()}
    off, kept = buf.expert_offset.cpu().numpy(), buf.expert_kept.cpu().numpy()
    rows = torch.from_numpy(np.concatenate(
        [np.arange(off[e], off[e] + kept[e]) for e in range(cfg.E)]).astype(np.int64)).to(DEV)
    ref_eo = buf.expert_out[rows].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in list(outs.values()) + [buf.expert_out]:  # eager work between replays
            t.view(torch.uint8).fill_(0xA5 if rep % 2 else 0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t.view(torch.uint8), ref[n].view(torch.uint8)), (rep, n)
        assert torch.equal(buf.expert_out[rows].view(torch.int16), ref_eo.view(torch.int16)), rep
    del g


@pytest.mark.parametrize("k", [2, 8])
def test_identity_experts_round_trip_on_gpu(k):
    """Dispatch then combine with identity experts and nothing dropped gives x
    back bit for bit (k = E = 8 included)."""
    cfg = CONFIGS["tiny"].with_(k=k, cf=INF)
    inp = make_inputs(cfg, DEV, experts=False)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    api.moe_route(shape, inp["x"], inp["w_gate"], None, buf.logits, buf.topk_idx, buf.topk_w,
                  buf.workspace)
    _run_dispatch(shape, inp["x"], buf.topk_idx, buf)
    api.moe_combine(shape, buf.send_buf, buf.slot, buf.topk_w, None, buf.y)
    torch.cuda.synchronize()
    assert torch.equal(buf.y.view(torch.int16), inp["x"].view(torch.int16))


def test_zero_tokens():
    """T = 0: nothing to route; dispatch still writes zero counts and counters."""
    shape = api.Shape(T=0, d=128, E=8, k=2, H=128, D=2, capacity_factor=1.25)
    buf = api.LayerBuffers.allocate(shape, DEV)
    buf.expert_count.fill_(-7)
    buf.expert_offset.fill_(-7)
    buf.stats.fill_(-7)
    x = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    _run_dispatch(shape, x, idx, buf)
    assert buf.expert_count.cpu().tolist() == [0] * 8
    assert buf.expert_offset.cpu().tolist() == [0] * 9
    st = api.stats_dict(buf.stats)
    assert st["assignments"] == 0 and st["kept"] == 0 and st["capacity"] == 0
    inp = make_inputs(CONFIGS["tiny"].with_(T=0, d=128, H=128), DEV)
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"], inp["w2"], buf)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Full-size workloads: the whole path at its real shape, checked on the parts
# the oracle can compute one by one (all routing and accounting; a sample of
# experts and tokens for the FFN and the combine).
# ---------------------------------------------------------------------------

def _expert_weights(inp, e):
    return (bf16_bits(inp["w1"][e]), bf16_bits(inp["w3"][e]), bf16_bits(inp["w2"][e]))


FULL_VARIANTS = {
    "dsv3_prefill_g8m4_shared": CONFIGS["dsv3_prefill"].with_(n_groups=8, group_limit=4,
                                                              shared_H=2048),
    "skewed_by_gate": CONFIGS["skewed"].with_(drop_policy=1),
    "dsv3_prefill_fp8": CONFIGS["dsv3_prefill"].with_(dispatch_fp8=1),
    "mixtral_fp8": CONFIGS["mixtral"].with_(dispatch_fp8=1),
}


@pytest.mark.parametrize("name", ["mixtral", "dsv3_prefill", "dsv3_decode", "skewed",
                                  "skewed_by_gate", "dsv3_prefill_fp8", "mixtral_fp8",
                                  "dsv3_prefill_g8m4_shared"])
def test_full_size_config(name):
    cfg = FULL_VARIANTS.get(name) or CONFIGS[name]
    fp8 = bool(cfg.dispatch_fp8)
    print(f"\n[full {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} H={cfg.H}", flush=True)
    inp = make_inputs(cfg, DEV)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV)
    shared = (inp["w1s"], inp["w3s"], inp["w2s"]) if cfg.shared_H else None
    api.moe_layer_fwd(shape, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                      inp["w2"], buf, shared=shared)
    torch.cuda.synchronize()
    x = bf16_bits(inp["x"])
    wg = bf16_bits(inp["w_gate"])
    G, M = cfg.n_groups, cfg.group_limit
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    # routing: every token
    lg_ref = oracle.logits(x, wg, bias)
    lg = buf.logits.cpu().numpy()
    assert np.all(np.abs(lg.astype(np.float64) - lg_ref) <= logit_tolerance(
        bits_to_f64(x), bits_to_f64(wg)))
    idx = buf.topk_idx.cpu().numpy()
    w = buf.topk_w.cpu().numpy()
    o_idx, o_w, _ = oracle.topk(lg, cfg.k, G, M)
    np.testing.assert_array_equal(idx, o_idx)
    np.testing.assert_allclose(w, o_w, rtol=4e-6, atol=1e-7)
    r_idx, _, gap = oracle.topk(lg_ref, cfg.k, G, M)
    flips = np.any(idx != r_idx, axis=1)
    bad = routing_mismatch(idx, r_idx, lg_ref, gap)
    print(f"  tokens routed differently from the oracle's logits: {int(flips.sum())} "
          f"(beyond near-ties: {int(bad.sum())})", flush=True)
    assert not bad.any()
    # accounting and layout: bit-exact on the GPU's routing (send buffer sampled)
    r = oracle.dispatch(x, idx, T=cfg.T, d=cfg.d, E=cfg.E, D=cfg.D, my_rank=cfg.my_rank,
                        cf=cfg.cf, with_send_buf=False, drop_policy=cfg.drop_policy, topk_w=w,
                        fp8=fp8)
    for key in ("expert_count", "expert_kept", "expert_offset", "rank_rows", "slot"):
        np.testing.assert_array_equal(getattr(buf, key).cpu().numpy(), r[key], err_msg=key)
    st = api.stats_dict(buf.stats)
    assert st == r["stats"]
    print(f"  stats: {st}", flush=True)
    rng = np.random.default_rng(0)
    slot = r["slot"]
    for t in rng.choice(cfg.T, min(cfg.T, 64), replace=False):
        if fp8:
            q, sc = oracle.fp8_quantize_rows(x[t:t + 1])
        for s in range(cfg.k):
            if slot[t, s] < 0:
                continue
            if fp8:
                np.testing.assert_array_equal(buf.send_buf[slot[t, s]].cpu().numpy(), q[0])
                assert buf.send_scale[slot[t, s]].item() == sc[0]
            else:
                assert torch.equal(buf.send_buf[slot[t, s]].view(torch.int16),
                                   inp["x"][t].view(torch.int16))
    if r["stats"]["capacity"] > 0:
        kept = r["expert_kept"]
        C = r["stats"]["capacity"]
        for e in rng.choice(cfg.E, min(cfg.E, 8), replace=False):
            pads = buf.send_buf[e * C + kept[e]:(e + 1) * C]
            assert torch.count_nonzero(pads) == 0
    # expert FFN, stage by stage on the GPU's own hidden values: the busiest,
    # the quietest non-empty and another expert; all their rows where the
    # oracle's work stays near 10 G multiply-adds per expert, else a sample
    eo = bf16_bits(buf.expert_out)
    sb = buf.send_buf.cpu().numpy() if fp8 else bf16_bits(buf.send_buf)
    ss = buf.send_scale.cpu().numpy() if fp8 else None
    kept = r["expert_kept"]
    hb = _gpu_h(shape, buf.send_buf, buf.send_scale, buf.expert_offset, buf.expert_kept,
                inp["w1"], inp["w3"], buf.workspace)
    nz = np.nonzero(kept)[0]
    picks = [int(nz[np.argmax(kept[nz])]), int(nz[np.argmin(kept[nz])])]
    picks += [int(e) for e in rng.permutation(nz) if e not in picks][:1]
    experts = sorted(set(picks))
    max_rows = max(32, int(1e10 // (3 * cfg.d * cfg.H)))
    for e in experts:
        lo, n = int(r["expert_offset"][e]), int(kept[e])
        rows = (np.arange(lo, lo + n) if n <= max_rows else
                np.sort(rng.choice(n, max_rows, replace=False)) + lo)
        src = dict(codes=sb[rows], scales=ss[rows]) if fp8 else dict(rows=sb[rows])
        check_expert_rows(f"{name} expert {e} ({len(rows)} of {n} rows)",
                          *_expert_weights(inp, e), hb[rows], eo[rows], **src)
    del hb
    # shared expert: sampled tokens
    toks = np.sort(rng.choice(cfg.T, min(cfg.T, 256), replace=False))
    so = so_e2e = None
    if cfg.shared_H:
        hx = dict(x=x, **{n: bf16_bits(inp[n]) for n in ("w1s", "w3s", "w2s")})
        _check_shared(cfg, inp, hx, buf.shared_out, toks[:48])
        so = bf16_bits(buf.shared_out)[toks]
    # combine: sampled tokens on the GPU's expert outputs (stage parity)
    yref = oracle.combine(eo, slot[toks], w[toks], so)
    y = bf16_bits(buf.y)
    assert_bf16_close(bits_to_f64(y[toks]), bits_to_f64(yref), f"{name} combine",
                      combine_floor(bits_to_f64(eo), slot[toks], w[toks],
                                    None if so is None else bits_to_f64(so)))
    # end to end for a few tokens, every step by the oracle from x
    for t in toks[:2]:
        outs, bnds = [], []
        for s in range(cfg.k):
            e = int(idx[t, s])
            if fp8:
                q, sc = oracle.fp8_quantize_rows(x[t:t + 1])
                o, ob = oracle.expert_ffn_fp8(q, sc, *_expert_weights(inp, e), bound=True)
            else:
                o, ob = oracle.expert_ffn(x[t:t + 1], *_expert_weights(inp, e), bound=True)
            outs.append(o[0])
            bnds.append(ob[0])
        eo_t, eb_t = np.stack(outs), np.stack(bnds)
        slot_t = np.where(slot[t:t + 1] >= 0, np.arange(cfg.k)[None, :], -1).astype(np.int32)
        so_t = sb_t = None
        if cfg.shared_H:
            so_t, sb_t = oracle.expert_ffn(x[t:t + 1], hx["w1s"], hx["w3s"], hx["w2s"],
                                           bound=True)
        ref_row = oracle.combine(eo_t, slot_t, w[t:t + 1], so_t)
        assert_bf16_close(bits_to_f64(y[t:t + 1]), bits_to_f64(ref_row), f"{name} token {t}",
                          combine_floor(bits_to_f64(eo_t), slot_t, w[t:t + 1],
                                        None if so_t is None else bits_to_f64(so_t),
                                        o_dev=expert_dev(eo_t, eb_t),
                                        shared_dev=None if so_t is None else
                                        expert_dev(so_t, sb_t)))
    del inp, buf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fp8", [False, True])
def test_rank_local_expert_share(fp8):
    """The expert GEMMs on one rank's share under 8-way expert parallelism:
    8 * 4096 DeepSeek-V3-shaped tokens are routed and dispatched, and the two
    grouped GEMMs run with E/D = 32 experts on the rows of experts 0..31
    (about 1024 each, several full 256-row tiles).  Rows of at least three
    distinct experts match the oracle stage by stage; rows of other experts
    are left untouched.  With E4M3 rows the share ends well before the send
    buffer does, and the gate/up GEMM's widened path (a workspace holding a
    non-zero pattern) gives the register path's bits on every kept row."""
    base = CONFIGS["dsv3_prefill"].with_(dispatch_fp8=int(fp8))
    cfg = base.with_(T=base.T * base.D)
    print(f"\n[rank-local] fp8={fp8} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} H={cfg.H}",
          flush=True)
    inp = make_inputs(cfg, DEV, experts=False)
    el = cfg.E // cfg.D
    w = make_inputs(base.with_(E=el, T=1), DEV)  # weights of experts 0..31
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, DEV, keep_logits=False)
    api.moe_route(shape, inp["x"], inp["w_gate"], None, None, buf.topk_idx, buf.topk_w,
                  buf.workspace)
    _run_dispatch(shape, inp["x"], buf.topk_idx, buf)
    torch.cuda.synchronize()
    kept = buf.expert_kept.cpu().numpy()
    off = buf.expert_offset.cpu().numpy()
    rows = int(off[el])
    assert rows == int(kept[:el].sum()) and kept[:el].max() > 256
    loc = api.Shape(cfg.T, cfg.d, el, cfg.k, cfg.H, 1, 0, INF, dispatch_fp8=int(fp8))
    h = torch.empty(buf.send_buf.shape[0], cfg.H, dtype=torch.bfloat16, device=DEV)
    out = torch.full(buf.send_buf.shape, 0x1234, dtype=torch.int16, device=DEV)
    ws = None
    if fp8:
        _, _, ws_bytes = api.moe_query(loc)
        ws = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device=DEV)
    api.moe_expert_gate_up(loc, buf.send_buf, buf.send_scale, buf.expert_offset, buf.expert_kept,
                           w["w1"], w["w3"], h, workspace=ws)
    if fp8:
        hr = torch.empty_like(h)
        api.moe_expert_gate_up(loc, buf.send_buf, buf.send_scale, buf.expert_offset,
                               buf.expert_kept, w["w1"], w["w3"], hr)
    api.moe_expert_down(loc, h, buf.expert_offset, buf.expert_kept, w["w2"],
                        out.view(torch.bfloat16))
    torch.cuda.synchronize()
    if fp8:
        assert rows < buf.send_buf.shape[0] // 2
        assert torch.equal(h[:rows].view(torch.int16), hr[:rows].view(torch.int16))
        del hr
    tail = out[rows:rows + 4096]
    assert torch.all(tail == 0x1234), "rows past the share were written"
    rng = np.random.default_rng(1)
    sb = buf.send_buf[:rows].cpu().numpy() if fp8 else bf16_bits(buf.send_buf[:rows])
    ss = buf.send_scale[:rows].cpu().numpy() if fp8 else None
    eo = bf16_bits(out[:rows].view(torch.bfloat16))
    hb = bf16_bits(h[:rows])
    picks = [int(np.argmax(kept[:el])), int(np.argmin(kept[:el]))]
    picks += [int(e) for e in rng.permutation(el) if e not in picks][:2]
    assert len(set(picks)) >= 3
    for e in sorted(set(picks)):
        lo, n = int(off[e]), int(kept[e])
        r = np.sort(rng.choice(n, min(n, 48), replace=False)) + lo
        src = dict(codes=sb[r], scales=ss[r]) if fp8 else dict(rows=sb[r])
        check_expert_rows(f"rank-local expert {e}", *_expert_weights(w, e), hb[r], eo[r], **src)
    del inp, w, buf, h, out, ws
    torch.cuda.empty_cache()
