"""Backward of the scan (ssm_scan_bwd) vs the fp64 oracle's gradients, through
the C ABI (needs an MI355X).

Bar per output tensor: max|got - want| <= tol * max|want|, with tol 1e-4 for
fp32 outputs (dA, dB, dC, dD, ddelta_bias, dh0, and du/ddelta/dz with fp32
io) and 2e-2 for the bf16 outputs (du, ddelta, dz with bf16 io, rounded to
bf16 like y).  The oracle runs on the identical (bf16-rounded) inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
IO_TOL = {"f32": 1e-4, "bf16": 2e-2}
F32_TOL = 1e-4


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def check(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    scale = float(np.max(np.abs(want)))
    err = float(np.max(np.abs(got - want)))
    assert err <= tol * scale + 1e-30, "%s: max err %.3e > %.1e * %.3e" % (what, err, tol, scale)


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def grads_inputs(x, seed, with_dlast=True):
    rng = np.random.default_rng([seed, 11])
    dy = rng.standard_normal(x.u.shape).astype(np.float32)
    if x.io == "bf16":
        dy = inputs.round_bf16(dy)
    dlast = rng.standard_normal((x.shape[0], x.shape[1], x.shape[2])).astype(np.float32) if with_dlast else None
    return dy, dlast


def gpu_bwd(x, dy, dlast):
    t = inputs.to_torch(x, DEV)
    dyt = torch.from_numpy(dy).to(DEV, t["u"].dtype)
    dlt = None if dlast is None else torch.from_numpy(dlast).to(DEV)
    g = binding.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dyt, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=x.softplus, h0=t["h0"], dlast=dlt)
    torch.cuda.synchronize()
    return g


def oracle_bwd(x, dy, dlast):
    return oracle.scan_bwd_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0, dy=dy,
                               dlast=dlast)


def compare(g, r, io, x, what):
    for k in ("du", "ddelta", "dz"):
        if r.get(k) is not None and g.get(k) is not None:
            check(np64(g[k]), r[k], IO_TOL[io], "%s %s" % (what, k))
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        if g.get(k) is not None and r.get(k) is not None:
            check(np64(g[k]), r[k], F32_TOL, "%s %s" % (what, k))


# (2, 70, 16, 200): 25 steps of 8 tokens, so the kernel's per-line groups of
# held stores (8 steps of bf16, 4 of fp32) end in a one-step group, over a
# dim whose second channel group is mostly idle lanes.
SHAPES = [(192, 64, 16, 64), (200, 64, 8, 24), (256, 33, 4, 16), (2, 8, 16, 40), (3, 130, 16, 8), (2, 70, 16, 200)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%dx%dx%d" % s for s in SHAPES])
def test_bwd_matches_oracle(io, shape):
    b, d, n, l = shape
    for mask in (31, 0, 21, 10):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=1000 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        if not sp:
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        dy, dlast = grads_inputs(x, 1000 + mask, with_dlast=(mask % 2 == 1))
        say("bwd shape=%s io=%s mask=%d" % (shape, io, mask))
        g = gpu_bwd(x, dy, dlast)
        r = oracle_bwd(x, dy, dlast)
        compare(g, r, io, x, "mask=%d" % mask)


# 5 and 6 channel groups of 64: the reduce kernel's lanes then sum unequal
# numbers of groups (lane q takes groups q, q + 4, ...), which dB and dC see.
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 320, 16, 32), (1, 384, 16, 48)], ids=["2x320x16x32", "1x384x16x48"])
def test_bwd_group_counts_dB_dC(io, shape):
    b, d, n, l = shape
    for mask in (31, 6):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=1200 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        if not sp:
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        dy, dlast = grads_inputs(x, 1200 + mask)
        say("bwd group counts shape=%s io=%s mask=%d" % (shape, io, mask))
        g = gpu_bwd(x, dy, dlast)
        r = oracle_bwd(x, dy, dlast)
        compare(g, r, io, x, "groups mask=%d" % mask)
        for k in ("dB", "dC"):
            assert g[k] is not None and r[k] is not None, k


def test_bwd_mamba130m_layer_full():
    x = inputs.scan_config(1)
    dy, dlast = grads_inputs(x, 1001)
    say("bwd Mamba-130M layer (8x1536x16x2048 fp32), every gradient against the full oracle")
    g = gpu_bwd(x, dy, dlast)
    r = oracle_bwd(x, dy, dlast)
    compare(g, r, "f32", x, "130M")


def test_bwd_mamba1p4b_layer_sampled():
    """Full Mamba-1.4B-layer backward; the per-channel gradients (du, ddelta,
    dz, dh0) and the per-channel sums (dA, dD, ddelta_bias) are checked on
    sampled channels, each an exact oracle problem of its own (batch rows of
    one channel); dB and dC sum over all channels and are covered by the
    full 130M-layer test."""
    x = inputs.scan_config(2)
    dy, dlast = grads_inputs(x, 1002)
    say("bwd Mamba-1.4B layer (4x4096x16x4096 bf16), sampled channels")
    g = gpu_bwd(x, dy, dlast)
    bsz, dim, n, l = x.shape
    for d in (0, 1, 777, 2048, 4095):
        sl = lambda a: None if a is None else a[:, d:d + 1]
        r = oracle.scan_bwd_f64(sl(x.u), sl(x.delta), x.A[d:d + 1], x.B, x.C, x.D[d:d + 1], sl(x.z),
                                x.delta_bias[d:d + 1], x.softplus, sl(x.h0), dy=sl(dy), dlast=sl(dlast))
        for k in ("du", "ddelta", "dz"):
            check(np64(g[k][:, d:d + 1]), r[k], IO_TOL["bf16"], "channel %d %s" % (d, k))
        check(np64(g["dh0"][:, d:d + 1]), r["dh0"], F32_TOL, "channel %d dh0" % d)
        check(np64(g["dA"][d:d + 1]), r["dA"], F32_TOL, "channel %d dA" % d)
        check(np64(g["dD"][d:d + 1]), r["dD"], F32_TOL, "channel %d dD" % d)
        check(np64(g["ddelta_bias"][d:d + 1]), r["ddelta_bias"], F32_TOL, "channel %d dbias" % d)


def test_bwd_deterministic_and_unsupported():
    x = inputs.make_scan_inputs(192, 64, 16, 48, io="bf16", seed=1100, h0=True)
    dy, dlast = grads_inputs(x, 1100)
    say("bwd determinism")
    g1 = gpu_bwd(x, dy, dlast)
    g2 = gpu_bwd(x, dy, dlast)
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k
    for shape in ((2, 8, 5, 16), (2, 8, 16, 20)):
        y = inputs.make_scan_inputs(*shape, io="f32", seed=1101)
        dy2, _ = grads_inputs(y, 1101, with_dlast=False)
        with pytest.raises(binding.SsmError) as e:
            gpu_bwd(y, dy2, None)
        assert e.value.name == "SSM_ERR_UNSUPPORTED"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_saved_checkpoints_match_recompute(io):
    """scan_fwd_save + scan_bwd_saved equal scan_fwd + scan_bwd bit for bit (single-pass shapes), on a split
    shape and on one that scan_fwd runs segmented (y then matches to the usual bar)."""
    for shape in ((192, 64, 16, 64), (1, 64, 8, 2048)):
        b, d, n, l = shape
        say("saved checkpoints shape=%s io=%s" % (shape, io))
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=1700, h0=True)
        dy, dlast = grads_inputs(x, 1700)
        t = inputs.to_torch(x, DEV)
        dyt = torch.from_numpy(dy).to(DEV, t["u"].dtype)
        dlt = torch.from_numpy(dlast).to(DEV)
        y1, h1, ck = binding.scan_fwd_save(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                           delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])
        y2, h2 = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])
        g1 = binding.scan_bwd_saved(t["u"], t["delta"], t["A"], t["B"], t["C"], dyt, ck, D=t["D"], z=t["z"],
                                    delta_bias=t["delta_bias"], delta_softplus=True, dlast=dlt)
        g2 = binding.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dyt, D=t["D"], z=t["z"],
                              delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], dlast=dlt)
        torch.cuda.synchronize()
        split = binding.scan_plan(b, d, n, l, t["u"].dtype, with_path=True)[0] == "split"
        if split:
            assert torch.equal(y1, y2) and torch.equal(h1, h2)
        else:
            check(np64(y1), np64(y2), IO_TOL[io], "y (segmented scan_fwd)")
            check(np64(h1), np64(h2), F32_TOL, "last_state (segmented scan_fwd)")
        for k in g2:
            if g2[k] is not None:
                assert torch.equal(g1[k], g2[k]), k


ZOH_SHAPES = [(192, 64, 16, 64), (256, 33, 4, 16), (2, 8, 16, 40), (3, 130, 8, 24), (3, 130, 16, 8)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ZOH_SHAPES, ids=["%dx%dx%dx%d" % s for s in ZOH_SHAPES])
def test_bwd_zoh_matches_oracle(io, shape):
    """Gradients under exact zero-order hold (ssm_scan_bwd_ex), with A holding a zero and a tiny entry."""
    b, d, n, l = shape
    for mask in (31, 10):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=1800 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        x.A = x.A.copy()
        x.A[::5, 0] = 0.0
        x.A[1::5, n - 1] = -1e-6
        if not sp:
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        dy, dlast = grads_inputs(x, 1800 + mask)
        say("bwd zoh shape=%s io=%s mask=%d" % (shape, io, mask))
        t = inputs.to_torch(x, DEV)
        g = binding.scan_bwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                torch.from_numpy(dy).to(DEV, t["u"].dtype), D=t["D"], z=t["z"],
                                delta_bias=t["delta_bias"], delta_softplus=sp, h0=t["h0"],
                                dlast=torch.from_numpy(dlast).to(DEV), disc="zoh")
        torch.cuda.synchronize()
        r = oracle.scan_bwd_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0, dy=dy,
                                dlast=dlast, zoh=True)
        compare(g, r, io, x, "zoh mask=%d" % mask)


def test_bwd_zoh_mamba1p4b_layer_sampled():
    """Full Mamba-1.4B-layer backward under exact zero-order hold; the per-channel gradients and
    sums checked on sampled channels against the oracle's ZOH backward of those channels."""
    x = inputs.scan_config(2)
    dy, dlast = grads_inputs(x, 1003)
    say("bwd zoh Mamba-1.4B layer (4x4096x16x4096 bf16), sampled channels")
    t = inputs.to_torch(x, DEV)
    g = binding.scan_bwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], torch.from_numpy(dy).to(DEV, t["u"].dtype),
                            D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=t["h0"],
                            dlast=torch.from_numpy(dlast).to(DEV), disc="zoh")
    torch.cuda.synchronize()
    for d in (0, 1500, 4095):
        sl = lambda a: None if a is None else a[:, d:d + 1]
        r = oracle.scan_bwd_f64(sl(x.u), sl(x.delta), x.A[d:d + 1], x.B, x.C, x.D[d:d + 1], sl(x.z),
                                x.delta_bias[d:d + 1], x.softplus, sl(x.h0), dy=sl(dy), dlast=sl(dlast), zoh=True)
        for k in ("du", "ddelta", "dz"):
            check(np64(g[k][:, d:d + 1]), r[k], IO_TOL["bf16"], "channel %d %s" % (d, k))
        check(np64(g["dh0"][:, d:d + 1]), r["dh0"], F32_TOL, "channel %d dh0" % d)
        check(np64(g["dA"][d:d + 1]), r["dA"], F32_TOL, "channel %d dA" % d)
        check(np64(g["dD"][d:d + 1]), r["dD"], F32_TOL, "channel %d dD" % d)
        check(np64(g["ddelta_bias"][d:d + 1]), r["ddelta_bias"], F32_TOL, "channel %d dbias" % d)


def test_bwd_ex_delta_b_is_scan_bwd_bitwise():
    x = inputs.make_scan_inputs(192, 64, 16, 64, io="bf16", seed=1900, h0=True)
    dy, dlast = grads_inputs(x, 1900)
    t = inputs.to_torch(x, DEV)
    dyt = torch.from_numpy(dy).to(DEV, t["u"].dtype)
    dlt = torch.from_numpy(dlast).to(DEV)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], dlast=dlt)
    g1 = binding.scan_bwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], dyt, disc="delta_b", **kw)
    g2 = binding.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dyt, **kw)
    torch.cuda.synchronize()
    for k in g2:
        if g2[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
