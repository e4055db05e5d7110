"""Causal depthwise conv fused in front of the scan (ssm_conv_scan_fwd) vs the
fp64 oracle, through the C ABI (needs an MI355X).

The reference is oracle.conv1d_f64 followed by oracle.scan_f64 on that u
rounded to the io dtype (the kernel rounds the conv output exactly as a stored
u would be).  y is held to the scan's bar (1e-4 of max|y| for fp32 io, 2e-2
for bf16); u_out to the rounding of one io element.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}
U_TOL = {"f32": 2e-6, "bf16": 2.0 ** -8}


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


def conv_inputs(b, d, n, l, io, width, seed, with_prev=True, with_bias=True, **kw):
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=seed, **kw)
    rng = np.random.default_rng([seed, 7])
    w = (0.5 * rng.standard_normal((d, width))).astype(np.float32)
    cb = (0.1 * rng.standard_normal(d)).astype(np.float32) if with_bias else None
    prev = rng.standard_normal((b, d, width - 1)).astype(np.float32) if with_prev and width > 1 else None
    if io == "bf16" and prev is not None:
        prev = inputs.round_bf16(prev)
    return x, w, cb, prev


def io_round(a, io):
    a = np.asarray(a, np.float64).astype(np.float32)
    return inputs.round_bf16(a) if io == "bf16" else a


def run(x, w, cb, prev, silu, u_out=True, out=None, uo=None, h0=None):
    t = inputs.to_torch(x, DEV)
    dt = t["u"].dtype
    wt = torch.from_numpy(w).to(DEV)
    cbt = None if cb is None else torch.from_numpy(cb).to(DEV)
    pt = None if prev is None else torch.from_numpy(prev).to(DEV, dt)
    if uo is None and u_out:
        uo = torch.empty_like(t["u"])
    y, last = binding.conv_scan_fwd(t["u"], wt, t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                    delta_bias=t["delta_bias"], delta_softplus=x.softplus, conv_bias=cbt, x_prev=pt,
                                    conv_silu=silu, h0=t["h0"] if h0 is None else h0, out=out, u_out=uo)
    torch.cuda.synchronize()
    return y, last, uo, t


def reference(x, w, cb, prev, silu, io):
    u64 = oracle.conv1d_f64(x.u, w, cb, prev, silu=silu)
    yr, hr = oracle.scan_f64(io_round(u64, io), x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    return u64, yr, hr


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


FUSED_SHAPES = [(192, 64, 16, 72), (200, 64, 8, 24), (256, 33, 4, 16)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=["%dx%dx%dx%d" % s for s in FUSED_SHAPES])
def test_fused_path(io, shape):
    b, d, n, l = shape
    path = binding.scan_plan(b, d, n, l, torch.float32 if io == "f32" else torch.bfloat16, with_path=True)[0]
    assert path == "split"
    for width in (1, 2, 3, 4):
        for silu, with_prev, with_bias in ((True, True, True), (False, False, False), (True, False, True)):
            say("conv fused shape=%s io=%s K=%d silu=%s prev=%s" % (shape, io, width, silu, with_prev))
            x, w, cb, prev = conv_inputs(b, d, n, l, io, width, 500 + width, with_prev, with_bias, h0=True)
            y, last, uo, _ = run(x, w, cb, prev, silu)
            u64, yr, hr = reference(x, w, cb, prev, silu, io)
            check(np64(uo), u64, U_TOL[io], "u_out K=%d" % width)
            check(np64(y), yr, TOL[io], "y K=%d silu=%s prev=%s" % (width, silu, with_prev))
            check(np64(last), hr, TOL["f32"], "last_state K=%d" % width)


# Shapes off the single-pass kernel: the conv is fused into the chunked,
# segmented and per-token kernels too (history carried across lanes, tiles,
# lines and segments).  Chunked: 1x64x16x4096, 1x40x16x24 (lane 1 half past
# the end), 2x37x16x2064 (three tiles, the last partial; ragged blocks),
# 1x2560x16x1048 (channels split by state).
OTHER_SHAPES = [(1, 16, 4, 64), (2, 63, 16, 63), (1, 3, 16, 7), (1, 64, 16, 4097), (1, 64, 16, 4096),
                (2, 100, 8, 1536), (1, 40, 16, 24), (2, 37, 16, 2064), (1, 2560, 16, 1048)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", OTHER_SHAPES, ids=["%dx%dx%dx%d" % s for s in OTHER_SHAPES])
def test_other_paths(io, shape):
    b, d, n, l = shape
    for width in (2, 4):
        say("conv other path shape=%s io=%s K=%d plan=%s" % (shape, io, width, binding.scan_plan(
            b, d, n, l, torch.float32 if io == "f32" else torch.bfloat16, with_path=True)))
        x, w, cb, prev = conv_inputs(b, d, n, l, io, width, 600 + width, h0=True)
        for u_out in (True, False):
            y, last, uo, _ = run(x, w, cb, prev, True, u_out=u_out)
            u64, yr, hr = reference(x, w, cb, prev, True, io)
            if u_out:
                check(np64(uo), u64, U_TOL[io], "u_out K=%d" % width)
            check(np64(y), yr, TOL[io], "y K=%d u_out=%s" % (width, u_out))
            check(np64(last), hr, TOL["f32"], "last_state K=%d" % width)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n", [16, 8])
def test_long_rows_with_conv(io, n):
    """1 x 2560 x 32768 with the conv in front.  dstate 16 runs the chunked
    kernel (32 tiles, two channels of each block split by state); dstate 8 a
    segmented plan whose aggregate launch runs each segment in two pieces (52
    segments of 640 tokens), each piece starting its conv from the four
    inputs before it.  Checked on sampled channels."""
    b, d, l = 1, 2560, 32768
    dt = torch.float32 if io == "f32" else torch.bfloat16
    want = ("chunked", 1, l, 0) if n == 16 else ("segmented", 52, 640, 0)
    assert binding.scan_plan(b, d, n, l, dt, with_path=True, conv_width=4) == want
    say("conv on long rows io=%s n=%d path=%s" % (io, n, want[0]))
    x, w, cb, prev = conv_inputs(b, d, n, l, io, 4, 700, h0=True)
    y, last, uo, _ = run(x, w, cb, prev, True)
    ch = inputs.sample_channels(b, d, 6, seed=5) + [(0, 8), (0, 2559)]   # two split channels of the chunked plan
    di = [c[1] for c in ch]
    u64 = oracle.conv1d_f64(x.u[:, di], w[di], None if cb is None else cb[di], None if prev is None else prev[:, di],
                            silu=True)
    ur = io_round(u64, io)
    sub = lambda a: None if a is None else a[:, di]
    yr, hr = oracle.scan_f64(ur, sub(x.delta), x.A[di], x.B, x.C, None if x.D is None else x.D[di], sub(x.z),
                             None if x.delta_bias is None else x.delta_bias[di], x.softplus, sub(x.h0))
    dti = torch.tensor(di, device=DEV)
    check(np64(uo[:, dti]), u64, U_TOL[io], "u_out")
    check(np64(y[:, dti]), yr, TOL[io], "y")
    check(np64(last[:, dti]), hr, TOL["f32"], "last_state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(192, 64, 16, 96), (1, 64, 16, 2056)], ids=["split", "chunked"])
def test_fused_equals_conv_then_scan(io, shape):
    """The fused kernel's y is bitwise the plain scan of the u it reports, and
    that u is bitwise the per-token kernel's conv (a misaligned u_out sends the
    call there; its scan then differs in summation order, so y is held to the
    usual bar)."""
    b, d, n, l = shape
    x, w, cb, prev = conv_inputs(b, d, n, l, io, 4, 700, h0=True)
    say("conv fused vs conv+scan io=%s shape=%s" % (io, shape))
    y, last, uo, t = run(x, w, cb, prev, True)
    y2, last2 = binding.scan_fwd(uo, t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                 delta_softplus=True, h0=t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(last, last2)
    es = 2 if io == "bf16" else 4
    big = torch.empty(b * d * l + 8, dtype=uo.dtype, device=DEV)
    uo_mis = big[1:1 + b * d * l].view(b, d, l)      # element-aligned, not 16-byte aligned
    assert uo_mis.data_ptr() % 16 == es
    y3, last3, _, _ = run(x, w, cb, prev, True, uo=uo_mis)
    assert torch.equal(uo_mis, uo)
    check(np64(y3), np64(y), TOL[io], "y via the per-token kernel")
    check(np64(last3), np64(last), TOL["f32"], "last_state via the per-token kernel")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(192, 64, 16, 160, 72), (1, 48, 16, 3072, 1040)], ids=["split", "chunked"])
def test_conv_carry_across_calls(io, shape):
    """Two calls, the second fed the first's last K-1 inputs and final state,
    equal one call over the whole sequence."""
    b, d, n, l, cut = shape
    x, w, cb, prev = conv_inputs(b, d, n, l, io, 4, 800, h0=True)
    say("conv carry io=%s" % io)
    y, last, uo, t = run(x, w, cb, prev, True)
    wt = torch.from_numpy(w).to(DEV)
    cbt = torch.from_numpy(cb).to(DEV)
    pt = torch.from_numpy(prev).to(DEV, t["u"].dtype)
    kw = dict(D=t["D"], delta_bias=t["delta_bias"], delta_softplus=True, conv_bias=cbt, conv_silu=True)
    sl = lambda v, a_, b_: v[..., a_:b_].contiguous()
    y1, h1 = binding.conv_scan_fwd(sl(t["u"], 0, cut), wt, sl(t["delta"], 0, cut), t["A"], sl(t["B"], 0, cut),
                                   sl(t["C"], 0, cut), z=sl(t["z"], 0, cut), x_prev=pt, h0=t["h0"], **kw)
    y2, h2 = binding.conv_scan_fwd(sl(t["u"], cut, l), wt, sl(t["delta"], cut, l), t["A"], sl(t["B"], cut, l),
                                   sl(t["C"], cut, l), z=sl(t["z"], cut, l), x_prev=sl(t["u"], cut - 3, cut), h0=h1,
                                   **kw)
    torch.cuda.synchronize()
    check(np64(torch.cat([y1, y2], dim=-1)), np64(y), 1e-6, "carried y")
    check(np64(h2), np64(last), 1e-6, "carried state")


# (shape, (batch, channel, token) of the Inf): the single-pass kernel; the
# chunked kernel with the Inf two tokens before a lane boundary (its taps
# reach the next lane's first outputs) and two before a tile boundary.
NONFINITE = [((192, 64, 16, 48), (3, 5, 17)), ((1, 40, 16, 2048), (0, 7, 30)), ((1, 40, 16, 2048), (0, 9, 1022))]


@pytest.mark.parametrize("shape,at", NONFINITE, ids=["split", "chunked-lane", "chunked-tile"])
def test_conv_nonfinite_reaches_exactly_k_outputs(shape, at):
    b, d, n, l = shape
    bi, di, li = at
    for width in (1, 2, 4):
        x, w, cb, prev = conv_inputs(b, d, n, l, "f32", width, 900 + width, h0=True)
        x.u = x.u.copy()
        x.u[bi, di, li] = np.inf
        say("conv inf K=%d shape=%s at=%s" % (width, shape, at))
        _, _, uo, _ = run(x, w, cb, prev, False)
        bad = ~torch.isfinite(uo.cpu())
        want = torch.zeros_like(bad)
        want[bi, di, li:li + width] = True
        assert torch.equal(bad, want), "K=%d non-finite at %s" % (width, torch.nonzero(bad).tolist()[:8])
