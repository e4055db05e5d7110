"""The chunked prefill kernel (lanes along the sequence, a DPP lane scan of
the chunks' affine maps, a running carry across tiles) against the fp64
oracle, through the C ABI.

Shapes are chosen around the kernel's geometry: 16 tokens per lane, 1024
per tile, seqlen a multiple of 8 (so a lane's last chunk may be half past the
end), 8 to 12 channels per block (ragged last blocks), one or more batch rows.
Bar as everywhere: max|got - want| <= tol * max|want|, tol 1e-4 (fp32 io) or
2e-2 (bf16 io) for y, 1e-4 for the fp32 last_state.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def check(got, want, io, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    scale = float(np.max(np.abs(want)))
    err = float(np.max(np.abs(got - want)))
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    assert err <= TOL[io] * scale + 1e-30, "%s: max err %.3e > %.1e * %.3e" % (what, err, TOL[io], scale)
    return err / max(scale, 1e-30)


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run(x, **kw):
    t = inputs.to_torch(x, DEV)
    y, last = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=t["h0"], **kw)
    torch.cuda.synchronize()
    return y, last


# (batch, dim, seqlen): 8 tokens (lane 0 half full), 24 (lane 1 half full),
# one tile + 8, one tile + 520 (a lane half full mid-tile), two batch rows of
# a dim no block size divides, three whole tiles, 12 channels (a block of 8
# and one of 4 live waves), two rows of 1300 channels (blocks of 11, the
# last of each row 2 wide).
SHAPES = [(1, 40, 8), (1, 40, 24), (1, 100, 1032), (1, 23, 1544), (2, 37, 2064), (1, 130, 3072), (1, 12, 4096),
          (2, 1300, 1040)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%dx%d" % s for s in SHAPES])
def test_chunked_shapes(io, shape):
    b, d, l = shape
    dt = torch.float32 if io == "f32" else torch.bfloat16
    assert binding.scan_plan(b, d, 16, l, dt, with_path=True)[0] == "chunked"
    x = inputs.make_scan_inputs(b, d, 16, l, io=io, seed=5100 + l, h0=True)
    say("chunked shape=%s io=%s" % (shape, io))
    y, last = run(x)
    yr, hr = oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    check(np64(y), yr, io, "y")
    check(np64(last), hr, "f32", "last_state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_flags(io):
    """Every combination of z, D, bias, softplus and h0 (all optional)."""
    b, d, l = 1, 24, 2056
    for mask in range(32):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, 16, l, io=io, seed=5200 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        if not sp:
            # Without softplus the step is delta + bias as given; keep it
            # positive so the test system stays stable (|Abar| <= 1).
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        say("chunked flags z=%d D=%d bias=%d softplus=%d h0=%d io=%s" % (z, D, bias, sp, h0, io))
        y, last = run(x)
        yr, hr = oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
        check(np64(y), yr, io, "y mask=%d" % mask)
        check(np64(last), hr, "f32", "last_state mask=%d" % mask)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_block_sizes(io):
    """Channel counts that give each block size from 8 to 12 waves (256
    blocks of 8, 9, 10, 11 and 12 channels), over two tiles, the second 24
    tokens long."""
    seen = set()
    for dim in (2048, 2304, 2560, 2816, 3072):
        x = inputs.make_scan_inputs(1, dim, 16, 1048, io=io, seed=5300 + dim, h0=True)
        say("chunked block sizes dim=%d io=%s" % (dim, io))
        y, last = run(x)
        ch = [(0, c) for c in sorted(set(np.linspace(0, dim - 1, 12).astype(int).tolist()))]
        yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
        di = torch.tensor([c[1] for c in ch], device=DEV)
        check(np64(y[0, di]), yr, io, "y dim=%d" % dim)
        check(np64(last[0, di]), hr, "f32", "last_state dim=%d" % dim)
        seen.add(dim)
    assert len(seen) == 5


def test_chunked_deterministic():
    x = inputs.make_scan_inputs(1, 64, 16, 8192, io="f32", seed=5400, h0=True)
    say("chunked determinism")
    y1, h1 = run(x)
    y2, h2 = run(x)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_chunked_carry_across_calls():
    """Four calls carrying last_state equal one call (the long-sequence
    workload's split-and-carry property, at a smaller size)."""
    b, d, l = 1, 48, 8192
    x = inputs.make_scan_inputs(b, d, 16, l, io="f32", seed=5500, h0=True)
    say("chunked carry across calls")
    t = inputs.to_torch(x, DEV)
    y_full, h_full = run(x)
    state = t["h0"].clone()
    parts = []
    for k in range(4):
        s = slice(k * l // 4, (k + 1) * l // 4)
        y, _ = binding.scan_fwd(t["u"][..., s].contiguous(), t["delta"][..., s].contiguous(), t["A"],
                                t["B"][..., s].contiguous(), t["C"][..., s].contiguous(), D=t["D"],
                                z=t["z"][..., s].contiguous(), delta_bias=t["delta_bias"], delta_softplus=True,
                                h0=state, last_state=state)
        parts.append(y)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    check(np64(torch.cat(parts, -1)), yr, "f32", "y over four calls")
    check(np64(state), hr, "f32", "carried state")
    check(np64(y_full), yr, "f32", "y in one call")


def test_chunked_nonfinite_propagates():
    """An Inf in one token's u reaches that channel's outputs from that token
    on and no other channel."""
    b, d, l = 1, 20, 2048
    x = inputs.make_scan_inputs(b, d, 16, l, io="f32", seed=5600, h0=False)
    x.u = x.u.copy()
    x.u[0, 7, 1500] = np.inf
    say("chunked inf propagation")
    y, _ = run(x)
    yy = y.cpu().numpy()
    assert np.isfinite(yy[0, 7, :1500]).all()
    assert not np.isfinite(yy[0, 7, 1500]).all()
    others = np.delete(yy[0], 7, axis=0)
    assert np.isfinite(others).all()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_split_channels_every_channel(io):
    """2560 channels run in blocks of 10 channels on 12 waves: channels 8 and 9
    of every block are split by state between two waves, which hand y over
    through LDS and each store their own final states.  Every channel of every
    block against the oracle, over a partial last tile, with an initial state."""
    b, d, l = 1, 2560, 1048
    x = inputs.make_scan_inputs(b, d, 16, l, io=io, seed=5700, h0=True)
    say("chunked split channels, every channel, io=%s" % io)
    y, last = run(x)
    yr, hr = oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    check(np64(y), yr, io, "y")
    check(np64(last), hr, "f32", "last_state")
