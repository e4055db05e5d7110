"""Backward of the causal depthwise conv (ssm_conv_bwd) vs the fp64 oracle,
through the C ABI (needs an MI355X).

x, du and x_prev are drawn, rounded to the io dtype and handed to both sides
as the same values, so the only differences are the kernel's fp32 arithmetic
and, for bf16 io, the rounding of dx and dx_prev to bf16.  dx and dx_prev are
held to 1e-4 of their largest magnitude for fp32 io and 2e-2 for bf16 (one
bf16 rounding is 2^-8 relative); dconv_weight and dconv_bias are fp32 sums
over every (batch, token) and are held to 1e-4 of their largest magnitude
for both io dtypes.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
IO_TOL = {"f32": 1e-4, "bf16": 2e-2}
SUM_TOL = 1e-4
SILU_SLOPE_MAX = 1.0998  # max over v of |d silu(v) / dv|


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def check(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= tol * scale + 1e-30, "%s: max err %.3e > %.1e * %.3e" % (what, err, tol, scale)


def io_round(a, io):
    a = np.asarray(a, np.float32)
    return inputs.round_bf16(a) if io == "bf16" else a


def draw(batch, dim, seqlen, width, io, seed, with_prev=True, with_bias=True):
    rng = np.random.default_rng([seed, batch, dim, seqlen, width])
    w, cb = inputs.conv_params(dim, width, seed=seed)
    x = io_round(rng.standard_normal((batch, dim, seqlen)), io)
    du = io_round(rng.standard_normal((batch, dim, seqlen)), io)
    prev = io_round(rng.standard_normal((batch, dim, width - 1)), io) if with_prev and width > 1 else None
    return x, w, (cb if with_bias else None), prev, du


def to_dev(a, io):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, torch.bfloat16 if io == "bf16" else torch.float32)


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run(x, w, cb, prev, du, silu, io):
    g = binding.conv_bwd(to_dev(x, io), torch.from_numpy(w).to(DEV), to_dev(du, io),
                         conv_bias=None if cb is None else torch.from_numpy(cb).to(DEV), x_prev=to_dev(prev, io),
                         conv_silu=silu)
    torch.cuda.synchronize()
    return g


def compare(g, want, io, what):
    check(np64(g["dx"]), want["dx"], IO_TOL[io], what + " dx")
    check(np64(g["dconv_weight"]), want["dweight"], SUM_TOL, what + " dconv_weight")
    check(np64(g["dconv_bias"]), want["dbias"], SUM_TOL, what + " dconv_bias")
    check(np64(g["dx_prev"]), want["dx_prev"], IO_TOL[io], what + " dx_prev")


# (batch, dim, seqlen): one token; part of one item; ragged tails past one
# and two items (items of 2048 tokens, 8 per thread, for rows read element by
# element and for 5000; 4096 tokens, 16 per thread, for 4096 and 8000); one
# whole item; a dim that is not a multiple of 64.
SHAPES = [(1, 1, 1), (2, 33, 17), (2, 64, 2051), (1, 5, 5000), (2, 3, 8000), (2, 3, 4096), (3, 70, 300)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("width", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", SHAPES)
def test_conv_bwd_parity(shape, width, io):
    b, d, l = shape
    say("conv_bwd %s K=%d io=%s" % (shape, width, io))
    x, w, cb, prev, du = draw(b, d, l, width, io, seed=65100)
    g = run(x, w, cb, prev, du, True, io)
    want = oracle.conv1d_bwd_f64(x, w, du, cb, prev, silu=True)
    compare(g, want, io, "%s K=%d %s" % (shape, width, io))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("with_prev,with_bias,silu", [(False, False, True), (False, True, False),
                                                      (True, False, False), (True, True, False)])
def test_conv_bwd_options(with_prev, with_bias, silu, io):
    b, d, l, width = 2, 40, 2300, 4
    say("conv_bwd options prev=%s bias=%s silu=%s io=%s" % (with_prev, with_bias, silu, io))
    x, w, cb, prev, du = draw(b, d, l, width, io, seed=65101, with_prev=with_prev, with_bias=with_bias)
    g = run(x, w, cb, prev, du, silu, io)
    want = oracle.conv1d_bwd_f64(x, w, du, cb, prev, silu=silu)
    compare(g, want, io, "options")


def test_conv_bwd_short_rows_use_x_prev():
    """seqlen below K - 1: the taps of every token reach into x_prev, and dx_prev
    slots past the last token take nothing from the next chunk."""
    x, w, cb, prev, du = draw(2, 9, 2, 4, "f32", seed=65102)
    g = run(x, w, cb, prev, du, True, "f32")
    compare(g, oracle.conv1d_bwd_f64(x, w, du, cb, prev, silu=True), "f32", "seqlen 2")


def test_conv_bwd_deterministic():
    """Two calls on the same inputs give the same bits (fixed-order sums)."""
    x, w, cb, prev, du = draw(2, 64, 6000, 4, "bf16", seed=65103)
    g1 = run(x, w, cb, prev, du, True, "bf16")
    g2 = run(x, w, cb, prev, du, True, "bf16")
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_conv_bwd_mamba1p4b_layer():
    """The Mamba-1.4B layer (batch 4, dim 4096, seqlen 4096, K = 4, bf16 io), every output."""
    x = inputs.scan_config(2)
    batch, dim, _, _ = x.shape
    w, cb = inputs.conv_params(dim, 4)
    rng = np.random.default_rng(65104)
    prev = io_round(rng.standard_normal((batch, dim, 3)), "bf16")
    du = inputs.grad_output(x)
    say("conv_bwd Mamba-1.4B layer %s" % (x.u.shape,))
    g = run(x.u, w, cb, prev, du, True, "bf16")
    want = oracle.conv1d_bwd_f64(x.u, w, du, cb, prev, silu=True)
    compare(g, want, "bf16", "Mamba-1.4B layer")


def test_conv_bwd_mamba130m_layer():
    """The Mamba-130M layer (batch 8, dim 1536, seqlen 2048, K = 4, fp32 io), every output: the
    fp32 rows that take their neighbouring tokens across lanes."""
    x = inputs.scan_config(1)
    batch, dim, _, _ = x.shape
    w, cb = inputs.conv_params(dim, 4)
    rng = np.random.default_rng(65110)
    prev = rng.standard_normal((batch, dim, 3)).astype(np.float32)
    du = inputs.grad_output(x)
    say("conv_bwd Mamba-130M layer %s" % (x.u.shape,))
    g = run(x.u, w, cb, prev, du, True, "f32")
    want = oracle.conv1d_bwd_f64(x.u, w, du, cb, prev, silu=True)
    compare(g, want, "f32", "Mamba-130M layer")


def test_conv_scan_training_chain():
    """conv_scan_fwd, scan_bwd on the u it stored, then conv_bwd on that du, against
    the same three steps in fp64 (fp32 io).

    The bar for dx and the conv's sums adds to this kernel's own 1e-4 the scan
    backward's error in du (1e-4 of max|du|) carried through the conv's
    gradient: at most sum_k |w_k| * max|silu'| times it for dx, and
    sum over (batch, token) of |x| * max|silu'| times it for dconv_weight.
    """
    b, d, n, l, width = 2, 96, 16, 712, 4  # the scan backward takes seqlen in multiples of 8
    say("conv + scan training chain (%d, %d, %d, %d)" % (b, d, n, l))
    x = inputs.make_scan_inputs(b, d, n, l, io="f32", seed=65105)
    w, cb = inputs.conv_params(d, width, seed=65106)
    rng = np.random.default_rng(65107)
    prev = rng.standard_normal((b, d, width - 1)).astype(np.float32)
    dy = inputs.grad_output(x, seed=65108)
    t = inputs.to_torch(x, DEV)
    xs = t["u"]
    wt, cbt, pt = (torch.from_numpy(a).to(DEV) for a in (w, cb, prev))
    u_out = torch.empty_like(xs)
    binding.conv_scan_fwd(xs, wt, t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                          delta_bias=t["delta_bias"], delta_softplus=x.softplus, conv_bias=cbt, x_prev=pt,
                          conv_silu=True, h0=t["h0"], u_out=u_out)
    gs = binding.scan_bwd(u_out, t["delta"], t["A"], t["B"], t["C"], torch.from_numpy(dy).to(DEV), D=t["D"],
                          z=t["z"], delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=t["h0"])
    gc = binding.conv_bwd(xs, wt, gs["du"], conv_bias=cbt, x_prev=pt, conv_silu=True)
    torch.cuda.synchronize()

    u64 = oracle.conv1d_f64(x.u, w, cb, prev, silu=True)
    ws = oracle.scan_bwd_f64(u64, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0, dy=dy)
    wc = oracle.conv1d_bwd_f64(x.u, w, ws["du"], cb, prev, silu=True)

    du_err = 1e-4 * float(np.max(np.abs(ws["du"])))
    gain_dx = float(np.max(np.sum(np.abs(w), axis=1))) * SILU_SLOPE_MAX
    xabs = np.abs(np.concatenate([prev.astype(np.float64), x.u.astype(np.float64)], axis=2))
    gain_dw = float(np.max(np.sum(xabs, axis=(0, 2)))) * SILU_SLOPE_MAX
    gain_db = b * l * SILU_SLOPE_MAX
    for got, want, gain, what in ((gc["dx"], wc["dx"], gain_dx, "dx"),
                                  (gc["dconv_weight"], wc["dweight"], gain_dw, "dconv_weight"),
                                  (gc["dconv_bias"], wc["dbias"], gain_db, "dconv_bias"),
                                  (gc["dx_prev"], wc["dx_prev"], gain_dx, "dx_prev")):
        gv = np64(got)
        assert np.isfinite(gv).all(), what
        err = float(np.max(np.abs(gv - want)))
        bound = 1e-4 * float(np.max(np.abs(want))) + gain * du_err
        assert err <= bound, "%s: max err %.3e > %.3e" % (what, err, bound)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_bwd_misaligned_rows(io):
    """x and du starting one element past a 16-byte boundary (seqlen a multiple
    of 8): the element-wise load path, same results."""
    b, d, l, width = 2, 24, 2056, 4
    say("conv_bwd misaligned io=%s" % io)
    x, w, cb, prev, du = draw(b, d, l, width, io, seed=65109)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    n = b * d * l

    def shifted(a):
        buf = torch.zeros(n + 1, dtype=dt, device=DEV)
        buf[1:] = torch.from_numpy(a.reshape(-1)).to(DEV, dt)
        return buf[1:].view(b, d, l)

    xs, dus = shifted(x), shifted(du)
    assert xs.data_ptr() % 16 != 0 and dus.data_ptr() % 16 != 0
    wt, cbt, pt = torch.from_numpy(w).to(DEV), torch.from_numpy(cb).to(DEV), to_dev(prev, io)
    g = binding.conv_bwd(xs, wt, dus, conv_bias=cbt, x_prev=pt, conv_silu=True)
    torch.cuda.synchronize()
    compare(g, oracle.conv1d_bwd_f64(x, w, du, cb, prev, silu=True), io, "misaligned")
