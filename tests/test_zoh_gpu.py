"""Exact zero-order hold for B (ssm_scan_fwd_ex / ssm_state_update_ex with
SSM_DISC_ZOH) against the fp64 oracle, through the C ABI (needs an MI355X).

Bar as for the Delta*B scan: max|got - want| <= tol * max|want| per output,
tol = 1e-4 for fp32 io and 2e-2 for bf16 io (states: 1e-4 for both, the state
being fp32 arithmetic on identical inputs).  Every kernel path is covered
(single pass, segmented, generic, decode), with A holding zeros, tiny values
and (decode) a small positive entry, and step sizes on both sides of the |Delta A| =
1/16 switch between the series and exp(Delta A) - 1.
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


def awkward_A(x, positive=False):
    """Zeros and tiny magnitudes in A; with positive, also a small positive entry
    (a growing state: only for a few tokens, or fp32 growth would swamp the bar)."""
    A = x.A.copy()
    dim, n = A.shape
    A[::3, 0] = 0.0
    A[1::3, min(1, n - 1)] = -1e-6
    if positive:
        A[2::5, n - 1] = 0.05
    x.A = A
    return x


def wide_steps(x, seed):
    """Step sizes spread over 1e-4 .. 3 (softplus off, no bias), so |Delta A| crosses 1/16."""
    rng = np.random.default_rng(seed)
    d = np.exp(rng.uniform(np.log(1e-4), np.log(3.0), size=x.delta.shape)).astype(np.float32)
    x.delta = inputs.round_bf16(d) if x.io == "bf16" else d
    x.softplus = False
    x.delta_bias = None
    return x


def run_ex(x, disc="zoh"):
    t = inputs.to_torch(x, DEV)
    y, last = binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=t["h0"], disc=disc)
    torch.cuda.synchronize()
    return y, last


def oracle_zoh(x):
    return oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0, zoh=True)


# (shape, expected path): the single-pass kernel, the chunked kernel (the
# second shape ends in a partial tile), the segmented path (dstate 8), the
# generic path (dstate 12; seqlen 63).
SHAPES = [((192, 64, 16, 96), "split"), ((200, 64, 8, 40), "split"), ((256, 33, 4, 24), "split"),
          ((1, 64, 16, 4096), "chunked"), ((1, 64, 16, 2056), "chunked"), ((2, 96, 8, 1536), "segmented"),
          ((2, 63, 12, 72), "generic"), ((3, 40, 16, 63), "generic")]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape,path", SHAPES, ids=["%dx%dx%dx%d" % s for s, _ in SHAPES])
def test_zoh_scan_paths(io, shape, path):
    b, d, n, l = shape
    dt = torch.float32 if io == "f32" else torch.bfloat16
    assert binding.scan_plan(b, d, n, l, dt, with_path=True, disc="zoh")[0] == path
    for variant in ("workload", "awkward_A", "wide_steps"):
        say("zoh shape=%s io=%s path=%s variant=%s" % (shape, io, path, variant))
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=3000 + n + l, h0=True)
        if variant != "workload":
            x = awkward_A(x)
        if variant == "wide_steps":
            x = wide_steps(x, 3100 + l)
        y, last = run_ex(x)
        yr, hr = oracle_zoh(x)
        check(np64(y), yr, TOL[io], "y %s" % variant)
        check(np64(last), hr, TOL["f32"], "last_state %s" % variant)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_delta_b_disc_is_scan_fwd_bitwise(io):
    for shape in ((192, 64, 16, 64), (1, 64, 16, 2048), (2, 63, 12, 40)):
        say("disc=delta_b vs scan_fwd shape=%s io=%s" % (shape, io))
        x = inputs.make_scan_inputs(*shape, io=io, seed=3200, h0=True)
        y1, h1 = run_ex(x, disc="delta_b")
        t = inputs.to_torch(x, DEV)
        y2, h2 = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_zoh_differs_from_delta_b():
    """The switch is live: with Delta of order 1 the two rules give clearly different outputs."""
    x = inputs.make_scan_inputs(192, 64, 16, 64, io="f32", seed=3300)
    x = wide_steps(x, 3301)
    y1, _ = run_ex(x, disc="delta_b")
    y2, _ = run_ex(x, disc="zoh")
    assert float((y1 - y2).abs().max()) > 1e-2 * float(y1.abs().max())


def test_zoh_mamba1p4b_layer_sampled():
    x = inputs.scan_config(2)
    say("zoh Mamba-1.4B layer (4x4096x16x4096 bf16), sampled channels")
    y, last = run_ex(x)
    ch = inputs.sample_channels(4, 4096, 24, seed=5)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0,
                                      zoh=True)
    yg = np64(y)
    hg = np64(last)
    check(np.stack([yg[b, d] for b, d in ch]), yr, TOL["bf16"], "y")
    check(np.stack([hg[b, d] for b, d in ch]), hr, TOL["f32"], "last_state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dstate", [16, 4, 5])
def test_zoh_decode(io, dstate):
    batch, dim, steps = 8, 96, 6
    rng = np.random.default_rng(3400 + dstate)
    x = inputs.make_scan_inputs(batch, dim, dstate, 1, io=io, seed=3400 + dstate)
    x = awkward_A(x, positive=True)
    state = (0.1 * rng.standard_normal((batch, dim, dstate))).astype(np.float32)
    st_gpu = torch.from_numpy(state).to(DEV)
    st_ref = state.astype(np.float64)
    A = torch.from_numpy(x.A).to(DEV)
    Dt = torch.from_numpy(x.D).to(DEV)
    bt = torch.from_numpy(x.delta_bias).to(DEV)
    dt = torch.float32 if io == "f32" else torch.bfloat16
    for s in range(steps):
        say("zoh decode io=%s dstate=%d step=%d" % (io, dstate, s))
        r = np.random.default_rng([3401, dstate, s])
        f = {k: r.standard_normal(shp).astype(np.float32)
             for k, shp in (("u", (batch, dim)), ("delta", (batch, dim)), ("z", (batch, dim)),
                            ("B", (batch, dstate)), ("C", (batch, dstate)))}
        f["delta"] *= np.float32(0.5)
        if io == "bf16":
            f = {k: inputs.round_bf16(v) for k, v in f.items()}
        tt = {k: torch.from_numpy(v).to(DEV, dt) for k, v in f.items()}
        y = binding.state_update_ex(st_gpu, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=Dt, z=tt["z"], delta_bias=bt,
                                    delta_softplus=True, disc="zoh")
        torch.cuda.synchronize()
        yr = oracle.state_update_f64(st_ref, f["u"], f["delta"], x.A, f["B"], f["C"], x.D, f["z"], x.delta_bias,
                                     softplus=True, zoh=True)
        check(np64(y), yr, TOL[io], "y step %d" % s)
        check(np64(st_gpu), st_ref, TOL["f32"], "state step %d" % s)


def test_zoh_decode_equals_one_token_scan():
    x = inputs.make_scan_inputs(4, 128, 16, 1, io="f32", seed=3500, h0=True)
    x = awkward_A(x)
    t = inputs.to_torch(x, DEV)
    y_scan, last = binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                       delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], disc="zoh")
    st = t["h0"].clone()
    y_dec = binding.state_update_ex(st, t["u"][..., 0], t["delta"][..., 0], t["A"], t["B"][..., 0].contiguous(),
                                    t["C"][..., 0].contiguous(), D=t["D"], z=t["z"][..., 0].contiguous(),
                                    delta_bias=t["delta_bias"], delta_softplus=True, disc="zoh")
    torch.cuda.synchronize()
    check(np64(y_dec), np64(y_scan[..., 0]), 1e-6, "y")
    check(np64(st), np64(last), 1e-6, "state")


def test_binding_rejects_unknown_disc():
    x = inputs.make_scan_inputs(1, 8, 4, 8, io="f32", seed=3600)
    t = inputs.to_torch(x, DEV)
    with pytest.raises(ValueError):
        binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], disc="bilinear")
