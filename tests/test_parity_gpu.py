"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Bar (per output tensor): max|got - want| <= tol * max|want| with tol = 1e-4
for fp32 io and 2e-2 for bf16 io; `want` is the fp64 oracle on the identical
(bf16-rounded where applicable) inputs.  Full-size workloads are checked on
sampled (batch, channel) rows, which the oracle computes exactly because
channels are independent.
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
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    assert err <= TOL[io] * scale + 1e-30, "%s: max err %.3e > %.1e * %.3e" % (what, err, TOL[io], scale)
    return err / max(scale, 1e-30)


def gpu_scan(x, h0=None, last_state=True, **kw):
    t = inputs.to_torch(x, DEV)
    if h0 is None:
        h0 = t["h0"]
    y, last = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=h0,
                               return_last_state=last_state, **kw)
    torch.cuda.synchronize()
    return y, last


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_full(x):
    return oracle.scan_f64(x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)


# ---------------------------------------------------------------------------
# The workloads


def test_tiny_config_full():
    x = inputs.scan_config(0)
    say("tiny config 1x16x4x64 fp32")
    y, last = gpu_scan(x)
    yr, hr = oracle_full(x)
    check(np64(y), yr, "f32", "y")
    check(np64(last), hr, "f32", "last_state")


@pytest.mark.parametrize("cfg,k", [(1, 48), (2, 48)])
def test_layer_configs_sampled(cfg, k):
    x = inputs.scan_config(cfg)
    b, d, n, l = x.shape
    say("config %d %dx%dx%dx%d %s" % (cfg, b, d, n, l, x.io))
    y, last = gpu_scan(x)
    ch = inputs.sample_channels(b, d, k, seed=cfg)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    bi = torch.tensor([c[0] for c in ch], device=DEV)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    check(np64(y[bi, di]), yr, x.io, "y")
    # The state is fp32 arithmetic on identical inputs for either io dtype.
    check(np64(last[bi, di]), hr, "f32", "last_state")


@pytest.mark.parametrize("cfg,k", [(1, 24), (2, 24), (3, 4)])
def test_ssm_part_alone_full_size(cfg, k):
    """The workloads with D = null and z = null: y is then C.h alone, which the
    D.u skip otherwise dominates.  Each output is normalised by its own max."""
    x = inputs.scan_config(cfg, D=False, z=False)
    b, d, n, l = x.shape
    say("diagnostic config %d %dx%dx%dx%d %s, D and z null" % (cfg, b, d, n, l, x.io))
    y, last = gpu_scan(x)
    ch = inputs.sample_channels(b, d, k, seed=100 + cfg)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    bi = torch.tensor([c[0] for c in ch], device=DEV)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    ey = check(np64(y[bi, di]), yr, x.io, "y (C.h alone)")
    eh = check(np64(last[bi, di]), hr, "f32", "last_state")
    say("diagnostic config %d: y rel err %.2e, last_state rel err %.2e" % (cfg, ey, eh))


def test_layer_shape_varied_channels_sampled():
    """The Mamba-1.4B layer shape with a per-channel A row and D (test recipe)."""
    x = inputs.scan_config(2, channel_params_kind="varied")
    b, d, n, l = x.shape
    assert np.unique(x.D).size > 1000 and np.unique(x.A[:, 0]).size > 1000
    say("config 2 shape with per-channel A and D")
    y, last = gpu_scan(x)
    ch = inputs.sample_channels(b, d, 32, seed=12)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    bi = torch.tensor([c[0] for c in ch], device=DEV)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    check(np64(y[bi, di]), yr, x.io, "y")
    check(np64(last[bi, di]), hr, "f32", "last_state")


# Segmented plans whose aggregate launch cuts each segment into pieces: 1 x
# 2560 channels x 32768 tokens gives 52 segments of 640 tokens, a multiple of
# 128 whose halves are >= 256 tokens, and 40 groups x 51 segments x 2 pieces
# fit the aggregate launch's 4096 waves, so every segment but the last is
# aggregated in two pieces and the carry launch folds 102 pieces.
PIECE_CASES = [("f32", 16, "delta_b"), ("bf16", 16, "delta_b"), ("f32", 5, "delta_b"), ("f32", 16, "zoh"),
               ("bf16", 8, "zoh")]


@pytest.mark.parametrize("io,n,disc", PIECE_CASES, ids=["%s-n%d-%s" % c for c in PIECE_CASES])
def test_segmented_aggregate_pieces(io, n, disc):
    b, d, l = 1, 2560, 32768
    dt = torch.float32 if io == "f32" else torch.bfloat16
    path, seg, seglen, scratch = binding.scan_plan(b, d, n, l, dt, with_path=True, disc=disc)
    if n == 16:   # dstate 16 runs the chunked kernel instead
        assert (path, seg, seglen, scratch) == ("chunked", 1, l, 0)
    else:
        assert (seg, seglen, scratch) == (52, 640, 0) and path == ("segmented" if n in (4, 8, 16) else "generic")
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=2100 + n, h0=True)
    say("aggregate pieces %s n=%d %s path=%s" % (io, n, disc, path))
    t = inputs.to_torch(x, DEV)
    y, last = binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], disc=disc)
    torch.cuda.synchronize()
    ch = inputs.sample_channels(b, d, 6, seed=n)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, True, x.h0,
                                      zoh=disc == "zoh")
    di = torch.tensor([c[1] for c in ch], device=DEV)
    check(np64(y[0, di]), yr, io, "y")
    check(np64(last[0, di]), hr, "f32", "last_state")


LONG_ROWS = [("f32", "delta_b", 16), ("bf16", "zoh", 16), ("f32", "zoh", 8), ("bf16", "delta_b", 8)]


@pytest.mark.parametrize("io,disc,n", LONG_ROWS, ids=["%s-%s-n%d" % c for c in LONG_ROWS])
def test_long_rows_two_batch_rows_ragged_dim(io, disc, n):
    """Two batch rows of 1300 channels over 31360 tokens, with an initial
    state; sampled channels of both rows, the ragged channel blocks included.
    dstate 16 runs the chunked kernel (31 tiles, the last 640 tokens long;
    the last block of each row only partly filled); dstate 8 runs segmented:
    49 segments of 640 tokens, each aggregated in two pieces (42 x 48 x 2 =
    4032 waves, the last group 20 channels wide)."""
    b, d, l = 2, 1300, 31360
    dt = torch.float32 if io == "f32" else torch.bfloat16
    want = ("chunked", 1, l, 0) if n == 16 else ("segmented", 49, 640, 0)
    assert binding.scan_plan(b, d, n, l, dt, with_path=True, disc=disc) == want
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=2200 + n, h0=True)
    say("long rows, 2 batch rows, ragged dim, io=%s disc=%s n=%d path=%s" % (io, disc, n, want[0]))
    t = inputs.to_torch(x, DEV)
    y, last = binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=t["h0"], disc=disc)
    torch.cuda.synchronize()
    ch = inputs.sample_channels(b, d, 8, seed=22) + [(0, d - 1), (1, d - 2), (1, d - 20), (0, d - 21)]
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0,
                                      zoh=disc == "zoh")
    bi = torch.tensor([c[0] for c in ch], device=DEV)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    check(np64(y[bi, di]), yr, io, "y")
    check(np64(last[bi, di]), hr, "f32", "last_state")


def test_long_sequence_sampled_and_carry():
    x = inputs.scan_config(3)
    b, d, n, l = x.shape
    say("config 3 %dx%dx%dx%d one pass" % (b, d, n, l))
    y, last = gpu_scan(x)
    ch = inputs.sample_channels(b, d, 6, seed=3)
    yr, hr = oracle.scan_channels_f64(ch, x.u, x.delta, x.A, x.B, x.C, x.D, x.z, x.delta_bias, x.softplus, x.h0)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    check(np64(y[0, di]), yr, "f32", "y one pass")
    check(np64(last[0, di]), hr, "f32", "last_state one pass")
    say("config 3 four segments with last_state carry")
    t = inputs.to_torch(x, DEV)
    h = None
    seg = l // 4
    ys = []
    for s in range(4):
        sl = slice(s * seg, (s + 1) * seg)
        ys_, h = binding.scan_fwd(t["u"][..., sl].contiguous(), t["delta"][..., sl].contiguous(), t["A"],
                                  t["B"][..., sl].contiguous(), t["C"][..., sl].contiguous(), D=t["D"],
                                  z=t["z"][..., sl].contiguous(), delta_bias=t["delta_bias"], delta_softplus=True,
                                  h0=h)
        ys.append(ys_[0, di])
    torch.cuda.synchronize()
    check(np64(torch.cat(ys, dim=-1)), yr, "f32", "y carried")
    check(np64(h[0, di]), hr, "f32", "last_state carried")


def test_decode_workload():
    dec = inputs.decode_config()
    bsz, dim, n = dec.batch, dec.dim, dec.dstate
    say("decode %dx%dx%d, %d steps" % (bsz, dim, n, dec.steps))
    ch = inputs.sample_channels(bsz, dim, 64, seed=4)
    bi = torch.tensor([c[0] for c in ch], device=DEV)
    di = torch.tensor([c[1] for c in ch], device=DEV)
    state = torch.from_numpy(dec.state0).to(DEV)
    A = torch.from_numpy(dec.A).to(DEV)
    D = torch.from_numpy(dec.D).to(DEV)
    bias = torch.from_numpy(dec.delta_bias).to(DEV)
    ref_state = np.ascontiguousarray(dec.state0[[c[0] for c in ch], [c[1] for c in ch]], dtype=np.float64)
    ys_gpu = torch.empty((dec.steps, len(ch)), device=DEV)
    ys_ref = np.empty((dec.steps, len(ch)))
    for s in range(dec.steps):
        st = dec.step(s)
        tt = {k: torch.from_numpy(v).to(DEV, torch.bfloat16) for k, v in st.items()}
        y = binding.state_update(state, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"], delta_bias=bias,
                                 delta_softplus=True)
        ys_gpu[s] = y[bi, di].float()
        ys_ref[s] = oracle.state_update_channels_f64(ch, ref_state, st["u"], st["delta"], dec.A, st["B"], st["C"],
                                                     dec.D, st["z"], dec.delta_bias, softplus=True)
    torch.cuda.synchronize()
    got = ys_gpu.cpu().numpy().astype(np.float64)
    for s in range(dec.steps):
        check(got[s], ys_ref[s], "bf16", "decode y step %d" % s)
    check(np64(state[bi, di]), ref_state, "f32", "decode final state")


def test_decode_varied_channels():
    """64 decode steps at 32x1024x16 with a per-channel A row and D."""
    dec = inputs.decode_config(batch=32, dim=1024, steps=64, channel_params_kind="varied")
    say("decode %dx%dx%d, %d steps, per-channel A and D" % (dec.batch, dec.dim, dec.dstate, dec.steps))
    state = torch.from_numpy(dec.state0).to(DEV)
    A = torch.from_numpy(dec.A).to(DEV)
    D = torch.from_numpy(dec.D).to(DEV)
    bias = torch.from_numpy(dec.delta_bias).to(DEV)
    ref_state = dec.state0.astype(np.float64)
    for s in range(dec.steps):
        st = dec.step(s)
        tt = {k: torch.from_numpy(v).to(DEV, torch.bfloat16) for k, v in st.items()}
        y = binding.state_update(state, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"], delta_bias=bias,
                                 delta_softplus=True)
        yr = oracle.state_update_f64(ref_state, st["u"], st["delta"], dec.A, st["B"], st["C"], dec.D, st["z"],
                                     dec.delta_bias, softplus=True)
        check(np64(y), yr, "bf16", "decode y step %d" % s)
    torch.cuda.synchronize()
    check(np64(state), ref_state, "f32", "decode final state")


# ---------------------------------------------------------------------------
# Flags, shapes, edge cases


FLAG_SHAPES = [(2, 80, 16, 200), (1, 70, 16, 1000), (1, 70, 8, 1000)]   # chunked, chunked, segmented


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", FLAG_SHAPES, ids=["%dx%dx%dx%d" % s for s in FLAG_SHAPES])
def test_flag_matrix(io, shape):
    b, d, n, l = shape
    for mask in range(32):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=100 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        if not sp:
            # Without softplus the step is delta + bias as given; keep it
            # positive so the test system stays stable (|Abar| <= 1).
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        say("flags z=%d D=%d bias=%d softplus=%d h0=%d shape=%s io=%s" % (z, D, bias, sp, h0, shape, io))
        y, last = gpu_scan(x)
        yr, hr = oracle_full(x)
        check(np64(y), yr, io, "y mask=%d" % mask)
        check(np64(last), hr, "f32", "last_state mask=%d" % mask)


ODD = [(1, 1, 16, 1), (1, 3, 16, 7), (2, 63, 16, 63), (1, 65, 16, 65), (1, 64, 16, 4097), (1, 33, 1, 40),
       (2, 17, 3, 29), (1, 40, 5, 300), (1, 70, 8, 520), (1, 100, 4, 3000), (3, 129, 16, 264), (1, 64, 12, 777)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ODD, ids=["%dx%dx%dx%d" % s for s in ODD])
def test_odd_shapes(io, shape):
    b, d, n, l = shape
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=7, h0=True)
    say("odd shape %s io=%s plan=%s" % (shape, io, binding.scan_plan(b, d, n, l, torch.float32 if io == "f32"
                                                                     else torch.bfloat16)))
    y, last = gpu_scan(x)
    yr, hr = oracle_full(x)
    check(np64(y), yr, io, "y")
    check(np64(last), hr, "f32", "last_state")


def test_long_sequence_plans():
    # The long-sequence workload runs the chunked kernel (one launch, nothing
    # but y and last_state written), under either discretization of B and
    # with the conv; at dstate 8 it runs segmented, with its aggregates and
    # carries in y.  Neither takes scratch.
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True) == ("chunked", 1, 131072, 0)
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True, disc="zoh") == \
        ("chunked", 1, 131072, 0)
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True, conv_width=4) == \
        ("chunked", 1, 131072, 0)
    path, seg, seglen, scratch = binding.scan_plan(1, 2560, 8, 131072, torch.float32, with_path=True)
    assert path == "segmented" and seg > 1 and scratch == 0


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("n,path", [(16, "chunked"), (8, "segmented")])
def test_h0_aliases_last_state(io, n, path):
    b, d, l = 1, 96, 4096
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=9, h0=True)
    assert binding.scan_plan(b, d, n, l, torch.float32, with_path=True)[0] == path
    t = inputs.to_torch(x, DEV)
    say("h0 aliasing last_state io=%s n=%d path=%s" % (io, n, path))
    state = t["h0"].clone()
    y, last = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               delta_bias=t["delta_bias"], delta_softplus=True, h0=state, last_state=state)
    torch.cuda.synchronize()
    assert last.data_ptr() == state.data_ptr()
    yr, hr = oracle_full(x)
    check(np64(y), yr, io, "y")
    check(np64(state), hr, "f32", "state carried in place")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_equals_one_token_scan(io):
    b, d, n = 3, 200, 16
    x = inputs.make_scan_inputs(b, d, n, 1, io=io, seed=21, h0=True)
    t = inputs.to_torch(x, DEV)
    say("decode vs one-token scan io=%s" % io)
    y_scan, h_scan = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                      delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])
    state = t["h0"].clone()
    y_dec = binding.state_update(state, t["u"][..., 0].contiguous(), t["delta"][..., 0].contiguous(), t["A"],
                                 t["B"][..., 0].contiguous(), t["C"][..., 0].contiguous(), D=t["D"],
                                 z=t["z"][..., 0].contiguous(), delta_bias=t["delta_bias"], delta_softplus=True)
    torch.cuda.synchronize()
    yr, hr = oracle_full(x)
    check(np64(y_dec), yr[..., 0], io, "decode y")
    check(np64(state), hr, "f32", "decode state")
    check(np64(y_dec), np64(y_scan[..., 0]), io, "decode vs scan y")
    assert torch.allclose(state, h_scan, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("n", [1, 5, 8, 4])
def test_decode_generic_dstate(n):
    b, d = 2, 37
    x = inputs.make_scan_inputs(b, d, n, 1, io="f32", seed=22, h0=True)
    t = inputs.to_torch(x, DEV)
    say("decode dstate=%d" % n)
    state = t["h0"].clone()
    y = binding.state_update(state, t["u"][..., 0].contiguous(), t["delta"][..., 0].contiguous(), t["A"],
                             t["B"][..., 0].contiguous(), t["C"][..., 0].contiguous(), D=t["D"],
                             z=t["z"][..., 0].contiguous(), delta_bias=t["delta_bias"], delta_softplus=True)
    torch.cuda.synchronize()
    yr, hr = oracle_full(x)
    check(np64(y), yr[..., 0], "f32", "y")
    check(np64(state), hr, "f32", "state")


def test_run_to_run_bitwise():
    x = inputs.make_scan_inputs(4, 256, 16, 2048, io="bf16", seed=31, h0=True)
    say("determinism")
    y1, h1 = gpu_scan(x)
    y2, h2 = gpu_scan(x)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    x = inputs.make_scan_inputs(1, 64, 16, 8192, io="f32", seed=32)
    y1, h1 = gpu_scan(x)
    y2, h2 = gpu_scan(x)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_misaligned_rows_segmented(io):
    """Rows one element off 16-byte alignment on a segmented shape: the generic
    kernel, with the segment slots in a y that is only element-aligned."""
    b, d, n, l = 1, 70, 16, 2000
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=42, h0=True)
    # The plan (for aligned rows) is the chunked kernel; rows that are not
    # 16-byte aligned run the per-token kernel over the segmented plan (the
    # one dstate 8 would take).
    assert binding.scan_plan(b, d, 8, l, torch.float32 if io == "f32" else torch.bfloat16)[0] > 1
    t = inputs.to_torch(x, DEV)
    say("misaligned segmented io=%s" % io)

    def shifted(a):
        flat = torch.empty(a.numel() + 1, dtype=a.dtype, device=DEV)
        v = flat[1:].view(a.shape)
        v.copy_(a)
        return v

    ybuf = torch.empty(b * d * l + 1, dtype=t["u"].dtype, device=DEV)
    y = ybuf[1:].view(b, d, l)
    _, last = binding.scan_fwd(shifted(t["u"]), shifted(t["delta"]), t["A"], shifted(t["B"]), shifted(t["C"]),
                               D=t["D"], z=shifted(t["z"]), delta_bias=t["delta_bias"], delta_softplus=True,
                               h0=t["h0"], out=y)
    torch.cuda.synchronize()
    yr, hr = oracle_full(x)
    check(np64(y), yr, io, "y")
    check(np64(last), hr, "f32", "last_state")


def test_misaligned_rows_take_the_generic_path():
    b, d, n, l = 1, 70, 16, 96
    x = inputs.make_scan_inputs(b, d, n, l, io="f32", seed=41, h0=True)
    t = inputs.to_torch(x, DEV)
    say("misaligned base pointers")

    def shifted(a):
        flat = torch.empty(a.numel() + 1, dtype=a.dtype, device=DEV)
        v = flat[1:].view(a.shape)
        v.copy_(a)
        return v

    y, last = binding.scan_fwd(shifted(t["u"]), shifted(t["delta"]), t["A"], shifted(t["B"]), shifted(t["C"]),
                               D=t["D"], z=shifted(t["z"]), delta_bias=t["delta_bias"], delta_softplus=True,
                               h0=t["h0"])
    torch.cuda.synchronize()
    yr, hr = oracle_full(x)
    check(np64(y), yr, "f32", "y")
    check(np64(last), hr, "f32", "last_state")


def test_nan_and_inf_propagate():
    b, d, n, l = 1, 64, 16, 64
    x = inputs.make_scan_inputs(b, d, n, l, io="f32", seed=51)
    x.u[0, 3, 10] = np.nan
    x.z[0, 5, 20] = np.inf
    say("nan/inf propagation")
    y, _ = gpu_scan(x)
    yr, _ = oracle_full(x)
    got = np64(y)
    assert np.array_equal(np.isnan(got), np.isnan(yr))
    assert np.array_equal(np.isinf(got), np.isinf(yr))
    fin = np.isfinite(yr)
    assert np.max(np.abs(got[fin] - yr[fin])) <= 1e-4 * np.max(np.abs(yr[fin]))


def test_binding_rejects_aliasing():
    x = inputs.make_scan_inputs(1, 8, 4, 16, io="f32", seed=61)
    t = inputs.to_torch(x, DEV)
    with pytest.raises(binding.SsmError) as e:
        binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], out=t["u"])
    assert e.value.name == "SSM_ERR_ALIAS"


# Shapes with at least 192 channel groups take the single-pass state-split
# kernel; keep them small in seqlen so the full oracle stays cheap.
SPLIT_SHAPES = [(192, 64, 16, 72), (96, 130, 16, 40), (200, 64, 8, 24), (256, 33, 4, 8), (192, 64, 16, 256)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=["%dx%dx%dx%d" % s for s in SPLIT_SHAPES])
def test_split_path(io, shape):
    b, d, n, l = shape
    path, seg, seglen, scratch = binding.scan_plan(b, d, n, l, torch.float32 if io == "f32" else torch.bfloat16,
                                                   with_path=True)
    assert path == "split" and seg == 1
    for mask in (0, 31, 5, 26):
        z, D, bias, sp, h0 = [(mask >> i) & 1 == 1 for i in range(5)]
        x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=300 + mask, z=z, D=D, bias=bias, softplus=sp, h0=h0)
        if not sp:
            x.delta = inputs.round_bf16(np.abs(x.delta) * np.float32(0.2)) if io == "bf16" else \
                np.abs(x.delta) * np.float32(0.2)
            if bias:
                x.delta_bias = np.full(d, 0.01, np.float32)
        say("split path shape=%s io=%s mask=%d" % (shape, io, mask))
        y, last = gpu_scan(x)
        yr, hr = oracle_full(x)
        check(np64(y), yr, io, "y mask=%d" % mask)
        check(np64(last), hr, "f32", "last_state mask=%d" % mask)


def test_split_path_determinism_and_alias():
    b, d, n, l = 192, 64, 16, 128
    x = inputs.make_scan_inputs(b, d, n, l, io="bf16", seed=400, h0=True)
    t = inputs.to_torch(x, DEV)
    say("split path determinism + in-place state")
    y1, h1 = gpu_scan(x)
    y2, h2 = gpu_scan(x)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    state = t["h0"].clone()
    y3, _ = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["delta_bias"], delta_softplus=True, h0=state, last_state=state)
    torch.cuda.synchronize()
    assert torch.equal(y3, y1) and torch.equal(state, h1)
