"""The decode step and the single-pass prefill captured in a HIP graph (through
torch.cuda.CUDAGraph, which records the library's launches on the capture
stream): every replay equals the eager result bit for bit, with eager work and
synchronisations between replays.  Neither path allocates or clears memory,
so a capture holds only their kernel launches.
"""
import numpy as np
import pytest
import torch

from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def test_decode_steps_in_a_graph():
    dec = inputs.decode_config(batch=16, dim=512, steps=4, channel_params_kind="varied")
    A = torch.from_numpy(dec.A).to(DEV)
    D = torch.from_numpy(dec.D).to(DEV)
    bias = torch.from_numpy(dec.delta_bias).to(DEV)
    st = dec.step(0)
    tt = {k: torch.from_numpy(v).to(DEV, torch.bfloat16) for k, v in st.items()}
    state0 = torch.from_numpy(dec.state0).to(DEV)

    # Eager reference: three steps from state0.
    ref_state = state0.clone()
    ref_y = []
    for _ in range(3):
        ref_y.append(binding.state_update(ref_state, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"],
                                          delta_bias=bias, delta_softplus=True).clone())
    torch.cuda.synchronize()

    state = state0.clone()
    y = torch.empty_like(tt["u"])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm the library up on the capture stream
        binding.state_update(state.clone(), tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"], delta_bias=bias,
                             delta_softplus=True, out=torch.empty_like(y))
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        binding.state_update(state, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"], delta_bias=bias,
                             delta_softplus=True, out=y)
    state.copy_(state0)
    torch.cuda.synchronize()
    for i in range(3):
        say("decode graph replay %d" % i)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y[i]), "replay %d: y" % i
        _ = (state * 2.0).sum().item()  # eager work between replays
    assert torch.equal(state, ref_state)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_prefill_in_a_graph(io):
    x = inputs.make_scan_inputs(192, 64, 16, 128, io=io, seed=77, h0=True)
    assert binding.scan_plan(192, 64, 16, 128, torch.float32 if io == "f32" else torch.bfloat16,
                             with_path=True)[0] == "split"
    t = inputs.to_torch(x, DEV)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])
    y_ref, h_ref = binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    last = torch.empty_like(h_ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], out=torch.empty_like(y),
                         last_state=torch.empty_like(last), **kw)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], out=y, last_state=last, **kw)
    for i in range(3):
        say("prefill graph replay %d io=%s" % (i, io))
        y.zero_()
        last.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(last, h_ref), "replay %d" % i
        _ = float(np.float64(y.float().abs().sum().item()))  # eager work between replays


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("conv", [False, True])
def test_segmented_prefill_in_a_graph(io, conv):
    """The chunked path (dstate 16, the plain scan) and the segmented path
    (dstate 8, the conv fused into it; three launches, aggregates and carries
    in y) allocate nothing, so a capture holds only launches."""
    b, d, l = 1, 128, 4096
    n = 8 if conv else 16
    dt = torch.float32 if io == "f32" else torch.bfloat16
    path, seg = binding.scan_plan(b, d, n, l, dt, with_path=True, conv_width=4 if conv else 0)[:2]
    assert (path, seg > 1) == (("segmented", True) if conv else ("chunked", False))
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=78, h0=True)
    t = inputs.to_torch(x, DEV)
    w = torch.from_numpy((0.5 * np.random.default_rng(79).standard_normal((d, 4))).astype(np.float32)).to(DEV)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"])

    def call(out, last):
        if conv:
            return binding.conv_scan_fwd(t["u"], w, t["delta"], t["A"], t["B"], t["C"], conv_silu=True, out=out,
                                         last_state=last, **kw)
        return binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], out=out, last_state=last, **kw)

    y_ref, h_ref = call(None, None)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    last = torch.empty_like(h_ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(torch.empty_like(y), torch.empty_like(last))
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(y, last)
    for i in range(3):
        say("segmented prefill graph replay %d io=%s conv=%s" % (i, io, conv))
        y.fill_(7.0)
        last.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(last, h_ref), "replay %d" % i
        _ = float(np.float64(y.float().abs().sum().item()))  # eager work between replays
