"""ssm_scan_bwd_saved_noalloc -- the saved-checkpoint backward with its scratch
in the library's fixed device array -- against ssm_scan_bwd_saved (the same
kernels with pool scratch), through the C ABI (needs an MI355X).  The two
must agree bit for bit: two calls in a row, the second smaller than the
first, so that nothing the first left in the shared array can leak into the
second's gradients."""
import numpy as np
import pytest
import torch

from selective_state_space_65_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def compare(shape, io, seed):
    b, d, n, l = shape
    x = inputs.make_scan_inputs(b, d, n, l, io=io, seed=seed)
    t = inputs.to_torch(x, DEV)
    dy = torch.from_numpy(inputs.grad_output(x, seed=seed + 1)).to(DEV, t["u"].dtype)
    dlast = torch.from_numpy(np.random.default_rng([seed, 2]).standard_normal((b, d, n)).astype(np.float32)).to(DEV)
    fw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True)
    _, _, ck = binding.scan_fwd_save(t["u"], t["delta"], t["A"], t["B"], t["C"], **fw)
    ref = binding.scan_bwd_saved(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, ck, dlast=dlast, **fw)
    got = binding.scan_bwd_saved_noalloc(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, ck, dlast=dlast, **fw)
    torch.cuda.synchronize()
    for k, v in ref.items():
        if v is None:
            assert got[k] is None, k
            continue
        assert torch.equal(got[k], v), "%s %s: %s differs" % (shape, io, k)


def test_noalloc_backward_two_calls_second_smaller():
    say("no-alloc backward: Mamba-130M layer (8x1536x16x2048 fp32, 49 MiB of scratch)")
    compare((8, 1536, 16, 2048), "f32", 5100)
    say("no-alloc backward: then 3x200x8x264 bf16")
    compare((3, 200, 8, 264), "bf16", 5200)
