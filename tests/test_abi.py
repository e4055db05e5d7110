"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid calls on the host before any HIP call (no compute here)."""
import ctypes
import os
import re

import pytest

from selective_state_space_65_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_state_update", "ssm_scan_fwd_plan", "ssm_status_string", "ssm_abi_version",
              "ssm_last_hip_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(binding.SIGNATURES)


def test_abi_version(lib):
    m = re.search(r"#define SSM_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.ssm_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(10):
        s = lib.ssm_status_string(code)
        assert s and s != b"unknown status"
    assert lib.ssm_status_string(99) == b"unknown status"


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        binding.load_library(str(tmp_path / "nope.so"))


# Fake, never-dereferenced device addresses: every call below fails validation
# on the host, before the library touches HIP.
BASE = 1 << 40


def addr(k):
    return BASE + k * (1 << 32)


def fwd(lib, batch=2, dim=8, dstate=4, seqlen=16, io=0, **over):
    args = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
                sp=1, h0=addr(9), y=addr(10), last=addr(11))
    args.update(over)
    return lib.ssm_scan_fwd(batch, dim, dstate, seqlen, io, args["u"], args["delta"], args["A"], args["B"],
                            args["C"], args["D"], args["z"], args["bias"], args["sp"], args["h0"], args["y"],
                            args["last"], None)


def upd(lib, batch=2, dim=8, dstate=4, io=0, **over):
    args = dict(state=addr(1), u=addr(2), delta=addr(3), A=addr(4), B=addr(5), C=addr(6), D=addr(7), z=addr(8),
                bias=addr(9), sp=1, y=addr(10))
    args.update(over)
    return lib.ssm_state_update(batch, dim, dstate, io, args["state"], args["u"], args["delta"], args["A"],
                                args["B"], args["C"], args["D"], args["z"], args["bias"], args["sp"], args["y"], None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "y"])
def test_scan_null_required(lib, field):
    assert fwd(lib, **{field: None}) == 1  # SSM_ERR_NULL


@pytest.mark.parametrize("sizes", [dict(batch=0), dict(dim=0), dict(seqlen=0), dict(dstate=0), dict(batch=-3),
                                   dict(batch=1 << 40, dim=1 << 30)])
def test_scan_bad_sizes(lib, sizes):
    assert fwd(lib, **sizes) == 2  # SSM_ERR_SHAPE


def test_scan_dstate_too_large(lib):
    assert fwd(lib, dstate=17) == 3


def test_scan_bad_dtype(lib):
    assert fwd(lib, io=7) == 4


def test_scan_misaligned(lib):
    assert fwd(lib, u=addr(1) + 2) == 5  # fp32 needs 4-byte alignment
    assert fwd(lib, io=1, u=addr(1) + 1) == 5  # bf16 needs 2-byte alignment
    assert fwd(lib, A=addr(3) + 2) == 5


def test_scan_aliasing(lib):
    assert fwd(lib, y=addr(1) + 64) == 6            # y inside u
    assert fwd(lib, y=addr(5)) == 6                 # y on C
    assert fwd(lib, last=addr(1)) == 6              # last_state on u
    assert fwd(lib, last=addr(9) + 16) == 6         # last_state overlapping h0 but not equal to it


def test_update_validation(lib):
    assert upd(lib, state=None) == 1
    assert upd(lib, y=None) == 1
    assert upd(lib, dim=0) == 2
    assert upd(lib, dstate=32) == 3
    assert upd(lib, io=5) == 4
    assert upd(lib, state=addr(1) + 1) == 5
    assert upd(lib, y=addr(1)) == 6                 # y on the state
    assert upd(lib, state=addr(2)) == 6             # state on u


def fwd_ex(lib, disc, batch=2, dim=8, dstate=4, seqlen=16, io=0, **over):
    args = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
                sp=1, h0=addr(9), y=addr(10), last=addr(11))
    args.update(over)
    return lib.ssm_scan_fwd_ex(batch, dim, dstate, seqlen, io, disc, args["u"], args["delta"], args["A"], args["B"],
                               args["C"], args["D"], args["z"], args["bias"], args["sp"], args["h0"], args["y"],
                               args["last"], None)


def upd_ex(lib, disc, batch=2, dim=8, dstate=4, io=0, **over):
    args = dict(state=addr(1), u=addr(2), delta=addr(3), A=addr(4), B=addr(5), C=addr(6), D=addr(7), z=addr(8),
                bias=addr(9), sp=1, y=addr(10))
    args.update(over)
    return lib.ssm_state_update_ex(batch, dim, dstate, io, disc, args["state"], args["u"], args["delta"], args["A"],
                                   args["B"], args["C"], args["D"], args["z"], args["bias"], args["sp"], args["y"],
                                   None)


def test_ex_validation(lib):
    for disc in (0, 1):
        assert fwd_ex(lib, disc, u=None) == 1
        assert fwd_ex(lib, disc, seqlen=0) == 2
        assert fwd_ex(lib, disc, dstate=17) == 3
        assert fwd_ex(lib, disc, io=3) == 4
        assert fwd_ex(lib, disc, A=addr(3) + 2) == 5
        assert fwd_ex(lib, disc, y=addr(5)) == 6
        assert upd_ex(lib, disc, state=None) == 1
        assert upd_ex(lib, disc, dstate=20) == 3
        assert upd_ex(lib, disc, y=addr(1)) == 6
    for disc in (2, -1, 99):   # not an ssm_disc_t value; otherwise valid calls
        assert fwd_ex(lib, disc) == 8
        assert upd_ex(lib, disc) == 8


def cplx(lib, batch=2, dim=8, dstate=4, seqlen=16, io=0, **over):
    args = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
                sp=1, h0=addr(9), y=addr(10), last=addr(11))
    args.update(over)
    return lib.ssm_scan_fwd_complex(batch, dim, dstate, seqlen, io, args["u"], args["delta"], args["A"], args["B"],
                                    args["C"], args["D"], args["z"], args["bias"], args["sp"], args["h0"], args["y"],
                                    args["last"], None)


def test_complex_validation(lib):
    assert cplx(lib, u=None) == 1
    assert cplx(lib, dstate=0) == 2
    assert cplx(lib, dstate=9) == 3            # above 16 real numbers per channel
    assert cplx(lib, dstate=1 << 62) == 3
    assert cplx(lib, io=9) == 4
    assert cplx(lib, B=addr(4) + 2) == 5
    assert cplx(lib, y=addr(2) + 8) == 6
    # A is (dim, dstate, 2): last_state overlapping A's second half is an alias.
    assert cplx(lib, last=addr(3) + 8 * 4 * 4) == 6
    # (Every valid shape runs: the other complex shapes are tested on the GPU.)


def cupd(lib, batch=2, dim=8, dstate=4, io=0, **over):
    args = dict(state=addr(1), u=addr(2), delta=addr(3), A=addr(4), B=addr(5), C=addr(6), D=addr(7), z=addr(8),
                bias=addr(9), sp=1, y=addr(10))
    args.update(over)
    return lib.ssm_state_update_complex(batch, dim, dstate, io, args["state"], args["u"], args["delta"], args["A"],
                                        args["B"], args["C"], args["D"], args["z"], args["bias"], args["sp"], args["y"],
                                        None)


def test_complex_update_validation(lib):
    assert cupd(lib, state=None) == 1
    assert cupd(lib, dim=0) == 2
    assert cupd(lib, dstate=9) == 3
    assert cupd(lib, io=4) == 4
    assert cupd(lib, A=addr(4) + 1) == 5
    assert cupd(lib, y=addr(1) + 64) == 6            # y inside the state (2 x 8 x 4 x 2 floats)
    assert cupd(lib, u=addr(1) + 2 * 8 * 4 * 2 * 4 - 4) == 6   # u overlapping the state's last float


def test_saved_checkpoint_validation(lib):
    nb = ctypes.c_int64(0)
    assert lib.ssm_scan_ckpt_bytes(2, 8, 4, 33, 0, ctypes.byref(nb)) == 0
    assert nb.value == 3 * 2 * 4 * 8 * 4                      # ceil(33/16) tiles x batch x dstate x dim floats
    assert lib.ssm_scan_ckpt_bytes(2, 8, 17, 33, 0, None) == 3
    assert lib.ssm_scan_ckpt_bytes(0, 8, 4, 33, 0, None) == 2

    def save(**over):
        args = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
                    h0=None, y=addr(10), last=addr(11), ck=addr(12), seqlen=16, dstate=4)
        args.update(over)
        return lib.ssm_scan_fwd_save(2, 8, args["dstate"], args["seqlen"], 0, args["u"], args["delta"], args["A"],
                                     args["B"], args["C"], args["D"], args["z"], args["bias"], 1, args["h0"], args["y"],
                                     args["last"], args["ck"], None)
    assert save(ck=None) == 1
    assert save(ck=addr(12) + 2) == 5
    assert save(ck=addr(1) + 16) == 6          # checkpoints inside u
    assert save(ck=addr(10)) == 6              # checkpoints on y
    assert save(dstate=5) == 8                 # outside the single-pass kernel
    assert save(seqlen=12) == 8

    def saved(**over):
        args = dict(ck=addr(12), dy=addr(13), du=addr(14), dd=addr(15), dA=addr(16), dB=addr(17), dC=addr(18))
        args.update(over)
        return lib.ssm_scan_bwd_saved(2, 8, 4, 16, 0, addr(1), addr(2), addr(3), addr(4), addr(5), None, None, None, 1,
                                      args["ck"], args["dy"], None, args["du"], args["dd"], args["dA"], args["dB"],
                                      args["dC"], None, None, None, None, None)
    assert saved(ck=None) == 1
    assert saved(ck=addr(12) + 1) == 5
    assert saved(du=addr(12)) == 6             # an output on the checkpoints


def test_bwd_ex_validation(lib):
    def call(disc, **over):
        args = dict(u=addr(1), dy=addr(13), du=addr(14), dd=addr(15), dA=addr(16), dB=addr(17), dC=addr(18))
        args.update(over)
        return lib.ssm_scan_bwd_ex(2, 8, 4, 16, 0, disc, args["u"], addr(2), addr(3), addr(4), addr(5), None, None, None,
                                   1, None, args["dy"], None, args["du"], args["dd"], args["dA"], args["dB"],
                                   args["dC"], None, None, None, None, None)
    assert call(1, u=None) == 1
    assert call(1, du=addr(1)) == 6
    for disc in (2, -1):
        assert call(disc) == 8


def test_bwd_complex_validation(lib):
    def call(**over):
        args = dict(batch=2, dstate=4, seqlen=16, u=addr(1), du=addr(14), dA=addr(16))
        args.update(over)
        return lib.ssm_scan_bwd_complex(args["batch"], 8, args["dstate"], args["seqlen"], 0, args["u"], addr(2), addr(3),
                                        addr(4), addr(5), None, None, None, 1, None, addr(13), None, args["du"],
                                        addr(15), args["dA"], addr(17), addr(18), None, None, None, None, None)
    assert call(u=None) == 1
    assert call(dstate=9) == 3
    assert call(dstate=0) == 2
    assert call(dstate=3) == 8                  # complex backward: 4 or 8 complex states
    assert call(seqlen=12) == 8
    assert call(du=addr(1)) == 6
    assert call(dA=addr(3) + 8) == 6            # dA on A (dim x dstate x 2 floats)


def cfwd(lib, batch=2, dim=8, dstate=4, seqlen=16, width=4, io=0, **over):
    args = dict(x=addr(1), w=addr(12), cb=addr(13), xp=addr(14), silu=1, delta=addr(2), A=addr(3), B=addr(4),
                C=addr(5), D=addr(6), z=addr(7), bias=addr(8), sp=1, h0=addr(9), y=addr(10), last=addr(11),
                uo=addr(15))
    args.update(over)
    return lib.ssm_conv_scan_fwd(batch, dim, dstate, seqlen, width, io, args["x"], args["w"], args["cb"], args["xp"],
                                 args["silu"], args["delta"], args["A"], args["B"], args["C"], args["D"], args["z"],
                                 args["bias"], args["sp"], args["h0"], args["y"], args["last"], args["uo"], None)


def cbwd(lib, batch=2, dim=8, seqlen=16, width=4, io=0, **over):
    args = dict(x=addr(1), w=addr(2), cb=addr(3), xp=addr(4), silu=1, du=addr(5), dx=addr(6), dw=addr(7), db=addr(8),
                dxp=addr(9))
    args.update(over)
    return lib.ssm_conv_bwd(batch, dim, seqlen, width, io, args["x"], args["w"], args["cb"], args["xp"], args["silu"],
                            args["du"], args["dx"], args["dw"], args["db"], args["dxp"], None)


@pytest.mark.parametrize("field", ["x", "w", "du", "dx", "dw"])
def test_conv_bwd_null_required(lib, field):
    assert cbwd(lib, **{field: None}) == 1


def test_conv_bwd_validation(lib):
    assert cbwd(lib, width=0) == 2
    assert cbwd(lib, width=5) == 2
    assert cbwd(lib, seqlen=0) == 2
    assert cbwd(lib, batch=1 << 62) == 2                 # sizes that overflow
    assert cbwd(lib, io=7) == 4
    assert cbwd(lib, batch=1, dim=1, seqlen=1 << 30, io=1) == 8   # rows of 2^31 bytes
    assert cbwd(lib, batch=1, dim=1, seqlen=1 << 29, io=0) == 8
    assert cbwd(lib, dx=addr(6) + 2) == 5               # fp32 dx needs 4-byte alignment
    assert cbwd(lib, io=1, xp=addr(4) + 1) == 5         # bf16 x_prev needs 2-byte alignment
    assert cbwd(lib, dw=addr(7) + 2) == 5
    assert cbwd(lib, dx=addr(1)) == 6                   # dx on x
    assert cbwd(lib, dx=addr(5) + 4) == 6               # dx overlapping du
    assert cbwd(lib, dw=addr(2) + 4) == 6               # dconv_weight overlapping conv_weight
    assert cbwd(lib, db=addr(6)) == 6                   # two outputs on one buffer
    assert cbwd(lib, dxp=addr(4)) == 6                  # dx_prev on x_prev


@pytest.mark.parametrize("field", ["x", "w", "delta", "A", "B", "C", "y"])
def test_conv_scan_null_required(lib, field):
    assert cfwd(lib, **{field: None}) == 1


@pytest.mark.parametrize("width", [0, 5, -1])
def test_conv_scan_bad_width(lib, width):
    assert cfwd(lib, width=width) == 2


def test_conv_scan_misaligned_and_aliasing(lib):
    assert cfwd(lib, xp=addr(14) + 2) == 5          # fp32 x_prev needs 4-byte alignment
    assert cfwd(lib, w=addr(12) + 2) == 5
    assert cfwd(lib, io=1, uo=addr(15) + 1) == 5    # bf16 u_out needs 2-byte alignment
    assert cfwd(lib, uo=addr(1)) == 6               # u_out on x
    assert cfwd(lib, uo=addr(10)) == 6              # u_out on y
    assert cfwd(lib, uo=addr(11)) == 6              # u_out on last_state
    assert cfwd(lib, y=addr(12)) == 6               # y on the conv weights
    assert cfwd(lib, y=addr(14)) == 6               # y on x_prev
    assert cfwd(lib, last=addr(13)) == 6            # last_state on the conv bias


def bwd(lib, batch=2, dim=8, dstate=4, seqlen=16, io=0, **over):
    args = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8), sp=1,
                h0=addr(9), dy=addr(10), dlast=addr(11), du=addr(20), ddelta=addr(21), dA=addr(22), dB=addr(23),
                dC=addr(24), dD=addr(25), dz=addr(26), dbias=addr(27), dh0=addr(28))
    args.update(over)
    return lib.ssm_scan_bwd(batch, dim, dstate, seqlen, io, args["u"], args["delta"], args["A"], args["B"], args["C"],
                            args["D"], args["z"], args["bias"], args["sp"], args["h0"], args["dy"], args["dlast"],
                            args["du"], args["ddelta"], args["dA"], args["dB"], args["dC"], args["dD"], args["dz"],
                            args["dbias"], args["dh0"], None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "dy", "du", "ddelta", "dA", "dB", "dC"])
def test_bwd_null_required(lib, field):
    assert bwd(lib, **{field: None}) == 1


def test_bwd_validation(lib):
    assert bwd(lib, dstate=0) == 2
    assert bwd(lib, dstate=17) == 3
    assert bwd(lib, io=3) == 4
    assert bwd(lib, dy=addr(10) + 2) == 5             # fp32 dy needs 4-byte alignment
    assert bwd(lib, dB=addr(23) + 1) == 5
    assert bwd(lib, du=addr(1)) == 6                  # du on u
    assert bwd(lib, dA=addr(3) + 4) == 6              # dA overlapping A
    assert bwd(lib, dz=addr(20)) == 6                 # two outputs on one buffer
    assert bwd(lib, dh0=addr(11)) == 6                # dh0 on dlast
    assert bwd(lib, dstate=5) == 8                    # valid, but the backward takes dstate 4, 8, 16 only
    assert bwd(lib, seqlen=20) == 8                   # ... and seqlen a multiple of 8
    assert bwd(lib, u=addr(1) + 4) == 8               # ... and 16-byte aligned rows
    assert bwd(lib, batch=1, dim=1, seqlen=1 << 25, io=1) == 8   # ... and rows under 2^26 bytes (bf16)
    assert bwd(lib, batch=1, dim=1, seqlen=1 << 24) == 8         # (fp32)


def test_plan(lib):
    import torch
    path, seg, seglen, scratch = binding.scan_plan(4, 4096, 16, 4096, torch.bfloat16, with_path=True)
    assert (path, seg, seglen, scratch) == ("split", 1, 4096, 0)          # Mamba-1.4B layer: single pass
    assert binding.scan_plan(8, 1536, 16, 2048, torch.float32, with_path=True) == ("split", 1, 2048, 0)
    # Long sequence: the chunked kernel at dstate 16 (under either
    # discretization, with or without the conv); dstate 8 runs segmented.  No
    # path takes scratch: the segment aggregates and carries live in y.  The
    # last segment ends at seqlen and holds at least 64 tokens.
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True) == ("chunked", 1, 131072, 0)
    assert binding.scan_plan(1, 2560, 16, 131072, torch.bfloat16, with_path=True) == ("chunked", 1, 131072, 0)
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True, conv_width=4)[0] == "chunked"
    assert binding.scan_plan(1, 2560, 16, 131072, torch.float32, with_path=True, disc="zoh")[0] == "chunked"
    path, seg, seglen, scratch = binding.scan_plan(1, 2560, 8, 131072, torch.float32, with_path=True, conv_width=4)
    assert path == "segmented" and seg > 1 and scratch == 0
    assert (seg - 1) * seglen < 131072 and 131072 - (seg - 1) * seglen >= 64
    path, seg, seglen, scratch = binding.scan_plan(1, 64, 16, 4097, torch.float32, with_path=True)
    assert path == "generic" and seg == 16 and seglen == 256 and scratch == 0   # a 1-token remainder joins segment 15
    assert seglen % 64 == 0
    assert binding.scan_plan(1, 16, 4, 64, torch.float32, with_path=True) == ("segmented", 1, 64, 0)
    assert binding.scan_plan(1, 16, 4, 63, torch.float32, with_path=True)[0] == "generic"
    assert binding.scan_plan(256, 64, 5, 64, torch.float32, with_path=True)[0] == "generic"
    assert binding.scan_plan(2, 8, 16, 16, torch.float32) == (1, 16, 0)
    path, seg = ctypes.c_int(), ctypes.c_int64()
    for disc, width in ((2, 0), (-1, 0), (0, 5), (0, -1)):
        st = lib.ssm_scan_fwd_plan_ex(1, 64, 16, 64, 0, disc, width, ctypes.byref(path), ctypes.byref(seg), None, None)
        assert st == 8   # SSM_ERR_UNSUPPORTED


def test_product_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "selective_state_space_65_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "ssm_oracle" not in text and "oracle_scan" not in text, f


def test_noalloc_backward_limit(lib):
    """ssm_scan_bwd_saved_noalloc refuses, on the host, a call whose scratch exceeds
    its fixed 64 MiB device array (the Mamba-1.4B layer: 129 MiB); its other checks
    are ssm_scan_bwd_saved's."""
    big = 1 << 36  # far-apart fake addresses: the arrays of a large call must not overlap

    def call(batch, dim, dstate, seqlen, ck=True):
        a = [big * (k + 1) for k in range(20)]
        return lib.ssm_scan_bwd_saved_noalloc(batch, dim, dstate, seqlen, 1, a[1], a[2], a[3], a[4], a[5], None, None,
                                              None, 1, a[12] if ck else None, a[13], None, a[14], a[15], a[16], a[17],
                                              a[18], None, None, None, None, None)
    assert call(4, 4096, 16, 4096) == 9                  # SSM_ERR_WORKSPACE
    assert lib.ssm_status_string(9).startswith(b"the call needs more scratch")
    assert call(4, 4096, 16, 4096, ck=False) == 1        # SSM_ERR_NULL first
    assert call(0, 4096, 16, 4096) == 2
    assert call(4, 4096, 5, 4096) == 8                   # outside the backward kernel, as ssm_scan_bwd_saved
