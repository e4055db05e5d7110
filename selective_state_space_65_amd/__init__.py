"""MI355X (gfx950) selective state-space scan (S6).

The compute lives in libssm_scan.so (HIP kernels behind a C ABI, see
include/ssm_scan.h); `scan_fwd`, `conv_scan_fwd`, `scan_bwd`, `conv_bwd`,
`state_update` and their variants are the ctypes wrappers.
The binding is imported lazily so that `inputs` (the seeded synthetic-input
generators) can be used without the library.
"""

__all__ = ["scan_fwd", "scan_fwd_ex", "scan_fwd_complex", "conv_scan_fwd", "scan_bwd", "conv_bwd", "state_update",
           "state_update_ex", "state_update_complex", "scan_fwd_save", "scan_bwd_saved", "scan_bwd_ex", "scan_bwd_complex",
           "ckpt_shape", "scan_plan", "SsmError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
