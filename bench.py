#!/usr/bin/env python3
"""Selective-scan benchmark on one MI355X.

One step = one ssm_scan_fwd call over the Mamba-1.4B-layer workload (batch 4,
dim 4096, dstate 16, seqlen 4096; u, delta, z, B, C, y in bf16; A, D, bias and
the state in fp32; gate and softplus on), with inputs resident in HBM before
the timed region.  Prints one JSON line:

  value        whole-job HBM throughput, algorithmic bytes / wall time per step (GB/s)
  roofline     the scan call against its binding roof (see below), timed with
               HIP events on the launch stream
  cpu_baseline the fp64 oracle on the host cores, on a bounded sample of the
               same workload
  decode       the one-token state update at the decode workload (batch 256,
               dim 5120, dstate 16), per step
  conv_scan    ssm_conv_scan_fwd (causal conv of width 4 fused in front of the
               scan) on the same workload, and its backward ssm_conv_bwd
  zoh          ssm_scan_fwd_ex with exact zero-order hold for B, same workload
  complex      ssm_scan_fwd_complex, 8 complex states (16 real numbers per channel)
  backward     ssm_scan_bwd (every gradient) on the same workload

Algorithmic bytes: read u, delta, z and write y once (4 x io bytes per
element), read B and C once per (batch, token), read A, D and the bias once,
write the final state once.  The (batch, dim, seqlen, dstate) expanded state
is not counted: the method never stores it.

roofline: HBM is the roof the line is measured against: frac = algorithmic
bytes / call time / 8 TB/s.  The path is in fact bound by plain ALU issue:
each (element, state) needs one exp2 and four fp32 VALU operations (Delta*A,
B*x, the state FMA and the C.h FMA).  The rate probe (csrc/rate_probe.hip)
measures on the GPU at hand how many FMA issue slots an exp2 and the scan's
per-(element, state) body take; alu_frac is the call's (element, state) rate
against 256 CU x 64 lanes x 2.4 GHz = 39.3 T lane-slots/s at that cost.

configs: the Mamba-130M-layer (fp32) and long-sequence (fp32) workloads
timed the same way, one call per step.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "selective-scan HBM GB/s (% of MI355X peak) + (B·D·L)/s at Mamba-1.4B shape"

# HBM bytes per call of the scan workloads measured with rocprofv3
# (FETCH_SIZE and WRITE_SIZE scaled by the factors a 1 GiB copy gives these
# counters in the same run), valid only for the kernel sources they were
# measured on (KERNEL_SOURCES, hashed together): when one changes, the figures
# are reported as null until re-measured.  Keys are the workload indices of
# inputs.scan_config.
MEASURED_TRAFFIC = {
    "source_sha256": "27d2d2e89572f694b958218bb97a4d41aa195019fa91a2aecfdf45075c6e62f0",
    "per_call": {
        2: {"read_bytes": 481_076_329, "write_bytes": 137_641_344},
        1: {"read_bytes": 359_579_236, "write_bytes": 103_075_296},
        3: {"read_bytes": 4_183_883_467, "write_bytes": 1_353_745_008},
    },
}
HBM_PEAK_GBS = 8000.0
LANE_SLOTS_PEAK = 256 * 64 * 2.4e9  # fp32 VALU lane-slots per second
SLOTS_PER_ELEM_STATE = 6            # exp2 (2 slots, half rate) + 4 fp32 ops


KERNELS = {"split": "scan_split_kernel", "segmented": "aggregate_kernel + carry_kernel + scan_kernel",
           "generic": "scan_kernel (per-token)", "chunked": "scan_chunked_kernel"}


def algorithmic_bytes(batch, dim, dstate, seqlen, io_bytes, has_z=True, has_h0=False):
    streams = (4 if has_z else 3) * batch * dim * seqlen * io_bytes      # u, delta, (z) in, y out
    bc = 2 * batch * dstate * seqlen * io_bytes
    params = dim * dstate * 4 + 2 * dim * 4
    state = batch * dim * dstate * 4 * (2 if has_h0 else 1)
    return streams + bc + params + state


def decode_bytes(batch, dim, dstate, io_bytes):
    return (2 * batch * dim * dstate * 4 + 4 * batch * dim * io_bytes + 2 * batch * dstate * io_bytes
            + dim * dstate * 4 + 2 * dim * 4)


KERNEL_SOURCES = ("ssm_scan.hip", "scan_chunked.hip", "device_common.h")


def kernel_source_digest():
    """sha256 over the kernel sources (csrc/, in KERNEL_SOURCES order)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "selective_state_space_65_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_traffic(config):
    """Counter-measured HBM bytes per call (read + written), or None if the
    kernel sources changed since the measurement or the workload has none."""
    digest = kernel_source_digest()
    m = MEASURED_TRAFFIC
    if digest != m["source_sha256"] or config not in m["per_call"]:
        return None
    return m["per_call"][config]["read_bytes"] + m["per_call"][config]["write_bytes"]


def cpu_cores():
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, budget_s, one_thread_s=5.0):
    """Time the fp64 oracle on whole batch rows of the workload until budget_s has elapsed,
    then on one thread over a slice of channels of batch row 0."""
    import numpy as np
    import oracle
    b, d, n, l = x.shape
    o = oracle.default()
    io_bytes = 2 if x.io == "bf16" else 4
    cores = cpu_cores()
    oracle.set_threads(cores)
    done = 0
    spent = 0.0
    rows = 0
    for bi in range(b):
        sl = slice(bi, bi + 1)
        args = [np.ascontiguousarray(a[sl], dtype=np.float64) for a in (x.u, x.delta, x.B, x.C, x.z)]
        t0 = time.perf_counter()
        o.scan_f64(args[0], args[1], x.A, args[2], args[3], x.D, args[4], x.delta_bias, x.softplus, None)
        spent += time.perf_counter() - t0
        done += d * l
        rows += 1
        if spent >= budget_s:
            break
    gbs = algorithmic_bytes(rows, d, n, l, io_bytes) / spent / 1e9
    out = dict(value=round(gbs, 3), unit="GB/s", cores=cores, kind="oracle", cpu_model=cpu_model(),
               sample="%d of %d batch rows (%d channels x %d tokens, dstate %d), fp64, OpenMP over channels"
               % (rows, b, rows * d, l, n), seconds=round(spent, 3), elements_per_s=round(done / spent, 1))
    # One thread: channels of batch row 0, 64 at a time, until one_thread_s has elapsed.
    oracle.set_threads(1)
    spent1, ch1 = 0.0, 0
    try:
        while ch1 < d and spent1 < one_thread_s:
            cs = slice(ch1, min(d, ch1 + 64))
            args = [np.ascontiguousarray(a[0:1, cs], dtype=np.float64) for a in (x.u, x.delta, x.z)]
            t0 = time.perf_counter()
            o.scan_f64(args[0], args[1], x.A[cs], np.ascontiguousarray(x.B[0:1], dtype=np.float64),
                       np.ascontiguousarray(x.C[0:1], dtype=np.float64), x.D[cs], args[2], x.delta_bias[cs],
                       x.softplus, None)
            spent1 += time.perf_counter() - t0
            ch1 += cs.stop - cs.start
    finally:
        oracle.set_threads(cores)
    el1 = ch1 * l
    out["one_thread"] = dict(elements_per_s=round(el1 / spent1, 1), seconds=round(spent1, 3),
                             sample="%d channels x %d tokens of batch row 0" % (ch1, l),
                             gbs=round(el1 * (4 * io_bytes) / spent1 / 1e9, 4))
    return out


def time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return wall / steps * 1e3, sum(per) / len(per), per[len(per) // 2]


def bench_decode(dev, steps, warmup):
    import torch
    from selective_state_space_65_amd import binding, inputs
    dec = inputs.decode_config()
    st = dec.step(0)
    state = torch.from_numpy(dec.state0).to(dev)
    A = torch.from_numpy(dec.A).to(dev)
    D = torch.from_numpy(dec.D).to(dev)
    bias = torch.from_numpy(dec.delta_bias).to(dev)
    tt = {k: torch.from_numpy(v).to(dev, torch.bfloat16) for k, v in st.items()}
    y = torch.empty_like(tt["u"])

    def fn():
        binding.state_update(state, tt["u"], tt["delta"], A, tt["B"], tt["C"], D=D, z=tt["z"], delta_bias=bias,
                             delta_softplus=True, out=y)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    # A decode loop as a serving stack would run it: GRAPH_STEPS consecutive
    # steps, each reading its own staged input slot, captured once in a HIP
    # graph and replayed (no host launch between steps).  The state is
    # updated in place by every step, as in the loop.
    graph_us = loop_us = None
    GRAPH_STEPS = 16
    try:
        slots = []
        for j in range(GRAPH_STEPS):
            sj = dec.step(j + 1)
            slots.append({k: torch.from_numpy(v).to(dev, torch.bfloat16) for k, v in sj.items()})
        ys = [torch.empty_like(y) for _ in range(GRAPH_STEPS)]

        def loop():
            for j in range(GRAPH_STEPS):
                sl = slots[j]
                binding.state_update(state, sl["u"], sl["delta"], A, sl["B"], sl["C"], D=D, z=sl["z"],
                                     delta_bias=bias, delta_softplus=True, out=ys[j])

        # The same 16 slots launched one by one: the like-for-like baseline
        # of the replay (16 staged input sets do not stay in the caches the
        # way the single set above does).
        reps = max(2, steps // GRAPH_STEPS)
        loop()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            loop()
        e1.record()
        torch.cuda.synchronize()
        loop_us = round(e0.elapsed_time(e1) / (reps * GRAPH_STEPS) * 1e3, 2)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            loop()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = round(e0.elapsed_time(e1) / (reps * GRAPH_STEPS) * 1e3, 2)
        del slots, ys
    except RuntimeError:
        graph_us = None
    nbytes = decode_bytes(dec.batch, dec.dim, dec.dstate, 2)
    return dict(workload="decode state update, batch %d, dim %d, dstate %d, bf16 io, fp32 state"
                % (dec.batch, dec.dim, dec.dstate), us_per_step=round(avg_ms * 1e3, 2),
                graph_replay_us_per_step=graph_us, graph_steps_per_replay=GRAPH_STEPS,
                staged_loop_us_per_step=loop_us,
                effective_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1), bytes_per_step=nbytes,
                note="algorithmic bytes per step / step time; the 84 MB state fits in the 256 MB Infinity "
                     "Cache, which sits behind the L2 and may serve part of it, so this is not pure HBM traffic")


def bench_conv_scan(dev, x, t, steps, warmup):
    """ssm_conv_scan_fwd on the same workload with u replaced by the conv input x
    (width 4, bias and silu on, no history): the conv rides in the scan's prologue."""
    import torch
    from selective_state_space_65_amd import binding, inputs
    b, d, n, l = x.shape
    w, cb = inputs.conv_params(d, 4)
    wt, cbt = torch.from_numpy(w).to(dev), torch.from_numpy(cb).to(dev)
    y = torch.empty_like(t["u"])
    last = torch.empty((b, d, n), dtype=torch.float32, device=dev)

    def fn():
        binding.conv_scan_fwd(t["u"], wt, t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                              delta_bias=t["delta_bias"], delta_softplus=x.softplus, conv_bias=cbt, conv_silu=True,
                              out=y, last_state=last)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    io_bytes = 2 if x.io == "bf16" else 4
    nbytes = algorithmic_bytes(b, d, n, l, io_bytes, has_z=x.z is not None) + d * 4 * 4 + d * 4
    out = dict(workload="causal conv (width 4, bias, silu) fused in front of the scan, same shape",
               us_per_call=round(avg_ms * 1e3, 2), us_median=round(med_ms * 1e3, 2),
               algorithmic_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1), algorithmic_bytes=nbytes)

    # Its backward (ssm_conv_bwd) for dL/du = the scan backward's du: read x and
    # du, write dx (3 io values per element); the filter, bias and their
    # gradients are a few KB.
    du = torch.from_numpy(inputs.grad_output(x)).to(dev, t["u"].dtype)

    def bwd():
        binding.conv_bwd(t["u"], wt, du, conv_bias=cbt, conv_silu=True)

    _, b_ms, b_med = time_calls(bwd, steps, warmup)
    bbytes = 3 * b * d * l * io_bytes + 2 * (d * 4 * 4 + d * 4)
    out["backward"] = dict(workload="ssm_conv_bwd: dx, dconv_weight, dconv_bias, same shape",
                           us_per_call=round(b_ms * 1e3, 2), us_median=round(b_med * 1e3, 2),
                           algorithmic_gbs=round(bbytes / (b_ms * 1e-3) / 1e9, 1), algorithmic_bytes=bbytes,
                           hbm_frac=round(bbytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    return out


ZOH_SLOTS_PER_ELEM_STATE = 14  # the 6 of the Delta*B rule + u/A, the series (3 FMAs, 1 mul), e*iu - iu, select (2)


def bench_zoh(dev, x, t, steps, warmup):
    """ssm_scan_fwd_ex with exact zero-order hold for B on the same workload."""
    import torch
    from selective_state_space_65_amd import binding
    b, d, n, l = x.shape
    y = torch.empty_like(t["u"])
    last = torch.empty((b, d, n), dtype=torch.float32, device=dev)

    def fn():
        binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                            delta_softplus=x.softplus, disc="zoh", out=y, last_state=last)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    io_bytes = 2 if x.io == "bf16" else 4
    nbytes = algorithmic_bytes(b, d, n, l, io_bytes, has_z=x.z is not None)
    slots = ZOH_SLOTS_PER_ELEM_STATE * b * d * l * n
    return dict(workload="exact zero-order hold for B (ssm_scan_fwd_ex), same shape and flags",
                us_per_call=round(avg_ms * 1e3, 2), us_median=round(med_ms * 1e3, 2),
                algorithmic_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1),
                alu_frac=round(slots / (avg_ms * 1e-3) / LANE_SLOTS_PEAK, 4),
                lane_slots_per_elem_state=ZOH_SLOTS_PER_ELEM_STATE)


# Per (element, complex state): Delta Re A, exp2 (2), Delta Im A, fract, cos (2), sin (2), the two Abar
# products, Delta u times Re B and Im B, four FMAs of the complex update, two for Re(C h).
CPLX_SLOTS_PER_ELEM_STATE = 19


def bench_complex(dev, x, t, steps, warmup):
    """ssm_scan_fwd_complex on the same shape with 8 complex states (16 real numbers per channel, as the
    real workload's 16 states): A = -1/2 + i pi n, B and C with N(0, 1) real and imaginary parts."""
    import numpy as np
    import torch
    from selective_state_space_65_amd import binding, inputs
    b, d, n, l = x.shape
    nc = n // 2
    rng = np.random.default_rng(inputs.SEED_BASE + 30)
    k = np.arange(nc, dtype=np.float32)
    A = np.stack([np.full((d, nc), -0.5, np.float32), np.broadcast_to(np.float32(np.pi) * k, (d, nc))], -1)
    B = rng.standard_normal((b, nc, l, 2)).astype(np.float32)
    C = rng.standard_normal((b, nc, l, 2)).astype(np.float32)
    At = torch.from_numpy(np.ascontiguousarray(A)).to(dev)
    Bt = torch.from_numpy(B).to(dev, t["u"].dtype)
    Ct = torch.from_numpy(C).to(dev, t["u"].dtype)
    y = torch.empty_like(t["u"])
    last = torch.empty((b, d, nc, 2), dtype=torch.float32, device=dev)

    def fn():
        binding.scan_fwd_complex(t["u"], t["delta"], At, Bt, Ct, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                 delta_softplus=x.softplus, out=y, last_state=last)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    io_bytes = 2 if x.io == "bf16" else 4
    nbytes = algorithmic_bytes(b, d, n, l, io_bytes, has_z=x.z is not None) + d * n * 4  # A holds 2 numbers per state
    slots = CPLX_SLOTS_PER_ELEM_STATE * b * d * l * nc
    dy = torch.from_numpy(inputs.grad_output(x)).to(dev, t["u"].dtype)

    def bwd():
        binding.scan_bwd_complex(t["u"], t["delta"], At, Bt, Ct, dy, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                 delta_softplus=x.softplus)

    _, bwd_ms, _ = time_calls(bwd, max(3, steps // 4), 2)
    return dict(workload="complex diagonal A (ssm_scan_fwd_complex), 8 complex states, same shape and flags",
                us_per_call=round(avg_ms * 1e3, 2), us_median=round(med_ms * 1e3, 2),
                algorithmic_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1),
                alu_frac=round(slots / (avg_ms * 1e-3) / LANE_SLOTS_PEAK, 4),
                lane_slots_per_elem_complex_state=CPLX_SLOTS_PER_ELEM_STATE,
                backward_us_per_call=round(bwd_ms * 1e3, 2))


BWD_SLOTS_PER_ELEM_STATE = 20  # 6 for the checkpointing forward + 14 for the adjoint walk


def bench_backward(dev, x, t, steps, warmup):
    """ssm_scan_bwd on the same workload: every gradient of sum(dy * y)."""
    import torch
    from selective_state_space_65_amd import binding, inputs
    b, d, n, l = x.shape
    dy = torch.from_numpy(inputs.grad_output(x)).to(dev, t["u"].dtype)

    def fn():
        binding.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=x.softplus, h0=None)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    io_bytes = 2 if x.io == "bf16" else 4
    el = b * d * l
    # read u, delta, z, dy, B, C (+ A, D, bias); write du, ddelta, dz, dB, dC (fp32), dA, dD, dbias
    nbytes = 4 * el * io_bytes + 2 * b * n * l * io_bytes + d * n * 4 + 2 * d * 4 + 3 * el * io_bytes \
        + 2 * b * n * l * 4 + d * n * 4 + 2 * d * 4
    slots = BWD_SLOTS_PER_ELEM_STATE * el * n
    out = dict(workload="ssm_scan_bwd (every gradient), same shape and flags", us_per_call=round(avg_ms * 1e3, 2),
               us_median=round(med_ms * 1e3, 2), algorithmic_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1),
               algorithmic_bytes=nbytes, alu_frac=round(slots / (avg_ms * 1e-3) / LANE_SLOTS_PEAK, 4),
               lane_slots_per_elem_state=BWD_SLOTS_PER_ELEM_STATE,
               vs_forward=None)
    # A training step with the forward's checkpoints kept for the backward:
    # ssm_scan_fwd_save, then ssm_scan_bwd_saved (no recompute pass).
    from selective_state_space_65_amd import binding as _b
    try:
        y = torch.empty_like(t["u"])
        last = torch.empty((b, d, n), dtype=torch.float32, device=dev)
        ck = torch.empty(_b.ckpt_shape(b, d, n, l), dtype=torch.float32, device=dev)

        def fwd_save():
            binding.scan_fwd_save(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=x.softplus, out=y, last_state=last, ckpt=ck)

        def bwd_saved():
            binding.scan_bwd_saved(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, ck, D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], delta_softplus=x.softplus)

        _, fs_ms, _ = time_calls(fwd_save, steps, warmup)
        _, bs_ms, _ = time_calls(bwd_saved, steps, warmup)
        out["saved_checkpoints"] = dict(fwd_save_us=round(fs_ms * 1e3, 2), bwd_saved_us=round(bs_ms * 1e3, 2),
                                        training_step_us=round((fs_ms + bs_ms) * 1e3, 2),
                                        checkpoint_mb=round(ck.numel() * 4 / 1e6, 1))
    except _b.SsmError as e:
        out["saved_checkpoints"] = dict(skipped=str(e))

    def bwd_zoh():
        binding.scan_bwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, D=t["D"], z=t["z"],
                            delta_bias=t["delta_bias"], delta_softplus=x.softplus, disc="zoh")

    _, z_ms, _ = time_calls(bwd_zoh, steps, warmup)
    out["zoh_us_per_call"] = round(z_ms * 1e3, 2)
    return out


def rate_probe(dev):
    """Issue rates of FMA, exp2 and the scan's per-(element, state) body on this GPU
    (csrc/rate_probe.hip), each probe at 2 and at 8 waves per SIMD."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_65_amd", "librate_probe.so"))
    lib.rate_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.rate_probe_launch.restype = ctypes.c_int
    lib.rate_probe_ops_per_iter.argtypes = [ctypes.c_int]
    lib.rate_probe_ops_per_iter.restype = ctypes.c_int
    names = {0: "fma", 1: "exp2", 2: "scan_body", 3: "exp2_plus_4fma"}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {}
    for waves_per_simd in (2, 8):
        blocks = cus * waves_per_simd  # blocks of 4 waves: one wave per SIMD each
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        rates = {}
        for kind, name in names.items():
            iters = 4000

            def launch():
                rc = lib.rate_probe_launch(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                           ctypes.c_void_p(stream))
                if rc != 0:
                    raise RuntimeError("rate probe launch failed: %d" % rc)

            launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                launch()
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 3 * 1e-3
            ops = blocks * 256 * iters * lib.rate_probe_ops_per_iter(kind)
            rates[name] = ops / sec
        res[waves_per_simd] = rates
    best = {k: max(res[w][k] for w in res) for k in names.values()}
    fma = best["fma"]
    return dict(
        kernel="csrc/rate_probe.hip", compute_units=cus,
        fma_lane_ops_per_s=round(fma, -9), exp2_lane_ops_per_s=round(best["exp2"], -9),
        scan_units_per_s=round(best["scan_body"], -9), exp2_plus_4fma_units_per_s=round(best["exp2_plus_4fma"], -9),
        exp2_cost_in_fma_slots=round(fma / best["exp2"], 3),
        exp2_plus_4fma_cost_in_fma_slots=round(4.0 * fma / (4.0 * best["exp2_plus_4fma"]), 3),
        scan_body_cost_in_fma_slots=round(fma / best["scan_body"], 3),
        implied_clock_ghz=round(fma / (cus * 64) / 1e9, 3),
        per_waves_per_simd={str(w): {k: round(v, -9) for k, v in r.items()} for w, r in res.items()},
        note="costs are FMA issue slots per operation (clock-independent); exp2 does not co-issue with FMA if "
             "exp2_plus_4fma costs 4 + exp2_cost")


def device_copy(dev, nbytes=1 << 30):
    """A plain device-to-device copy of nbytes (torch copy_): the HBM rate a
    streaming kernel reaches on this GPU, beside the 8 TB/s peak."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def fn():
        dst.copy_(src)

    _, avg_ms, med_ms = time_calls(fn, 5, 2)
    del src, dst
    torch.cuda.empty_cache()
    moved = 2 * nbytes
    return dict(bytes_per_copy=moved, us_per_copy=round(avg_ms * 1e3, 1),
                gbs=round(moved / (avg_ms * 1e-3) / 1e9, 1), frac_of_peak=round(moved / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def bench_config(dev, cfg, steps, warmup):
    """One scan workload (fp32 configs 1 and 3) timed call by call with HIP events."""
    import torch
    from selective_state_space_65_amd import binding, inputs
    x = inputs.scan_config(cfg)
    b, d, n, l = x.shape
    io_bytes = 2 if x.io == "bf16" else 4
    t = inputs.to_torch(x, dev)
    y = torch.empty_like(t["u"])
    last = torch.empty((b, d, n), dtype=torch.float32, device=dev)

    def fn():
        binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=x.softplus, h0=None, out=y, last_state=last)

    wall_ms, avg_ms, med_ms = time_calls(fn, steps, warmup)
    nbytes = algorithmic_bytes(b, d, n, l, io_bytes, has_z=x.z is not None)
    path, seg, seglen, scratch = binding.scan_plan(b, d, n, l, t["u"].dtype, with_path=True)
    variants = {}
    if cfg == 3:
        # The same long rows under exact zero-order hold and with the width-4
        # conv (+ silu) fused in front: the other two entry points the
        # one-pass kernel serves.
        def fn_zoh():
            binding.scan_fwd_ex(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                delta_bias=t["delta_bias"], delta_softplus=x.softplus, h0=None, out=y, last_state=last,
                                disc="zoh")

        cw = inputs.conv_params(d, 4)
        cwt = torch.from_numpy(cw[0]).to(dev)
        cbt = torch.from_numpy(cw[1]).to(dev)

        def fn_conv():
            binding.conv_scan_fwd(t["u"], cwt, t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], delta_softplus=x.softplus, conv_bias=cbt, conv_silu=True,
                                  out=y, last_state=last)

        for name, f, kw in (("zoh", fn_zoh, {"disc": "zoh"}), ("conv_scan", fn_conv, {"conv_width": 4})):
            _, v_ms, v_med = time_calls(f, max(3, steps // 2), 1)
            variants[name] = dict(us_per_call=round(v_ms * 1e3, 2), us_median=round(v_med * 1e3, 2),
                                  kernel_path=binding.scan_plan(b, d, n, l, t["u"].dtype, with_path=True, **kw)[0])
    del t, y, last
    torch.cuda.empty_cache()
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg)
    alu_frac = SLOTS_PER_ELEM_STATE * b * d * l * n / (avg_ms * 1e-3) / LANE_SLOTS_PEAK
    return dict(workload=x.meta["name"], batch=b, dim=d, dstate=n, seqlen=l, io=x.io, kernel_path=path,
                segments=seg, us_per_call=round(avg_ms * 1e3, 2), us_median=round(med_ms * 1e3, 2),
                algorithmic_bytes=nbytes, algorithmic_gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                alu_frac=round(alu_frac, 4), elements_per_s=round(b * d * l / (avg_ms * 1e-3), 1),
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                              traffic_ratio=None if traffic is None else round(traffic / nbytes, 3),
                              kernel="ssm_scan_fwd call: %s" % KERNELS[path],
                              alu=dict(frac=round(alu_frac, 4), lane_slots_per_elem_state=SLOTS_PER_ELEM_STATE)),
                **variants)


def sweep_seqlen(dev, steps, warmup, lengths):
    """Time and algorithmic bytes at fixed channels (batch 1, dim 2560, dstate 16, fp32) over seqlen."""
    import torch
    from selective_state_space_65_amd import binding, inputs
    lmax = max(lengths)
    x = inputs.make_scan_inputs(1, 2560, 16, lmax, io="f32", seed=inputs.SEED_BASE + 3,
                                channel_params_kind="workload")
    full = inputs.to_torch(x, dev)
    rows = []
    for l in lengths:
        t = {k: (None if v is None else (v[..., :l].contiguous() if k in ("u", "delta", "z", "B", "C") else v))
             for k, v in full.items()}
        y = torch.empty_like(t["u"])
        last = torch.empty((1, 2560, 16), dtype=torch.float32, device=dev)

        def fn():
            binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["delta_bias"], delta_softplus=True, h0=None, out=y, last_state=last)

        _, avg_ms, med_ms = time_calls(fn, steps, warmup)
        nbytes = algorithmic_bytes(1, 2560, 16, l, 4)
        path, seg, seglen, _ = binding.scan_plan(1, 2560, 16, l, torch.float32, with_path=True)
        row = dict(seqlen=l, us_per_call=round(avg_ms * 1e3, 2), us_per_1k_tokens=round(avg_ms * 1e6 / l, 3),
                   algorithmic_bytes=nbytes, algorithmic_gbs=round(nbytes / (avg_ms * 1e-3) / 1e9, 1),
                   kernel_path=path, segments=seg)
        print(json.dumps(row), flush=True)
        rows.append(row)
        del t, y, last
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="scan workload (default 2: Mamba-1.4B layer)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true", help="skip the fused conv + scan line")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward line")
    ap.add_argument("--no-zoh", action="store_true", help="skip the zero-order-hold line")
    ap.add_argument("--no-complex", action="store_true", help="skip the complex-A line")
    ap.add_argument("--no-configs", action="store_true", help="skip the Mamba-130M and long-sequence sub-lines")
    ap.add_argument("--no-probe", action="store_true", help="skip the instruction-rate probe")
    ap.add_argument("--probe-only", action="store_true", help="only run the instruction-rate probe")
    ap.add_argument("--sweep-seqlen", action="store_true",
                    help="only time batch 1 x dim 2560 x dstate 16 fp32 over seqlen 1k .. 128k")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB three times (reference kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: every box here has a single MI355X, and this path is not "
              "sharded across GPUs (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_65_amd import binding, inputs

    dev = "cuda:0"
    if args.copy_calibration:
        # A plain device copy of known size: 1 GiB read + 1 GiB written per
        # launch.  Profiled with the same counters as the scan, it gives the
        # factor between FETCH_SIZE / WRITE_SIZE and the true bytes.
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes_per_launch=src.numel() * 4, launches=3)))
        return
    if args.probe_only:
        print(json.dumps(rate_probe(dev)), flush=True)
        return
    if args.sweep_seqlen:
        rows = sweep_seqlen(dev, max(3, args.steps // 4), 2, [1024 << i for i in range(8)])
        print(json.dumps(dict(sweep="seqlen", channels="batch 1 x dim 2560 x dstate 16, fp32", rows=rows)))
        return
    x = inputs.scan_config(args.config)
    b, d, n, l = x.shape
    io_bytes = 2 if x.io == "bf16" else 4
    t = inputs.to_torch(x, dev)
    y = torch.empty_like(t["u"])
    last = torch.empty((b, d, n), dtype=torch.float32, device=dev)

    def step():
        binding.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=x.softplus, h0=None, out=y, last_state=last)

    wall_ms, avg_ms, med_ms = time_calls(step, args.steps, args.warmup)
    nbytes = algorithmic_bytes(b, d, n, l, io_bytes, has_z=x.z is not None)
    elems = b * d * l
    gbs = nbytes / (wall_ms * 1e-3) / 1e9
    path, seg, seglen, scratch = binding.scan_plan(b, d, n, l, t["u"].dtype, with_path=True)

    call_gbs = nbytes / (avg_ms * 1e-3) / 1e9
    slots = SLOTS_PER_ELEM_STATE * elems * n
    alu_rate = slots / (avg_ms * 1e-3)
    hbm_frac = call_gbs / HBM_PEAK_GBS
    alu_frac = alu_rate / LANE_SLOTS_PEAK
    traffic = measured_traffic(args.config)
    roof = dict(bound="hbm", achieved=round(call_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(hbm_frac, 4),
                traffic=traffic, traffic_ratio=None if traffic is None else round(traffic / nbytes, 3),
                kernel="ssm_scan_fwd call: %s" % KERNELS[path],
                call_us_avg=round(avg_ms * 1e3, 2), call_us_median=round(med_ms * 1e3, 2),
                algorithmic_bytes=nbytes,
                alu=dict(frac=round(alu_frac, 4), achieved=round(alu_rate / 1e12, 2),
                         peak=round(LANE_SLOTS_PEAK / 1e12, 2), unit="T lane-slots/s",
                         lane_slots_per_elem_state=SLOTS_PER_ELEM_STATE, algorithmic_lane_slots=slots,
                         note="the binding roof: exp2 (2 FMA slots, see rate_probe) + 4 fp32 ops per "
                              "(element, state); packed FP32 is not used"))

    out = dict(metric=METRIC, value=round(gbs, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=round(wall_ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
               data="synthetic",
               config=dict(workload=x.meta["name"], batch=b, dim=d, dstate=n, seqlen=l, io=x.io, gate=True,
                           softplus=True, kernel_path=path, segments=seg, segment_len=seglen),
               hbm_frac_of_peak=round(gbs / HBM_PEAK_GBS, 4), elements_per_s=round(elems / (wall_ms * 1e-3), 1),
               roofline=roof)
    if not args.no_probe:
        out["rate_probe"] = rate_probe(dev)
        out["device_copy"] = device_copy(dev)
        roof["alu"]["probe_scan_body_cost_in_fma_slots"] = out["rate_probe"]["scan_body_cost_in_fma_slots"]
    if not args.no_configs:
        out["configs"] = {str(c): bench_config(dev, c, max(5, args.steps // 2), 2) for c in (1, 3)
                          if c != args.config}
    if not args.no_decode:
        out["decode"] = bench_decode(dev, 50, 5)
    if not args.no_conv:
        out["conv_scan"] = bench_conv_scan(dev, x, t, args.steps, args.warmup)
    if not args.no_zoh:
        out["zoh"] = bench_zoh(dev, x, t, args.steps, args.warmup)
    if not args.no_complex:
        from selective_state_space_65_amd import binding as _b
        try:
            out["complex"] = bench_complex(dev, x, t, args.steps, args.warmup)
        except _b.SsmError as e:
            out["complex"] = dict(skipped=str(e))
    if not args.no_backward:
        bw = bench_backward(dev, x, t, max(3, args.steps // 4), 2)
        bw["vs_forward"] = round(bw["us_per_call"] / (avg_ms * 1e3), 2)
        sc = bw.get("saved_checkpoints", {})
        if "training_step_us" in sc:
            sc["recompute_training_step_us"] = round(avg_ms * 1e3 + bw["us_per_call"], 2)
        out["backward"] = bw
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
