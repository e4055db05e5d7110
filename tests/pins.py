"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
the mathematics, each written independently of the oracle's loop.

Every pin takes an oracle object (oracle.Oracle) and raises AssertionError on
a mismatch, so the same pins run against the real oracle and against
deliberately broken copies of it (tests/test_oracle_mutants.py).

  worked_examples   hand-derived values (tests/golden/worked_examples.json)
  lti_closed_form   constant Delta, B, C: the scan equals a causal convolution
                    with kernel K_k = sum_n C_n Abar_n^k Delta B_n (the pages'
                    recurrence-vs-global-convolution equivalence for S4, in the
                    Chinese explainer's stage 2/3 and the Hebrew overview's
                    linear-time-invariance section)
  bruteforce        time-varying case, tiny L, evaluated in 50-digit mpmath
                    from the product form h_t = (prod Abar) h0 + sum (prod Abar) Bbar u
  single_step       L = 1 by hand formula
  persistence       Delta = 0 leaves the state unchanged (small step: keep the
                    state, ignore the input -- the explainer's gating section)
  forgetting        huge Delta forgets the past (large step: reset the state)
  split_carry       cutting the sequence and carrying last_state equals one pass
                    (segments combine in any grouping -- the parallel scan)
  linearity         with h0 = 0 the output is linear in u
  softplus_silu     the scalar helpers against numpy / scipy library routines
  decode_is_scan    the one-token update equals a one-token scan
  channel_subset    scanning a subset of channels equals the rows of a full scan
  conv_library      the causal depthwise conv (+ silu) in front of the scan against
                    numpy's correlate over [x_prev, x] and scipy's logistic
  conv_taps         a filter that keeps only the current tap returns x; one that
                    keeps only the oldest tap shifts x by K-1, fed by x_prev
  conv_causality    changing x at position p changes exactly u[p .. p+K-1]
  conv_split_carry  convolving in two pieces, the second fed the first's last K-1
                    inputs as x_prev, equals one pass
  bwd_finite_diff   the hand-written reverse-mode gradients against central finite
                    differences of the forward oracle, every input, every flag
  bwd_autograd      the same gradients against torch autograd (fp64, CPU) through an
                    independently written vectorised forward
  zoh_van_loan      exact zero-order hold for B: every step equals the block matrix
                    exponential expm([[a, b u], [0, 0]] Delta) per state (scipy), which
                    holds Abar and Bbar u of the held-input ODE; A with zeros included
  zoh_fixed_point   constant input: the ZOH state converges to -B u / A whatever
                    Delta is (the ODE's equilibrium), the Delta*B rule's does not
  zoh_limits        at A = 0 ZOH equals the Delta*B rule, and for small |Delta A|
                    its factor follows the series Delta (1 + Delta A / 2 + ...)
  zoh_decode        the one-token ZOH update equals a one-token ZOH scan
  zoh_bwd           the ZOH backward against finite differences (A with zero and tiny
                    entries) and torch autograd through expm1(Delta A) / A
  complex_real_limit   complex A, B, C, h0 with zero imaginary parts equal the real
                    scan with C doubled (a real state and its conjugate partner)
  complex_block_expm   each complex state a + ib is the real two-state system with
                    block [[a, -b], [b, a]]: stepped with scipy's expm of that block,
                    input (Re B, Im B) u and output 2 (Re C, -Im C)
  complex_lti       constant Delta, B, C: y = 2 Re(sum_k K_k u_{t-k}) + D u with
                    K_k = sum_n C_n Abar_n^k Delta B_n (numpy complex powers, np.convolve)
  complex_bwd       the complex-A gradients (d/dRe + i d/dIm) against central finite
                    differences of the complex forward and torch's complex autograd
  conv_bwd_finite_diff  the conv's gradients (x, weight, bias, x_prev) against central
                    finite differences of the conv oracle, every width, silu on and off
  conv_bwd_autograd the same gradients against torch autograd (fp64, CPU) through
                    torch.nn.functional.conv1d (groups = dim) over [x_prev, x]
"""
import json
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "worked_examples.json")


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, "%s: shape %s vs %s" % (what, got.shape, want.shape)
    err = np.abs(got - want)
    tol = atol + rtol * np.abs(want)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: max err %.3e at %s (got %r want %r)" % (
        what, float(err.max()), np.unravel_index(int(np.argmax(err)), err.shape), got.flat[np.argmax(err)],
        want.flat[np.argmax(err)])


def _rng(seed):
    return np.random.default_rng(seed)


def _random_problem(rng, batch, dim, dstate, seqlen, z=True, D=True, bias=True, h0=True):
    A = -rng.uniform(0.2, 3.0, size=(dim, dstate))
    return dict(
        u=rng.standard_normal((batch, dim, seqlen)),
        delta=0.5 * rng.standard_normal((batch, dim, seqlen)),
        A=A,
        B=rng.standard_normal((batch, dstate, seqlen)),
        C=rng.standard_normal((batch, dstate, seqlen)),
        D=rng.standard_normal(dim) if D else None,
        z=rng.standard_normal((batch, dim, seqlen)) if z else None,
        delta_bias=rng.uniform(-2.0, 0.5, size=dim) if bias else None,
        h0=rng.standard_normal((batch, dim, dstate)) if h0 else None,
    )


# ---------------------------------------------------------------------------


def worked_examples(o):
    data = json.load(open(GOLDEN))
    env = {"ln2": math.log(2.0), "ln3": math.log(3.0), "__builtins__": {}}

    def ev(x):
        if x is None:
            return None
        if isinstance(x, list):
            return np.array([ev(v) for v in x], dtype=np.float64)
        if isinstance(x, str):
            return float(eval(x, env))
        return float(x)

    for case in data["cases"]:
        args = {k: ev(case[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
        y, last = o.scan_f64(softplus=case["softplus"], zoh=case.get("zoh", False), **args)
        _close(y, ev(case["expected_y"]), 1e-14, 1e-14, case["name"] + " y")
        _close(last, ev(case["expected_last_state"]), 1e-14, 1e-14, case["name"] + " last_state")


def lti_closed_form(o):
    rng = _rng(11)
    batch, dim, dstate, seqlen = 2, 3, 4, 40
    for with_h0 in (False, True):
        p = _random_problem(rng, batch, dim, dstate, seqlen, z=True, D=True, bias=True, h0=with_h0)
        # Time-invariant system: one raw step per channel, one B and C per batch row.
        p["delta"] = np.repeat(0.5 * rng.standard_normal((batch, dim, 1)), seqlen, axis=2)
        Bc = rng.standard_normal((batch, dstate, 1))
        Cc = rng.standard_normal((batch, dstate, 1))
        p["B"] = np.repeat(Bc, seqlen, axis=2)
        p["C"] = np.repeat(Cc, seqlen, axis=2)
        y, last = o.scan_f64(softplus=True, **p)
        k = np.arange(seqlen)
        for b in range(batch):
            for d in range(dim):
                step = np.logaddexp(0.0, p["delta"][b, d, 0] + p["delta_bias"][d])
                abar = np.exp(step * p["A"][d])                             # (dstate,)
                powers = abar[None, :] ** k[:, None]                         # (seqlen, dstate)
                K = powers @ (Cc[b, :, 0] * step * Bc[b, :, 0])              # convolution kernel
                conv = np.convolve(p["u"][b, d], K)[:seqlen]
                ref = conv + p["D"][d] * p["u"][b, d]
                if with_h0:
                    ref = ref + (abar[None, :] ** (k[:, None] + 1)) @ (Cc[b, :, 0] * p["h0"][b, d])
                zz = p["z"][b, d]
                from scipy.special import expit
                ref = ref * zz * expit(zz)
                _close(y[b, d], ref, 1e-11, 1e-12, "LTI convolution b=%d d=%d h0=%s" % (b, d, with_h0))
                h_ref = (abar ** seqlen) * (p["h0"][b, d] if with_h0 else 0.0) + np.array(
                    [np.sum(abar[n] ** (seqlen - 1 - k) * step * Bc[b, n, 0] * p["u"][b, d]) for n in range(dstate)])
                _close(last[b, d], h_ref, 1e-11, 1e-12, "LTI final state b=%d d=%d" % (b, d))


def bruteforce(o):
    import itertools
    import mpmath as mp
    mp.mp.dps = 50
    rng = _rng(12)
    batch, dim, dstate, seqlen = 2, 2, 3, 5
    for flags in itertools.product([False, True], repeat=5):
        zf, Df, bf, spf, hf = flags
        p = _random_problem(rng, batch, dim, dstate, seqlen, z=zf, D=Df, bias=bf, h0=hf)
        y, last = o.scan_f64(softplus=spf, **p)
        for b in range(batch):
            for d in range(dim):
                steps = []
                for t in range(seqlen):
                    x = mp.mpf(p["delta"][b, d, t]) + (mp.mpf(p["delta_bias"][d]) if bf else 0)
                    steps.append(mp.log(1 + mp.exp(x)) if spf else x)
                abar = [[mp.exp(steps[t] * mp.mpf(p["A"][d, n])) for n in range(dstate)] for t in range(seqlen)]
                for t in range(seqlen):
                    acc = mp.mpf(0)
                    hs = []
                    for n in range(dstate):
                        prod_all = mp.fprod(abar[s][n] for s in range(t + 1))
                        h = prod_all * (mp.mpf(p["h0"][b, d, n]) if hf else 0)
                        for s in range(t + 1):
                            tail = mp.fprod(abar[r][n] for r in range(s + 1, t + 1))
                            h += tail * steps[s] * mp.mpf(p["B"][b, n, s]) * mp.mpf(p["u"][b, d, s])
                        hs.append(h)
                        acc += mp.mpf(p["C"][b, n, t]) * h
                    if Df:
                        acc += mp.mpf(p["D"][d]) * mp.mpf(p["u"][b, d, t])
                    if zf:
                        zz = mp.mpf(p["z"][b, d, t])
                        acc *= zz / (1 + mp.exp(-zz))
                    _close(y[b, d, t], float(acc), 1e-13, 1e-14, "brute force y flags=%s" % (flags,))
                    if t == seqlen - 1:
                        _close(last[b, d], [float(v) for v in hs], 1e-13, 1e-14, "brute force h flags=%s" % (flags,))


def single_step(o):
    rng = _rng(13)
    p = _random_problem(rng, 3, 4, 5, 1)
    y, last = o.scan_f64(softplus=True, **p)
    step = np.logaddexp(0.0, p["delta"][..., 0] + p["delta_bias"][None, :])           # (b, d)
    abar = np.exp(step[..., None] * p["A"][None])                                     # (b, d, n)
    h = abar * p["h0"] + step[..., None] * p["B"][:, None, :, 0] * p["u"][..., 0][..., None]
    ref = np.einsum("bdn,bn->bd", h, p["C"][..., 0]) + p["D"][None] * p["u"][..., 0]
    zz = p["z"][..., 0]
    ref = ref * zz / (1.0 + np.exp(-zz))
    _close(y[..., 0], ref, 1e-13, 1e-14, "single step y")
    _close(last, h, 1e-13, 1e-14, "single step h")


def persistence(o):
    rng = _rng(14)
    p = _random_problem(rng, 2, 3, 4, 17, z=False, bias=False, h0=True)
    p["delta"] = np.zeros_like(p["delta"])
    y, last = o.scan_f64(softplus=False, **p)
    assert np.array_equal(last, p["h0"]), "zero step must leave the state unchanged"
    ref = np.einsum("bdn,bnl->bdl", p["h0"], p["C"]) + p["D"][None, :, None] * p["u"]
    _close(y, ref, 1e-14, 1e-14, "persistence y")


def forgetting(o):
    rng = _rng(15)
    p = _random_problem(rng, 2, 3, 4, 12, bias=False, h0=True)
    p["A"] = -rng.uniform(1.0, 4.0, size=p["A"].shape)
    p["delta"] = np.full_like(p["delta"], 50.0)
    y1, _ = o.scan_f64(softplus=False, **p)
    q = dict(p)
    for t in range(1, 12):
        q["u"] = p["u"].copy()
        q["u"][..., :t] += rng.standard_normal(q["u"][..., :t].shape) * 10.0
        q["h0"] = p["h0"] + 100.0
        y2, _ = o.scan_f64(softplus=False, **q)
        _close(y2[..., t:], y1[..., t:], 1e-15, 1e-12, "forgetting t=%d" % t)
        # and the past did matter before t (the perturbation is visible there)
        assert np.abs(y2[..., :t] - y1[..., :t]).max() > 1e-3


def split_carry(o):
    rng = _rng(16)
    p = _random_problem(rng, 2, 3, 4, 50)
    y, last = o.scan_f64(softplus=True, **p)
    for cuts in ([1], [7, 8], [13, 29, 30, 49]):
        h = p["h0"]
        pieces = []
        edges = [0] + cuts + [50]
        for a, b in zip(edges[:-1], edges[1:]):
            q = dict(p)
            for k in ("u", "delta", "B", "C", "z"):
                q[k] = p[k][..., a:b]
            q["h0"] = h
            yy, h = o.scan_f64(softplus=True, **q)
            pieces.append(yy)
        _close(np.concatenate(pieces, axis=-1), y, 1e-12, 1e-13, "split %s y" % cuts)
        _close(h, last, 1e-12, 1e-13, "split %s state" % cuts)


def linearity(o):
    rng = _rng(17)
    p = _random_problem(rng, 2, 3, 4, 30, h0=False)
    u1, u2 = p["u"], rng.standard_normal(p["u"].shape)
    a, b = 0.75, -2.5
    y1, h1 = o.scan_f64(softplus=True, **dict(p, u=u1))
    y2, h2 = o.scan_f64(softplus=True, **dict(p, u=u2))
    y3, h3 = o.scan_f64(softplus=True, **dict(p, u=a * u1 + b * u2))
    _close(y3, a * y1 + b * y2, 1e-12, 1e-12, "linearity y")
    _close(h3, a * h1 + b * h2, 1e-12, 1e-12, "linearity h")


def softplus_silu(o):
    from scipy.special import expit
    for x in (-800.0, -60.0, -20.0, -7.0, -1e-3, 0.0, 1e-3, 1.0, 19.0, 21.0, 60.0, 800.0):
        _close(o.softplus_f64(x), np.logaddexp(0.0, x), 1e-15, 0.0, "softplus(%g)" % x)
        _close(o.silu_f64(x), x * expit(x), 1e-15, 1e-300, "silu(%g)" % x)


def decode_is_scan(o):
    rng = _rng(18)
    p = _random_problem(rng, 3, 5, 4, 1)
    y_scan, h_scan = o.scan_f64(softplus=True, **p)
    state = p["h0"].copy()
    y_dec = o.state_update_f64(state, p["u"][..., 0], p["delta"][..., 0], p["A"], p["B"][..., 0], p["C"][..., 0],
                               p["D"], p["z"][..., 0], p["delta_bias"], softplus=True)
    _close(y_dec, y_scan[..., 0], 1e-15, 1e-15, "decode y")
    _close(state, h_scan, 1e-15, 1e-15, "decode state")


def channel_subset(o):
    rng = _rng(19)
    p = _random_problem(rng, 3, 5, 4, 9)
    y, last = o.scan_f64(softplus=True, **p)
    ch = [(0, 0), (1, 3), (2, 4), (0, 2)]
    ys, hs = o.scan_channels_f64(ch, softplus=True, **p)
    for i, (b, d) in enumerate(ch):
        assert np.array_equal(ys[i], y[b, d]) and np.array_equal(hs[i], last[b, d])


def _conv_problem(rng, batch, dim, seqlen, width):
    return dict(x=rng.standard_normal((batch, dim, seqlen)), weight=rng.standard_normal((dim, width)),
                bias=rng.standard_normal(dim), x_prev=rng.standard_normal((batch, dim, width - 1)))


def conv_library(o):
    from scipy.special import expit
    rng = _rng(20)
    batch, dim, seqlen = 2, 3, 23
    for width in (1, 2, 3, 4):
        for silu in (False, True):
            for with_prev in (False, True):
                for with_bias in (False, True):
                    p = _conv_problem(rng, batch, dim, seqlen, width)
                    u = o.conv1d_f64(p["x"], p["weight"], p["bias"] if with_bias else None,
                                     p["x_prev"] if with_prev else None, silu=silu)
                    for b in range(batch):
                        for d in range(dim):
                            head = p["x_prev"][b, d] if with_prev else np.zeros(width - 1)
                            ref = np.correlate(np.concatenate([head, p["x"][b, d]]), p["weight"][d], mode="valid")
                            if with_bias:
                                ref = ref + p["bias"][d]
                            if silu:
                                ref = ref * expit(ref)
                            _close(u[b, d], ref, 1e-13, 1e-14,
                                   "conv K=%d silu=%s prev=%s bias=%s" % (width, silu, with_prev, with_bias))


def conv_taps(o):
    rng = _rng(21)
    x = rng.standard_normal((2, 3, 17))
    for width in (1, 2, 3, 4):
        keep_current = np.zeros((3, width))
        keep_current[:, width - 1] = 1.0
        assert np.array_equal(o.conv1d_f64(x, keep_current, silu=False), x), "current tap must return x (K=%d)" % width
        keep_oldest = np.zeros((3, width))
        keep_oldest[:, 0] = 1.0
        prev = rng.standard_normal((2, 3, width - 1))
        u = o.conv1d_f64(x, keep_oldest, x_prev=prev, silu=False)
        assert np.array_equal(u[..., width - 1:], x[..., :17 - (width - 1)]), "oldest tap must shift (K=%d)" % width
        assert np.array_equal(u[..., :width - 1], prev), "oldest tap must read x_prev first (K=%d)" % width
        u0 = o.conv1d_f64(x, keep_oldest, silu=False)
        assert not u0[..., :width - 1].any(), "no x_prev means zero history (K=%d)" % width


def conv_causality(o):
    rng = _rng(22)
    for width in (2, 4):
        p = _conv_problem(rng, 1, 2, 20, width)
        u = o.conv1d_f64(p["x"], p["weight"], p["bias"], p["x_prev"], silu=True)
        for pos in (0, 7, 19):
            x2 = p["x"].copy()
            x2[..., pos] += 3.0
            u2 = o.conv1d_f64(x2, p["weight"], p["bias"], p["x_prev"], silu=True)
            changed = np.abs(u2 - u).max(axis=(0, 1)) > 0
            want = np.zeros(20, bool)
            want[pos:pos + width] = True
            assert np.array_equal(changed, want), "K=%d pos=%d changed %s" % (width, pos, np.nonzero(changed)[0])


def conv_split_carry(o):
    rng = _rng(23)
    for width in (2, 3, 4):
        p = _conv_problem(rng, 2, 3, 30, width)
        u = o.conv1d_f64(p["x"], p["weight"], p["bias"], p["x_prev"], silu=True)
        for cut in (width - 1, 11, 29):
            u1 = o.conv1d_f64(p["x"][..., :cut], p["weight"], p["bias"], p["x_prev"], silu=True)
            tail = np.concatenate([p["x_prev"], p["x"][..., :cut]], axis=-1)[..., -(width - 1):]
            u2 = o.conv1d_f64(p["x"][..., cut:], p["weight"], p["bias"], tail, silu=True)
            _close(np.concatenate([u1, u2], axis=-1), u, 1e-15, 1e-15, "conv split K=%d cut=%d" % (width, cut))


GRAD_OF = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias", h0="dh0")


def bwd_finite_diff(o):
    rng = _rng(24)
    batch, dim, dstate, seqlen = 2, 2, 3, 9
    eps = 1e-6
    for zf, Df, bf, spf, hf, dlf in ((True, True, True, True, True, True), (False, False, False, False, False, False),
                                     (True, False, True, False, True, False), (False, True, False, True, False, True)):
        p = _random_problem(rng, batch, dim, dstate, seqlen, z=zf, D=Df, bias=bf, h0=hf)
        dy = rng.standard_normal((batch, dim, seqlen))
        dlast = rng.standard_normal((batch, dim, dstate)) if dlf else None
        g = o.scan_bwd_f64(softplus=spf, dy=dy, dlast=dlast, **p)

        def loss(q):
            y, h = o.scan_f64(softplus=spf, **q)
            return float((dy * y).sum() + ((dlast * h).sum() if dlf else 0.0))

        for name, key in GRAD_OF.items():
            if p.get(name) is None:
                continue
            base = p[name]
            num = np.empty_like(base)
            for i in range(base.size):
                up, dn = base.copy(), base.copy()
                up.flat[i] += eps
                dn.flat[i] -= eps
                num.flat[i] = (loss(dict(p, **{name: up})) - loss(dict(p, **{name: dn}))) / (2 * eps)
            if name == "h0" and not hf:
                continue
            scale = max(float(np.abs(num).max()), 1e-12)
            _close(g[key] / scale, num / scale, 0.0, 1e-6, "d/d%s flags=%s" % (name, (zf, Df, bf, spf, hf, dlf)))
        if not hf:  # without h0 the state starts at zero; dh0 is still the gradient at that zero state
            zero = np.zeros((batch, dim, dstate))
            num = np.empty_like(zero)
            for i in range(zero.size):
                up, dn = zero.copy(), zero.copy()
                up.flat[i] += eps
                dn.flat[i] -= eps
                num.flat[i] = (loss(dict(p, h0=up)) - loss(dict(p, h0=dn))) / (2 * eps)
            _close(g["dh0"], num, 1e-6, 1e-9, "dh0 at a zero state")


def _torch_loss(p, softplus, dy, dlast, zoh=False):
    import torch
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True)) for k, v in p.items()}
    x = t["delta"] + (t["delta_bias"][None, :, None] if t["delta_bias"] is not None else 0.0)
    step = torch.logaddexp(x, torch.zeros_like(x)) if softplus else x
    batch, dim, seqlen = t["u"].shape
    dstate = t["A"].shape[1]
    h = t["h0"] if t["h0"] is not None else torch.zeros(batch, dim, dstate, dtype=torch.float64)
    loss = 0.0
    for l in range(seqlen):
        abar = torch.exp(step[:, :, l, None] * t["A"][None])
        phi = torch.expm1(step[:, :, l, None] * t["A"][None]) / t["A"][None] if zoh else step[:, :, l, None]
        h = abar * h + phi * t["B"][:, None, :, l] * t["u"][:, :, l, None]
        s = (t["C"][:, None, :, l] * h).sum(-1)
        if t["D"] is not None:
            s = s + t["D"][None] * t["u"][:, :, l]
        if t["z"] is not None:
            zz = t["z"][:, :, l]
            s = s * zz * torch.sigmoid(zz)
        loss = loss + (torch.tensor(dy[:, :, l]) * s).sum()
    if dlast is not None:
        loss = loss + (torch.tensor(dlast) * h).sum()
    loss.backward()
    return {k: (None if v is None else v.grad.numpy()) for k, v in t.items()}


def bwd_autograd(o):
    rng = _rng(25)
    batch, dim, dstate, seqlen = 3, 4, 5, 17
    for flags in ((True, True, True, True, True), (False, True, False, True, False), (True, False, True, False, True)):
        zf, Df, bf, spf, hf = flags
        p = _random_problem(rng, batch, dim, dstate, seqlen, z=zf, D=Df, bias=bf, h0=hf)
        dy = rng.standard_normal((batch, dim, seqlen))
        dlast = rng.standard_normal((batch, dim, dstate))
        g = o.scan_bwd_f64(softplus=spf, dy=dy, dlast=dlast, **p)
        ref = _torch_loss(p, spf, dy, dlast)
        for name, key in GRAD_OF.items():
            if p.get(name) is None:
                continue
            _close(g[key], ref[name], 1e-11, 1e-12, "autograd d/d%s flags=%s" % (name, flags))


def zoh_van_loan(o):
    from scipy.linalg import expm
    rng = _rng(30)
    batch, dim, dstate, seqlen = 2, 3, 4, 7
    for flags in ((True, True, True, True, True), (False, False, False, False, False), (True, False, True, True, False)):
        zf, Df, bf, spf, hf = flags
        p = _random_problem(rng, batch, dim, dstate, seqlen, z=zf, D=Df, bias=bf, h0=hf)
        p["A"][0, 1] = 0.0         # a non-decaying state
        p["A"][2, 3] = -1e-9       # nearly non-decaying
        y, last = o.scan_f64(softplus=spf, zoh=True, **p)
        x = p["delta"] + (p["delta_bias"][None, :, None] if bf else 0.0)
        step = np.logaddexp(x, 0.0) if spf else x
        for b in range(batch):
            for d in range(dim):
                h = p["h0"][b, d].copy() if hf else np.zeros(dstate)
                for t in range(seqlen):
                    # A is diagonal, so the (N+1)-square block exponential splits
                    # into one 2 x 2 block per state (scipy's expm of the whole
                    # block matrix loses ~1e-8 when its diagonal spans 1e-9..3).
                    for n in range(dstate):
                        m = np.array([[p["A"][d, n], p["B"][b, n, t] * p["u"][b, d, t]], [0.0, 0.0]])
                        e = expm(m * step[b, d, t])
                        h[n] = e[0, 0] * h[n] + e[0, 1]
                    v = float(p["C"][b, :, t] @ h) + (p["D"][d] * p["u"][b, d, t] if Df else 0.0)
                    if zf:
                        zz = p["z"][b, d, t]
                        v *= zz / (1.0 + math.exp(-zz))
                    _close(y[b, d, t], v, 1e-11, 1e-13, "zoh van loan y b=%d d=%d t=%d" % (b, d, t))
                _close(last[b, d], h, 1e-11, 1e-13, "zoh van loan state b=%d d=%d" % (b, d))


def zoh_fixed_point(o):
    dim, dstate, seqlen = 3, 4, 400
    A = -np.array([[0.5, 1.0, 2.0, 3.0], [1.0, 1.5, 2.5, 4.0], [0.7, 0.9, 1.1, 5.0]])
    Bc = np.array([1.0, -2.0, 0.5, 3.0])
    for dt in (0.25, 1.0, 3.0):
        u = np.full((1, dim, seqlen), 1.5)
        delta = np.full((1, dim, seqlen), dt)
        B = np.repeat(Bc[None, :, None], seqlen, axis=2)
        C = np.ones((1, dstate, seqlen))
        _, last = o.scan_f64(u, delta, A, B, C, zoh=True)
        want = -Bc[None, :] * 1.5 / A
        _close(last[0], want, 1e-12, 1e-14, "zoh fixed point dt=%g" % dt)


def zoh_limits(o):
    rng = _rng(31)
    p = _random_problem(rng, 2, 3, 4, 9)
    p["A"][:, 0] = 0.0
    ys, ls = o.scan_f64(softplus=True, zoh=False, **dict(p, A=p["A"][:, :1], B=p["B"][:, :1], C=p["C"][:, :1]))
    yz, lz = o.scan_f64(softplus=True, zoh=True, **dict(p, A=p["A"][:, :1], B=p["B"][:, :1], C=p["C"][:, :1]))
    _close(yz, ys, 1e-15, 1e-15, "zoh at A = 0 is the Delta*B rule (y)")
    _close(lz, ls, 1e-15, 1e-15, "zoh at A = 0 is the Delta*B rule (state)")
    for dt in (1e-3, 0.1, 1.0):
        for a in (-1e-12, -1e-6, 1e-6, -1e-3):
            x = dt * a
            series = dt * (1.0 + x / 2.0 + x * x / 6.0 + x ** 3 / 24.0)
            _close(o.zoh_b_f64(dt, a), series, 1e-14, 0.0, "zoh factor series dt=%g a=%g" % (dt, a))
        assert o.zoh_b_f64(dt, 0.0) == dt, "zoh factor at a = 0"
        for a in (-0.5, -4.0, 2.0):
            _close(o.zoh_b_f64(dt, a), (math.exp(dt * a) - 1.0) / a, 1e-13, 0.0, "zoh factor dt=%g a=%g" % (dt, a))


def zoh_bwd(o):
    """The zero-order-hold backward: finite differences (A with a zero and a tiny entry, where the
    factor's A-derivative comes from its series) and torch autograd through expm1(Delta A) / A."""
    rng = _rng(33)
    batch, dim, dstate, seqlen = 2, 2, 3, 8
    eps = 1e-6
    p = _random_problem(rng, batch, dim, dstate, seqlen)
    p["A"][0, 0] = 0.0
    p["A"][1, 2] = -1e-7
    dy = rng.standard_normal((batch, dim, seqlen))
    dlast = rng.standard_normal((batch, dim, dstate))
    g = o.scan_bwd_f64(softplus=True, dy=dy, dlast=dlast, zoh=True, **p)

    def loss(q):
        y, h = o.scan_f64(softplus=True, zoh=True, **q)
        return float((dy * y).sum() + (dlast * h).sum())

    for name, key in GRAD_OF.items():
        base = p[name]
        num = np.empty_like(base)
        for i in range(base.size):
            up, dn = base.copy(), base.copy()
            up.flat[i] += eps
            dn.flat[i] -= eps
            num.flat[i] = (loss(dict(p, **{name: up})) - loss(dict(p, **{name: dn}))) / (2 * eps)
        scale = max(float(np.abs(num).max()), 1e-12)
        _close(g[key] / scale, num / scale, 0.0, 1e-6, "zoh d/d%s" % name)
    q = _random_problem(rng, 3, 4, 5, 13)
    dy = rng.standard_normal((3, 4, 13))
    dlast = rng.standard_normal((3, 4, 5))
    g = o.scan_bwd_f64(softplus=True, dy=dy, dlast=dlast, zoh=True, **q)
    ref = _torch_loss(q, True, dy, dlast, zoh=True)
    for name, key in GRAD_OF.items():
        _close(g[key], ref[name], 1e-11, 1e-12, "zoh autograd d/d%s" % name)
    # the factor's A-derivative: its series at small |Delta A|, the closed form elsewhere, Delta^2/2 at A = 0
    for dt in (1e-3, 0.3, 2.0):
        assert abs(o.zoh_b_da_f64(dt, 0.0) - dt * dt / 2) <= 1e-16 * dt * dt
        for a in (-3.0, -0.4, -1e-5, 1e-5, 0.7):
            h = 1e-4  # central difference: truncation ~ h^2 dt^4, rounding ~ 1e-16 dt / h
            num = (o.zoh_b_f64(dt, a + h) - o.zoh_b_f64(dt, a - h)) / (2 * h)
            _close(o.zoh_b_da_f64(dt, a), num, 1e-7, 1e-13, "d phi / dA at dt=%g a=%g" % (dt, a))


def zoh_decode(o):
    rng = _rng(32)
    p = _random_problem(rng, 3, 5, 4, 1)
    p["A"][1, 2] = 0.0
    y_scan, last_scan = o.scan_f64(softplus=True, zoh=True, **p)
    st = p["h0"].copy()
    y_dec = o.state_update_f64(st, p["u"][..., 0], p["delta"][..., 0], p["A"], p["B"][..., 0], p["C"][..., 0],
                               p["D"], p["z"][..., 0], p["delta_bias"], softplus=True, zoh=True)
    _close(y_dec, y_scan[..., 0], 1e-15, 1e-15, "zoh decode y")
    _close(st, last_scan, 1e-15, 1e-15, "zoh decode state")


def _complex_problem(rng, batch, dim, dstate, seqlen, h0=True):
    p = _random_problem(rng, batch, dim, dstate, seqlen, h0=False)
    p["A"] = p["A"] + 1j * rng.uniform(-6.0, 6.0, size=(dim, dstate))
    p["B"] = p["B"] + 1j * rng.standard_normal((batch, dstate, seqlen))
    p["C"] = p["C"] + 1j * rng.standard_normal((batch, dstate, seqlen))
    p["h0"] = (rng.standard_normal((batch, dim, dstate)) + 1j * rng.standard_normal((batch, dim, dstate))) if h0 else None
    return p


def complex_real_limit(o):
    rng = _rng(40)
    p = _random_problem(rng, 2, 3, 4, 11, h0=True)
    y, last = o.scan_f64(softplus=True, **dict(p, C=2.0 * p["C"]))
    q = dict(p, A=p["A"] + 0j, B=p["B"] + 0j, C=p["C"] + 0j, h0=p["h0"] + 0j)
    yc, lc = o.scan_complex_f64(softplus=True, **q)
    _close(yc, y, 1e-13, 1e-14, "complex with real parameters: y")
    _close(lc.real, last, 1e-13, 1e-14, "complex with real parameters: state")
    assert not lc.imag.any(), "imaginary state from real parameters"


def complex_block_expm(o):
    from scipy.linalg import expm
    rng = _rng(41)
    batch, dim, dstate, seqlen = 2, 2, 3, 6
    for flags in ((True, True, True, True, True), (False, False, False, False, False)):
        zf, Df, bf, spf, hf = flags
        p = _complex_problem(rng, batch, dim, dstate, seqlen, h0=hf)
        if not zf:
            p["z"] = None
        if not Df:
            p["D"] = None
        if not bf:
            p["delta_bias"] = None
        y, last = o.scan_complex_f64(softplus=spf, **p)
        x = p["delta"] + (p["delta_bias"][None, :, None] if bf else 0.0)
        step = np.logaddexp(x, 0.0) if spf else x
        for b in range(batch):
            for d in range(dim):
                h = np.zeros((dstate, 2))
                if hf:
                    h[:, 0], h[:, 1] = p["h0"][b, d].real, p["h0"][b, d].imag
                for t in range(seqlen):
                    v = 0.0
                    for n in range(dstate):
                        a, w = p["A"][d, n].real, p["A"][d, n].imag
                        e = expm(np.array([[a, -w], [w, a]]) * step[b, d, t])
                        bv = np.array([p["B"][b, n, t].real, p["B"][b, n, t].imag])
                        h[n] = e @ h[n] + step[b, d, t] * bv * p["u"][b, d, t]
                        v += 2.0 * (p["C"][b, n, t].real * h[n, 0] - p["C"][b, n, t].imag * h[n, 1])
                    if Df:
                        v += p["D"][d] * p["u"][b, d, t]
                    if zf:
                        zz = p["z"][b, d, t]
                        v *= zz / (1.0 + math.exp(-zz))
                    _close(y[b, d, t], v, 1e-11, 1e-13, "complex block y b=%d d=%d t=%d" % (b, d, t))
                _close(last[b, d].real, h[:, 0], 1e-11, 1e-13, "complex block state re")
                _close(last[b, d].imag, h[:, 1], 1e-11, 1e-13, "complex block state im")


def complex_lti(o):
    rng = _rng(42)
    dim, dstate, seqlen = 3, 4, 40
    A = -rng.uniform(0.1, 1.0, size=(dim, dstate)) + 1j * rng.uniform(-3.0, 3.0, size=(dim, dstate))
    Bc = rng.standard_normal(dstate) + 1j * rng.standard_normal(dstate)
    Cc = rng.standard_normal(dstate) + 1j * rng.standard_normal(dstate)
    u = rng.standard_normal((1, dim, seqlen))
    dt = 0.3
    delta = np.full((1, dim, seqlen), dt)
    B = np.repeat(Bc[None, :, None], seqlen, axis=2)
    C = np.repeat(Cc[None, :, None], seqlen, axis=2)
    D = rng.standard_normal(dim)
    y, _ = o.scan_complex_f64(u, delta, A, B, C, D=D)
    k = np.arange(seqlen)
    for d in range(dim):
        abar = np.exp(dt * A[d])
        K = (Cc[None, :] * abar[None, :] ** k[:, None] * dt * Bc[None, :]).sum(axis=1)
        want = 2.0 * np.convolve(K, u[0, d])[:seqlen].real + D[d] * u[0, d]
        _close(y[0, d], want, 1e-11, 1e-12, "complex LTI d=%d" % d)


def _complex_loss_torch(p, softplus, dy, dlast):
    import torch
    c = {k: (None if p.get(k) is None else torch.tensor(p[k], dtype=torch.complex128 if np.iscomplexobj(p[k])
                                                          else torch.float64, requires_grad=True))
         for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
    x = c["delta"] + (c["delta_bias"][None, :, None] if c["delta_bias"] is not None else 0.0)
    step = torch.logaddexp(x, torch.zeros_like(x)) if softplus else x
    batch, dim, seqlen = c["u"].shape
    dstate = c["A"].shape[1]
    h = c["h0"] if c["h0"] is not None else torch.zeros(batch, dim, dstate, dtype=torch.complex128)
    loss = 0.0
    for l in range(seqlen):
        abar = torch.exp(step[:, :, l, None] * c["A"][None])
        h = abar * h + step[:, :, l, None] * c["B"][:, None, :, l] * c["u"][:, :, l, None]
        s_ = 2.0 * (c["C"][:, None, :, l] * h).sum(-1).real
        if c["D"] is not None:
            s_ = s_ + c["D"][None] * c["u"][:, :, l]
        if c["z"] is not None:
            zz = c["z"][:, :, l]
            s_ = s_ * zz * torch.sigmoid(zz)
        loss = loss + (torch.tensor(dy[:, :, l]) * s_).sum()
    dl = torch.tensor(dlast)
    loss = loss + (dl.real * h.real + dl.imag * h.imag).sum()
    loss.backward()
    return {k: (None if v is None else v.grad.numpy()) for k, v in c.items()}


def complex_bwd(o):
    rng = _rng(43)
    batch, dim, dstate, seqlen = 2, 2, 3, 7
    for flags in ((True, True, True, True, True), (False, False, False, False, True)):
        zf, Df, bf, spf, hf = flags
        p = _complex_problem(rng, batch, dim, dstate, seqlen, h0=hf)
        if not zf:
            p["z"] = None
        if not Df:
            p["D"] = None
        if not bf:
            p["delta_bias"] = None
        dy = rng.standard_normal((batch, dim, seqlen))
        dlast = rng.standard_normal((batch, dim, dstate)) + 1j * rng.standard_normal((batch, dim, dstate))
        g = o.scan_complex_bwd_f64(softplus=spf, dy=dy, dlast=dlast, **p)

        def loss(q):
            y, h = o.scan_complex_f64(softplus=spf, **q)
            return float((dy * y).sum() + (dlast.real * h.real + dlast.imag * h.imag).sum())

        eps = 1e-6
        for name, key in GRAD_OF.items():
            if p.get(name) is None:
                continue
            base = p[name]
            parts = (1.0, 1j) if np.iscomplexobj(base) else (1.0,)
            num = np.zeros(base.shape, complex if np.iscomplexobj(base) else float)
            for part in parts:
                for i in range(base.size):
                    up, dn = base.copy(), base.copy()
                    up.flat[i] += eps * part
                    dn.flat[i] -= eps * part
                    dv = (loss(dict(p, **{name: up})) - loss(dict(p, **{name: dn}))) / (2 * eps)
                    num.flat[i] += dv * part
            scale = max(float(np.abs(num).max()), 1e-12)
            _close(np.abs(g[key] - num) / scale, np.zeros(base.shape), 0.0, 1e-6, "complex d/d%s" % name)
        ref = _complex_loss_torch(p, spf, dy, dlast)
        for name, key in GRAD_OF.items():
            if p.get(name) is None:
                continue
            _close(np.abs(g[key] - ref[name]), np.zeros(np.shape(ref[name])), 0.0,
                   1e-11 * max(1.0, float(np.abs(ref[name]).max())), "complex autograd d/d%s" % name)


def conv_bwd_finite_diff(o):
    rng = _rng(24)
    batch, dim, seqlen = 2, 3, 9
    eps = 1e-6
    for width in (1, 2, 3, 4):
        for silu in (False, True):
            p = _conv_problem(rng, batch, dim, seqlen, width)
            du = rng.standard_normal((batch, dim, seqlen))
            g = o.conv1d_bwd_f64(p["x"], p["weight"], du, bias=p["bias"], x_prev=p["x_prev"], silu=silu)

            def loss(q):
                return float((du * o.conv1d_f64(q["x"], q["weight"], q["bias"], q["x_prev"], silu=silu)).sum())

            for name, key in (("x", "dx"), ("weight", "dweight"), ("bias", "dbias"), ("x_prev", "dx_prev")):
                base = p[name]
                num = np.zeros(base.shape)
                for i in range(base.size):
                    up, dn = base.copy(), base.copy()
                    up.flat[i] += eps
                    dn.flat[i] -= eps
                    num.flat[i] = (loss(dict(p, **{name: up})) - loss(dict(p, **{name: dn}))) / (2 * eps)
                _close(g[key], num, 0.0, 2e-8, "conv K=%d silu=%s d/d%s" % (width, silu, name))
    # No x_prev: the history is zero and its gradient is still reported (as what x_prev would get).
    p = _conv_problem(rng, 1, 2, 6, 3)
    du = rng.standard_normal((1, 2, 6))
    g0 = o.conv1d_bwd_f64(p["x"], p["weight"], du, bias=p["bias"], x_prev=None, silu=True)
    gz = o.conv1d_bwd_f64(p["x"], p["weight"], du, bias=p["bias"], x_prev=np.zeros((1, 2, 2)), silu=True)
    for k in ("dx", "dweight", "dbias", "dx_prev"):
        _close(g0[k], gz[k], 1e-15, 1e-15, "conv no x_prev %s" % k)


def conv_bwd_autograd(o):
    import torch
    import torch.nn.functional as F
    rng = _rng(25)
    batch, dim, seqlen = 3, 4, 17
    for width in (1, 2, 4):
        for silu in (False, True):
            p = _conv_problem(rng, batch, dim, seqlen, width)
            du = rng.standard_normal((batch, dim, seqlen))
            g = o.conv1d_bwd_f64(p["x"], p["weight"], du, bias=p["bias"], x_prev=p["x_prev"], silu=silu)
            t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
            xin = torch.cat([t["x_prev"], t["x"]], dim=-1)  # [x_prev, x]: the K-1 inputs before token 0 first
            v = F.conv1d(xin, t["weight"].unsqueeze(1), t["bias"], groups=dim)
            u = F.silu(v) if silu else v
            (u * torch.tensor(du)).sum().backward()
            for name, key in (("x", "dx"), ("weight", "dweight"), ("bias", "dbias"), ("x_prev", "dx_prev")):
                _close(g[key], t[name].grad.numpy(), 1e-12, 1e-12, "conv autograd K=%d silu=%s d/d%s" %
                       (width, silu, name))


ALL = [worked_examples, lti_closed_form, bruteforce, single_step, persistence, forgetting, split_carry, linearity,
       softplus_silu, decode_is_scan, channel_subset, conv_library, conv_taps, conv_causality, conv_split_carry,
       bwd_finite_diff, bwd_autograd, zoh_van_loan, zoh_fixed_point, zoh_limits, zoh_decode, zoh_bwd, complex_real_limit,
       complex_block_expm, complex_lti, complex_bwd, conv_bwd_finite_diff, conv_bwd_autograd]
