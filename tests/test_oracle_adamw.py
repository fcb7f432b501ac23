"""Pins for the oracle's AdamW phase, skip path and loss scaler (not GPU).

* First step from m = v = 0: the bias corrections cancel the moment weights,
  so master1 = master0 * (1 - lr*wd) - lr * g / (|g| + eps) (closed form), and
  exactly master0 * (1 - lr*wd) where g = 0.
* torch.optim.AdamW (CPU, fp32, foreach=False) from the same state and the same
  gradient: the published algorithm (decoupled decay, bias-corrected moments,
  eps outside the root) agrees to a few ulp of each term.  This pins the
  formula, not our operation order.
* The fp32 step stays within a few ulp of the same update evaluated in fp64.
* Overflow skips the step: state bit-unchanged, t unchanged, scale halved.
* Scale invariance: power-of-two loss scales give bit-identical updates.
* Union invariant (ZeRO 优化器 training loop: reduce to owners, each owner
  steps its own parameters): all owners stepped with the global norm equal one
  unsharded step over the whole flat buffer, bit for bit.
* Loss scaler: closed forms for the fragmented-bucket schedule and a brute-force
  window check.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W

FP16, BF16 = oracle.FP16, oracle.BF16
EPS32 = 2.0 ** -23


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(np.maximum(x, np.float32(2.0 ** -126))).astype(np.float64)


def _grads(n, world, dtype, sigma, scale, seed=7, step=1, first=0):
    spec = synth.normal_spec(sigma, dtype)
    if scale != 1.0:
        spec = synth.scaled(spec, scale)
    out = []
    for r in range(world):
        a = np.empty(n, np.uint16)
        synth.fill_host(a, first, synth.stream_key(seed, synth.KIND_GRAD, step, r), spec)
        out.append(a)
    return out


def _param16(n, dtype, seed=7):
    a = np.empty(n, np.uint16)
    synth.fill_host(a, 0, synth.stream_key(seed, synth.KIND_INIT, 0, 0),
                    synth.normal_spec(0.02, dtype))
    return a


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_first_step_closed_form(dtype):
    n = 4096
    p16 = _param16(n, dtype)
    st = oracle.OwnerState.from_param16(p16, dtype)
    master0 = st.master.copy()
    g16 = _grads(n, 1, dtype, 1e-3, 1.0)[0]
    g16[:64] = 0                                   # zero gradients
    hp = oracle.HParams(max_grad_norm=0.0)
    oracle.adamw(st.master, st.exp_avg, st.exp_avg_sq, st.param16, g16, dtype, 1.0, 0.0, 0, hp, 1)
    c = oracle.adam_consts(hp, 1)
    decayed = (master0 * np.float32(c["decay"])).astype(np.float32)
    g = oracle.decode16(g16, dtype)
    want = decayed.astype(np.float64) - float(np.float32(hp.lr)) * g / (np.abs(g) + float(np.float32(hp.eps)))
    # g = 0: exactly the decayed weight
    assert np.array_equal(st.master[:64], decayed[:64])
    err = np.abs(st.master.astype(np.float64) - want)
    assert (err <= 2 * _ulp32(want) + 8 * EPS32 * hp.lr).all()
    # when |g| >> eps the step is lr * sign(g)
    big = np.abs(g) > 1e-5
    assert np.allclose(st.master[big], decayed[big] - hp.lr * np.sign(g[big]), rtol=0, atol=1e-6)
    # the 16-bit copy is the rounded master
    assert np.array_equal(st.param16, oracle.encode16(st.master, dtype))


@pytest.mark.parametrize("max_norm", [0.05, 1.0])
def test_matches_torch_adamw_step_by_step(max_norm):
    """torch.nn.utils.clip_grad_norm_ on the unscaled gradient, then
    torch.optim.AdamW.  max_norm 0.05 clips every step (the norm is ~0.14),
    1.0 never does."""
    n = 5000
    dtype = FP16
    hp = oracle.HParams(lr=float(np.float32(1e-3)), beta1=float(np.float32(0.9)),
                        beta2=float(np.float32(0.999)), eps=float(np.float32(1e-8)),
                        weight_decay=float(np.float32(0.01)), max_grad_norm=max_norm)
    st = oracle.OwnerState.from_param16(_param16(n, dtype), dtype)
    scale = 2.0 ** 16
    worst = {"m": 0.0, "v": 0.0, "p": 0.0}
    for t in range(1, 11):
        red = oracle.reduce(_grads(n, 4, dtype, 1e-3, scale, step=t), dtype)
        inv = 1.0 / scale
        flag, sumsq = oracle.check(red, dtype, inv)
        g_unscaled = (oracle.decode16(red, dtype).astype(np.float32)
                      * np.float32(inv)).astype(np.float32)

        p = torch.nn.Parameter(torch.from_numpy(st.master.copy()))
        p.grad = torch.from_numpy(g_unscaled.copy())
        norm = float(torch.nn.utils.clip_grad_norm_([p], max_norm))
        assert (norm > max_norm) == (max_norm < 1.0)
        g = p.grad.numpy().copy()
        opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                                weight_decay=hp.weight_decay, foreach=False, fused=False)
        # give torch the oracle's state as of step t-1
        opt.state[p]["step"] = torch.tensor(float(t - 1))
        opt.state[p]["exp_avg"] = torch.from_numpy(st.exp_avg.copy())
        opt.state[p]["exp_avg_sq"] = torch.from_numpy(st.exp_avg_sq.copy())
        m_prev, v_prev, p_prev = st.exp_avg.copy(), st.exp_avg_sq.copy(), st.master.copy()
        opt.step()
        oracle.adamw(st.master, st.exp_avg, st.exp_avg_sq, st.param16, red, dtype, inv, sumsq,
                     flag, hp, t)

        gd = g.astype(np.float64)
        mag_m = hp.beta1 * np.abs(m_prev) + (1 - hp.beta1) * np.abs(gd)
        mag_v = hp.beta2 * v_prev + (1 - hp.beta2) * gd * gd
        dm = np.abs(st.exp_avg - opt.state[p]["exp_avg"].numpy()) / (mag_m + 1e-30)
        dv = np.abs(st.exp_avg_sq - opt.state[p]["exp_avg_sq"].numpy()) / (mag_v + 1e-30)
        upd = np.abs(p_prev.astype(np.float64) - st.master)
        # torch's fp32 clip coefficient differs from the oracle's by a few ulp;
        # through m that moves the update by lr*(1-b1)|g|*delta/bc1/(sqrt(vh)+eps)
        delta = 0.0 if max_norm >= 1.0 else 8 * EPS32
        bc1, bc2 = 1 - hp.beta1 ** t, 1 - hp.beta2 ** t
        via_m = (hp.lr * (1 - hp.beta1) * np.abs(gd) * delta / bc1
                 / (np.sqrt(st.exp_avg_sq / bc2) + hp.eps))
        dp = np.abs(st.master - p.detach().numpy()) / (_ulp32(st.master) + 8 * EPS32 * upd + via_m)
        worst = {"m": max(worst["m"], dm.max()), "v": max(worst["v"], dv.max()),
                 "p": max(worst["p"], dp.max())}
    # clipping adds torch's fp32 norm and coefficient (a few ulp) to both sides' terms
    tol = 4 * EPS32 if max_norm >= 1.0 else 12 * EPS32
    assert worst["m"] <= tol
    # unclipped, v = b2*v + (1-b2)*g^2 rounds three times on each side: 4 ulp
    # of its magnitude bound the difference.  Clipped, both g^2 terms carry
    # twice the relative difference of the two fp32 clip factors.
    assert worst["v"] <= (tol if max_norm >= 1.0 else 2 * tol)
    assert worst["p"] <= 2.0


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_fp32_step_within_bound_of_fp64_step(dtype):
    n = 20000
    hp = oracle.HParams(max_grad_norm=1.0)
    st = oracle.OwnerState.from_param16(_param16(n, dtype), dtype)
    scale = 2.0 ** 16 if dtype == FP16 else 1.0
    sigma = 1e-3 if dtype == FP16 else 1e-4
    for t in range(1, 6):
        red = oracle.reduce(_grads(n, 8, dtype, sigma, scale, step=t), dtype)
        inv = 1.0 / scale
        flag, sumsq = oracle.check(red, dtype, inv)
        coef = oracle.clip_coef(hp.max_grad_norm, sumsq)
        pm, mm, vm = oracle.adamw_f64(st.master, st.exp_avg, st.exp_avg_sq, red, dtype, inv,
                                      float(np.float32(coef)), hp, t)
        prev = st.master.copy()
        m_prev, v_prev = st.exp_avg.astype(np.float64), st.exp_avg_sq.astype(np.float64)
        oracle.adamw(st.master, st.exp_avg, st.exp_avg_sq, st.param16, red, dtype, inv, sumsq,
                     flag, hp, t)
        # Each stored value is within a few roundings of the terms that formed
        # it: m = b1*m + (1-b1)*g and v = b2*v + (1-b2)*g^2 round at most three
        # times; the update adds the propagated error of m.
        g = np.abs(oracle.decode16(red, dtype) * inv * float(np.float32(coef)))
        mag_m = hp.beta1 * np.abs(m_prev) + (1 - hp.beta1) * g
        mag_v = hp.beta2 * v_prev + (1 - hp.beta2) * g * g
        assert (np.abs(st.exp_avg - mm) <= 3 * EPS32 * mag_m).all()
        assert (np.abs(st.exp_avg_sq - vm) <= 4 * EPS32 * mag_v).all()
        bc1 = 1 - hp.beta1 ** t
        bc2 = 1 - hp.beta2 ** t
        upd = np.abs(prev.astype(np.float64) - pm)
        from_m = hp.lr * (3 * EPS32 * mag_m / bc1) / (np.sqrt(vm / bc2) + hp.eps)
        assert (np.abs(st.master - pm) <= 2 * _ulp32(pm) + from_m + 12 * EPS32 * upd).all()


def test_skip_on_overflow_leaves_state_untouched():
    n = 3000
    dtype = FP16
    st = oracle.OwnerState.from_param16(_param16(n, dtype), dtype)
    hp = oracle.HParams()
    scaler = oracle.Scaler(2.0 ** 16)
    t = 0
    for s in range(1, 4):
        grads = _grads(n, 8, dtype, 1e-3, scaler.scale, step=s)
        res, t = oracle.step([st], [grads], dtype, hp, scaler, t)
        assert res.applied
    before = st.copy()
    grads = _grads(n, 8, dtype, 1e-3, scaler.scale, step=4)
    grads[3][1234] = synth.POS_INF[FP16]
    # the AdamW phase on its own writes nothing when handed the flag
    red = oracle.reduce(grads, dtype)
    flag, sumsq = oracle.check(red, dtype, 1.0 / scaler.scale)
    assert flag == 1
    oracle.adamw(st.master, st.exp_avg, st.exp_avg_sq, st.param16, red, dtype,
                 1.0 / scaler.scale, sumsq, flag, hp, t + 1)
    for a, b in ((st.master, before.master), (st.exp_avg, before.exp_avg),
                 (st.exp_avg_sq, before.exp_avg_sq), (st.param16, before.param16)):
        assert np.array_equal(a.view(np.uint32 if a.dtype == np.float32 else np.uint16),
                              b.view(np.uint32 if b.dtype == np.float32 else np.uint16))
    res, t2 = oracle.step([st], [grads], dtype, hp, scaler, t)
    assert res.overflow == 1 and not res.applied and t2 == t
    for a, b in ((st.master, before.master), (st.exp_avg, before.exp_avg),
                 (st.exp_avg_sq, before.exp_avg_sq), (st.param16, before.param16)):
        assert np.array_equal(a.view(np.uint32 if a.dtype == np.float32 else np.uint16),
                              b.view(np.uint32 if b.dtype == np.float32 else np.uint16))
    assert scaler.scale == 2.0 ** 15 and scaler.clean == 0 and scaler.skipped == 1
    # a finite pair whose sum overflows binary16 also trips the flag
    grads = _grads(n, 8, dtype, 1e-3, scaler.scale, step=5)
    for r in range(8):
        grads[r][10] = 0x7B53          # 8 x 60000 > 65504
    res, _ = oracle.step([st], [grads], dtype, hp, scaler, t)
    assert res.overflow == 1


def test_scale_invariance():
    n = 4000
    dtype = FP16
    hp = oracle.HParams(max_grad_norm=1.0)
    finals = []
    for scale in (1.0, 2.0 ** 8, 2.0 ** 16):
        st = oracle.OwnerState.from_param16(_param16(n, dtype), dtype)
        scaler = oracle.Scaler(scale, window=10 ** 9)
        t = 0
        for s in range(1, 6):
            res, t = oracle.step([st], [_grads(n, 8, dtype, 1e-3, scale, step=s)], dtype, hp,
                                 scaler, t)
            assert res.applied
        finals.append(st)
    for other in finals[1:]:
        assert np.array_equal(finals[0].master.view(np.uint32), other.master.view(np.uint32))
        assert np.array_equal(finals[0].exp_avg.view(np.uint32), other.exp_avg.view(np.uint32))
        assert np.array_equal(finals[0].exp_avg_sq.view(np.uint32),
                              other.exp_avg_sq.view(np.uint32))
        assert np.array_equal(finals[0].param16, other.param16)


def test_divisor_averages_the_gradient():
    """Averaging over N ranks is the sum divided by N, folded into the
    unscale factor 1/(S*N): for N = 8 (a power of two, so every scaling is
    exact) the squared norm is the summed one / 64, and the update equals the
    one from the summed gradient at loss scale 8*S, bit for bit."""
    n = 3000
    dtype = FP16
    hp = oracle.HParams(max_grad_norm=0.05)
    a = oracle.OwnerState.from_param16(_param16(n, dtype), dtype)
    b = a.copy()
    plain = a.copy()
    grads = _grads(n, 8, dtype, 1e-3, 1024.0)
    ra, _ = oracle.step([a], [grads], dtype, hp, oracle.Scaler(1024.0), 0, divisor=8)
    rb, _ = oracle.step([b], [grads], dtype, hp, oracle.Scaler(8 * 1024.0), 0)
    rp, _ = oracle.step([plain], [grads], dtype, hp, oracle.Scaler(1024.0), 0)
    assert ra.sumsq == rp.sumsq / 64 and ra.sumsq == rb.sumsq
    for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert not np.array_equal(a.exp_avg.view(np.uint32), plain.exp_avg.view(np.uint32))


@pytest.mark.parametrize("world,clip", [(2, 0.0), (3, 1.0), (8, 0.5)])
def test_union_of_owner_steps_equals_unsharded_step(world, clip):
    # a small flat group: ragged tensor sizes, padded tail
    numels = [37, 1, 250, 1024, 3, 77]
    dtype = FP16
    offs, parts, padded = oracle.layout(numels, world, 2)
    phi = sum(numels)
    hp = oracle.HParams(max_grad_norm=clip)
    full16 = np.zeros(padded, np.uint16)
    full16[:phi] = _param16(phi, dtype)
    whole = oracle.OwnerState.from_param16(full16, dtype)
    owners = [oracle.OwnerState.from_param16(full16[parts[p]:parts[p + 1]], dtype)
              for p in range(world)]
    sc_whole, sc_owner = oracle.Scaler(2.0 ** 16), oracle.Scaler(2.0 ** 16)
    t_whole = t_owner = 0
    for s in range(1, 5):
        ranks = []
        for g in _grads(phi, world, dtype, 1e-3, 2.0 ** 16, step=s):
            full = np.zeros(padded, np.uint16)
            full[:phi] = g
            ranks.append(full)
        res_w, t_whole = oracle.step([whole], [ranks], dtype, hp, sc_whole, t_whole)
        per_owner = [[r[parts[p]:parts[p + 1]] for r in ranks] for p in range(world)]
        res_o, t_owner = oracle.step(owners, per_owner, dtype, hp, sc_owner, t_owner)
        assert res_w.overflow == res_o.overflow
        assert res_w.sumsq == pytest.approx(res_o.sumsq, rel=1e-15)
    glued = {k: np.concatenate([getattr(o, k) for o in owners])
             for k in ("master", "exp_avg", "exp_avg_sq", "param16")}
    assert np.array_equal(glued["master"].view(np.uint32), whole.master.view(np.uint32))
    assert np.array_equal(glued["exp_avg"].view(np.uint32), whole.exp_avg.view(np.uint32))
    assert np.array_equal(glued["exp_avg_sq"].view(np.uint32), whole.exp_avg_sq.view(np.uint32))
    assert np.array_equal(glued["param16"], whole.param16)
    # padding never moves: zero master, zero grads -> stays exactly zero
    assert (whole.master[phi:] == 0).all() and (whole.param16[phi:] == 0).all()


def test_loss_scaler_fragmented_bucket_schedule():
    """Inf/NaN in every 4th of 40 steps, window 1000: ten halvings from 2^16
    to 2^6 = 64, ten skipped steps, t = 30 applied steps."""
    sc = oracle.Scaler(2.0 ** 16, min_scale=1.0, window=1000)
    t = 0
    for s in range(1, 41):
        overflow = int(s % 4 == 0)
        if not overflow:
            t += 1
        sc.update(overflow)
    assert sc.scale == 64.0 and sc.skipped == 10 and t == 30


def test_loss_scaler_window_and_floor():
    # window 3: doubles after three clean steps in a row, halves on overflow
    sc = oracle.Scaler(8.0, min_scale=1.0, window=3)
    seq = [0, 0, 0, 0, 1, 0, 0, 1, 1, 1, 1, 1, 0, 0, 0]
    want = [8, 8, 16, 16, 8, 8, 8, 4, 2, 1, 1, 1, 1, 1, 2]
    got = []
    for f in seq:
        sc.update(f)
        got.append(sc.scale)
    assert got == want
    assert sc.skipped == 6


def test_workload_init_is_master_clone():
    # the fp32 master is the float of the 16-bit partition, so rounding it back
    # gives the 16-bit partition again
    wl = W.WORKLOADS["toy"]
    p16 = _param16(10000, wl.dtype)
    st = oracle.OwnerState.from_param16(p16, wl.dtype)
    assert np.array_equal(oracle.encode16(st.master, wl.dtype), p16)
    assert (st.exp_avg == 0).all() and (st.exp_avg_sq == 0).all()
