"""Seeded random configurations of the checkpoint kernels against the oracle: layer
count, units per layer, unit size, keep probability (empty and full masks included),
checkpoint / private slot maps.  FP32 pack / restore bit-exact; INT8 pack: scales
bit-exact, codes off by at most 1 on at most 0.1% of values; INT8 restore of the oracle's
checkpoint bit-exact; the fused restore + replay against the oracle's restore then replay
and bit for bit against the library's two calls.  Slots no pair names keep their sentinel
bytes."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, need_gpu, torch

pytestmark = pytest.mark.gpu
N_CASES = 10
CODE_FRAC = 1e-3


def _keep(g):
    u = g.random()
    return 0.0 if u < 0.1 else 1.0 if u < 0.2 else float(g.uniform(0.05, 0.95))


def _maps(g, S_src, S_dst):
    N = int(g.integers(1, min(S_src, S_dst) + 1))
    return (g.permutation(S_src)[:N].astype(np.int32), g.permutation(S_dst)[:N].astype(np.int32))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_pack_restore_fp32(i):
    hla = need_gpu()
    g = np.random.default_rng(7100 + i)
    ub = int(g.choice([16, 48, 512, 1040, 4096, 65536]))
    L = int(g.integers(1, 6))
    n_units = int(g.integers(1, 41 if ub <= 4096 else 5))
    S_act = int(g.integers(1, 7))
    active = g.integers(0, 256, size=(L, S_act, n_units, ub), dtype=np.uint8)
    mask = (g.random((L, n_units)) < _keep(g)).astype(np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    S_ckpt = S_act + int(g.integers(0, 3))
    src, dst = _maps(g, S_act, S_ckpt)
    packed = torch.full((max(S_ckpt * R * ub, 16),), 0xCD, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    act_d = dev(active.reshape(-1))
    hla.dasc_pack(act_d, S_act * n_units * ub, S_act, L, n_units, ub, dev(offsets),
                  dev(unit_index), R, dev(src), dev(dst), packed, S_ckpt, err_flag=err)
    ref = oracle.dasc_pack(active, offsets, unit_index, src, dst, S_ckpt)
    got = host(packed)[: S_ckpt * R * ub].reshape(S_ckpt, R, ub)
    for d_ in dst:
        assert np.array_equal(got[d_], ref[d_])
    others = sorted(set(range(S_ckpt)) - set(dst.tolist()))
    assert (got[others] == 0xCD).all()
    S_dst = S_act + int(g.integers(0, 3))
    src2, dst2 = _maps(g, S_ckpt, S_dst)
    out0 = g.integers(0, 256, size=(L, S_dst, n_units, ub), dtype=np.uint8)
    out = dev(out0.reshape(-1))
    ckpt = dev(ref.reshape(-1)) if R else dev(np.zeros(16, np.uint8))  # no unit kept: any buffer
    hla.dasc_restore(ckpt, S_ckpt, R, dev(unit_pos.reshape(-1)), L, n_units, ub,
                     dev(src2), dev(dst2), out, S_dst * n_units * ub, S_dst, err_flag=err)
    ref_out = out0.copy()
    oracle.dasc_restore(ref, offsets, unit_index, L, n_units, src2, dst2, ref_out)
    assert np.array_equal(host(out).reshape(ref_out.shape), ref_out)
    assert int(err.item()) == 0


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_pack_restore_int8(i):
    hla = need_gpu()
    g = np.random.default_rng(7200 + i)
    unit_rows = int(g.choice([1, 2, 4, 8, 128]))
    dv = int(g.choice([64, 128]))
    L = int(g.integers(1, 5))
    n_units = int(g.integers(1, 41 if unit_rows <= 8 else 6))
    S_ = int(g.integers(1, 6))
    act = (g.standard_normal((L, S_, n_units, unit_rows, dv)) * g.uniform(0.01, 2.0)).astype(
        np.float32)
    mask = (g.random((L, n_units)) < _keep(g)).astype(np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    S_ckpt = S_ + int(g.integers(0, 3))
    src, dst = _maps(g, S_, S_ckpt)
    codes = torch.full((max(S_ckpt * R * unit_rows * dv, 16),), 99, dtype=torch.int8,
                       device="cuda")
    scales = torch.full((max(S_ckpt * R * unit_rows, 4),), -1.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_pack_int8(dev(act), S_ * n_units * unit_rows * dv * 4, S_, L, n_units, unit_rows,
                       dv, dev(offsets), dev(unit_index), R, dev(src), dev(dst), codes, scales,
                       S_ckpt, err_flag=err)
    c_o, s_o = oracle.dasc_pack_int8(act, offsets, unit_index, src, dst, S_ckpt)
    n_c, n_s = S_ckpt * R * unit_rows * dv, S_ckpt * R * unit_rows
    c_g = host(codes)[:n_c].reshape(c_o.shape)
    s_g = host(scales)[:n_s].reshape(s_o.shape)
    for d_ in dst:
        assert np.array_equal(s_g[d_], s_o[d_])
        diff = np.abs(c_g[d_].astype(int) - c_o[d_].astype(int))
        assert diff.max(initial=0) <= 1 and (diff.size == 0 or (diff > 0).mean() <= CODE_FRAC)
    others = [s for s in range(S_ckpt) if s not in dst]
    assert (c_g[others] == 99).all() and (s_g[others] == -1.0).all()
    S_dst = S_ + int(g.integers(0, 3))
    src2, dst2 = _maps(g, S_ckpt, S_dst)
    out0 = np.full((L, S_dst, n_units, unit_rows, dv), 3.5, np.float32)
    out = dev(out0)
    hla.dasc_restore_int8(dev(c_o.reshape(-1)) if R else dev(np.zeros(16, np.int8)),  # R = 0:
                          dev(s_o.reshape(-1)) if R else dev(np.zeros(4, np.float32)),  # any buffer
                          S_ckpt, R, dev(unit_pos.reshape(-1)), L, n_units, unit_rows, dv,
                          dev(src2), dev(dst2), out, S_dst * n_units * unit_rows * dv * 4, S_dst,
                          err_flag=err)
    ref = oracle.dasc_restore_int8(c_o, s_o, offsets, unit_index, L, n_units, src2, dst2,
                                   out0.copy())
    assert np.array_equal(host(out), ref)
    assert int(err.item()) == 0


@pytest.mark.parametrize("i", range(6))
def test_random_refresh_local(i):
    """The dasc-wr copy-back of the local units (the inverted mask's plan) from scratch
    slots into active slots, bit-exact; every other byte of the active state untouched."""
    hla = need_gpu()
    g = np.random.default_rng(7300 + i)
    ub = int(g.choice([16, 48, 512, 1040, 4096]))
    L, n_units = int(g.integers(1, 5)), int(g.integers(1, 41))
    S_s, S_a = int(g.integers(1, 5)), int(g.integers(1, 7))
    scratch = g.integers(0, 256, size=(L, S_s, n_units, ub), dtype=np.uint8)
    active = g.integers(0, 256, size=(L, S_a, n_units, ub), dtype=np.uint8)
    local = 1 - (g.random((L, n_units)) < _keep(g)).astype(np.uint8)
    offsets, unit_index, _, R_local = hla.dasc_plan(local)
    src, dst = _maps(g, S_s, S_a)
    act_d = dev(active.reshape(-1))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_refresh_local(dev(scratch.reshape(-1)), S_s * n_units * ub, S_s, act_d,
                           S_a * n_units * ub, S_a, L, n_units, ub, dev(offsets),
                           dev(unit_index), R_local, dev(src), dev(dst), err_flag=err)
    ref = oracle.dasc_refresh_local(scratch, active.copy(), local, src, dst)
    assert np.array_equal(host(act_d).reshape(active.shape), ref)
    assert int(err.item()) == 0


def test_refresh_local_device_errors():
    """A pair whose scratch or active slot is past its bound is skipped (HLA_DEVERR_SLOT);
    a local-plan entry past the units is skipped (HLA_DEVERR_PLAN); the rest is copied."""
    hla = need_gpu()
    g = np.random.default_rng(7399)
    L, S_s, S_a, n_units, ub = 2, 3, 4, 9, 64
    scratch = g.integers(0, 256, size=(L, S_s, n_units, ub), dtype=np.uint8)
    active = g.integers(0, 256, size=(L, S_a, n_units, ub), dtype=np.uint8)
    local = np.zeros((L, n_units), np.uint8)
    local[0, [1, 4]] = 1
    local[1, [0, 8]] = 1
    offsets, unit_index, _, R_local = hla.dasc_plan(local)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    act_d = dev(active.reshape(-1))
    src, dst = np.array([0, 7, 1], np.int32), np.array([2, 0, 9], np.int32)
    hla.dasc_refresh_local(dev(scratch.reshape(-1)), S_s * n_units * ub, S_s, act_d,
                           S_a * n_units * ub, S_a, L, n_units, ub, dev(offsets),
                           dev(unit_index), R_local, dev(src), dev(dst), err_flag=err)
    assert int(err.item()) == hla.DEVERR_SLOT
    ref = oracle.dasc_refresh_local(scratch, active.copy(), local, src[:1], dst[:1])
    assert np.array_equal(host(act_d).reshape(active.shape), ref)
    # a plan entry naming unit 12 of 9: that unit is skipped, the others are copied
    bad = unit_index.copy()
    bad[2] = 12                                # layer 1's first local unit (unit 0)
    act2 = dev(active.reshape(-1))
    err.zero_()
    hla.dasc_refresh_local(dev(scratch.reshape(-1)), S_s * n_units * ub, S_s, act2,
                           S_a * n_units * ub, S_a, L, n_units, ub, dev(offsets), dev(bad),
                           R_local, dev(src[:1]), dev(dst[:1]), err_flag=err)
    assert int(err.item()) == hla.DEVERR_PLAN
    ref2 = ref.copy()
    ref2[1, 2, 0] = active[1, 2, 0]            # not copied
    assert np.array_equal(host(act2).reshape(active.shape), ref2)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_restore_replay(i):
    """The fused restore + replay on random geometry (layers, heads, head shape, unit size
    from one key channel to a whole head, draft count, input and readout types or no
    readouts, decay kind, FP32 or INT8 checkpoints, masks from empty to full, slot maps,
    accepted counts with out-of-range values): against the oracle's restore then replay,
    and bit for bit against the library's restore followed by replay_accepted per
    layer."""
    import oracle_par

    hla = need_gpu()
    g = np.random.default_rng(7300 + i)
    L = int(g.integers(1, 5))
    H = int(g.integers(1, 7))
    dk, dv = (int(g.choice([64, 128])) for _ in range(2))
    K = int(g.integers(1, 17))
    vec = bool(g.integers(0, 2))
    in_dt = str(g.choice(["f32", "bf16", "f16"]))
    out_dt = str(g.choice(["f32", "bf16", "f16"]))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    ur = int(g.choice([1, 2, 8, dk]))  # key channels per unit
    n_units = H * dk // ur
    mask = (g.random((L, n_units)) < _keep(g)).astype(np.uint8)
    _, _, unit_pos, R = hla.dasc_plan(mask)
    S_ckpt, S_dst = int(g.integers(1, 6)), int(g.integers(1, 8))
    src, dst = _maps(g, S_ckpt, S_dst)
    N = len(src)
    packed = (g.standard_normal((S_ckpt, R, ur * dv)) * 0.05).astype(np.float32)
    q8 = bool(g.integers(0, 2))          # an INT8 checkpoint: the state starts as code x scale
    want_out = bool(g.integers(0, 4))    # three cases in four with readouts
    if q8:
        codes = g.integers(-127, 128, size=(S_ckpt, R, ur, dv)).astype(np.int8)
        scales = (g.uniform(0.5, 2.0, size=(S_ckpt, R, ur)) * 0.05 / 127).astype(np.float32)
        packed = (codes.astype(np.float32) * scales[..., None]).reshape(S_ckpt, R, ur * dv)
    # inputs: q, k unit vectors, stored in the input type; values the kernel reads exactly
    qk = g.standard_normal((2, L, N, K, H, dk))
    qk /= np.linalg.norm(qk, axis=-1, keepdims=True)
    v = g.standard_normal((L, N, K, H, dv)) * 0.5
    x_t = {n: torch.from_numpy(a).to(tdt[in_dt])
           for n, a in (("q", qk[0]), ("k", qk[1]), ("v", v))}
    alpha = g.uniform(0.9, 0.9999, size=(L, N, K, H) + ((dk,) if vec else ())).astype(np.float32)
    beta = g.uniform(0.05, 0.95, size=(L, N, K, H)).astype(np.float32)
    n_acc = g.integers(-2, K + 3, size=N).astype(np.int32)
    n_eff = np.clip(n_acc, 0, K)
    xd = {n: t.cuda() for n, t in x_t.items()}
    xd.update(alpha=dev(alpha), beta=dev(beta))
    pk = dev(packed)
    pos = dev(unit_pos.reshape(-1))
    if q8:
        cd, sc = dev(codes), dev(scales)

    def fused():
        st = torch.full((L, S_dst, H, dk, dv), 3.0, device="cuda")
        out = torch.full((L, N, K, H, dv), 5.0, device="cuda", dtype=tdt[out_dt])
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        args = (pos, dev(src), dev(dst), st, xd["q"], xd["k"], xd["v"], xd["alpha"],
                xd["beta"], dev(n_acc), int(vec))
        o = out if want_out else None
        if q8:
            hla.dasc_restore_int8_replay(cd, sc, *args, out=o, err_flag=err)
        else:
            hla.dasc_restore_replay(pk, *args, out=o, err_flag=err)
        return st, out, int(err.item())

    st, out, err = fused()
    assert err == (hla.DEVERR_ACCEPT if (n_acc != n_eff).any() else 0)
    # the two-call chain
    st2 = torch.full((L, S_dst, H, dk, dv), 3.0, device="cuda")
    out2 = torch.full((L, N, K, H, dv), 5.0, device="cuda", dtype=tdt[out_dt])
    ub = ur * dv * 4
    if q8:
        hla.dasc_restore_int8(cd if R else dev(np.zeros(16, np.int8)),
                              sc if R else dev(np.zeros(4, np.float32)), S_ckpt, R, pos, L,
                              n_units, ur, dv, dev(src), dev(dst), st2, S_dst * n_units * ub,
                              S_dst)
    else:
        hla.dasc_restore(pk if R else dev(np.zeros(4, np.float32)), S_ckpt, R, pos, L,
                         n_units, ub, dev(src), dev(dst), st2, S_dst * n_units * ub, S_dst)
    for l in range(L):
        hla.replay_accepted(st2[l], xd["q"][l], xd["k"][l], xd["v"][l], xd["alpha"][l],
                            xd["beta"][l], dev(n_acc), int(vec),
                            out=out2[l] if want_out else None, slot=dev(dst),
                            want_out=want_out)
    assert torch.equal(st, st2) and torch.equal(out, out2)
    # the oracle
    got, o = host(st), host(out)
    x64 = {"q": x_t["q"].double().numpy(), "k": x_t["k"].double().numpy(),
           "v": x_t["v"].double().numpy(), "alpha": alpha.astype(np.float64),
           "beta": beta.astype(np.float64)}
    tol_o = 1e-5 if out_dt == "f32" else (2.0 ** -8 if out_dt == "bf16" else 2.0 ** -10)
    for l in range(L):
        S64 = np.zeros((N, H * dk // ur, ur, dv))
        for u in range(n_units):
            if unit_pos[l, u] >= 0:
                S64[:, u] = packed[src, unit_pos[l, u]].reshape(N, ur, dv)
        S64 = S64.reshape(N, H, dk, dv)
        o_ref, scale = oracle_par.replay_terms(S64, {n: x64[n][l] for n in x64}, n_acc,
                                               per_channel=vec)
        assert oracle_par.rel_err_tiles(got[l][dst], S64) <= 1e-5
        if not want_out:
            assert (o[l] == 5.0).all()
            continue
        rows = np.arange(K)[None, :] < n_eff[:, None]
        e = np.where(rows[:, :, None, None], np.abs(o[l] - o_ref), 0.0).max(axis=-1)
        assert float((e / np.maximum(scale, 1e-30)).max()) <= tol_o
        assert (o[l][~rows] == 5.0).all()
    others = sorted(set(range(S_dst)) - set(dst.tolist()))
    assert (got[:, others] == 3.0).all()
