"""GPU parity of dasc_restore_replay: a checkpoint of whole-head units restored into
private slots with each request's accepted drafts replayed on the way ([dasc] §4.2
dasc-nr; [K3] "Speculative decoding without state snapshots").

Every case is checked twice:

* against the oracle: its restore of the same packed bits (retained heads copied,
  omitted heads zero), then its replay of the first n_b drafts of each layer in float64
  (state within 1e-5 of max|oracle| per head tile, each accepted readout within 1e-5
  of the size of its terms, max_j sum_i |S_t[i][j] q_t,i|, per head and token);
* bit for bit against the library's two-call chain, dasc_restore followed by
  replay_accepted on each layer, which the fused kernel must reproduce exactly (same
  per-token arithmetic, the state held in registers in between).

Small cases span GDN / KDA decay, FP32 / BF16 / FP16 inputs and readouts, all four
head shapes, K = 1, 5 and 16, accepted counts from 0 to K with clamping, slot maps that
permute, leave destination slots alone and name bad slots, a plan entry past the
checkpoint, a checkpoint that retains nothing, no pairs, and units smaller than a head
(1 to 32 key channels).  The full-size cases are the two checkpoint workloads: 4 layers x
512 requests x 32 heads x 128 x 128, K = 8 drafts, one accepted count per request for
every layer; GDN heads with 64 of 128 layer-heads retained, and KDA single key channels
selected by static horizons."""
import numpy as np
import pytest

import oracle
import oracle_par
import synth
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")
TORCH_DT = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def _cfg(kind, dk, dv, in_dtype, K, H=4, L=3, S=7, seed=0):
    base = synth.CONFIGS["dasc_gdn"]
    return synth.shrink(base, H=H, dk=dk, dv=dv, in_dtype=in_dtype, K=K, L=L, slots=S,
                        decay="vector" if kind == "kda" else "scalar",
                        seed=base.seed + 11 * dk + 5 * dv + K + seed
                        + (3 if kind == "kda" else 0), plan_seed=base.plan_seed + seed)


def _checkpoint(cfg, mask):
    """The oracle's pack of every slot's retained heads (uint8 [S, R, dk*dv*4]) and the
    plan tables."""
    hla = need_gpu()
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    ub = cfg.dk * cfg.dv * 4
    act = np.stack([synth.initial_state(cfg, S=cfg.slots, layer=l) for l in range(cfg.L)])
    ids = np.arange(cfg.slots, dtype=np.int32)
    packed = oracle.dasc_pack(act.view(np.uint8).reshape(cfg.L, cfg.slots, cfg.H, ub),
                              offsets, unit_index, ids, ids, cfg.slots)
    return packed, offsets, unit_index, unit_pos, R


def _drafts(cfg, N):
    """Each layer's draft projections for N requests, stacked [L, N, K, H, ...]."""
    xs = [synth.replay_inputs(cfg, l, B=N) for l in range(cfg.L)]
    return {n: np.stack([x[n] for x in xs]) for n in NAMES}


def _fused(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc, out_dtype, init):
    L, H = cfg.L, cfg.H
    st = torch.full((L, S_dst, H, cfg.dk, cfg.dv), init, device="cuda")
    out = torch.full((L, len(src), cfg.K, H, cfg.dv), 5.0, device="cuda",
                     dtype=getattr(torch, TORCH_DT[out_dtype]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = dev(np.ascontiguousarray(unit_pos, np.int32).reshape(-1))
    hla.dasc_restore_replay(packed_d, pos, dev(src), dev(dst), st, xd["q"], xd["k"], xd["v"],
                            xd["alpha"], xd["beta"], dev(n_acc),
                            1 if cfg.decay == "vector" else 0, out=out, err_flag=err)
    return st, out, int(err.item())


def _chain(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc, out_dtype, init,
           unit_rows=None):
    """dasc_restore, then replay_accepted layer by layer into the restored slots."""
    L, H = cfg.L, cfg.H
    ur = cfg.dk if unit_rows is None else unit_rows
    ub = ur * cfg.dv * 4
    n_units = H * cfg.dk // ur
    st = torch.full((L, S_dst, H, cfg.dk, cfg.dv), init, device="cuda")
    out = torch.full((L, len(src), cfg.K, H, cfg.dv), 5.0, device="cuda",
                     dtype=getattr(torch, TORCH_DT[out_dtype]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    S_ck, R = packed_d.shape[:2]
    src_d, dst_d, n_d = dev(src), dev(dst), dev(n_acc)
    pos = dev(np.ascontiguousarray(unit_pos, np.int32).reshape(-1))
    hla.dasc_restore(packed_d, S_ck, R, pos, L, n_units, ub, src_d, dst_d, st,
                     S_dst * n_units * ub, S_dst, err_flag=err)
    for l in range(L):
        hla.replay_accepted(st[l], xd["q"][l], xd["k"][l], xd["v"][l], xd["alpha"][l],
                            xd["beta"][l], n_d, 1 if cfg.decay == "vector" else 0, out=out[l],
                            slot=dst_d, err_flag=err)
    return st, out, int(err.item())


def _oracle(cfg, packed, offsets, unit_index, src, dst, S_dst, x64, n_acc, init,
            zero_heads=(), unit_rows=None, zero_rows=()):
    """The oracle's restore into a state filled with `init` (the heads (l, h) listed in
    zero_heads then zero-filled in the restored slots), then its replay per layer.
    Returns the state [L, S_dst, H, dk, dv] (float64), readouts [L, N, K, H, dv] and the
    readouts' term sizes [L, N, K, H]."""
    L, H, dk, dv = cfg.L, cfg.H, cfg.dk, cfg.dv
    ur = dk if unit_rows is None else unit_rows
    rest = np.full((L, S_dst, H, dk, dv), init, np.float32)
    oracle.dasc_restore(packed, offsets, unit_index, L, H * dk // ur, src, dst,
                        rest.view(np.uint8).reshape(L, S_dst, H * dk // ur, ur * dv * 4))
    for l, h in zero_heads:
        rest[l, dst, h] = 0.0
    for l, h, r0, r1 in zero_rows:
        rest[l, dst, h, r0:r1] = 0.0
    return _oracle_replay(cfg, rest, dst, x64, n_acc)


def _oracle_replay(cfg, rest, dst, x64, n_acc):
    """The oracle's replay of each layer's drafts into the restored slots dst of `rest`."""
    S64 = rest.astype(np.float64)
    outs, scales = [], []
    for l in range(cfg.L):
        Sl = np.ascontiguousarray(S64[l][dst])
        o, sc = oracle_par.replay_terms(Sl, {n: x64[n][l] for n in NAMES}, n_acc,
                                        per_channel=(cfg.decay == "vector"))
        S64[l][dst] = Sl
        outs.append(o)
        scales.append(sc)
    return S64, np.stack(outs), np.stack(scales)


def _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, K):
    got = host(st)
    assert oracle_par.rel_err_tiles(got.reshape(-1, *got.shape[-2:]),
                                    ref_st.reshape(-1, *ref_st.shape[-2:])) <= TOL
    o = host(out)
    rows = np.arange(K)[None, :] < np.clip(n_acc, 0, K)[:, None]       # [N, K]
    rows = np.broadcast_to(rows[None], o.shape[:3])
    assert (o[~rows] == 5.0).all()                                      # rows t >= n_b
    err = np.where(rows[..., None, None], np.abs(o - ref_out), 0.0).max(axis=-1)
    return float((err / np.maximum(scale, 1e-30)).max())


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("in_dtype,out_dtype", [("f32", "f32"), ("bf16", "f32"),
                                                ("f16", "f16"), ("bf16", "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_restore_replay_matches_oracle_and_chain(kind, in_dtype, out_dtype, dk, dv):
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, in_dtype, K=5)
    mask = synth.dasc_masks(cfg)
    packed, offsets, unit_index, unit_pos, R = _checkpoint(cfg, mask)
    assert 0 < R < cfg.L * cfg.H
    src = np.array([3, 0, 6, 2, 5], np.int32)                # checkpoint slots, permuted
    dst = np.array([1, 7, 4, 0, 2], np.int32)                # slots 3, 5, 6 are left alone
    n_acc = np.array([0, 5, 2, 7, -1], np.int32)             # 7 and -1 clamp to 5 and 0
    S_dst = 8
    x = _drafts(cfg, len(src))
    xd = dev_inputs(x, in_dtype)
    packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, dk * dv))
    st, out, err = _fused(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc,
                          out_dtype, 7.0)
    assert err == hla.DEVERR_ACCEPT
    st2, out2, err2 = _chain(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc,
                             out_dtype, 7.0)
    assert err2 == hla.DEVERR_ACCEPT
    assert torch.equal(st, st2) and torch.equal(out, out2)
    ref_st, ref_out, scale = _oracle(cfg, packed, offsets, unit_index, src, dst, S_dst,
                                     f64_inputs(x, in_dtype), n_acc, 7.0)
    err_o = _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, cfg.K)
    tol_o = TOL if out_dtype == "f32" else (2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -10)
    assert err_o <= tol_o
    # requests with nothing accepted hold the restored bits exactly; slots no pair names
    # keep what they held
    got = host(st)
    assert np.array_equal(got[:, [1, 2]], ref_st[:, [1, 2]].astype(np.float32))
    assert (got[:, [3, 5, 6]] == 7.0).all()


@pytest.mark.parametrize("kind,in_dtype", [("gdn", "bf16"), ("kda", "f32")])
@pytest.mark.parametrize("K", [1, 16])
def test_restore_replay_draft_counts_at_the_limits(K, kind, in_dtype):
    """K = 16 with FP32 inputs and a per-channel decay stages the most bytes per token in
    LDS (2 KiB per token at 128 x 128)."""
    hla = need_gpu()
    cfg = _cfg(kind, 128, 128, in_dtype, K=K, L=2, S=4, seed=1)
    packed, offsets, unit_index, unit_pos, R = _checkpoint(cfg, synth.dasc_masks(cfg))
    src = np.array([0, 1, 2, 3], np.int32)
    dst = np.array([3, 2, 1, 0], np.int32)
    n_acc = np.array([K, 0, K // 2, 1], np.int32)
    x = _drafts(cfg, 4)
    xd = dev_inputs(x, in_dtype)
    packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, -1))
    st, out, err = _fused(hla, cfg, packed_d, unit_pos, src, dst, 4, xd, n_acc, "f32", 0.0)
    st2, out2, _ = _chain(hla, cfg, packed_d, unit_pos, src, dst, 4, xd, n_acc, "f32", 0.0)
    assert err == 0 and torch.equal(st, st2) and torch.equal(out, out2)
    ref_st, ref_out, scale = _oracle(cfg, packed, offsets, unit_index, src, dst, 4,
                                     f64_inputs(x, in_dtype), n_acc, 0.0)
    assert _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, K) <= TOL


def test_restore_replay_device_errors_and_degenerate_plans():
    """Bad slots are skipped, a plan entry past the checkpoint starts its head from zero;
    both are reported.  A checkpoint that retains nothing starts every head from zero;
    no pairs touches nothing."""
    hla = need_gpu()
    cfg = _cfg("kda", 64, 64, "f32", K=4, L=2, S=5, seed=2)
    mask = synth.dasc_masks(cfg)
    packed, offsets, unit_index, unit_pos, R = _checkpoint(cfg, mask)
    packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, -1))
    src = np.array([0, 5, 2, -1, 4], np.int32)   # 5 and -1: not checkpoint slots
    dst = np.array([0, 1, 6, 3, 2], np.int32)    # 6: not a private slot
    n_acc = np.array([4, 2, 3, 1, 2], np.int32)
    x = _drafts(cfg, len(src))
    xd = dev_inputs(x, "f32")
    pos = unit_pos.copy()
    h_bad = int(np.flatnonzero(pos[1] >= 0)[0])
    pos[1, h_bad] = R + 3                        # a bad plan entry: that head starts at zero
    st, out, err = _fused(hla, cfg, packed_d, pos, src, dst, 6, xd, n_acc, "f32", 7.0)
    assert err == hla.DEVERR_SLOT | hla.DEVERR_PLAN
    good = np.array([0, 4])
    xg = {n: a[:, good] for n, a in x.items()}
    st2, out2, err2 = _chain(hla, cfg, packed_d, pos, src[good], dst[good], 6,
                             dev_inputs(xg, "f32"), n_acc[good], "f32", 7.0)
    assert err2 == hla.DEVERR_PLAN
    assert torch.equal(st, st2) and torch.equal(out[:, good], out2)
    assert (host(out)[:, [1, 2, 3]] == 5.0).all()         # skipped pairs: no readout
    assert (host(st)[:, [1, 3, 4, 5]] == 7.0).all()       # and no state written
    # the oracle's restore with the bad entry's head zero-filled, as an omitted head
    ref_st, ref_out, scale = _oracle(cfg, packed, offsets, unit_index, src[good], dst[good], 6,
                                     f64_inputs(xg, "f32"), n_acc[good], 7.0,
                                     zero_heads=[(1, h_bad)])
    assert _check_vs_oracle(st2, out2, ref_st, ref_out, scale, n_acc[good], cfg.K) <= TOL

    # nothing retained: every head starts from zero
    none = np.zeros_like(mask)
    _, _, pos0, R0 = hla.dasc_plan(none)
    assert R0 == 0 and (pos0 < 0).all()
    empty = torch.empty((cfg.slots, 0, cfg.dk * cfg.dv), device="cuda")
    src0, dst0 = np.array([1, 0], np.int32), np.array([0, 1], np.int32)
    x0 = {n: a[:, :2] for n, a in x.items()}
    st0, out0, err0 = _fused(hla, cfg, empty, pos0, src0, dst0, 2, dev_inputs(x0, "f32"),
                             n_acc[:2], "f32", 7.0)
    assert err0 == 0
    for l in range(cfg.L):
        Z = np.zeros((2, cfg.H, cfg.dk, cfg.dv))
        o, sc = oracle_par.replay_terms(Z, {n: f64_inputs(x0, "f32")[n][l] for n in NAMES},
                                        n_acc[:2], per_channel=True)
        assert oracle_par.rel_err_tiles(host(st0)[l], Z) <= TOL
        e = np.nan_to_num(np.abs(host(out0)[l] - o)).max(axis=-1) / np.maximum(sc, 1e-30)
        assert float(e.max()) <= TOL

    # no pairs: nothing is launched and nothing changes
    stn, outn, errn = _fused(hla, cfg, packed_d, unit_pos, np.zeros(0, np.int32),
                             np.zeros(0, np.int32), 2,
                             {n: t[:, :0].contiguous() for n, t in xd.items()},
                             np.zeros(0, np.int32), "f32", 7.0)
    assert errn == 0 and (host(stn) == 7.0).all()


def test_restore_replay_full_size():
    """The checkpoint workload at full size: bitwise against the two-call chain over the
    whole 4 GiB of private state and every readout, and against the oracle on sampled
    requests (every layer and head of each)."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    L, S_, H, dk, dv, K = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv, cfg.K
    mask = synth.dasc_masks(cfg)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    assert R == 64
    # the checkpoint's heads are drawn as the active state's are
    packed = synth.initial_state(synth.shrink(cfg, H=R), S=S_).reshape(S_, R, dk * dv)
    g = synth.rng(cfg.seed, 99)
    src = g.permutation(S_).astype(np.int32)
    dst = g.permutation(S_).astype(np.int32)
    n_acc = synth.replay_inputs(cfg, 0)["n_accept"]
    x = _drafts(cfg, S_)
    xd = dev_inputs(x, cfg.in_dtype)
    packed_d = dev(packed)
    print(f"full size: {L} layers x {S_} requests x {H} heads, {R} heads retained, "
          f"{int(n_acc.sum())} accepted tokens per layer", flush=True)
    st, out, err = _fused(hla, cfg, packed_d, unit_pos, src, dst, S_, xd, n_acc, "f32", 7.0)
    assert err == 0
    st2, out2, err2 = _chain(hla, cfg, packed_d, unit_pos, src, dst, S_, xd, n_acc, "f32", 7.0)
    assert err2 == 0
    assert torch.equal(st, st2)
    del st2
    assert torch.equal(out, out2)
    del out2
    # the oracle on sampled requests: their heads start from the packed bits (or zero)
    pick = np.sort(g.choice(S_, size=24, replace=False))
    n_p = n_acc[pick]
    x64 = f64_inputs({n: a[:, pick] for n, a in x.items()}, cfg.in_dtype)
    st_h = st[:, torch.from_numpy(dst[pick]).long().cuda()].cpu().numpy()
    out_h = out[:, torch.from_numpy(pick).long().cuda()].cpu().numpy()
    for l in range(L):
        S64 = np.zeros((len(pick), H, dk, dv))
        for h in range(H):
            if unit_pos[l, h] >= 0:
                S64[:, h] = packed[src[pick], unit_pos[l, h]].reshape(-1, dk, dv)
        o, sc = oracle_par.replay_terms(S64, {n: x64[n][l] for n in NAMES}, n_p,
                                        per_channel=False)
        err_s = oracle_par.rel_err_tiles(st_h[l], S64)
        rows = np.arange(K)[None, :] < n_p[:, None]
        e = np.where(rows[:, :, None, None], np.abs(out_h[l] - o), 0.0).max(axis=-1)
        err_o = float((e / np.maximum(sc, 1e-30)).max())
        print(f"layer {l}: sampled requests' state err {err_s:.2e}, readout err {err_o:.2e} "
              f"of its terms' size", flush=True)
        assert err_s <= TOL and err_o <= TOL
        assert (out_h[l][~rows] == 5.0).all()


def _row_checkpoint(cfg, unit_rows, keep, seed):
    """Every slot's state, a seeded random mask over units of unit_rows key channels
    ([L, H * dk / unit_rows]) and the oracle's pack of the retained units."""
    hla = need_gpu()
    n_units = cfg.H * cfg.dk // unit_rows
    g = np.random.default_rng(seed)
    mask = (g.random((cfg.L, n_units)) < keep).astype(np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    act = np.stack([synth.initial_state(cfg, S=cfg.slots, layer=l) for l in range(cfg.L)])
    ids = np.arange(cfg.slots, dtype=np.int32)
    packed = oracle.dasc_pack(act.view(np.uint8).reshape(cfg.L, cfg.slots, n_units,
                                                         unit_rows * cfg.dv * 4),
                              offsets, unit_index, ids, ids, cfg.slots)
    return packed, offsets, unit_index, unit_pos, R


@pytest.mark.parametrize("kind,dk,dv", [("kda", 128, 128), ("gdn", 128, 64), ("kda", 64, 128)])
@pytest.mark.parametrize("unit_rows", [1, 4, 16, 32])
def test_restore_replay_row_units(kind, dk, dv, unit_rows):
    """Units of unit_rows key channels (1: the KDA checkpoints' single channels): each
    lane looks up the unit of every row it holds."""
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, "f32", K=8, L=2, S=5, seed=3 + unit_rows)
    packed, offsets, unit_index, unit_pos, R = _row_checkpoint(cfg, unit_rows, 0.35,
                                                               70 + unit_rows + dk)
    src = np.array([4, 0, 2, 1], np.int32)
    dst = np.array([2, 5, 0, 3], np.int32)       # slots 1 and 4 are left alone
    n_acc = np.array([8, 0, 3, 11], np.int32)    # 11 clamps to 8
    S_dst = 6
    x = _drafts(cfg, len(src))
    xd = dev_inputs(x, "f32")
    packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, unit_rows * dv))
    st, out, err = _fused(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc, "f32", 7.0)
    assert err == hla.DEVERR_ACCEPT
    st2, out2, err2 = _chain(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc, "f32",
                             7.0, unit_rows=unit_rows)
    assert err2 == hla.DEVERR_ACCEPT
    assert torch.equal(st, st2) and torch.equal(out, out2)
    ref_st, ref_out, scale = _oracle(cfg, packed, offsets, unit_index, src, dst, S_dst,
                                     f64_inputs(x, "f32"), n_acc, 7.0, unit_rows=unit_rows)
    assert _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, cfg.K) <= TOL
    assert (host(st)[:, [1, 4]] == 7.0).all()


def test_restore_replay_row_units_bad_plan_entry():
    """A single-channel unit whose plan entry is past the checkpoint starts from zero and
    is reported, as the restore writes it."""
    hla = need_gpu()
    cfg = _cfg("kda", 128, 128, "f32", K=4, L=2, S=3, seed=9)
    packed, offsets, unit_index, unit_pos, R = _row_checkpoint(cfg, 1, 0.3, 90)
    pos = unit_pos.copy()
    u_bad = int(np.flatnonzero(pos[1] >= 0)[3])
    pos[1, u_bad] = R + 5
    src = np.array([2, 0], np.int32)
    dst = np.array([0, 1], np.int32)
    n_acc = np.array([4, 2], np.int32)
    x = _drafts(cfg, 2)
    xd = dev_inputs(x, "f32")
    packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, cfg.dv))
    st, out, err = _fused(hla, cfg, packed_d, pos, src, dst, 2, xd, n_acc, "f32", 7.0)
    assert err == hla.DEVERR_PLAN
    st2, out2, err2 = _chain(hla, cfg, packed_d, pos, src, dst, 2, xd, n_acc, "f32", 7.0,
                             unit_rows=1)
    assert err2 == hla.DEVERR_PLAN
    assert torch.equal(st, st2) and torch.equal(out, out2)
    h, r = divmod(u_bad, cfg.dk)
    ref_st, ref_out, scale = _oracle(cfg, packed, offsets, unit_index, src, dst, 2,
                                     f64_inputs(x, "f32"), n_acc, 7.0, unit_rows=1,
                                     zero_rows=[(1, h, r, r + 1)])
    assert _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, cfg.K) <= TOL


def test_restore_replay_full_size_kda_channel_rows():
    """The KDA checkpoint workload: 4 layers x 512 requests x 32 heads x 128 x 128 with
    units of single key channels selected by static horizons (4,124 of 16,384), per-channel
    decay, K = 8 drafts.  Bit for bit against the two calls over the whole 4 GiB state and
    every readout; against the oracle on sampled requests."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_kda"]
    L, S_, H, dk, dv, K = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv, cfg.K
    A, d = synth.gate_params(cfg)
    _, mask3 = hla.dasc_static_horizon(A, d, hla.GATE_SOFTPLUS, cfg.a_s, cfg.W_max)
    mask = mask3.reshape(L, H * dk)
    _, _, unit_pos, R = hla.dasc_plan(mask)
    # the checkpoint's rows are drawn as the active state's are
    packed = synth.initial_state(synth.shrink(cfg, H=R, dk=1), S=S_).reshape(S_, R, dv)
    g = synth.rng(cfg.seed, 98)
    src = g.permutation(S_).astype(np.int32)
    dst = g.permutation(S_).astype(np.int32)
    n_acc = synth.replay_inputs(cfg, 0)["n_accept"]
    x = _drafts(cfg, S_)
    xd = dev_inputs(x, cfg.in_dtype)
    packed_d = dev(packed)
    print(f"full size: {L} layers x {S_} requests x {H} heads, {R} of {L * H * dk} channel "
          f"rows retained, {int(n_acc.sum())} accepted tokens per layer", flush=True)
    st, out, err = _fused(hla, cfg, packed_d, unit_pos, src, dst, S_, xd, n_acc, "f32", 7.0)
    assert err == 0
    st2, out2, err2 = _chain(hla, cfg, packed_d, unit_pos, src, dst, S_, xd, n_acc, "f32", 7.0,
                             unit_rows=1)
    assert err2 == 0
    assert torch.equal(st, st2)
    del st2
    assert torch.equal(out, out2)
    del out2
    pick = np.sort(g.choice(S_, size=16, replace=False))
    n_p = n_acc[pick]
    x64 = f64_inputs({n: a[:, pick] for n, a in x.items()}, cfg.in_dtype)
    st_h = st[:, torch.from_numpy(dst[pick]).long().cuda()].cpu().numpy()
    out_h = out[:, torch.from_numpy(pick).long().cuda()].cpu().numpy()
    for l in range(L):
        S64 = np.zeros((len(pick), H, dk, dv))
        pl = unit_pos[l].reshape(H, dk)
        for h in range(H):
            kept = np.flatnonzero(pl[h] >= 0)
            S64[:, h, kept] = packed[src[pick]][:, pl[h][kept]]
        o, sc = oracle_par.replay_terms(S64, {n: x64[n][l] for n in NAMES}, n_p,
                                        per_channel=True)
        err_s = oracle_par.rel_err_tiles(st_h[l], S64)
        rows = np.arange(K)[None, :] < n_p[:, None]
        e = np.where(rows[:, :, None, None], np.abs(out_h[l] - o), 0.0).max(axis=-1)
        err_o = float((e / np.maximum(sc, 1e-30)).max())
        print(f"layer {l}: {int((pl >= 0).sum())} rows retained; sampled requests' state err "
              f"{err_s:.2e}, readout err {err_o:.2e} of its terms' size", flush=True)
        assert err_s <= TOL and err_o <= TOL


# ------------------------------------------------------------------ INT8 checkpoints

def _int8_checkpoint(cfg, unit_rows, keep, seed):
    """The oracle's INT8 pack ([dasc] App. E.1) of every slot's state over a seeded random
    mask of units of unit_rows key channels: codes [S, R, unit_rows, dv], scales
    [S, R, unit_rows] and the plan."""
    hla = need_gpu()
    n_units = cfg.H * cfg.dk // unit_rows
    g = np.random.default_rng(seed)
    mask = (g.random((cfg.L, n_units)) < keep).astype(np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    act = np.stack([synth.initial_state(cfg, S=cfg.slots, layer=l) for l in range(cfg.L)])
    ids = np.arange(cfg.slots, dtype=np.int32)
    codes, scales = oracle.dasc_pack_int8(
        act.reshape(cfg.L, cfg.slots, n_units, unit_rows, cfg.dv), offsets, unit_index, ids,
        ids, cfg.slots)
    return codes, scales, offsets, unit_index, unit_pos, R


def _fused8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_dst, xd, n_acc, out_dtype,
            init):
    st = torch.full((cfg.L, S_dst, cfg.H, cfg.dk, cfg.dv), init, device="cuda")
    out = torch.full((cfg.L, len(src), cfg.K, cfg.H, cfg.dv), 5.0, device="cuda",
                     dtype=getattr(torch, TORCH_DT[out_dtype]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = dev(np.ascontiguousarray(unit_pos, np.int32).reshape(-1))
    hla.dasc_restore_int8_replay(codes_d, scales_d, pos, dev(src), dev(dst), st, xd["q"],
                                 xd["k"], xd["v"], xd["alpha"], xd["beta"], dev(n_acc),
                                 1 if cfg.decay == "vector" else 0, out=out, err_flag=err)
    return st, out, int(err.item())


def _chain8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_dst, xd, n_acc, out_dtype, init,
            unit_rows):
    """dasc_restore_int8, then replay_accepted layer by layer into the restored slots."""
    L, H, dv = cfg.L, cfg.H, cfg.dv
    n_units = H * cfg.dk // unit_rows
    st = torch.full((L, S_dst, H, cfg.dk, dv), init, device="cuda")
    out = torch.full((L, len(src), cfg.K, H, dv), 5.0, device="cuda",
                     dtype=getattr(torch, TORCH_DT[out_dtype]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    S_ck, R = codes_d.shape[:2]
    src_d, dst_d, n_d = dev(src), dev(dst), dev(n_acc)
    pos = dev(np.ascontiguousarray(unit_pos, np.int32).reshape(-1))
    hla.dasc_restore_int8(codes_d, scales_d, S_ck, R, pos, L, n_units, unit_rows, dv, src_d,
                          dst_d, st, S_dst * H * cfg.dk * dv * 4, S_dst, err_flag=err)
    for l in range(L):
        hla.replay_accepted(st[l], xd["q"][l], xd["k"][l], xd["v"][l], xd["alpha"][l],
                            xd["beta"][l], n_d, 1 if cfg.decay == "vector" else 0, out=out[l],
                            slot=dst_d, err_flag=err)
    return st, out, int(err.item())


def _oracle8(cfg, codes, scales, offsets, unit_index, src, dst, S_dst, x64, n_acc, init,
             unit_rows):
    """The oracle's INT8 restore (code x scale in FP32) into a state filled with `init`,
    then its replay per layer."""
    L, H, dk, dv = cfg.L, cfg.H, cfg.dk, cfg.dv
    n_units = H * dk // unit_rows
    rest = np.full((L, S_dst, H, dk, dv), init, np.float32)
    view = rest.reshape(L, S_dst, n_units, unit_rows, dv)
    oracle.dasc_restore_int8(codes, scales, offsets, unit_index, L, n_units, src, dst, view)
    return _oracle_replay(cfg, rest, dst, x64, n_acc)


@pytest.mark.parametrize("kind,dk,dv,in_dtype", [("kda", 128, 128, "f32"),
                                                 ("gdn", 128, 64, "bf16"),
                                                 ("kda", 64, 128, "f16")])
@pytest.mark.parametrize("unit_rows", [1, 16, "dk"])
def test_restore_int8_replay_matches_oracle_and_chain(kind, dk, dv, in_dtype, unit_rows):
    """An INT8 checkpoint restored and replayed in one pass: against the oracle's INT8
    restore then replay, and bit for bit against dasc_restore_int8 then replay_accepted."""
    hla = need_gpu()
    ur = dk if unit_rows == "dk" else unit_rows
    cfg = _cfg(kind, dk, dv, in_dtype, K=8, L=2, S=5, seed=17 + ur)
    codes, scales, offsets, unit_index, unit_pos, R = _int8_checkpoint(cfg, ur, 0.4, 40 + ur)
    src = np.array([4, 0, 2, 1], np.int32)
    dst = np.array([2, 5, 0, 3], np.int32)
    n_acc = np.array([8, 0, 3, 11], np.int32)    # 11 clamps to 8
    S_dst = 6
    x = _drafts(cfg, len(src))
    xd = dev_inputs(x, in_dtype)
    codes_d, scales_d = dev(codes), dev(scales)
    st, out, err = _fused8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_dst, xd, n_acc,
                           "f32", 7.0)
    assert err == hla.DEVERR_ACCEPT
    st2, out2, err2 = _chain8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_dst, xd, n_acc,
                              "f32", 7.0, ur)
    assert err2 == hla.DEVERR_ACCEPT
    assert torch.equal(st, st2) and torch.equal(out, out2)
    ref_st, ref_out, scale = _oracle8(cfg, codes, scales, offsets, unit_index, src, dst, S_dst,
                                      f64_inputs(x, in_dtype), n_acc, 7.0, ur)
    assert _check_vs_oracle(st, out, ref_st, ref_out, scale, n_acc, cfg.K) <= TOL
    assert (host(st)[:, [1, 4]] == 7.0).all()


@pytest.mark.parametrize("kind,dk,dv,in_dtype", [("gdn", 128, 128, "bf16"),
                                                 ("kda", 128, 128, "f32"),
                                                 ("gdn", 64, 128, "f16"),
                                                 ("kda", 128, 64, "bf16")])
@pytest.mark.parametrize("unit_rows", [1, "dk"])
@pytest.mark.parametrize("q8", [False, True])
def test_restore_replay_without_readouts(kind, dk, dv, in_dtype, unit_rows, q8):
    """With out NULL the fused restore + replay forms no readout terms and reads no q: the
    private state must be the same bits as with readouts, and as the restore followed by
    replays without readouts (FP32 and INT8 checkpoints, head and channel-row units, 0 to
    K accepted drafts)."""
    hla = need_gpu()
    ur = dk if unit_rows == "dk" else unit_rows
    cfg = _cfg(kind, dk, dv, in_dtype, K=8, L=2, S=5, seed=29 + ur)
    L, H = cfg.L, cfg.H
    n_units = H * dk // ur
    src = np.array([4, 0, 2, 1, 3], np.int32)
    dst = np.array([2, 5, 0, 3, 1], np.int32)
    n_acc = np.array([8, 0, 3, 7, 6], np.int32)  # staged in LDS by every fused call
    S_dst = 6
    x = _drafts(cfg, len(src))
    xd = dev_inputs(x, in_dtype)
    vec = 1 if kind == "kda" else 0
    src_d, dst_d, n_d = dev(src), dev(dst), dev(n_acc)
    stride = S_dst * H * dk * dv * 4
    if q8:
        codes, scales, _, _, unit_pos, R = _int8_checkpoint(cfg, ur, 0.4, 50 + ur)
        codes_d, scales_d = dev(codes), dev(scales)
        pos = dev(unit_pos.reshape(-1))
        st, _, _ = _fused8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_dst, xd, n_acc,
                           "f32", 7.0)

        def fused_nr(s_):
            hla.dasc_restore_int8_replay(codes_d, scales_d, pos, src_d, dst_d, s_, xd["q"],
                                         xd["k"], xd["v"], xd["alpha"], xd["beta"], n_d, vec)

        def restore(s_):
            hla.dasc_restore_int8(codes_d, scales_d, cfg.slots, R, pos, L, n_units, ur, dv,
                                  src_d, dst_d, s_, stride, S_dst)
    else:
        packed, _, _, unit_pos, R = _row_checkpoint(cfg, ur, 0.4, 50 + ur)
        packed_d = dev(packed.view(np.float32).reshape(cfg.slots, R, ur * dv))
        pos = dev(unit_pos.reshape(-1))
        st, _, _ = _fused(hla, cfg, packed_d, unit_pos, src, dst, S_dst, xd, n_acc, "f32", 7.0)

        def fused_nr(s_):
            hla.dasc_restore_replay(packed_d, pos, src_d, dst_d, s_, xd["q"], xd["k"], xd["v"],
                                    xd["alpha"], xd["beta"], n_d, vec)

        def restore(s_):
            hla.dasc_restore(packed_d, cfg.slots, R, pos, L, n_units, ur * dv * 4, src_d, dst_d,
                             s_, stride, S_dst)
    st_nr = torch.full_like(st, 7.0)
    fused_nr(st_nr)
    assert torch.equal(st_nr, st)
    st_c = torch.full_like(st, 7.0)
    restore(st_c)
    for l in range(L):
        hla.replay_accepted(st_c[l], xd["q"][l], xd["k"][l], xd["v"][l], xd["alpha"][l],
                            xd["beta"][l], n_d, vec, slot=dst_d, want_out=False)
    assert torch.equal(st_c, st)


@pytest.mark.parametrize("name", ["dasc_gdn", "dasc_kda"])
def test_restore_int8_replay_full_size(name):
    """The two checkpoint workloads with INT8 checkpoints (the library's pack of a random
    state): bit for bit against dasc_restore_int8 then replay_accepted over the whole 4 GiB
    private state and every readout; against the oracle (its INT8 restore of the same codes
    and scales, then its replay) on sampled requests."""
    hla = need_gpu()
    cfg = synth.CONFIGS[name]
    L, S_, H, dk, dv, K = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv, cfg.K
    if cfg.decay == "vector":
        A, d = synth.gate_params(cfg)
        _, mask3 = hla.dasc_static_horizon(A, d, hla.GATE_SOFTPLUS, cfg.a_s, cfg.W_max)
        mask, ur = mask3.reshape(L, H * dk), 1
    else:
        mask, ur = synth.dasc_masks(cfg), dk
    n_units = H * dk // ur
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    act = torch.randn((L, S_, n_units, ur, dv), device="cuda", generator=gen) * 0.05
    codes_d = torch.empty((S_, R, ur, dv), dtype=torch.int8, device="cuda")
    scales_d = torch.empty((S_, R, ur), device="cuda")
    ids_h = np.arange(S_, dtype=np.int32)
    hla.dasc_pack_int8(act, S_ * H * dk * dv * 4, S_, L, n_units, ur, dv, dev(offsets),
                       dev(unit_index), R, dev(ids_h), dev(ids_h), codes_d, scales_d, S_)
    del act
    g = synth.rng(cfg.seed, 97)
    src = g.permutation(S_).astype(np.int32)
    dst = g.permutation(S_).astype(np.int32)
    n_acc = synth.replay_inputs(cfg, 0)["n_accept"]
    x = _drafts(cfg, S_)
    xd = dev_inputs(x, cfg.in_dtype)
    print(f"{name}: {R} of {L * n_units} units of {ur} channels retained, "
          f"{int(n_acc.sum())} accepted tokens per layer", flush=True)
    st, out, err = _fused8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_, xd, n_acc,
                           "f32", 7.0)
    assert err == 0
    st2, out2, err2 = _chain8(hla, cfg, codes_d, scales_d, unit_pos, src, dst, S_, xd, n_acc,
                              "f32", 7.0, ur)
    assert err2 == 0
    assert torch.equal(st, st2)
    del st2
    assert torch.equal(out, out2)
    del out2
    pick = np.sort(g.choice(S_, size=16, replace=False))
    codes = codes_d[torch.from_numpy(src[pick]).long().cuda()].cpu().numpy()
    scs = scales_d[torch.from_numpy(src[pick]).long().cuda()].cpu().numpy()
    sub = np.arange(len(pick), dtype=np.int32)
    x64 = f64_inputs({n: a[:, pick] for n, a in x.items()}, cfg.in_dtype)
    rest = np.zeros((L, len(pick), H, dk, dv), np.float32)
    oracle.dasc_restore_int8(codes, scs, offsets, unit_index, L, n_units, sub, sub,
                             rest.reshape(L, len(pick), n_units, ur, dv))
    ref_st, ref_out, scale = _oracle_replay(cfg, rest, sub, x64, n_acc[pick])
    st_h = st[:, torch.from_numpy(dst[pick]).long().cuda()].cpu().numpy()
    out_h = out[:, torch.from_numpy(pick).long().cuda()].cpu().numpy()
    for l in range(L):
        err_s = oracle_par.rel_err_tiles(st_h[l], ref_st[l])
        rows = np.arange(K)[None, :] < n_acc[pick][:, None]
        e = np.where(rows[:, :, None, None], np.abs(out_h[l] - ref_out[l]), 0.0).max(axis=-1)
        err_o = float((e / np.maximum(scale[l], 1e-30)).max())
        print(f"layer {l}: sampled requests' state err {err_s:.2e}, readout err {err_o:.2e} "
              f"of its terms' size", flush=True)
        assert err_s <= TOL and err_o <= TOL
