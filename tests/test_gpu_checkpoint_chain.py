"""The checkpoint workload run as one chain, at full size, against the oracle's chain.

4 layers x 512 request states x 32 GDN heads x 128 x 128 FP32 (4 GiB), seeded ragged
head masks retaining 64 of the 128 layer-heads ([dasc] §4.1, App. B "Ragged
(Scheme 2)"):

1. pack every state's retained heads into the flat checkpoint (2 GiB);
2. restore the checkpoint into 512 private slots, zero-filling the omitted heads
   ([dasc] §4.2, dasc-nr);
3. replay each request's accepted draft projections (K = 8 drafts, accepted counts
   U{0..8}, drawn per layer) into its restored state, layer by layer ([K3]
   "Speculative decoding without state snapshots").

The oracle runs the same chain from the same bits (its pack, its restore, its replay
on every host thread).  Pack and restore are compared bit for bit over the whole 6 GiB;
the replayed states within 1e-5 of max|oracle| per head tile, and every accepted
readout within 1e-5 of the size of its terms, max_j sum_i |S_t[i][j] q_t,i|
per head and token (the readout is a dot product evaluated in FP32: its rounding error
is relative to those terms, not to the result, and a head the restore zero-filled makes
its first readout beta (q . k) v, whose terms cancel whenever q and k are nearly
orthogonal).  The restore∘pack identity (retained heads equal the active state, omitted
heads zero) is also checked over the whole state on the GPU."""
import numpy as np
import pytest

import oracle
import oracle_par
import synth
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")


def test_pack_restore_replay_chain_full_size():
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    L, S_, H, dk, dv = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv
    ub = dk * dv * 4
    mask = synth.dasc_masks(cfg)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    assert R == 64
    act_h = np.empty((L, S_, H, dk, dv), np.float32)
    for l in range(L):
        act_h[l] = synth.initial_state(cfg, S=S_, layer=l)
    active = dev(act_h)
    ids_h = np.arange(S_, dtype=np.int32)
    ids = dev(ids_h)
    stride = S_ * H * ub
    packed = torch.empty((S_, R, ub // 4), device="cuda")
    hla.dasc_pack(active, stride, S_, L, H, ub, dev(offsets), dev(unit_index), R, ids, ids,
                  packed, S_)
    restored = torch.full_like(active, float("nan"))
    hla.dasc_restore(packed, S_, R, dev(unit_pos.reshape(-1)), L, H, ub, ids, ids, restored,
                     stride, S_)
    keep = torch.from_numpy(mask.astype(bool)).cuda()[:, None, :, None, None]
    assert torch.equal(torch.where(keep, active, torch.zeros_like(active)), restored)
    del active

    # the oracle's chain from the same bits: pack, then restore, bit for bit
    a8 = act_h.view(np.uint8).reshape(L, S_, H, ub)
    ref_packed = oracle.dasc_pack(a8, offsets, unit_index, ids_h, ids_h, S_)
    del a8, act_h
    assert np.array_equal(packed.cpu().numpy().view(np.uint8).reshape(S_, R, ub), ref_packed)
    del packed
    ref_rest = np.full((L, S_, H, ub), 0xA5, np.uint8)
    oracle.dasc_restore(ref_packed, offsets, unit_index, L, H, ids_h, ids_h, ref_rest)
    del ref_packed
    got_rest = restored.cpu().numpy()
    assert np.array_equal(got_rest.view(np.uint8).reshape(ref_rest.shape), ref_rest)
    del got_rest

    # replay each layer's accepted drafts into the restored private states
    for l in range(L):
        x = synth.replay_inputs(cfg, l)
        n_acc = x["n_accept"]
        xd = dev_inputs({n: x[n] for n in NAMES}, cfg.in_dtype)
        out = torch.full((S_, cfg.K, H, dv), 5.0, device="cuda")
        st = restored[l]
        hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                            dev(n_acc), 0, out=out)
        S64 = ref_rest[l].view(np.float32).reshape(S_, H, dk, dv).astype(np.float64)
        o_ref, scale = oracle_par.replay_terms(
            S64, f64_inputs({n: x[n] for n in NAMES}, cfg.in_dtype), n_acc, per_channel=False)
        got = host(st)
        err_s = oracle_par.rel_err_tiles(got, S64)
        idle = n_acc == 0
        assert np.array_equal(got[idle].view(np.uint8).reshape(-1, H, ub),
                              ref_rest[l][idle])       # n = 0: the restored bits as they are
        o = host(out)
        rows = np.arange(cfg.K)[None, :] < n_acc[:, None]
        assert (o[~rows] == 5.0).all()                 # rows t >= n_b are left alone
        err = np.where(rows[:, :, None, None], np.abs(o - o_ref), 0.0).max(axis=-1)
        err_o = float((err / np.maximum(scale, 1e-30)).max())
        err_plain = oracle_par.rel_err_tiles(np.where(rows[:, :, None, None], o, 0.0),
                                             np.where(rows[:, :, None, None], o_ref, 0.0), 1)
        print(f"layer {l}: {int(mask[l].sum())} of {H} heads restored, {int((~idle).sum())} "
              f"requests replay {int(n_acc.sum())} tokens; state err {err_s:.2e}; readout err "
              f"{err_o:.2e} of its terms' size ({err_plain:.2e} of its own size)")
        assert err_s <= TOL and err_o <= TOL
