"""GPU parity of dasc_pack / dasc_restore against the oracle: bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, need_gpu, torch

pytestmark = pytest.mark.gpu


def _bytes_dev(a: np.ndarray):
    return dev(np.ascontiguousarray(a).view(np.uint8).reshape(-1))


def _case(rng, L, S_act, n_units, ub, p_keep, empty_layer=False):
    active = rng.integers(0, 256, size=(L, S_act, n_units, ub), dtype=np.uint8)
    mask = (rng.random((L, n_units)) < p_keep).astype(np.uint8)
    if empty_layer:
        mask[L // 2] = 0
    return active, mask


@pytest.mark.parametrize("L,S_act,n_units,ub,p_keep", [
    (3, 6, 7, 48, 0.5),         # odd unit count, 3 vectors per unit
    (4, 5, 32, 512, 0.4),       # KDA-like channel rows of dv fp32 values
    (2, 4, 4, 65536, 0.5),      # GDN-like whole-head units
    (1, 3, 1, 16, 1.0),         # a single one-vector unit
    (5, 4, 9, 1040, 0.7),       # unit larger than a wave's 1 KiB, not a power of two
])
def test_pack_restore_bit_exact(L, S_act, n_units, ub, p_keep):
    hla = need_gpu()
    rng = np.random.default_rng(L * 1000 + n_units * 10 + ub)
    active, mask = _case(rng, L, S_act, n_units, ub, p_keep, empty_layer=L > 2)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    S_ckpt = S_act + 1
    N = S_act
    src = rng.permutation(S_act).astype(np.int32)
    dst = rng.permutation(S_ckpt)[:N].astype(np.int32)
    # GPU pack into a sentinel-filled checkpoint buffer
    packed = torch.full((S_ckpt * max(R, 1) * ub,), 0xCD, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_pack(_bytes_dev(active), S_act * n_units * ub, S_act, L, n_units, ub,
                  dev(offsets), dev(unit_index), R, dev(src), dev(dst), packed, S_ckpt,
                  err_flag=err)
    ref = oracle.dasc_pack(active, offsets, unit_index, src, dst, S_ckpt)  # zeros elsewhere
    got = packed.cpu().numpy()[: S_ckpt * R * ub].reshape(S_ckpt, R, ub)
    for d in dst:
        assert np.array_equal(got[d], ref[d])
    untouched = sorted(set(range(S_ckpt)) - set(dst.tolist()))
    assert (got[untouched] == 0xCD).all()
    # GPU restore of the oracle's checkpoint into sentinel-filled private slots
    S_dst = S_act + 2
    dst2 = rng.permutation(S_dst)[:N].astype(np.int32)
    out0 = rng.integers(0, 256, size=(L, S_dst, n_units, ub), dtype=np.uint8)
    out = _bytes_dev(out0)
    hla.dasc_restore(_bytes_dev(ref), S_ckpt, R, dev(unit_pos.reshape(-1)), L, n_units, ub,
                     dev(dst), dev(dst2), out, S_dst * n_units * ub, S_dst, err_flag=err)
    ref_out = out0.copy()
    oracle.dasc_restore(ref, offsets, unit_index, L, n_units, dst, dst2, ref_out)
    assert np.array_equal(out.cpu().numpy().reshape(ref_out.shape), ref_out)
    assert int(err.item()) == 0


def test_empty_and_full_masks():
    hla = need_gpu()
    rng = np.random.default_rng(3)
    L, S_, n_units, ub = 2, 3, 5, 64
    active = rng.integers(0, 256, size=(L, S_, n_units, ub), dtype=np.uint8)
    idx = dev(np.arange(S_, dtype=np.int32))
    for full in (False, True):
        mask = np.full((L, n_units), int(full), np.uint8)
        offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
        packed = torch.zeros(max(S_ * R * ub, 16), dtype=torch.uint8, device="cuda")
        hla.dasc_pack(_bytes_dev(active), S_ * n_units * ub, S_, L, n_units, ub, dev(offsets),
                      dev(unit_index), R, idx, idx, packed, S_)
        out = torch.full((active.size,), 0xEE, dtype=torch.uint8, device="cuda")
        hla.dasc_restore(packed, S_, R, dev(unit_pos.reshape(-1)), L, n_units, ub, idx, idx, out,
                         S_ * n_units * ub, S_)
        got = out.cpu().numpy().reshape(active.shape)
        if full:
            assert np.array_equal(got, active)  # dense hit: a plain copy
        else:
            assert R == 0 and not got.any()     # nothing retained: all zero


def test_checkpoint_workload_full_size():
    """4 layers x 512 request states x 32 heads x 64 KiB, seeded ragged head masks with
    64 retained heads: pack all 512 states, restore into 512 private slots.  The restored
    state equals the active state on retained heads and is zero elsewhere (checked over the
    whole 4 GiB on the GPU); 8 sampled pairs are checked bit-exact against the oracle."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    L, S_, H, ub = cfg.L, cfg.slots, cfg.H, cfg.dk * cfg.dv * 4
    mask = synth.dasc_masks(cfg)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    assert R == 64
    g = torch.Generator(device="cuda").manual_seed(11)
    active = torch.randn((L, S_, H, cfg.dk * cfg.dv), device="cuda", generator=g)
    packed = torch.empty((S_, R, ub // 4), device="cuda")
    ids = dev(np.arange(S_, dtype=np.int32))
    hla.dasc_pack(active, S_ * H * ub, S_, L, H, ub, dev(offsets), dev(unit_index), R, ids, ids,
                  packed, S_)
    restored = torch.full_like(active, float("nan"))
    hla.dasc_restore(packed, S_, R, dev(unit_pos.reshape(-1)), L, H, ub, ids, ids, restored,
                     S_ * H * ub, S_)
    keep = torch.from_numpy(mask.astype(bool)).cuda()[:, None, :, None]
    assert torch.equal(torch.where(keep, active, torch.zeros_like(active)), restored)
    # sampled pairs against the oracle, bit-exact
    rng = np.random.default_rng(2)
    for s in rng.choice(S_, size=8, replace=False):
        act_s = active[:, s:s + 1].cpu().numpy().view(np.uint8).reshape(L, 1, H, ub)
        ref = oracle.dasc_pack(act_s, offsets, unit_index, np.zeros(1, np.int32),
                               np.zeros(1, np.int32), 1)
        assert np.array_equal(packed[s].cpu().numpy().view(np.uint8).reshape(R, ub), ref[0])


def test_bad_slots_and_plan_entries_set_flags():
    hla = need_gpu()
    L, S_, n_units, ub = 2, 3, 4, 32
    active = torch.zeros(L * S_ * n_units * ub, dtype=torch.uint8, device="cuda")
    mask = np.ones((L, n_units), np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    packed = torch.zeros(S_ * R * ub, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_pack(active, S_ * n_units * ub, S_, L, n_units, ub, dev(offsets), dev(unit_index),
                  R, dev(np.array([0, 7], np.int32)), dev(np.array([1, 0], np.int32)), packed, S_,
                  err_flag=err)
    assert int(err.item()) == hla.DEVERR_SLOT
    err.zero_()
    bad_index = unit_index.copy()
    bad_index[2] = 99
    hla.dasc_pack(active, S_ * n_units * ub, S_, L, n_units, ub, dev(offsets), dev(bad_index), R,
                  dev(np.array([0], np.int32)), dev(np.array([1], np.int32)), packed, S_,
                  err_flag=err)
    assert int(err.item()) == hla.DEVERR_PLAN
    err.zero_()
    bad_pos = unit_pos.reshape(-1).copy()
    bad_pos[1] = R + 5
    hla.dasc_restore(packed, S_, R, dev(bad_pos), L, n_units, ub, dev(np.array([0], np.int32)),
                     dev(np.array([2], np.int32)), active, S_ * n_units * ub, S_, err_flag=err)
    assert int(err.item()) == hla.DEVERR_PLAN
