"""The C ABI on the CPU: the library loads, exports every entry point that
include/hla.h declares, and rejects bad arguments on the host before launching
anything.  No call here reaches a kernel launch (every call is either invalid or
empty), so these tests need no GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

hla = pytest.importorskip("hybrid_linear_attention_step_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hla.LIB_PATH):
        pytest.skip("libhla.so not built (run __graft_entry__.build())")
    return hla.lib()


OK, NULL, SHAPE, ALIGN, DTYPE, PLAN, ALIAS, UNSUP = 0, 1, 2, 3, 4, 5, 6, 7


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"HLA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"gdn_step", "kda_step", "damp_step", "dasc_pack", "dasc_restore",
            "replay_accepted"} <= names
    for n in names:
        assert hasattr(L, n), n
        assert n in hla.SIGNATURES, n


def test_status_strings(L):
    for code in range(9):
        assert len(hla.status_str(code)) > 0
    assert hla.status_str(0) == "ok"
    assert hla.status_str(99) == "unknown status"
    assert L.hla_version() == 101


# Fake device addresses: never dereferenced, because every call below fails
# validation (or is empty) before anything is launched.
class Fake:
    def __init__(self):
        self.next = 0x7F0000000000

    def __call__(self, nbytes=1 << 30):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return ctypes.c_void_p(p)


def _gdn(L, f, **kw):
    a = dict(state=f(), n_slots=4, slot=None, B=4, H=2, dk=128, dv=128, q=f(), k=f(), v=f(),
             in_dtype=1, alpha=f(), beta=f(), out=f(), out_dtype=0, err=None, stream=None)
    a.update(kw)
    return L.gdn_step(*a.values())


def test_step_validation(L):
    f = Fake()
    assert _gdn(L, f, state=None) == NULL
    assert _gdn(L, f, q=None) == NULL
    assert _gdn(L, f, dk=96) == UNSUP
    assert _gdn(L, f, dv=256) == UNSUP
    assert _gdn(L, f, in_dtype=5) == DTYPE
    assert _gdn(L, f, out_dtype=-1) == DTYPE
    assert _gdn(L, f, B=-1) == SHAPE
    assert _gdn(L, f, H=0) == SHAPE
    assert _gdn(L, f, n_slots=3) == SHAPE  # identity slot map needs n_slots >= B
    assert _gdn(L, f, q=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert _gdn(L, f, state=ctypes.c_void_p(f().value + 8)) == ALIGN
    q = f()
    assert _gdn(L, f, q=q, out=q) == ALIAS
    st = f()
    assert _gdn(L, f, state=st, v=ctypes.c_void_p(st.value + 4096)) == ALIAS
    assert _gdn(L, f, B=0) == OK  # empty batch: nothing to launch


def test_kda_and_replay_validation(L):
    f = Fake()
    args = [f(), 4, None, 4, 2, 64, 64, f(), f(), f(), 0]
    # KDA's per-channel decay is read with 16-byte loads
    assert L.kda_step(*args, ctypes.c_void_p(f().value + 4), f(), f(), 0, None, None) == ALIGN
    base = dict(state=f(), n_slots=4, slot=None, B=4, H=2, dk=64, dv=64, K=8, q=f(), k=f(),
                v=f(), in_dtype=0, alpha=f(), decay=0, beta=f(), n_accept=f(), out=None,
                out_dtype=0, err=None, stream=None)

    def rp(**kw):
        a = dict(base)
        a.update(kw)
        return L.replay_accepted(*a.values())

    assert rp(K=0) == SHAPE and rp(K=17) == SHAPE
    assert rp(n_accept=None) == NULL
    assert rp(decay=2) == DTYPE
    assert rp(B=0) == OK

    # replay fused with the bonus token
    bonus = dict(base)
    n_out = bonus.pop("out_dtype")
    tail = dict(err=bonus.pop("err"), stream=bonus.pop("stream"))
    bonus.update(qb=f(), kb=f(), vb=f(), ab=f(), bb=f(), out_b=f(), out_dtype=n_out, **tail)

    def rb(**kw):
        a = dict(bonus)
        a.update(kw)
        return L.replay_accepted_bonus(*a.values())

    assert rb(qb=None) == NULL and rb(bb=None) == NULL and rb(n_accept=None) == NULL
    assert rb(kb=ctypes.c_void_p(f().value + 8)) == ALIGN
    assert rb(out_b=ctypes.c_void_p(f().value + 4)) == ALIGN
    st = f()
    assert rb(state=st, out_b=st) == ALIAS
    assert rb(qb=st, state=st) == ALIAS
    assert rb(K=0) == SHAPE and rb(B=0) == OK
    # the verify pass: readouts are required, the state is only read
    ver = {k: base[k] for k in ("state", "n_slots", "slot", "B", "H", "dk", "dv", "K", "q",
                                "k", "v", "in_dtype", "alpha", "decay", "beta")}
    ver.update(out=f(), out_dtype=0, err=None, stream=None)

    def vd(**kw):
        a = dict(ver)
        a.update(kw)
        return L.verify_drafts(*a.values())

    assert vd(out=None) == NULL
    assert vd(K=17) == SHAPE and vd(decay=5) == DTYPE
    assert vd(out=st, state=st) == ALIAS
    assert vd(B=0) == OK


def test_damp_validation(L):
    f = Fake()
    base = dict(hi=f(), lo=f(), sc=f(), n_slots=4, perm=None, K_hi=16, group=128,
                val_perm=None, val_scale=None, slot=None, B=4, H=2, dk=128, dv=128, q=f(),
                k=f(), v=f(), in_dtype=1, alpha=f(), decay=1, beta=f(), out=f(), out_dtype=0,
                err=None, stream=None)

    def dm(**kw):
        a = dict(base)
        a.update(kw)
        return L.damp_step(*a.values())

    assert dm(K_hi=129) == SHAPE and dm(K_hi=-1) == SHAPE
    assert dm(hi=None) == NULL
    # no FP16 rows: hi may be NULL (the misaligned q is reported instead; nothing launches)
    assert dm(hi=None, K_hi=0, q=ctypes.c_void_p(f().value + 2)) == ALIGN
    assert dm(lo=None) == NULL
    assert dm(dk=32) == UNSUP
    # scale groups: one per row (group = dv) or per 32 values; nothing else is built
    assert dm(group=64) == UNSUP and dm(group=0) == UNSUP and dm(group=16) == UNSUP
    assert dm(group=32, q=ctypes.c_void_p(f().value + 2)) == ALIGN
    hi = f()
    assert dm(hi=hi, lo=hi) == ALIAS
    # the value-transform tables are inputs: an output written over one is an alias
    vs = f()
    assert dm(val_scale=vs, out=vs) == ALIAS
    assert dm(val_perm=hi, hi=hi) == ALIAS
    assert L.damp_quantize(f(), 2, 2, 128, 128, None, 200, 128, None, None, f(), f(), f(),
                           None) == SHAPE
    assert L.damp_quantize(f(), 2, 2, 128, 128, None, 16, 48, None, None, f(), f(), f(),
                           None) == UNSUP
    assert L.damp_dequantize(f(), f(), f(), 2, 2, 100, 128, None, 16, 128, None, None, f(),
                             None) == UNSUP
    # dequantise must not write its state over a plan table
    st = f()
    assert L.damp_dequantize(f(), f(), f(), 2, 2, 128, 128, None, 16, 32, st, None, st,
                             None) == ALIAS


def test_dasc_validation(L):
    f = Fake()
    base = dict(active=f(), stride=512 * 32 * 65536, S_act=512, L=4, n_units=32,
                unit_bytes=65536, offsets=f(), unit_index=f(), R_total=64, src=f(), dst=f(),
                N=8, packed=f(), S_ckpt=8, err=None, stream=None)

    def pk(**kw):
        a = dict(base)
        a.update(kw)
        return L.dasc_pack(*a.values())

    assert pk(unit_bytes=24) == ALIGN
    assert pk(R_total=129) == PLAN
    assert pk(offsets=None) == NULL
    assert pk(stride=1024) == SHAPE  # layers would overlap
    act = f()
    assert pk(active=act, packed=ctypes.c_void_p(act.value + 65536)) == ALIAS
    assert pk(N=0) == OK
    assert L.dasc_restore(f(), 8, 64, None, 4, 32, 65536, f(), f(), 8, f(), 512 * 32 * 65536,
                          512, None, None) == NULL


def test_dasc_plan_matches_oracle(L, orc):
    g = np.random.default_rng(40)
    for trial in range(20):
        Lr, n = int(g.integers(1, 9)), int(g.integers(1, 300))
        mask = (g.random((Lr, n)) < g.random()).astype(np.uint8)
        off, idx, pos, R = hla.dasc_plan(mask)
        o_off, o_idx = orc.dasc_plan(mask)
        assert R == o_off[-1]
        assert np.array_equal(off, o_off) and np.array_equal(idx, o_idx)
        for l in range(Lr):
            for u in range(n):
                p = pos[l, u]
                if mask[l, u]:
                    assert off[l] <= p < off[l + 1] and idx[p] == u
                else:
                    assert p == -1


def test_dasc_plan_errors(L):
    mask = np.ones((2, 5), np.uint8)
    off = np.zeros(3, np.int32)
    idx = np.zeros(4, np.int32)
    R = ctypes.c_int32()
    assert L.dasc_plan(mask.ctypes.data, 2, 5, off.ctypes.data, idx.ctypes.data, 4, None,
                       ctypes.byref(R)) == PLAN
    assert L.dasc_plan(None, 2, 5, off.ctypes.data, idx.ctypes.data, 4, None,
                       ctypes.byref(R)) == NULL
    assert L.dasc_plan(mask.ctypes.data, 0, 5, off.ctypes.data, idx.ctypes.data, 4, None,
                       ctypes.byref(R)) == SHAPE


# ---------------------------------------------------------------- static selection (host)

def test_static_horizon_and_mask_match_oracle(orc):
    """The library's host horizons (float64) equal the oracle's, and the masks are
    bit-exact, on the KDA checkpoint workload's synthetic gate parameters and on the
    bounded gate."""
    import synth

    import hybrid_linear_attention_step_amd as hla

    cfg = synth.CONFIGS["dasc_kda"]
    A, d = synth.gate_params(cfg)
    for gate, a_s in ((hla.GATE_SOFTPLUS, cfg.a_s), (hla.GATE_BOUNDED, 0.8)):
        H, m = hla.dasc_static_horizon(A, d, gate, a_s, cfg.W_max)
        Ho = orc.static_horizon(A.astype(np.float64), d.astype(np.float64), gate, a_s)
        np.testing.assert_allclose(H, Ho, rtol=1e-15)
        assert np.array_equal(m, orc.static_mask(Ho, cfg.W_max))
        if gate == hla.GATE_SOFTPLUS:
            assert 0.05 < m.mean() < 0.95  # a mixed selection, not all or nothing


@pytest.mark.parametrize("H,mask,n_p,W_max", [
    ([3.0, 4.0, 4.5, 9.0, 0.5], [0, 0, 0, 0, 0], 100, 16),
    ([3.0, 9.0, 40.0], [0, 0, 1], 7, 16),
    ([30.0, 40.0], [1, 1], 100, 16),
    ([0.0, -1.0, 1e300], [0, 0, 0], 10 ** 6, 64),
    ([32.0, 64.0, 33.0], [0, 0, 1], 1000, 64),
])
def test_replay_window_matches_oracle(orc, H, mask, n_p, W_max):
    import hybrid_linear_attention_step_amd as hla

    H, mask = np.array(H), np.array(mask, np.uint8)
    assert hla.dasc_replay_window(H, mask, n_p, W_max)[0] == orc.replay_window(H, mask, n_p,
                                                                                W_max)[0]
    assert np.array_equal(hla.dasc_replay_window(H, mask, n_p, W_max)[1],
                          orc.replay_window(H, mask, n_p, W_max)[1])


def test_selection_and_int8_validation(L):
    f = Fake()
    A = (ctypes.c_float * 4)()
    H = (ctypes.c_double * 4)()
    m = (ctypes.c_uint8 * 4)()
    W = ctypes.c_int32(0)
    assert L.dasc_static_horizon(A, A, 4, 2, -0.3, 1e-3, 16.0, H, m) == UNSUP
    assert L.dasc_static_horizon(A, A, 4, 0, -0.3, 0.0, 16.0, H, m) == SHAPE
    assert L.dasc_static_horizon(A, A, 4, 0, -0.3, 1e-3, 16.0, None, None) == NULL
    assert L.dasc_static_horizon(None, A, 0, 0, -0.3, 1e-3, 16.0, None, None) == OK
    assert L.dasc_replay_window(H, m, 4, 10, 3, None, ctypes.byref(W)) == SHAPE
    assert L.dasc_replay_window(H, m, 4, 10, 16, None, None) == NULL
    base = dict(active=f(), stride=512 * 4096 * 512, S_act=512, L=4, n_units=4096,
                unit_rows=1, dv=128, offsets=f(), unit_index=f(), R=4096, src=f(), dst=f(),
                N=8, codes=f(), scales=f(), S_ckpt=8, err=None, stream=None)

    def pk(**kw):
        a = dict(base)
        a.update(kw)
        return L.dasc_pack_int8(*a.values())

    assert pk(unit_rows=3) == SHAPE and pk(unit_rows=512) == SHAPE
    assert pk(dv=96) == UNSUP
    assert pk(scales=None) == NULL
    assert pk(scales=ctypes.c_void_p(f().value + 2)) == ALIGN
    assert pk(codes=ctypes.c_void_p(f().value + 8)) == ALIGN
    act = f()
    assert pk(active=act, codes=ctypes.c_void_p(act.value + 4096)) == ALIAS
    assert pk(N=0) == OK
    rs = dict(codes=f(), scales=f(), S_ckpt=8, R=4096, unit_pos=f(), L=4, n_units=4096,
              unit_rows=1, dv=128, src=f(), dst=f(), N=8, out=f(), stride=512 * 4096 * 512,
              S_dst=512, err=None, stream=None)
    assert L.dasc_restore_int8(*dict(rs, dv=32).values()) == UNSUP
    assert L.dasc_restore_int8(*dict(rs, unit_pos=None).values()) == NULL
    # copy-back: the scratch and active states must not overlap
    st = f()
    cb = dict(scratch=st, s_stride=64 * 32 * 65536, S_s=64, active=f(), stride=512 * 32 * 65536,
              S_act=512, L=4, n_units=32, unit_bytes=65536, offsets=f(), unit_index=f(), R=64,
              src=f(), dst=f(), N=8, err=None, stream=None)
    assert L.dasc_refresh_local(*dict(cb, active=ctypes.c_void_p(st.value + 65536)).values()) \
        == ALIAS
    assert L.dasc_refresh_local(*dict(cb, unit_bytes=65540).values()) == ALIGN



def test_binding_rejects_host_tensors_and_bad_dtypes():
    """The Python binding refuses CPU tensors and wrong element types before any call
    into the library (nothing here touches a GPU)."""
    torch = pytest.importorskip("torch")
    import hybrid_linear_attention_step_amd as hla

    z = lambda *s, **kw: torch.zeros(*s, **kw)  # noqa: E731
    st = z(2, 2, 64, 64)
    with pytest.raises(ValueError, match="GPU"):
        hla.gdn_step(st, z(2, 2, 64), z(2, 2, 64), z(2, 2, 64), z(2, 2), z(2, 2))
    with pytest.raises(ValueError):
        hla.damp_quantize(z(2, 2, 64, 64, dtype=torch.float64), None, 8)
