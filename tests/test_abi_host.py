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
    assert L.hla_version() == 102


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
    # an output written over a plan table or slot map the kernel reads while it writes
    pkd = f()
    for table in ("offsets", "unit_index", "src", "dst"):
        assert pk(packed=pkd, **{table: ctypes.c_void_p(pkd.value + 4096)}) == ALIAS, table
    rs = dict(packed=f(), S_ckpt=8, R=64, unit_pos=f(), L=4, n_units=32, unit_bytes=65536,
              src=f(), dst=f(), N=8, out=f(), stride=512 * 32 * 65536, S_dst=512, err=None,
              stream=None)
    out = f()
    for table in ("unit_pos", "src", "dst"):
        a = dict(rs, out=out, **{table: ctypes.c_void_p(out.value + 3 * 512 * 32 * 65536)})
        assert L.dasc_restore(*a.values()) == ALIAS, table


def test_restore_replay_validation(L):
    """The fused restore + replay: the checks of both halves, on the host."""
    f = Fake()
    ub = 128 * 128 * 4
    base = dict(packed=f(), S_ckpt=512, R_total=64, unit_pos=f(), L=4, unit_rows=128,
                src=f(), dst=f(), N=512, active_out=f(4 * 512 * 32 * ub), stride=512 * 32 * ub,
                S_dst=512, H=32,
                dk=128, dv=128, K=8, q=f(), k=f(), v=f(), in_dtype=1, alpha=f(), decay=0,
                beta=f(), n_accept=f(), out=None, out_dtype=0, err=None, stream=None)

    def rr(**kw):
        a = dict(base)
        a.update(kw)
        return L.dasc_restore_replay(*a.values())

    assert rr(N=0) == OK
    assert rr(K=0) == SHAPE and rr(K=17) == SHAPE and rr(L=0) == SHAPE
    assert rr(R_total=129) == PLAN
    # the unit count follows unit_rows (N = 0: the checks run, nothing is launched)
    assert rr(R_total=129, unit_rows=64, N=0) == OK
    assert rr(R_total=4 * 32 * 128, unit_rows=1, N=0) == OK
    assert rr(R_total=4 * 32 * 128 + 1, unit_rows=1, N=0) == PLAN
    for bad in (0, 3, 256, -1):
        assert rr(unit_rows=bad) == SHAPE, bad
    assert rr(dk=96) == UNSUP and rr(in_dtype=7) == DTYPE and rr(decay=3) == DTYPE
    for name in ("unit_pos", "src", "dst", "active_out", "q", "k", "v", "alpha", "beta",
                 "n_accept"):
        assert rr(**{name: None}) == NULL, name
    assert rr(packed=None) == NULL
    assert rr(stride=512 * 32 * ub - 16) == SHAPE     # layers would overlap
    assert rr(stride=512 * 32 * ub + 4) == ALIGN
    assert rr(v=ctypes.c_void_p(f().value + 8)) == ALIGN
    assert rr(unit_pos=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert rr(decay=1, alpha=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert rr(out=ctypes.c_void_p(f().value + 2), out_dtype=1) == ALIGN
    assert rr(L=1 << 12, N=1 << 12, H=1 << 8) == SHAPE  # workgroups beyond 32-bit indices
    # the private state over the checkpoint, an input or a table it reads while it writes;
    # the readout over an input or the state
    act = base["active_out"]
    inside = ctypes.c_void_p(act.value + 3 * 512 * 32 * ub)
    for name in ("packed", "unit_pos", "src", "dst", "q", "v", "alpha", "beta", "n_accept"):
        assert rr(**{name: inside}) == ALIAS, name
    o = f()
    assert rr(out=o, q=ctypes.c_void_p(o.value + 64)) == ALIAS
    assert rr(out=inside) == ALIAS


def test_restore_int8_replay_validation(L):
    """The INT8-checkpoint form: the codes and scales join the checks of the FP32 form."""
    f = Fake()
    ub = 128 * 128 * 4
    act = f(4 * 512 * 32 * ub)
    base = dict(codes=f(), scales=f(), S_ckpt=512, R_total=4124, unit_pos=f(), L=4,
                unit_rows=1, src=f(), dst=f(), N=512, active_out=act, stride=512 * 32 * ub,
                S_dst=512, H=32, dk=128, dv=128, K=8, q=f(), k=f(), v=f(), in_dtype=0,
                alpha=f(), decay=1, beta=f(), n_accept=f(), out=None, out_dtype=0, err=None,
                stream=None)

    def rr(**kw):
        a = dict(base)
        a.update(kw)
        return L.dasc_restore_int8_replay(*a.values())

    assert rr(N=0) == OK
    assert rr(scales=None) == NULL and rr(codes=None) == NULL
    assert rr(scales=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert rr(unit_rows=5) == SHAPE and rr(R_total=4 * 32 * 128 + 1, N=0) == PLAN
    inside = ctypes.c_void_p(act.value + 2 * 512 * 32 * ub)
    assert rr(codes=inside) == ALIAS and rr(scales=inside) == ALIAS


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
    out = f()
    assert L.dasc_restore_int8(*dict(rs, out=out, unit_pos=ctypes.c_void_p(out.value + 64))
                               .values()) == ALIAS
    sc = f()
    assert pk(scales=sc, dst=ctypes.c_void_p(sc.value + 16)) == ALIAS
    cd = f()
    assert pk(codes=cd, offsets=ctypes.c_void_p(cd.value + 1024)) == ALIAS
    # copy-back: the scratch and active states must not overlap
    st = f()
    cb = dict(scratch=st, s_stride=64 * 32 * 65536, S_s=64, active=f(), stride=512 * 32 * 65536,
              S_act=512, L=4, n_units=32, unit_bytes=65536, offsets=f(), unit_index=f(), R=64,
              src=f(), dst=f(), N=8, err=None, stream=None)
    assert L.dasc_refresh_local(*dict(cb, active=ctypes.c_void_p(st.value + 65536)).values()) \
        == ALIAS
    assert L.dasc_refresh_local(*dict(cb, unit_bytes=65540).values()) == ALIGN
    act = f()
    assert L.dasc_refresh_local(*dict(cb, active=act, unit_index=ctypes.c_void_p(act.value + 64))
                                .values()) == ALIAS



def test_binding_rejects_host_tensors_and_bad_dtypes():
    """The Python binding refuses CPU tensors and wrong element types before any call
    into the library (nothing here touches a GPU)."""
    torch = pytest.importorskip("torch")
    import hybrid_linear_attention_step_amd as hla

    z = lambda *s, **kw: torch.zeros(*s, **kw)  # noqa: E731
    st = z(2, 2, 64, 64)
    with pytest.raises(ValueError, match="GPU"):
        hla.gdn_step(st, z(2, 2, 64), z(2, 2, 64), z(2, 2, 64), z(2, 2), z(2, 2))
    with pytest.raises(TypeError, match="dtype"):
        hla.damp_quantize(z(2, 2, 64, 64, dtype=torch.float64), None, 8)


# ---------------------------------------------------------------- binding argument checks
#
# The C entry points size every access from the sizes they are given, so the binding must
# refuse a tensor whose shape disagrees with those sizes, or that lives in host memory,
# before the call.  Shapes are checked before devices, so these run on CPU tensors.

def _t():
    return pytest.importorskip("torch")


def _step_args(torch, B=3, H=2, dk=64, dv=64, kda=False):
    z = torch.zeros
    return dict(state=z(B, H, dk, dv), q=z(B, H, dk), k=z(B, H, dk), v=z(B, H, dv),
                alpha=z(B, H, dk) if kda else z(B, H), beta=z(B, H))


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("bad,shape", [
    ("q", (3, 2, 32)), ("k", (3, 3, 64)), ("v", (2, 2, 64)), ("beta", (3, 1)),
    ("alpha", (3, 2, 64, 1)),
])
def test_binding_rejects_misshaped_step_operands(kda, bad, shape):
    torch = _t()
    a = _step_args(torch, kda=kda)
    a[bad] = torch.zeros(shape)
    fn = hla.kda_step if kda else hla.gdn_step
    with pytest.raises(ValueError, match=bad):
        fn(**a)


def test_binding_rejects_wrong_decay_shape_and_lengths():
    torch = _t()
    a = _step_args(torch)
    with pytest.raises(ValueError, match="alpha"):  # KDA given a GDN-shaped decay
        hla.kda_step(**a)
    with pytest.raises(ValueError, match="alpha"):  # GDN given a KDA-shaped decay
        hla.gdn_step(**_step_args(torch, kda=True))
    with pytest.raises(ValueError, match="slot"):
        hla.gdn_step(**a, slot=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        hla.gdn_step(**a, out=torch.zeros(3, 2, 32))
    with pytest.raises(ValueError, match="err_flag"):
        hla.gdn_step(**a, err_flag=torch.zeros(0, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):    # right shapes, host memory
        hla.gdn_step(**a)


def _draft_args(torch, B=3, K=4, H=2, dk=64, dv=64):
    z = torch.zeros
    return dict(state=z(B, H, dk, dv), q=z(B, K, H, dk), k=z(B, K, H, dk), v=z(B, K, H, dv),
                alpha=z(B, K, H), beta=z(B, K, H))


def test_binding_rejects_misshaped_draft_operands():
    torch = _t()
    i32 = torch.int32
    a = _draft_args(torch)
    n = torch.zeros(3, dtype=i32)
    with pytest.raises(ValueError, match="n_accept"):
        hla.replay_accepted(**a, n_accept=torch.zeros(4, dtype=i32), decay_kind=0)
    with pytest.raises(ValueError, match="alpha"):
        hla.replay_accepted(**a, n_accept=n, decay_kind=1)
    with pytest.raises(ValueError, match="out"):
        hla.replay_accepted(**a, n_accept=n, decay_kind=0, out=torch.zeros(3, 3, 2, 64))
    with pytest.raises(ValueError, match="v"):
        hla.verify_drafts(**dict(a, v=torch.zeros(3, 4, 2, 32)), decay_kind=0)
    z = torch.zeros
    bonus = dict(q_bonus=z(3, 2, 64), k_bonus=z(3, 2, 64), v_bonus=z(3, 2, 64),
                 alpha_bonus=z(3, 2), beta_bonus=z(3, 2))
    with pytest.raises(ValueError, match="k_bonus"):
        hla.replay_accepted_bonus(**a, n_accept=n, decay_kind=0,
                                  **dict(bonus, k_bonus=z(3, 2, 32)))
    with pytest.raises(ValueError, match="alpha_bonus"):
        hla.replay_accepted_bonus(**a, n_accept=n, decay_kind=0,
                                  **dict(bonus, alpha_bonus=z(3, 2, 64)))
    with pytest.raises(ValueError, match="GPU"):
        hla.replay_accepted_bonus(**a, n_accept=n, decay_kind=0, **bonus)


def test_binding_checks_packed_state_operands():
    torch = _t()
    S, H, dk, dv, K_hi = 3, 2, 64, 64, 8
    hi, lo, sc = hla.damp_alloc(S, H, dk, dv, K_hi, device="cpu")
    z = torch.zeros
    x = dict(q=z(S, H, dk), k=z(S, H, dk), v=z(S, H, dv), alpha=z(S, H, dk), beta=z(S, H))
    with pytest.raises(ValueError, match="lo"):
        hla.damp_step(hi, lo[:, :, 1:].contiguous(), sc, None, K_hi, decay_kind=1, **x)
    with pytest.raises(ValueError, match="lo_scale"):
        hla.damp_step(hi, lo, z(S, H, dk - K_hi + 1), None, K_hi, decay_kind=1, **x)
    with pytest.raises(ValueError, match="key_perm"):
        hla.damp_step(hi, lo, sc, z(H, dk - 1, dtype=torch.int32), K_hi, decay_kind=1, **x)
    with pytest.raises(ValueError, match="alpha"):
        hla.damp_step(hi, lo, sc, None, K_hi, decay_kind=0, **x)
    with pytest.raises(ValueError, match="K_hi"):
        hla.damp_step(hi, lo, sc, None, dk + 1, decay_kind=1, **x)
    with pytest.raises(ValueError, match="GPU"):
        hla.damp_step(hi, lo, sc, None, K_hi, decay_kind=1, **x)
    # quantise / dequantise check caller-supplied packed regions and the state alike
    st = z(S, H, dk, dv)
    with pytest.raises(ValueError, match="GPU"):
        hla.damp_quantize(st, None, K_hi, hi=hi, lo=lo, lo_scale=sc)
    with pytest.raises(ValueError, match="hi"):
        hla.damp_quantize(st, None, K_hi, hi=hi[:2].contiguous(), lo=lo, lo_scale=sc)
    with pytest.raises(ValueError, match="all of"):
        hla.damp_quantize(st, None, K_hi, hi=hi)
    with pytest.raises(ValueError, match="GPU"):
        hla.damp_dequantize(hi, lo, sc, None, K_hi, dk)
    with pytest.raises(ValueError, match="state"):
        hla.damp_dequantize(hi, lo, sc, None, K_hi, dk, out=z(S, H, dk, dv + 1))
    with pytest.raises(ValueError, match="val_scale"):
        hla.damp_dequantize(hi, lo, sc, None, K_hi, dk, val_scale=z(H, dv - 1))


def test_binding_checks_checkpoint_buffer_sizes():
    torch = _t()
    i32 = torch.int32
    L, S, n_units, ub = 2, 3, 4, 32
    stride = S * n_units * ub
    active = torch.zeros(L * stride, dtype=torch.uint8)
    offsets = torch.tensor([0, 2, 4], dtype=i32)
    idx = torch.tensor([0, 1, 2, 3], dtype=i32)
    ids = torch.arange(S, dtype=i32)
    packed = torch.zeros(S * 4 * ub, dtype=torch.uint8)
    pk = dict(active=active, layer_stride_bytes=stride, S_act=S, L=L, n_units=n_units,
              unit_bytes=ub, offsets=offsets, unit_index=idx, R_total=4, src_slot=ids,
              dst_slot=ids, packed=packed, S_ckpt=S)
    with pytest.raises(ValueError, match="active"):
        hla.dasc_pack(**dict(pk, active=active[:-16]))
    with pytest.raises(ValueError, match="packed"):
        hla.dasc_pack(**dict(pk, packed=packed[:-16]))
    with pytest.raises(ValueError, match="offsets"):
        hla.dasc_pack(**dict(pk, offsets=offsets[:2]))
    with pytest.raises(ValueError, match="unit_index"):
        hla.dasc_pack(**dict(pk, unit_index=idx[:3]))
    with pytest.raises(ValueError, match="dst_slot"):
        hla.dasc_pack(**dict(pk, dst_slot=ids[:2]))
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_pack(**pk)
    pos = torch.arange(L * n_units, dtype=i32)
    rs = dict(packed=packed, S_ckpt=S, R_total=4, unit_pos=pos, L=L, n_units=n_units,
              unit_bytes=ub, src_slot=ids, dst_slot=ids, active_out=active,
              layer_stride_bytes=stride, S_dst=S)
    with pytest.raises(ValueError, match="unit_pos"):
        hla.dasc_restore(**dict(rs, unit_pos=pos[:-1]))
    with pytest.raises(ValueError, match="active_out"):
        hla.dasc_restore(**dict(rs, S_dst=S + 1))
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_restore(**rs)
    # restore fused with the replay: shapes follow the private state [L, S, H, dk, dv]
    z = torch.zeros
    H, dk, N, K = 2, 64, 3, 4
    pk64 = z(S, 4, dk * dk)
    st = z(L, S, H, dk, dk)
    rr = dict(packed=pk64, unit_pos=z(L, H, dtype=i32), src_slot=ids, dst_slot=ids,
              active_out=st, q=z(L, N, K, H, dk), k=z(L, N, K, H, dk), v=z(L, N, K, H, dk),
              alpha=z(L, N, K, H), beta=z(L, N, K, H), n_accept=z(N, dtype=i32), decay_kind=0)
    with pytest.raises(ValueError, match="unit_pos"):
        hla.dasc_restore_replay(**dict(rr, unit_pos=z(L * H + 1, dtype=i32)))
    with pytest.raises(ValueError, match="packed"):
        hla.dasc_restore_replay(**dict(rr, packed=z(S, 4, dk * dk - 1)))
    with pytest.raises(ValueError, match="alpha"):
        hla.dasc_restore_replay(**dict(rr, decay_kind=1))
    with pytest.raises(ValueError, match="k"):
        hla.dasc_restore_replay(**dict(rr, k=z(L, N, K + 1, H, dk)))
    with pytest.raises(ValueError, match="n_accept"):
        hla.dasc_restore_replay(**dict(rr, n_accept=z(N + 1, dtype=i32)))
    with pytest.raises(ValueError, match="out"):
        hla.dasc_restore_replay(**rr, out=z(L, N, K, H, dk + 1))
    with pytest.raises(TypeError, match="q"):
        hla.dasc_restore_replay(**dict(rr, q=z(L, N, K, H, dk, dtype=torch.float64)))
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_restore_replay(**rr)
    # the INT8 form: codes int8, one scale per checkpoint row
    r8 = dict(rr)
    del r8["packed"]
    codes = torch.zeros((S, 4, 8, dk), dtype=torch.int8)      # units of 8 channels
    pos8 = z(L, H * dk // 8, dtype=i32)
    with pytest.raises(TypeError, match="codes"):
        hla.dasc_restore_int8_replay(codes.float(), z(S * 4 * 8), **dict(r8, unit_pos=pos8))
    with pytest.raises(ValueError, match="scales"):
        hla.dasc_restore_int8_replay(codes, z(S * 4 * 8 - 1), **dict(r8, unit_pos=pos8))
    with pytest.raises(ValueError, match="unit_pos"):
        hla.dasc_restore_int8_replay(codes, z(S * 4 * 8), **r8)
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_restore_int8_replay(codes, z(S * 4 * 8), **dict(r8, unit_pos=pos8))
    # INT8 checkpoints: codes and scales sized by rows, the FP32 state by the geometry
    rows, dv = 2, 4
    act32 = torch.zeros(L * S * n_units * rows * dv)
    codes = torch.zeros(S * 4 * rows * dv, dtype=torch.int8)
    scales = torch.zeros(S * 4 * rows)
    p8 = dict(active=act32, layer_stride_bytes=S * n_units * rows * dv * 4, S_act=S, L=L,
              n_units=n_units, unit_rows=rows, dv=dv, offsets=offsets, unit_index=idx,
              R_total=4, src_slot=ids, dst_slot=ids, codes=codes, scales=scales, S_ckpt=S)
    with pytest.raises(ValueError, match="scales"):
        hla.dasc_pack_int8(**dict(p8, scales=scales[:-1]))
    with pytest.raises(ValueError, match="codes"):
        hla.dasc_pack_int8(**dict(p8, codes=codes[:-1]))
    with pytest.raises(TypeError, match="active"):
        hla.dasc_pack_int8(**dict(p8, active=act32.double()))
    r8 = dict(codes=codes, scales=scales, S_ckpt=S, R_total=4, unit_pos=pos, L=L,
              n_units=n_units, unit_rows=rows, dv=dv, src_slot=ids, dst_slot=ids,
              active_out=act32, layer_stride_bytes=S * n_units * rows * dv * 4, S_dst=S)
    with pytest.raises(ValueError, match="active_out"):
        hla.dasc_restore_int8(**dict(r8, active_out=act32[:-1]))
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_restore_int8(**r8)
    cb = dict(scratch=active, scratch_layer_stride_bytes=stride, S_scratch=S, active=active,
              layer_stride_bytes=stride, S_act=S, L=L, n_units=n_units, unit_bytes=ub,
              offsets_local=offsets, unit_index_local=idx, R_local=4, src_slot=ids,
              dst_slot=ids)
    with pytest.raises(ValueError, match="scratch"):
        hla.dasc_refresh_local(**dict(cb, scratch=active[:-1]))
    with pytest.raises(ValueError, match="GPU"):
        hla.dasc_refresh_local(**cb)
