"""The C-ABI library without a GPU: it loads, exports every entry point that
include/mla_dsa.h declares, and its host-side validation returns the documented status
before any HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re
import subprocess

import pytest

import mla_latent_kv_dsa_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_dsa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla_dsa.so is not built (python -m mla_latent_kv_dsa_amd.build)")
    return mla.lib()


def test_header_declares_the_five_calls():
    fns = _declared_functions()
    for name in ("mla_rope_interleave", "dsa_index_scores", "dsa_topk_select", "mla_absorbed_decode",
                 "mla_prefill_nonabsorbed"):
        assert name in fns
    assert set(fns) == set(mla.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for fn in _declared_functions():
        assert fn in exported, fn
        assert hasattr(L, fn)


def test_status_strings(L):
    assert mla.mla_status_string(0) == "MLA_OK"
    assert mla.mla_status_string(-3) == "MLA_ERR_WORKSPACE"
    assert mla.mla_status_string(-99) == "MLA_ERR_UNKNOWN"


# Fake (never dereferenced) device addresses: every call below fails host validation first.
FAKE = ctypes.c_void_p(0x1000)


def _no_gpu():
    # On a GPU machine an unexpected pass of validation would launch on fake pointers;
    # these checks are host logic and run where no GPU is visible.
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation tests run without a GPU")


def _view(**kw):
    v = mla.mla_kv_view()
    v.lc, v.rc, v.ic = 0x1000, 0x2000, 0x3000
    v.rows, v.kv_dtype, v.index_hd = 4096, mla.MLA_BF16, 128
    v.block_table, v.block_size, v.max_blocks = None, 0, 0
    v.seq_stride, v.seq_len, v.max_seq_len = 4096, 0x4000, 4096
    for k, val in kw.items():
        setattr(v, k, val)
    return v


def _dims(**kw):
    d = mla.mla_dims()
    d.n_heads, d.qk_nope, d.qk_rope, d.v_head, d.kv_lora = 64, 192, 64, 256, 512
    for k, val in kw.items():
        setattr(d, k, val)
    return d


def test_rope_validation(L):
    _no_gpu()
    r = lambda **kw: L.mla_rope_interleave(FAKE, kw.get("dt", 0), kw.get("n", 4), kw.get("h", 2),
                                            kw.get("ts", 512), kw.get("hs", 256), kw.get("off", 192),
                                            kw.get("rd", 64), FAKE, kw.get("theta", 1e4), None)
    assert r(rd=63) == mla.MLA_ERR_ARG
    assert r(rd=0) == mla.MLA_ERR_ARG
    assert r(rd=1024) == mla.MLA_ERR_UNSUPPORTED
    assert r(dt=7) == mla.MLA_ERR_ARG
    assert r(theta=-1.0) == mla.MLA_ERR_ARG
    assert r(hs=100) == mla.MLA_ERR_ARG          # heads overlap
    assert r(ts=300) == mla.MLA_ERR_ARG          # tokens overlap
    assert r(n=0) == mla.MLA_OK                  # nothing to do, nothing launched
    assert "rope" in mla.mla_last_error() or mla.mla_last_error() == ""


def test_index_validation(L):
    _no_gpu()
    f = lambda B=1, n_ih=32, v=None, t_max=4096: L.dsa_index_scores(FAKE, FAKE, B, n_ih, ctypes.byref(v or _view()), t_max, FAKE, None)
    assert f(n_ih=0) == mla.MLA_ERR_ARG
    assert f(n_ih=65) == mla.MLA_ERR_UNSUPPORTED
    assert f(v=_view(ic=None)) == mla.MLA_ERR_ARG
    assert f(v=_view(index_hd=130)) == mla.MLA_ERR_ARG
    assert f(v=_view(index_hd=512)) == mla.MLA_ERR_UNSUPPORTED
    assert f(v=_view(seq_len=None)) == mla.MLA_ERR_ARG
    assert f(B=2, v=_view(seq_stride=100)) == mla.MLA_ERR_ARG          # sequences overlap
    assert f(B=2, v=_view(rows=5000)) == mla.MLA_ERR_ARG               # second sequence past the pool
    assert f(v=_view(block_table=0x5000, block_size=64, max_blocks=10)) == mla.MLA_ERR_ARG  # table too short
    assert f(v=_view(block_table=0x5000, block_size=64, max_blocks=64, rows=4000)) == mla.MLA_ERR_ARG
    assert f(t_max=1 << 31) == mla.MLA_ERR_UNSUPPORTED
    assert f(B=0) == mla.MLA_OK


def test_topk_validation(L):
    _no_gpu()
    f = lambda B=1, t=4096, k=2048, ws=None, wsb=0: L.dsa_topk_select(FAKE, B, t, FAKE, k, FAKE, FAKE, ws, wsb, None)
    assert f(k=0) == mla.MLA_ERR_ARG
    assert f(k=70000) == mla.MLA_ERR_UNSUPPORTED
    assert f(B=-1) == mla.MLA_ERR_ARG
    assert f(t=1 << 31) == mla.MLA_ERR_UNSUPPORTED
    assert L.dsa_topk_select(FAKE, 1, 4096, None, 8, FAKE, FAKE, None, 0, None) == mla.MLA_ERR_ARG
    need = L.dsa_topk_workspace_bytes(1, 4096, 2048)
    if need:
        assert f(ws=None) == mla.MLA_ERR_WORKSPACE
        assert f(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE
    assert f(B=0) == mla.MLA_OK


def test_index_select_validation(L):
    _no_gpu()

    def f(B=1, n_ih=32, t=4096, k=2048, v=None, ws=None, wsb=0, scores=FAKE):
        return L.dsa_index_select(FAKE, FAKE, B, n_ih, ctypes.byref(v or _view()), t, k, scores, FAKE, FAKE, ws, wsb,
                                  None)
    need = L.dsa_index_select_workspace_bytes(1, 4096, 2048)
    assert need > 0
    assert f() == mla.MLA_ERR_WORKSPACE
    assert f(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE
    assert f(k=0) == mla.MLA_ERR_ARG
    assert f(k=70000) == mla.MLA_ERR_UNSUPPORTED
    assert f(n_ih=0) == mla.MLA_ERR_ARG
    assert f(B=-1) == mla.MLA_ERR_ARG
    assert f(t=1 << 31) == mla.MLA_ERR_UNSUPPORTED
    assert f(scores=None, ws=FAKE, wsb=need) == mla.MLA_ERR_ARG
    assert f(v=_view(ic=None)) == mla.MLA_ERR_ARG
    assert f(B=0) == mla.MLA_OK
    assert L.dsa_index_select_workspace_bytes(1, 300000, 2048) >= L.dsa_topk_workspace_bytes(1, 300000, 2048)


def test_decode_validation(L):
    _no_gpu()
    d = _dims()

    def f(d=d, B=1, v=None, q_dt=1, w_dt=1, sel=None, nsel=None, sel_stride=0, ws=None, wsb=0, scale=0.0625):
        return L.mla_absorbed_decode(FAKE, FAKE, q_dt, FAKE, w_dt, ctypes.byref(d), B, ctypes.byref(v or _view()),
                                     sel, nsel, sel_stride, scale, FAKE, ws, wsb, None)
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 4096)
    assert need > 0
    assert f() == mla.MLA_ERR_WORKSPACE
    assert f(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE
    assert f(d=_dims(n_heads=0)) == mla.MLA_ERR_ARG
    assert f(d=_dims(kv_lora=4096)) == mla.MLA_ERR_UNSUPPORTED
    assert f(q_dt=0) == mla.MLA_ERR_UNSUPPORTED         # mixed dtypes
    assert f(q_dt=5) == mla.MLA_ERR_ARG
    assert f(sel=FAKE, nsel=None, sel_stride=2048) == mla.MLA_ERR_ARG
    assert f(sel=FAKE, nsel=FAKE, sel_stride=0) == mla.MLA_ERR_ARG
    assert f(v=_view(lc=None)) == mla.MLA_ERR_ARG
    assert f(scale=float("inf")) == mla.MLA_ERR_ARG
    assert f(B=0) == mla.MLA_OK


def test_decode_split_validation(L):
    _no_gpu()
    d = _dims()

    def a(d=d, B=1, q_dt=1, w_dt=1, q=FAKE, w=FAKE, ws=None, wsb=0):
        return L.mla_decode_absorb(q, q_dt, w, w_dt, ctypes.byref(d), B, ws, wsb, None)

    def t(d=d, B=1, v=None, q_dt=1, w_dt=1, sel=None, nsel=None, sel_stride=0, ws=None, wsb=0, scale=0.0625):
        return L.mla_decode_attend(FAKE, q_dt, FAKE, w_dt, ctypes.byref(d), B, ctypes.byref(v or _view()), sel, nsel,
                                   sel_stride, scale, FAKE, ws, wsb, None)
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 4096)
    assert a() == mla.MLA_ERR_WORKSPACE                  # the absorb step still needs its part
    assert a(ws=FAKE, wsb=1) == mla.MLA_ERR_WORKSPACE
    assert a(q_dt=0) == mla.MLA_ERR_UNSUPPORTED
    assert a(q=None, ws=FAKE, wsb=need) == mla.MLA_ERR_ARG
    assert a(d=_dims(n_heads=0)) == mla.MLA_ERR_ARG
    assert a(B=-1) == mla.MLA_ERR_ARG
    assert a(B=0) == mla.MLA_OK
    assert t() == mla.MLA_ERR_WORKSPACE
    assert t(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE
    assert t(sel=FAKE, nsel=None, sel_stride=2048) == mla.MLA_ERR_ARG
    assert t(v=_view(lc=None)) == mla.MLA_ERR_ARG
    assert t(scale=float("nan")) == mla.MLA_ERR_ARG
    assert t(B=0) == mla.MLA_OK


def test_prefill_validation(L):
    _no_gpu()
    d = _dims()

    def f(S=4096, pb=0, v=None, ws=None, wsb=0, out_dt=0):
        return L.mla_prefill_nonabsorbed(FAKE, 1, FAKE, 1, ctypes.byref(d), ctypes.byref(v or _view(seq_len=None)),
                                         S, pb, 0.0625, FAKE, out_dt, ws, wsb, None)
    need = L.mla_prefill_workspace_bytes(ctypes.byref(d), 4096, 4096)
    assert need > 0
    assert f() == mla.MLA_ERR_WORKSPACE
    assert f(S=-1) == mla.MLA_ERR_ARG
    assert f(out_dt=9) == mla.MLA_ERR_ARG
    assert f(S=4000, pb=200) == mla.MLA_ERR_ARG          # rows 0..4199 exceed the 4096-row pool
    assert f(S=0) == mla.MLA_OK


def test_workspace_queries_are_host_only(L):
    d = _dims()
    assert L.mla_decode_workspace_bytes(ctypes.byref(d), 32, 2048) >= L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 2048)
    assert L.mla_decode_workspace_bytes(None, 1, 2048) == 0
    assert L.mla_prefill_workspace_bytes(ctypes.byref(d), 4096, 4096) >= 4096 * 64 * (192 + 256) * 2
    assert L.dsa_topk_workspace_bytes(0, 10, 10) == 0


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mla.lib()


def test_dsa_decode_validation(L):
    _no_gpu()
    d = _dims()

    def f(d=d, B=1, v=None, q_dt=1, w_dt=1, theta=1e4, n_ih=32, t=4096, k=2048, scale=0.0625, ws=None, wsb=0,
          scores=FAKE, out=FAKE):
        return L.mla_dsa_decode(FAKE, FAKE, q_dt, theta, FAKE, FAKE, n_ih, FAKE, w_dt, ctypes.byref(d), B,
                                ctypes.byref(v or _view()), t, k, scale, scores, FAKE, FAKE, out, ws, wsb, None)
    need = L.mla_dsa_decode_workspace_bytes(ctypes.byref(d), 1, 4096, 2048)
    assert need >= L.dsa_index_select_workspace_bytes(1, 4096, 2048) + L.mla_decode_workspace_bytes(
        ctypes.byref(d), 1, 2048)
    assert f() == mla.MLA_ERR_WORKSPACE
    assert f(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE
    assert f(d=_dims(n_heads=0)) == mla.MLA_ERR_ARG
    assert f(q_dt=0) == mla.MLA_ERR_UNSUPPORTED          # mixed dtypes
    assert f(theta=0.0) == mla.MLA_ERR_ARG
    assert f(theta=float("nan")) == mla.MLA_ERR_ARG
    assert f(scale=float("inf")) == mla.MLA_ERR_ARG
    assert f(n_ih=0) == mla.MLA_ERR_ARG
    assert f(k=0) == mla.MLA_ERR_ARG
    assert f(k=70000) == mla.MLA_ERR_UNSUPPORTED
    assert f(t=-1) == mla.MLA_ERR_ARG
    assert f(t=1 << 31) == mla.MLA_ERR_UNSUPPORTED
    assert f(v=_view(ic=None)) == mla.MLA_ERR_ARG
    assert f(v=_view(lc=None)) == mla.MLA_ERR_ARG
    assert f(v=_view(seq_len=None)) == mla.MLA_ERR_ARG
    assert f(v=_view(index_hd=6)) == mla.MLA_ERR_ARG
    assert f(out=None, ws=FAKE, wsb=need) == mla.MLA_ERR_ARG
    assert f(scores=None, ws=FAKE, wsb=need) == mla.MLA_ERR_ARG
    assert f(B=0) == mla.MLA_OK


def test_tiled_index_pool_validation(L):
    _no_gpu()

    def f(v):
        return L.dsa_index_scores(FAKE, FAKE, 2, 32, ctypes.byref(v), 4096, FAKE, None)
    assert f(_view(ic_layout=2)) == mla.MLA_ERR_ARG
    assert f(_view(ic_layout=mla.MLA_IC_TILE64, rows=4100)) == mla.MLA_ERR_ARG          # rows % 64
    assert f(_view(ic_layout=mla.MLA_IC_TILE64, rows=2 * 4160, seq_stride=4100)) == mla.MLA_ERR_ARG   # stride % 64
    bt = ctypes.c_void_p(0x5000)
    assert f(_view(ic_layout=mla.MLA_IC_TILE64, block_table=bt.value, block_size=16, max_blocks=256)) == mla.MLA_ERR_ARG


def test_misaligned_pointers_rejected_alike(L):
    """On the matrix-core geometry a tensor that is not 16-byte aligned gives MLA_ERR_UNSUPPORTED in
    every decode and prefill call (fused, split, whole step, prefill), before anything is launched:
    no call switches kernels because of where a pointer sits.  fp32 inputs take the generic kernels."""
    _no_gpu()
    d = _dims()
    MIS = ctypes.c_void_p(0x1002)
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 4096)
    ws = ctypes.c_void_p(0x100000)
    for args in ((MIS, FAKE, FAKE), (FAKE, MIS, FAKE), (FAKE, FAKE, MIS)):
        qn, qr, kvb = args
        st = L.mla_absorbed_decode(qn, qr, 1, kvb, 1, ctypes.byref(d), 1, ctypes.byref(_view()), None, None, 0,
                                   0.0625, FAKE, ws, need, None)
        assert st == mla.MLA_ERR_UNSUPPORTED, args
    st = L.mla_absorbed_decode(FAKE, FAKE, 1, FAKE, 1, ctypes.byref(d), 1, ctypes.byref(_view(lc=0x1002)), None,
                               None, 0, 0.0625, FAKE, ws, need, None)
    assert st == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_decode_absorb(MIS, 1, FAKE, 1, ctypes.byref(d), 1, ws, need, None) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_decode_attend(FAKE, 1, FAKE, 1, ctypes.byref(d), 1, ctypes.byref(_view(rc=0x2002)), None, None, 0,
                               0.0625, FAKE, ws, need, None) == mla.MLA_ERR_UNSUPPORTED
    need2 = L.mla_dsa_decode_workspace_bytes(ctypes.byref(d), 1, 4096, 2048)
    assert L.mla_dsa_decode(MIS, FAKE, 1, 1e4, FAKE, FAKE, 32, FAKE, 1, ctypes.byref(d), 1, ctypes.byref(_view()),
                            4096, 2048, 0.0625, FAKE, FAKE, FAKE, FAKE, ws, need2, None) == mla.MLA_ERR_UNSUPPORTED
    needp = L.mla_prefill_workspace_bytes(ctypes.byref(d), 4096, 4096)
    for q, out, v in ((MIS, FAKE, _view(seq_len=None)), (FAKE, MIS, _view(seq_len=None)),
                      (FAKE, FAKE, _view(seq_len=None, lc=0x1008))):
        assert L.mla_prefill_nonabsorbed(q, 1, FAKE, 1, ctypes.byref(d), ctypes.byref(v), 4096, 0, 0.0625, out, 0,
                                         ws, needp, None) == mla.MLA_ERR_UNSUPPORTED
    assert "16-byte aligned" in mla.mla_last_error()


def test_noalloc_decode_validation(L):
    """mla_dsa_decode_noalloc validates like mla_dsa_decode, and a step whose workspace exceeds the
    library's static scratch is refused with MLA_ERR_WORKSPACE before any HIP call."""
    _no_gpu()
    d = _dims()
    BT = ctypes.c_void_p(0x5000)

    def f(B=1, v=None, t=4096, k=2048, q_dt=1, out=FAKE):
        return L.mla_dsa_decode_noalloc(FAKE, FAKE, q_dt, 1e4, FAKE, FAKE, 32, FAKE, 1, ctypes.byref(d), B,
                                        ctypes.byref(v or _view()), t, k, 0.0625, FAKE, FAKE, FAKE, out, None)
    assert f(q_dt=0) == mla.MLA_ERR_UNSUPPORTED
    assert f(out=None) == mla.MLA_ERR_ARG
    assert f(k=0) == mla.MLA_ERR_ARG
    assert f(B=0) == mla.MLA_OK
    paged = _view(block_table=BT.value, block_size=64, max_blocks=2048, rows=4096, max_seq_len=131072)
    need = L.mla_dsa_decode_workspace_bytes(ctypes.byref(d), 32, 131072, 2048)
    assert need > (64 << 20)
    assert f(B=32, v=paged, t=131072) == mla.MLA_ERR_WORKSPACE
    assert "static scratch" in mla.mla_last_error()


def test_cache_write_and_shared_decode_validation(L):
    _no_gpu()
    d = _dims()

    def cw(n=4, dt=1, ik=FAKE, nseq=2, kvl=512, rope=64, off=64, rd=64, eps=1e-6, v=None):
        return L.mla_cache_write(FAKE, ik, dt, n, FAKE, FAKE, nseq, kvl, rope, None, None, None, off, rd, eps, 1e-6,
                                 1e4, ctypes.byref(v or _view(seq_len=None)), None)
    assert cw(dt=3) == mla.MLA_ERR_ARG
    assert cw(n=-1) == mla.MLA_ERR_ARG
    assert cw(nseq=0) == mla.MLA_ERR_ARG
    assert cw(rope=63) == mla.MLA_ERR_ARG
    assert cw(kvl=4096) == mla.MLA_ERR_UNSUPPORTED
    assert cw(eps=0.0) == mla.MLA_ERR_ARG
    assert cw(off=100, rd=64) == mla.MLA_ERR_ARG            # slice past the 128-wide key
    assert cw(rd=3) == mla.MLA_ERR_ARG
    assert cw(v=_view(seq_len=None, ic=None)) == mla.MLA_ERR_ARG   # ik given, no indexer pool
    assert cw(n=0, nseq=1) == mla.MLA_OK

    def sh(sel=FAKE, nsel=FAKE, k=2048, ws=None, wsb=0, theta=1e4):
        return L.mla_dsa_decode_shared(FAKE, FAKE, 1, theta, FAKE, 1, ctypes.byref(d), 1, ctypes.byref(_view()), sel,
                                       nsel, k, 0.0625, FAKE, ws, wsb, None)
    need = L.mla_dsa_decode_shared_workspace_bytes(ctypes.byref(d), 1, 2048)
    assert need >= L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 2048)
    assert sh(sel=None) == mla.MLA_ERR_ARG
    assert sh(k=0) == mla.MLA_ERR_ARG
    assert sh(theta=-1.0) == mla.MLA_ERR_ARG
    assert sh() == mla.MLA_ERR_WORKSPACE
    assert sh(ws=FAKE, wsb=need - 1) == mla.MLA_ERR_WORKSPACE


def test_g_absorb_rule_and_attention_validation(L):
    """colibri-analysis 06, sec. 2.3: g_absorb -1 absorbs when S <= 4, 0 never, 1 always."""
    assert [L.mla_attention_absorbs(S, -1) for S in (1, 2, 3, 4, 5, 64, 4096)] == [1, 1, 1, 1, 0, 0, 0]
    assert [L.mla_attention_absorbs(S, 0) for S in (1, 4, 4096)] == [0, 0, 0]
    assert [L.mla_attention_absorbs(S, 1) for S in (1, 4, 4096)] == [1, 1, 1]
    _no_gpu()
    d = _dims()

    def f(S=4, pb=100, g=-1, sel=None, nsel=None, stride=0, ws=None, wsb=0):
        return L.mla_attention(FAKE, 1, FAKE, 1, ctypes.byref(d), ctypes.byref(_view(seq_len=None)), S, pb, sel, nsel,
                               stride, 0.0625, g, FAKE, ws, wsb, None)
    need = L.mla_attention_workspace_bytes(ctypes.byref(d), 4, 100, 0, -1)
    assert need > 0
    assert f() == mla.MLA_ERR_WORKSPACE
    assert f(g=2) == mla.MLA_ERR_ARG
    assert f(S=-1) == mla.MLA_ERR_ARG
    assert f(sel=FAKE, nsel=None, stride=8) == mla.MLA_ERR_ARG
    assert f(S=8, g=0, sel=FAKE, nsel=FAKE, stride=1 << 19) == mla.MLA_ERR_UNSUPPORTED   # the key bitmap's limit
    assert f(S=4000, pb=200) == mla.MLA_ERR_ARG          # rows beyond the 4096-row pool
    assert f(S=0) == mla.MLA_OK
    assert L.mla_attention_workspace_bytes(ctypes.byref(d), 4096, 0, 2048, 0) > \
        L.mla_attention_workspace_bytes(ctypes.byref(d), 4096, 0, 0, 0)      # the key bitmap

    def ps(S=8, pb=100, k=16, n_ih=32, ws=None, wsb=0):
        return L.dsa_prefill_select(FAKE, FAKE, n_ih, ctypes.byref(_view(seq_len=None)), S, pb, k, FAKE, FAKE, FAKE,
                                    ws, wsb, None)
    assert ps() == mla.MLA_ERR_WORKSPACE
    assert ps(k=0) == mla.MLA_ERR_ARG
    assert ps(n_ih=65) == mla.MLA_ERR_UNSUPPORTED
    assert ps(S=0) == mla.MLA_OK


def test_quantized_decode_validation(L):
    _no_gpu()
    d = _dims()
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 1, 4096)

    def f(fmt=1, codes=FAKE, scales=FAKE, dd=None, q_dt=1, ws=FAKE, wsb=None):
        w = mla.mla_qweights()
        w.codes, w.scales, w.format = codes.value if codes else None, scales.value if scales else None, fmt
        return L.mla_absorbed_decode_q(FAKE, FAKE, q_dt, ctypes.byref(w), ctypes.byref(dd or d), 1,
                                       ctypes.byref(_view()), None, None, 0, 0.0625, FAKE, ws,
                                       need if wsb is None else wsb, None)
    assert f(fmt=0) == mla.MLA_ERR_ARG
    assert f(fmt=4) == mla.MLA_ERR_ARG
    assert f(codes=None) == mla.MLA_ERR_ARG
    assert f(scales=ctypes.c_void_p(0x1002)) == mla.MLA_ERR_UNSUPPORTED     # 4-byte alignment
    assert f(dd=_dims(kv_lora=256)) == mla.MLA_ERR_UNSUPPORTED              # not the matrix-core geometry
    assert f(q_dt=0) == mla.MLA_ERR_UNSUPPORTED
    assert f(wsb=need - 1) == mla.MLA_ERR_WORKSPACE
