"""C-ABI contract tests that need no GPU: the library loads, exports every
declared call, and rejects bad arguments on the host before any HIP call.

Pointers passed here are fake (never dereferenced): every case below fails
validation, which runs before anything touches the device."""
import ctypes

import pytest

from block_sparse_long_rbs_amd import _lib
from oracle import rbs_oracle as orc

E = _lib
P = 0x10000          # fake 16-byte aligned "device" pointer
PM = 0x10004         # misaligned for 16-byte loads


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_library_exports_every_declared_symbol(L):
    names = _lib.declared_symbols()
    assert set(names) >= {"rbs_block_stats", "rbs_select", "blocksparse_attn_fwd",
                          "block_mask_attn_fwd", "rbs_select_capacity", "rbs_status_string"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert _lib.status_string(0) == "ok"
    assert "argument" in _lib.status_string(1)


def stats(L, **kw):
    a = dict(dt=0, q=P, k=P, S=1024, Hq=8, Hkv=2, D=128, B=128, c=P, r=P, qr=P, qn=P)
    a.update(kw)
    return L.rbs_block_stats(a["dt"], a["q"], a["k"], a["S"], a["Hq"], a["Hkv"], a["D"], a["B"],
                             a["c"], a["r"], a["qr"], a["qn"], None)


def test_block_stats_validation(L):
    assert stats(L, q=None) == E.RBS_E_ARG
    assert stats(L, k=PM) == E.RBS_E_ARG
    assert stats(L, c=None) == E.RBS_E_ARG
    assert stats(L, Hq=6, Hkv=4) == E.RBS_E_ARG
    assert stats(L, S=-1) == E.RBS_E_ARG
    assert stats(L, Hkv=0) == E.RBS_E_ARG
    assert stats(L, dt=7) == E.RBS_E_ARG
    assert stats(L, D=96) == E.RBS_E_UNSUPPORTED
    assert stats(L, B=100) == E.RBS_E_UNSUPPORTED
    assert stats(L, B=512) == E.RBS_E_UNSUPPORTED
    assert stats(L, S=0) == E.RBS_OK         # empty input: nothing to do, nothing enqueued


def select(L, ws=None, wsz=1 << 30, cap=1 << 30, **kw):
    a = dict(c=P, r=P, qr=P, qn=P, beta=None, Hkv=4, nb=64, D=128, rc=0.1, rr=0.1, flags=0,
             bo=None, rp=P, ci=P)
    a.update(kw)
    size = ctypes.c_size_t(wsz)
    st = L.rbs_select(a["c"], a["r"], a["qr"], a["qn"], a["beta"], a["Hkv"], a["nb"], a["D"],
                      a["rc"], a["rr"], a["flags"], a["bo"], a["rp"], a["ci"], cap, ws,
                      ctypes.byref(size), None)
    return st, size.value


def test_select_workspace_query_and_capacity(L):
    st, need = select(L, ws=None, wsz=0)
    assert st == E.RBS_OK and need >= 256 + 4 * 256
    assert select(L, ws=0x100000, wsz=need - 1)[0] == E.RBS_E_CAPACITY
    cap = L.rbs_select_capacity(4, 64, 0.1, 0.1, 0)
    assert cap == orc.select_capacity(4, 64, 0.1, 0.1, False)
    assert select(L, ws=0x100000, wsz=need, cap=cap - 1)[0] == E.RBS_E_CAPACITY
    assert L.rbs_select_capacity(4, 1024, 0.03, 0.03, 1) == orc.select_capacity(4, 1024, 0.03, 0.03, True)
    assert L.rbs_select_capacity(1, 16, 0.25, 0.25, 0) == orc.select_capacity(1, 16, 0.25, 0.25, False)
    assert L.rbs_select_capacity(0, 16, 0.25, 0.25, 0) == -1


def test_select_validation(L):
    assert select(L, rc=0.0)[0] == E.RBS_E_ARG
    assert select(L, rr=1.5)[0] == E.RBS_E_ARG
    assert select(L, rc=float("nan"))[0] == E.RBS_E_ARG
    assert select(L, flags=0x4)[0] == E.RBS_E_ARG
    assert select(L, Hkv=0)[0] == E.RBS_E_ARG
    assert select(L, D=80)[0] == E.RBS_E_UNSUPPORTED
    assert select(L, nb=100000)[0] == E.RBS_E_UNSUPPORTED
    assert select(L, ws=0x100001)[0] == E.RBS_E_ARG            # workspace not 256-aligned
    assert select(L, ws=0x100000, rp=None)[0] == E.RBS_E_ARG
    st = L.rbs_select(P, P, P, P, None, 4, 64, 128, 0.1, 0.1, 0, None, P, P, 0, None, None, None)
    assert st == E.RBS_E_ARG                                     # no workspace size pointer


def attn(L, **kw):
    a = dict(dt=0, q=P, k=P, v=P, S=1024, Hq=8, Hkv=2, D=128, B=128, rp=P, ci=P, sc=0.0, o=P,
             lse=None)
    a.update(kw)
    return L.blocksparse_attn_fwd(a["dt"], a["q"], a["k"], a["v"], a["S"], a["Hq"], a["Hkv"],
                                  a["D"], a["B"], a["rp"], a["ci"], a["sc"], a["o"], a["lse"], None)


def test_attention_validation(L):
    assert attn(L, v=None) == E.RBS_E_ARG
    assert attn(L, o=PM) == E.RBS_E_ARG
    assert attn(L, Hq=10, Hkv=4) == E.RBS_E_ARG
    assert attn(L, sc=float("inf")) == E.RBS_E_ARG
    assert attn(L, D=96, B=128) == E.RBS_E_UNSUPPORTED           # head dim 64 or 128 only
    assert attn(L, D=128, B=256) == E.RBS_E_UNSUPPORTED          # block 64 or 128 only
    assert attn(L, dt=1, D=96, B=64) == E.RBS_E_UNSUPPORTED
    assert attn(L, S=0) == E.RBS_OK


def bmask(L, seg=(0, 128, 256, 300), rer=(0, 128, 0), ws=P, wsz=0, size_out=None, **kw):
    a = dict(dt=0, q=P, k=P, v=P, S=300, Hq=8, Hkv=2, D=128, theta=5e5, qrb=0, sc=0.0, o=P,
             lse=None)
    a.update(kw)
    n = len(seg) - 1
    ss = (ctypes.c_int32 * len(seg))(*seg)
    rr = (ctypes.c_int32 * max(1, len(rer)))(*rer)
    sz = ctypes.c_size_t(wsz)
    r = L.block_mask_attn_fwd(a["dt"], a["q"], a["k"], a["v"], a["S"], a["Hq"], a["Hkv"],
                              a["D"], n, ss, rr, a["theta"], a["qrb"], a["sc"], a["o"],
                              a["lse"], ws, ctypes.byref(sz), None)
    if size_out is not None:
        size_out.append(sz.value)
    return r


def test_block_mask_validation(L):
    assert bmask(L, seg=(0, 256, 128, 300)) == E.RBS_E_ARG      # not increasing
    assert bmask(L, seg=(0, 128, 256, 299)) == E.RBS_E_ARG      # does not end at S
    assert bmask(L, seg=(1, 128, 256, 300)) == E.RBS_E_ARG      # does not start at 0
    assert bmask(L, rer=(0, -5, 0)) == E.RBS_E_ARG
    assert bmask(L, theta=0.0) == E.RBS_E_ARG
    assert bmask(L, qrb=301) == E.RBS_E_ARG
    assert bmask(L, seg=(0, 100, 256, 300)) == E.RBS_E_UNSUPPORTED  # start not on a 128 tile
    assert bmask(L, dt=1) == E.RBS_E_UNSUPPORTED
    assert bmask(L, D=64) == E.RBS_E_UNSUPPORTED
    assert bmask(L, qrb=300) == E.RBS_OK                          # no rows requested


def test_block_mask_workspace_query(L):
    def query(**kw):
        got = []
        assert bmask(L, ws=None, size_out=got, **kw) == E.RBS_OK
        return got[0]

    # no offsets and a short final block: nothing to re-encode or split
    assert query(rer=(0, 0, 0)) == 0
    # an offset: the re-encoded keys (S * Hkv * D bf16) and the cos/sin table
    # (n_segments * D/2 float pairs), each rounded up to 256 bytes
    assert query() == 300 * 2 * 128 * 2 + 1536
    # no rows requested: nothing is needed
    assert query(qrb=300) == 0
    # 20 passages of 1536 tokens + a 512-token final block: the final block's
    # 4 query tiles see 241..244 key tiles and are split into 4 chunks of 64
    seg = tuple(range(0, 30721, 1536)) + (31232,)
    rer = tuple(range(0, 30720, 1536)) + (0,)
    kw = dict(seg=seg, rer=rer, S=31232, Hq=32, Hkv=8)
    keys = 31232 * 8 * 128 * 2 + 21 * 64 * 8
    need = query(**kw)
    assert need == keys + 4 * 32 * 4 * 128 * 132 * 4
    # too small a workspace is refused before anything is enqueued
    assert bmask(L, wsz=need - 1, **kw) == E.RBS_E_CAPACITY
    # computing only the final block's last tile still splits its rows
    assert query(qrb=31232 - 100, **kw) == keys + 1 * 32 * 4 * 128 * 132 * 4
    # a misaligned workspace is refused
    assert bmask(L, ws=P + 16, wsz=need, **kw) == E.RBS_E_ARG


def test_per_head_entry_points_validate_before_launch(L):
    sz = ctypes.c_size_t(0)
    # size query: one list per query head (8 heads x 300 rows' worth of workspace)
    r = L.rbs_select_per_head(None, None, None, None, None, 8, 2, 300, 128, 0.1, 0.1, 0, None,
                              None, None, 0, None, ctypes.byref(sz), None)
    assert r == E.RBS_OK and sz.value > 0
    sz2 = ctypes.c_size_t(0)
    r = L.rbs_select(None, None, None, None, None, 8, 300, 128, 0.1, 0.1, 0, None, None, None, 0,
                     None, ctypes.byref(sz2), None)
    assert r == E.RBS_OK and sz2.value == sz.value    # same rows, same workspace
    # query heads not a multiple of KV heads
    r = L.rbs_select_per_head(None, None, None, None, None, 7, 2, 300, 128, 0.1, 0.1, 0, None,
                              None, None, 0, None, ctypes.byref(sz), None)
    assert r == E.RBS_E_ARG
    # stats: missing per-head outputs, bad head dim
    r = L.rbs_block_stats_per_head(0, P, P, 300, 8, 2, 128, 128, P, P, None, None, None)
    assert r == E.RBS_E_ARG
    r = L.rbs_block_stats_per_head(0, P, P, 300, 8, 2, 96, 128, P, P, P, P, None)
    assert r == E.RBS_E_UNSUPPORTED
    # attention: the same shape checks as the group call
    r = L.blocksparse_attn_fwd_per_head(0, P, P, P, 300, 8, 2, 96, 128, P, P, 0.0, P, None, None)
    assert r == E.RBS_E_UNSUPPORTED
    r = L.blocksparse_attn_fwd_per_head(0, P, P, P, 0, 8, 2, 128, 128, P, P, 0.0, P, None, None)
    assert r == E.RBS_OK


def attn8(L, **kw):
    a = dict(q=P, k=P, v=P, S=1024, Hq=8, Hkv=2, D=128, B=128, rp=P, ci=P, sc=0.0, qd=1.0, kd=1.0,
             vd=1.0, o=P, lse=None)
    a.update(kw)
    return L.blocksparse_attn_fwd_fp8(a["q"], a["k"], a["v"], a["S"], a["Hq"], a["Hkv"], a["D"],
                                      a["B"], a["rp"], a["ci"], a["sc"], a["qd"], a["kd"], a["vd"],
                                      a["o"], a["lse"], None)


def test_fp8_attention_validation(L):
    assert attn8(L, q=None) == E.RBS_E_ARG
    assert attn8(L, o=PM) == E.RBS_E_ARG
    assert attn8(L, Hq=10, Hkv=4) == E.RBS_E_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert attn8(L, qd=bad) == E.RBS_E_ARG
        assert attn8(L, kd=bad) == E.RBS_E_ARG
        assert attn8(L, vd=bad) == E.RBS_E_ARG
    assert attn8(L, D=64, B=128) == E.RBS_E_UNSUPPORTED   # head dim 128 only
    assert attn8(L, D=128, B=64) == E.RBS_E_UNSUPPORTED   # block 128 only
    assert attn8(L, S=0) == E.RBS_OK


def test_sizes_beyond_the_supported_range_are_refused(L):
    """A Q (or O) of more than 2^40 elements is refused on the host with
    RBS_E_UNSUPPORTED, before anything is enqueued."""
    big = dict(S=2 ** 30, Hq=16, Hkv=2, D=128)          # 2^41 elements in Q
    assert stats(L, **big) == E.RBS_E_UNSUPPORTED
    assert attn(L, **big) == E.RBS_E_UNSUPPORTED
    assert bmask(L, seg=(0, 2 ** 30), rer=(0,), **big) == E.RBS_E_UNSUPPORTED


def test_select_static_refuses_on_the_host(L):
    """The no-allocation selection entry checks its arguments and the size of
    its static scratch before touching the device; the binding's copy of the
    scratch size equals the header's."""
    import re
    with open(_lib.HEADER) as f:
        m = re.search(r"#define RBS_SELECT_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.RBS_SELECT_STATIC_SCRATCH_BYTES
    s = L.rbs_select_static
    assert s(P, P, P, P, None, 4, 64, 128, 0.0, 0.1, 0, None, P, P, 1 << 20, None) == E.RBS_E_ARG
    assert s(P, P, P, P, None, 4, 64, 80, 0.1, 0.1, 0, None, P, P, 1 << 20, None) \
        == E.RBS_E_UNSUPPORTED
    # one list per query head at 128K needs far more scratch than the array holds
    assert s(P, P, P, P, None, 32, 1024, 128, 0.03, 0.03, 0, None, P, P, 1 << 24, None) \
        == E.RBS_E_CAPACITY


def test_shared_query_validation(L):
    f = L.blocksparse_attn_fwd_shared_query
    ok = dict(dt=0, q=P, k=P, v=P, S=1024, Hq=8, Hkv=2, D=128, B=128, rp=P, ci=P, sc=0.0, o=P)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dt"], a["q"], a["k"], a["v"], a["S"], a["Hq"], a["Hkv"], a["D"], a["B"],
                 a["rp"], a["ci"], a["sc"], a["o"], None, None)
    assert call(dt=1) == E.RBS_E_UNSUPPORTED       # fp32: the vector-ALU path has no pair mode
    assert call(D=64) == E.RBS_E_UNSUPPORTED
    assert call(B=64) == E.RBS_E_UNSUPPORTED
    assert call(q=PM) == E.RBS_E_ARG
    assert call(Hq=7) == E.RBS_E_ARG
    assert call(dt=5) == E.RBS_E_ARG
    assert call(S=0) == E.RBS_OK
