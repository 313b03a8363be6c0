"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects every invalid argument with its status code before any HIP call
(so no device is touched: the pointers passed here are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

from block_sparse_attention_spa2_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libspa2.so not built (run __graft_entry__.build())")

FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\*?(spa2_[a-z_]+)\s*\(",
                                 text, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert {"spa2_mask", "spa2_fwd", "spa2_bwd", "spa2_select", "spa2_pool"} <= set(names)
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def good(**kw):
    d = dict(B=1, H=2, N=1000, D=128, BQ=128, BKV=64, dtype=_lib.BF16)
    d.update(kw)
    return _lib.Desc(**d)


def bm(**kw):
    m = dict(mask=FAKE, row_cnt=FAKE, row_idx=FAKE, col_cnt=FAKE, col_idx=FAKE)
    m.update(kw)
    return _lib.BlockMaskC(**m)


def mask_call(desc=None, q=FAKE, k=FAKE, kf=0.1, pf=0.5, out=None, ws=FAKE, wsb=1 << 40):
    L = _lib.lib()
    return L.spa2_mask(C.byref(desc or good()), q, k, kf, pf, C.byref(out or bm()), None, ws,
                       wsb, None)


def test_status_strings():
    L = _lib.lib()
    for s in range(9):
        assert L.spa2_status_str(s) != b"unknown status"
    assert L.spa2_status_str(9) == b"unknown status"
    assert L.spa2_num_blocks(32760, 128) == 256 and L.spa2_num_blocks(75600, 64) == 1182
    assert L.spa2_num_blocks(0, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), _lib.E_SHAPE), (dict(N=(1 << 20) + 1), _lib.E_SHAPE), (dict(B=0), _lib.E_SHAPE),
    (dict(H=-1), _lib.E_SHAPE), (dict(D=96), _lib.E_SHAPE), (dict(D=256), _lib.E_SHAPE),
    (dict(BQ=32), _lib.E_SHAPE), (dict(BQ=512), _lib.E_SHAPE), (dict(BQ=96), _lib.E_SHAPE),
    (dict(BKV=16), _lib.E_SHAPE), (dict(BKV=256), _lib.E_SHAPE), (dict(BKV=48), _lib.E_SHAPE),
    (dict(N=4096 * 64 + 1), _lib.E_SHAPE), (dict(N=4096 * 32 + 1, BKV=32), _lib.E_SHAPE),
    (dict(B=1 << 12, H=1 << 12, N=4096), _lib.E_SHAPE),  # B*H*T_m past the grid bound
    (dict(dtype=7), _lib.E_DTYPE),
])
def test_bad_desc(kw, code):
    assert mask_call(desc=good(**kw)) == code
    L = _lib.lib()
    d = good(**kw)
    assert L.spa2_fwd(C.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None) == code
    assert L.spa2_bwd(C.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE,
                      FAKE, FAKE, 1 << 40, None) == code
    assert L.spa2_bwd_prep(C.byref(d), FAKE, None, FAKE, FAKE, None) == code
    assert L.spa2_bwd_dkdv(C.byref(d), *[FAKE] * 6, None, FAKE, FAKE, None) == code
    assert L.spa2_bwd_dq(C.byref(d), *[FAKE] * 6, 1 << 40, None, FAKE, None) == code
    assert L.spa2_bwd_dq_rowterm(C.byref(d), *[FAKE] * 4, None, FAKE, FAKE, None, FAKE, 1 << 40,
                                 FAKE, None) == code
    n = C.c_size_t(0)
    assert L.spa2_mask_workspace_size(C.byref(d), C.byref(n)) == code


@pytest.mark.parametrize("kf,pf", [(-0.1, 0.5), (1.5, 0.5), (0.1, -1e-9), (0.1, 1.0000001),
                                   (float("nan"), 0.5), (0.1, float("nan")), (0.0, 0.0)])
def test_bad_fractions(kf, pf):
    assert mask_call(kf=kf, pf=pf) == _lib.E_PARAM
    L = _lib.lib()
    assert L.spa2_select(C.byref(good()), FAKE, kf, pf, C.byref(bm()), None) == _lib.E_PARAM


def test_null_pointers():
    L = _lib.lib()
    assert mask_call(q=None) == _lib.E_NULL
    assert mask_call(k=None) == _lib.E_NULL
    for field in ("mask", "row_cnt", "row_idx", "col_cnt", "col_idx"):
        assert mask_call(out=bm(**{field: None})) == _lib.E_NULL
    assert L.spa2_mask(None, FAKE, FAKE, 0.1, 0.5, C.byref(bm()), None, FAKE, 1, None) == _lib.E_NULL
    d = C.byref(good())
    args = [FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None]  # q k v m o lse o_f32 stream
    for i in (0, 1, 2, 4, 5):
        a = list(args)
        a[i] = None
        assert L.spa2_fwd(d, *a) == _lib.E_NULL
    # a mask without row lists
    assert L.spa2_fwd(d, FAKE, FAKE, FAKE, C.byref(bm(row_idx=None)), FAKE, FAKE, None,
                      None) == _lib.E_NULL
    # q k v o o_f32 lse dout m dq dk dv ws ws_bytes stream
    bargs = [FAKE] * 4 + [None] + [FAKE] * 2 + [None] + [FAKE] * 4 + [1 << 40, None]
    for i in (0, 1, 2, 3, 5, 6, 8, 9, 10):
        a = list(bargs)
        a[i] = None
        assert L.spa2_bwd(d, *a) == _lib.E_NULL, i
    assert L.spa2_bwd(d, *bargs[:7], C.byref(bm(col_cnt=None)), *bargs[8:]) == _lib.E_NULL
    # the staged backward: prep (o, o_f32, dout, dvec), dkdv, dq
    assert L.spa2_bwd_prep(d, FAKE, None, None, FAKE, None) == _lib.E_NULL
    assert L.spa2_bwd_prep(d, FAKE, None, FAKE, None, None) == _lib.E_NULL
    st = [FAKE] * 6  # q k v lse dout dvec (dkdv) / workspace (dq)
    for i in range(6):
        a = list(st)
        a[i] = None
        assert L.spa2_bwd_dkdv(d, *a, None, FAKE, FAKE, None) == _lib.E_NULL
        # a missing workspace is a workspace error, like spa2_bwd's
        want = _lib.E_WORKSPACE if i == 5 else _lib.E_NULL
        assert L.spa2_bwd_dq(d, *a, 1 << 40, None, FAKE, None) == want, i
    assert L.spa2_bwd_dkdv(d, *st, C.byref(bm(col_idx=None)), FAKE, FAKE, None) == _lib.E_NULL
    assert L.spa2_bwd_dq(d, *st, 1 << 40, C.byref(bm(row_cnt=None)), FAKE, None) == _lib.E_NULL
    assert L.spa2_bwd_dq(d, *st, 1 << 40, None, None, None) == _lib.E_NULL
    # dQ with the row term: q k v o o_f32 lse dout m ws ws_bytes dq stream
    rargs = [FAKE] * 4 + [None] + [FAKE] * 2 + [None] + [FAKE, 1 << 40, FAKE, None]
    for i in (0, 1, 2, 3, 5, 6, 10):
        a = list(rargs)
        a[i] = None
        assert L.spa2_bwd_dq_rowterm(d, *a) == _lib.E_NULL, i
    assert L.spa2_bwd_dq_rowterm(d, *rargs[:7], C.byref(bm(row_idx=None)),
                                 *rargs[8:]) == _lib.E_NULL
    assert L.spa2_pool(d, FAKE, None, FAKE, FAKE, None) == _lib.E_NULL
    assert L.spa2_mask_lists(d, C.byref(bm(mask=None)), None) == _lib.E_NULL


def test_workspace_checks():
    L = _lib.lib()
    d = good()
    n = C.c_size_t(0)
    assert L.spa2_mask_workspace_size(C.byref(d), C.byref(n)) == _lib.OK
    tm, tn = 8, 16
    # pooled rows padded to D + 2 doubles, plus 256 bytes of alignment slack
    assert n.value == 2 * ((tm + tn) * 130 + tm * tn) * 8 + 256
    assert mask_call(ws=None) == _lib.E_WORKSPACE
    assert mask_call(wsb=n.value - 1) == _lib.E_WORKSPACE
    assert L.spa2_bwd_workspace_size(C.byref(d), C.byref(n)) == _lib.OK
    # bf16: the row term, 256 bytes of alignment slack, a bf16 mean key per 64-key tile
    assert n.value == 2 * 1000 * 4 + 256 + 2 * tn * 128 * 2
    head = [FAKE] * 4 + [None] + [FAKE] * 2 + [None] + [FAKE] * 3
    assert L.spa2_bwd(C.byref(d), *head, FAKE, n.value - 1, None) == _lib.E_WORKSPACE
    assert L.spa2_bwd(C.byref(d), *head, None, n.value, None) == _lib.E_WORKSPACE
    # the staged dQ passes check the same size
    st = [FAKE] * 5  # q k v lse dout
    assert L.spa2_bwd_dq(C.byref(d), *st, FAKE, n.value - 1, None, FAKE, None) == _lib.E_WORKSPACE
    rowterm = [FAKE] * 4 + [None] + [FAKE] * 2 + [None]
    assert L.spa2_bwd_dq_rowterm(C.byref(d), *rowterm, FAKE, n.value - 1, FAKE,
                                 None) == _lib.E_WORKSPACE
    # fp32 keeps no mean keys; 128-key blocks run two 64-key tiles each
    assert L.spa2_bwd_workspace_size(C.byref(good(dtype=_lib.F32)), C.byref(n)) == _lib.OK
    assert n.value == 2 * 1000 * 4
    assert L.spa2_bwd_workspace_size(C.byref(good(BKV=128, D=64)), C.byref(n)) == _lib.OK
    assert n.value == 2 * 1000 * 4 + 256 + 2 * (2 * 8) * 64 * 2


def test_bwd_noalloc_validation():
    """The no-allocation backward validates like spa2_bwd and rejects a problem whose row
    term exceeds its built-in scratch with SPA2_E_SCRATCH, all before any HIP call."""
    L = _lib.lib()
    args = [FAKE] * 4 + [None] + [FAKE] * 2 + [None] + [FAKE] * 3 + [None]
    # q k v o o_f32 lse dout m dq dk dv stream
    assert L.spa2_bwd_noalloc(C.byref(good(D=96)), *args) == _lib.E_SHAPE
    a = list(args)
    a[2] = None
    assert L.spa2_bwd_noalloc(C.byref(good()), *a) == _lib.E_NULL
    a = list(args)
    a[0] = ODD
    assert L.spa2_bwd_noalloc(C.byref(good()), *a) == _lib.E_ALIGN
    # the scratch holds the whole backward workspace: 40 heads of 75,600 tokens fit, at
    # 64- and 32-key blocks; 80 heads do not, nor a workspace one step over the size
    cap = _lib.NOALLOC_SCRATCH_BYTES
    for kw in (dict(H=40, N=75600), dict(H=40, N=75600, BKV=128), dict(H=24, N=75600, BKV=32)):
        assert L.spa2_bwd_workspace_bytes(C.byref(good(**kw))) <= cap, kw
    big = good(B=1, H=80, N=75600)
    assert L.spa2_bwd_workspace_bytes(C.byref(big)) > cap
    assert L.spa2_bwd_noalloc(C.byref(big), *args) == _lib.E_SCRATCH
    assert L.spa2_bwd_noalloc(C.byref(good(B=2, H=40, N=75600)), *args) == _lib.E_SCRATCH
    # fp32 (no mean keys): the largest head count whose row term fits, and one more
    h = cap // (4 * 65536)
    assert L.spa2_bwd_workspace_bytes(C.byref(good(H=h, N=65536, dtype=_lib.F32))) == cap
    assert L.spa2_bwd_noalloc(C.byref(good(H=h + 1, N=65536, dtype=_lib.F32)),
                              *args) == _lib.E_SCRATCH


def test_bwd_workspace_bytes():
    """The size as a return value equals the status-returning size call for every valid
    descriptor, and is 0 for an invalid descriptor or NULL."""
    L = _lib.lib()
    n = C.c_size_t(0)
    for kw in (dict(), dict(B=2, H=3, N=777, D=64, dtype=_lib.F32), dict(N=75600, H=40),
               dict(N=777, BKV=32, D=64)):
        d = good(**kw)
        assert L.spa2_bwd_workspace_size(C.byref(d), C.byref(n)) == _lib.OK
        tiles = -(-d.N // d.BKV) * (2 if d.BKV == 128 else 1)
        kmean = 256 + d.B * d.H * tiles * d.D * 2 if d.dtype == _lib.BF16 else 0
        assert L.spa2_bwd_workspace_bytes(C.byref(d)) == n.value == d.B * d.H * d.N * 4 + kmean
    assert L.spa2_bwd_workspace_bytes(C.byref(good(D=96))) == 0
    assert L.spa2_bwd_workspace_bytes(C.byref(good(dtype=9))) == 0
    assert L.spa2_bwd_workspace_bytes(None) == 0


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    """The Python layer has no fallback: a missing library is an import-time error."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.lib()


@pytest.mark.parametrize("bq,bkv", [(64, 32), (64, 128), (128, 32), (128, 128), (256, 32),
                                    (256, 64), (256, 128)])
def test_block_size_variants_accepted(bq, bkv):
    """Every b_q in {64, 128, 256} and b_kv in {32, 64, 128} passes validation (checked
    through the workspace-size calls, which launch nothing)."""
    L = _lib.lib()
    n = C.c_size_t(0)
    d = good(BQ=bq, BKV=bkv)
    assert L.spa2_mask_workspace_size(C.byref(d), C.byref(n)) == _lib.OK
    assert n.value > 0
    assert L.spa2_bwd_workspace_size(C.byref(d), C.byref(n)) == _lib.OK


ODD = C.c_void_p(0x1008)  # 8-byte aligned, not 16
ODD4 = C.c_void_p(0x1002)  # not 4-byte aligned


def test_misaligned_pointers():
    """Pointers the kernels would load from with wider vector accesses than their alignment
    allows are rejected before any HIP call."""
    L = _lib.lib()
    d = C.byref(good())
    assert mask_call(q=ODD) == _lib.E_ALIGN
    assert mask_call(out=bm(row_idx=ODD4)) == _lib.E_ALIGN
    fargs = [FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None]  # q k v m o lse o_f32 stream
    for i, bad in ((0, ODD), (2, ODD), (4, ODD), (5, ODD4), (6, ODD)):
        a = list(fargs)
        a[i] = bad
        assert L.spa2_fwd(d, *a) == _lib.E_ALIGN, i
    assert L.spa2_fwd(d, FAKE, FAKE, FAKE, C.byref(bm(col_cnt=ODD4)), FAKE, FAKE, None,
                      None) == _lib.E_ALIGN
    # q k v o o_f32 lse dout m dq dk dv ws ws_bytes stream
    bargs = [FAKE] * 4 + [None] + [FAKE] * 2 + [None] + [FAKE] * 4 + [1 << 40, None]
    for i, bad in ((1, ODD), (3, ODD), (5, ODD4), (6, ODD), (10, ODD), (11, ODD4)):
        a = list(bargs)
        a[i] = bad
        assert L.spa2_bwd(d, *a) == _lib.E_ALIGN, i
    assert L.spa2_select(d, ODD4, 0.1, 0.5, C.byref(bm()), None) == _lib.E_ALIGN
    assert L.spa2_pool(d, FAKE, ODD, FAKE, FAKE, None) == _lib.E_ALIGN
    assert L.spa2_mask_lists(d, C.byref(bm(row_cnt=ODD4)), None) == _lib.E_ALIGN


def test_build_rejects_register_spills():
    """The build reads the compiler's per-kernel resource report and names every kernel
    that spills vector registers (a build error for all but the fp32 attention kernels)."""
    from block_sparse_attention_spa2_amd import build
    report = "\n".join([
        "fwd.hip:9:1: remark: Function Name: _ZN4spa210fwd_kernelIDF16bLi128E",
        "fwd.hip:9:1: remark:     VGPRs: 168",
        "fwd.hip:9:1: remark:     VGPRs Spill: 0",
        "bwd.hip:5:1: remark: Function Name: _ZN4spa213bwd_dq_kernelIDF16bLi128E",
        "bwd.hip:5:1: remark:     VGPRs Spill: 12",
        "bwd.hip:7:1: remark: Function Name: _ZN4spa215bwd_dkdv_kernelIfLi128E",
        "bwd.hip:7:1: remark:     VGPRs Spill: 104",
    ])
    assert build._spills(report) == [("_ZN4spa213bwd_dq_kernelIDF16bLi128E", 12),
                                     ("_ZN4spa215bwd_dkdv_kernelIfLi128E", 104)]
    assert build._spills("") == []
