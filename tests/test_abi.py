"""The C-ABI library loads, exports every function include/idx.h declares, and rejects
invalid arguments on the host before any HIP call (CPU only: nothing here launches)."""
import ctypes
import os
import re

import pytest

from key_scoring_exact_amd import _lib
from key_scoring_exact_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")


@pytest.fixture(scope="module")
def L():
    B.ensure_built()
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)
    # the dynamic symbol table holds them as C symbols
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(r"\bT " + n + r"$", out, flags=re.M), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ["IDX_HEADS", "IDX_DIM", "IDX_PAGE_SIZE", "IDX_KMAX", "IDX_GROUP_ROWS", "IDX_MAX_REQ",
                 "IDX_OK", "IDX_EINVAL", "IDX_EUNSUPPORTED", "IDX_EWORKSPACE", "IDX_EHIP", "IDX_EDEVICE",
                 "IDX_ESCRATCH", "IDX_ABI_VERSION"]:
        m = re.search(r"#define " + name + r"\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(_lib, name), name
    for name, expr in [("IDX_MAX_KEYS", r"\(1 << (\d+)\)"), ("IDX_NOALLOC_SCRATCH_BYTES", r"\((\d+)u << 20\)")]:
        m = re.search(r"#define " + name + r"\s+" + expr, text)
        assert m, name
        v = (1 << int(m.group(1))) if name == "IDX_MAX_KEYS" else int(m.group(1)) << 20
        assert v == getattr(_lib, name), name
    # the struct mirrors the header's field order
    body = re.search(r"typedef struct idx_problem \{(.*?)\} idx_problem;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\*?\s*([a-z_]+);", body)
    assert fields == [f for f, _ in _lib.IdxProblem._fields_]


def test_abi_version_and_strerror(L):
    assert L.idx_abi_version() == 3
    for c in range(7):
        assert len(L.idx_strerror(c)) > 0
    assert b"unknown" in L.idx_strerror(99)
    assert L.idx_last_hip_error() is not None


def test_workspace_bytes(L):
    out = ctypes.c_size_t(0)
    assert L.idx_workspace_bytes(4, 131072, 2048, ctypes.byref(out)) == 0
    big = out.value
    assert big % 256 == 0 and big >= 4 * 256 * 128 * 8     # candidate slots: rows x chunks x 128 x 8 B
    assert L.idx_workspace_bytes(1, 4096, 2048, ctypes.byref(out)) == 0
    assert 0 < out.value < big
    assert L.idx_workspace_bytes(0, 10, 2048, ctypes.byref(out)) == _lib.IDX_EINVAL
    assert L.idx_workspace_bytes(1, -1, 2048, ctypes.byref(out)) == _lib.IDX_EINVAL
    assert L.idx_workspace_bytes(1, 10, 0, ctypes.byref(out)) == _lib.IDX_EINVAL
    assert L.idx_workspace_bytes(1, 10, 2049, ctypes.byref(out)) == _lib.IDX_EINVAL
    assert L.idx_workspace_bytes(1, 10, 8, None) == _lib.IDX_EINVAL


def test_workspace_bytes_monotone(L):
    """A workspace sized for (rows, max_keys) serves every call with fewer rows or keys:
    a call checks its workspace against idx_workspace_bytes of its own shape, and the
    size never decreases in either argument (the chunk plan of a smaller key count can
    use more, smaller chunks)."""
    out = ctypes.c_size_t(0)
    for rows in (1, 4, 16):
        prev = 0
        for m in list(range(0, 140000, 257)) + [262143, 300000, 524287, 1 << 20]:
            assert L.idx_workspace_bytes(rows, m, 2048, ctypes.byref(out)) == 0
            assert out.value >= prev, (rows, m)
            prev = out.value
    for m in (0, 30000, 40000, 131072):
        sizes = []
        for rows in (1, 2, 4, 8, 64):
            assert L.idx_workspace_bytes(rows, m, 2048, ctypes.byref(out)) == 0
            sizes.append(out.value)
        assert sizes == sorted(sizes), m


FAKE = 0x10000000  # an aligned address that validation never dereferences


def make_problem(**over):
    ip = (ctypes.c_int32 * 3)(0, 4, 6)
    kw = dict(rows=6, num_req=2, req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)), heads=64, dim=128,
              page_size=64, num_pages=100, max_pages=50, max_keys=3200, q=FAKE, w=FAKE, k_cache=FAKE,
              k_scale=FAKE, page_table=FAKE, n_keys=FAKE, req_max_keys=None)
    kw.update(over)
    return _lib.IdxProblem(**kw), ip


def ws_size(L, rows, max_keys, k=2048):
    out = ctypes.c_size_t(0)
    assert L.idx_workspace_bytes(rows, max_keys, k, ctypes.byref(out)) == 0
    return out.value


def call_all(L, p, k=2048, ld=3200, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ws_size(L, p.rows if p.rows > 0 else 1, max(0, p.max_keys))
    r1 = L.idx_score(ctypes.byref(p), FAKE, ld, ws, ws_bytes, None)
    r2 = L.idx_score_topk(ctypes.byref(p), k, FAKE, ld, FAKE, ws, ws_bytes, None)
    return r1, r2


@pytest.mark.parametrize("field,value,code", [
    ("heads", 32, _lib.IDX_EUNSUPPORTED),
    ("dim", 64, _lib.IDX_EUNSUPPORTED),
    ("page_size", 16, _lib.IDX_EUNSUPPORTED),
    ("rows", 0, _lib.IDX_EINVAL),
    ("num_req", 0, _lib.IDX_EINVAL),
    ("num_req", 300, _lib.IDX_EUNSUPPORTED),
    ("num_pages", 0, _lib.IDX_EINVAL),
    ("max_pages", 0, _lib.IDX_EINVAL),
    ("max_keys", -1, _lib.IDX_EINVAL),
    ("max_keys", 50 * 64 + 1, _lib.IDX_EINVAL),
    ("q", None, _lib.IDX_EINVAL),
    ("q", FAKE + 8, _lib.IDX_EINVAL),
    ("w", None, _lib.IDX_EINVAL),
    ("w", FAKE + 2, _lib.IDX_EINVAL),
    ("k_cache", None, _lib.IDX_EINVAL),
    ("k_cache", FAKE + 4, _lib.IDX_EINVAL),
    ("k_scale", None, _lib.IDX_EINVAL),
    ("page_table", None, _lib.IDX_EINVAL),
    ("n_keys", None, _lib.IDX_EINVAL),
])
def test_problem_validation(L, field, value, code):
    p, keep = make_problem(**{field: value})
    assert call_all(L, p) == (code, code)


def test_req_indptr_validation(L):
    for vals, code in [((0, 4, 5), _lib.IDX_EINVAL),      # last != rows
                       ((1, 4, 6), _lib.IDX_EINVAL),      # first != 0
                       ((0, 0, 6), _lib.IDX_EINVAL)]:     # empty request
        ip = (ctypes.c_int32 * 3)(*vals)
        p, keep = make_problem(req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)))
        assert call_all(L, p) == (code, code), vals
    # a request of more than IDX_GROUP_ROWS rows is split into row groups; more than
    # IDX_MAX_REQ groups in all is refused (1,025 rows in one request: 257 groups; 2 x 512
    # rows: exactly 256)
    for rows, ptr, code in [(1025, (0, 1025), _lib.IDX_EUNSUPPORTED), (1025, (0, 1, 1025), _lib.IDX_EUNSUPPORTED)]:
        ip = (ctypes.c_int32 * len(ptr))(*ptr)
        p, keep = make_problem(rows=rows, num_req=len(ptr) - 1,
                               req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)))
        assert call_all(L, p) == (code, code), ptr
    p, keep = make_problem(req_indptr=None)
    assert call_all(L, p) == (_lib.IDX_EINVAL, _lib.IDX_EINVAL)
    rm = (ctypes.c_int32 * 2)(3200, 3201)                  # a request bound above max_keys
    p, keep = make_problem(req_max_keys=ctypes.cast(rm, ctypes.POINTER(ctypes.c_int32)))
    assert call_all(L, p) == (_lib.IDX_EINVAL, _lib.IDX_EINVAL)


def test_output_and_workspace_validation(L):
    p, keep = make_problem()
    need = ws_size(L, 6, 3200)
    assert L.idx_score(ctypes.byref(p), None, 3200, FAKE, need, None) == _lib.IDX_EINVAL
    assert L.idx_score(ctypes.byref(p), FAKE, 3199, FAKE, need, None) == _lib.IDX_EINVAL      # ld < max_keys
    assert L.idx_score(ctypes.byref(p), FAKE, 3200, None, need, None) == _lib.IDX_EWORKSPACE
    assert L.idx_score(ctypes.byref(p), FAKE, 3200, FAKE + 64, need, None) == _lib.IDX_EWORKSPACE
    assert L.idx_score(ctypes.byref(p), FAKE, 3200, FAKE, need - 256, None) == _lib.IDX_EWORKSPACE
    for k in (0, -3, 2049):
        assert L.idx_score_topk(ctypes.byref(p), k, FAKE, 3200, FAKE, FAKE, need, None) == _lib.IDX_EINVAL
    assert L.idx_score_topk(ctypes.byref(p), 16, FAKE, 3200, None, FAKE, need, None) == _lib.IDX_EINVAL
    assert L.idx_score_topk(ctypes.byref(p), 16, FAKE, 3200, FAKE, FAKE, need - 256, None) == _lib.IDX_EWORKSPACE
    assert L.idx_score(None, FAKE, 3200, FAKE, need, None) == _lib.IDX_EINVAL


def test_topk_validation(L):
    need = ws_size(L, 4, 5000)
    args = dict(scores=FAKE, ld=5000, n_keys=FAKE, rows=4, max_keys=5000, k=2048, topk=FAKE, ws=FAKE, wsb=need)

    def call(**over):
        a = dict(args); a.update(over)
        return L.idx_topk(a["scores"], a["ld"], a["n_keys"], a["rows"], a["max_keys"], a["k"], a["topk"],
                          a["ws"], a["wsb"], None)
    assert call(scores=None) == _lib.IDX_EINVAL
    assert call(scores=FAKE + 2) == _lib.IDX_EINVAL
    assert call(n_keys=None) == _lib.IDX_EINVAL
    assert call(topk=None) == _lib.IDX_EINVAL
    assert call(rows=0) == _lib.IDX_EINVAL
    assert call(max_keys=-1) == _lib.IDX_EINVAL
    assert call(ld=4999) == _lib.IDX_EINVAL
    assert call(k=0) == _lib.IDX_EINVAL
    assert call(k=2049) == _lib.IDX_EINVAL
    assert call(ws=None) == _lib.IDX_EWORKSPACE
    assert call(wsb=need - 256) == _lib.IDX_EWORKSPACE


def test_workspace_init_and_status_validation(L):
    assert L.idx_workspace_init(None, 1024, None) == _lib.IDX_EINVAL
    assert L.idx_workspace_init(FAKE + 16, 1024, None) == _lib.IDX_EINVAL
    assert L.idx_workspace_init(FAKE, 100, None) == _lib.IDX_EINVAL
    assert L.idx_workspace_init(FAKE, 1000, None) == _lib.IDX_EINVAL
    assert L.idx_device_status(None, 1024, None, None) == _lib.IDX_EINVAL



def test_prep_query_validation(L):
    """idx_prep_query refuses bad arguments before any launch."""
    ok = dict(q=FAKE, c=FAKE, s=FAKE, rows=4, rope=64, il=0, out=FAKE + 0x100000)
    cases = [dict(q=None), dict(out=None), dict(rows=0), dict(rope=-2), dict(rope=3), dict(rope=130),
             dict(il=2), dict(c=None), dict(s=None), dict(q=FAKE + 2), dict(out=FAKE + 2), dict(c=FAKE + 1)]
    for over in cases:
        a = dict(ok, **over)
        rc = L.idx_prep_query(a["q"], a["c"], a["s"], a["rows"], a["rope"], a["il"], a["out"], None)
        assert rc == _lib.IDX_EINVAL, over


def test_append_validation(L):
    """idx_score_topk_append refuses a missing or misaligned new-key set and requests of
    more than 16 rows before any launch."""
    p, keep = make_problem()
    need = ws_size(L, 6, 3200)
    def call(nk, prob=p):
        return L.idx_score_topk_append(ctypes.byref(prob), nk, 2048, FAKE, 3200, FAKE, FAKE, need, None)
    good = dict(codes=FAKE, scales=FAKE, pos=FAKE)
    assert call(None) == _lib.IDX_EINVAL
    for over in (dict(codes=None), dict(scales=None), dict(pos=None), dict(codes=FAKE + 4), dict(scales=FAKE + 2),
                 dict(pos=FAKE + 1)):
        nk = _lib.IdxNewKeys(**dict(good, **over))
        assert call(ctypes.byref(nk)) == _lib.IDX_EINVAL, over
    ip = (ctypes.c_int32 * 2)(0, 17)
    p17, keep17 = make_problem(rows=17, num_req=1, req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)))
    nk = _lib.IdxNewKeys(**good)
    assert call(ctypes.byref(nk), p17) == _lib.IDX_EUNSUPPORTED


def test_max_keys_limit(L):
    """Rows above IDX_MAX_KEYS keys are refused before any launch (the selection's score
    offsets are 32-bit)."""
    out = ctypes.c_size_t(0)
    assert L.idx_workspace_bytes(4, _lib.IDX_MAX_KEYS, 2048, ctypes.byref(out)) == 0
    assert L.idx_workspace_bytes(4, _lib.IDX_MAX_KEYS + 1, 2048, ctypes.byref(out)) == _lib.IDX_EUNSUPPORTED
    big = _lib.IDX_MAX_KEYS + 1
    p, keep = make_problem(max_pages=(big + 63) // 64, max_keys=big)
    assert call_all(L, p, ld=big, ws_bytes=1 << 40) == (_lib.IDX_EUNSUPPORTED, _lib.IDX_EUNSUPPORTED)
    rc = L.idx_topk(FAKE, big, FAKE, 4, big, 2048, FAKE, FAKE, 1 << 40, None)
    assert rc == _lib.IDX_EUNSUPPORTED


def test_build_hash_matches_sources(L):
    """The loaded library was built from the current sources and flags."""
    assert L.idx_build_hash().decode() == B.source_hash() == B.library_hash()


def test_tagged_validation(L):
    p, keep = make_problem()
    need = ws_size(L, 6, 3200)
    call = lambda tg: L.idx_score_topk_tagged(ctypes.byref(p), 2048, FAKE, 3200, FAKE, tg, 7, FAKE, need, None)
    assert call(None) == _lib.IDX_EINVAL
    assert call(FAKE + 4) == _lib.IDX_EINVAL
    bad, keep2 = make_problem(heads=32)
    assert L.idx_score_topk_tagged(ctypes.byref(bad), 2048, FAKE, 3200, FAKE, FAKE, 7, FAKE, need, None) == \
        _lib.IDX_EUNSUPPORTED


def test_noalloc_validation(L):
    """idx_score_topk_noalloc checks its arguments like idx_score_topk, and refuses a problem
    whose workspace need exceeds the static scratch, before any HIP call."""
    p, keep = make_problem()
    call = lambda prob, k=2048, sc=FAKE, tk=FAKE, ld=3200: L.idx_score_topk_noalloc(ctypes.byref(prob), k, sc, ld, tk,
                                                                                     None)
    assert call(p, k=0) == _lib.IDX_EINVAL
    assert call(p, tk=None) == _lib.IDX_EINVAL
    assert call(p, sc=None) == _lib.IDX_EINVAL
    assert call(p, ld=3199) == _lib.IDX_EINVAL
    bad, keep2 = make_problem(q=None)
    assert call(bad) == _lib.IDX_EINVAL
    # 64 rows of 131,072 keys need 16 MiB + 256 B of candidate blocks: one header too many
    rows = 64
    ip = (ctypes.c_int32 * 17)(*range(0, rows + 1, 4))
    big, keep3 = make_problem(rows=rows, num_req=16, req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)),
                              max_pages=2048, max_keys=131072, num_pages=2048)
    assert ws_size(L, rows, 131072) > _lib.IDX_NOALLOC_SCRATCH_BYTES
    assert call(big, ld=131072) == _lib.IDX_ESCRATCH
    rows = 60
    ip = (ctypes.c_int32 * 16)(*range(0, rows + 1, 4))
    assert ws_size(L, rows, 131072) <= _lib.IDX_NOALLOC_SCRATCH_BYTES
