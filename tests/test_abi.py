"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and validates its arguments on the host before any launch.  No call here
reaches a kernel (every call either has an invalid argument or touches no
device memory), so the file is safe with or without a GPU."""
import ctypes
import os
import re

import pytest

import latent_kv_attention_lr_amd as lr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lr_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lr_attn_\w+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ("lr_attn_append_latent", "lr_attn_decode", "lr_attn_decode_explicit",
                 "lr_attn_plan_create", "lr_attn_workspace_bytes"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lr.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def _plan(**kw):
    args = dict(n_layers=1, batch=2, n_heads=4, capacity=300, qfmt=lr.LR_Q_INT8_TOKEN,
                io_dtype=lr.LR_DT_BF16, rank_k=[32, 16, 8, 128], rank_v=[40, 96, 64, 8])
    args.update(kw)
    return lr.lr_attn_plan_create(**args)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=64), lr.LR_EUNSUPPORTED),
    (dict(n_heads=129, rank_k=[32] * 129, rank_v=[32] * 129), lr.LR_EUNSUPPORTED),
    (dict(rank_k=[32, 16, 8, 136]), lr.LR_EUNSUPPORTED),
    (dict(rank_k=[32, 16, 0, 128]), lr.LR_EUNSUPPORTED),
    (dict(rank_v=[40, 96, 64, 12]), lr.LR_EUNSUPPORTED),
    (dict(batch=0), lr.LR_EINVAL),
    (dict(capacity=0), lr.LR_EINVAL),
    (dict(capacity=(1 << 24) + 1), lr.LR_ERANGE),
    (dict(qfmt=7), lr.LR_EINVAL),
    (dict(io_dtype=9), lr.LR_EINVAL),
    (dict(max_splits=-1), lr.LR_EINVAL),
    (dict(wg_waves=6), lr.LR_EINVAL),
    (dict(wg_waves=32), lr.LR_EINVAL),
])
def test_plan_create_rejects(bad, status):
    with pytest.raises(lr.LrAttnError) as e:
        _plan(**bad)
    assert e.value.status == status


def test_plan_layout_is_consistent():
    for qfmt in (lr.LR_Q_INT8_TOKEN, lr.LR_Q_INT4_G32):
        p = _plan(qfmt=qfmt)
        try:
            total = lr.lr_attn_cache_bytes(p, 0)
            assert lr.lr_attn_latent_elems(p, 0, 0) == 32 + 16 + 8 + 128
            assert lr.lr_attn_latent_elems(p, 0, 1) == 40 + 96 + 64 + 8
            assert lr.lr_attn_factor_elems(p, 0, 1) == (40 + 96 + 64 + 8) * 128
            regions = []
            lk = lv = 0
            for h in range(4):
                hl = lr.lr_attn_head_layout_get(p, 0, h)
                for kv in "kv":
                    r = hl["rank_" + kv]
                    rb = r if qfmt == lr.LR_Q_INT8_TOKEN else r // 2
                    sb = 4 if qfmt == lr.LR_Q_INT8_TOKEN else 2 * ((r + 31) // 32)
                    assert hl["row_bytes_" + kv] == rb and hl["scale_bytes_" + kv] == sb
                    assert hl["tile_bytes_" + kv] == 64 * (rb + sb)
                    assert hl["plane_bytes_" + kv] == 5 * 64 * (rb + sb)  # ceil(300 / 64) tiles
                    off = hl[kv + "_offset"]
                    assert off % 256 == 0
                    regions.append((off, off + 2 * hl["plane_bytes_" + kv]))
                assert hl["latent_offset_k"] == lk and hl["latent_offset_v"] == lv
                assert hl["factor_offset_k"] == lk * 128 and hl["factor_offset_v"] == lv * 128
                lk += hl["rank_k"]
                lv += hl["rank_v"]
            regions.sort()
            for (a0, a1), (b0, b1) in zip(regions, regions[1:]):
                assert a1 <= b0
            assert regions[-1][1] <= total
        finally:
            lr.lr_attn_plan_destroy(p)


def test_query_functions_reject_bad_indices():
    p = _plan()
    try:
        assert lr.lr_attn_cache_bytes(p, 1) == 0
        assert lr.lr_attn_latent_elems(p, 0, 2) == 0
        assert lr.lr_attn_workspace_bytes(p, 0) == 0
        assert lr.lr_attn_workspace_bytes(p, 301) == 0
        with pytest.raises(lr.LrAttnError) as e:
            lr.lr_attn_head_layout_get(p, 0, 4)
        assert e.value.status == lr.LR_ERANGE
    finally:
        lr.lr_attn_plan_destroy(p)


def test_workspace_grows_with_context_and_is_aligned():
    # one sequence, 8 heads: few work-groups, so long contexts are split
    p = lr.lr_attn_plan_create(1, 1, 8, 40000, lr.LR_Q_INT4_G32, lr.LR_DT_BF16, [48] * 8, [48] * 8)
    try:
        sizes = [lr.lr_attn_workspace_bytes(p, n) for n in (1, 64, 600, 4096, 32832, 40000)]
        assert all(s % 256 == 0 for s in sizes)
        assert sizes == sorted(sizes)
        assert sizes[0] == 0 and sizes[-1] > 0
    finally:
        lr.lr_attn_plan_destroy(p)


def test_many_sequences_need_no_workspace():
    # 16 x 32 (b, h) work-groups fill the GPU without splitting the context
    p = lr.lr_attn_plan_create(1, 16, 32, 4224, lr.LR_Q_INT8_TOKEN, lr.LR_DT_BF16, [32] * 32, [32] * 32)
    try:
        assert lr.lr_attn_workspace_bytes(p, 4224) == 0
    finally:
        lr.lr_attn_plan_destroy(p)


FAKE = 1 << 20  # a 256-aligned non-null address that is never dereferenced


def _append(p, **kw):
    a = dict(layer=0, cache=FAKE, ck=FAKE, cv=FAKE, pos=FAKE, n_new=1)
    a.update(kw)
    return lr._lib.lr_attn_append_latent(p, a["layer"], a["cache"], a["ck"], a["cv"], a["pos"],
                                         a["n_new"], None)


def _decode(p, fn="lr_attn_decode", **kw):
    a = dict(layer=0, cache=FAKE, len=FAKE, max_len=100, q=FAKE, bk=FAKE, bv=FAKE, scale=0.088,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return getattr(lr._lib, fn)(p, a["layer"], a["cache"], a["len"], a["max_len"], a["q"], a["bk"],
                                a["bv"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_append_argument_errors_before_launch():
    p = _plan()
    try:
        assert _append(None) == lr.LR_EINVAL
        assert _append(p, layer=1) == lr.LR_ERANGE
        assert _append(p, layer=-1) == lr.LR_ERANGE
        assert _append(p, cache=None) == lr.LR_EINVAL
        assert _append(p, ck=None) == lr.LR_EINVAL
        assert _append(p, pos=None) == lr.LR_EINVAL
        assert _append(p, n_new=-1) == lr.LR_EINVAL
        assert _append(p, n_new=301) == lr.LR_ERANGE
        assert _append(p, cache=FAKE + 16) == lr.LR_EINVAL   # cache must be 256-aligned
        assert _append(p, ck=FAKE + 4) == lr.LR_EINVAL       # latents 16-aligned
        assert _append(p, n_new=0) == lr.LR_OK               # no-op, no launch
    finally:
        lr.lr_attn_plan_destroy(p)


@pytest.mark.parametrize("fn", ["lr_attn_decode", "lr_attn_decode_explicit"])
def test_decode_argument_errors_before_launch(fn):
    p = _plan(capacity=3000)
    try:
        assert _decode(None, fn) == lr.LR_EINVAL
        assert _decode(p, fn, layer=3) == lr.LR_ERANGE
        assert _decode(p, fn, max_len=0) == lr.LR_ERANGE
        assert _decode(p, fn, max_len=3001) == lr.LR_ERANGE
        for name in ("cache", "len", "q", "bk", "bv", "out"):
            assert _decode(p, fn, **{name: None}) == lr.LR_EINVAL, name
        assert _decode(p, fn, scale=float("nan")) == lr.LR_EINVAL
        assert _decode(p, fn, scale=float("inf")) == lr.LR_EINVAL
        assert _decode(p, fn, q=FAKE + 8) == lr.LR_EINVAL
        assert _decode(p, fn, cache=FAKE + 64) == lr.LR_EINVAL
        if fn == "lr_attn_decode":   # the explicit form needs no workspace
            need = lr.lr_attn_workspace_bytes(p, 3000)
            assert need > 0
            assert _decode(p, fn, max_len=3000, ws=None) == lr.LR_EWORKSPACE
            assert _decode(p, fn, max_len=3000, ws_bytes=need - 1) == lr.LR_EWORKSPACE
    finally:
        lr.lr_attn_plan_destroy(p)


def _append_decode(p, **kw):
    a = dict(layer=0, cache=FAKE, ck=FAKE, cv=FAKE, pos=FAKE, len=FAKE, max_len=100, q=FAKE,
             bk=FAKE, bv=FAKE, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lr._lib.lr_attn_append_decode(p, a["layer"], a["cache"], a["ck"], a["cv"], a["pos"],
                                         a["len"], a["max_len"], a["q"], a["bk"], a["bv"],
                                         a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_append_decode_argument_errors_before_launch():
    p = _plan(capacity=3000)
    try:
        assert _append_decode(None) == lr.LR_EINVAL
        assert _append_decode(p, layer=3) == lr.LR_ERANGE
        assert _append_decode(p, max_len=0) == lr.LR_ERANGE
        assert _append_decode(p, max_len=3001) == lr.LR_ERANGE
        for name in ("cache", "ck", "cv", "pos", "len", "q", "bk", "bv", "out"):
            assert _append_decode(p, **{name: None}) == lr.LR_EINVAL, name
        assert _append_decode(p, ck=FAKE + 4) == lr.LR_EINVAL      # latents 16-aligned
        assert _append_decode(p, pos=FAKE + 2) == lr.LR_EINVAL     # pos 4-aligned
        assert _append_decode(p, cache=FAKE + 64) == lr.LR_EINVAL
        assert _append_decode(p, scale=float("nan")) == lr.LR_EINVAL
        need = lr.lr_attn_workspace_bytes(p, 3000)
        assert _append_decode(p, max_len=3000, ws=None) == lr.LR_EWORKSPACE
        assert _append_decode(p, max_len=3000, ws_bytes=need - 1) == lr.LR_EWORKSPACE
    finally:
        lr.lr_attn_plan_destroy(p)


def _project(p, **kw):
    a = dict(layer=0, x=FAKE, n=16, embed=4096, packed=FAKE, ck=FAKE, cv=FAKE)
    a.update(kw)
    return lr._lib.lr_attn_project_latent(p, a["layer"], a["x"], a["n"], a["embed"], a["packed"],
                                          a["ck"], a["cv"], None)


def _project_append(p, **kw):
    a = dict(layer=0, cache=FAKE, x=FAKE, embed=4096, packed=FAKE, pos=FAKE, n_new=1,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lr._lib.lr_attn_project_append(p, a["layer"], a["cache"], a["x"], a["embed"],
                                          a["packed"], a["pos"], a["n_new"], a["ws"],
                                          a["ws_bytes"], None)


def test_project_argument_errors_before_launch():
    p = _plan()
    try:
        assert _project(None) == lr.LR_EINVAL
        assert _project(p, layer=1) == lr.LR_ERANGE
        for name in ("x", "packed", "ck", "cv"):
            assert _project(p, **{name: None}) == lr.LR_EINVAL, name
            assert _project(p, **{name: FAKE + 8}) == lr.LR_EINVAL, name   # 16-aligned
        for e in (0, 16, 48, 4095, -32):
            assert _project(p, embed=e) == lr.LR_EINVAL, e                  # multiple of 32, >= 32
        assert _project(p, n=-1) == lr.LR_EINVAL
        assert _project(p, n=0) == lr.LR_OK                                 # no-op, no launch
    finally:
        lr.lr_attn_plan_destroy(p)


def test_pack_projection_size_and_argument_errors():
    p = _plan()
    try:
        # rank_k sums to 184 (12 tiles of 16 rows), rank_v to 208 (13 tiles)
        assert lr.lr_attn_packed_projection_elems(p, 0, 64) == (12 + 13) * 16 * 64
        assert lr.lr_attn_packed_projection_elems(p, 0, 4096) == 25 * 16 * 4096
        for e in (0, 16, 100):
            assert lr.lr_attn_packed_projection_elems(p, 0, e) == 0
        assert lr.lr_attn_packed_projection_elems(p, 1, 64) == 0
        assert lr.lr_attn_packed_projection_elems(None, 0, 64) == 0
        pack = lr._lib.lr_attn_pack_projection
        assert pack(None, 0, 64, FAKE, FAKE, FAKE, None) == lr.LR_EINVAL
        assert pack(p, 1, 64, FAKE, FAKE, FAKE, None) == lr.LR_ERANGE
        assert pack(p, 0, 48, FAKE, FAKE, FAKE, None) == lr.LR_EINVAL
        assert pack(p, 0, 64, None, FAKE, FAKE, None) == lr.LR_EINVAL
        assert pack(p, 0, 64, FAKE, FAKE + 2, FAKE, None) == lr.LR_EINVAL
        assert pack(p, 0, 64, FAKE, FAKE, None, None) == lr.LR_EINVAL
    finally:
        lr.lr_attn_plan_destroy(p)


def test_project_workspace_bytes():
    p = _plan()
    try:
        # rank_k sums to 184, rank_v to 208; batch 2
        for n_new in (1, 3, 300):
            n = 2 * n_new
            want = -(-n * 184 * 4 // 256) * 256 + -(-n * 208 * 4 // 256) * 256
            assert lr.lr_attn_project_workspace_bytes(p, n_new) == want
        assert lr.lr_attn_project_workspace_bytes(p, 0) == 0
        assert lr.lr_attn_project_workspace_bytes(p, 301) == 0
        assert lr.lr_attn_project_workspace_bytes(None, 1) == 0
    finally:
        lr.lr_attn_plan_destroy(p)


def test_append_rejects_more_rows_than_one_grid_holds():
    """batch x n_heads x n_new above 2^26 is a range error, not a launch."""
    p = _plan(batch=1 << 17, n_heads=128, capacity=8, rank_k=[8] * 128, rank_v=[8] * 128)
    try:
        assert _append(p, n_new=5) == lr.LR_ERANGE
        assert _project_append(p, n_new=5) == lr.LR_ERANGE
    finally:
        lr.lr_attn_plan_destroy(p)


def _append_decode_noalloc(p, **kw):
    a = dict(layer=0, cache=FAKE, ck=FAKE, cv=FAKE, pos=FAKE, len=FAKE, max_len=100, q=FAKE,
             bk=FAKE, bv=FAKE, scale=0.088, out=FAKE)
    a.update(kw)
    return lr._lib.lr_attn_append_decode_noalloc(p, a["layer"], a["cache"], a["ck"], a["cv"], a["pos"],
                                                 a["len"], a["max_len"], a["q"], a["bk"], a["bv"],
                                                 a["scale"], a["out"], None)


def test_append_decode_noalloc_argument_errors_before_launch():
    p = _plan(capacity=3000)
    try:
        assert _append_decode_noalloc(None) == lr.LR_EINVAL
        assert _append_decode_noalloc(p, layer=1) == lr.LR_ERANGE
        assert _append_decode_noalloc(p, max_len=0) == lr.LR_ERANGE
        assert _append_decode_noalloc(p, max_len=3001) == lr.LR_ERANGE
    finally:
        lr.lr_attn_plan_destroy(p)


NOALLOC_SCRATCH_BYTES = 2 << 20   # LR_NOALLOC_SCRATCH_BYTES in the header


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define\s+LR_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("qfmt", [lr.LR_Q_INT8_TOKEN, lr.LR_Q_INT4_G32])
@pytest.mark.parametrize("rank", [8, 32, 64, 96, 128])
def test_split_partials_of_any_plan_fit_the_noalloc_scratch(qfmt, rank):
    """The context split keeps (b, h) units x splits below 2048 whatever the
    shape, so every plan's workspace fits the allocation-free entry point's
    array: checked over batch x heads from 1 to 4096 and contexts up to 2^24."""
    worst = 0
    for units in (1, 2, 3, 5, 8, 13, 32, 63, 64, 100, 255, 256, 511, 512, 1000, 1023, 1024, 4096):
        heads = min(units, 128)
        while units % heads:
            heads -= 1
        for cap in (64, 4097, 1 << 16, 1 << 24):
            for waves in (0, 4, 8, 16):
                try:   # caches past 2^40 bytes are a range error of the plan
                    p = _plan(batch=units // heads, n_heads=heads, capacity=cap, qfmt=qfmt,
                              rank_k=[rank] * heads, rank_v=[rank] * heads, wg_waves=waves)
                except lr.LrAttnError as e:
                    assert e.status == lr.LR_ERANGE
                    continue
                try:
                    for ml in sorted({1, 64, 65, cap // 2 + 1, cap}):
                        worst = max(worst, lr.lr_attn_workspace_bytes(p, ml))
                finally:
                    lr.lr_attn_plan_destroy(p)
    assert 0 < worst <= NOALLOC_SCRATCH_BYTES, worst


def _project_append_decode(p, **kw):
    a = dict(layer=0, cache=FAKE, x=FAKE, embed=4096, packed=FAKE, pos=FAKE, len=FAKE, max_len=100,
             q=FAKE, bk=FAKE, bv=FAKE, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lr._lib.lr_attn_project_append_decode(p, a["layer"], a["cache"], a["x"], a["embed"], a["packed"],
                                                 a["pos"], a["len"], a["max_len"], a["q"], a["bk"],
                                                 a["bv"], a["scale"], a["out"], a["ws"], a["ws_bytes"],
                                                 None)


def test_project_append_decode_argument_errors_before_launch():
    p = _plan(capacity=3000)
    try:
        assert _project_append_decode(None) == lr.LR_EINVAL
        assert _project_append_decode(p, layer=1) == lr.LR_ERANGE
        for name in ("cache", "x", "packed", "pos", "len", "q", "bk", "bv", "out"):
            assert _project_append_decode(p, **{name: None}) == lr.LR_EINVAL, name
        assert _project_append_decode(p, x=FAKE + 8) == lr.LR_EINVAL
        assert _project_append_decode(p, pos=FAKE + 2) == lr.LR_EINVAL
        assert _project_append_decode(p, cache=FAKE + 16) == lr.LR_EINVAL
        assert _project_append_decode(p, embed=40) == lr.LR_EINVAL
        assert _project_append_decode(p, embed=0) == lr.LR_EINVAL
        assert _project_append_decode(p, max_len=0) == lr.LR_ERANGE
        assert _project_append_decode(p, max_len=3001) == lr.LR_ERANGE
        assert _project_append_decode(p, scale=float("nan")) == lr.LR_EINVAL
        need = lr.lr_attn_project_decode_workspace_bytes(p, 3000, 4096)
        assert need >= lr.lr_attn_workspace_bytes(p, 3000) + 2 * 2 * 4 * (32 + 16 + 8 + 128)
        assert _project_append_decode(p, max_len=3000, ws=None) == lr.LR_EWORKSPACE
        assert _project_append_decode(p, max_len=3000, ws_bytes=need - 1) == lr.LR_EWORKSPACE
        assert _project_append_decode(p, ws=FAKE + 16) == lr.LR_EINVAL   # 256-aligned
        assert lr.lr_attn_project_decode_workspace_bytes(p, 3001, 4096) == 0
        assert lr.lr_attn_project_decode_workspace_bytes(p, 100, 48) == 0
    finally:
        lr.lr_attn_plan_destroy(p)


def test_project_latent_parts_argument_errors_before_launch():
    p = _plan()
    f = lr._lib.lr_attn_project_latent_parts
    try:
        assert lr.lr_attn_project_parts(p, 0, 2, 4096) >= 1
        assert lr.lr_attn_project_parts(p, 1, 2, 4096) == 0
        assert lr.lr_attn_project_parts(p, 0, 0, 4096) == 0
        assert lr.lr_attn_project_parts(p, 0, 2, 48) == 0
        assert lr.lr_attn_project_parts(p, 0, 2, 32) == 1       # never more parts than steps / 8
        assert f(None, 0, FAKE, 2, 4096, FAKE, 2, FAKE, FAKE, None) == lr.LR_EINVAL
        assert f(p, 1, FAKE, 2, 4096, FAKE, 2, FAKE, FAKE, None) == lr.LR_ERANGE
        assert f(p, 0, FAKE, 2, 4096, FAKE, 0, FAKE, FAKE, None) == lr.LR_EINVAL
        assert f(p, 0, FAKE, 2, 4096, FAKE, 9, FAKE, FAKE, None) == lr.LR_EINVAL
        assert f(p, 0, FAKE, 2, 64, FAKE, 3, FAKE, FAKE, None) == lr.LR_EINVAL   # 2 steps of E
        assert f(p, 0, FAKE, 2, 4096, FAKE, 2, FAKE + 4, FAKE, None) == lr.LR_EINVAL
        assert f(p, 0, FAKE, -1, 4096, FAKE, 2, FAKE, FAKE, None) == lr.LR_EINVAL
        assert f(p, 0, FAKE, 0, 4096, FAKE, 2, FAKE, FAKE, None) == lr.LR_OK   # no-op
    finally:
        lr.lr_attn_plan_destroy(p)


def test_decode_rejects_more_threads_than_one_grid_holds():
    """batch x n_heads work-groups of 512-1024 threads above 2^32 threads in
    all is a range error for every decode entry point, not a launch."""
    p = _plan(batch=1 << 18, n_heads=64, capacity=8, rank_k=[32] * 64, rank_v=[32] * 64)
    try:
        assert _decode(p, max_len=8) == lr.LR_ERANGE
        assert _decode(p, fn="lr_attn_decode_explicit", max_len=8) == lr.LR_ERANGE
        assert _append_decode(p, max_len=8) == lr.LR_ERANGE
    finally:
        lr.lr_attn_plan_destroy(p)


def test_project_append_argument_errors_before_launch():
    p = _plan()
    try:
        assert _project_append(None) == lr.LR_EINVAL
        assert _project_append(p, layer=2) == lr.LR_ERANGE
        for name in ("cache", "x", "packed", "pos"):
            assert _project_append(p, **{name: None}) == lr.LR_EINVAL, name
        assert _project_append(p, cache=FAKE + 16) == lr.LR_EINVAL
        assert _project_append(p, pos=FAKE + 2) == lr.LR_EINVAL
        assert _project_append(p, embed=40) == lr.LR_EINVAL
        assert _project_append(p, n_new=-1) == lr.LR_EINVAL
        assert _project_append(p, n_new=301) == lr.LR_ERANGE
        need = lr.lr_attn_project_workspace_bytes(p, 5)
        assert _project_append(p, n_new=5, ws=None) == lr.LR_EWORKSPACE
        assert _project_append(p, n_new=5, ws_bytes=need - 1) == lr.LR_EWORKSPACE
        assert _project_append(p, n_new=5, ws=FAKE + 16) == lr.LR_EINVAL   # 256-aligned
        assert _project_append(p, n_new=0) == lr.LR_OK                     # no-op, no launch
    finally:
        lr.lr_attn_plan_destroy(p)


def test_explicit_form_rejects_fp32_io_before_launch():
    p = _plan(io_dtype=lr.LR_DT_F32)
    try:
        assert _decode(p, "lr_attn_decode_explicit") == lr.LR_EUNSUPPORTED
    finally:
        lr.lr_attn_plan_destroy(p)


def test_strerror_covers_every_status():
    seen = {lr.lr_attn_strerror(s) for s in range(6)}
    assert len(seen) == 6 and "unknown status" not in seen
    assert lr.lr_attn_strerror(99) == "unknown status"


def test_product_package_never_loads_the_oracle():
    pkg = os.path.join(ROOT, "latent_kv_attention_lr_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
    assert "oracle" not in open(HEADER).read().lower()


@pytest.mark.parametrize("src,nbytes,sink", [
    (None, 1 << 20, 0x1000),        # null source
    (0x1000, 1 << 20, None),        # null sink
    (0x1000, 8, 0x2000),            # fewer than 16 bytes
    (0x1008, 1 << 20, 0x2000),      # source not 16-byte aligned
    (0x1000, 1 << 20, 0x2002),      # sink not 4-byte aligned
])
def test_probe_read_rejects_bad_arguments(src, nbytes, sink):
    # rejected on the host: these addresses are never dereferenced
    st = lr._lib.lr_attn_probe_read(src, nbytes, sink, None)
    assert st == lr.LR_EINVAL
