"""Host checks of the C ABI: libmsa.so loads without a GPU, exports every entry point that
include/msa.h declares, and rejects invalid arguments before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(ROOT, "block_sparse_attention_nvfp4_amd", "libmsa.so")


def declared_functions():
    """Every function the headers under include/ declare (msa.h and msa_probe.h)."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def msa():
    if not os.path.exists(LIB):
        import importlib.util
        path = os.path.join(os.path.dirname(LIB), "build.py")
        spec = importlib.util.spec_from_file_location("msa_build", path)
        build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build)
        build.build()
    import block_sparse_attention_nvfp4_amd as m
    return m


def test_header_declares_the_path(msa):
    fns = declared_functions()
    for f in ("msa_kv_insert_nvfp4", "msa_indexer_score", "msa_block_topk", "msa_sparse_attn_decode"):
        assert f in fns
    assert set(fns) == set(msa.EXPORTED)


def test_library_exports_every_declared_symbol(msa):
    for path in (LIB, msa.CHECKED_LIB_PATH):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                             check=True).stdout
        exported = set(re.findall(r"\bT (msa_[a-z0-9_]+)$", out, flags=re.M))
        missing = set(declared_functions()) - exported
        assert not missing, (path, missing)
    for f in declared_functions():
        assert hasattr(msa.lib, f)


def test_checked_library_and_its_diagnostics(msa):
    """libmsa.so counts nothing (MSA_ERR_UNSUPPORTED); libmsa_checked.so is the same library
    with the kernels' checks; NULL pointers are rejected before any GPU call in both."""
    c, s = ctypes.c_uint32(7), ctypes.c_uint32(7)
    assert msa.lib.msa_debug_checks(ctypes.byref(c), ctypes.byref(s)) == msa.MSA_ERR_UNSUPPORTED
    assert (c.value, s.value) == (0, 0)
    assert msa.lib.msa_debug_checks(None, ctypes.byref(s)) == msa.MSA_ERR_INVALID_ARG
    try:
        msa.use_library(True)
        assert "checked" in msa.msa_version()
        assert msa.lib.msa_debug_checks(ctypes.byref(c), None) == msa.MSA_ERR_INVALID_ARG
        assert msa.lib.msa_block_topk(None, None, 16, None, None) == msa.MSA_ERR_INVALID_ARG
    finally:
        msa.use_library(False)
    assert "checked" not in msa.msa_version()


def test_constants_and_version(msa):
    assert msa.msa_page_bytes(0) == 4 * 9216 == msa.msa_page_bytes(1)
    assert msa.msa_page_bytes(2) == 9216 and msa.msa_page_bytes(7) == 0
    assert "gfx950" in msa.msa_version()
    # 72 B per 128-element vector: 4.5 bits per element
    assert 9216 / 128 == 72 and 72 * 8 / 128 == 4.5


def _cache(k=1, v=1, ik=1, pages=4):
    import block_sparse_attention_nvfp4_amd as m
    return m._Cache(k, v, ik, pages)


def _batch(bt=1, cl=1, b=1, mb=1, q=1):
    import block_sparse_attention_nvfp4_amd as m
    return m._Batch(bt, cl, b, mb, q)


def test_invalid_arguments_return_codes_without_launch(msa):
    L = msa.lib
    by = ctypes.byref
    # insert
    assert L.msa_kv_insert_nvfp4(None, 1, 1, 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert_nvfp4(by(_cache()), None, 1, 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert_nvfp4(by(_cache()), 1, None, None, None, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert_nvfp4(by(_cache()), 1, 1, 1, 1, -1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert_nvfp4(by(_cache(pages=0)), 1, 1, 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_kv_insert_nvfp4(by(_cache(k=None)), 1, 1, None, None, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert "NULL" in msa.msa_last_error()
    assert L.msa_kv_insert_nvfp4(by(_cache()), 1, 1, 1, 1, 0, None) == msa.MSA_OK  # n = 0: no-op
    # indexer
    assert L.msa_indexer_score(by(_cache(ik=None)), by(_batch()), 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_indexer_score(by(_cache()), by(_batch(q=0)), 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_indexer_score(by(_cache()), by(_batch(bt=None)), 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_indexer_score(by(_cache()), by(_batch()), None, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_indexer_score(by(_cache()), by(_batch(b=70000)), 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    # indexer with a reduction choice
    ix = L.msa_indexer_score_ex
    assert ix(by(_cache()), by(_batch()), 1, 2, 1, None) == msa.MSA_ERR_UNSUPPORTED
    assert ix(by(_cache()), by(_batch()), None, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert ix(by(_cache(ik=None)), by(_batch()), 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert ix(by(_cache()), by(_batch(q=0)), 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    sp = L.msa_indexer_score_shared_prefix
    assert sp(by(_cache()), by(_batch(mb=4)), 1, -1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert sp(by(_cache()), by(_batch(mb=4)), 1, 5, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert sp(by(_cache()), by(_batch(mb=4)), None, 2, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert sp(by(_cache(ik=None)), by(_batch(mb=4)), 1, 2, 1, None) == msa.MSA_ERR_INVALID_ARG
    # the indexer over a shard (args: cache shard begin stride total q_idx scores stream)
    sh = L.msa_indexer_score_shard
    for bad in ((-1, 1, 8), (0, 0, 8), (0, 1, 0), (5, 1, 8), (1, 3, 8), (0, 1, 1 << 30)):
        assert sh(by(_cache()), by(_batch(mb=4)), *bad, 1, 1, None) == msa.MSA_ERR_INVALID_ARG, bad
    assert sh(by(_cache()), by(_batch(mb=4)), 0, 1, 8, None, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert sh(by(_cache()), by(_batch(mb=4)), 0, 1, 8, 1, None, None) == msa.MSA_ERR_INVALID_ARG
    assert sh(by(_cache(ik=None)), by(_batch(mb=4)), 0, 1, 8, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert sh(by(_cache()), by(_batch(mb=4, q=0)), 0, 1, 8, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert "total_blocks" in msa.msa_last_error() or "q_len" in msa.msa_last_error()
    # top-k
    assert L.msa_block_topk(1, by(_batch()), 8, 1, None) == msa.MSA_ERR_UNSUPPORTED
    assert "topk" in msa.msa_last_error()
    assert L.msa_block_topk(None, by(_batch()), 16, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_block_topk(1, by(_batch(mb=0)), 16, 1, None) == msa.MSA_ERR_INVALID_ARG
    # attention over rows of 1..64 ids (args: cache batch q ids topk scale out ws ws_bytes stream)
    at = L.msa_sparse_attn_decode_topk
    for bad in (0, 65, -3):
        assert at(by(_cache()), by(_batch()), 1, 1, bad, 0.1, 1, None, 0, None) == msa.MSA_ERR_UNSUPPORTED
    assert "topk" in msa.msa_last_error()
    assert at(by(_cache()), by(_batch()), None, 1, 16, 0.1, 1, None, 0, None) == msa.MSA_ERR_INVALID_ARG
    assert at(by(_cache()), by(_batch()), 1, None, 16, 0.1, 1, None, 0, None) == msa.MSA_ERR_INVALID_ARG
    assert at(by(_cache(k=None)), by(_batch()), 1, 1, 16, 0.1, 1, None, 0, None) == msa.MSA_ERR_INVALID_ARG
    assert at(by(_cache()), by(_batch(q=0)), 1, 1, 16, 0.1, 1, None, 0, None) == msa.MSA_ERR_INVALID_ARG
    # selection with the window knobs (args: scores batch topk init local ids stream)
    win = L.msa_block_topk_window
    assert win(1, by(_batch(mb=8)), 0, 0, 1, 1, None) == msa.MSA_ERR_UNSUPPORTED
    assert win(1, by(_batch(mb=8)), 65, 0, 1, 1, None) == msa.MSA_ERR_UNSUPPORTED
    assert win(1, by(_batch(mb=5000)), 16, 0, 1, 1, None) == msa.MSA_ERR_UNSUPPORTED
    for init, local in ((-1, 1), (0, -1), (10, 7)):
        assert win(1, by(_batch(mb=8)), 16, init, local, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert win(None, by(_batch(mb=8)), 16, 0, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert win(1, by(_batch(mb=8)), 16, 0, 1, None, None) == msa.MSA_ERR_INVALID_ARG
    # shard-local lists and their merge (args: scores ld begin stride n_cols batch topk ids keys)
    loc = L.msa_block_topk_local
    mb8 = by(_batch(mb=8))
    assert loc(1, 4, 0, 1, 4, mb8, 8, 1, 1, None) == msa.MSA_ERR_UNSUPPORTED
    for bad in ([None, 4, 0, 1, 4], [1, 3, 0, 1, 4], [1, 4, 0, 1, 0], [1, 4, -1, 1, 4],
                [1, 4, 0, 0, 4], [1, 4, 5, 1, 4], [1, 4, 1, 3, 4], [1, 5000, 0, 1, 4097]):
        assert loc(*bad, mb8, 16, 1, 1, None) == msa.MSA_ERR_INVALID_ARG, bad
    assert loc(1, 4, 0, 1, 4, mb8, 16, None, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert loc(1, 4, 0, 1, 4, mb8, 16, 1, None, None) == msa.MSA_ERR_INVALID_ARG
    assert loc(1, 4, 0, 1, 4, by(_batch(cl=None, mb=8)), 16, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    mrg = L.msa_block_topk_merge
    assert mrg(1, 1, 2, mb8, 8, 1, None) == msa.MSA_ERR_UNSUPPORTED
    for n_shards in (0, 17):
        assert mrg(1, 1, n_shards, mb8, 16, 1, None) == msa.MSA_ERR_INVALID_ARG
    for i in range(3):
        a = [1, 1, 1]
        a[i] = None
        assert mrg(a[0], a[1], 2, mb8, 16, a[2], None) == msa.MSA_ERR_INVALID_ARG, i
    assert mrg(1, 1, 2, by(_batch(q=0)), 16, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert mrg(1, 1, 2, None, 16, 1, None) == msa.MSA_ERR_INVALID_ARG
    # attention
    small = by(_batch(b=1, q=1))
    need = L.msa_sparse_attn_workspace_bytes(small)
    assert need > 0
    assert L.msa_sparse_attn_decode(by(_cache()), small, 1, 1, 0.1, 1, None, 0, None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_sparse_attn_decode(by(_cache()), small, 1, 1, 0.1, 1, 256, need - 1, None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_sparse_attn_decode(by(_cache()), small, 1, 1, 0.1, 1, 257, need, None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_sparse_attn_decode(by(_cache(v=None)), small, 1, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_INVALID_ARG
    assert L.msa_sparse_attn_decode(by(_cache()), small, None, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_INVALID_ARG
    # large batches need no workspace (one workgroup per row group covers the chip)
    assert L.msa_sparse_attn_workspace_bytes(by(_batch(b=256, q=1))) == 0
    # attention over a shared prefix (args: cache batch q ids prefix scale out ws bytes stream)
    spa = L.msa_sparse_attn_decode_shared_prefix
    spn = L.msa_sparse_attn_shared_prefix_workspace_bytes(by(_batch(b=2, q=3, mb=8)))
    assert spn == 2 * 3 * 4 * 16 * 4224
    mb8q3 = by(_batch(b=2, q=3, mb=8))
    for bad_prefix in (-1, 9):
        assert spa(by(_cache()), mb8q3, 1, 1, bad_prefix, 0.1, 1, 256, spn, None) == msa.MSA_ERR_INVALID_ARG
    assert spa(by(_cache()), mb8q3, None, 1, 2, 0.1, 1, 256, spn, None) == msa.MSA_ERR_INVALID_ARG
    assert spa(by(_cache()), mb8q3, 1, None, 2, 0.1, 1, 256, spn, None) == msa.MSA_ERR_INVALID_ARG
    assert spa(by(_cache()), mb8q3, 1, 1, 2, 0.1, None, 256, spn, None) == msa.MSA_ERR_INVALID_ARG
    assert spa(by(_cache(v=None)), mb8q3, 1, 1, 2, 0.1, 1, 256, spn, None) == msa.MSA_ERR_INVALID_ARG
    assert spa(by(_cache()), mb8q3, 1, 1, 2, 0.1, 1, None, 0, None) == msa.MSA_ERR_WORKSPACE
    assert spa(by(_cache()), mb8q3, 1, 1, 2, 0.1, 1, 256, spn - 1, None) == msa.MSA_ERR_WORKSPACE
    assert spa(by(_cache()), mb8q3, 1, 1, 2, 0.1, 1, 257, spn, None) == msa.MSA_ERR_WORKSPACE
    big = by(_batch(b=257, q=4, mb=8))  # 1,028 rows
    assert spa(by(_cache()), big, 1, 1, 2, 0.1, 1, 256, 1 << 40, None) == msa.MSA_ERR_UNSUPPORTED
    # selection + attention in one launch: the checks of both calls
    sel = L.msa_select_attn_decode
    assert sel(by(_cache()), small, 1, 8, 1, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_UNSUPPORTED
    assert sel(by(_cache()), small, None, 16, 1, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_INVALID_ARG
    assert sel(by(_cache()), small, 1, 16, None, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_INVALID_ARG
    assert sel(by(_cache(k=None)), small, 1, 16, 1, 1, 0.1, 1, 256, need, None) == msa.MSA_ERR_INVALID_ARG
    assert sel(by(_cache()), small, 1, 16, 1, 1, 0.1, 1, None, 0, None) == msa.MSA_ERR_WORKSPACE
    assert sel(by(_cache()), small, 1, 16, 1, 1, 0.1, 1, 257, need, None) == msa.MSA_ERR_WORKSPACE
    # the whole step: the checks of insert, indexer and selection + attention
    st = L.msa_decode_step
    args = [1, 1, 1, 1, 1, 16, 0.1, 1, 1, 1, 256, need, None]  # k v ik q_idx q topk scale scores ids out ws bytes stream
    def call(cache=None, batch=small, **over):
        a = list(args)
        for i, val in over.items():
            a[int(i[1:])] = val
        return st(by(cache or _cache()), batch, *a)
    assert call(a5=8) == msa.MSA_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 4, 7, 8, 9):
        assert call(**{f"a{i}": None}) == msa.MSA_ERR_INVALID_ARG, i
    assert call(cache=_cache(ik=None)) == msa.MSA_ERR_INVALID_ARG
    assert call(cache=_cache(v=None)) == msa.MSA_ERR_INVALID_ARG
    assert call(batch=by(_batch(q=0))) == msa.MSA_ERR_INVALID_ARG
    assert call(a10=None, a11=0) == msa.MSA_ERR_WORKSPACE
    assert call(a10=257) == msa.MSA_ERR_WORKSPACE
    # the step with the window knobs: k v ik q_idx q topk init local scale scores ids out ws bytes
    sw = L.msa_decode_step_window
    wargs = [1, 1, 1, 1, 1, 64, 1, 2, 0.1, 1, 1, 1, 256, need, None]
    def wcall(cache=None, batch=small, **over):
        a = list(wargs)
        for i, val in over.items():
            a[int(i[1:])] = val
        return sw(by(cache or _cache()), batch, *a)
    for bad in (0, 65):
        assert wcall(a5=bad) == msa.MSA_ERR_UNSUPPORTED
    assert "topk" in msa.msa_last_error()
    for init, local in ((-1, 1), (0, -1), (40, 30)):
        assert wcall(a6=init, a7=local) == msa.MSA_ERR_INVALID_ARG, (init, local)
    assert wcall(batch=by(_batch(mb=5000))) == msa.MSA_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 4, 9, 10, 11):
        assert wcall(**{f"a{i}": None}) == msa.MSA_ERR_INVALID_ARG, i
    assert wcall(cache=_cache(ik=None)) == msa.MSA_ERR_INVALID_ARG
    assert wcall(a12=None, a13=0) == msa.MSA_ERR_WORKSPACE
    ii = L.msa_insert_indexer_score
    for i in range(5):
        a = [1] * 5
        a[i] = None
        assert ii(by(_cache()), small, *a, None) == msa.MSA_ERR_INVALID_ARG, i
    assert ii(by(_cache(k=None)), small, 1, 1, 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG
    assert ii(by(_cache()), by(_batch(mb=0)), 1, 1, 1, 1, 1, None) == msa.MSA_ERR_INVALID_ARG


def test_stream_read_probe_rejects_bad_arguments(msa):
    """The measurement probe of include/msa_probe.h checks its pointers and alignment on the host
    and launches nothing on an error (no GPU here)."""
    L = msa.lib
    assert L.msa_probe_sink_words() >= 256
    assert L.msa_probe_stream_read(None, 1024, 16, None) == -1
    assert L.msa_probe_stream_read(16, 1024, None, None) == -1
    assert L.msa_probe_stream_read(16, 1000, 16, None) == -1   # not a multiple of 16 bytes
    assert L.msa_probe_stream_read(8, 1024, 16, None) == -1    # misaligned buffer
    assert L.msa_probe_stream_read(16, 0, 16, None) == 0       # nothing to read
