"""Host-only checks of the C ABI: the library loads without a GPU, exports
every function declared in include/mla.h, and rejects bad arguments before
launching anything (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

api = pytest.importorskip("mla_latent_kv_24_amd.api", reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = api.raw()
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strings():
    lib = api.raw()
    declared = int(re.search(r"#define MLA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.mla_abi_version() == declared
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(3) == b"MLA_ERR_WORKSPACE_TOO_SMALL"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _status(fn, *args):
    return fn(*args)


def test_dims_validation():
    lib = api.raw()
    d = api.dims(16)
    bad = api.dims(16, d_c=256)
    assert lib.mla_append_kv(None, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.mla_append_kv(ctypes.byref(bad), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    odd = api.dims(16, d_hR=63)
    assert lib.mla_append_kv(ctypes.byref(odd), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.mla_append_kv(ctypes.byref(d), 7, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1  # dtype
    zero_heads = api.dims(0)
    assert lib.mla_absorb_q(ctypes.byref(zero_heads), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    nan_base = api.dims(16, rope_base=float("nan"))
    assert lib.mla_append_kv(ctypes.byref(nan_base), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert b"rope_base" in lib.mla_last_error()
    for kw, word in ((dict(yarn_factor=float("nan")), b"yarn_factor"), (dict(yarn_factor=-2.0), b"yarn_factor"),
                     (dict(yarn_factor=40.0, yarn_orig_ctx=0.0), b"yarn_orig_ctx"),
                     (dict(yarn_factor=40.0, yarn_alpha=32.0, yarn_beta=1.0), b"yarn_alpha"),
                     (dict(yarn_factor=40.0, yarn_alpha=0.0), b"yarn_alpha")):
        y = api.dims(16, **kw)
        assert lib.mla_append_kv(ctypes.byref(y), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1, kw
        assert word in lib.mla_last_error(), kw
    # a factor of 1 (or 0) is the plain RoPE: the YaRN fields are not looked at
    off = api.dims(16, yarn_factor=1.0, yarn_orig_ctx=0.0, yarn_alpha=5.0, yarn_beta=1.0)
    assert lib.mla_append_kv(ctypes.byref(off), 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) != 1 or \
        b"yarn" not in lib.mla_last_error()


def test_append_absorb_validation():
    """mla_append_absorb checks what mla_append_kv and mla_absorb_q check; an empty
    half may pass NULL pointers, a non-empty one may not."""
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    f = lib.mla_append_absorb
    assert f(d, 1, 0, None, None, None, None, None, 0, None, None, None, None, None, None, None) == 0  # both empty
    assert f(d, 1, -1, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert f(d, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert f(d, 1, 2, None, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert f(d, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None, None, None) == 1  # q_lat NULL
    assert f(d, 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1  # lo with f32
    assert f(d, 7, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1  # dtype
    assert f(None, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1


def test_null_and_size_validation():
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    assert lib.mla_append_kv(d, 1, 0, None, None, None, None, None, None) == 0      # n_tok = 0: no-op
    assert lib.mla_append_kv(d, 1, -1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.mla_append_kv(d, 1, 4, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.mla_absorb_q(d, 1, 2, FAKE, None, FAKE, FAKE, FAKE, None, None) == 1
    # decode partials: batch, lengths, stride, splits
    args = lambda B, st, L, S: (d, 1, B, FAKE, None, FAKE, st, FAKE, L, S, FAKE, FAKE, None)
    assert lib.mla_decode_partials(*args(0, 100, 10, 1)) == 1
    assert lib.mla_decode_partials(*args(2, 100, 0, 1)) == 1
    assert lib.mla_decode_partials(*args(2, 9, 10, 1)) == 1      # stride < max_seq_len
    assert lib.mla_decode_partials(*args(2, 100, 10, 0)) == 1
    assert lib.mla_decode_partials(*args(2, 100, 10, 70000)) == 1
    assert lib.mla_combine_project(d, 1, 0, 1, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.mla_combine_project(d, 1, 4, 1, FAKE, FAKE, None, FAKE, None, None) == 1


def test_workspace_validation():
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    need = lib.mla_decode_workspace_bytes(d, 1, 64, 8192)
    S = lib.mla_decode_num_splits(d, 1, 64, 8192)
    assert need >= 64 * S * 128 * 512 * 4
    st = lib.mla_decode(d, 1, 64, FAKE, None, FAKE, 8192, FAKE, 8192, FAKE, FAKE, None, FAKE, need - 1, None)
    assert st == 3
    assert b"workspace" in lib.mla_last_error()
    pneed = lib.mla_prefill_workspace_bytes(d, 1, 1, 4096, 4096)
    assert pneed >= 4096 * 128 * 512 * 4
    assert lib.mla_prefill(d, 1, 1, 4096, FAKE, None, FAKE, 8191, FAKE, 4096, FAKE, FAKE, FAKE, pneed, None) == 1
    assert lib.mla_prefill(d, 1, 1, 4096, FAKE, None, FAKE, 8192, FAKE, 4096, FAKE, FAKE, FAKE, pneed - 1, None) == 3


def test_split_plan_covers_every_row():
    for L in (1, 31, 32, 33, 4096, 8192, 32768, 131072):
        for S in (1, 2, 3, 7, 64):
            R = api.split_rows(L, S)
            assert R % 32 == 0 and R * S >= L and (R - 32) * S < L + 32 * S
    d = api.dims(128)
    assert api.num_splits(d, api.BF16, 64, 8192) == 4          # 64 x 4 = 256 workgroups
    assert api.num_splits(d, api.BF16, 4, 131072) == 64
    assert api.num_splits(d, api.BF16, 4096, 8192) == 1          # 16 rounds of queries: no cap
    assert api.num_splits(api.dims(16), api.BF16, 1, 100) == 1
    assert api.num_splits(api.dims(16), api.BF16, 32, 4096) == 8   # one round of 256
    assert api.num_splits(api.dims(16), api.BF16, 128, 32768) == 10  # ragged: 3,328-row cap
    for B, L in ((1, 100), (3, 5000), (64, 8192), (128, 32768), (4, 131072), (4096, 8192)):
        S = api.num_splits(d, api.BF16, B, L)
        assert api.split_rows(L, S) <= 3328 or B >= 1024


def test_paged_validation():
    """Paged entry points reject bad descriptors on the host (nothing launches)."""
    lib = api.raw()
    d = ctypes.byref(api.dims(128))

    def pc(page_rows=64, max_pages=4, num_pages=10, pool=FAKE, table=FAKE):
        return api.PagedCache(pool, table, num_pages, page_rows, max_pages)

    def dec(c, max_len=200):
        return lib.mla_decode_paged(d, 1, 2, FAKE, None, ctypes.byref(c) if c is not None else None, FAKE, max_len,
                                    FAKE, FAKE, None, FAKE, 1 << 30, None)

    assert dec(None) == 1
    for bad in (pc(page_rows=48), pc(page_rows=16), pc(page_rows=1 << 17), pc(max_pages=0), pc(num_pages=0),
                pc(num_pages=1 << 31), pc(pool=None), pc(table=None)):
        assert dec(bad) == 1
    assert dec(pc(page_rows=64, max_pages=3), max_len=193) == 1      # 193 rows need 4 pages of 64
    assert b"max_pages" in lib.mla_last_error()
    assert lib.mla_decode_partials_paged(d, 1, 2, FAKE, None, ctypes.byref(pc()), FAKE, 200, 0, FAKE, FAKE, None) == 1
    assert lib.mla_prefill_paged(d, 1, 1, 100, FAKE, None, ctypes.byref(pc(page_rows=32, max_pages=4)), FAKE, 29,
                                 FAKE, FAKE, FAKE, 1 << 30, None) == 1   # 29 + 100 > 128
    assert lib.mla_prefill_unabsorbed_paged(ctypes.byref(api.dims(12)), 1, 1, 8, FAKE, FAKE, ctypes.byref(pc()),
                                            FAKE, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2   # n_h % 8
    # a workspace too small is still caught after the descriptor passes
    need = lib.mla_decode_workspace_bytes(d, 1, 2, 200)
    assert lib.mla_decode_paged(d, 1, 2, FAKE, None, ctypes.byref(pc()), FAKE, 200, FAKE, FAKE, None, FAKE,
                                need - 1, None) == 3


def test_paged_block_table_recipe():
    """The seeded block table hands every sequence distinct pages of the pool."""
    from mla_latent_kv_24_amd import workloads as W
    lens = [1, 31, 32, 33, 700, 4096]
    for P in (32, 64, 256):
        table, num_pages = W.paged_block_table(lens, P, seed=5, spare_pages=7)
        used = []
        for b, L in enumerate(lens):
            n = -(-L // P)
            assert np.all(table[b, :n] >= 0) and np.all(table[b, :n] < num_pages)
            assert np.all(table[b, n:] == -1)
            used.extend(table[b, :n].tolist())
        assert len(set(used)) == len(used) == num_pages - 7
        rows = W.paged_rows(table, P, np.repeat(np.arange(len(lens)), lens),
                            np.concatenate([np.arange(L) for L in lens]))
        assert len(np.unique(rows)) == sum(lens) and rows.max() < num_pages * P


def test_append_kv_from_hidden_validation():
    lib = api.raw()
    d = ctypes.byref(api.dims(16))
    need = lib.mla_append_kv_from_hidden_workspace_bytes(d, 1, 64, 5120)
    assert need >= 64 * 576 * 4

    def call(n_tok=64, dm=5120, eps=1e-6, h=FAKE, ws=need):
        return lib.mla_append_kv_from_hidden(d, 1, n_tok, dm, h, FAKE, FAKE, None, eps, FAKE, FAKE, FAKE, FAKE, ws,
                                             None)

    assert lib.mla_append_kv_from_hidden(d, 1, 0, 5120, None, None, None, None, 1e-6, None, None, None, None, 0,
                                         None) == 0          # n_tok = 0: no-op
    assert call(n_tok=-1) == 1
    assert call(n_tok=70000) == 1
    assert call(dm=0) == 1
    assert call(eps=float("nan")) == 1
    assert call(eps=-1.0) == 1
    assert call(h=None) == 1
    assert call(ws=need - 1) == 3


def test_projection_entry_points_validation():
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    need = lib.mla_absorb_q_from_hidden_workspace_bytes(d, 64, 5120, 1536)
    assert need >= 64 * (1536 + 128 * 192) * 2

    def q(n_q=64, dm=5120, dcq=1536, eps=1e-6, h=FAKE, ws=need):
        return lib.mla_absorb_q_from_hidden(d, n_q, dm, dcq, h, FAKE, None, eps, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                            FAKE, ws, None)

    assert q(n_q=-1) == 1 and q(dcq=5000) == 1 and q(eps=float("inf")) == 1 and q(h=None) == 1
    assert q(ws=need - 1) == 3
    oneed = lib.mla_output_projection_workspace_bytes(d, 64, 5120)
    assert oneed >= 64 * 128 * 128 * 2
    assert lib.mla_output_projection(d, 64, 0, FAKE, FAKE, FAKE, FAKE, oneed, None) == 1
    assert lib.mla_output_projection(d, 64, 5120, FAKE, None, FAKE, FAKE, oneed, None) == 1
    assert lib.mla_output_projection(d, 64, 5120, FAKE, FAKE, FAKE, FAKE, oneed - 1, None) == 3


def test_fp8_entry_points_validation():
    """The FP8 cache's entry points reject bad descriptors and sizes before any
    device work (no GPU needed: every pointer here is fake)."""
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    good = api.FP8Cache(FAKE, FAKE, FAKE)
    no_scale = api.FP8Cache(FAKE, FAKE, None)
    for cache, word in ((None, b"descriptor"), (no_scale, b"NULL array")):
        c = ctypes.byref(cache) if cache is not None else None
        assert lib.mla_append_kv_fp8(d, 4, FAKE, FAKE, FAKE, FAKE, c, None) == 1
        assert word in lib.mla_last_error()
        assert lib.mla_decode_partials_fp8(d, 2, FAKE, None, c, 100, FAKE, 100, 1, FAKE, FAKE, None) == 1
        assert lib.mla_prefill_fp8(d, 1, 8, FAKE, None, c, 100, FAKE, 10, FAKE, FAKE, FAKE, 1 << 30, None) == 1
        assert word in lib.mla_last_error()
    g = ctypes.byref(good)
    assert lib.mla_append_kv_fp8(d, 0, None, None, None, None, None, None) == 0          # no-op
    assert lib.mla_append_kv_fp8(d, -1, FAKE, FAKE, FAKE, FAKE, g, None) == 1
    assert lib.mla_decode_partials_fp8(d, 2, FAKE, None, g, 50, FAKE, 100, 1, FAKE, FAKE, None) == 1   # stride < max len
    # prefill: prefix + chunk beyond the stride, empty chunk, workspace too small
    assert lib.mla_prefill_fp8(d, 1, 8, FAKE, None, g, 100, FAKE, 95, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert b"cache_seq_stride" in lib.mla_last_error()
    assert lib.mla_prefill_fp8(d, 1, 0, FAKE, None, g, 100, FAKE, 10, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.mla_prefill_fp8(d, 1, 8, FAKE, None, g, 100, FAKE, 10, FAKE, FAKE, FAKE, 16, None) == 3
    f32 = ctypes.byref(api.dims(128, d_hR=32))
    assert lib.mla_prefill_fp8(f32, 1, 8, FAKE, None, g, 100, FAKE, 10, FAKE, FAKE, FAKE, 1 << 30, None) == 2


def test_lo_plane_rules():
    """The absorbed queries' lo plane: bf16 only (rejected with MLA_F32 before
    any launch), and the attended length below which the attention reads it."""
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    assert lib.mla_absorb_q(d, 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert b"q_lat_lo" in lib.mla_last_error()
    assert lib.mla_decode_partials(d, 0, 2, FAKE, FAKE, FAKE, 100, FAKE, 10, 1, FAKE, FAKE, None) == 1
    assert lib.mla_decode(d, 0, 2, FAKE, FAKE, FAKE, 100, FAKE, 10, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.mla_prefill(d, 0, 1, 8, FAKE, FAKE, FAKE, 100, FAKE, 10, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    all_rows = 2 ** 31 - 1
    assert api.precise_rows(api.dims(128), api.BF16) == 4096
    assert api.precise_rows(api.dims(64), api.BF16) == 4096
    assert api.precise_rows(api.dims(32), api.BF16) == 4096
    assert api.precise_rows(api.dims(16), api.BF16) == all_rows
    assert api.precise_rows(api.dims(8), api.BF16) == all_rows          # generic kernels: always hi + lo
    assert api.precise_rows(api.dims(128, yarn_factor=40.0), api.BF16) == all_rows
    assert api.precise_rows(api.dims(128), api.F32) == 0
    assert api.precise_rows(api.dims(128, d_c=256), api.BF16) == 0      # bad dims


def test_split_plan_of_the_precise_path():
    """When every query takes the 16-head-group path, each (query, split) is
    n_h / 16 workgroups and the plan counts them."""
    d = api.dims(128)
    assert api.num_splits(d, api.BF16, 64, 8192) == 4     # wide kernel: 64 x 4 workgroups
    assert api.num_splits(d, api.BF16, 64, 2048) == 1     # grouped: 64 x 1 x 8 = 512 workgroups
    assert api.num_splits(d, api.BF16, 8, 3000) == 4      # grouped: 8 x 4 x 8 = 256
    y = api.dims(128, yarn_factor=40.0)
    assert api.num_splits(y, api.BF16, 64, 8192) == 3     # grouped; the 3,328-row cap sets it
    assert api.num_splits(y, api.BF16, 4, 131072) == 40   # 131,072 rows / 3,328


def test_noalloc_decode_validates_before_touching_the_device():
    """mla_decode_noalloc checks every argument, and that the plan's partials
    fit the library's scratch array, before any device call (none here)."""
    lib = api.raw()
    d = ctypes.byref(api.dims(128))
    cap = 128 << 20
    assert lib.mla_decode_workspace_bytes(d, 1, 64, 8192) <= cap          # the V2 decode step fits
    assert lib.mla_decode_workspace_bytes(d, 1, 1024, 8192) > cap
    call = lambda B, L, q=FAKE, lo=None, dt=1, stride=8192: lib.mla_decode_noalloc(
        d, dt, B, q, lo, FAKE, stride, FAKE, L, FAKE, FAKE, None, None)
    assert call(1024, 8192) == 3 and b"scratch" in lib.mla_last_error()
    assert call(4, 8192, q=None) == 1
    assert call(0, 8192) == 1 and call(4, 0) == 1
    assert call(4, 8192, stride=100) == 1
    assert call(4, 8192, lo=FAKE, dt=0) == 1 and b"q_lat_lo" in lib.mla_last_error()
