"""Thin Python binding of the MLA C ABI (include/mla.h).

Argument marshalling only: tensors -> device pointers, torch's current HIP
stream -> hipStream_t.  Every step runs in the HIP library; if the library is
missing this module raises on import instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

if not os.path.exists(LIB):
    raise ImportError(f"MLA HIP library not built ({LIB}); run __graft_entry__.build()")

_lib = ctypes.CDLL(LIB)

MLA_OK = 0
STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARGUMENT", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE_TOO_SMALL", 4: "MLA_ERR_HIP"}
F32, BF16 = 0, 1


class Dims(ctypes.Structure):
    _fields_ = [("d_c", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_hR", ctypes.c_int32),
                ("n_h", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("softmax_scale", ctypes.c_double), ("yarn_factor", ctypes.c_double),
                ("yarn_orig_ctx", ctypes.c_double), ("yarn_alpha", ctypes.c_double),
                ("yarn_beta", ctypes.c_double)]


def dims(n_h: int, d_c: int = 512, d_h: int = 128, d_hR: int = 64, rope_base: float = 10000.0,
         softmax_scale: float = 0.0, yarn_factor: float = 0.0, yarn_orig_ctx: float = 4096.0,
         yarn_alpha: float = 1.0, yarn_beta: float = 32.0) -> Dims:
    """Model dimensions; yarn_factor > 1 selects the long-context RoPE frequencies
    and temperature (DeepSeek-V2: 40 over a 4,096-position pretraining context)."""
    return Dims(d_c, d_h, d_hR, n_h, rope_base, softmax_scale, yarn_factor, yarn_orig_ctx, yarn_alpha, yarn_beta)


class MLAError(RuntimeError):
    def __init__(self, status: int, func: str):
        detail = _lib.mla_last_error().decode()
        super().__init__(f"{func}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER(Dims)


class PagedCache(ctypes.Structure):
    """mla_paged_cache: pool [num_pages][page_rows][d_c + d_hR], block_table [batch][max_pages] int32."""
    _fields_ = [("pool", _vp), ("block_table", _vp), ("num_pages", _i64), ("page_rows", _i32),
                ("max_pages", _i32)]


_PC = ctypes.POINTER(PagedCache)


class FP8Cache(ctypes.Structure):
    """mla_fp8_cache: codes uint8 [rows][d_c], rope bf16 [rows][d_hR], scale float [rows]."""
    _fields_ = [("codes", _vp), ("rope", _vp), ("scale", _vp)]


_FC = ctypes.POINTER(FP8Cache)
_SIGS = {
    "mla_abi_version": (_i32, []),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_append_kv": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mla_append_kv_from_hidden_workspace_bytes": (_sz, [_P, ctypes.c_int, _i32, _i32]),
    "mla_append_kv_from_hidden": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp,
                                                 ctypes.c_double, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_absorb_q_from_hidden_workspace_bytes": (_sz, [_P, _i32, _i32, _i32]),
    "mla_absorb_q_from_hidden": (ctypes.c_int, [_P, _i32, _i32, _i32, _vp, _vp, _vp, ctypes.c_double, _vp, _vp,
                                                _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_output_projection_workspace_bytes": (_sz, [_P, _i32, _i32]),
    "mla_output_projection": (ctypes.c_int, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_absorb_q": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mla_append_absorb": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp]),
    "mla_precise_rows": (_i32, [_P, ctypes.c_int]),
    "mla_decode_num_splits": (_i32, [_P, ctypes.c_int, _i32, _i32]),
    "mla_split_rows": (_i64, [_i32, _i32]),
    "mla_decode_partials": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _i32,
                                           _vp, _vp, _vp]),
    "mla_combine_project": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mla_decode_workspace_bytes": (_sz, [_P, ctypes.c_int, _i32, _i32]),
    "mla_decode": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp,
                                  _vp, _sz, _vp]),
    "mla_decode_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp,
                                          _vp]),
    "mla_prefill_workspace_bytes": (_sz, [_P, ctypes.c_int, _i32, _i32, _i32]),
    "mla_prefill_unabsorbed_workspace_bytes": (_sz, [_P, ctypes.c_int, _i32, _i32, _i32]),
    "mla_prefill_unabsorbed": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i32,
                                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_prefill": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp,
                                   _vp, _sz, _vp]),
    "mla_append_kv_fp8": (ctypes.c_int, [_P, _i32, _vp, _vp, _vp, _vp, _FC, _vp]),
    "mla_decode_partials_fp8": (ctypes.c_int, [_P, _i32, _vp, _vp, _FC, _i64, _vp, _i32, _i32, _vp, _vp, _vp]),
    "mla_decode_fp8": (ctypes.c_int, [_P, _i32, _vp, _vp, _FC, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_prefill_fp8": (ctypes.c_int, [_P, _i32, _i32, _vp, _vp, _FC, _i64, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "mla_decode_partials_paged": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _PC, _vp, _i32, _i32, _vp,
                                                 _vp, _vp]),
    "mla_decode_paged": (ctypes.c_int, [_P, ctypes.c_int, _i32, _vp, _vp, _PC, _vp, _i32, _vp, _vp, _vp, _vp,
                                        _sz, _vp]),
    "mla_prefill_paged": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _PC, _vp, _i32, _vp, _vp, _vp,
                                         _sz, _vp]),
    "mla_prefill_unabsorbed_paged": (ctypes.c_int, [_P, ctypes.c_int, _i32, _i32, _vp, _vp, _PC, _vp, _i32,
                                                    _vp, _vp, _vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def raw():
    """The ctypes handle (for tests of the C ABI itself)."""
    return _lib


def _check(status: int, func: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, func)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"storage dtype must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def append_kv(d: Dims, c_kv, k_r, pos, row, cache) -> None:
    """A1: cache[row[t]] = [c_kv[t]; RoPE(k_r[t], pos[t])]."""
    n = c_kv.shape[0]
    assert pos.dtype == torch.int32 and row.dtype == torch.int64
    _check(_lib.mla_append_kv(ctypes.byref(d), _dtype(cache), n, _ptr(c_kv), _ptr(k_r), _ptr(pos),
                              _ptr(row), _ptr(cache), _stream(cache.device)), "mla_append_kv")


def append_kv_from_hidden_workspace_bytes(d: Dims, dtype: int, n_tok: int, d_model: int) -> int:
    return _lib.mla_append_kv_from_hidden_workspace_bytes(ctypes.byref(d), dtype, n_tok, d_model)


def append_kv_from_hidden(d: Dims, h, w_dkv, w_kr, norm_weight, eps: float, pos, row, cache,
                          workspace=None) -> None:
    """A1 from hidden states: cache[row[t]] = [RMSNorm(w_dkv @ h[t]) * norm_weight;
    RoPE(w_kr @ h[t], pos[t])]; h [n_tok, d_model], w_dkv [d_c, d_model], w_kr [d_hR, d_model],
    norm_weight [d_c] or None."""
    assert pos.dtype == torch.int32 and row.dtype == torch.int64
    n, dm = h.shape
    dt = _dtype(cache)
    if workspace is None:
        need = append_kv_from_hidden_workspace_bytes(d, dt, n, dm)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=cache.device)
    _check(_lib.mla_append_kv_from_hidden(ctypes.byref(d), dt, n, dm, _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                                          _ptr(norm_weight), float(eps), _ptr(pos), _ptr(row), _ptr(cache),
                                          _ptr(workspace), workspace.numel(), _stream(cache.device)),
           "mla_append_kv_from_hidden")


class QLat:
    """Absorbed queries (A2's output, mla.h): `hi` [*lead, n_h, d_c + d_hR] in the
    storage dtype and, for bf16, an optional `lo` plane of the same shape
    (lo = bf16(v - hi)); the attention calls read lo for the queries that
    mla_precise_rows() names."""

    def __init__(self, hi: torch.Tensor, lo: torch.Tensor | None = None):
        if lo is not None:
            assert lo.shape == hi.shape and lo.dtype == hi.dtype == torch.bfloat16
        self.hi, self.lo = hi, lo

    @property
    def shape(self):
        return self.hi.shape

    @property
    def dtype(self):
        return self.hi.dtype

    @property
    def device(self):
        return self.hi.device

    def view(self, *shape) -> "QLat":
        return QLat(self.hi.view(*shape), None if self.lo is None else self.lo.view(*shape))

    def __getitem__(self, idx) -> "QLat":
        return QLat(self.hi[idx], None if self.lo is None else self.lo[idx])


def q_lat_empty(d: Dims, storage: torch.dtype, *lead: int, device="cuda", lo: bool = True) -> QLat:
    """Absorbed query buffers [*lead, n_h, d_c + d_hR] of `storage` dtype, with the
    bf16 lo plane when `lo` (ignored for float32)."""
    if storage not in (torch.bfloat16, torch.float32):
        raise TypeError(f"storage dtype must be bfloat16 or float32, got {storage}")
    shape = (*lead, d.n_h, d.d_c + d.d_hR)
    hi = torch.empty(shape, dtype=storage, device=device)
    return QLat(hi, torch.empty_like(hi) if (lo and storage == torch.bfloat16) else None)


def q_lat_value(q_lat) -> torch.Tensor:
    """fp32 value of absorbed queries (hi + lo where the lo plane exists)."""
    if isinstance(q_lat, QLat):
        v = q_lat.hi.float()
        return v + q_lat.lo.float() if q_lat.lo is not None else v
    return q_lat.float()


def _q(q_lat):
    """(hi, lo) device pointers of absorbed queries (a QLat or a bare hi tensor)."""
    if isinstance(q_lat, QLat):
        return _ptr(q_lat.hi), _ptr(q_lat.lo)
    return _ptr(q_lat), None


def precise_rows(d: Dims, dtype: int) -> int:
    """mla_precise_rows: queries attending fewer rows read the lo plane."""
    return _lib.mla_precise_rows(ctypes.byref(d), dtype)


def absorb_q(d: Dims, q_c, q_r, q_pos, w_uk, q_lat) -> None:
    """A2: q_lat[n, i] = [q_c[n, i] @ w_uk[i]; RoPE(q_r[n, i], q_pos[n])] (hi, and lo
    when the QLat has that plane)."""
    assert q_pos.dtype == torch.int32 and q_lat.dtype == w_uk.dtype
    hi, lo = _q(q_lat)
    _check(_lib.mla_absorb_q(ctypes.byref(d), _dtype(w_uk), q_c.shape[0], _ptr(q_c), _ptr(q_r),
                             _ptr(q_pos), _ptr(w_uk), hi, lo, _stream(q_lat.device)),
           "mla_absorb_q")


def append_absorb(d: Dims, c_kv, k_r, pos, row, cache, q_c, q_r, q_pos, w_uk, q_lat) -> None:
    """A1 + A2 of a decode step in one call: append_kv(c_kv, k_r, pos, row, cache)
    and absorb_q(q_c, q_r, q_pos, w_uk, q_lat), bit for bit (one launch on the
    bf16 fast path)."""
    assert pos.dtype == torch.int32 and row.dtype == torch.int64 and q_pos.dtype == torch.int32
    assert q_lat.dtype == w_uk.dtype == cache.dtype
    hi, lo = _q(q_lat)
    _check(_lib.mla_append_absorb(ctypes.byref(d), _dtype(cache), c_kv.shape[0], _ptr(c_kv), _ptr(k_r), _ptr(pos),
                                  _ptr(row), _ptr(cache), q_c.shape[0], _ptr(q_c), _ptr(q_r), _ptr(q_pos),
                                  _ptr(w_uk), hi, lo, _stream(cache.device)), "mla_append_absorb")


def num_splits(d: Dims, dtype: int, batch: int, max_seq_len: int) -> int:
    return _lib.mla_decode_num_splits(ctypes.byref(d), dtype, batch, max_seq_len)


def split_rows(max_seq_len: int, splits: int) -> int:
    return _lib.mla_split_rows(max_seq_len, splits)


def decode_partials(d: Dims, q_lat, cache, stride: int, seq_lens, max_seq_len: int, splits: int,
                    z_part, lse_part) -> None:
    """A3: split-KV partials (z_part [B, S, n_h, d_c] fp32, lse_part [B, S, n_h] fp32)."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == cache.dtype
    _check(_lib.mla_decode_partials(ctypes.byref(d), _dtype(cache), q_lat.shape[0], *_q(q_lat),
                                    _ptr(cache), stride, _ptr(seq_lens), max_seq_len, splits,
                                    _ptr(z_part), _ptr(lse_part), _stream(cache.device)),
           "mla_decode_partials")


def combine_project(d: Dims, z_part, lse_part, w_uv, out, out_latent=None) -> None:
    """A4 + A5: out[n, i] = w_uv[i] @ combine_s(z_part[n, s, i])."""
    n_q, S = z_part.shape[0], z_part.shape[1]
    _check(_lib.mla_combine_project(ctypes.byref(d), _dtype(w_uv), n_q, S, _ptr(z_part),
                                    _ptr(lse_part), _ptr(w_uv), _ptr(out), _ptr(out_latent),
                                    _stream(out.device)), "mla_combine_project")


def decode_workspace_bytes(d: Dims, dtype: int, batch: int, max_seq_len: int) -> int:
    return _lib.mla_decode_workspace_bytes(ctypes.byref(d), dtype, batch, max_seq_len)


def decode(d: Dims, q_lat, cache, stride: int, seq_lens, max_seq_len: int, w_uv, out,
           out_latent=None, workspace=None) -> None:
    """A3 + A4 + A5 with the automatic split plan."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == cache.dtype
    dt = _dtype(cache)
    need = decode_workspace_bytes(d, dt, q_lat.shape[0], max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=cache.device)
    _check(_lib.mla_decode(ctypes.byref(d), dt, q_lat.shape[0], *_q(q_lat), _ptr(cache), stride,
                           _ptr(seq_lens), max_seq_len, _ptr(w_uv), _ptr(out), _ptr(out_latent),
                           _ptr(workspace), workspace.numel(), _stream(cache.device)), "mla_decode")


NOALLOC_SCRATCH_BYTES = 128 << 20


def decode_noalloc(d: Dims, q_lat, cache, stride: int, seq_lens, max_seq_len: int, w_uv, out,
                   out_latent=None) -> None:
    """decode() with the split partials in the library's own device array (no
    workspace, no allocation; calls on one GPU must not overlap)."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == cache.dtype
    _check(_lib.mla_decode_noalloc(ctypes.byref(d), _dtype(cache), q_lat.shape[0], *_q(q_lat), _ptr(cache), stride,
                                   _ptr(seq_lens), max_seq_len, _ptr(w_uv), _ptr(out), _ptr(out_latent),
                                   _stream(cache.device)), "mla_decode_noalloc")


def prefill_workspace_bytes(d: Dims, dtype: int, batch: int, chunk: int, max_prefix_len: int) -> int:
    return _lib.mla_prefill_workspace_bytes(ctypes.byref(d), dtype, batch, chunk, max_prefix_len)


def prefill(d: Dims, q_lat, cache, stride: int, prefix_lens, max_prefix_len: int, w_uv, out,
            workspace=None) -> None:
    """A6: causal prefill; q_lat [B, chunk, n_h, 576] (QLat), out [B, chunk, n_h, d_h]."""
    assert prefix_lens.dtype == torch.int32 and q_lat.dtype == cache.dtype
    dt = _dtype(cache)
    B, chunk = q_lat.shape[0], q_lat.shape[1]
    need = prefill_workspace_bytes(d, dt, B, chunk, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=cache.device)
    _check(_lib.mla_prefill(ctypes.byref(d), dt, B, chunk, *_q(q_lat), _ptr(cache), stride,
                            _ptr(prefix_lens), max_prefix_len, _ptr(w_uv), _ptr(out),
                            _ptr(workspace), workspace.numel(), _stream(cache.device)),
           "mla_prefill")


def prefill_unabsorbed_workspace_bytes(d: Dims, dtype: int, batch: int, chunk: int, max_prefix_len: int) -> int:
    return _lib.mla_prefill_unabsorbed_workspace_bytes(ctypes.byref(d), dtype, batch, chunk, max_prefix_len)


def prefill_unabsorbed(d: Dims, q_c, q_r, cache, stride: int, prefix_lens, max_prefix_len: int, w_uk, w_uv,
                       out, workspace=None) -> None:
    """A6 in the unabsorbed form: q_c [B, chunk, n_h, d_h], q_r [B, chunk, n_h, d_hR] (before RoPE),
    out [B, chunk, n_h, d_h] fp32."""
    assert prefix_lens.dtype == torch.int32 and q_c.dtype == cache.dtype == q_r.dtype == w_uk.dtype
    dt = _dtype(cache)
    B, chunk = q_c.shape[0], q_c.shape[1]
    need = prefill_unabsorbed_workspace_bytes(d, dt, B, chunk, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=cache.device)
    _check(_lib.mla_prefill_unabsorbed(ctypes.byref(d), dt, B, chunk, _ptr(q_c), _ptr(q_r), _ptr(cache), stride,
                                       _ptr(prefix_lens), max_prefix_len, _ptr(w_uk), _ptr(w_uv), _ptr(out),
                                       _ptr(workspace), workspace.numel(), _stream(cache.device)),
           "mla_prefill_unabsorbed")


def paged_cache(pool, block_table) -> PagedCache:
    """Descriptor of a paged latent cache: pool [num_pages, page_rows, d_c + d_hR] (storage dtype),
    block_table [batch, max_pages] int32; row r of sequence b is pool[block_table[b, r // page_rows],
    r % page_rows].  The tensors must outlive every call that uses the descriptor."""
    assert pool.dim() == 3 and block_table.dim() == 2 and block_table.dtype == torch.int32
    return PagedCache(_ptr(pool), _ptr(block_table), pool.shape[0], pool.shape[1], block_table.shape[1])


def decode_partials_paged(d: Dims, q_lat, pool, block_table, seq_lens, max_seq_len: int, splits: int,
                          z_part, lse_part) -> None:
    """decode_partials() over a paged cache (see paged_cache)."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == pool.dtype
    pc = paged_cache(pool, block_table)
    _check(_lib.mla_decode_partials_paged(ctypes.byref(d), _dtype(pool), q_lat.shape[0], *_q(q_lat),
                                          ctypes.byref(pc), _ptr(seq_lens), max_seq_len, splits, _ptr(z_part),
                                          _ptr(lse_part), _stream(pool.device)), "mla_decode_partials_paged")


def decode_paged(d: Dims, q_lat, pool, block_table, seq_lens, max_seq_len: int, w_uv, out,
                 out_latent=None, workspace=None) -> None:
    """decode() over a paged cache (see paged_cache)."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == pool.dtype
    dt = _dtype(pool)
    need = decode_workspace_bytes(d, dt, q_lat.shape[0], max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=pool.device)
    pc = paged_cache(pool, block_table)
    _check(_lib.mla_decode_paged(ctypes.byref(d), dt, q_lat.shape[0], *_q(q_lat), ctypes.byref(pc),
                                 _ptr(seq_lens), max_seq_len, _ptr(w_uv), _ptr(out), _ptr(out_latent),
                                 _ptr(workspace), workspace.numel(), _stream(pool.device)), "mla_decode_paged")


def prefill_paged(d: Dims, q_lat, pool, block_table, prefix_lens, max_prefix_len: int, w_uv, out,
                  workspace=None) -> None:
    """prefill() over a paged cache (see paged_cache)."""
    assert prefix_lens.dtype == torch.int32 and q_lat.dtype == pool.dtype
    dt = _dtype(pool)
    B, chunk = q_lat.shape[0], q_lat.shape[1]
    need = prefill_workspace_bytes(d, dt, B, chunk, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=pool.device)
    pc = paged_cache(pool, block_table)
    _check(_lib.mla_prefill_paged(ctypes.byref(d), dt, B, chunk, *_q(q_lat), ctypes.byref(pc),
                                  _ptr(prefix_lens), max_prefix_len, _ptr(w_uv), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(pool.device)), "mla_prefill_paged")


def prefill_unabsorbed_paged(d: Dims, q_c, q_r, pool, block_table, prefix_lens, max_prefix_len: int, w_uk,
                             w_uv, out, workspace=None) -> None:
    """prefill_unabsorbed() over a paged cache (see paged_cache)."""
    assert prefix_lens.dtype == torch.int32 and q_c.dtype == pool.dtype == q_r.dtype == w_uk.dtype
    dt = _dtype(pool)
    B, chunk = q_c.shape[0], q_c.shape[1]
    need = prefill_unabsorbed_workspace_bytes(d, dt, B, chunk, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=pool.device)
    pc = paged_cache(pool, block_table)
    _check(_lib.mla_prefill_unabsorbed_paged(ctypes.byref(d), dt, B, chunk, _ptr(q_c), _ptr(q_r),
                                             ctypes.byref(pc), _ptr(prefix_lens), max_prefix_len, _ptr(w_uk),
                                             _ptr(w_uv), _ptr(out), _ptr(workspace), workspace.numel(),
                                             _stream(pool.device)), "mla_prefill_unabsorbed_paged")


def fp8_cache_empty(rows: int, d_c: int = 512, d_hR: int = 64, device="cuda"):
    """(codes, rope, scale) device tensors of an FP8 latent cache of `rows` rows."""
    return (torch.empty((rows, d_c), dtype=torch.uint8, device=device),
            torch.empty((rows, d_hR), dtype=torch.bfloat16, device=device),
            torch.empty((rows,), dtype=torch.float32, device=device))


def _fp8(cache) -> FP8Cache:
    codes, rope, scale = cache
    assert codes.dtype == torch.uint8 and rope.dtype == torch.bfloat16 and scale.dtype == torch.float32
    return FP8Cache(_ptr(codes), _ptr(rope), _ptr(scale))


def append_kv_fp8(d: Dims, c_kv, k_r, pos, row, cache) -> None:
    """A1 into the FP8 cache (codes, rope, scale): c_kv, k_r bf16."""
    assert pos.dtype == torch.int32 and row.dtype == torch.int64 and c_kv.dtype == torch.bfloat16
    fc = _fp8(cache)
    _check(_lib.mla_append_kv_fp8(ctypes.byref(d), c_kv.shape[0], _ptr(c_kv), _ptr(k_r), _ptr(pos), _ptr(row),
                                  ctypes.byref(fc), _stream(c_kv.device)), "mla_append_kv_fp8")


def decode_partials_fp8(d: Dims, q_lat, cache, stride: int, seq_lens, max_seq_len: int, splits: int,
                        z_part, lse_part) -> None:
    """A3 over the FP8 cache (bf16 absorbed queries)."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == torch.bfloat16
    fc = _fp8(cache)
    _check(_lib.mla_decode_partials_fp8(ctypes.byref(d), q_lat.shape[0], *_q(q_lat), ctypes.byref(fc), stride,
                                        _ptr(seq_lens), max_seq_len, splits, _ptr(z_part), _ptr(lse_part),
                                        _stream(q_lat.device)), "mla_decode_partials_fp8")


def decode_fp8(d: Dims, q_lat, cache, stride: int, seq_lens, max_seq_len: int, w_uv, out, out_latent=None,
               workspace=None) -> None:
    """A3 + A4 + A5 over the FP8 cache."""
    assert seq_lens.dtype == torch.int32 and q_lat.dtype == torch.bfloat16
    need = decode_workspace_bytes(d, BF16, q_lat.shape[0], max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_lat.device)
    fc = _fp8(cache)
    _check(_lib.mla_decode_fp8(ctypes.byref(d), q_lat.shape[0], *_q(q_lat), ctypes.byref(fc), stride,
                               _ptr(seq_lens), max_seq_len, _ptr(w_uv), _ptr(out), _ptr(out_latent),
                               _ptr(workspace), workspace.numel(), _stream(q_lat.device)), "mla_decode_fp8")


def absorb_q_from_hidden(d: Dims, h, w_dq, norm_weight, eps: float, w_uq, w_qr, q_pos, w_uk, q_lat,
                         workspace=None) -> None:
    """The query path into A2: c^Q = RMSNorm(w_dq @ h) * norm_weight, q^C = w_uq @ c^Q,
    q^R = w_qr @ c^Q, then absorb_q (bf16 throughout; h [n_q, d_model], w_dq [d_cq, d_model])."""
    assert q_pos.dtype == torch.int32 and h.dtype == torch.bfloat16
    n_q, d_model = h.shape
    d_cq = w_dq.shape[0]
    if workspace is None:
        need = _lib.mla_absorb_q_from_hidden_workspace_bytes(ctypes.byref(d), n_q, d_model, d_cq)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check(_lib.mla_absorb_q_from_hidden(ctypes.byref(d), n_q, d_model, d_cq, _ptr(h), _ptr(w_dq), _ptr(norm_weight),
                                         float(eps), _ptr(w_uq), _ptr(w_qr), _ptr(q_pos), _ptr(w_uk), *_q(q_lat),
                                         _ptr(workspace), workspace.numel(), _stream(h.device)),
           "mla_absorb_q_from_hidden")


def output_projection(d: Dims, o, w_o, out, workspace=None) -> None:
    """out [n_q, d_model] = W^O o for o [n_q, n_h, d_h] fp32 and w_o [d_model, n_h * d_h] bf16."""
    n_q, d_model = out.shape
    if workspace is None:
        need = _lib.mla_output_projection_workspace_bytes(ctypes.byref(d), n_q, d_model)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=out.device)
    _check(_lib.mla_output_projection(ctypes.byref(d), n_q, d_model, _ptr(o), _ptr(w_o), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(out.device)), "mla_output_projection")


def prefill_fp8(d: Dims, q_lat, cache, stride: int, prefix_lens, max_prefix_len: int, w_uv, out,
                workspace=None) -> None:
    """A6 over the FP8 cache (codes, rope, scale); q_lat [B, chunk, n_h, 576] bf16 (QLat)."""
    assert prefix_lens.dtype == torch.int32 and q_lat.dtype == torch.bfloat16
    B, chunk = q_lat.shape[0], q_lat.shape[1]
    need = prefill_workspace_bytes(d, BF16, B, chunk, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_lat.device)
    fc = _fp8(cache)
    _check(_lib.mla_prefill_fp8(ctypes.byref(d), B, chunk, *_q(q_lat), ctypes.byref(fc), stride, _ptr(prefix_lens),
                                max_prefix_len, _ptr(w_uv), _ptr(out), _ptr(workspace), workspace.numel(),
                                _stream(q_lat.device)), "mla_prefill_fp8")
