"""Device-side setup and one decode/prefill step over the C ABI.

Plumbing only: torch allocates device memory and supplies the stream; every
computation is a call into the HIP library (api.py).
"""
from __future__ import annotations

import numpy as np
import torch

from . import api
from .workloads import D_C, D_R, ROW, DecodeInputs, PrefillInputs, paged_block_table, paged_rows


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array (uint16 bf16 bits or float32) -> device tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device, non_blocking=False)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class DecodeState:
    """All device buffers of one decode workload, with the cache filled by A1.

    cache rows: sequence b owns rows [b*stride, (b+1)*stride); rows at and past
    len_b hold NaN so that any read past a length shows up in the output.
    With page_rows set, the cache is a pool of pages of that many rows instead,
    handed out by a seeded block table (workloads.paged_block_table); unused
    pool rows hold NaN likewise.
    """

    def __init__(self, inp: DecodeInputs, device="cuda", out_latent=False, page_rows=None,
                 spare_pages=0, table_seed=0, fp8=False, q_lo=None):
        w = inp.w
        self.inp = inp
        self.device = device
        self.dt = w.dtype
        tdt = torch_dtype(w.dtype)
        self.d = api.dims(w.n_h, rope_base=w.rope_base, yarn_factor=w.yarn_factor)
        self.batch, self.stride = w.batch, inp.stride
        lens = inp.seq_lens.astype(np.int64)
        self.max_len = int(lens.max())
        self.total_rows = int(lens.sum())
        self.page_rows = page_rows
        self.fp8 = fp8
        if fp8:
            # FP8 latent cache (codes, RoPE keys, scales), rows as the contiguous layout
            assert page_rows is None and w.dtype == "bf16"
            self.cache = api.fp8_cache_empty(self.batch * self.stride, device=device)
            self.cache[0].fill_(0x7F)                   # NaN codes past every length
            self.cache[1].fill_(float("nan"))
            self.cache[2].fill_(float("nan"))
            self.block_table = None
            row_of = lambda b, j: np.asarray(b, dtype=np.int64) * self.stride + np.asarray(j, dtype=np.int64)
        elif page_rows is None:
            self.cache = torch.full((self.batch * self.stride, ROW), float("nan"), dtype=tdt, device=device)
            self.block_table = None
            row_of = lambda b, j: np.asarray(b, dtype=np.int64) * self.stride + np.asarray(j, dtype=np.int64)
        else:
            table, num_pages = paged_block_table(lens, page_rows, table_seed, spare_pages)
            self.cache = torch.full((num_pages, page_rows, ROW), float("nan"), dtype=tdt, device=device)
            self.block_table = torch.from_numpy(table).to(device)
            row_of = lambda b, j: paged_rows(table, page_rows, b, j)
        self.seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
        # fill: every valid row goes through A1 (RoPE of k_raw at its position)
        b_idx = np.repeat(np.arange(self.batch, dtype=np.int64), lens)
        j_idx = np.concatenate([np.arange(L, dtype=np.int64) for L in lens])
        self.fill_rows = torch.from_numpy(row_of(b_idx, j_idx)).to(device)
        self.fill_pos = torch.from_numpy(j_idx.astype(np.int32)).to(device)
        self.fill_c = to_device(inp.c_kv[b_idx, j_idx], w.dtype, device)
        self.fill_k = to_device(inp.k_raw[b_idx, j_idx], w.dtype, device)
        # the step's new token of each sequence = its last row
        last = lens - 1
        self.new_rows = torch.from_numpy(row_of(np.arange(self.batch), last)).to(device)
        self.new_pos = torch.from_numpy(last.astype(np.int32)).to(device)
        self.new_c = to_device(inp.c_kv[np.arange(self.batch), last], w.dtype, device)
        self.new_k = to_device(inp.k_raw[np.arange(self.batch), last], w.dtype, device)
        self.q_c = to_device(inp.q_c, w.dtype, device)
        self.q_r = to_device(inp.q_r, w.dtype, device)
        self.q_pos = self.new_pos
        self.w_uk = to_device(inp.w_uk, w.dtype, device)
        self.w_uv = to_device(inp.w_uv, w.dtype, device)
        # the lo plane of the absorbed queries only where a query reads it (q_lo=None:
        # some sequence is shorter than mla_precise_rows)
        if q_lo is None:
            q_lo = int(lens.min()) < api.precise_rows(self.d, self._api_dtype())
        self.q_lat = api.q_lat_empty(self.d, tdt, self.batch, device=device, lo=q_lo)
        self.out = torch.empty((self.batch, w.n_h, 128), dtype=torch.float32, device=device)
        self.out_latent = (torch.empty((self.batch, w.n_h, D_C), dtype=torch.float32, device=device)
                           if out_latent else None)
        self.splits = api.num_splits(self.d, self._api_dtype(), self.batch, self.max_len)
        self.z_part = torch.empty((self.batch, self.splits, w.n_h, D_C), dtype=torch.float32, device=device)
        self.lse_part = torch.empty((self.batch, self.splits, w.n_h), dtype=torch.float32, device=device)
        self.fill_cache()

    def _api_dtype(self):
        return api.BF16 if self.dt == "bf16" else api.F32

    def _append(self, c, k, pos, rows):
        if self.fp8:
            api.append_kv_fp8(self.d, c, k, pos, rows, self.cache)
        else:
            api.append_kv(self.d, c, k, pos, rows, self.cache)

    def fill_cache(self):
        self._append(self.fill_c, self.fill_k, self.fill_pos, self.fill_rows)

    # --- the steps of one decode pass (A1, A2, A3, A4+A5)
    def append_new(self):
        self._append(self.new_c, self.new_k, self.new_pos, self.new_rows)

    def absorb(self):
        api.absorb_q(self.d, self.q_c, self.q_r, self.q_pos, self.w_uk, self.q_lat)

    def append_absorb(self):
        """A1 and A2 of the step in one call (one launch on the bf16 fast path)."""
        if self.fp8:
            self.append_new()
            self.absorb()
        else:
            api.append_absorb(self.d, self.new_c, self.new_k, self.new_pos, self.new_rows, self.cache,
                              self.q_c, self.q_r, self.q_pos, self.w_uk, self.q_lat)

    def attention(self, splits=None, z_part=None, lse_part=None):
        S = self.splits if splits is None else splits
        z = self.z_part if z_part is None else z_part
        lse = self.lse_part if lse_part is None else lse_part
        if self.fp8:
            api.decode_partials_fp8(self.d, self.q_lat, self.cache, self.stride, self.seq_lens, self.max_len,
                                    S, z, lse)
        elif self.block_table is None:
            api.decode_partials(self.d, self.q_lat, self.cache, self.stride, self.seq_lens, self.max_len,
                                S, z, lse)
        else:
            api.decode_partials_paged(self.d, self.q_lat, self.cache, self.block_table, self.seq_lens,
                                      self.max_len, S, z, lse)
        return z, lse

    def combine(self, z=None, lse=None):
        api.combine_project(self.d, self.z_part if z is None else z, self.lse_part if lse is None else lse,
                            self.w_uv, self.out, self.out_latent)

    def step(self):
        """One decode step of one layer: append the new rows and absorb (one call), attend, combine."""
        self.append_absorb()
        self.attention()
        self.combine()
        return self.out

    def capture(self, fn=None, repeat=1):
        """Capture `repeat` calls of fn (default: step) into a HIP graph.

        Every launch goes to torch's current stream, which torch.cuda.graph
        makes its capture stream, so replaying the graph reruns the same kernels
        on the same buffers with no host work in between."""
        fn = fn or self.step
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(repeat):
                fn()
        return g


class PrefillState:
    """One sequence: prefix rows appended first, then the chunk's rows; chunk queries."""

    def __init__(self, inp: PrefillInputs, device="cuda", q_lo=None):
        w = inp.w
        self.inp = inp
        tdt = torch_dtype(w.dtype)
        self.d = api.dims(w.n_h, rope_base=w.rope_base, yarn_factor=w.yarn_factor)
        self.dt = w.dtype
        total = inp.prefix + inp.chunk
        self.stride = total
        self.prefix, self.chunk = inp.prefix, inp.chunk
        self.cache = torch.full((total, ROW), float("nan"), dtype=tdt, device=device)
        self.rows = torch.arange(total, dtype=torch.int64, device=device)
        self.pos = torch.arange(total, dtype=torch.int32, device=device)
        self.c_kv = to_device(inp.c_kv, w.dtype, device)
        self.k_raw = to_device(inp.k_raw, w.dtype, device)
        self.q_c = to_device(inp.q_c, w.dtype, device)
        self.q_r = to_device(inp.q_r, w.dtype, device)
        self.q_pos = torch.arange(inp.prefix, total, dtype=torch.int32, device=device)
        self.prefix_lens = torch.tensor([inp.prefix], dtype=torch.int32, device=device)
        self.w_uk = to_device(inp.w_uk, w.dtype, device)
        self.w_uv = to_device(inp.w_uv, w.dtype, device)
        dtc = api.BF16 if w.dtype == "bf16" else api.F32
        if q_lo is None:   # the first query attends prefix + 1 rows
            q_lo = inp.prefix + 1 < api.precise_rows(self.d, dtc)
        self.q_lat = api.q_lat_empty(self.d, tdt, 1, inp.chunk, device=device, lo=q_lo)
        self.out = torch.empty((1, inp.chunk, w.n_h, 128), dtype=torch.float32, device=device)
        ws = api.prefill_workspace_bytes(self.d, dtc, 1, inp.chunk, inp.prefix)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.workspace_x = None            # expanded rows of the unabsorbed form, on first use

    def append_all(self):
        api.append_kv(self.d, self.c_kv, self.k_raw, self.pos, self.rows, self.cache)

    def absorb(self):
        api.absorb_q(self.d, self.q_c, self.q_r, self.q_pos, self.w_uk, self.q_lat.view(-1, *self.q_lat.shape[2:]))

    def attend(self):
        api.prefill(self.d, self.q_lat, self.cache, self.stride, self.prefix_lens, self.prefix,
                    self.w_uv, self.out, self.workspace)

    def attend_unabsorbed(self, out=None):
        """A6 in the unabsorbed form (explicit per-head keys and values), into `out` (default self.out)."""
        if self.workspace_x is None:
            n = api.prefill_unabsorbed_workspace_bytes(self.d, api.BF16, 1, self.chunk, self.prefix)
            self.workspace_x = torch.empty(n, dtype=torch.uint8, device=self.cache.device)
        api.prefill_unabsorbed(self.d, self.q_c.view(1, *self.q_c.shape), self.q_r.view(1, *self.q_r.shape),
                               self.cache, self.stride, self.prefix_lens, self.prefix, self.w_uk, self.w_uv,
                               self.out if out is None else out, self.workspace_x)

    def step(self):
        self.append_all()
        self.absorb()
        self.attend()
        return self.out
