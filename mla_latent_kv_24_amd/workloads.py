"""Seeded synthetic workloads for MLA latent-KV decode and causal prefill.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic (no RoPE, no softmax, no
absorption): the CPU oracle and the HIP library both receive the arrays it
returns, so both see bit-identical inputs.

Shapes follow the DeepSeek-V2 pages:
  * the jiphyeonjeon.kr review of DeepSeek-V2 (arXiv 2405.04434v5), section 2
    (c^KV = W^DKV h, 512-d latent; query latent of 1,536), section 3 (per-head
    128-d content query/key, 64-d RoPE query per head, one 64-d RoPE key per
    token) and section 4 (60 layers, d_c = 512, d_h^R = 64);
  * the axforge.ai DeepSeek-V2-Lite model card, section 5 (hidden 2048,
    16 heads of 128, KV latent 512, RoPE dim 64, queries not compressed).

Recipe (all draws float32 from numpy's PCG64 via SeedSequence children):
  root = SeedSequence(seed); [s_len, s_cache, s_query, s_weight] = root.spawn(4)
  lengths  <- default_rng(seed) itself, drawn first (ragged workloads only:
              integers in [1, T_max]); s_len is left unused
  cache    <- s_cache.spawn(B) (sequence b: c_kv [T_b, 512] then k_raw [T_b, 64], N(0,1))
  queries  <- s_query          (h, then query weights; see query_path)
  weights  <- s_weight         (W_UK then W_UV, N(0, 1/512), stored [n_h][d_h][d_c])
Values are rounded to bfloat16 with round-to-nearest-even for bf16
workloads; fp32 workloads keep the float32 draws.  "N(0, 1/fan_in)" is read
as variance 1/fan_in (std = fan_in ** -0.5).
"""
from __future__ import annotations

import dataclasses
import numpy as np

D_C = 512      # KV latent width d_c
D_H = 128      # per-head content dim d_h
D_R = 64       # decoupled RoPE dim d_h^R
ROW = D_C + D_R  # one cached row: [c_kv ; k_R]


# --------------------------------------------------------------------------
# bfloat16 storage helpers (IEEE round-to-nearest-even on the fp32 bits)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> storage array (uint16 bf16 bits, or float32)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> the exact float64 values it holds."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16" storage; accumulation is fp32
    batch: int
    seq_len: int          # fixed length, or the maximum for ragged draws
    n_h: int
    ragged: bool = False
    query_path: str = "direct"   # "direct" | "lite" | "v2"
    hidden: int = 0
    d_cq: int = 0                # query latent width d_c' (v2 path)
    prefill_chunk: int = 0       # >0: causal prefill of this many tokens after seq_len-chunk prefix
    rope_base: float = 10000.0
    yarn_factor: float = 0.0     # >1: long-context RoPE scale over a 4,096-position pretraining context
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(D_H + D_R))


WORKLOADS = {
    # tiny fp32 decode: batch 1, T=256, 16 heads, q ~ N(0,1) directly
    "tiny_f32": Workload("tiny_f32", "f32", 1, 256, 16),
    # V2-Lite shaped decode: 32 x 4096, 16 heads, uncompressed queries from hidden 2048
    "lite_decode": Workload("lite_decode", "bf16", 32, 4096, 16, query_path="lite", hidden=2048),
    # ragged V2-Lite decode: 128 sequences, lengths uniform in [1, 32768]
    "lite_ragged": Workload("lite_ragged", "bf16", 128, 32768, 16, ragged=True,
                            query_path="lite", hidden=2048),
    # V2 shaped decode: 64 x 8192, 128 heads, query latent 1536 from hidden 5120
    "v2_decode": Workload("v2_decode", "bf16", 64, 8192, 128, query_path="v2",
                          hidden=5120, d_cq=1536),
    # V2 long context decode: 4 x 131072 (plain RoPE, base 10000)
    "v2_long": Workload("v2_long", "bf16", 4, 131072, 128, query_path="v2",
                        hidden=5120, d_cq=1536),
    # V2 causal prefill: 4096-token chunk appended to a 4096-token prefix
    "v2_prefill": Workload("v2_prefill", "bf16", 1, 8192, 128, query_path="v2",
                           hidden=5120, d_cq=1536, prefill_chunk=4096),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (small parity cases)."""
    return dataclasses.replace(w, **changes)


# --------------------------------------------------------------------------
# Drawing
# --------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def draw_lengths(w: Workload) -> np.ndarray:
    """Per-sequence lengths (int32).  Ragged: uniform integers in [1, seq_len],
    the first draw of default_rng(seed) (seed 0, 128 x [1, 32768]: sum 2,142,301,
    min 90, max 32,677)."""
    if not w.ragged:
        return np.full(w.batch, w.seq_len, dtype=np.int32)
    rng = np.random.default_rng(w.seed)
    return rng.integers(1, w.seq_len + 1, w.batch).astype(np.int32)


def draw_sequence_rows(w: Workload, b: int, n_rows: int):
    """Rows 0..n_rows-1 of sequence b: c_kv [n, 512] and pre-RoPE k_raw [n, 64] (float32)."""
    s_cache = np.random.SeedSequence(w.seed).spawn(4)[1]
    rng = np.random.default_rng(s_cache.spawn(w.batch)[b])
    c_kv = _normal(rng, (n_rows, D_C))
    k_raw = _normal(rng, (n_rows, D_R))
    return c_kv, k_raw


def _rms_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    # Input-synthesis step of the V2 query path (unit-weight RMSNorm of the
    # query latent).  It is upstream of every library call.
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True)
    return (x / np.sqrt(ms + np.float32(eps))).astype(np.float32)


def draw_queries(w: Workload, n_q: int):
    """Content and pre-RoPE queries q_c [n_q, n_h, 128], q_r [n_q, n_h, 64] (float32).

    direct: q_c, q_r ~ N(0,1).
    lite:   h ~ N(0,1) [n_q, hidden]; q_c = W^Q h, q_r = W^QR h with
            W^Q [n_h*128, hidden], W^QR [n_h*64, hidden] ~ N(0, 1/hidden).
    v2:     h ~ N(0,1) [n_q, hidden]; c^Q = RMSNorm(W^DQ h), W^DQ [d_cq, hidden]
            ~ N(0, 1/hidden); q_c = W^UQ c^Q, q_r = W^QR c^Q with
            W^UQ [n_h*128, d_cq], W^QR [n_h*64, d_cq] ~ N(0, 1/d_cq).
    """
    s_query = np.random.SeedSequence(w.seed).spawn(4)[2]
    rng = np.random.default_rng(s_query)
    if w.query_path == "direct":
        q_c = _normal(rng, (n_q, w.n_h, D_H))
        q_r = _normal(rng, (n_q, w.n_h, D_R))
        return q_c, q_r
    h = _normal(rng, (n_q, w.hidden))
    if w.query_path == "lite":
        w_q = _normal(rng, (w.n_h * D_H, w.hidden), w.hidden ** -0.5)
        w_qr = _normal(rng, (w.n_h * D_R, w.hidden), w.hidden ** -0.5)
        src = h
    elif w.query_path == "v2":
        w_dq = _normal(rng, (w.d_cq, w.hidden), w.hidden ** -0.5)
        src = _rms_normalise(h @ w_dq.T)
        w_q = _normal(rng, (w.n_h * D_H, w.d_cq), w.d_cq ** -0.5)
        w_qr = _normal(rng, (w.n_h * D_R, w.d_cq), w.d_cq ** -0.5)
    else:
        raise ValueError(w.query_path)
    q_c = (src @ w_q.T).reshape(n_q, w.n_h, D_H)
    q_r = (src @ w_qr.T).reshape(n_q, w.n_h, D_R)
    return q_c.astype(np.float32), q_r.astype(np.float32)


def draw_weights(w: Workload):
    """W_UK, W_UV as [n_h][d_h][d_c] float32 ~ N(0, 1/d_c)."""
    s_weight = np.random.SeedSequence(w.seed).spawn(4)[3]
    rng = np.random.default_rng(s_weight)
    w_uk = _normal(rng, (w.n_h, D_H, D_C), D_C ** -0.5)
    w_uv = _normal(rng, (w.n_h, D_H, D_C), D_C ** -0.5)
    return w_uk, w_uv


@dataclasses.dataclass
class DecodeInputs:
    """Storage-dtype arrays for one decode step (uint16 bf16 bits or float32).

    c_kv [B, stride, 512] and k_raw [B, stride, 64] hold rows 0..len_b-1 of
    each sequence; rows at and beyond len_b are filled with `pad` (NaN poison
    by default for bf16 and f32) so that any read past the length shows.
    q_c [B, n_h, 128], q_r [B, n_h, 64] are the queries of the token at
    position len_b - 1; w_uk, w_uv are [n_h, 128, 512].
    """
    w: Workload
    seq_lens: np.ndarray
    stride: int
    c_kv: np.ndarray
    k_raw: np.ndarray
    q_c: np.ndarray
    q_r: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray

    @property
    def q_pos(self) -> np.ndarray:
        return (self.seq_lens - 1).astype(np.int32)


def _nan_storage(dtype: str):
    return np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)


def make_decode_inputs(w: Workload, poison: bool = True, threads: int = 8) -> DecodeInputs:
    """Draw every input of one decode step of workload `w`."""
    lens = draw_lengths(w)
    stride = int(w.seq_len)
    sd = np.uint16 if w.dtype == "bf16" else np.float32
    c_kv = np.empty((w.batch, stride, D_C), dtype=sd)
    k_raw = np.empty((w.batch, stride, D_R), dtype=sd)

    def fill(b):
        n = int(lens[b])
        c, k = draw_sequence_rows(w, b, n)
        c_kv[b, :n] = to_storage(c, w.dtype)
        k_raw[b, :n] = to_storage(k, w.dtype)
        if n < stride:
            pad = _nan_storage(w.dtype) if poison else sd(0)
            c_kv[b, n:] = pad
            k_raw[b, n:] = pad

    if threads > 1 and w.batch > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(w.batch)))
    else:
        for b in range(w.batch):
            fill(b)
    q_c, q_r = draw_queries(w, w.batch)
    w_uk, w_uv = draw_weights(w)
    return DecodeInputs(w, lens, stride, c_kv, k_raw,
                        to_storage(q_c, w.dtype), to_storage(q_r, w.dtype),
                        to_storage(w_uk, w.dtype), to_storage(w_uv, w.dtype))


@dataclasses.dataclass
class PrefillInputs:
    """One sequence: rows 0..total-1 of the cache source (c_kv, k_raw), of
    which the last `chunk` rows are the new tokens, plus the chunk's queries
    q_c [chunk, n_h, 128], q_r [chunk, n_h, 64] at positions prefix..total-1."""
    w: Workload
    prefix: int
    chunk: int
    c_kv: np.ndarray
    k_raw: np.ndarray
    q_c: np.ndarray
    q_r: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray


def make_prefill_inputs(w: Workload) -> PrefillInputs:
    total = int(w.seq_len)
    chunk = int(w.prefill_chunk)
    prefix = total - chunk
    c, k = draw_sequence_rows(w, 0, total)
    q_c, q_r = draw_queries(w, chunk)
    w_uk, w_uv = draw_weights(w)
    return PrefillInputs(w, prefix, chunk, to_storage(c, w.dtype), to_storage(k, w.dtype),
                         to_storage(q_c, w.dtype), to_storage(q_r, w.dtype),
                         to_storage(w_uk, w.dtype), to_storage(w_uv, w.dtype))


def random_storage(seed, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    """Generic seeded draw N(0, std^2) rounded to the storage dtype (per-kernel test inputs)."""
    rng = np.random.default_rng(seed)
    return to_storage(_normal(rng, shape, std), dtype)


def random_ints(seed, low: int, high: int, shape) -> np.ndarray:
    """Seeded integers in [low, high) (positions, lengths, row indices of test inputs)."""
    return np.random.default_rng(seed).integers(low, high, shape)


def paged_block_table(lens, page_rows: int, seed: int = 0, spare_pages: int = 0):
    """Block table of a paged cache for sequences of the given lengths.

    Sequence b needs ceil(len_b / page_rows) pages; all pages of the batch
    (plus `spare_pages` that no sequence uses) are handed out in a seeded
    random order, so a sequence's consecutive pages sit far apart in the pool,
    as in a server whose pages were freed and reused.  Returns
    (table [B, max_pages] int32, num_pages); entries past a sequence's pages
    are -1 (never read for lengths within the table)."""
    lens = np.asarray(lens, dtype=np.int64)
    need = (lens + page_rows - 1) // page_rows
    max_pages = max(int(need.max()), 1)
    num_pages = int(need.sum()) + int(spare_pages)
    order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = order[k:k + n]
        k += int(n)
    return table, num_pages


def paged_rows(table: np.ndarray, page_rows: int, b_idx, j_idx) -> np.ndarray:
    """Pool row of logical row j of sequence b under `table` (int64)."""
    b_idx = np.asarray(b_idx, dtype=np.int64)
    j_idx = np.asarray(j_idx, dtype=np.int64)
    return table[b_idx, j_idx // page_rows].astype(np.int64) * page_rows + j_idx % page_rows
