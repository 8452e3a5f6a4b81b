"""CPU oracle for MLA latent-KV attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The HIP library never calls it and shares no code with
it.  Everything here is plain float64 numpy (or pure Python loops for the
brute-force form); it is slow on purpose and follows the pages' equations
in their own order.

Sources (page title, then the part of it followed):
  [R2]  jiphyeonjeon.kr deep review "DeepSeek-V2: A Strong, Economical, and
        Efficient Mixture-of-Experts Language Model", section 2 -- joint
        low-rank compression c^KV = W^DKV h, k^C = W^UK c^KV, v^C = W^UV c^KV;
        the absorption identity (q^C)^T U^K_i c = ((U^K_i)^T q^C)^T c and
        sum_j a_ij U^V_i c_j = U^V_i sum_j a_ij c_j.
  [R3]  same review, section 3 -- decoupled RoPE: per-head 128-d content
        query/key, per-head 64-d RoPE query, ONE 64-d RoPE key per token;
        score l_ij = ((q^C_ti)^T k^C_ji + (q^R_ti)^T k^R_j) / sqrt(128 + 64),
        a_ij = softmax_j(l_ij); the scale stays sqrt(128+64) after absorption.
  [R4]  same review, section 4 -- per-token cache element counts (MHA 2 H d_h L,
        GQA 2 G d_h L, MQA 2 d_h L, MLA (d_c + d_h^R) L) and the worked
        byte counts behind the 93.3% figure.
  [L1]  irregular6612.github.io notes on the same paper, section 2.1.2
        (Low-Rank Key-Value Joint Compression).
  [V3]  xyznot.com "Laporan Teknis DeepSeek-V3", Metode 1 (MLA):
        k^R_t = RoPE(W^KR h_t), k_{t,i} = [k^C_{t,i}; k^R_t]; only c^KV and
        k^R are cached.

Readings where the pages are silent (the decoupled-RoPE section of [L1] has
no body, and no page defines RoPE itself):
  * RoPE rotates interleaved pairs (x[2k], x[2k+1]) by angle p * theta_k,
    theta_k = base ** (-2k / d_h^R), base 10000, angle formed in float64.
  * Decode: the new token's row is already in the cache; the query sits at
    position len-1 and attends to rows 0..len-1 (itself included).
  * Prefill: query i of a chunk sits at position prefix+i and attends to rows
    0..prefix+i (inclusive causal mask).
  * W^UK and W^UV are stored per head as [n_h][d_h][d_c]; U^K_i = w_uk[i].
  * The cache is a tensor of the storage dtype ([V3]: c^KV and k^R are what is
    cached; [R4]: d_c + d_h^R elements per token), so the RoPE key that the
    attention reads is RoPE(k_raw) rounded to that dtype (`store=` below;
    round to nearest even, float64 -> float32 -> bfloat16).  c^KV needs no
    rounding: it is stored as given.
  * Rows made from hidden states ([L1], [V3]: c^KV = W^DKV h, k^R =
    RoPE(W^KR h); [R2]: the model normalises the compressed latent with an
    RMSNorm): c^KV = RMSNorm(W^DKV h) * weight, over the d_c latent channels
    only, with eps 1e-6 unless given (the pages give no value) and a
    per-channel weight supplied by the caller (1 if absent); the width
    bottleneck scaling that [R2] mentions has no value on the pages and is
    taken as folded into that weight.  The cache holds the normalised latent
    (the one W^UK and W^UV consume); k^R is not normalised.  Both halves of
    the row are rounded to the storage dtype once, from their exact values.

  * Query side: c^Q = RMSNorm(W^DQ h) * weight over the d_c' = 1,536 query
    latent channels (as for c^KV), q^C = W^UQ c^Q and the decoupled RoPE
    query q^R = W^QR c^Q (no page prints W^QR; the per-head 64-d RoPE query of
    [R3] is read as coming from the query latent), RoPE applied at absorption.
  * Quantised latent cache (the pages report a cache of about 6 bits per
    element for the served model -- review section 4 -- without giving a
    format): c^KV is stored as FP8 E4M3 (the OCP 8-bit float: 1 sign, 4
    exponent bits of bias 7, 3 mantissa bits, no infinities, 448 the largest
    finite value) with one float32 scale per row, s = amax|c| / 448, and the
    code of each element the round-to-nearest-even of c / s; k^R stays in
    bf16.  The scale and the codes are decided in float32 (the kernel's
    precision; divisions correctly rounded), so this oracle reproduces them
    exactly.  A row of zeros takes s = 1.

  * Long-context RoPE ([R2] section 6: the 4K-pretrained model is extended
    with YaRN at scale s = 40 towards a 160K target, 40 x 4K; the pages give
    no formula).  Taken as YaRN's published frequency interpolation (Peng et
    al., 2023, "NTK-by-parts" with its attention temperature): pair k keeps
    theta_k where its wavelength 2 pi / theta_k fits many times into the
    pretraining context L = 4,096, is slowed to theta_k / s where it does not
    fit once, and blends linearly in between -- with r_k = L theta_k / (2 pi)
    and gamma_k = clip((r_k - alpha) / (beta - alpha), 0, 1),
    theta'_k = (1 - gamma_k) theta_k / s + gamma_k theta_k, alpha = 1 and
    beta = 32 (that paper's values; the pages give none).  The temperature
    (sqrt(1/t) = 0.1 ln s + 1) multiplies the whole logit, content and RoPE
    halves alike, by (0.1 ln s + 1)^2.  RoPE acts on q^R and k^R only ([R3]).

Parity: every function below is pinned by tests that do not re-type its
formula (closed forms, brute force, a library attention routine, identities,
the pages' printed cache numbers).
"""
from __future__ import annotations

import math
import numpy as np

ROPE_BASE = 10000.0


# ---------------------------------------------------------------------------
# RoPE ([R3] rotates query and key by position; convention: see header)
# ---------------------------------------------------------------------------
def rope_frequencies(d: int, base=ROPE_BASE) -> np.ndarray:
    """Angular frequency of each of the d/2 pairs: base**(-2k/d) for a scalar
    base; an array of d/2 frequencies (yarn_frequencies') is taken as given."""
    if np.ndim(base) == 0:
        k = np.arange(d // 2, dtype=np.float64)
        return np.power(float(base), -2.0 * k / d)
    theta = np.asarray(base, dtype=np.float64)
    if theta.shape != (d // 2,):
        raise ValueError(f"need {d // 2} pair frequencies, got shape {theta.shape}")
    return theta


def yarn_frequencies(d: int, base: float, factor: float, orig_ctx: float = 4096.0,
                     alpha: float = 1.0, beta: float = 32.0) -> np.ndarray:
    """Pair frequencies of the long-context RoPE (header: YaRN reading).
    factor <= 1 leaves the plain frequencies."""
    theta = rope_frequencies(d, base)
    if factor <= 1.0:
        return theta
    turns = orig_ctx * theta / (2.0 * math.pi)          # wavelengths inside the context
    gamma = np.clip((turns - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * (theta / factor) + gamma * theta


def yarn_softmax_scale(d_h: int, d_r: int, factor: float) -> float:
    """The score scale with YaRN's temperature: (0.1 ln s + 1)^2 / sqrt(d_h + d_r)
    for s > 1, the plain scale otherwise."""
    m = 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0
    return m * m * default_scale(d_h, d_r)


def rope(x: np.ndarray, pos, base=ROPE_BASE) -> np.ndarray:
    """Rotate the last axis of x (even length d) by position(s) `pos`.

    x: [..., d]; pos broadcasts against x.shape[:-1].
    Pair k = (x[2k], x[2k+1]) is rotated by angle pos * theta_k, theta_k =
    base**(-2k/d), or the k-th entry of `base` when it is an array of pair
    frequencies.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even width")
    theta = rope_frequencies(d, base)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def round_to_storage(x, store: str) -> np.ndarray:
    """Values of x as a tensor of storage dtype `store` holds them, as float64.

    "f32": round to nearest even float32.  "bf16": float32 first, then round to
    nearest even on the upper 16 bits (bfloat16 keeps float32's sign and
    exponent and the top 7 mantissa bits); NaN stays NaN.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if store == "f32":
        return x32.astype(np.float64)
    if store != "bf16":
        raise ValueError(f"unknown storage dtype {store!r}")
    u = x32.view(np.uint32).astype(np.uint64)
    kept_lsb = (u >> 16) & 1
    r = (((u + 0x7FFF + kept_lsb) >> 16) << 16) & 0xFFFFFFFF
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x32), np.float32(np.nan), out).astype(np.float64)


def cached_rope_key(k_raw, pos, base: float = ROPE_BASE, store=None) -> np.ndarray:
    """k^R_j = RoPE(k_raw_j, pos_j) ([V3]) as the cache holds it: exact float64
    when store is None, else rounded to the storage dtype."""
    k = rope(k_raw, pos, base)
    return k if store is None else round_to_storage(k, store)


def softmax(logits: np.ndarray, axis: int = -1) -> np.ndarray:
    """Max-subtracted softmax in float64 ([R3] a_ij = softmax_j(l_ij))."""
    logits = np.asarray(logits, dtype=np.float64)
    m = np.max(logits, axis=axis, keepdims=True)
    e = np.exp(logits - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def default_scale(d_h: int, d_r: int) -> float:
    """[R3]: 1/sqrt(d_h + d_h^R) -- 1/sqrt(128+64) for V2 -- also after absorption."""
    return 1.0 / math.sqrt(d_h + d_r)


# ---------------------------------------------------------------------------
# A1: the cached row of a token ([V3] only c^KV and k^R are cached)
# ---------------------------------------------------------------------------
def append_rows(c_kv: np.ndarray, k_raw: np.ndarray, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Cache rows [c^KV_t ; RoPE(k_raw_t, pos_t)] -> [N, d_c + d_h^R]."""
    c_kv = np.asarray(c_kv, dtype=np.float64)
    return np.concatenate([c_kv, rope(k_raw, pos, base)], axis=-1)


# ---------------------------------------------------------------------------
# A1 from hidden states ([L1] / [V3] c^KV = W^DKV h, k^R = RoPE(W^KR h);
# [R2] RMSNorm after the compressed latent)
# ---------------------------------------------------------------------------
def rms_norm(x, weight=None, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, times a per-channel weight."""
    x = np.asarray(x, dtype=np.float64)
    inv = 1.0 / np.sqrt(np.mean(np.square(x), axis=-1, keepdims=True) + eps)
    out = x * inv
    return out if weight is None else out * np.asarray(weight, dtype=np.float64)


def kv_from_hidden(h, w_dkv, w_kr, norm_weight=None, eps: float = 1e-6):
    """(c^KV, k_raw) of tokens with hidden states h [N, d_model]:
    c^KV = RMSNorm(W^DKV h) * norm_weight  [N, d_c]   (w_dkv [d_c, d_model])
    k_raw = W^KR h                        [N, d_h^R] (w_kr [d_h^R, d_model]; RoPE comes at append)."""
    h = np.asarray(h, dtype=np.float64)
    latent = h @ np.asarray(w_dkv, dtype=np.float64).T
    k_raw = h @ np.asarray(w_kr, dtype=np.float64).T
    return rms_norm(latent, norm_weight, eps), k_raw


def append_rows_from_hidden(h, w_dkv, w_kr, pos, norm_weight=None, eps: float = 1e-6,
                            base: float = ROPE_BASE, store=None) -> np.ndarray:
    """Cache rows [c^KV_t ; RoPE(W^KR h_t, pos_t)] made from hidden states, each
    half rounded once to the storage dtype when `store` is given."""
    c, k_raw = kv_from_hidden(h, w_dkv, w_kr, norm_weight, eps)
    rows = append_rows(c, k_raw, pos, base)
    return rows if store is None else round_to_storage(rows, store)


# ---------------------------------------------------------------------------
# The projections around the path: the query side ([R2] queries pass through a
# 1,536-wide latent; [V3] c^Q; the latent normalised as c^KV is, [R2]) and the
# output side ([R2] u_t = sum_i O_i U^V_i sum_j a_ij c_j)
# ---------------------------------------------------------------------------
def query_from_hidden(h, w_dq, w_uq, w_qr, n_h: int, norm_weight=None, eps: float = 1e-6):
    """(q^C [N, n_h, d_h], q^R [N, n_h, d_h^R] before RoPE) of hidden states h [N, d_model]:
    c^Q = RMSNorm(W^DQ h) * norm_weight (w_dq [d_c', d_model]),
    q^C = W^UQ c^Q (w_uq [n_h d_h, d_c'], head i = rows i d_h ..), q^R = W^QR c^Q
    (w_qr [n_h d_h^R, d_c'])."""
    h = np.asarray(h, dtype=np.float64)
    c_q = rms_norm(h @ np.asarray(w_dq, dtype=np.float64).T, norm_weight, eps)
    q_c = c_q @ np.asarray(w_uq, dtype=np.float64).T
    q_r = c_q @ np.asarray(w_qr, dtype=np.float64).T
    return q_c.reshape(h.shape[0], n_h, -1), q_r.reshape(h.shape[0], n_h, -1)


def output_projection(o, w_o) -> np.ndarray:
    """u_t = sum_i O_i o_{t,i} with o [N, n_h, d_h] and w_o [d_model, n_h d_h],
    O_i = columns i d_h .. (i+1) d_h - 1 of w_o."""
    o = np.asarray(o, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    n_h, d_h = o.shape[1], o.shape[2]
    u = np.zeros((o.shape[0], w_o.shape[0]))
    for i in range(n_h):
        u += o[:, i, :] @ w_o[:, i * d_h:(i + 1) * d_h].T
    return u


# ---------------------------------------------------------------------------
# Quantised latent (FP8 E4M3 codes + one float32 scale per row; see header)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each 8-bit E4M3 code as float64: sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); the
    code with every exponent and mantissa bit set is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest finite E4M3 value, ties to the code with
    an even mantissa (round to nearest even), keeping the sign (a negative
    value that rounds to zero gives -0, code 0x80); |x| up to the midpoint 464
    above 448 rounds to +-448, beyond it raises (the quantiser never gets
    there)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) >= 464.0):
        raise ValueError("E4M3 encode: NaN or |x| >= 464")
    pos = np.arange(0x7F, dtype=np.uint8)              # codes 0x00..0x7E: 0 .. 448, increasing
    vals = e4m3_decode(pos)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((pos[hi] & 1) == 0))
    code = np.where(pick_hi, pos[hi], pos[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)   # the sign is kept, zero included


def quantize_rows_fp8(c):
    """(codes uint8 [N, d], scale float32 [N]) of latent rows c [N, d] (values
    exact in float32): s = amax / 448 and y = c / s in float32, codes = E4M3(y)."""
    c32 = np.asarray(c, dtype=np.float32)
    amax = np.max(np.abs(c32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (c32 / scale[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def dequantize_rows_fp8(codes, scale) -> np.ndarray:
    """float64 latent values the quantised rows stand for: E4M3(code) * s."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------------------------
# A2: the absorbed query ([R2] (U^K_i)^T q^C; [R3] RoPE query per head)
# ---------------------------------------------------------------------------
def absorb_query(q_c: np.ndarray, q_r: np.ndarray, q_pos, w_uk: np.ndarray,
                 base: float = ROPE_BASE) -> np.ndarray:
    """q_lat[n, i] = [(U^K_i)^T q^C_{n,i} ; RoPE(q^R_{n,i}, pos_n)].

    q_c [n, n_h, d_h], q_r [n, n_h, d_r], q_pos [n], w_uk [n_h, d_h, d_c]
    -> [n, n_h, d_c + d_r].
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    n, n_h, _ = q_c.shape
    lat = np.empty((n, n_h, w_uk.shape[2]), dtype=np.float64)
    for i in range(n_h):
        lat[:, i, :] = q_c[:, i, :] @ w_uk[i]           # ((U^K_i)^T q)^T = q^T U^K_i
    pos = np.asarray(q_pos, dtype=np.float64)[:, None]  # same position for all heads
    return np.concatenate([lat, rope(q_r, pos, base)], axis=-1)


# ---------------------------------------------------------------------------
# The definition: unabsorbed MLA attention for one query token
# ---------------------------------------------------------------------------
def attend_unabsorbed(q_c, q_r_rot, c, k_r_rot, w_uk, w_uv, scale=None):
    """Standard softmax attention with explicit per-head keys and values.

    q_c [n_h, d_h], q_r_rot [n_h, d_r] (already rotated), c [T, d_c],
    k_r_rot [T, d_r] (already rotated), w_uk / w_uv [n_h, d_h, d_c].
    For head i ([R2], [R3], [V3]):
        k^C_{j,i} = U^K_i c_j,  v^C_{j,i} = U^V_i c_j,  k_{j,i} = [k^C_{j,i}; k^R_j]
        q_i = [q^C_i ; q^R_i],  l_ij = q_i . k_{j,i} * scale,  a_i = softmax(l_i)
        o_i = sum_j a_ij v^C_{j,i}
    Returns (o [n_h, d_h], a [n_h, T]).
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r_rot = np.asarray(q_r_rot, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    k_r_rot = np.asarray(k_r_rot, dtype=np.float64)
    n_h, d_h = q_c.shape
    d_r = q_r_rot.shape[1]
    if scale is None:
        scale = default_scale(d_h, d_r)
    T = c.shape[0]
    out = np.empty((n_h, d_h), dtype=np.float64)
    probs = np.empty((n_h, T), dtype=np.float64)
    for i in range(n_h):
        u_k = np.asarray(w_uk[i], dtype=np.float64)       # [d_h, d_c]
        u_v = np.asarray(w_uv[i], dtype=np.float64)
        k_c = c @ u_k.T                                    # rows: U^K_i c_j
        v_c = c @ u_v.T                                    # rows: U^V_i c_j
        keys = np.concatenate([k_c, k_r_rot], axis=1)      # [T, d_h + d_r]
        q = np.concatenate([q_c[i], q_r_rot[i]])
        a = softmax(keys @ q * scale)
        out[i] = a @ v_c
        probs[i] = a
    return out, probs


def attend_absorbed(q_c, q_r_rot, c, k_r_rot, w_uk, w_uv, scale=None):
    """The same attention computed after absorption ([R2]).

    q~_i = (U^K_i)^T q^C_i, l_ij = (q~_i . c_j + q^R_i . k^R_j) * scale,
    z_i = sum_j a_ij c_j, o_i = U^V_i z_i.
    Returns (o [n_h, d_h], z [n_h, d_c], a [n_h, T]).
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r_rot = np.asarray(q_r_rot, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    k_r_rot = np.asarray(k_r_rot, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    n_h, d_h = q_c.shape
    if scale is None:
        scale = default_scale(d_h, q_r_rot.shape[1])
    q_lat = np.einsum("hd,hdc->hc", q_c, w_uk)
    logits = (q_lat @ c.T + q_r_rot @ k_r_rot.T) * scale
    a = softmax(logits, axis=1)
    z = a @ c
    out = np.einsum("hdc,hc->hd", w_uv, z)
    return out, z, a


# ---------------------------------------------------------------------------
# Decode over a batch and causal prefill
# ---------------------------------------------------------------------------
def decode(q_c, q_r, seq_lens, c_kv, k_raw, w_uk, w_uv, base=ROPE_BASE, scale=None,
           batch_idx=None, absorbed=False, store=None):
    """Decode one token per sequence.

    q_c [B, n_h, d_h], q_r [B, n_h, d_r] (pre-RoPE), seq_lens [B],
    c_kv [B, S, d_c], k_raw [B, S, d_r] (pre-RoPE; row j sits at position j).
    The query of sequence b sits at position len_b - 1 and attends rows
    0..len_b-1.  Returns (out [B', n_h, d_h], z [B', n_h, d_c]) for the
    sequences in `batch_idx` (all by default).  z is sum_j a_ij c_j.
    store: storage dtype of the cache ("bf16", "f32"), whose rounding of the
    RoPE key the attention reads; None keeps the exact key.
    """
    idx = range(len(seq_lens)) if batch_idx is None else list(batch_idx)
    outs, zs = [], []
    for b in idx:
        T = int(seq_lens[b])
        c = np.asarray(c_kv[b, :T], dtype=np.float64)
        k_rot = cached_rope_key(k_raw[b, :T], np.arange(T), base, store)
        q_rot = rope(q_r[b], T - 1, base)
        if absorbed:
            o, z, _ = attend_absorbed(q_c[b], q_rot, c, k_rot, w_uk, w_uv, scale)
        else:
            o, a = attend_unabsorbed(q_c[b], q_rot, c, k_rot, w_uk, w_uv, scale)
            z = a @ c
        outs.append(o)
        zs.append(z)
    return np.stack(outs), np.stack(zs)


def prefill(q_c, q_r, prefix, c_kv, k_raw, w_uk, w_uv, base=ROPE_BASE, scale=None,
            query_idx=None, store=None):
    """Causal prefill of one sequence.

    Rows 0..prefix+chunk-1 of (c_kv, k_raw) are cached (row j at position j).
    Query i (q_c [chunk, n_h, d_h], q_r pre-RoPE) sits at position prefix+i and
    attends rows 0..prefix+i.  Returns out [n, n_h, d_h] for the queries in
    `query_idx` (all by default), computed unabsorbed.  store: as in decode.
    """
    chunk = q_c.shape[0]
    idx = range(chunk) if query_idx is None else list(query_idx)
    total = prefix + chunk
    c = np.asarray(c_kv[:total], dtype=np.float64)
    k_rot = cached_rope_key(k_raw[:total], np.arange(total), base, store)
    n_h, d_h = q_c.shape[1], q_c.shape[2]
    d_r = q_r.shape[2]
    if scale is None:
        scale = default_scale(d_h, d_r)
    idx = list(idx)
    out = np.empty((len(idx), n_h, d_h), dtype=np.float64)
    q_rot = rope(np.asarray(q_r, dtype=np.float64)[idx],
                 (prefix + np.asarray(idx, dtype=np.float64))[:, None], base)
    for i in range(n_h):
        u_k = np.asarray(w_uk[i], dtype=np.float64)
        u_v = np.asarray(w_uv[i], dtype=np.float64)
        keys = np.concatenate([c @ u_k.T, k_rot], axis=1)          # [total, d_h + d_r]
        vals = c @ u_v.T                                           # [total, d_h]
        q = np.concatenate([np.asarray(q_c, dtype=np.float64)[idx, i], q_rot[:, i]], axis=1)
        logits = (q @ keys.T) * scale                              # [n, total]
        pos = prefix + np.asarray(idx)[:, None]
        logits = np.where(np.arange(total)[None, :] <= pos, logits, -np.inf)
        out[:, i, :] = softmax(logits, axis=1) @ vals
    return out


# ---------------------------------------------------------------------------
# A3/A4/A5 in latent space: split-KV partials, their combine, the W^UV step
# ---------------------------------------------------------------------------
def split_partials(q_lat, rows, seq_len, chunk, num_splits, scale, d_c=512):
    """Per split s (rows [s*chunk, min((s+1)*chunk, seq_len))), per head:
        lse_s = log sum_j exp(l_j),  Z_s = sum_j exp(l_j - lse_s) c_j,
    with l_j = (q_lat . row_j) * scale.  Empty split: lse = -inf, Z = 0.
    This is softmax_j of [R3] restricted to a range of j (re-associated).
    q_lat [n_h, d_c + d_r], rows [>= seq_len, d_c + d_r].
    Returns Z [S, n_h, d_c], lse [S, n_h].
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    n_h = q_lat.shape[0]
    Z = np.zeros((num_splits, n_h, d_c), dtype=np.float64)
    lse = np.full((num_splits, n_h), -np.inf, dtype=np.float64)
    for s in range(num_splits):
        lo, hi = s * chunk, min((s + 1) * chunk, int(seq_len))
        if lo >= hi:
            continue
        r = np.asarray(rows[lo:hi], dtype=np.float64)
        logits = (q_lat @ r.T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        l = e.sum(axis=1, keepdims=True)
        lse[s] = (m + np.log(l))[:, 0]
        Z[s] = (e / l) @ r[:, :d_c]
    return Z, lse


def combine_partials(Z, lse):
    """LSE = log sum_s exp(lse_s); z = sum_s exp(lse_s - LSE) Z_s.  [S, n_h, *] -> [n_h, *]."""
    Z = np.asarray(Z, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=0)
    w = np.exp(lse - m[None, :])
    tot = w.sum(axis=0)
    return np.einsum("sh,shc->hc", w / tot[None, :], Z), m + np.log(tot)


def project_uv(z, w_uv):
    """o_i = U^V_i z_i ([R2] value up-projection after the weighted sum)."""
    return np.einsum("hdc,...hc->...hd", np.asarray(w_uv, dtype=np.float64),
                     np.asarray(z, dtype=np.float64))


def latent_attention(q_lat, rows, seq_len, scale, d_c=512):
    """Absorbed attention straight from stored q_lat and cache rows:
    a = softmax((q_lat . row_j) * scale, j < seq_len); z = sum_j a_j c_j."""
    r = np.asarray(rows[:seq_len], dtype=np.float64)
    a = softmax((np.asarray(q_lat, dtype=np.float64) @ r.T) * scale, axis=1)
    return a @ r[:, :d_c]


# ---------------------------------------------------------------------------
# Brute force: pure Python scalar loops, tiny inputs only
# ---------------------------------------------------------------------------
def decode_bruteforce(q_c, q_r, pos_q, c, k_raw, w_uk, w_uv, base=ROPE_BASE, scale=None):
    """One query, one sequence, every step a scalar loop.  Rows 0..T-1 at positions 0..T-1."""
    n_h, d_h = len(q_c), len(q_c[0])
    d_r = len(q_r[0])
    d_c = len(c[0])
    T = len(c)
    if scale is None:
        scale = 1.0 / math.sqrt(d_h + d_r)

    def rot(vec, p):
        outv = [0.0] * d_r
        for k in range(d_r // 2):
            ang = p * (base ** (-2.0 * k / d_r))
            cs, sn = math.cos(ang), math.sin(ang)
            a0, a1 = float(vec[2 * k]), float(vec[2 * k + 1])
            outv[2 * k] = a0 * cs - a1 * sn
            outv[2 * k + 1] = a0 * sn + a1 * cs
        return outv

    krot = [rot(k_raw[j], j) for j in range(T)]
    out = [[0.0] * d_h for _ in range(n_h)]
    for i in range(n_h):
        qr = rot(q_r[i], pos_q)
        logit = []
        vals = []
        for j in range(T):
            s = 0.0
            v = [0.0] * d_h
            for r in range(d_h):
                kc = 0.0
                vc = 0.0
                for e in range(d_c):
                    kc += float(w_uk[i][r][e]) * float(c[j][e])
                    vc += float(w_uv[i][r][e]) * float(c[j][e])
                s += float(q_c[i][r]) * kc
                v[r] = vc
            for r in range(d_r):
                s += qr[r] * krot[j][r]
            logit.append(s * scale)
            vals.append(v)
        mx = max(logit)
        ws = [math.exp(x - mx) for x in logit]
        tot = sum(ws)
        for j in range(T):
            for r in range(d_h):
                out[i][r] += ws[j] / tot * vals[j][r]
    return out


# ---------------------------------------------------------------------------
# Cache accounting ([R4] per-token elements; bytes at a given bit width)
# ---------------------------------------------------------------------------
def cache_elements(kind: str, layers: int, d_h: int = 128, heads: int = 0, groups: int = 0,
                   d_c: int = 512, d_r: int = 64) -> int:
    """Per-token KV-cache elements: MHA 2*H*d_h*L, GQA 2*G*d_h*L, MQA 2*d_h*L,
    MLA (d_c + d_h^R)*L."""
    if kind == "mha":
        return 2 * heads * d_h * layers
    if kind == "gqa":
        return 2 * groups * d_h * layers
    if kind == "mqa":
        return 2 * d_h * layers
    if kind == "mla":
        return (d_c + d_r) * layers
    raise ValueError(kind)


def cache_bytes(elements: int, bits_per_element: float) -> float:
    return elements * bits_per_element / 8.0
