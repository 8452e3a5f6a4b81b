"""Shared helpers of the GPU parity tests: oracle adapters and error metrics."""
import numpy as np

import oracle as O
from mla_latent_kv_24_amd import workloads as W

TOL = {"bf16": 2e-2, "f32": 1e-4}   # max|gpu - ref| / rms(ref), per workload output


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref)) / np.sqrt(np.mean(np.square(ref))))


def f64(a, dtype):
    return W.to_f64(a, dtype)


def rope_freq(w):
    """What the oracle's RoPE takes for workload w: the frequency base, or the
    long-context pair frequencies when the workload extends its context."""
    return O.yarn_frequencies(W.D_R, w.rope_base, w.yarn_factor) if w.yarn_factor > 1 else w.rope_base


def score_scale(w):
    return O.yarn_softmax_scale(W.D_H, W.D_R, w.yarn_factor)


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def oracle_decode(inp, b, heads=None, absorbed=False):
    """fp64 oracle for sequence b (selected heads): (out [h, 128], z [h, 512]),
    over the cache as stored (RoPE key rounded to the workload's dtype).
    Unabsorbed by default; absorbed=True takes the oracle's absorbed form
    (pinned equal to the unabsorbed one to 1e-10), which is cheap enough to run
    over every sequence of a large batch."""
    dt = inp.w.dtype
    L = int(inp.seq_lens[b])
    heads = np.arange(inp.w.n_h) if heads is None else np.asarray(heads)
    c = f64(inp.c_kv[b, :L], dt)
    k_rot = O.cached_rope_key(f64(inp.k_raw[b, :L], dt), np.arange(L), rope_freq(inp.w), store=dt)
    q_rot = O.rope(f64(inp.q_r[b][heads], dt), L - 1, rope_freq(inp.w))
    args = (f64(inp.q_c[b][heads], dt), q_rot, c, k_rot, f64(inp.w_uk[heads], dt), f64(inp.w_uv[heads], dt),
            score_scale(inp.w))
    if absorbed:
        o, z, _ = O.attend_absorbed(*args)
        return o, z
    o, a = O.attend_unabsorbed(*args)
    return o, a @ c


def oracle_prefill(pinp, queries, heads=None):
    dt = pinp.w.dtype
    heads = np.arange(pinp.w.n_h) if heads is None else np.asarray(heads)
    return O.prefill(f64(pinp.q_c[:, heads], dt), f64(pinp.q_r[:, heads], dt), pinp.prefix,
                     f64(pinp.c_kv, dt), f64(pinp.k_raw, dt), f64(pinp.w_uk[heads], dt),
                     f64(pinp.w_uv[heads], dt), rope_freq(pinp.w), score_scale(pinp.w), query_idx=queries,
                     store=dt)


def absorbed_layout(q32, dtype):
    """Absorbed query input for the device: fp32 as is, or for bf16 storage the
    hi plane (bf16(q)) and the lo plane (bf16(q - hi)).  Returns (hi, lo or
    None, the fp64 value hi + lo carries: what the oracle is given)."""
    q32 = np.asarray(q32, dtype=np.float32)
    if dtype != "bf16":
        return q32, None, q32.astype(np.float64)
    hi = W.f32_to_bf16_bits(q32)
    lo = W.f32_to_bf16_bits(q32 - W.bf16_bits_to_f32(hi))
    value = W.bf16_bits_to_f32(hi).astype(np.float64) + W.bf16_bits_to_f32(lo).astype(np.float64)
    return hi, lo, value


def oracle_decode_fp8(inp, b, heads=None):
    """fp64 oracle for sequence b over the FP8 latent cache: the oracle's own
    E4M3 codes and per-row scales of c^KV (dequantised exactly), the RoPE key
    rounded to bf16 as stored.  Absorbed form (pinned to the unabsorbed one)."""
    L = int(inp.seq_lens[b])
    heads = np.arange(inp.w.n_h) if heads is None else np.asarray(heads)
    codes, scale = O.quantize_rows_fp8(f64(inp.c_kv[b, :L], "bf16"))
    c = O.dequantize_rows_fp8(codes, scale)
    k_rot = O.cached_rope_key(f64(inp.k_raw[b, :L], "bf16"), np.arange(L), rope_freq(inp.w), store="bf16")
    q_rot = O.rope(f64(inp.q_r[b][heads], "bf16"), L - 1, rope_freq(inp.w))
    o, z, _ = O.attend_absorbed(f64(inp.q_c[b][heads], "bf16"), q_rot, c, k_rot, f64(inp.w_uk[heads], "bf16"),
                                f64(inp.w_uv[heads], "bf16"), score_scale(inp.w))
    return o, z
