"""GPU parity of A1 from hidden states (KV down-projection, post-latent
RMSNorm, RoPE key, cache store) against the fp64 oracle.

Bound per element, from the arithmetic: the kernel sums the projections in
fp32 (relative error ~sqrt(d_model) 2^-24, below 1e-5 of the row's scale
here) and rounds each value once to the storage dtype, so
|gpu - exact| <= half an ulp of the stored value + 1e-5 rms(row half)."""
import numpy as np
import pytest

import oracle as O
from mla_latent_kv_24_amd import workloads as W
from helpers import TOL, f64, rel_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    from mla_latent_kv_24_amd import api as A
    return A


def dev(a, dtype):
    from mla_latent_kv_24_amd.pipeline import to_device
    return to_device(a, dtype)


def _inputs(dtype, n_tok, d_model, weighted, seed):
    h = W.random_storage(seed, (n_tok, d_model), dtype)
    w_dkv = W.random_storage(seed + 1, (512, d_model), dtype, d_model ** -0.5)
    w_kr = W.random_storage(seed + 2, (64, d_model), dtype, d_model ** -0.5)
    gamma = (W.to_storage(1.0 + 0.25 * np.random.default_rng(seed + 3).standard_normal(512).astype(np.float32),
                          dtype) if weighted else None)
    pos = W.random_ints(seed + 4, 0, 131072, n_tok).astype(np.int32)
    pos[: min(3, n_tok)] = [0, 4095, 131071][: min(3, n_tok)]
    return h, w_dkv, w_kr, gamma, pos


def _check_rows(got, exact, dtype):
    for half in (slice(0, 512), slice(512, 576)):
        g, e = got[:, half], exact[:, half]
        rms = np.sqrt(np.mean(e * e))
        if dtype == "bf16":
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), 1e-30))) - 7)
            bound = 0.5 * ulp + 1e-5 * rms
        else:
            bound = 1e-5 * rms + 2.0 ** -24 * np.abs(e)
        assert np.all(np.abs(g - e) <= bound), (half, float(np.max(np.abs(g - e) - bound)))


# V2 decode step (64 tokens of hidden 5120), V2-Lite (2048), a ragged token
# block, a d_model the MFMA tiling takes in 5 slices of 128, the generic bf16
# path (d_model not a multiple of 128), fp32 storage, a prefill chunk; from
# 256 tokens the LDS-tiled product, also with one token past a tile and k
# slices of 5, 5 and 3 stages of 64 (d_model 832)
CASES = [("bf16", 64, 5120, True), ("bf16", 1, 2048, False), ("bf16", 300, 2048, True),
         ("bf16", 70, 640, True), ("bf16", 5, 200, True), ("f32", 9, 300, True), ("bf16", 4096, 5120, True),
         ("bf16", 257, 832, False)]


@pytest.mark.parametrize("dtype,n_tok,d_model,weighted", CASES)
def test_rows_from_hidden(api, dtype, n_tok, d_model, weighted):
    print(f"kv projection {dtype} n_tok={n_tok} d_model={d_model}", flush=True)
    h, w_dkv, w_kr, gamma, pos = _inputs(dtype, n_tok, d_model, weighted, 50 + n_tok)
    cap = n_tok + 37
    rows = np.random.default_rng(7).permutation(cap)[:n_tok].astype(np.int64)
    d = api.dims(16)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = torch.full((cap, 576), float("nan"), dtype=tdt, device="cuda")
    eps = 1e-6
    args = (d, dev(h, dtype), dev(w_dkv, dtype), dev(w_kr, dtype),
            None if gamma is None else dev(gamma, dtype), eps, torch.from_numpy(pos).cuda(),
            torch.from_numpy(rows).cuda(), cache)
    api.append_kv_from_hidden(*args)
    torch.cuda.synchronize()
    first = cache.clone()
    api.append_kv_from_hidden(*args)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(first.view(bits), cache.view(bits))   # bitwise reproducible (NaN rows included)
    got = f64(to_np(cache)[rows], dtype)
    exact = O.append_rows_from_hidden(f64(h, dtype), f64(w_dkv, dtype), f64(w_kr, dtype), pos,
                                      None if gamma is None else f64(gamma, dtype), eps)
    _check_rows(got, exact, dtype)
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert np.all(np.isnan(f64(to_np(cache)[untouched], dtype)))


def test_rows_from_hidden_then_decode(api):
    """Two sequences' caches filled from hidden states, then decoded: the
    output meets the decode bar against the oracle fed the same hidden states."""
    n_h, d_model, lens, dtype = 128, 5120, (300, 77), "bf16"
    d = api.dims(n_h)
    stride = max(lens)
    h, w_dkv, w_kr, gamma, _ = _inputs(dtype, sum(lens), d_model, True, 91)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    rows = np.concatenate([b * stride + np.arange(L) for b, L in enumerate(lens)]).astype(np.int64)
    cache = torch.full((len(lens) * stride, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.append_kv_from_hidden(d, dev(h, dtype), dev(w_dkv, dtype), dev(w_kr, dtype), dev(gamma, dtype), 1e-6,
                              torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda(), cache)
    q_c = W.random_storage(92, (len(lens), n_h, 128), dtype)
    q_r = W.random_storage(93, (len(lens), n_h, 64), dtype)
    w_uk = W.random_storage(94, (n_h, 128, 512), dtype, 512 ** -0.5)
    w_uv = W.random_storage(95, (n_h, 128, 512), dtype, 512 ** -0.5)
    q_pos = np.array([L - 1 for L in lens], dtype=np.int32)
    q_lat = api.q_lat_empty(d, torch.bfloat16, len(lens))
    api.absorb_q(d, dev(q_c, dtype), dev(q_r, dtype), torch.from_numpy(q_pos).cuda(), dev(w_uk, dtype), q_lat)
    out = torch.empty((len(lens), n_h, 128), dtype=torch.float32, device="cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    api.decode(d, q_lat, cache, stride, seq, max(lens), dev(w_uv, dtype), out)
    got = out.cpu().numpy()
    c_all, k_all = O.kv_from_hidden(f64(h, dtype), f64(w_dkv, dtype), f64(w_kr, dtype), f64(gamma, dtype), 1e-6)
    off = 0
    for b, L in enumerate(lens):
        # the cache holds both halves rounded to bf16 (the oracle's storage reading)
        c = O.round_to_storage(c_all[off:off + L], dtype)
        k_rot = O.cached_rope_key(k_all[off:off + L], np.arange(L), 10000.0, store=dtype)
        q_rot = O.rope(f64(q_r[b], dtype), L - 1)
        o, _ = O.attend_unabsorbed(f64(q_c[b], dtype), q_rot, c, k_rot, f64(w_uk, dtype), f64(w_uv, dtype))
        assert rel_err(got[b], o) < TOL[dtype]
        off += L
