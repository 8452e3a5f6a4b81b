"""GPU tests of the FP8 latent cache: A1's codes and scales bit for bit
against the oracle's quantiser (both decide in fp32), and decode over the
quantised cache against the oracle over its own dequantised rows, at the
bf16 bar (the codes are shared, so the bar covers only the kernel's own
roundings, as on the bf16 path)."""
import numpy as np
import pytest

import oracle as O
from mla_latent_kv_24_amd import workloads as W
from helpers import TOL, f64, oracle_decode, oracle_decode_fp8, rel_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    from mla_latent_kv_24_amd import api as A
    return A


@pytest.fixture(scope="module")
def pipeline():
    from mla_latent_kv_24_amd import pipeline as P
    return P


def dev(a, dtype):
    from mla_latent_kv_24_amd.pipeline import to_device
    return to_device(a, dtype)


def test_append_fp8_codes_and_scales_bit_exact(api):
    n, cap = 700, 1000
    r = np.random.default_rng(60)
    c = r.standard_normal((n, 512)).astype(np.float32) * r.choice([1e-3, 1.0, 40.0], (n, 1)).astype(np.float32)
    c[0] = 0.0                                          # zero row: scale 1, codes 0
    c[1] = 0.0
    c[1, 17] = -3.0                                     # one element: it maps to -448
    c[2] = -c[2]
    c[3, ::2] = -0.0                                    # negative zeros keep their sign
    c = W.to_storage(c, "bf16")
    k = W.random_storage(61, (n, 64), "bf16")
    pos = W.random_ints(62, 0, 131072, n).astype(np.int32)
    rows = r.permutation(cap)[:n].astype(np.int64)
    d = api.dims(128)
    cache = api.fp8_cache_empty(cap)
    cache[0].fill_(0x7F)
    cache[1].fill_(float("nan"))
    cache[2].fill_(float("nan"))
    api.append_kv_fp8(d, dev(c, "bf16"), dev(k, "bf16"), torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda(),
                      cache)
    torch.cuda.synchronize()
    codes = cache[0].cpu().numpy()[rows]
    scale = cache[2].cpu().numpy()[rows]
    ref_codes, ref_scale = O.quantize_rows_fp8(f64(c, "bf16"))
    assert np.array_equal(scale.view(np.uint32), ref_scale.view(np.uint32))
    assert np.array_equal(codes, ref_codes)
    assert scale[0] == 1.0 and np.all(codes[0] == 0) and codes[1, 17] == 0xFE
    # the RoPE half: one rounding of the exact rotation to bf16
    ref_k = O.cached_rope_key(f64(k, "bf16"), pos, 10000.0)
    got_k = f64(to_np(cache[1])[rows], "bf16")
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_k), 1e-30))) - 7)
    assert np.all(np.abs(got_k - ref_k) <= ulp + 1e-30)
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert np.all(cache[0].cpu().numpy()[untouched] == 0x7F)


# 128 heads and 16 heads (matrix-core kernels) at several lengths, ragged
# tails and ragged batches (at 128 heads one that mixes queries under and over
# the precise-path threshold; at 16 heads one of more workgroups than compute
# units, which take their units longest first); 32 heads (generic kernel)
CASES = [("v2_decode", dict(batch=3, seq_len=1000)), ("v2_decode", dict(batch=2, seq_len=4099)),
         ("v2_decode", dict(batch=5, seq_len=65)), ("v2_decode", dict(batch=1, seq_len=1)),
         ("v2_decode", dict(batch=2, seq_len=33)), ("lite_decode", dict(batch=3, seq_len=300)),
         ("lite_decode", dict(batch=2, seq_len=4113)), ("lite_decode", dict(batch=3, seq_len=17)),
         ("lite_ragged", dict(batch=6, seq_len=3000)), ("lite_decode", dict(batch=2, seq_len=300, n_h=32)),
         ("v2_decode", dict(batch=6, seq_len=9000, ragged=True)),
         ("lite_ragged", dict(batch=100, seq_len=5000))]   # 300 workgroups: units longest first


@pytest.mark.parametrize("name,changes", CASES, ids=[f"{c[0]}-{c[1]['batch']}x{c[1]['seq_len']}-h{c[1].get('n_h', '')}" for c in CASES])
def test_decode_fp8(pipeline, name, changes):
    w = W.scaled(W.WORKLOADS[name], **changes)
    inp = W.make_decode_inputs(w)
    print(f"fp8 decode {name} {changes}", flush=True)
    st = pipeline.DecodeState(inp, out_latent=True, fp8=True)
    st.absorb()
    st.attention()
    st.combine()
    out = st.out.cpu().numpy()
    lat = st.out_latent.cpu().numpy()
    assert np.all(np.isfinite(out))                       # NaN codes past every length are never read
    refs = [oracle_decode_fp8(inp, b) for b in range(w.batch)]
    tol = TOL["bf16"]
    e_out = rel_err(out, np.stack([r[0] for r in refs]))
    e_lat = rel_err(lat, np.stack([r[1] for r in refs]))
    print(f"fp8 parity: out {e_out:.3e}, latent {e_lat:.3e} (bar {tol})")
    assert e_out < tol and e_lat < tol
    # what the quantisation itself costs, against the bf16 cache's exact output
    # (informational; E4M3 rounds each latent element by up to 2^-4 relative,
    # about 3.6% rms, and the output's rms deviation is of that size)
    exact = np.stack([oracle_decode(inp, b, absorbed=True)[0] for b in range(w.batch)])
    q_rms = float(np.sqrt(np.mean((out - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))
    print(f"fp8 cache vs exact bf16-cache output: max {rel_err(out, exact):.3e}, rms {q_rms:.3e}")
    assert q_rms < 0.06


def test_decode_fp8_fused_equals_partials(api, pipeline):
    w = W.scaled(W.WORKLOADS["v2_decode"], batch=4, seq_len=2000)
    st = pipeline.DecodeState(W.make_decode_inputs(w), out_latent=True, fp8=True)
    st.absorb()
    st.attention()
    st.combine()
    torch.cuda.synchronize()
    out = torch.empty_like(st.out)
    lat = torch.empty_like(st.out_latent)
    api.decode_fp8(st.d, st.q_lat, st.cache, st.stride, st.seq_lens, st.max_len, st.w_uv, out, lat)
    torch.cuda.synchronize()
    assert torch.equal(out, st.out) and torch.equal(lat, st.out_latent)
    # deterministic across calls
    api.decode_fp8(st.d, st.q_lat, st.cache, st.stride, st.seq_lens, st.max_len, st.w_uv, out, lat)
    torch.cuda.synchronize()
    assert torch.equal(out, st.out)


# Query lengths 2001..2065, 301..340, 4061..4130 (straddling the precise-path
# threshold of 4,096 rows) and 1001..1070: every query ends in a ragged tile
# and the chunk crosses a tile boundary.
@pytest.mark.parametrize("n_h,prefix,chunk", [(128, 2000, 65), (128, 300, 40), (128, 4060, 70), (16, 1000, 70)])
def test_prefill_fp8(api, n_h, prefix, chunk):
    """Causal prefill over the FP8 cache against the oracle's prefill on its own
    dequantised rows (the RoPE key rounded to bf16 as stored)."""
    base = W.WORKLOADS["v2_prefill"] if n_h == 128 else W.scaled(W.WORKLOADS["lite_decode"], batch=1)
    pinp = W.make_prefill_inputs(W.scaled(base, seq_len=prefix + chunk, prefill_chunk=chunk, batch=1))
    total = prefix + chunk
    d = api.dims(n_h)
    cache = api.fp8_cache_empty(total)
    api.append_kv_fp8(d, dev(pinp.c_kv, "bf16"), dev(pinp.k_raw, "bf16"),
                      torch.arange(total, dtype=torch.int32, device="cuda"),
                      torch.arange(total, dtype=torch.int64, device="cuda"), cache)
    q_lat = api.q_lat_empty(d, torch.bfloat16, 1, chunk)
    api.absorb_q(d, dev(pinp.q_c, "bf16"), dev(pinp.q_r, "bf16"),
                 torch.arange(prefix, total, dtype=torch.int32, device="cuda"), dev(pinp.w_uk, "bf16"),
                 q_lat.view(chunk, n_h, 576))
    out = torch.empty((1, chunk, n_h, 128), dtype=torch.float32, device="cuda")
    api.prefill_fp8(d, q_lat, cache, total, torch.tensor([prefix], dtype=torch.int32, device="cuda"), prefix,
                    dev(pinp.w_uv, "bf16"), out)
    got = out.cpu().numpy()[0]
    codes, scale = O.quantize_rows_fp8(f64(pinp.c_kv, "bf16"))
    ref = O.prefill(f64(pinp.q_c, "bf16"), f64(pinp.q_r, "bf16"), prefix, O.dequantize_rows_fp8(codes, scale),
                    f64(pinp.k_raw, "bf16"), f64(pinp.w_uk, "bf16"), f64(pinp.w_uv, "bf16"), pinp.w.rope_base,
                    store="bf16")
    e = rel_err(got, ref)
    print(f"fp8 prefill parity: {e:.3e}")
    assert np.all(np.isfinite(got)) and e < TOL["bf16"]


def test_decode_fp8_long_context_rope(pipeline):
    """The FP8 cache under the long-context RoPE (YaRN at scale 40: its pair
    frequencies in the appended keys and the absorbed queries, its temperature
    in the score), 16 heads over 6,000 rows, against the oracle on its own
    dequantised rows with the same frequencies and scale.  The 16-head kernel
    scores with hi + lo queries, so the bf16 bar applies."""
    w = W.scaled(W.WORKLOADS["lite_decode"], batch=2, seq_len=6000, yarn_factor=40.0)
    inp = W.make_decode_inputs(w)
    st = pipeline.DecodeState(inp, out_latent=True, fp8=True)
    st.absorb()
    st.attention()
    st.combine()
    out = st.out.cpu().numpy()
    refs = [oracle_decode_fp8(inp, b) for b in range(w.batch)]
    e = rel_err(out, np.stack([r[0] for r in refs]))
    plain = W.make_decode_inputs(W.scaled(w, yarn_factor=0.0))
    e_plain = rel_err(out, np.stack([oracle_decode_fp8(plain, b)[0] for b in range(w.batch)]))
    print(f"fp8 yarn decode: {e:.3e} (plain-RoPE oracle {e_plain:.3e})")
    assert e < TOL["bf16"] and e_plain > 10 * TOL["bf16"]
