"""GPU parity of the projections around the path against the fp64 oracle:
the query path into A2 (W^DQ, RMSNorm, W^UQ / W^QR, absorption), the output
projection W^O, and one whole attention layer from hidden states (rows from
hidden states, the query path, decode, W^O).  Bar: max|gpu - ref| / rms(ref)
<= 2e-2, the bf16 bar; c^Q, q^C and the heads' outputs pass between
launches rounded once to bf16 (2^-9 relative each), q^R in fp32."""
import math

import numpy as np
import pytest

import oracle as O
from mla_latent_kv_24_amd import workloads as W
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    from mla_latent_kv_24_amd import api as A
    return A


def dev(a, dtype="bf16"):
    from mla_latent_kv_24_amd.pipeline import to_device
    return to_device(a, dtype)


def _query_weights(seed, n_h, d_model, d_cq):
    w_dq = W.random_storage(seed, (d_cq, d_model), "bf16", d_model ** -0.5)
    g_q = W.to_storage((1.0 + 0.25 * np.random.default_rng(seed + 1).standard_normal(d_cq)).astype(np.float32), "bf16")
    w_uq = W.random_storage(seed + 2, (n_h * 128, d_cq), "bf16", d_cq ** -0.5)
    w_qr = W.random_storage(seed + 3, (n_h * 64, d_cq), "bf16", d_cq ** -0.5)
    w_uk = W.random_storage(seed + 4, (n_h, 128, 512), "bf16", 512 ** -0.5)
    return w_dq, g_q, w_uq, w_qr, w_uk


# V2 (128 heads, hidden 5120, query latent 1536), 16 heads, a ragged token
# count, and shapes that take the generic kernels (d_model, d_cq not
# multiples of 128)
@pytest.mark.parametrize("n_h,n_q,d_model,d_cq", [(128, 64, 5120, 1536), (16, 37, 2048, 1536),
                                                   (128, 130, 5120, 1536), (16, 5, 200, 96)])
def test_absorb_q_from_hidden(api, n_h, n_q, d_model, d_cq):
    print(f"query path n_h={n_h} n_q={n_q} d_model={d_model} d_cq={d_cq}", flush=True)
    h = W.random_storage(70, (n_q, d_model), "bf16")
    w_dq, g_q, w_uq, w_qr, w_uk = _query_weights(71, n_h, d_model, d_cq)
    pos = W.random_ints(76, 0, 131072, n_q).astype(np.int32)
    d = api.dims(n_h)
    q_lat = api.q_lat_empty(d, torch.bfloat16, n_q)
    api.absorb_q_from_hidden(d, dev(h), dev(w_dq), dev(g_q), 1e-6, dev(w_uq), dev(w_qr), torch.from_numpy(pos).cuda(),
                             dev(w_uk), q_lat)
    got = api.q_lat_value(q_lat).cpu().numpy().astype(np.float64)
    q_c, q_r = O.query_from_hidden(f64(h, "bf16"), f64(w_dq, "bf16"), f64(w_uq, "bf16"), f64(w_qr, "bf16"), n_h,
                                   f64(g_q, "bf16"), 1e-6)
    ref = O.absorb_query(q_c, q_r, pos, f64(w_uk, "bf16"))
    e_lat, e_rope = rel_err(got[..., :512], ref[..., :512]), rel_err(got[..., 512:], ref[..., 512:])
    print(f"query path parity: latent part {e_lat:.3e}, RoPE part {e_rope:.3e}")
    assert e_lat < TOL["bf16"] and e_rope < TOL["bf16"]


@pytest.mark.parametrize("n_h,n_q,d_model", [(128, 64, 5120), (16, 33, 2048), (128, 3, 5120)])
def test_output_projection(api, n_h, n_q, d_model):
    print(f"output projection n_h={n_h} n_q={n_q} d_model={d_model}", flush=True)
    o = np.random.default_rng(80).standard_normal((n_q, n_h, 128)).astype(np.float32) * 0.1
    w_o = W.random_storage(81, (d_model, n_h * 128), "bf16", (n_h * 128) ** -0.5)
    d = api.dims(n_h)
    out = torch.empty((n_q, d_model), dtype=torch.float32, device="cuda")
    api.output_projection(d, torch.from_numpy(o).cuda(), dev(w_o), out)
    ref = O.output_projection(o.astype(np.float64), f64(w_o, "bf16"))
    e = rel_err(out.cpu().numpy(), ref)
    print(f"output projection parity: {e:.3e}")
    assert e < TOL["bf16"]


def test_attention_layer_from_hidden_states(api):
    """Hidden states in, layer output out: the cache rows and the queries made
    by the projections, decode over that cache, W^O -- against the oracle's
    chain on the same inputs (the cache as stored: both row halves rounded to
    bf16, reading of the storage dtype)."""
    n_h, d_model, d_cq, lens = 128, 5120, 1536, (300, 77)
    B, stride = len(lens), max(lens)
    d = api.dims(n_h)
    rng_seed = 90
    h_kv = W.random_storage(rng_seed, (sum(lens), d_model), "bf16")
    w_dkv = W.random_storage(rng_seed + 1, (512, d_model), "bf16", d_model ** -0.5)
    w_kr = W.random_storage(rng_seed + 2, (64, d_model), "bf16", d_model ** -0.5)
    g_kv = W.to_storage((1.0 + 0.25 * np.random.default_rng(rng_seed + 3).standard_normal(512)).astype(np.float32), "bf16")
    h_q = W.random_storage(rng_seed + 4, (B, d_model), "bf16")
    w_dq, g_q, w_uq, w_qr, w_uk = _query_weights(rng_seed + 5, n_h, d_model, d_cq)
    w_uv = W.random_storage(rng_seed + 10, (n_h, 128, 512), "bf16", 512 ** -0.5)
    w_o = W.random_storage(rng_seed + 11, (d_model, n_h * 128), "bf16", (n_h * 128) ** -0.5)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    rows = np.concatenate([b * stride + np.arange(L) for b, L in enumerate(lens)]).astype(np.int64)
    cache = torch.full((B * stride, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.append_kv_from_hidden(d, dev(h_kv), dev(w_dkv), dev(w_kr), dev(g_kv), 1e-6, torch.from_numpy(pos).cuda(),
                              torch.from_numpy(rows).cuda(), cache)
    q_pos = np.array([L - 1 for L in lens], dtype=np.int32)
    q_lat = api.q_lat_empty(d, torch.bfloat16, B)
    api.absorb_q_from_hidden(d, dev(h_q), dev(w_dq), dev(g_q), 1e-6, dev(w_uq), dev(w_qr),
                             torch.from_numpy(q_pos).cuda(), dev(w_uk), q_lat)
    o = torch.empty((B, n_h, 128), dtype=torch.float32, device="cuda")
    api.decode(d, q_lat, cache, stride, torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), dev(w_uv), o)
    u = torch.empty((B, d_model), dtype=torch.float32, device="cuda")
    api.output_projection(d, o, dev(w_o), u)
    got = u.cpu().numpy()
    # oracle chain
    c_all, k_all = O.kv_from_hidden(f64(h_kv, "bf16"), f64(w_dkv, "bf16"), f64(w_kr, "bf16"), f64(g_kv, "bf16"), 1e-6)
    q_c, q_r = O.query_from_hidden(f64(h_q, "bf16"), f64(w_dq, "bf16"), f64(w_uq, "bf16"), f64(w_qr, "bf16"), n_h,
                                   f64(g_q, "bf16"), 1e-6)
    outs, off = [], 0
    for b, L in enumerate(lens):
        c = O.round_to_storage(c_all[off:off + L], "bf16")
        k_rot = O.cached_rope_key(k_all[off:off + L], np.arange(L), 10000.0, store="bf16")
        ob, _ = O.attend_unabsorbed(q_c[b], O.rope(q_r[b], L - 1), c, k_rot, f64(w_uk, "bf16"), f64(w_uv, "bf16"))
        outs.append(ob)
        off += L
    ref = O.output_projection(np.stack(outs), f64(w_o, "bf16"))
    e = rel_err(got, ref)
    tol = TOL["bf16"]
    print(f"attention layer from hidden states: {e:.3e} (bar {tol})")
    assert np.all(np.isfinite(got)) and e < tol
