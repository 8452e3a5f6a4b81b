"""GPU parity: every step of the HIP path against the fp64 CPU oracle on the
same seeded inputs.  Tolerance: max|gpu - ref| / rms(ref) <= 2e-2 (bf16
storage) or 1e-4 (fp32 storage), as stated for this method's outputs."""
import math

import numpy as np
import pytest

import oracle as O
from mla_latent_kv_24_amd import workloads as W
from helpers import TOL, absorbed_layout, f64, oracle_decode, oracle_prefill, rel_err, to_np

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


# ---------------------------------------------------------------- A1 append
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_kv_rows(api, dtype):
    n, cap = 300, 1000
    c = W.random_storage(1, (n, 512), dtype)
    k = W.random_storage(2, (n, 64), dtype)
    pos = W.random_ints(3, 0, 131072, n).astype(np.int32)
    pos[:4] = [0, 1, 4095, 131071]
    rows = np.random.default_rng(4).permutation(cap)[:n].astype(np.int64)
    d = api.dims(16)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = torch.full((cap, 576), float("nan"), dtype=tdt, device="cuda")
    api.append_kv(d, dev(c, dtype), dev(k, dtype), torch.from_numpy(pos).cuda(),
                  torch.from_numpy(rows).cuda(), cache)
    got = to_np(cache)[rows]
    ref = O.append_rows(f64(c, dtype), f64(k, dtype), pos)
    # the latent half is a copy: bit exact
    assert np.array_equal(got[:, :512], c)
    g = f64(got[:, 512:], dtype)
    if dtype == "bf16":
        # fp32 rotation then one RNE rounding vs the exact value: within one bf16 ulp
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref[:, 512:]), 1e-30))) - 7)
        assert np.all(np.abs(g - ref[:, 512:]) <= ulp + 1e-30)
    else:
        assert np.max(np.abs(g - ref[:, 512:])) < 1e-5
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert np.all(np.isnan(f64(to_np(cache)[untouched], dtype)))


# ---------------------------------------------------------------- A2 absorb
@pytest.mark.parametrize("dtype,n_h,n_q", [("bf16", 16, 1), ("bf16", 16, 37), ("bf16", 128, 64),
                                           ("bf16", 128, 300), ("bf16", 8, 5), ("f32", 16, 9)])
def test_absorb_q(api, dtype, n_h, n_q):
    q_c = W.random_storage(10, (n_q, n_h, 128), dtype)
    q_r = W.random_storage(11, (n_q, n_h, 64), dtype)
    w_uk = W.random_storage(12, (n_h, 128, 512), dtype, 512 ** -0.5)
    pos = W.random_ints(13, 0, 131072, n_q).astype(np.int32)
    d = api.dims(n_h)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q_lat = api.q_lat_empty(d, tdt, n_q)
    api.absorb_q(d, dev(q_c, dtype), dev(q_r, dtype), torch.from_numpy(pos).cuda(), dev(w_uk, dtype), q_lat)
    got = api.q_lat_value(q_lat).cpu().numpy().astype(np.float64)
    ref = O.absorb_query(f64(q_c, dtype), f64(q_r, dtype), pos, f64(w_uk, dtype))
    # fp32 sums of 128 exact bf16 products and an fp32 RoPE rotation: within
    # 1e-5 of rms(ref).  The bf16 layout then carries each fp32 value v as
    # hi + lo with |hi + lo - v| <= 2^-9 |v - hi| <= 2^-17 |v| (two RNE
    # roundings), an elementwise term on top.
    rms = np.sqrt(np.mean(np.square(ref)))
    pair = 2.0 ** -17 * np.abs(ref) if dtype == "bf16" else 0.0
    assert np.all(np.abs(got - ref) <= 1e-5 * rms + pair * (1 + 2.0 ** -8))
    if dtype == "bf16":
        # layout: hi is the bf16 rounding of hi + lo, i.e. |lo| <= half an ulp of hi
        hi = q_lat.hi.float().cpu().numpy().astype(np.float64)
        lo = q_lat.lo.float().cpu().numpy().astype(np.float64)
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(hi), 1e-30))) - 8)
        assert np.all(np.abs(lo) <= half_ulp * (1 + 2.0 ** -7) + 1e-30)
        # without a lo plane the same hi plane, bit for bit (lo is not written)
        q_hi = api.q_lat_empty(d, tdt, n_q, lo=False)
        assert q_hi.lo is None
        api.absorb_q(d, dev(q_c, dtype), dev(q_r, dtype), torch.from_numpy(pos).cuda(), dev(w_uk, dtype), q_hi)
        assert torch.equal(q_hi.hi, q_lat.hi)


# ------------------------------------------- A1 + A2 in one call (one launch)
def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype,n_h,n_tok,n_q,lo", [
    ("bf16", 128, 64, 64, False),    # the V2 decode step: one row per sequence
    ("bf16", 128, 600, 3, True),     # more rows than the launch's 512 workgroups
    ("bf16", 16, 100, 37, True),     # 64 workgroups: several rows each
    ("bf16", 16, 32, 32, False),
    ("bf16", 128, 0, 7, True),       # empty halves
    ("bf16", 128, 5, 0, False),
    ("bf16", 8, 9, 5, True),         # no fused kernel: the two launches
    ("f32", 16, 9, 4, False)])
def test_append_absorb_matches_separate_calls(api, dtype, n_h, n_tok, n_q, lo):
    """mla_append_absorb writes the cache rows and absorbed queries of
    mla_append_kv followed by mla_absorb_q, bit for bit."""
    cap = 1000
    c = W.random_storage(51, (max(n_tok, 1), 512), dtype)[:n_tok]
    k = W.random_storage(52, (max(n_tok, 1), 64), dtype)[:n_tok]
    pos = W.random_ints(53, 0, 131072, max(n_tok, 1)).astype(np.int32)[:n_tok]
    rows = np.random.default_rng(54).permutation(cap)[:n_tok].astype(np.int64)
    q_c = W.random_storage(55, (max(n_q, 1), n_h, 128), dtype)[:n_q]
    q_r = W.random_storage(56, (max(n_q, 1), n_h, 64), dtype)[:n_q]
    qpos = W.random_ints(57, 0, 131072, max(n_q, 1)).astype(np.int32)[:n_q]
    w_uk = W.random_storage(58, (n_h, 128, 512), dtype, 512 ** -0.5)
    d = api.dims(n_h)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda a: dev(a, dtype)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    outs = []
    for fused in (False, True):
        cache = torch.full((cap, 576), float("nan"), dtype=tdt, device="cuda")
        q_lat = api.q_lat_empty(d, tdt, n_q, lo=lo)
        q_lat.hi.fill_(float("nan"))
        if q_lat.lo is not None:
            q_lat.lo.fill_(float("nan"))
        args = (t(c), t(k), i32(pos), i32(rows))
        if fused:
            api.append_absorb(d, *args, cache, t(q_c), t(q_r), i32(qpos), t(w_uk), q_lat)
        else:
            if n_tok:
                api.append_kv(d, *args, cache)
            if n_q:
                api.absorb_q(d, t(q_c), t(q_r), i32(qpos), t(w_uk), q_lat)
        torch.cuda.synchronize()
        outs.append((_bits(cache), _bits(q_lat.hi), None if q_lat.lo is None else _bits(q_lat.lo)))
    (c0, h0, l0), (c1, h1, l1) = outs
    assert np.array_equal(c0, c1)
    assert np.array_equal(h0, h1)
    assert (l0 is None and l1 is None) or np.array_equal(l0, l1)
    if n_tok:   # and the rows are the appended ones (the rest stays NaN)
        assert np.array_equal(c1[rows][:, :512], c.view(np.int16) if dtype == "bf16" else c.view(np.int32))


# ---------------------------------------------------- A3 split-KV partials
def _partials_case(api, dtype, n_h, lens, splits, stride=None, seed=20, tol=None):
    B = len(lens)
    max_len = int(max(lens))
    stride = stride or max_len + 5
    q32 = W.random_storage(seed, (B, n_h, 576), "f32", 0.06)
    q_hi, q_lo, q_lat = absorbed_layout(q32, dtype)     # device planes, and the value they carry
    q_in = api.QLat(dev(q_hi, dtype), None if q_lo is None else dev(q_lo, dtype))
    rows = W.random_storage(seed + 1, (B, stride, 576), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache_np = rows.copy()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    for b, L in enumerate(lens):
        cache_np[b, L:] = nan                       # poison past each length
    cache = dev(cache_np.reshape(B * stride, 576), dtype)
    # NaN everywhere first: a unit that no workgroup computed shows up
    z = torch.full((B, splits, n_h, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, splits, n_h), float("nan"), dtype=torch.float32, device="cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    api.decode_partials(api.dims(n_h), q_in, cache, stride, seq, max_len, splits, z, lse)
    torch.cuda.synchronize()
    R = api.split_rows(max_len, splits)
    scale = 1.0 / math.sqrt(192.0)
    zg, lg = z.cpu().numpy(), lse.cpu().numpy()
    for b, L in enumerate(lens):
        Zr, lr = O.split_partials(q_lat[b].astype(np.float64), f64(rows[b], dtype), L, R, splits, scale)
        for s in range(splits):
            if np.isneginf(lr[s]).all():
                assert np.all(np.isneginf(lg[b, s])) and np.all(zg[b, s] == 0)
                continue
            assert np.all(np.isfinite(zg[b, s]))
            assert np.max(np.abs(lg[b, s] - lr[s])) < (2e-3 if dtype == "bf16" else 1e-5)
            bar = tol(L) if callable(tol) else (tol or TOL[dtype])
            assert rel_err(zg[b, s], Zr[s]) < bar, (b, L, s, rel_err(zg[b, s], Zr[s]))
    return zg, lg


@pytest.mark.parametrize("n_h", [16, 32, 64, 128, 8])
def test_splitkv_partials_bf16(api, n_h):
    _partials_case(api, "bf16", n_h, [1, 37, 500, 64], 3)


@pytest.mark.parametrize("splits", [1, 2, 7, 16])
def test_splitkv_partials_split_counts(api, splits):
    _partials_case(api, "bf16", 128, [33, 300, 1000], splits, seed=30 + splits)


@pytest.mark.parametrize("n_h,lens,splits", [(128, [4100, 4500, 5000], 2), (128, [50, 4100, 300, 5000], 3),
                                             (64, [4096, 70, 4200], 2), (32, [5000, 1], 4)])
def test_splitkv_partials_wide_and_mixed(api, n_h, lens, splits):
    """32 to 128 heads over queries of 4,096 rows or more (the wide kernels'
    single-bf16 path) and mixed with short ones (the same launch runs their
    16-head groups with hi + lo products).  Short queries' partials match the
    oracle to 1e-4; long ones to the bf16 bar."""
    assert api.precise_rows(api.dims(n_h), api.BF16) == 4096
    _partials_case(api, "bf16", n_h, lens, splits, seed=60 + n_h,
                   tol=lambda L: 1e-4 if L < 4096 else TOL["bf16"])


@pytest.mark.parametrize("n_h", [16, 128])
def test_longest_first_order_covers_every_unit(api, n_h):
    """A decode launch of more workgroups than compute units (40 queries x 8
    splits, x 8 head groups at 128 heads) takes its (query, split) units
    longest first: full splits, partial ones by length class, empty ones.
    Lengths hit every kind: 0, 1, exact multiples of the 256-row split, one
    row past one, the maximum, and random ones.  Every unit is computed exactly
    once: all partials (NaN-filled before) match the oracle."""
    rng = np.random.default_rng(70 + n_h)
    lens = [0, 1, 256, 257, 512, 2000, 1999, 255, 768, 1024] + rng.integers(1, 2001, 30).tolist()
    assert api.split_rows(2000, 8) == 256
    _partials_case(api, "bf16", n_h, lens, 8, seed=71 + n_h, tol=lambda L: 1e-4)


def test_splitkv_partials_f32(api):
    _partials_case(api, "f32", 16, [5, 300], 2)


@pytest.mark.parametrize("n_h,dtype", [(128, "bf16"), (16, "bf16"), (32, "bf16"), (8, "bf16"), (16, "f32")])
def test_decode_empty_sequences(api, n_h, dtype):
    """Sequences of length 0 inside a batch (every kernel family): all their
    splits are empty (lse = -inf, z = 0); the combine then gives them z = 0 and
    out = 0, while the other sequences meet the oracle."""
    zg, lg = _partials_case(api, dtype, n_h, [0, 37, 0, 500], 3, seed=50)
    assert np.all(np.isneginf(lg[[0, 2]])) and np.all(zg[[0, 2]] == 0)
    w_uv = W.random_storage(51, (n_h, 128, 512), dtype, 512 ** -0.5)
    out = torch.full((4, n_h, 128), float("nan"), dtype=torch.float32, device="cuda")
    lat = torch.full((4, n_h, 512), float("nan"), dtype=torch.float32, device="cuda")
    api.combine_project(api.dims(n_h), torch.from_numpy(zg).cuda(), torch.from_numpy(lg).cuda(),
                        dev(w_uv, dtype), out, lat)
    o, z = out.cpu().numpy(), lat.cpu().numpy()
    assert np.all(o[[0, 2]] == 0) and np.all(z[[0, 2]] == 0)
    for n in (1, 3):
        z_ref = O.combine_partials(zg[n].astype(np.float64), lg[n].astype(np.float64))[0]
        assert rel_err(z[n], z_ref) < 1e-5
        assert rel_err(o[n], O.project_uv(z_ref, f64(w_uv, dtype))) < 1e-4


@pytest.mark.parametrize("name,n_h,opts", [("v2_decode", 128, {}), ("lite_ragged", 16, {}),
                                           ("v2_decode", 128, dict(fp8=True)), ("lite_ragged", 16, dict(fp8=True)),
                                           ("v2_decode", 128, dict(page_rows=64)),
                                           ("lite_ragged", 16, dict(page_rows=32))])
def test_decode_zero_length_on_device(pipeline, name, n_h, opts):
    """A device-side length set to 0 after the split plan is fixed (the FP8
    and paged caches included): that sequence's output and latent are exactly
    0, the others are bitwise what they were."""
    w = W.scaled(W.WORKLOADS[name], batch=4, seq_len=900, n_h=n_h)
    st = pipeline.DecodeState(W.make_decode_inputs(w), out_latent=True, **opts)
    print(f"zero length {name} {opts}", flush=True)
    st.absorb()
    st.attention()
    st.combine()
    out0, lat0 = st.out.clone(), st.out_latent.clone()
    st.seq_lens[2] = 0
    st.attention()
    st.combine()
    torch.cuda.synchronize()
    assert torch.all(st.out[2] == 0) and torch.all(st.out_latent[2] == 0)
    keep = [0, 1, 3]
    assert torch.equal(st.out[keep], out0[keep]) and torch.equal(st.out_latent[keep], lat0[keep])


# ------------------------------------------------------ A4 + A5 combine/lift
@pytest.mark.parametrize("dtype,n_h,S,n_q", [("bf16", 128, 4, 45), ("bf16", 16, 1, 45), ("bf16", 16, 64, 45),
                                             ("f32", 16, 3, 45), ("bf16", 128, 64, 4), ("bf16", 128, 5, 45),
                                             ("bf16", 128, 17, 33), ("bf16", 16, 16, 32),
                                             # 21 blocks of 32 queries, two per workgroup (the last
                                             # workgroup takes one, the last block 10 queries)
                                             ("bf16", 128, 1, 650), ("bf16", 128, 2, 650)])
def test_combine_project(api, dtype, n_h, S, n_q):
    Z = np.random.default_rng(40).standard_normal((n_q, S, n_h, 512)).astype(np.float32)
    lse = (np.random.default_rng(41).standard_normal((n_q, S, n_h)) * 3).astype(np.float32)
    if S > 1:
        lse[::3, -1] = -np.inf
        Z[::3, -1] = 0.0
    w_uv = W.random_storage(42, (n_h, 128, 512), dtype, 512 ** -0.5)
    out = torch.empty((n_q, n_h, 128), dtype=torch.float32, device="cuda")
    lat = torch.empty((n_q, n_h, 512), dtype=torch.float32, device="cuda")
    api.combine_project(api.dims(n_h), torch.from_numpy(Z).cuda(), torch.from_numpy(lse).cuda(),
                        dev(w_uv, dtype), out, lat)
    z_ref = np.stack([O.combine_partials(Z[n].astype(np.float64), lse[n].astype(np.float64))[0]
                      for n in range(n_q)])
    o_ref = O.project_uv(z_ref, f64(w_uv, dtype))
    assert rel_err(lat.cpu().numpy(), z_ref) < 1e-5
    assert rel_err(out.cpu().numpy(), o_ref) < 1e-4


# --------------------------------------------------------- end-to-end decode
SMALL = [
    ("tiny_f32", {}),
    ("lite_decode", dict(batch=3, seq_len=777)),
    ("lite_ragged", dict(batch=6, seq_len=3000)),
    ("v2_decode", dict(batch=2, seq_len=1000)),
    ("v2_long", dict(batch=1, seq_len=4099)),
    ("v2_decode", dict(batch=5, seq_len=65)),
    ("v2_decode", dict(batch=3, seq_len=4200, ragged=True)),
]


@pytest.mark.parametrize("name,changes", SMALL, ids=[f"{s[0]}-{i}" for i, s in enumerate(SMALL)])
def test_decode_small(pipeline, name, changes):
    w = W.scaled(W.WORKLOADS[name], **changes)
    inp = W.make_decode_inputs(w)
    st = pipeline.DecodeState(inp, out_latent=True)
    st.absorb()
    st.attention()
    st.combine()
    out = st.out.cpu().numpy()
    lat = st.out_latent.cpu().numpy()
    assert np.all(np.isfinite(out))
    refs = [oracle_decode(inp, b) for b in range(w.batch)]
    o_ref = np.stack([r[0] for r in refs])
    z_ref = np.stack([r[1] for r in refs])
    assert rel_err(out, o_ref) < TOL[w.dtype], name
    assert rel_err(lat, z_ref) < TOL[w.dtype], name


@pytest.mark.parametrize("max_len", [4096, 12000])
def test_decode_ragged_128_heads(pipeline, max_len):
    """128 heads, lengths uniform in [1, max_len]: short sequences' outputs are
    several times the batch rms, so every rounding of theirs shows in the
    whole-tensor metric.  Every sequence against the oracle's absorbed form
    (pinned equal to the definition), the shortest and the longest against
    the definition itself, all over the whole tensor's rms; at 12,000 rows the
    launch mixes both 128-head paths."""
    w = W.scaled(W.WORKLOADS["v2_decode"], batch=16, seq_len=max_len, ragged=True, seed=3)
    inp = W.make_decode_inputs(w)
    print(f"ragged 128 heads, lengths {sorted(inp.seq_lens.tolist())}", flush=True)
    st = pipeline.DecodeState(inp, out_latent=True)
    st.absorb()
    st.attention()
    st.combine()
    out, lat = st.out.cpu().numpy(), st.out_latent.cpu().numpy()
    refs = [oracle_decode(inp, b, absorbed=True) for b in range(w.batch)]
    o_ref, z_ref = np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs])
    assert rel_err(out, o_ref) < TOL["bf16"] and rel_err(lat, z_ref) < TOL["bf16"]
    rms = np.sqrt(np.mean(np.square(o_ref)))
    for b in (int(np.argmin(inp.seq_lens)), int(np.argmax(inp.seq_lens))):
        o_def, _ = oracle_decode(inp, b)
        assert np.max(np.abs(out[b] - o_def)) / rms < TOL["bf16"], b


def test_absent_lo_plane_reads_as_zero(api, pipeline):
    """Without the lo plane the precise path scores with hi alone: bitwise the
    result of a lo plane of zeros (short queries, 128 heads)."""
    w = W.scaled(W.WORKLOADS["v2_decode"], batch=3, seq_len=500)
    st = pipeline.DecodeState(W.make_decode_inputs(w), out_latent=True)
    st.absorb()
    outs = []
    for lo in (None, torch.zeros_like(st.q_lat.hi)):
        out, lat = torch.empty_like(st.out), torch.empty_like(st.out_latent)
        api.decode(st.d, api.QLat(st.q_lat.hi, lo), st.cache, st.stride, st.seq_lens, st.max_len, st.w_uv, out, lat)
        outs.append((out, lat))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_decode_is_deterministic_and_split_invariant(pipeline):
    w = W.scaled(W.WORKLOADS["v2_decode"], batch=3, seq_len=2000)
    st = pipeline.DecodeState(W.make_decode_inputs(w))
    st.absorb()
    st.attention()
    st.combine()
    a = st.out.clone()
    st.attention()
    st.combine()
    assert torch.equal(a, st.out)                         # bitwise determinism
    outs = []
    for S in (1, 2, 7, 16):
        z = torch.empty((3, S, 128, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((3, S, 128), dtype=torch.float32, device="cuda")
        st.attention(S, z, lse)
        st.combine(z, lse)
        outs.append(st.out.cpu().numpy())
    for o in outs[1:]:
        assert rel_err(o, outs[0]) < 1e-2


@pytest.mark.parametrize("name", ["v2_decode", "lite_ragged"])
def test_fused_decode_equals_partials_then_combine(api, pipeline, name):
    """mla_decode (A3 + A4 + A5 in one call, partials in the caller's workspace)
    gives bitwise the result of the separate calls under the same split plan."""
    w = W.scaled(W.WORKLOADS[name], batch=5, seq_len=1500)
    st = pipeline.DecodeState(W.make_decode_inputs(w), out_latent=True)
    st.absorb()
    st.attention()
    st.combine()
    torch.cuda.synchronize()
    out = torch.empty_like(st.out)
    lat = torch.empty_like(st.out_latent)
    api.decode(st.d, st.q_lat, st.cache, st.stride, st.seq_lens, st.max_len, st.w_uv, out, lat)
    torch.cuda.synchronize()
    assert torch.equal(out, st.out) and torch.equal(lat, st.out_latent)


def test_prefill_two_sequences(api, pipeline):
    """One mla_prefill call over two sequences with different prefix lengths
    (sequence slots of a shared cache), each against the oracle."""
    C, prefixes, n_h, dtype = 40, (70, 5), 128, "bf16"
    pinps = [W.make_prefill_inputs(W.scaled(W.WORKLOADS["v2_prefill"], seq_len=p + C, prefill_chunk=C,
                                            seed=7 + b)) for b, p in enumerate(prefixes)]
    w_uk, w_uv = pinps[0].w_uk, pinps[0].w_uv          # one layer: shared weights
    stride = max(prefixes) + C + 3
    d = api.dims(n_h)
    cache = torch.full((2 * stride, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b, pi in enumerate(pinps):
        tot = pi.prefix + pi.chunk
        api.append_kv(d, dev(pi.c_kv, dtype), dev(pi.k_raw, dtype),
                      torch.arange(tot, dtype=torch.int32, device="cuda"),
                      torch.arange(tot, dtype=torch.int64, device="cuda") + b * stride, cache)
    q_c = np.concatenate([pi.q_c for pi in pinps])
    q_r = np.concatenate([pi.q_r for pi in pinps])
    q_pos = np.concatenate([np.arange(p, p + C) for p in prefixes]).astype(np.int32)
    q_lat = api.q_lat_empty(d, torch.bfloat16, 2, C)
    api.absorb_q(d, dev(q_c, dtype), dev(q_r, dtype), torch.from_numpy(q_pos).cuda(), dev(w_uk, dtype),
                 q_lat.view(2 * C, n_h, 576))
    out = torch.empty((2, C, n_h, 128), dtype=torch.float32, device="cuda")
    plen = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    api.prefill(d, q_lat, cache, stride, plen, max(prefixes), dev(w_uv, dtype), out)
    got = out.cpu().numpy()
    for b, pi in enumerate(pinps):
        ref = O.prefill(f64(pi.q_c, dtype), f64(pi.q_r, dtype), pi.prefix, f64(pi.c_kv, dtype),
                        f64(pi.k_raw, dtype), f64(w_uk, dtype), f64(w_uv, dtype), pi.w.rope_base,
                        store=dtype)
        assert np.all(np.isfinite(got[b]))
        assert rel_err(got[b], ref) < TOL["bf16"]


@pytest.mark.parametrize("name", ["v2_decode", "lite_decode"])
def test_step_graph_replay(pipeline, name):
    """The decode step captured as a HIP graph reproduces the eager step bitwise
    on every replay, with eager kernels and synchronisations between replays."""
    w = W.scaled(W.WORKLOADS[name], batch=3, seq_len=700)
    st = pipeline.DecodeState(W.make_decode_inputs(w), out_latent=True)
    st.step()
    torch.cuda.synchronize()
    ref, ref_lat = st.out.clone(), st.out_latent.clone()
    g = st.capture()
    for _ in range(3):
        st.out.zero_()
        st.out_latent.zero_()
        st.absorb()                      # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref) and torch.equal(st.out_latent, ref_lat)


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 63, 64, 65, 97, 4097])
def test_decode_tile_edges(pipeline, T):
    w = W.scaled(W.WORKLOADS["v2_decode"], batch=1, seq_len=T)
    inp = W.make_decode_inputs(w)
    st = pipeline.DecodeState(inp)
    st.absorb()
    st.attention()
    st.combine()
    o_ref, _ = oracle_decode(inp, 0)
    assert rel_err(st.out.cpu().numpy()[0], o_ref) < TOL["bf16"]
    if T == 1:
        # closed form: a single row gives U^V c_0 for every head
        c0 = f64(inp.c_kv[0, 0], "bf16")
        expect = np.einsum("hdc,c->hd", f64(inp.w_uv, "bf16"), c0)
        assert rel_err(st.out.cpu().numpy()[0], expect) < 1e-3


def test_poison_past_length_is_never_read(pipeline):
    """NaN rows past each length vs. zero rows there: identical outputs, bit for bit."""
    w = W.scaled(W.WORKLOADS["lite_ragged"], batch=8, seq_len=700)
    inp_nan = W.make_decode_inputs(w, poison=True)
    inp_zero = W.make_decode_inputs(w, poison=False)
    outs = []
    for inp in (inp_nan, inp_zero):
        st = pipeline.DecodeState(inp)
        if inp is inp_zero:
            st.cache.zero_()
            st.fill_cache()
        st.absorb()
        st.attention()
        st.combine()
        outs.append(st.out.cpu())
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])


# ----------------------------------------------------------------- prefill
@pytest.mark.parametrize("n_h,prefix,chunk", [(16, 40, 70), (128, 0, 33), (128, 100, 65), (128, 300, 40),
                                              (128, 2000, 65), (128, 4060, 70)])
def test_prefill_small(pipeline, n_h, prefix, chunk):
    """Causal prefill against the oracle at the bf16 bar; at 128 heads the
    chunk over 4,060..4,129 rows straddles the precise-path threshold."""
    tol = TOL["bf16"]
    base = W.WORKLOADS["v2_prefill"] if n_h == 128 else W.scaled(W.WORKLOADS["lite_decode"], batch=1)
    w = W.scaled(base, seq_len=prefix + chunk, prefill_chunk=chunk, batch=1)
    pinp = W.make_prefill_inputs(w)
    st = pipeline.PrefillState(pinp)
    st.step()
    got = st.out.cpu().numpy()[0]
    ref = oracle_prefill(pinp, range(chunk))
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) < tol


def test_prefill_causal_rows(pipeline):
    """Rewriting row j changes exactly the queries at positions >= j, bit for bit."""
    w = W.scaled(W.WORKLOADS["v2_prefill"], seq_len=160, prefill_chunk=96)
    pinp = W.make_prefill_inputs(w)
    st = pipeline.PrefillState(pinp)
    st.step()
    before = st.out.clone()
    j = 64 + 40                                    # inside the chunk
    new_c = dev(W.random_storage(99, (1, 512), "bf16"), "bf16")
    new_k = dev(W.random_storage(98, (1, 64), "bf16"), "bf16")
    from mla_latent_kv_24_amd import api as A
    A.append_kv(st.d, new_c, new_k, torch.tensor([j], dtype=torch.int32, device="cuda"),
                torch.tensor([j], dtype=torch.int64, device="cuda"), st.cache)
    st.attend()
    after = st.out
    for i in range(96):
        same = torch.equal(before[0, i], after[0, i])
        assert same == (64 + i < j), i


# ------------------------------------------------- prefill, unabsorbed form
# Shapes cover: both precisions (a workgroup of 256 queries takes hi + lo
# products when its first query sees fewer than 2,048 keys), a chunk whose
# query blocks straddle that threshold, ragged last tiles and query blocks,
# and 16 heads.  The bar is the plain 2e-2 at every length.
@pytest.mark.parametrize("n_h,prefix,chunk", [(128, 0, 33), (128, 100, 65), (128, 2000, 65), (128, 2100, 300),
                                              (128, 1900, 600), (16, 40, 70), (16, 3000, 257)])
def test_prefill_unabsorbed(pipeline, n_h, prefix, chunk):
    base = W.WORKLOADS["v2_prefill"] if n_h == 128 else W.scaled(W.WORKLOADS["lite_decode"], batch=1)
    w = W.scaled(base, seq_len=prefix + chunk, prefill_chunk=chunk, batch=1)
    pinp = W.make_prefill_inputs(w)
    st = pipeline.PrefillState(pinp)
    st.append_all()
    st.attend_unabsorbed()
    got = st.out.cpu().numpy()[0]
    queries = range(chunk) if chunk <= 80 else sorted({0, 1, 31, 32, 63, 64, 255, 256, chunk // 2, chunk - 1})
    heads = None if n_h == 16 else [0, 1, 37, 64, 127]
    ref = oracle_prefill(pinp, list(queries), heads)
    g = got[list(queries)] if heads is None else got[list(queries)][:, heads]
    assert np.all(np.isfinite(got))
    assert rel_err(g, ref) < TOL["bf16"], (n_h, prefix, chunk, rel_err(g, ref))


def test_prefill_unabsorbed_two_sequences(api):
    """One call over two sequences with different prefixes (slots of a shared
    cache, shared weights), each against the oracle at the plain bar."""
    C, prefixes, n_h, dtype = 40, (70, 5), 128, "bf16"
    pinps = [W.make_prefill_inputs(W.scaled(W.WORKLOADS["v2_prefill"], seq_len=p + C, prefill_chunk=C,
                                            seed=7 + b)) for b, p in enumerate(prefixes)]
    w_uk, w_uv = pinps[0].w_uk, pinps[0].w_uv
    stride = max(prefixes) + C + 3
    d = api.dims(n_h)
    cache = torch.full((2 * stride, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b, pi in enumerate(pinps):
        tot = pi.prefix + pi.chunk
        api.append_kv(d, dev(pi.c_kv, dtype), dev(pi.k_raw, dtype),
                      torch.arange(tot, dtype=torch.int32, device="cuda"),
                      torch.arange(tot, dtype=torch.int64, device="cuda") + b * stride, cache)
    q_c = dev(np.stack([pi.q_c for pi in pinps]), dtype)
    q_r = dev(np.stack([pi.q_r for pi in pinps]), dtype)
    out = torch.empty((2, C, n_h, 128), dtype=torch.float32, device="cuda")
    plen = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    api.prefill_unabsorbed(d, q_c, q_r, cache, stride, plen, max(prefixes), dev(w_uk, dtype), dev(w_uv, dtype), out)
    got = out.cpu().numpy()
    for b, pi in enumerate(pinps):
        ref = O.prefill(f64(pi.q_c, dtype), f64(pi.q_r, dtype), pi.prefix, f64(pi.c_kv, dtype),
                        f64(pi.k_raw, dtype), f64(w_uk, dtype), f64(w_uv, dtype), pi.w.rope_base,
                        store=dtype)
        assert np.all(np.isfinite(got[b]))
        assert rel_err(got[b], ref) < TOL["bf16"]


# The expansion gives a workgroup 8, 16 or 32 heads (as many as still leave
# 256 workgroups) and maps workgroups to XCDs by head range.  The small shapes
# above take 8 heads and the full v2_prefill 32; these batches take 16 (batch
# 2, 16 row blocks) and 32 over an odd count of row blocks (batch 4, 17 row
# blocks: the plain mapping), with prefixes on both sides of the hi + lo
# threshold's row range.
@pytest.mark.parametrize("prefixes", [(1800, 1750), (1800, 1750, 1900, 1650)])
def test_prefill_unabsorbed_head_ranges(api, prefixes):
    import dataclasses
    C, n_h, dtype = 200, 128, "bf16"
    pinps = [W.make_prefill_inputs(W.scaled(W.WORKLOADS["v2_prefill"], seq_len=p + C, prefill_chunk=C,
                                            seed=11 + b)) for b, p in enumerate(prefixes)]
    w_uk, w_uv = pinps[0].w_uk, pinps[0].w_uv
    pinps = [dataclasses.replace(pi, w_uk=w_uk, w_uv=w_uv) for pi in pinps]
    stride = max(prefixes) + C
    d = api.dims(n_h)
    cache = torch.full((len(prefixes) * stride, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b, pi in enumerate(pinps):
        tot = pi.prefix + pi.chunk
        api.append_kv(d, dev(pi.c_kv, dtype), dev(pi.k_raw, dtype),
                      torch.arange(tot, dtype=torch.int32, device="cuda"),
                      torch.arange(tot, dtype=torch.int64, device="cuda") + b * stride, cache)
    q_c = dev(np.stack([pi.q_c for pi in pinps]), dtype)
    q_r = dev(np.stack([pi.q_r for pi in pinps]), dtype)
    out = torch.empty((len(prefixes), C, n_h, 128), dtype=torch.float32, device="cuda")
    plen = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    api.prefill_unabsorbed(d, q_c, q_r, cache, stride, plen, max(prefixes), dev(w_uk, dtype), dev(w_uv, dtype), out)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    queries, heads = [0, 1, 63, 100, C - 1], [0, 7, 8, 15, 16, 31, 64, 127]
    for b, pi in enumerate(pinps):
        ref = oracle_prefill(pi, queries, heads)
        g = got[b][queries][:, heads]
        assert rel_err(g, ref) < TOL["bf16"], (prefixes, b, rel_err(g, ref))


# ------------------------------------------------------- long-context RoPE
YARN = dict(yarn_factor=40.0)            # DeepSeek-V2's scale over 4,096 pretraining positions
# YaRN's temperature multiplies every logit by (0.1 ln 40 + 1)^2 = 1.87 and
# sharpens the softmax so that a few heads' outputs are ~20x the tensor's rms;
# the library then takes hi + lo products for every query (both prefill
# forms included), and every output is held to the plain bf16 bar against the
# oracle alone.


def test_yarn_rows_and_absorbed_queries(api):
    """A1's RoPE key and A2's absorbed query with the long-context frequencies,
    element by element, at the bars of the plain-RoPE tests (positions up to
    160K, where the interpolated pairs matter)."""
    n, n_h = 200, 128
    c = W.random_storage(41, (n, 512), "bf16")
    k = W.random_storage(42, (n, 64), "bf16")
    pos = W.random_ints(43, 0, 163840, n).astype(np.int32)
    pos[:3] = [0, 4095, 163839]
    d = api.dims(n_h, **YARN)
    freq = O.yarn_frequencies(64, 10000.0, 40.0)
    cache = torch.full((n, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    api.append_kv(d, dev(c, "bf16"), dev(k, "bf16"), torch.from_numpy(pos).cuda(),
                  torch.arange(n, dtype=torch.int64, device="cuda"), cache)
    g = f64(to_np(cache)[:, 512:], "bf16")
    ref = O.cached_rope_key(f64(k, "bf16"), pos, freq)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(g - ref) <= ulp + 1e-30)
    assert np.max(np.abs(g - O.cached_rope_key(f64(k, "bf16"), pos))) > 0.5   # not the plain frequencies
    q_c = W.random_storage(44, (n, n_h, 128), "bf16")
    q_r = W.random_storage(45, (n, n_h, 64), "bf16")
    w_uk = W.random_storage(46, (n_h, 128, 512), "bf16", 512 ** -0.5)
    q_lat = api.q_lat_empty(d, torch.bfloat16, n)
    api.absorb_q(d, dev(q_c, "bf16"), dev(q_r, "bf16"), torch.from_numpy(pos).cuda(), dev(w_uk, "bf16"), q_lat)
    got = api.q_lat_value(q_lat).cpu().numpy().astype(np.float64)
    ref = O.absorb_query(f64(q_c, "bf16"), f64(q_r, "bf16"), pos, f64(w_uk, "bf16"), freq)
    rms = np.sqrt(np.mean(np.square(ref)))
    assert np.all(np.abs(got - ref) <= 1e-5 * rms + 2.0 ** -17 * np.abs(ref) * (1 + 2.0 ** -8))


@pytest.mark.parametrize("n_h", [128, 16])
def test_yarn_decode_and_prefill(pipeline, n_h):
    """Decode and causal prefill (absorbed and unabsorbed) with the
    long-context RoPE (frequencies and temperature), end to end through
    append, absorption and attention, against the oracle at the bf16 bar.  The
    plain-RoPE oracle misses by many times the bar (the fields are honoured)."""
    base = W.WORKLOADS["v2_decode"] if n_h == 128 else W.WORKLOADS["lite_decode"]
    w = W.scaled(base, batch=2, seq_len=6000, **YARN)
    inp = W.make_decode_inputs(w)
    print(f"yarn decode n_h={n_h}", flush=True)
    st = pipeline.DecodeState(inp, out_latent=True)
    assert st.q_lat.lo is not None                 # every query reads the lo plane under YaRN
    st.absorb()
    st.attention()
    st.combine()
    out, lat = st.out.cpu().numpy(), st.out_latent.cpu().numpy()
    refs = [oracle_decode(inp, b, absorbed=True) for b in range(w.batch)]
    exact, z_exact = np.stack([r[0] for r in refs]), np.stack([r[1] for r in refs])
    plain = W.make_decode_inputs(W.scaled(w, yarn_factor=0.0))
    e_plain = rel_err(out, np.stack([oracle_decode(plain, b, absorbed=True)[0] for b in range(w.batch)]))
    e, e_z = rel_err(out, exact), rel_err(lat, z_exact)
    print(f"yarn decode: out {e:.3e}, latent {e_z:.3e}; plain-RoPE oracle {e_plain:.3e}", flush=True)
    assert e < TOL["bf16"] and e_z < TOL["bf16"]
    assert e_plain > 5 * TOL["bf16"]
    o_def, _ = oracle_decode(inp, 0, heads=[0, 63, 127] if n_h == 128 else None)
    h = [0, 63, 127] if n_h == 128 else slice(None)
    assert np.max(np.abs(out[0][h] - o_def)) / np.sqrt(np.mean(np.square(exact))) < TOL["bf16"]

    pbase = W.WORKLOADS["v2_prefill"] if n_h == 128 else W.scaled(W.WORKLOADS["lite_decode"], batch=1)
    prefix, chunk = 5000, 65
    pw = W.scaled(pbase, seq_len=prefix + chunk, prefill_chunk=chunk, batch=1, **YARN)
    pinp = W.make_prefill_inputs(pw)
    heads = None if n_h == 16 else [0, 37, 127]
    exact = oracle_prefill(pinp, range(chunk), heads)
    pst = pipeline.PrefillState(pinp)
    pst.step()
    got = pst.out.cpu().numpy()[0]
    pst.attend_unabsorbed()
    got_u = pst.out.cpu().numpy()[0]
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_u))
    sel = (lambda x: x) if heads is None else (lambda x: x[:, heads])
    e_a, e_u = rel_err(sel(got), exact), rel_err(sel(got_u), exact)
    print(f"yarn prefill: absorbed {e_a:.3e}, unabsorbed {e_u:.3e}", flush=True)
    assert e_a < TOL["bf16"] and e_u < TOL["bf16"]
