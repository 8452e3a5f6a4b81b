"""Measurements of the board and of the 128-head decode kernel's tile loop (a measurement tool).

    python3 -m mla_latent_kv_24_amd.build --probe     # libmla_probe.so
    python3 -m mla_latent_kv_24_amd.probe phases      # the kernel's tile loop at v2_decode
    python3 -m mla_latent_kv_24_amd.probe read        # streaming-read ceiling
    python3 -m mla_latent_kv_24_amd.probe lds         # ds_read_b128 bytes per cycle per CU
    python3 -m mla_latent_kv_24_amd.probe mfma        # bf16 MFMA rate and clock on random operands
    python3 -m mla_latent_kv_24_amd.probe overlap     # does VALU work overlap MFMA work on a SIMD?
    python3 -m mla_latent_kv_24_amd.probe floor       # the V2 decode attention's bytes and products alone

The probe library is the product library built with MLA_PHASE_STAMPS: the
128-head kernel sums s_memtime cycles per phase of each tile step (the wait
for the tile and the first barrier; phase 1, the score products of tile t+1
with tile t's softmax; the second barrier; phase 2, the value products of
tile t) and stamps s_memrealtime (100 MHz) around its loop, and three probe
kernels (mla_probe.hip) are added.  Each subcommand prints one JSON line.
`phases` runs the decode step (append, absorb and combine from libmla.so, A3
from the probe library) for 2 s to settle the board's power state and reads
one more A3 launch.  The product never loads the probe library.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import time

import numpy as np
import torch

from . import api, workloads as W
from .build import PROBE_LIB

CUS = 256


def _lib():
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mla_probe_phase_stamps.argtypes = [vp]
    lib.mla_probe_read.argtypes = [vp, i64, vp, i32, vp]
    lib.mla_probe_lds.argtypes = [i32, vp, i32, vp]
    lib.mla_probe_mfma.argtypes = [i32, vp, vp, i32, vp]
    lib.mla_probe_overlap.argtypes = [i32, i32, i32, vp, vp, i32, vp]
    lib.mla_probe_floor.argtypes = [vp, i64, i32, vp, vp, i32, vp]
    for f in (lib.mla_probe_phase_stamps, lib.mla_probe_read, lib.mla_probe_lds, lib.mla_probe_mfma,
              lib.mla_probe_overlap, lib.mla_probe_floor):
        f.restype = ctypes.c_int
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _timed(launch, reps):
    """Mean milliseconds of `reps` launches after a 1 s settle of the same launch."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        launch()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def phases(lib, workload):
    from .pipeline import DecodeState
    fn = lib.mla_decode_partials
    fn.argtypes = api._lib.mla_decode_partials.argtypes
    fn.restype = api._lib.mla_decode_partials.restype
    w = W.WORKLOADS[workload]
    assert w.n_h == 128, "the stamps are in the 128-head kernel"
    st = DecodeState(W.make_decode_inputs(w))
    hi, lo = api._q(st.q_lat)

    def attention():
        r = fn(ctypes.byref(st.d), api.BF16, st.batch, hi, lo, st.cache.data_ptr(), st.stride,
               st.seq_lens.data_ptr(), st.max_len, st.splits, st.z_part.data_ptr(), st.lse_part.data_ptr(),
               torch.cuda.current_stream().cuda_stream)
        assert r == 0, r

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 2.0:
        for _ in range(20):
            st.append_new()
            st.absorb()
            attention()
            st.combine()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.append_new()
    st.absorb()
    e0.record()
    attention()
    e1.record()
    st.combine()
    torch.cuda.synchronize()
    buf = np.zeros(1024 * 4 * 8, dtype=np.uint64)
    assert lib.mla_probe_phase_stamps(buf.ctypes.data) == 0
    nwg = min(st.batch * st.splits, 1024)
    d = buf.reshape(1024, 4, 8)[:nwg].astype(np.float64)
    tiles = float(d[..., 6].mean())
    names = ["wait for the tile + barrier", "phase 1: score t+1, softmax t", "barrier", "phase 2: value t"]
    loop, ticks = float(d[..., 4].mean()), float(d[..., 5].mean())
    return {"probe": "phases", "workload": w.name, "workgroups": nwg, "tiles_per_workgroup": tiles,
            "a3_event_us": round(e0.elapsed_time(e1) * 1e3, 1),
            "cycles_per_tile_and_wave": {nm: round(float(d[..., k].mean()) / tiles, 1) for k, nm in enumerate(names)},
            "loop_to_end_cycles_per_wave": round(loop), "loop_to_end_us": round(ticks / 100.0, 1),
            "shader_clock_ghz": round(loop / (ticks * 10.0), 3)}


def read(lib):
    nbytes = 2 << 30
    src = torch.randint(0, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros(4 * CUS, dtype=torch.int32, device="cuda")
    out = {"probe": "read", "bytes": nbytes, "loads_in_flight_per_lane": 8}
    for per_cu in (1, 2, 4):
        wg = CUS * per_cu
        ms = _timed(lambda: lib.mla_probe_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                               ctypes.c_void_p(sink.data_ptr()), wg, _stream()), 10)
        out[f"tb_s_{per_cu}_workgroups_per_cu"] = round(nbytes / (ms * 1e-3) / 1e12, 3)
    return out


def lds(lib):
    iters = 4096
    out_t = torch.zeros(2 * CUS, dtype=torch.int64, device="cuda")
    _timed(lambda: lib.mla_probe_lds(iters, ctypes.c_void_p(out_t.data_ptr()), CUS, _stream()), 3)
    d = out_t.view(CUS, 2).cpu().numpy().astype(np.float64)
    bpc = d[:, 1] / d[:, 0]
    return {"probe": "lds", "instruction": "ds_read_b128, 64 lanes x 16 B consecutive", "workgroups": CUS,
            "bytes_per_cycle_per_cu_mean": round(float(bpc.mean()), 1), "min": round(float(bpc.min()), 1),
            "max": round(float(bpc.max()), 1)}


def mfma(lib):
    iters = 20000
    wg = CUS  # one workgroup of 4 waves per CU: one wave per SIMD
    out_t = torch.zeros(2 * wg, dtype=torch.int64, device="cuda")
    sink = torch.zeros(wg, dtype=torch.float32, device="cuda")
    ms = _timed(lambda: lib.mla_probe_mfma(iters, ctypes.c_void_p(out_t.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                           wg, _stream()), 5)
    d = out_t.view(wg, 2).cpu().numpy().astype(np.float64)
    flop = float(iters) * 4 * 32 * 32 * 16 * 2 * 4 * wg
    return {"probe": "mfma", "instruction": "v_mfma_f32_32x32x16_bf16, 4 chains per wave, random operands",
            "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "shader_clock_ghz": round(float((d[:, 0] / (d[:, 1] * 10.0)).mean()), 3),
            "cycles_per_mfma": round(float(d[:, 0].mean()) / (iters * 4), 2)}


def overlap(lib):
    """Cycles per iteration (8 MFMAs and/or 64 or 128 FMAs) of each wave, two waves per SIMD: each kind alone,
    split over the SIMD's two waves, and mixed in every wave.  MFMA and VALU overlap iff split/mixed take about
    the larger of the parts rather than their sum."""
    iters, wg = 2000, CUS  # 8 waves per workgroup, one workgroup per CU: two waves per SIMD
    out_t = torch.zeros(8 * wg, dtype=torch.int64, device="cuda")
    sink = torch.zeros(wg, dtype=torch.float32, device="cuda")
    res = {"probe": "overlap", "mfma": "v_mfma_f32_32x32x16_bf16", "valu": "v_fma_f32", "waves_per_simd": 2,
           "unit": "cycles per iteration of each wave (mean over waves 0-3 / 4-7)"}
    cases = [("both_waves_8_mfma", 2, 64), ("both_waves_64_fma", 3, 64), ("both_waves_128_fma", 3, 128),
             ("one_wave_8_mfma_other_64_fma", 1, 64), ("one_wave_8_mfma_other_128_fma", 1, 128),
             ("both_waves_8_mfma_and_64_fma", 0, 64), ("both_waves_8_mfma_and_128_fma", 0, 128)]
    for name, mode, nv in cases:
        _timed(lambda: lib.mla_probe_overlap(iters, mode, nv, ctypes.c_void_p(out_t.data_ptr()),
                                             ctypes.c_void_p(sink.data_ptr()), wg, _stream()), 3)
        d = out_t.view(wg, 8).cpu().numpy().astype(np.float64) / iters
        res[name] = [round(float(d[:, :4].mean()), 1), round(float(d[:, 4:].mean()), 1)]
    return res


def floor(lib):
    """The decode attention's work at v2_decode with nothing else: 256 workgroups (one per CU) stream 64 tiles
    of 36,864 B each (603,979,776 B, the cache of 64 sequences x 8,192 rows) and issue 68 bf16 32x32x16
    products per tile and wave (1.4603e11 FLOP, 2,176 x 128 per row).  Mode both / products alone / loads
    alone; each after a 1.5 s settle on its own load, timed back to back and after a 512 MB read that evicts
    the Infinity Cache (the attention kernel's roofline protocol)."""
    tiles, wg = 64, CUS
    nbytes = wg * tiles * 36864
    data = torch.randn(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    out_t = torch.zeros(2 * wg, dtype=torch.int64, device="cuda")
    sink = torch.zeros(wg, dtype=torch.float32, device="cuda")
    flush_buf = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    flush_sum = torch.zeros((), dtype=torch.float32, device="cuda")
    res = {"probe": "floor", "bytes": nbytes, "flop": 2176 * 128 * (nbytes // 1152), "workgroups": wg,
           "tiles_per_workgroup": tiles, "mfma_per_tile_and_wave": 68}
    for mode, name in ((0, "loads_and_products"), (1, "products_alone"), (2, "loads_alone")):
        def launch():
            assert lib.mla_probe_floor(ctypes.c_void_p(data.data_ptr()), tiles, mode, ctypes.c_void_p(out_t.data_ptr()),
                                       ctypes.c_void_p(sink.data_ptr()), wg, _stream()) == 0
        b2b = _timed(launch, 20) * 1e3
        d = out_t.view(wg, 2).cpu().numpy().astype(np.float64)
        ghz = float((d[:, 0] / (d[:, 1] * 10.0)).mean())
        ts = []
        for _ in range(20):
            torch.sum(flush_buf, dim=0, out=flush_sum)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.mean(ts))
        res[name] = {"us_flushed": round(us, 1), "us_back_to_back": round(b2b, 1), "shader_clock_ghz": round(ghz, 3),
                     "tb_s": round(nbytes / (us * 1e-6) / 1e12, 2) if mode != 1 else None,
                     "pflop_s": round(res["flop"] / (us * 1e-6) / 1e15, 3) if mode != 2 else None}
    return res


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["phases", "read", "lds", "mfma", "overlap", "floor"])
    ap.add_argument("--workload", default="v2_decode")
    args = ap.parse_args()
    lib = _lib()
    res = {"phases": lambda: phases(lib, args.workload), "read": lambda: read(lib), "lds": lambda: lds(lib),
           "mfma": lambda: mfma(lib), "overlap": lambda: overlap(lib), "floor": lambda: floor(lib)}[args.what]()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
