#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X; prints ONE JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
  prefill  the four Qwen3-8B-like layers at M = 8192 tokens, each
           quantize_nvfp4(X bf16) -> gemm_w4a4(-> Y bf16)     (quantize is timed)
  decode   the same four layer shapes, W4A16 (INT4 group-128) at M = 16
  decode   the three Gemma3-12B-like layers, LUT2 at M = 8
Inputs and packed weights are resident in HBM before the timed region.

value = the step's algorithmic FLOPs / ms_per_step (TFLOP/s); the prefill
FLOPs dominate (decode adds < 0.3 %).  ``parts`` breaks the step down with HIP
events (torch.cuda.Event on the stream every kernel is launched on):
per-layer quantize and GEMM times, the GEMM-only TFLOP/s as fractions of the
fp16 (the dtype the MFMAs run), FP8 and FP4 dense peaks, and a separate
decode sweep (all batch sizes) that rotates through > 512 MiB of weight copies
so the 256 MiB Infinity Cache cannot serve repeats.

``roofline`` describes the dominant kernel (gemm_w4a4); ``cpu_baseline`` times
the CPU oracle (test infrastructure) on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "W4A4 prefill GEMM TFLOPS (% FP4 peak); W4A16 decode GB/s (% HBM) on 1 MI355X"
PEAK = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}  # dense TFLOP/s
HBM_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))


def _pct(v, lo=10, hi=90):
    v = np.asarray(v, dtype=np.float64)
    return float(np.median(v)), float(np.percentile(v, lo)), float(np.percentile(v, hi))


def _progress(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _kernel_build_hash():
    """Hash of what decides the block-cooperative GEMM's machine code: its
    source, the internal header it includes, and its compile flags."""
    import hashlib
    from decode_nvfp4_rtn_amd import build as qbuild
    h = hashlib.sha256()
    for name in ("gemm_w4a4_coop.hip", "qlin_internal.hpp"):
        h.update(open(os.path.join(qbuild.CSRC, name), "rb").read())
    h.update(" ".join(qbuild.COMMON + qbuild.SOURCES["gemm_w4a4_coop.hip"]).encode())
    return h.hexdigest()[:16]


def _traffic_record():
    """HBM traffic of the dominant kernel from the committed rocprofv3 --pmc
    summary, if it was taken on the kernel as built now (hash match)."""
    path = os.path.join(ROOT, "profiles", "gemm_w4a4_qwen3_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("traffic:"):
            for kv in line.split()[1:]:
                k, v = kv.split("=")
                rec[k] = v
    if rec.get("kernel_sha256_16") != _kernel_build_hash():
        return None
    return float(rec["bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-reps", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of X per layer in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-sweep", action="store_true")
    ap.add_argument("--no-bf16-reference", action="store_true")
    ap.add_argument("--no-27b", action="store_true",
                    help="skip the 27B-class prefill measurement (M = 4096, 16384, 32768)")
    ap.add_argument("--no-small-m", action="store_true",
                    help="skip the smaller prefill batches (M = 512 / 1024 / 2048)")
    ap.add_argument("--no-odp", action="store_true",
                    help="skip the host-to-device weight streaming measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 3 device copies of 256 MiB (a kernel of known traffic, "
                         "to scale the FETCH_SIZE/WRITE_SIZE counters of a --pmc run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (sharded by "
              "output columns, each GPU would run the same kernels on its 1/N share of the "
              "weight rows).", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_nvfp4_rtn_amd import qlin, synth, configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ------------------------------------------------------------ set-up --
    pre = configs.QWEN3_PREFILL
    dec = configs.QWEN3_DECODE
    lut = configs.GEMMA3_LUT2
    M = pre.ms[0]
    M_DEC, M_LUT = 16, 8

    P = []   # prefill layers
    for li, L in enumerate(pre.layers):
        x = bf16(synth.activations_bf16(pre.cid, li, M, L.k, outliers=pre.outliers))
        wc, ws, wt = qlin.quantize_nvfp4(f32(synth.weights(pre.cid, li, L.n, L.k)))
        blob = qlin.repack_weights(qlin.QL_NVFP4, L.n, L.k, wc, ws, wt)
        del wc, ws
        P.append(dict(L=L, x=x, blob=blob,
                      codes=torch.empty((M, L.k // 2), dtype=torch.uint8, device=dev),
                      scales=torch.empty((M, L.k // 16), dtype=torch.uint8, device=dev),
                      ts=torch.empty(1, dtype=torch.float32, device=dev),
                      ws=torch.empty(max(16, qlin.quantize_nvfp4_workspace(M, L.k)),
                                     dtype=torch.uint8, device=dev),
                      y=torch.empty((M, L.n), dtype=torch.bfloat16, device=dev)))
        gb = qlin.gemm_w4a4_workspace(M, L.n, L.k)   # 0 when the tiles fill whole rounds
        P[-1]["gws"] = torch.empty(gb, dtype=torch.uint8, device=dev) if gb else None
    D = []   # W4A16 decode layers
    for li, L in enumerate(dec.layers):
        c, s = qlin.quantize_int4_g128(f32(synth.weights(dec.cid, li, L.n, L.k)))
        blob = qlin.repack_weights(qlin.QL_INT4_G128, L.n, L.k, c, s)
        x32 = {m: bf16(synth.decode_x_bf16(dec.cid, li, m, L.k)) for m in dec.ms}
        c24, s24 = qlin.quantize_int4_g128(f32(synth.weights(dec.cid, li, L.n, L.k)), sparse24=True)
        blob24 = qlin.repack_weights(qlin.QL_INT4_SP24, L.n, L.k, c24, s24)
        del c24, s24
        D.append(dict(L=L, blob=blob, blob24=blob24, x=x32,
                      y={m: torch.empty((m, L.n), dtype=torch.bfloat16, device=dev) for m in dec.ms}))
    U = []   # LUT2 decode layers
    for li, L in enumerate(lut.layers):
        i, c = qlin.fit_lut2(f32(synth.weights(lut.cid, li, L.n, L.k)))
        blob = qlin.repack_weights(qlin.QL_LUT2, L.n, L.k, i, c)
        xs = {m: bf16(synth.decode_x_bf16(lut.cid, li, m, L.k)) for m in lut.ms}
        U.append(dict(L=L, blob=blob, x=xs,
                      y={m: torch.empty((m, L.n), dtype=torch.bfloat16, device=dev) for m in lut.ms}))
    torch.cuda.synchronize()

    _progress("inputs and packed weights resident")
    prefill_flops = sum(2.0 * M * p["L"].n * p["L"].k for p in P)
    dec_flops = sum(2.0 * M_DEC * d["L"].n * d["L"].k for d in D)
    lut_flops = sum(2.0 * M_LUT * u["L"].n * u["L"].k for u in U)
    step_flops = prefill_flops + dec_flops + lut_flops

    E = torch.cuda.Event

    def step(ev=None):
        for i, p in enumerate(P):
            L = p["L"]
            if ev is not None:
                ev[i][0].record()
            qlin.quantize_nvfp4(p["x"], codes=p["codes"], scales=p["scales"],
                                workspace=p["ws"], ts_out=p["ts"])
            if ev is not None:
                ev[i][1].record()
            qlin.gemm_w4a4(p["codes"], p["scales"], p["ts"], p["blob"], M, L.n, L.k, y=p["y"],
                           workspace=p["gws"])
            if ev is not None:
                ev[i][2].record()
        if ev is not None:
            ev[len(P)][0].record()
        for d in D:
            qlin.gemm_w4a16(d["x"][M_DEC], d["blob"], d["L"].n, d["L"].k, y=d["y"][M_DEC])
        for u in U:
            qlin.gemm_lut2(u["x"][M_LUT], u["blob"], u["L"].n, u["L"].k, y=u["y"][M_LUT])
        if ev is not None:
            ev[len(P)][1].record()

    # -------------------------------------------------- warm-up + timing --
    # The timed region is K eager steps.  HIP events recorded on the stream the
    # kernels run on bracket every quantize, every GEMM and the decode block;
    # the host stays ahead of the GPU (each step queues ~3 ms of work for
    # ~0.2 ms of launch calls), so the events see back-to-back kernels.
    evs = [[[E(enable_timing=True) for _ in range(3)] for _ in range(len(P) + 1)]
           for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    q_ms = np.array([[evs[s][i][0].elapsed_time(evs[s][i][1]) for i in range(len(P))]
                     for s in range(args.steps)])
    g_ms = np.array([[evs[s][i][1].elapsed_time(evs[s][i][2]) for i in range(len(P))]
                     for s in range(args.steps)])
    d_ms = np.array([evs[s][len(P)][0].elapsed_time(evs[s][len(P)][1]) for s in range(args.steps)])
    _progress(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    layers = []
    for i, p in enumerate(P):
        L = p["L"]
        fl = 2.0 * M * L.n * L.k
        gq = float(np.median(g_ms[:, i]))
        qq = float(np.median(q_ms[:, i]))
        qbytes = 2.0 * M * L.k + M * L.k / 2 + M * L.k / 16
        layers.append({
            "layer": L.name, "n": L.n, "k": L.k,
            "gemm_us": round(gq * 1e3, 2), "gemm_tflops": round(fl / gq / 1e9, 1),
            "quantize_us": round(qq * 1e3, 2),
            "quantize_gbps_1pass_bytes": round(qbytes / qq / 1e6, 1),
            "prefill_tflops_incl_quantize": round(fl / (gq + qq) / 1e9, 1),
        })
    gemm_ms_step = float(np.median(g_ms.sum(axis=1)))
    quant_ms_step = float(np.median(q_ms.sum(axis=1)))
    gemm_tflops = prefill_flops / gemm_ms_step / 1e9
    prefill_tflops = prefill_flops / (gemm_ms_step + quant_ms_step) / 1e9

    # --------------------------------------- decode sweep (MALL defeated) --
    # Each (layer, batch) case is captured once in a HIP graph that launches the
    # kernel over enough weight copies (> 600 MB) that the 256 MiB Infinity
    # Cache cannot serve a repeat; the graph is replayed between two events.
    # Graph replay removes the host launch cost, which is larger than the
    # kernels themselves at these sizes.
    sweep = {}
    if not args.no_decode_sweep:
        combos = [("w4a16", li, m) for li in range(len(D)) for m in dec.ms] + \
                 [("w4a16_sp24", li, m) for li in range(len(D)) for m in dec.ms] + \
                 [("lut2", li, m) for li in range(len(U)) for m in lut.ms]
        fns = {"w4a16": qlin.gemm_w4a16, "w4a16_sp24": qlin.gemm_w4a16_sp24, "lut2": qlin.gemm_lut2}
        for kind, li, m in combos:
            rec = U[li] if kind == "lut2" else D[li]
            fn = fns[kind]
            src = rec["blob24"] if kind == "w4a16_sp24" else rec["blob"]
            L = rec["L"]
            if m == (lut.ms if kind == "lut2" else dec.ms)[0]:
                copies = [src.clone() for _ in range(int(np.ceil(600e6 / src.numel())))]
            x, y = rec["x"][m], rec["y"][m]
            for b in copies[:3]:
                fn(x, b, L.n, L.k, y=y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in copies:
                    fn(x, b, L.n, L.k, y=y)
            g.replay()
            torch.cuda.synchronize()
            t = []
            for _ in range(args.decode_reps):
                a, b = E(enable_timing=True), E(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                b.synchronize()
                t.append(a.elapsed_time(b) / len(copies))
            del g
            wbytes = {"w4a16": L.n * L.k / 2 + L.n * L.k / 64,
                      "w4a16_sp24": L.n * L.k / 4 + L.n * L.k / 8 + L.n * L.k / 64,
                      "lut2": L.n * L.k / 4 + 8 * L.n}[kind]
            by = wbytes + 2.0 * m * L.k + 2.0 * m * L.n
            med, p10, p90 = _pct(t)
            _progress(f"decode {kind}/{L.name}/m{m}: {med * 1e3:.2f} us")
            rec_out = {
                "us": round(med * 1e3, 2), "us_p10": round(p10 * 1e3, 2), "us_p90": round(p90 * 1e3, 2),
                "gbps": round(by / med / 1e6, 1), "hbm_frac": round(by / med / 1e6 / HBM_GBPS, 3)}
            if kind == "w4a16_sp24":
                dense = sweep.get(f"w4a16/{L.name}/m{m}")
                if dense:
                    rec_out["speedup_vs_w4a16"] = round(dense["us"] / (med * 1e3), 3)
            sweep[f"{kind}/{L.name}/m{m}"] = rec_out
            if m == (lut.ms if kind == "lut2" else dec.ms)[-1]:
                del copies
                torch.cuda.empty_cache()

    def _agg(kind, ms):
        out = {}
        for m in ms:
            vals = [v for k, v in sweep.items() if k.startswith(kind + "/") and k.endswith(f"/m{m}")]
            if vals:
                out[f"m{m}"] = round(float(np.mean([v["gbps"] for v in vals])), 1)
        return out

    # -------------------------------- weight streaming from host (ODP) ----
    # A layer block's packed weights (the four prefill layers) stream from
    # pinned host memory through two device buffers while the previous block
    # is quantized and multiplied (decode_nvfp4_rtn_amd.pipeline); a stack of
    # ODP_BLOCKS blocks with these weights is run.  Per batch size M: time of
    # the stack with resident weights, of the block copies alone, and of the
    # streamed stack; `exposed` is what the copies add.
    odp = {}
    if not args.no_odp:
        from decode_nvfp4_rtn_amd.pipeline import PrefillWeightStream
        ODP_BLOCKS = 4
        host = [p["blob"].cpu().pin_memory() for p in P]
        streamer = PrefillWeightStream([host], dev)
        wbytes = float(sum(h.numel() for h in host))
        shapes = [(p["L"].n, p["L"].k) for p in P]

        def timed(fn, stream=None, reps=5):
            out = []
            for _ in range(reps):
                torch.cuda.synchronize()
                a, b = E(enable_timing=True), E(enable_timing=True)
                st = stream if stream is not None else torch.cuda.current_stream()
                a.record(st)
                fn()
                b.record(st)
                torch.cuda.synchronize()
                out.append(a.elapsed_time(b))
            return float(np.median(out))

        def copies_alone():
            with torch.cuda.stream(streamer.copy_stream):
                for blk in range(ODP_BLOCKS):
                    for j, h in enumerate(host):
                        streamer._blob(blk % 2, 0, j).copy_(h, non_blocking=True)

        copy_ms = timed(copies_alone, stream=streamer.copy_stream)
        for m_odp in (512, 1024, 2048, 4096, 8192):
            xs = [p["x"][:m_odp] for p in P]
            cs = [p["codes"][:m_odp] for p in P]
            ss = [p["scales"][:m_odp] for p in P]
            ts = [p["ts"] for p in P]
            ws = [p["ws"] for p in P]
            ys = [p["y"][:m_odp] for p in P]

            def resident():
                for _ in range(ODP_BLOCKS):
                    for i, p in enumerate(P):
                        qlin.quantize_nvfp4(xs[i], codes=cs[i], scales=ss[i], workspace=ws[i],
                                            ts_out=ts[i])
                        qlin.gemm_w4a4(cs[i], ss[i], ts[i], p["blob"], m_odp, p["L"].n,
                                       p["L"].k, y=ys[i])

            comp_ms = timed(resident)
            strm_ms = timed(lambda: streamer.run([0] * ODP_BLOCKS, shapes, xs, ys, cs, ss, ts, ws))
            exposed = max(strm_ms - comp_ms, 0.0)
            # the first block's copy cannot overlap anything (pipeline fill)
            steady = max(strm_ms - comp_ms - copy_ms / ODP_BLOCKS, 0.0)
            odp[f"m{m_odp}"] = {"compute_ms": round(comp_ms, 4), "streamed_ms": round(strm_ms, 4),
                                "exposed_ms": round(exposed, 4),
                                "exposed_after_fill_ms": round(steady, 4),
                                "hidden_frac": round(1.0 - min(exposed / copy_ms, 1.0), 3),
                                "block_compute_ms": round(comp_ms / ODP_BLOCKS, 4)}
            _progress(f"odp m={m_odp}: compute {comp_ms:.3f} ms, streamed {strm_ms:.3f} ms")
        # batch size at which one block's compute equals one block's copy
        # (linear interpolation between the measured sizes)
        per_copy = copy_ms / ODP_BLOCKS
        ms_sorted = sorted(int(k[1:]) for k in odp)
        cross = None
        for a_m, b_m in zip(ms_sorted, ms_sorted[1:]):
            ca, cb = odp[f"m{a_m}"]["block_compute_ms"], odp[f"m{b_m}"]["block_compute_ms"]
            if ca < per_copy <= cb:
                cross = round(a_m + (per_copy - ca) * (b_m - a_m) / (cb - ca))
        odp["m_where_block_compute_equals_block_copy"] = cross
        odp["blocks"] = ODP_BLOCKS
        odp["copy_ms"] = round(copy_ms, 4)
        odp["h2d_gbps"] = round(ODP_BLOCKS * wbytes / copy_ms / 1e6, 1)
        odp["block_weights_mb"] = round(wbytes / 1e6, 1)
        del streamer, host

    # ------------------------------- 27B-class long-context prefill ----
    # NVFP4 W4A4 prefill (quantize + GEMM, bf16 out) of the 27B-class layer
    # set at M = 4096, 16384 and 32768 tokens, interleaved round-robin over
    # sizes and layers in this one process.  Activations: the first 4096 rows
    # of each layer's seeded draw (N(0,1), 0.1 % of elements x50, bf16),
    # repeated down to M rows (timing does not depend on the values; drawing
    # 1.1 G values on the host would take longer than the whole measurement).
    big = {}
    if not args.no_27b:
        b27 = configs.BIG27_PREFILL
        MB = max(b27.ms)
        R = []
        for li, L in enumerate(b27.layers):
            x0 = bf16(synth.activations_bf16(b27.cid, li, 4096, L.k, outliers=b27.outliers))
            x = x0.repeat(MB // 4096, 1)
            del x0
            wc, ws, wt = qlin.quantize_nvfp4(f32(synth.weights(b27.cid, li, L.n, L.k)))
            blob = qlin.repack_weights(qlin.QL_NVFP4, L.n, L.k, wc, ws, wt)
            del wc, ws
            R.append(dict(L=L, x=x, blob=blob,
                          codes=torch.empty((MB, L.k // 2), dtype=torch.uint8, device=dev),
                          scales=torch.empty((MB, L.k // 16), dtype=torch.uint8, device=dev),
                          ts=torch.empty(1, dtype=torch.float32, device=dev),
                          ws=torch.empty(max(16, qlin.quantize_nvfp4_workspace(MB, L.k)),
                                         dtype=torch.uint8, device=dev),
                          y=torch.empty((MB, L.n), dtype=torch.bfloat16, device=dev)))
            # k split of a partly filled last round of tiles (fp32 partials)
            R[-1]["gws_bytes"] = {m: qlin.gemm_w4a4_workspace(m, L.n, L.k) for m in b27.ms}
            nb = max(R[-1]["gws_bytes"].values())
            R[-1]["gws"] = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        torch.cuda.synchronize()
        _progress("27B-class inputs and packed weights resident")
        reps = 5
        tq = {(m, i): [] for m in b27.ms for i in range(len(R))}
        tg = {(m, i): [] for m in b27.ms for i in range(len(R))}
        for rep in range(reps + 1):
            for m in b27.ms:
                for i, r in enumerate(R):
                    L = r["L"]
                    e0, e1, e2 = E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)
                    e0.record()
                    qlin.quantize_nvfp4(r["x"][:m], codes=r["codes"][:m], scales=r["scales"][:m],
                                        workspace=r["ws"], ts_out=r["ts"])
                    e1.record()
                    qlin.gemm_w4a4(r["codes"][:m], r["scales"][:m], r["ts"], r["blob"], m, L.n, L.k,
                                   y=r["y"][:m],
                                   workspace=r["gws"] if r["gws_bytes"][m] else None)
                    e2.record()
                    if rep > 0:   # the first round is a warm-up
                        tq[(m, i)].append((e0, e1))
                        tg[(m, i)].append((e1, e2))
        torch.cuda.synchronize()
        for m in b27.ms:
            rows, fl_all, q_all, g_all = [], 0.0, 0.0, 0.0
            for i, r in enumerate(R):
                L = r["L"]
                q = float(np.median([a.elapsed_time(b) for a, b in tq[(m, i)]]))
                g = float(np.median([a.elapsed_time(b) for a, b in tg[(m, i)]]))
                fl = 2.0 * m * L.n * L.k
                fl_all, q_all, g_all = fl_all + fl, q_all + q, g_all + g
                rows.append({"layer": L.name, "n": L.n, "k": L.k, "gemm_us": round(g * 1e3, 1),
                             "gemm_tflops": round(fl / g / 1e9, 1), "quantize_us": round(q * 1e3, 1),
                             "k_split_workspace_mb": round(r["gws_bytes"][m] / 1e6, 1)})
            big[f"m{m}"] = {
                "layers": rows,
                "gemm_tflops": round(fl_all / g_all / 1e9, 1),
                "prefill_tflops_incl_quantize": round(fl_all / (g_all + q_all) / 1e9, 1),
                "gemm_frac_f16_peak": round(fl_all / g_all / 1e9 / PEAK["f16"], 4),
                "gemm_frac_fp8_peak": round(fl_all / g_all / 1e9 / PEAK["fp8"], 4),
                "gemm_frac_fp4_peak": round(fl_all / g_all / 1e9 / PEAK["fp4"], 4),
                "quantize_ms": round(q_all, 4), "gemm_ms": round(g_all, 4)}
            _progress(f"27b m={m}: GEMM {big[f'm{m}']['gemm_tflops']} TFLOP/s, "
                      f"with quantize {big[f'm{m}']['prefill_tflops_incl_quantize']}")
        big["activations"] = ("first 4096 rows of each layer's seeded draw repeated to M rows; "
                              "median of 5 interleaved rounds after one warm-up round")
        del R
        torch.cuda.empty_cache()

    # ------------------------------------------ smaller prefill batches ----
    # The Qwen3-8B-like layers at M = 512 / 1024 / 2048 (the first M rows of
    # the same inputs), quantize + GEMM, with a gemm_w4a4 workspace where a k
    # split applies.  With fewer 256 x 256 tiles than CUs these show the
    # GEMM's dispatch: the cooperative kernel above half a round of tiles,
    # its k split below that (workspace), never the per-wave kernel here.
    small = {}
    if not args.no_small_m:
        SM = (512, 1024, 2048)
        gws = {}
        for i, p in enumerate(P):
            for m in SM:
                nb = qlin.gemm_w4a4_workspace(m, p["L"].n, p["L"].k)
                gws[(m, i)] = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        tq = {(m, i): [] for m in SM for i in range(len(P))}
        tg = {(m, i): [] for m in SM for i in range(len(P))}
        for rep in range(6):
            for m in SM:
                for i, p in enumerate(P):
                    L = p["L"]
                    e0, e1, e2 = E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)
                    e0.record()
                    qlin.quantize_nvfp4(p["x"][:m], codes=p["codes"][:m], scales=p["scales"][:m],
                                        workspace=p["ws"], ts_out=p["ts"])
                    e1.record()
                    qlin.gemm_w4a4(p["codes"][:m], p["scales"][:m], p["ts"], p["blob"], m, L.n, L.k,
                                   y=p["y"][:m], workspace=gws[(m, i)])
                    e2.record()
                    if rep > 0:   # the first round is a warm-up
                        tq[(m, i)].append((e0, e1))
                        tg[(m, i)].append((e1, e2))
        torch.cuda.synchronize()
        for m in SM:
            rows, fl_all, q_all, g_all = [], 0.0, 0.0, 0.0
            for i, p in enumerate(P):
                L = p["L"]
                q = float(np.median([a.elapsed_time(b) for a, b in tq[(m, i)]]))
                g = float(np.median([a.elapsed_time(b) for a, b in tg[(m, i)]]))
                fl = 2.0 * m * L.n * L.k
                fl_all, q_all, g_all = fl_all + fl, q_all + q, g_all + g
                nb = 0 if gws[(m, i)] is None else gws[(m, i)].numel()
                rows.append({"layer": L.name, "gemm_us": round(g * 1e3, 1),
                             "gemm_tflops": round(fl / g / 1e9, 1), "quantize_us": round(q * 1e3, 1),
                             "k_split_workspace_mb": round(nb / 1e6, 1)})
            small[f"m{m}"] = {"layers": rows, "gemm_tflops": round(fl_all / g_all / 1e9, 1),
                              "prefill_tflops_incl_quantize": round(fl_all / (g_all + q_all) / 1e9, 1)}
            _progress(f"small m={m}: GEMM {small[f'm{m}']['gemm_tflops']} TFLOP/s")
        small["activations"] = "first M rows of the M = 8192 inputs; median of 5 interleaved rounds"
        del gws

    # ------------------------------------------- BF16 reference points ----
    # The pages state their speed-ups against BF16; torch's bf16 matmul
    # (hipBLASLt) on the same shapes is that reference here: prefill
    # Y = X W^T at M=8192 (TFLOP/s) and decode GEMV at M=1 and 16 (GB/s,
    # weights rotated over > 600 MB like the decode sweep).
    bf16_ref = {}
    if not args.no_bf16_reference:
        for p in P:
            L = p["L"]
            wb = torch.randn((L.n, L.k), dtype=torch.bfloat16, device=dev) * (L.k ** -0.5)
            ref_ms = []
            for _ in range(3):
                torch.matmul(p["x"], wb.t())
            torch.cuda.synchronize()
            for _ in range(10):
                a, b = E(enable_timing=True), E(enable_timing=True)
                a.record()
                torch.matmul(p["x"], wb.t())
                b.record()
                b.synchronize()
                ref_ms.append(a.elapsed_time(b))
            med = float(np.median(ref_ms))
            bf16_ref[f"prefill/{L.name}"] = {
                "us": round(med * 1e3, 1),
                "tflops": round(2.0 * M * L.n * L.k / med / 1e9, 1)}
            del wb
        for d in D:
            L = d["L"]
            copies = [torch.randn((L.n, L.k), dtype=torch.bfloat16, device=dev)
                      for _ in range(int(np.ceil(600e6 / (2.0 * L.n * L.k))))]
            for m in (1, 16):
                xb = d["x"][m]
                yb = torch.empty((m, L.n), dtype=torch.bfloat16, device=dev)
                for c in copies[:2]:
                    torch.matmul(xb, c.t(), out=yb)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for c in copies:
                        torch.matmul(xb, c.t(), out=yb)
                g.replay()
                torch.cuda.synchronize()
                t = []
                for _ in range(5):
                    a, b = E(enable_timing=True), E(enable_timing=True)
                    a.record()
                    g.replay()
                    b.record()
                    b.synchronize()
                    t.append(a.elapsed_time(b) / len(copies))
                del g
                med = float(np.median(t))
                by = 2.0 * L.n * L.k + 2.0 * m * L.k + 2.0 * m * L.n
                bf16_ref[f"decode/{L.name}/m{m}"] = {"us": round(med * 1e3, 2),
                                                    "gbps": round(by / med / 1e6, 1)}
            del copies
            torch.cuda.empty_cache()
        _progress("bf16 reference points measured")

    # --------------------------------------------------- CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_rows, pre, M)
        _progress(f"cpu baseline: {cpu['sample']}")

    traffic = _traffic_record()
    avg_launch_ms = gemm_ms_step / len(P)
    out = {
        "metric": METRIC,
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-like linear set: NVFP4 W4A4 prefill (quantize + GEMM, M=8192, "
                        "bf16 out) over qkv/o/gate_up/down, + W4A16 decode M=16 over the same "
                        "shapes, + Gemma3-12B-like LUT2 decode M=8",
            "m_prefill": M, "m_w4a16": M_DEC, "m_lut2": M_LUT,
            "prefill_layers_nk": [[p["L"].n, p["L"].k] for p in P],
            "lut2_layers_nk": [[u["L"].n, u["L"].k] for u in U],
        },
        "roofline": {
            "kernel": "w4a4_coop_kernel (gemm_w4a4)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK["f16"],
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK["f16"], 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
            "per_launch": "mean over the 4 prefill layers of 2*M*N*K FLOPs / mean event-timed "
                          "launch duration; traffic = HBM bytes per launch (mean over the layers)",
        },
        "cpu_baseline": cpu,
        "parts": {
            "prefill_tflops_incl_quantize": round(prefill_tflops, 1),
            "gemm_w4a4_tflops": round(gemm_tflops, 1),
            "gemm_w4a4_frac_fp4_peak": round(gemm_tflops / PEAK["fp4"], 4),
            "gemm_w4a4_frac_fp8_peak": round(gemm_tflops / PEAK["fp8"], 4),
            "gemm_w4a4_frac_f16_peak": round(gemm_tflops / PEAK["f16"], 4),
            "quantize_ms_per_step": round(quant_ms_step, 4),
            "gemm_ms_per_step": round(gemm_ms_step, 4),
            "decode_block_ms_per_step": round(float(np.median(d_ms)), 4),
            "layers": layers,
            "w4a16_gbps_mean_over_layers": _agg("w4a16", dec.ms),
            "lut2_gbps_mean_over_layers": _agg("lut2", lut.ms),
            "w4a16_sp24_gbps_mean_over_layers": _agg("w4a16_sp24", dec.ms),
            "decode_sweep": sweep,
            "bf16_reference": bf16_ref,
            "odp_weight_streaming": odp,
            "prefill_27b": big,
            "prefill_small_m": small,
            "w4a4_gemm_speedup_vs_bf16": (
                round(sum(v["us"] for k, v in bf16_ref.items() if k.startswith("prefill/"))
                      / (gemm_ms_step * 1e3), 3) if bf16_ref else None),
            "decode_timing": "events around the replay of a HIP graph of back-to-back launches "
                             "rotating over >600 MB of weight copies (Infinity Cache defeated)",
        },
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(rows, pre, M):
    """The oracle as it stands, timed on the host on a bounded sample: for each
    prefill layer, NVFP4-quantize `rows` rows of X (with the full tensor's
    scale) and run the oracle's fp64 W4A4 product against the layer's weights
    (weight quantization is offline, outside the timing, as on the GPU)."""
    sys.path.insert(0, ROOT)
    from oracle import nvfp4, gemm
    from decode_nvfp4_rtn_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    prep = []
    for li, L in enumerate(pre.layers):
        xb = synth.activations_bf16(pre.cid, li, rows, L.k, outliers=pre.outliers)
        w = synth.weights(pre.cid, li, L.n, L.k)
        prep.append((L, synth.bf16_bits_as_f32(xb), nvfp4.quantize(w)))
    t0 = time.perf_counter()
    flops = 0.0
    for L, x, wq in prep:
        aq = nvfp4.quantize(x)
        gemm.w4a4(*aq, *wq)
        flops += 2.0 * rows * L.n * L.k
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of the {M} token rows of each of the 4 prefill layers "
                      f"(quantize + fp64 product); {dt:.1f} s"}


if __name__ == "__main__":
    main()
