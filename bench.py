#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X; prints ONE JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
  prefill  the four 27B-class layers (qkv 7168x5120, o_proj 5120x5120,
           gate_up 34816x5120, down 5120x17408) at M = 32768 tokens, each
           quantize_nvfp4(X bf16) -> gemm_w4a4(-> Y bf16)     (quantize is timed)
  decode   W4A16 (INT4 group-128) at M = 16 over the four Qwen3-8B-like shapes
  decode   LUT2 at M = 8 over the three Gemma3-12B-like shapes
The activations are drawn at full size by the seeded generator (synth),
every row, in host threads; inputs and packed weights are resident in HBM
before the timed region.

value = the step's algorithmic FLOPs / ms_per_step (TFLOP/s; the prefill
FLOPs are 99.99 % of them).  HIP events recorded on the stream every kernel is
launched on time each quantize, each GEMM and the decode block.

``roofline`` describes the dominant kernel, the W4A4 GEMM
(w4a4_coop_kernel), against the dense FP4 peak the metric names (its fp16
fraction, the rate of the MFMA it runs on, is reported beside it);
``cpu_baseline`` times the CPU oracle (test infrastructure) on a bounded
sample of the same workload.  ``parts`` holds the other measurements: the
Qwen3-8B-like prefill set at M = 8192, the 27B-class set at M = 4096 and
16384, smaller prefill batches, a decode sweep over every batch size that
rotates through > 512 MiB of weight copies (so the 256 MiB Infinity Cache
cannot serve repeats), the 2:4 sparse decode, torch's bf16 GEMM/GEMV on the
same shapes, and weight streaming from host memory.
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


TRAFFIC_PROFILE = {"27b": os.path.join("profiles", "gemm_w4a4_27b_m32768_traffic.md"),
                   "qwen3": os.path.join("profiles", "gemm_w4a4_qwen3_m8192_traffic.md")}


def _traffic_record(prefill_set):
    """HBM bytes per launch of the dominant kernel on the step's prefill set,
    from the committed rocprofv3 --pmc summary, if it was taken on the kernel
    as built now (hash match)."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE[prefill_set])
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


def host_threads():
    """Cores this process may run on (the GPU machine's share of the host)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def draw_activations_bf16(cid, li, m, k, outliers):
    """synth.activations_bf16 of every row of [m, k], drawn in 2048-row
    ranges on host threads (synth seeds each 256-row block on its own, so this
    is the same tensor as one draw)."""
    from concurrent.futures import ThreadPoolExecutor
    from decode_nvfp4_rtn_amd import synth
    out = np.empty((m, k), dtype=np.uint16)
    step = 2048

    def one(r0):
        out[r0:min(m, r0 + step)] = synth.activations_bf16(cid, li, m, k, outliers=outliers,
                                                           rows=(r0, min(m, r0 + step)))
    with ThreadPoolExecutor(max_workers=max(1, min(16, host_threads()))) as ex:
        list(ex.map(one, range(0, m, step)))
    return out


def draw_weights(cid, li, n, k):
    """synth.weights of every row of [n, k], drawn in row ranges on host threads."""
    from concurrent.futures import ThreadPoolExecutor
    from decode_nvfp4_rtn_amd import synth
    out = np.empty((n, k), dtype=np.float32)
    step = 2048

    def one(r0):
        out[r0:min(n, r0 + step)] = synth.weights(cid, li, n, k, rows=(r0, min(n, r0 + step)))
    with ThreadPoolExecutor(max_workers=max(1, min(16, host_threads()))) as ex:
        list(ex.map(one, range(0, n, step)))
    return out


def decode_launches(spec, dev, bf16, f32):
    """Profiling workload (--decode-launches): the named decode cases in the
    given order, each as 3 direct launches, each launch after a 512 MiB device
    fill (twice the Infinity Cache) so the weights come from HBM."""
    import torch
    from decode_nvfp4_rtn_amd import qlin, synth, configs
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for case in spec.split(","):
        parts = case.strip().split("/")
        kind, name, m = parts[0], parts[1], int(parts[2])
        use_ws = parts[3:] == ["ws"]
        cfg = configs.GEMMA3_LUT2 if kind == "lut2" else configs.QWEN3_DECODE
        li = [L.name for L in cfg.layers].index(name)
        L = cfg.layers[li]
        w = f32(synth.weights(cfg.cid, li, L.n, L.k))
        if kind == "lut2":
            i, c = qlin.fit_lut2(w)
            blob = qlin.repack_weights(qlin.QL_LUT2, L.n, L.k, i, c)
            fn, wsf = qlin.gemm_lut2, qlin.gemm_lut2_workspace
        elif kind == "sp24":
            c, sc = qlin.quantize_int4_g128(w, sparse24=True)
            blob = qlin.repack_weights(qlin.QL_INT4_SP24, L.n, L.k, c, sc)
            fn, wsf = qlin.gemm_w4a16_sp24, qlin.gemm_w4a16_sp24_workspace
        else:
            c, sc = qlin.quantize_int4_g128(w)
            blob = qlin.repack_weights(qlin.QL_INT4_G128, L.n, L.k, c, sc)
            fn, wsf = qlin.gemm_w4a16, qlin.gemm_w4a16_workspace
        del w
        x = bf16(synth.decode_x_bf16(cfg.cid, li, m, L.k))
        y = torch.empty((m, L.n), dtype=torch.bfloat16, device=dev)
        kw = {}
        if use_ws:
            nb = wsf(m, L.n, L.k)
            if nb == 0:
                raise SystemExit(f"{case}: this shape has no k-split workspace")
            kw["workspace"] = torch.empty(nb, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for r in range(3):
            flush.fill_(r)
            fn(x, blob, L.n, L.k, y=y, **kw)
            torch.cuda.synchronize()
        print(f"case {case}: {L.n} x {L.k}, m {m}", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-reps", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="token rows per layer in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-sweep", action="store_true")
    ap.add_argument("--no-bf16-reference", action="store_true")
    ap.add_argument("--prefill-set", choices=("27b", "qwen3"), default="27b",
                    help="prefill layers of the timed step: the 27B-class set at M = 32768 "
                         "(default) or the Qwen3-8B-like set at M = 8192 (for profiling that "
                         "set alone; the other prefill measurements are then skipped)")
    ap.add_argument("--no-qwen3", action="store_true",
                    help="skip the Qwen3-8B-like prefill set (M = 8192) and the smaller batches")
    ap.add_argument("--no-27b-smaller", action="store_true",
                    help="skip the 27B-class prefill set at M = 4096 and 16384")
    ap.add_argument("--no-small-m", action="store_true",
                    help="skip the smaller prefill batches (M = 512 / 1024 / 2048)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip quantize_gemm_w4a4 against quantize_nvfp4 + gemm_w4a4")
    ap.add_argument("--no-odp", action="store_true",
                    help="skip the host-to-device weight streaming measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 3 device copies and 3 elementwise negations of 256 MiB "
                         "(kernels of known traffic, to scale the FETCH_SIZE/WRITE_SIZE "
                         "counters of a --pmc run)")
    ap.add_argument("--decode-launches", default=None, metavar="CASES",
                    help="profiling workload only: comma-separated decode cases "
                         "format/layer/M[/ws] (format w4a16, sp24 or lut2; layer as in the "
                         "decode sweep; ws: the workspace entry point), each launched 3 times "
                         "after a 512 MiB fill that evicts the weights from the Infinity "
                         "Cache; prints one line per case and no bench line")
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

    if args.decode_launches:
        decode_launches(args.decode_launches, dev, bf16, f32)
        return

    if args.copy_calibration:
        # kernels of known traffic: three runtime copies of 256 MiB, then three
        # elementwise negations of 256 MiB of fp32 (a plain vector kernel that
        # reads 256 MiB and writes 256 MiB with ordinary loads and stores)
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        af, bf = a.view(torch.float32), b.view(torch.float32)
        af.zero_()
        for _ in range(3):
            torch.neg(af, out=bf)
        torch.cuda.synchronize()
        del a, b, af, bf

    def prefill_set(cfg, m_max, ms):
        """Packed weights, full-size activations and output buffers of a
        prefill layer set, with a k-split workspace for every M that has one."""
        out = []
        for li, L in enumerate(cfg.layers):
            x = bf16(draw_activations_bf16(cfg.cid, li, m_max, L.k, cfg.outliers))
            wc, ws, wt = qlin.quantize_nvfp4(f32(draw_weights(cfg.cid, li, L.n, L.k)))
            blob = qlin.repack_weights(qlin.QL_NVFP4, L.n, L.k, wc, ws, wt)
            del wc, ws
            gws_bytes = {m: qlin.gemm_w4a4_workspace(m, L.n, L.k) for m in ms}
            nb = max(gws_bytes.values())
            out.append(dict(L=L, x=x, blob=blob, gws_bytes=gws_bytes,
                            gws=torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None,
                            codes=torch.empty((m_max, L.k // 2), dtype=torch.uint8, device=dev),
                            scales=torch.empty((m_max, L.k // 16), dtype=torch.uint8, device=dev),
                            ts=torch.empty(1, dtype=torch.float32, device=dev),
                            ws=torch.empty(max(16, qlin.quantize_nvfp4_workspace(m_max, L.k)),
                                           dtype=torch.uint8, device=dev),
                            y=torch.empty((m_max, L.n), dtype=torch.bfloat16, device=dev)))
        return out

    def prefill_layer(r, m, ev=None):
        """quantize_nvfp4 + gemm_w4a4 of one layer on its first m token rows;
        ev = (e0, e1, e2) events around the two calls."""
        L = r["L"]
        if ev is not None:
            ev[0].record()
        qlin.quantize_nvfp4(r["x"][:m], codes=r["codes"][:m], scales=r["scales"][:m],
                            workspace=r["ws"], ts_out=r["ts"])
        if ev is not None:
            ev[1].record()
        qlin.gemm_w4a4(r["codes"][:m], r["scales"][:m], r["ts"], r["blob"], m, L.n, L.k,
                       y=r["y"][:m], workspace=r["gws"] if r["gws_bytes"][m] else None)
        if ev is not None:
            ev[2].record()

    E = torch.cuda.Event

    def interleaved(R, ms, rounds=6, warm=2):
        """quantize + GEMM of every (M, layer), round-robin in this process:
        `warm` warm-up rounds, then the median of `rounds` rounds per case."""
        tq = {(m, i): [] for m in ms for i in range(len(R))}
        tg = {(m, i): [] for m in ms for i in range(len(R))}
        for rep in range(rounds + warm):
            for m in ms:
                for i, r in enumerate(R):
                    ev = (E(enable_timing=True), E(enable_timing=True), E(enable_timing=True))
                    prefill_layer(r, m, ev)
                    if rep >= warm:
                        tq[(m, i)].append((ev[0], ev[1]))
                        tg[(m, i)].append((ev[1], ev[2]))
        torch.cuda.synchronize()
        res = {}
        for m in ms:
            rows, fl_all, q_all, g_all = [], 0.0, 0.0, 0.0
            for i, r in enumerate(R):
                L = r["L"]
                q = float(np.median([a.elapsed_time(b) for a, b in tq[(m, i)]]))
                g = float(np.median([a.elapsed_time(b) for a, b in tg[(m, i)]]))
                fl = 2.0 * m * L.n * L.k
                fl_all, q_all, g_all = fl_all + fl, q_all + q, g_all + g
                qbytes = 2.0 * m * L.k + m * L.k / 2 + m * L.k / 16
                rows.append({"layer": L.name, "n": L.n, "k": L.k, "gemm_us": round(g * 1e3, 1),
                             "gemm_tflops": round(fl / g / 1e9, 1),
                             "quantize_us": round(q * 1e3, 1),
                             "quantize_gbps_1pass_bytes": round(qbytes / q / 1e6, 1),
                             "k_split_workspace_mb": round(r["gws_bytes"][m] / 1e6, 1)})
            res[f"m{m}"] = {
                "layers": rows,
                "gemm_tflops": round(fl_all / g_all / 1e9, 1),
                "prefill_tflops_incl_quantize": round(fl_all / (g_all + q_all) / 1e9, 1),
                "gemm_frac_fp4_peak": round(fl_all / g_all / 1e9 / PEAK["fp4"], 4),
                "gemm_frac_fp8_peak": round(fl_all / g_all / 1e9 / PEAK["fp8"], 4),
                "gemm_frac_f16_peak": round(fl_all / g_all / 1e9 / PEAK["f16"], 4),
                "quantize_ms": round(q_all, 4), "gemm_ms": round(g_all, 4)}
        return res

    def fused_vs_two_calls(R, ms, rounds=6, warm=2):
        """quantize_gemm_w4a4 (quantize folded into the GEMM's activation load)
        against quantize_nvfp4 + gemm_w4a4 (with its k-split workspace where
        the shape has one) on the same inputs, interleaved in this process;
        median per case."""
        gws = {}
        for m in ms:
            for i, r in enumerate(R):
                nb = qlin.gemm_w4a4_workspace(m, r["L"].n, r["L"].k)
                gws[(m, i)] = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        t2 = {key: [] for key in gws}
        tf = {key: [] for key in gws}
        for rep in range(rounds + warm):
            for m in ms:
                for i, r in enumerate(R):
                    L = r["L"]
                    e = [E(enable_timing=True) for _ in range(3)]
                    e[0].record()
                    qlin.quantize_nvfp4(r["x"][:m], codes=r["codes"][:m], scales=r["scales"][:m],
                                        workspace=r["ws"], ts_out=r["ts"])
                    qlin.gemm_w4a4(r["codes"][:m], r["scales"][:m], r["ts"], r["blob"], m, L.n,
                                   L.k, y=r["y"][:m], workspace=gws[(m, i)])
                    e[1].record()
                    qlin.quantize_gemm_w4a4(r["x"][:m], r["blob"], L.n, y=r["y"][:m],
                                            ts_out=r["ts"], workspace=r["ws"])
                    e[2].record()
                    if rep >= warm:
                        t2[(m, i)].append((e[0], e[1]))
                        tf[(m, i)].append((e[1], e[2]))
        torch.cuda.synchronize()
        res = {}
        for m in ms:
            rows, a_all, b_all = [], 0.0, 0.0
            for i, r in enumerate(R):
                a = float(np.median([x.elapsed_time(y) for x, y in t2[(m, i)]])) * 1e3
                b = float(np.median([x.elapsed_time(y) for x, y in tf[(m, i)]])) * 1e3
                a_all, b_all = a_all + a, b_all + b
                rows.append({"layer": r["L"].name, "two_calls_us": round(a, 1),
                             "fused_us": round(b, 1), "fused_speedup": round(a / b, 3)})
            res[f"m{m}"] = {"layers": rows, "two_calls_us": round(a_all, 1),
                            "fused_us": round(b_all, 1), "fused_speedup": round(a_all / b_all, 3)}
        return res

    # ------------------------------------------------------------ set-up --
    big = configs.BIG27_PREFILL if args.prefill_set == "27b" else configs.QWEN3_PREFILL
    dec = configs.QWEN3_DECODE
    lut = configs.GEMMA3_LUT2
    M = max(big.ms)          # 32768 tokens (8192 for the Qwen3-8B-like set)
    M_DEC, M_LUT = 16, 8

    def decode_ws(ws_fn, ms, L):
        """k-split workspace of each batch size that has one (else None)."""
        out = {}
        for m in ms:
            nb = ws_fn(m, L.n, L.k)
            out[m] = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        return out

    R = prefill_set(big, M, big.ms)
    D = []   # W4A16 decode layers
    for li, L in enumerate(dec.layers):
        w = f32(draw_weights(dec.cid, li, L.n, L.k))
        c, s = qlin.quantize_int4_g128(w)
        blob = qlin.repack_weights(qlin.QL_INT4_G128, L.n, L.k, c, s)
        c24, s24 = qlin.quantize_int4_g128(w, sparse24=True)
        blob24 = qlin.repack_weights(qlin.QL_INT4_SP24, L.n, L.k, c24, s24)
        del w, c, s, c24, s24
        x32 = {m: bf16(synth.decode_x_bf16(dec.cid, li, m, L.k)) for m in dec.ms}
        D.append(dict(L=L, blob=blob, blob24=blob24, x=x32,
                      y={m: torch.empty((m, L.n), dtype=torch.bfloat16, device=dev) for m in dec.ms},
                      ws=decode_ws(qlin.gemm_w4a16_workspace, dec.ms, L),
                      ws24=decode_ws(qlin.gemm_w4a16_sp24_workspace, dec.ms, L)))
    U = []   # LUT2 decode layers
    for li, L in enumerate(lut.layers):
        i, c = qlin.fit_lut2(f32(draw_weights(lut.cid, li, L.n, L.k)))
        blob = qlin.repack_weights(qlin.QL_LUT2, L.n, L.k, i, c)
        xs = {m: bf16(synth.decode_x_bf16(lut.cid, li, m, L.k)) for m in lut.ms}
        U.append(dict(L=L, blob=blob, x=xs,
                      y={m: torch.empty((m, L.n), dtype=torch.bfloat16, device=dev) for m in lut.ms},
                      ws=decode_ws(qlin.gemm_lut2_workspace, lut.ms, L)))
    torch.cuda.synchronize()

    _progress("inputs and packed weights resident")
    prefill_flops = sum(2.0 * M * r["L"].n * r["L"].k for r in R)
    dec_flops = sum(2.0 * M_DEC * d["L"].n * d["L"].k for d in D)
    lut_flops = sum(2.0 * M_LUT * u["L"].n * u["L"].k for u in U)
    step_flops = prefill_flops + dec_flops + lut_flops

    def step(ev=None):
        for i, r in enumerate(R):
            prefill_layer(r, M, None if ev is None else ev[i])
        if ev is not None:
            ev[len(R)][0].record()
        for d in D:
            qlin.gemm_w4a16(d["x"][M_DEC], d["blob"], d["L"].n, d["L"].k, y=d["y"][M_DEC],
                            workspace=d["ws"][M_DEC])
        for u in U:
            qlin.gemm_lut2(u["x"][M_LUT], u["blob"], u["L"].n, u["L"].k, y=u["y"][M_LUT],
                           workspace=u["ws"][M_LUT])
        if ev is not None:
            ev[len(R)][1].record()

    # -------------------------------------------------- warm-up + timing --
    # The timed region is K eager steps between two device synchronisations.
    # HIP events recorded on the stream the kernels run on bracket every
    # quantize, every GEMM and the decode block; the host stays ahead of the
    # GPU (each step queues ~17 ms of work for well under 1 ms of launch
    # calls), so the events see back-to-back kernels.
    evs = [[[E(enable_timing=True) for _ in range(3)] for _ in range(len(R) + 1)]
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
    q_ms = np.array([[evs[s][i][0].elapsed_time(evs[s][i][1]) for i in range(len(R))]
                     for s in range(args.steps)])
    g_ms = np.array([[evs[s][i][1].elapsed_time(evs[s][i][2]) for i in range(len(R))]
                     for s in range(args.steps)])
    d_ms = np.array([evs[s][len(R)][0].elapsed_time(evs[s][len(R)][1]) for s in range(args.steps)])
    _progress(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    layers = []
    for i, r in enumerate(R):
        L = r["L"]
        fl = 2.0 * M * L.n * L.k
        gq = float(np.median(g_ms[:, i]))
        qq = float(np.median(q_ms[:, i]))
        qbytes = 2.0 * M * L.k + M * L.k / 2 + M * L.k / 16
        layers.append({
            "layer": L.name, "n": L.n, "k": L.k,
            "gemm_us": round(gq * 1e3, 1), "gemm_tflops": round(fl / gq / 1e9, 1),
            "gemm_frac_fp4_peak": round(fl / gq / 1e9 / PEAK["fp4"], 4),
            "gemm_frac_f16_peak": round(fl / gq / 1e9 / PEAK["f16"], 4),
            "quantize_us": round(qq * 1e3, 1),
            "quantize_gbps_1pass_bytes": round(qbytes / qq / 1e6, 1),
            "prefill_tflops_incl_quantize": round(fl / (gq + qq) / 1e9, 1),
        })
    gemm_ms_step = float(np.median(g_ms.sum(axis=1)))
    quant_ms_step = float(np.median(q_ms.sum(axis=1)))
    gemm_tflops = prefill_flops / gemm_ms_step / 1e9
    prefill_tflops = prefill_flops / (gemm_ms_step + quant_ms_step) / 1e9
    # mean event-timed duration of the 4 x K timed GEMM launches
    avg_launch_ms = float(np.mean(g_ms))
    achieved = (prefill_flops / len(R)) / avg_launch_ms / 1e9

    # ---------------------------------- 27B-class set at smaller M ------
    big_parts = {f"m{M}": {"layers": layers, "gemm_tflops": round(gemm_tflops, 1),
                            "prefill_tflops_incl_quantize": round(prefill_tflops, 1),
                            "gemm_frac_fp4_peak": round(gemm_tflops / PEAK["fp4"], 4),
                            "gemm_frac_fp8_peak": round(gemm_tflops / PEAK["fp8"], 4),
                            "gemm_frac_f16_peak": round(gemm_tflops / PEAK["f16"], 4),
                            "quantize_ms": round(quant_ms_step, 4),
                            "gemm_ms": round(gemm_ms_step, 4),
                            "source": "the timed steps (median per layer)"}}
    if not args.no_27b_smaller and args.prefill_set == "27b":
        big_parts.update(interleaved(R, [m for m in big.ms if m != M]))
        for m in big.ms:
            if m != M:
                _progress(f"27b m={m}: GEMM {big_parts[f'm{m}']['gemm_tflops']} TFLOP/s")
    big_parts["activations"] = (f"every row drawn by the seeded generator at M = {M}; smaller "
                                "M are its first rows (the same tensors as draws at those M)")

    # ----------------------------------- Qwen3-8B-like prefill set ------
    qwen = {}
    P = []
    if args.prefill_set == "qwen3":
        qwen, big_parts, P = big_parts, {}, R
    elif not args.no_qwen3:
        pre = configs.QWEN3_PREFILL
        SM = () if args.no_small_m else (512, 1024, 2048)
        P = prefill_set(pre, pre.ms[0], (pre.ms[0],) + SM)
        qwen = interleaved(P, [pre.ms[0]])
        _progress(f"qwen3 m={pre.ms[0]}: GEMM {qwen[f'm{pre.ms[0]}']['gemm_tflops']} TFLOP/s")
        if SM:
            qwen.update(interleaved(P, list(SM)))
        qwen["activations"] = ("every row drawn by the seeded generator at M = 8192; smaller M "
                               "are its first rows")
    fused = {}
    if P and not args.no_fused:
        fused = fused_vs_two_calls(P, [16, 64, 128, 512, 2048])
        fused["timing"] = ("events around quantize_nvfp4 + gemm_w4a4 and around "
                           "quantize_gemm_w4a4 on the Qwen3-8B-like layers' first M rows, "
                           "interleaved, median of 6 rounds")
        _progress("fused quantize + GEMM: " + ", ".join(
            f"m{m} {fused[f'm{m}']['fused_speedup']}x" for m in (16, 64, 128, 512, 2048)))

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
            kw = {"workspace": rec["ws24" if kind == "w4a16_sp24" else "ws"][m]}
            for b in copies[:3]:
                fn(x, b, L.n, L.k, y=y, **kw)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in copies:
                    fn(x, b, L.n, L.k, y=y, **kw)
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
                "gbps": round(by / med / 1e6, 1), "hbm_frac": round(by / med / 1e6 / HBM_GBPS, 3),
                "k_split": bool(kw.get("workspace") is not None)}
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
    if not args.no_odp and P:
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

    # ------------------------------------------- BF16 reference points ----
    # The pages state their speed-ups against BF16; torch's bf16 matmul
    # (hipBLASLt) on the same shapes is that reference here: prefill
    # Y = X W^T on the 27B-class set at M = 32768 and the Qwen3-8B-like set at
    # M = 8192 (TFLOP/s), and decode GEMV at M = 1 and 16 (GB/s, weights
    # rotated over > 600 MB like the decode sweep).
    bf16_ref = {}
    same_loop = {}
    if not args.no_bf16_reference:
        sets = (("qwen3", P, 8192),) if args.prefill_set == "qwen3" else \
            (("27b", R, M), ("qwen3", P, 8192))
        for tag, S, m in sets:
            tot_b = tot_w = 0.0
            for r in S:
                L = r["L"]
                wb = torch.randn((L.n, L.k), dtype=torch.bfloat16, device=dev) * (L.k ** -0.5)
                yb = torch.empty((m, L.n), dtype=torch.bfloat16, device=dev)
                # this layer's activations quantized at m rows, for the W4A4
                # GEMM timed in the same loop as the bf16 product
                qlin.quantize_nvfp4(r["x"][:m], codes=r["codes"][:m], scales=r["scales"][:m],
                                    workspace=r["ws"], ts_out=r["ts"])
                gws = r["gws"] if r["gws_bytes"][m] else None

                def w4a4_gemm():
                    qlin.gemm_w4a4(r["codes"][:m], r["scales"][:m], r["ts"], r["blob"], m, L.n,
                                   L.k, y=r["y"][:m], workspace=gws)

                ref_ms, w_ms = [], []
                for _ in range(3):
                    torch.matmul(r["x"][:m], wb.t(), out=yb)
                    w4a4_gemm()
                torch.cuda.synchronize()
                for _ in range(10):   # alternating: the same clock and cache state for both
                    a, b = E(enable_timing=True), E(enable_timing=True)
                    a.record()
                    torch.matmul(r["x"][:m], wb.t(), out=yb)
                    b.record()
                    b.synchronize()
                    ref_ms.append(a.elapsed_time(b))
                    a, b = E(enable_timing=True), E(enable_timing=True)
                    a.record()
                    w4a4_gemm()
                    b.record()
                    b.synchronize()
                    w_ms.append(a.elapsed_time(b))
                med, wmed = float(np.median(ref_ms)), float(np.median(w_ms))
                bf16_ref[f"prefill_{tag}/{L.name}"] = {
                    "us": round(med * 1e3, 1),
                    "tflops": round(2.0 * m * L.n * L.k / med / 1e9, 1),
                    "w4a4_same_loop_us": round(wmed * 1e3, 1),
                    "w4a4_same_loop_tflops": round(2.0 * m * L.n * L.k / wmed / 1e9, 1)}
                tot_b, tot_w = tot_b + med, tot_w + wmed
                del wb, yb
            same_loop[f"{tag}_m{m}"] = round(tot_b / tot_w, 3)
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

    def speedup(tag, gemm_us):
        ref = [v["us"] for k, v in bf16_ref.items() if k.startswith(f"prefill_{tag}/")]
        return round(sum(ref) / gemm_us, 3) if ref else None

    # --------------------------------------------------- CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_rows, big, M)
        _progress(f"cpu baseline: {cpu['sample']}")

    traffic = _traffic_record(args.prefill_set)
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
            "workload": (("27B-class long-context prefill" if args.prefill_set == "27b" else
                          "Qwen3-8B-like prefill") +
                         f", NVFP4 W4A4 (quantize + GEMM, bf16 out) at M={M} tokens over "
                         "qkv/o_proj/gate_up/down, + W4A16 decode M=16 over the Qwen3-8B-like "
                         "shapes, + Gemma3-12B-like LUT2 decode M=8"),
            "m_prefill": M, "m_w4a16": M_DEC, "m_lut2": M_LUT,
            "prefill_layers_nk": [[L.n, L.k] for L in big.layers],
            "w4a16_layers_nk": [[L.n, L.k] for L in dec.layers],
            "lut2_layers_nk": [[L.n, L.k] for L in lut.layers],
            "activations": ("N(0,1), " + ("0.1% of elements x50" if args.prefill_set == "27b"
                                          else "1% of channels x10") +
                            ", bf16; every row drawn by the seeded generator"),
        },
        "roofline": {
            "kernel": "w4a4_coop_kernel (gemm_w4a4)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK["fp4"],
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK["fp4"], 4),
            "frac_f16_peak": round(achieved / PEAK["f16"], 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
            "per_launch": f"2*M*N*K FLOPs per launch averaged over the 4 layers "
                          f"({prefill_flops / len(R) / 1e12:.2f} TFLOP) / "
                          "mean event-timed duration of the timed launches; peak = dense FP4 "
                          "MFMA (the exact NVFP4 products run on the fp16 MFMA, whose dense "
                          "peak of 2500 TFLOP/s gives frac_f16_peak); traffic = HBM bytes per "
                          "launch averaged over the layers, from " +
                          TRAFFIC_PROFILE[args.prefill_set],
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
            "w4a4_gemm_speedup_vs_bf16": speedup(args.prefill_set, gemm_ms_step * 1e3),
            "prefill_27b": big_parts,
            "prefill_qwen3": qwen,
            "quantize_gemm_fused_qwen3": fused,
            "w4a4_gemm_speedup_vs_bf16_qwen3_m8192": (
                speedup("qwen3", sum(l["gemm_us"] for l in qwen["m8192"]["layers"]))
                if "m8192" in qwen else None),
            "w4a4_gemm_speedup_vs_bf16_same_loop": same_loop,
            "w4a16_gbps_mean_over_layers": _agg("w4a16", dec.ms),
            "lut2_gbps_mean_over_layers": _agg("lut2", lut.ms),
            "w4a16_sp24_gbps_mean_over_layers": _agg("w4a16_sp24", dec.ms),
            "decode_sweep": sweep,
            "bf16_reference": bf16_ref,
            "odp_weight_streaming": odp,
            "decode_timing": "events around the replay of a HIP graph of back-to-back launches "
                             "rotating over >600 MB of weight copies (Infinity Cache defeated)",
        },
    }
    print(json.dumps(out), flush=True)


def _oracle_weights(nvfp4, w):
    """The oracle's NVFP4 quantization of every weight row (row ranges on host
    threads; each row depends only on the whole tensor's scale)."""
    from concurrent.futures import ThreadPoolExecutor
    n, k = w.shape
    st = nvfp4.tensor_scale(w)
    codes = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // 16), dtype=np.uint8)

    def one(r0):
        c, s, _ = nvfp4.quantize(w[r0:r0 + 512], s_t=st)
        codes[r0:r0 + 512], scales[r0:r0 + 512] = c, s
    with ThreadPoolExecutor(max_workers=max(1, min(16, host_threads()))) as ex:
        list(ex.map(one, range(0, n, 512)))
    return codes, scales, st


def cpu_baseline(rows, cfg, M):
    """The oracle as it stands, timed on the host on a bounded sample of the
    headline workload.  For each of the four layers (weights quantized by the
    oracle beforehand, outside the timing: they are offline, as on the GPU):
    the tensor scale over the whole [M, K] activation (the method's first
    step), the NVFP4 quantization of the first `rows` token rows with that
    scale, and the fp64 W4A4 product of those rows with the layer's weights.
    value = 2 * rows * sum(N K) / the timed seconds."""
    sys.path.insert(0, ROOT)
    from oracle import nvfp4, gemm
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    cores = host_threads()
    dt, flops = 0.0, 0.0
    for li, L in enumerate(cfg.layers):
        wq = _oracle_weights(nvfp4, draw_weights(cfg.cid, li, L.n, L.k))
        xf = (draw_activations_bf16(cfg.cid, li, M, L.k, cfg.outliers).astype(np.uint32)
              << 16).view(np.float32)
        t0 = time.perf_counter()
        st = nvfp4.tensor_scale(xf)
        aq = nvfp4.quantize(xf[:rows], s_t=st)
        gemm.w4a4(*aq, *wq)
        dt += time.perf_counter() - t0
        flops += 2.0 * rows * L.n * L.k
        del xf, wq
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "blas_threads": blas, "kind": "oracle",
            "sample": f"the first {rows} of the {M} token rows of each of the 4 27B-class "
                      f"layers: tensor scale over all {M} rows, quantize of the sample, fp64 "
                      f"product; {dt:.1f} s of host time"}


if __name__ == "__main__":
    main()
