"""Benchmark of the 4-bit grouped MoE layer on one MI355X.

One step = one full layer call (moe_route -> moe_grouped_gemm_q4 ->
moe_combine) over the 512-token prefill workload (H 2048, I 512, 256 experts
top-8 + 1 shared expert of I 512, 4-bit g64 weights), inputs resident in HBM.
The weights' code words are put in the tile-packed order once at load time
(moe_q4_prepack, outside every timed region); --layout rows times the
row-major order instead, and the other layout's 512-token figure is always
reported next to it.
Prints ONE JSON line.  The 2048-token prefill, batch-1 decode over 1000
tokens and the skewed 8192-token prefill in chunks of 2048 are timed too and
reported under "extra".

Warm and cold: repeating one layer lets part of its 455 MB of packed weights
stay in the 256 MB Infinity Cache between calls.  The cold figures cycle
through 4 layer copies with distinct weight bytes (1.8 GB), call i on copy
i mod 4, as consecutive layers of a model would.  Copies 1-3 are made on the
device from copy 0 by XOR-ing every code word with a per-copy constant and
copying the scales and biases: same shapes and routing, different bytes.

--calibrate-copy MB runs only a plain device-to-device copy of MB megabytes
(five times); rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE over it gives the
scale between those counters and true bytes.

The pages' two ablations are timed on the 512-token workload as well
(extra "ablation_unfused" and "ablation_host_routing"): the weights expanded to
bf16 in memory before a GEMM over bf16 weights, and the grouping done on the
host after a synchronising copy of the top-k.

--sweep runs only the tiling and chunking sweeps and prints them as one JSON
line: block_rows 16 / 32 / 64 (the row-block height of the block map and of
the GEMM tiles) on the 512- and 2048-token prefill, and chunk sizes 512 /
1024 / 2048 / 4096 of the bounded-chunk driver on the skewed 8192-token
prefill.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 MFMA
BYTES_PER_WEIGHT = 0.5 + 4.0 / 64   # code nibble + bf16 scale and bias per 64 weights
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_prefill512.txt")
KERNEL_SRC = os.path.join(ROOT, "bit_quantized_grouped_amd", "csrc", "gemm_q4.hip")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def layer_flops(T, H, I, k, I_sh):
    return 2.0 * (T * k * 3 * H * I + T * 3 * H * I_sh)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first; the GPU needs about 30 ms of work to reach its steady clock")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of back-to-back calls before each timed line (clock ramp)")
    ap.add_argument("--block-rows", type=int, default=32)
    ap.add_argument("--layout", choices=("tiles", "tiles-codes", "rows"), default="tiles",
                    help="weight layout of the timed layer, made at load time: tile-packed code "
                         "words with packed gate/up scale|bias words (moe_q4_prepack, "
                         "moe_q4_pack_scales), tile-packed code words only, or row-major")
    ap.add_argument("--other-layout", action="store_true",
                    help="also time prefill512 with the other code-word layout")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extra workloads to run")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB")
    ap.add_argument("--sweep", action="store_true", help="tiling and chunking sweeps only")
    ap.add_argument("--decode-tokens", type=int, default=1000,
                    help="decode line over the first N of the 1000 tokens (counter runs: fewer dispatches)")
    ap.add_argument("--no-floor", action="store_true", help="skip the decode launch-floor chains")
    return ap.parse_args()


def only_set(args):
    return set(filter(None, args.only.split(",")))


def settle(fn, torch, ms=150.0, max_calls=20000):
    """Run fn back to back until about `ms` of wall time has passed.  After
    host-bound phases (the host-synced ablation, graph capture) the GPU clocks
    are low; a count-based warm-up of a few calls would time the ramp."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < max_calls:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                break
    torch.cuda.synchronize()


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps   # ms per call


def read_ceiling(torch, bq, dev, nbytes=1 << 30, reps=20):
    """HBM read ceiling in bytes/s: the library's streaming-read probe over a
    buffer 4x the 256 MB Infinity Cache, timed back to back."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.fill_(1)
    sink = torch.empty(bq.read_probe_sink_words(nbytes), dtype=torch.int32, device=dev)
    ms = timed(lambda: bq.moe_read_probe(buf, sink), reps, 5, torch)
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3)


def device_facts(torch, dev):
    props = torch.cuda.get_device_properties(dev)
    facts = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
             "compute_units": props.multi_processor_count, "max_clock_mhz": None}
    try:   # rocminfo lists the agent's peak engine clock
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        for block in out.split("Agent ")[1:]:
            if "gfx950" in block:
                m = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", block)
                facts["max_clock_mhz"] = int(m.group(1)) if m else None
                break
    except (OSError, subprocess.SubprocessError):
        pass
    return facts


def kernel_src_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(ln.strip().split("=", 1) for ln in f if "=" in ln and not ln.startswith("#"))
        if kv.get("kernel_src_sha") != kernel_src_sha():
            return None
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy(mb, torch):
    n = mb * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}))


def host_grouping(idx, E, block_rows, max_blocks):
    """Histogram, exclusive offsets, stable scatter and block map of the top-k
    on the host (numpy): the host-synced routing baseline."""
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    np.cumsum(counts, out=offsets[1:])
    sorted_assign = np.argsort(flat, kind="stable").astype(np.int32)
    assign_row = np.empty_like(sorted_assign)
    assign_row[sorted_assign] = np.arange(flat.size, dtype=np.int32)
    nb = (counts + block_rows - 1) // block_rows
    block_expert = np.full(max_blocks, -1, np.int32)
    block_row = np.full(max_blocks, -1, np.int32)
    be = np.repeat(np.arange(E, dtype=np.int32), nb)
    first = np.repeat(np.cumsum(nb) - nb, nb)
    block_expert[:be.size] = be
    block_row[:be.size] = offsets[be] + block_rows * (np.arange(be.size) - first)
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                assign_row=assign_row, block_expert=block_expert, block_row=block_row,
                n_blocks=np.array([be.size], np.int32))


def cold_copy_mats(bq, mats, i):
    """Layer copy i for the cold runs: every code word XOR-ed with a per-copy constant,
    scale arrays copied (same shapes, layout and routing; distinct weight bytes)."""
    def one(m):
        clone = lambda t: None if t is None else t.clone()  # noqa: E731
        plain = None if m.plain is None else tuple(clone(t) for t in m.plain)
        return bq.DeviceQMat(m.codes ^ (0x01010101 * i), clone(m.scales), clone(m.biases),
                             m.layout, plain=plain)
    return [None if m is None else one(m) for m in mats]


def sweep(args, torch, bq, dev):
    from workload import CONFIGS, make_activations, make_weights
    cfg = CONFIGS["prefill512"]
    w = make_weights(cfg, seed=0)
    base = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, dev, prepack=True)
    mats = base.weight_mats()
    out = {"sweep": "block_rows x prefill, chunk_tokens x skewed prefill", "unit": "tokens/s",
           "weight_layout": "tile-packed codes, packed gate/up scale|bias words",
           "warmup": args.warmup, "block_rows": {},
           "chunk_tokens": {}}
    for name in ("prefill512", "prefill2048"):
        c = CONFIGS[name]
        xb, lgn = make_activations(c)
        x, lg = bq.bf16_from_bits(xb, dev), torch.from_numpy(lgn).to(dev)
        for br in (16, 32, 64):
            L = bq.MoeLayer.from_device(mats, c.H, c.I, c.I_sh, c.E, c.k, dev, block_rows=br)
            ms = timed(lambda: L.forward(x, lg), max(20, args.steps // 4), args.warmup, torch)
            out["block_rows"].setdefault(name, {})[br] = c.T / (ms * 1e-3)
            log(f"sweep {name} block_rows {br}: {ms*1e3:.1f} us/call")
            del L
    c = CONFIGS["skew8192"]
    xb, lgn = make_activations(c)
    x, lg = bq.bf16_from_bits(xb, dev), torch.from_numpy(lgn).to(dev)
    y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
    for chunk in (512, 1024, 2048, 4096):
        ws = base.forward_chunked(x, lg, chunk, y)
        ms = timed(lambda: base.forward_chunked(x, lg, chunk, y, ws), 10,
                   max(2, args.warmup // 40), torch)
        out["chunk_tokens"][chunk] = c.T / (ms * 1e-3)
        log(f"sweep skew8192 chunk {chunk}: {ms*1e3:.1f} us per 8192 tokens")
        del ws
    print(json.dumps(out))


def decode_launch_shapes(c):
    """(grid, threads) of moe_decode_q4's two launches for a layer config."""
    rows_per_wg = 4 * 2                       # 4 waves x 2 gate/up row pairs
    gateup = (-(-(c.I_sh + c.k * c.I) // rows_per_wg), 256)
    down = (c.H // 4, 512)                    # 4 output columns per workgroup, 8 waves
    return [list(gateup), list(down)]


def oracle_baselines(w_big, only, no_extra):
    """The CPU oracle (numpy fp64) timed on this host, one bounded sample per
    workload, about 20-30 s in all; tokens/s = tokens of the sample / its time."""
    import oracle
    from threadpoolctl import threadpool_info
    from workload import CONFIGS, make_activations, make_weights
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools
                             if p.get("user_api") == "blas"})) or None
    common = {"unit": "tokens/s", "cores": threads, "kind": "oracle", "blas": blas,
              "host_cpus": len(os.sched_getaffinity(0))}

    def run(w, xb, lg, k):
        t0 = time.perf_counter()
        oracle.moe_layer(xb, lg, w.gate, w.up, w.down, k, w.sh_gate, w.sh_up, w.sh_down)
        return time.perf_counter() - t0

    out = {}
    names = ["prefill512"]
    if not no_extra:
        names += [n for n in ("tiny", "prefill2048", "decode", "skew8192") if not only or n in only]
    for name in names:
        c = CONFIGS[name]
        w = make_weights(c, seed=0) if name == "tiny" else w_big
        xb, lg = make_activations(c)
        if name == "decode":      # single-token calls, as the GPU line runs them
            n = 10
            dt = sum(run(w, xb[t:t + 1], lg[t:t + 1], c.k) for t in range(n))
            sample = f"the first {n} of the 1000 tokens, one single-token layer call each"
        elif name == "skew8192":  # one bounded chunk
            n = c.chunk
            dt = run(w, xb[:n], lg[:n], c.k)
            sample = f"the first {n}-token chunk of the 8192 tokens (one of the four chunk calls)"
        else:
            n = c.T
            dt = run(w, xb, lg, c.k)
            sample = f"one full {n}-token layer call"
        out[name] = dict(common, value=n / dt, seconds=dt,
                         sample=f"{sample} ({dt:.1f} s; numpy fp64, BLAS threads {threads}, "
                                f"elementwise work single-threaded)")
        log(f"cpu oracle {name}: {dt:.2f} s for {n} tokens ({n/dt:,.1f} tok/s)")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, torch)
        return
    import bit_quantized_grouped_amd as bq
    from workload import CONFIGS, make_activations, make_weights

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        sweep(args, torch, bq, dev)
        return
    cfg = CONFIGS["prefill512"]
    log("generating weights")
    w = make_weights(cfg, seed=0)
    layer_rows = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, dev,
                             block_rows=args.block_rows)
    # load time, outside every timed region: the same weights with tile-packed code words
    layer_tiles = bq.MoeLayer.from_device(
        bq.prepacked_mats(layer_rows.weight_mats(), pack_scales=args.layout != "tiles-codes"),
        cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, dev, block_rows=args.block_rows)
    torch.cuda.synchronize()
    layer, other = ((layer_rows, layer_tiles) if args.layout == "rows"
                    else (layer_tiles, layer_rows))
    log(f"weights resident (timed layout: {args.layout})")
    br = layer.block_rows
    layers = [layer] + [
        bq.MoeLayer.from_device(cold_copy_mats(bq, layer.weight_mats(), i), cfg.H, cfg.I, cfg.I_sh,
                                cfg.E, cfg.k, dev, block_rows=args.block_rows)
        for i in range(1, 4)]
    log("4 layer copies resident (cold runs)")

    def cold(fn_of_layer):
        state = [0]

        def step():
            fn_of_layer(layers[state[0] % len(layers)])
            state[0] += 1
        return step

    def prep(c):
        xb, lg = make_activations(c)
        return bq.bf16_from_bits(xb, dev), torch.from_numpy(lg).to(dev)

    def gateup_alone_us(L, c, xx, lgx, steps):
        """Mean duration of the gate/up call alone, back to back on the routing of one
        layer call over (xx, lgx) (events on the launch stream)."""
        L.forward(xx, lgx)
        b = L.buffers(c.T)
        fn = lambda: bq.moe_expert_gateup_q4(xx, c.I, c.I_sh, c.E, c.k, L.block_rows,  # noqa: E731
                                             b["routing"], L.gate, L.up, L.sh_gate, L.sh_up,
                                             b["gemm_ws"])
        settle(fn, torch)
        return timed(fn, steps, 5, torch) * 1e3

    # ---------------- headline: prefill 512 ----------------
    x, lg = prep(cfg)
    T = cfg.T
    # the clocks need tens of ms of back-to-back work to reach their steady state, more
    # than a few warm-up calls give: settle on wall time first, then the counted warm-up
    settle(lambda: layer.forward(x, lg), torch, ms=args.settle_ms)
    ms = timed(lambda: layer.forward(x, lg), args.steps, args.warmup, torch)
    settle(cold(lambda L: L.forward(x, lg)), torch, ms=args.settle_ms)
    ms_cold = timed(cold(lambda L: L.forward(x, lg)), args.steps, args.warmup, torch)
    # per-call durations (events around each call) for the median
    per_call = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.forward(x, lg)
        e1.record()
        per_call.append((e0, e1))
    torch.cuda.synchronize()
    median_us = float(np.median([a.elapsed_time(b) for a, b in per_call])) * 1e3
    bufs = layer.buffers(T)
    counts = bufs["routing"].counts.cpu().numpy()
    touched = int(np.count_nonzero(counts))

    # per-phase durations: events on the launch stream around each ABI call
    r, ws_r, ws_g = bufs["routing"], bufs["route_ws"], bufs["gemm_ws"]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev = evs[i]
        ev[0].record()
        bq.moe_route(lg, cfg.k, br, r, ws_r)
        ev[1].record()
        bq.moe_expert_gateup_q4(x, cfg.I, cfg.I_sh, cfg.E, cfg.k, br, r, layer.gate, layer.up,
                                layer.sh_gate, layer.sh_up, ws_g)
        ev[2].record()
        bq.moe_expert_down_q4(T, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, br, r, layer.down,
                              layer.sh_down, bufs["expert_out"], bufs["shared_out"], ws_g)
        ev[3].record()
        bq.moe_combine(bufs["expert_out"], bufs["shared_out"], r, cfg.k, bufs["y"])
        ev[4].record()
    torch.cuda.synchronize()
    phase = [float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs])) * 1e-3 for j in range(4)]
    t_route, t_gu, t_dn, t_comb = phase

    # the gate/up launch duration for the roofline: launches back to back on the headline's
    # routing, rotating over the 4 layer copies (distinct weight bytes: no copy is still in the
    # Infinity Cache when its turn comes), events around the whole run
    gu_calls = [lambda L=L: bq.moe_expert_gateup_q4(x, cfg.I, cfg.I_sh, cfg.E, cfg.k, br, r, L.gate,
                                                     L.up, L.sh_gate, L.sh_up, ws_g)
                for L in layers]

    def gu_run():
        for f in gu_calls:
            f()

    settle(gu_run, torch, ms=50.0)
    t_gu_launch = timed(gu_run, max(5, args.steps // 4), 2, torch) * 1e-3 / len(gu_calls)

    # algorithmic bytes: packed weights of touched experts + shared expert, x in, logits in, y out
    gu_bytes_per_expert = int(2 * cfg.I * cfg.H * BYTES_PER_WEIGHT)
    expert_bytes = int(3 * cfg.I * cfg.H * BYTES_PER_WEIGHT)
    gu_bytes = (touched + 1) * gu_bytes_per_expert + T * cfg.H * 2
    layer_bytes = (touched + 1) * expert_bytes + T * cfg.H * 2 + T * cfg.E * 4 + T * cfg.H * 2
    flops = layer_flops(T, cfg.H, cfg.I, cfg.k, cfg.I_sh)
    t_layer = ms * 1e-3
    t_roof = max(flops / MFMA_BF16_PEAK, layer_bytes / HBM_PEAK)
    achieved = gu_bytes / t_gu_launch
    ceiling = read_ceiling(torch, bq, dev)
    log(f"measured HBM read ceiling: {ceiling/1e9:.0f} GB/s")
    result = {
        "metric": "MoE-layer tokens/s (prefill 512 tokens, 256 experts top-8 + shared, 4-bit g64)",
        "value": T / t_layer,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill512", "T": T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "I_shared": cfg.I_sh, "block_rows": br,
                   "weights": "4-bit codes, bf16 scale+bias per 64 along K",
                   "weight_layout": {
                       "tiles": "made at load time: tile-packed code words (moe_q4_prepack), gate/up "
                                "scale|bias words packed per 64-row tile and group "
                                "(moe_q4_pack_scales)",
                       "tiles-codes": "tile-packed code words at load time (moe_q4_prepack)",
                       "rows": "row-major"}[args.layout]},
        "roofline": {"bound": "hbm", "kernel": "grouped_q4_kernel gate/up+SwiGLU (moe_expert_gateup_q4)",
                     "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": read_traffic(),
                     "algorithmic_bytes": gu_bytes, "avg_launch_us": t_gu_launch * 1e6,
                     "launch_timing": "gate/up launches back to back over the 4 layer copies "
                                      "(cold weights), HIP events around the run",
                     "measured_read_ceiling": ceiling / 1e9,
                     "frac_of_measured_ceiling": achieved / ceiling},
        "device": device_facts(torch, dev),
        "library": bq.lib_fingerprint(),
        "layer": {"route_us": t_route * 1e6, "gateup_us": t_gu * 1e6, "down_us": t_dn * 1e6,
                  "combine_us": t_comb * 1e6, "touched_experts": touched,
                  "algorithmic_bytes": layer_bytes, "algorithmic_flops": flops,
                  "roofline_frac": t_roof / t_layer,
                  "mfma_frac": flops / t_layer / MFMA_BF16_PEAK,
                  "hbm_frac": layer_bytes / t_layer / HBM_PEAK,
                  "median_us_per_call": median_us,
                  "cold_tokens_per_s": T / (ms_cold * 1e-3), "cold_us_per_call": ms_cold * 1e3,
                  "cold_hbm_frac": layer_bytes / (ms_cold * 1e-3) / HBM_PEAK},
    }
    log(f"prefill512: {ms*1e3:.1f} us/call, {T/t_layer:,.0f} tok/s | phases in the call: route "
        f"{t_route*1e6:.1f} gateup {t_gu*1e6:.1f} down {t_dn*1e6:.1f} combine {t_comb*1e6:.1f} us; "
        f"gate/up launch {t_gu_launch*1e6:.1f} us ({achieved/1e9:.0f} GB/s); "
        f"cold {ms_cold*1e3:.1f} us/call")

    # ---------------- the other code-word layout, same weights ----------------
    if args.other_layout:
        other_name = "tiles" if args.layout == "rows" else "rows"
        ms_ot = timed(lambda: other.forward(x, lg), args.steps, args.warmup, torch)
        result["layer"][f"{other_name}_layout_us_per_call"] = ms_ot * 1e3
        result["layer"][f"{other_name}_layout_tokens_per_s"] = T / (ms_ot * 1e-3)
        log(f"prefill512 with {other_name} code layout: {ms_ot*1e3:.1f} us/call "
            f"({T/(ms_ot*1e-3):,.0f} tok/s)")

    # ---------------- the pages' two ablations (512 tokens) ----------------
    extra = {}
    if not args.no_extra and (not only_set(args) or "ablations" in only_set(args)):
        # the expansion reads row-major code words
        ms_unf = timed(lambda: layer_rows.forward_unfused(x, lg), max(20, args.steps // 4), 5, torch)
        y_fused = layer.forward(x, lg)["y"].clone()
        y_unf = layer_rows.forward_unfused(x, lg)["y"]
        torch.cuda.synchronize()
        err = float((y_unf.float() - y_fused.float()).abs().max() / y_fused.float().abs().max())
        extra["ablation_unfused"] = {
            "us_per_call": ms_unf * 1e3, "tokens_per_s": T / (ms_unf * 1e-3),
            "fused_speedup": ms_unf / ms,
            "max_rel_diff_vs_fused": err,
            "what": "route; expand the routed and shared experts' weights to bf16 in HBM "
                    "(moe_dequant_q4_bf16); gate/up and down GEMMs over bf16 weights; combine"}
        log(f"ablation unfused: {ms_unf*1e3:.1f} us/call; fused is {ms_unf/ms:.2f}x faster "
            f"(max rel diff {err:.1e})")
        hb = layer.buffers(T)
        hr = hb["routing"]
        dev_arrays = {n: getattr(hr, n) for n in ("counts", "offsets", "sorted_assign",
                                                  "assign_row", "block_expert", "block_row",
                                                  "n_blocks")}

        def host_routed():
            bq.moe_route(lg, cfg.k, br, hr, hb["route_ws"])   # top-k (grouping redone below)
            idx = hr.topk_idx.cpu().numpy()                  # synchronising copy
            g = host_grouping(idx, cfg.E, br, hr.max_blocks)
            for n, t in dev_arrays.items():
                t.copy_(torch.from_numpy(g[n]))
            bq.moe_grouped_gemm_q4(x, cfg.I, cfg.I_sh, cfg.E, cfg.k, br, hr, layer.gate, layer.up,
                                   layer.down, layer.sh_gate, layer.sh_up, layer.sh_down,
                                   hb["expert_out"], hb["shared_out"], hb["gemm_ws"])
            bq.moe_combine(hb["expert_out"], hb["shared_out"], hr, cfg.k, hb["y"])
        ms_host = timed(host_routed, max(20, args.steps // 4), 5, torch)
        same = bool(torch.equal(hb["y"].view(torch.int16), y_fused.view(torch.int16)))
        extra["ablation_host_routing"] = {
            "us_per_call": ms_host * 1e3, "tokens_per_s": T / (ms_host * 1e-3),
            "gpu_routing_speedup": ms_host / ms, "y_identical_to_gpu_routing": same,
            "what": "top-k on the GPU, then a synchronising copy of topk_idx to the host, "
                    "histogram/scan/stable scatter/block map in numpy, copies back, GEMMs, combine"}
        log(f"ablation host routing: {ms_host*1e3:.1f} us/call; GPU-resident routing is "
            f"{ms_host/ms:.2f}x faster (y identical: {same})")

    # ---------------- router projection (the input of routing) ----------------
    if not args.no_extra and (not only_set(args) or "router" in only_set(args)):
        from workload import make_router
        wr_bits, wg_bits = make_router(cfg)
        wr, wg = bq.bf16_from_bits(wr_bits, dev), bq.bf16_from_bits(wg_bits, dev)
        lg_r = torch.empty((T, cfg.E), dtype=torch.float32, device=dev)
        g_r = torch.empty(T, dtype=torch.float32, device=dev)
        def graphed(fn, n=20):
            # n calls captured once, so the host's per-call cost does not pace the GPU
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(n):
                    fn()
            ms_ = timed(gr.replay, 10, 2, torch) / n
            del gr
            return ms_
        ms_r = graphed(lambda: bq.moe_router(x, wr, lg_r, wg, g_r))
        ms_r1 = graphed(lambda: bq.moe_router(x[:1], wr, lg_r[:1], wg, g_r[:1]))
        r_bytes = T * cfg.H * 2 + (cfg.E + 1) * cfg.H * 2 + T * (cfg.E + 1) * 4
        extra["router"] = {"us_512": ms_r * 1e3, "us_1": ms_r1 * 1e3,
                           "hbm_frac_512": r_bytes / (ms_r * 1e-3) / HBM_PEAK,
                           "what": "logits = x W_r^T for 256 experts plus the shared-expert gate row"}
        log(f"router: {ms_r*1e3:.1f} us at 512 tokens, {ms_r1*1e3:.1f} us at 1 token")

    # ---------------- secondary workloads ----------------
    only = only_set(args)
    if not args.no_extra:
        if not only or "tiny" in only:
            c = CONFIGS["tiny"]
            wt = make_weights(c, seed=0)
            tiny = bq.MoeLayer(wt, c.H, c.I, c.I_sh, c.E, c.k, dev, prepack=True)
            xt, lgt = prep(c)
            settle(lambda: tiny.forward(xt, lgt), torch)
            mst = timed(lambda: tiny.forward(xt, lgt), max(20, args.steps), 10, torch)
            # the same calls replayed from a captured graph: the GPU's time per call,
            # without the host's per-call cost (which paces the eager loop at this size)
            y_t = tiny.forward(xt, lgt)["y"]
            torch.cuda.synchronize()
            want = y_t.clone()
            n_g = 20
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(n_g):
                    tiny.forward(xt, lgt)
            same = True
            for _ in range(3):
                y_t.zero_()
                gr.replay()
                torch.cuda.synchronize()
                same = same and bool(torch.equal(y_t, want))
            msg = timed(gr.replay, 10, 2, torch) / n_g
            del gr
            extra["tiny"] = {"tokens_per_s": c.T / (mst * 1e-3), "us_per_call": mst * 1e3,
                             "graph_us_per_call": msg * 1e3,
                             "graph_tokens_per_s": c.T / (msg * 1e-3),
                             "graph_matches_eager": same,
                             "what": "T 64, H 256, I 128, 16 experts top-2 + shared I 128: "
                                     "launch-bound (four kernels for 1 MB of weights); eager "
                                     "calls from Python, and the same calls replayed from a "
                                     "captured graph (each replay checked against eager)"}
            log(f"tiny: {mst*1e3:.1f} us/call eager, {msg*1e3:.1f} us/call from a graph "
                f"({c.T/(msg*1e-3):,.0f} tok/s; graph == eager: {same})")
            del tiny
        if not only or "prefill2048" in only:
            c = CONFIGS["prefill2048"]
            x2, lg2 = prep(c)
            settle(lambda: layer.forward(x2, lg2), torch)
            ms2 = timed(lambda: layer.forward(x2, lg2), max(10, args.steps // 4), 5, torch)
            settle(cold(lambda L: L.forward(x2, lg2)), torch)
            ms2c = timed(cold(lambda L: L.forward(x2, lg2)), max(10, args.steps // 4), 5, torch)
            cnt = layer.buffers(c.T)["routing"].counts.cpu().numpy()
            tch = int(np.count_nonzero(cnt))
            fl = layer_flops(c.T, c.H, c.I, c.k, c.I_sh)
            by = (tch + 1) * expert_bytes + c.T * c.H * 4 + c.T * c.E * 4
            t = ms2 * 1e-3
            gu = gateup_alone_us(layer, c, x2, lg2, max(10, args.steps // 4))
            fl_gu = fl * 2 / 3     # gate and up: two of the three matrices
            extra["prefill2048"] = {"tokens_per_s": c.T / t, "us_per_call": ms2 * 1e3,
                                    "mfma_frac": fl / t / MFMA_BF16_PEAK,
                                    "hbm_frac": by / t / HBM_PEAK,
                                    "roofline_frac": max(fl / MFMA_BF16_PEAK, by / HBM_PEAK) / t,
                                    "cold_tokens_per_s": c.T / (ms2c * 1e-3),
                                    "cold_us_per_call": ms2c * 1e3,
                                    "gateup_alone_us": gu,
                                    "gateup_alone_mfma_frac": fl_gu / (gu * 1e-6) / MFMA_BF16_PEAK}
            log(f"prefill2048: {ms2*1e3:.1f} us/call, {c.T/t:,.0f} tok/s, "
                f"MFMA {100*fl/t/MFMA_BF16_PEAK:.1f}%; cold {ms2c*1e3:.1f} us/call; gate/up alone "
                f"{gu:.1f} us (MFMA {100*fl_gu/(gu*1e-6)/MFMA_BF16_PEAK:.1f}%)")
            del x2, lg2
        if not only or "decode" in only:
            c = CONFIGS["decode"]
            xd, lgd = prep(c)
            n_dec = max(1, min(args.decode_tokens, c.T))
            xd, lgd = xd[:n_dec].contiguous(), lgd[:n_dec].contiguous()
            yd = torch.empty((n_dec, c.H), dtype=torch.bfloat16, device=dev)
            wsd = torch.empty(bq.decode_workspace_bytes(c.H, c.I, c.I_sh, c.E, c.k),
                              dtype=torch.uint8, device=dev)
            # 1000 single-token launches enqueued back to back from C, one per token
            seq = lambda: bq.moe_decode_q4_sequential(xd, lgd, c.I, c.I_sh, c.k,
                                                      *layer.decode_mats(), yd, wsd)
            settle(seq, torch)
            msd = timed(seq, 3, 1, torch)
            t_tok = msd * 1e-3 / n_dec
            by_tok = 9 * expert_bytes + c.H * 4 + c.E * 4
            # the three-call path at T = 1 over the first 100 tokens, for comparison
            n3 = min(100, n_dec)
            xs = [xd[i:i + 1] for i in range(n3)]
            ls = [lgd[i:i + 1] for i in range(n3)]

            def run_tokens():
                for i in range(n3):
                    layer.forward(xs[i], ls[i])

            t_three = timed(run_tokens, 2, 1, torch) * 1e-3 / n3

            # cold: token t on layer copy t mod 4.  The 1000 single-token calls are
            # captured once into a graph (no memset nodes) so the host does not pace
            # them; each replay is checked bit for bit against the same calls run eagerly.
            def decode_calls(y_out):
                for t in range(n_dec):
                    L = layers[t % len(layers)]
                    bq.moe_decode_q4(xd[t:t + 1], lgd[t:t + 1], c.I, c.I_sh, c.k, L.block_rows,
                                     *L.decode_mats(), None, y_out[t:t + 1], wsd)
            y_eager = torch.empty_like(yd)
            decode_calls(y_eager)
            y_graph = torch.zeros_like(yd)
            graph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph):
                decode_calls(y_graph)
            torch.cuda.synchronize()
            graph_ok = True
            for _ in range(2):
                y_graph.zero_()
                graph.replay()
                torch.cuda.synchronize()
                graph_ok &= bool(torch.equal(y_graph.view(torch.int16), y_eager.view(torch.int16)))
            settle(graph.replay, torch)
            t_cold = timed(graph.replay, 3, 1, torch) * 1e-3 / n_dec
            del graph
            # the floor under per-token launches: the same chain of 2 launches per token with
            # the decode kernels' grid shapes, empty, then with one dependent read each
            pb = torch.zeros(3, dtype=torch.int32, device=dev)
            shapes = decode_launch_shapes(c)
            floor = {False: float("nan"), True: float("nan")}
            gfloor = {False: float("nan"), True: float("nan")}
            for dep in (() if args.no_floor else (False, True)):
                run = lambda: bq.moe_launch_probe(pb, 2 * n_dec, *shapes, dep)  # noqa: E731
                settle(run, torch, ms=50.0)
                floor[dep] = timed(run, 3, 1, torch) * 1e-3 / n_dec
                # the same chain replayed from a graph: no host enqueue cost, the GPU's own floor
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    run()
                settle(g.replay, torch, ms=50.0)
                gfloor[dep] = timed(g.replay, 3, 1, torch) * 1e-3 / n_dec
                del g
            # a graph with an explicit parallel branch: per token, a shared-expert-sized launch
            # S on a second stream beside launch A, joined before launch B (dependent reads)
            gbranch = float("nan")
            if not args.no_floor:
                s_side = torch.cuda.Stream(device=dev)
                s_main = torch.cuda.current_stream(dev)
                sh_shape = [max(1, c.I_sh // 8), 256]

                def branch_tokens():
                    for _ in range(n_dec):
                        s_side.wait_stream(s_main)
                        bq.moe_launch_probe(pb, 1, sh_shape, sh_shape, True, stream=s_side)
                        bq.moe_launch_probe(pb, 1, shapes[0], shapes[0], True)
                        s_main.wait_stream(s_side)
                        bq.moe_launch_probe(pb, 1, shapes[1], shapes[1], True)

                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    branch_tokens()
                settle(g.replay, torch, ms=50.0)
                gbranch = timed(g.replay, 3, 1, torch) * 1e-3 / n_dec
                del g
            extra_floor = {"empty_us_per_token": floor[False] * 1e6,
                           "dependent_us_per_token": floor[True] * 1e6,
                           "graph_empty_us_per_token": gfloor[False] * 1e6,
                           "graph_dependent_us_per_token": gfloor[True] * 1e6,
                           "graph_branch_us_per_token": gbranch * 1e6,
                           "launch_shapes": shapes,
                           "what": "2 launches per token with the decode kernels' grids: empty, "
                                   "then each reading the word the previous launch wrote; eager "
                                   "(host enqueue rate) and replayed from a captured graph (the "
                                   "GPU's kernel-boundary floor); graph_branch: the dependent "
                                   "chain with a shared-expert-sized launch on a parallel graph "
                                   "branch beside the first launch, joined before the second"}
            log(f"decode floor: eager {floor[False]*1e6:.2f} / {floor[True]*1e6:.2f} us/token, "
                f"graph {gfloor[False]*1e6:.2f} / {gfloor[True]*1e6:.2f} us/token "
                f"(empty / one dependent read per launch); graph with a parallel branch "
                f"{gbranch*1e6:.2f} us/token")
            extra["decode"] = {"tokens_per_s": 1.0 / t_tok, "us_per_token": t_tok * 1e6,
                               "launch_floor": extra_floor,
                               "hbm_frac": by_tok / t_tok / HBM_PEAK,
                               "algorithmic_bytes_per_token": by_tok,
                               "path": "moe_decode_q4: two launches per token "
                                       "(top-k + gate/up + SwiGLU, then down + weighted sum)",
                               "three_call_us_per_token": t_three * 1e6,
                               "cold_us_per_token": t_cold * 1e6,
                               "cold_hbm_frac": by_tok / t_cold / HBM_PEAK,
                               "cold_graph_matches_eager": graph_ok,
                               "tokens": n_dec,
                               "note": f"warm: {n_dec} single-token calls back to back on one "
                                       "layer; cold: token t on layer copy t mod 4, replayed from "
                                       "a graph"}
            log(f"decode: {t_tok*1e6:.2f} us/token, HBM {100*by_tok/t_tok/HBM_PEAK:.1f}%; "
                f"cold {t_cold*1e6:.2f} us/token (graph == eager: {graph_ok}); "
                f"three-call path {t_three*1e6:.1f} us/token")
        if not only or "skew8192" in only:
            c = CONFIGS["skew8192"]
            xs_, lgs_ = prep(c)
            y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
            ws = layer.forward_chunked(xs_, lgs_, c.chunk, y)
            settle(lambda: layer.forward_chunked(xs_, lgs_, c.chunk, y, ws), torch)
            mss = timed(lambda: layer.forward_chunked(xs_, lgs_, c.chunk, y, ws), 10, 2, torch)
            t = mss * 1e-3
            fl = layer_flops(c.T, c.H, c.I, c.k, c.I_sh)
            extra["skew8192"] = {"tokens_per_s": c.T / t, "us_per_8192": mss * 1e3,
                                 "mfma_frac": fl / t / MFMA_BF16_PEAK}
            log(f"skew8192: {mss*1e3:.1f} us per 4 chunks, {c.T/t:,.0f} tok/s, "
                f"MFMA {100*fl/t/MFMA_BF16_PEAK:.1f}%")
    result["extra"] = extra

    # ---------------- CPU oracle baselines (rank 0, N = 1) ----------------
    if not args.no_cpu_baseline:
        base = oracle_baselines(w, only, args.no_extra)
        result["cpu_baseline"] = base.pop("prefill512")
        for name, b in base.items():
            extra.setdefault(name, {})["cpu_baseline"] = b
    print(json.dumps(result))


if __name__ == "__main__":
    main()
