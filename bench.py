"""Benchmark: end-to-end 1920x1080 UNet denoise (input pass -> sixteen
3x3 convs -> output pass) on one MI355X, fp16 storage / fp32 accumulate.

Prints one JSON line.  `value` is megapixels of image per second over the
timed steps (inputs resident in HBM).  Per-kernel times come from HIP events
recorded between the launches of every N-th timed step (markers between
launches slow a step by ~10%, so the other steps run without them); the
roofline entry is the kernel symbol with the largest total time.  `cpu_baseline` times the CPU
oracle on one frame of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "megapixels/s for full UNet denoise at 1080p fp16; conv TFLOP/s and % MFMA peak"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30       # device copy timed for counter calibration
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv_kernels_1080p_hbm_traffic.md")
# Sources whose change invalidates the recorded traffic of the conv kernels.
TRAFFIC_SOURCES = ("unet_x3_convolution_amd/csrc/conv_f16.hip",
                   "unet_x3_convolution_amd/csrc/internal.h")


def conv_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_symbol(name):
    """'void oidn::(anonymous namespace)::conv3x3_f16_mfma<4, 8, false>(...)' -> 'conv3x3_f16_mfma<4, 8, false>'."""
    name = name.replace("(anonymous namespace)::", "").replace("oidn::", "").replace("void ", "")
    depth = 0
    for i, ch in enumerate(name):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


def recorded_traffic(symbol):
    """HBM bytes per launch of `symbol` from the committed counter summary,
    or None if there is none or the conv sources changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    block = text.split("```json", 1)[-1].split("```", 1)[0] if "```json" in text else ""
    try:
        rec = json.loads(block)
    except ValueError:
        return None
    if rec.get("source_sha256") != conv_source_hash():
        return None
    return rec.get("bytes_per_launch", {}).get(symbol)


def traffic_summary(fetch_dir, write_dir):
    """Writes TRAFFIC_FILE from two rocprofv3 --pmc runs of this script with
    --copy-calibration (FETCH_SIZE, then WRITE_SIZE): KiB per dispatch per
    kernel, each counter scaled by its reading for the 1 GiB device copy."""
    import csv
    import glob
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = []
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if len(copy) != 1:
            raise SystemExit(f"{d}: expected one device copy dispatch, found {len(copy)}")
        scale = COPY_BYTES / 1024.0 / copy[0]
        for r in rows:
            if "oidn::" not in r["Kernel_Name"]:
                continue
            e = per.setdefault(kernel_symbol(r["Kernel_Name"]), {})
            e.setdefault(counter, []).append(float(r["Counter_Value"]))
            e[counter + "_scale"] = scale
            e["copy_" + counter] = copy[0]
    lines = ["# HBM traffic per launch: kernels of the UNet denoise at 1920x1080, fp16", "",
             "Commands (repository root, one MI355X):", "", "```"]
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        lines.append(f"rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python -u bench.py "
                     "--steps 3 --warmup 1 --no-cpu-baseline --copy-calibration")
    lines += [f"python bench.py --traffic-summary {fetch_dir} {write_dir}", "```", ""]
    any_e = next(iter(per.values()))
    fs, ws = any_e["FETCH_SIZE_scale"], any_e["WRITE_SIZE_scale"]
    lines += [f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {any_e['copy_FETCH_SIZE']:.0f} KiB "
              f"and WRITE_SIZE = {any_e['copy_WRITE_SIZE']:.0f} KiB, so the counters are scaled by "
              f"{fs:.4f} (fetch) and {ws:.4f} (write).", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB per launch |",
              "|---|---|---|---|---|"]
    out = {}
    for sym, e in per.items():
        f = sum(e["FETCH_SIZE"]) / len(e["FETCH_SIZE"])
        w = sum(e["WRITE_SIZE"]) / len(e["WRITE_SIZE"])
        b = 1024.0 * (f * fs + w * ws)
        out[sym] = round(b)
        lines.append(f"| `{sym}` | {len(e['FETCH_SIZE'])} | {f:.0f} | {w:.0f} | {b / 1e6:.1f} |")
    lines += ["", "Averages are over every dispatch of the kernel symbol in the profiled run "
              "(all layers it serves), i.e. per launch.", "",
              "```json", json.dumps({"source_sha256": conv_source_hash(), "fetch_scale": fs,
                                     "write_scale": ws, "bytes_per_launch": out}, indent=1), "```"]
    open(TRAFFIC_FILE, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def standalone_passes(U, torch, W, H, tw, th, dtype, d_color, d_albedo, d_normal, launches):
    """The library's standalone bandwidth-bound passes at the 1080p shapes of
    the network (fp16 / bf16 storage): the input pass of the whole image into
    a tw x th tile, the output pass back, the 2x2 pool of enc_conv1's output
    and the materialised upsample + concat that dec_conv1a would read.  Each
    launch is timed alone with events on the stream it runs on, after 512 MB
    of other data were read (inputs not in the 256 MB Infinity Cache, which
    holds only clean lines, so the pass pays for no one else's write-back);
    reported: the median, its algorithmic bytes (inputs read once, outputs
    written once) and GB/s against the HBM peak."""
    import numpy as np
    dev = "cuda"
    h16 = torch.float16
    packed = torch.empty((th, tw, 12), dtype=h16, device=dev)
    net = torch.rand((th, tw, 4), dtype=torch.float32, device=dev)
    out = torch.empty((H, W, 4), dtype=torch.float32, device=dev)
    x32 = torch.rand((th, tw, 32), device=dev).to(h16)          # enc_conv1 output
    y32 = torch.empty((th // 2, tw // 2, 32), dtype=h16, device=dev)
    low = torch.rand((th // 2, tw // 2, 64), device=dev).to(h16)   # dec_conv2b output
    skip = torch.rand((th, tw, 12), device=dev).to(h16)          # packed input
    z = torch.empty((th, tw, 76), dtype=h16, device=dev)
    px, opx = tw * th, W * H
    cases = [
        ("input pass", "pack_input_kernel", opx * 48 + px * 24,
         lambda: U.oidn_pack_input(d_color, d_albedo, d_normal, W, H, 0, 0, tw, th, True,
                                   U.OIDN_TRANSFER_LOG, 1.0, packed, dtype)),
        ("output pass", "unpack_output_kernel", opx * (16 + 16 + 16),
         lambda: U.oidn_unpack_output(net, tw, th, 0, 0, d_color, W, H, 0, 0, W, H, True,
                                      U.OIDN_TRANSFER_LOG, 1.0, out)),
        ("pool2x2 32ch", "pool2x2_kernel", px * 64 + px // 4 * 64,
         lambda: U.oidn_pool2x2(x32, th, tw, 32, y32, dtype)),
        ("upsample+concat 64+12ch", "upcat_kernel", px // 4 * 128 + px * 24 + px * 152,
         lambda: U.oidn_upsample_concat(low, 64, skip, 12, th, tw, z, dtype)),
    ]
    flush = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = []
    for name, kernel, nbytes, launch in cases:
        launch()
        times = []
        for _ in range(launches):
            flush.sum()
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        gbs = nbytes / ms / 1e6
        res.append({"pass": name, "kernel": kernel, "us": round(ms * 1e3, 2),
                    "mb": round(nbytes / 1e6, 1), "gbs": round(gbs, 1),
                    "frac": round(gbs / PEAK_HBM_GBS, 4)})
        print(f"  {name:24s} {ms * 1e3:8.1f} us  {gbs:7.1f} GB/s  ({kernel}, inputs not cached)",
              file=sys.stderr)
    del flush
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--width", type=int, default=1920)
    ap.add_argument("--height", type=int, default=1080)
    ap.add_argument("--max-tile", type=int, default=0)
    ap.add_argument("--overlap", type=int, default=32)
    ap.add_argument("--cold-frames", type=int, default=20,
                    help="frames timed one by one after an Infinity Cache flush (0: none)")
    ap.add_argument("--dtype", choices=["f16", "bf16"], default="f16",
                    help="16-bit storage of the network (the metric is quoted on f16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass-launches", type=int, default=10,
                    help="cold-cache launches of each standalone bandwidth-bound pass (0: skip)")
    ap.add_argument("--events-every", type=int, default=10,
                    help="record per-kernel HIP events on every N-th timed step (event markers "
                         "between launches cost ~4 us each, so they are kept off the other steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the tiles of a frame, or whole frames, would be dealt out to one process "
              "per GPU)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as S
    import unet_x3_convolution_amd as U

    torch.cuda.set_device(0)
    W, H = args.width, args.height
    r = S.rng(0)
    color, albedo, normal = S.images(r, W, H)
    ws, bs = S.layer_params(r, U.unet_layer_shapes(9))
    dev = lambda a: torch.from_numpy(a).cuda()
    d_color, d_albedo, d_normal = dev(color), dev(albedo), dev(normal)
    DTYPE = {"f16": U.OIDN_F16, "bf16": U.OIDN_BF16}[args.dtype]
    wbuf = torch.empty(U.oidn_unet_weights_bytes(9, DTYPE), dtype=torch.uint8, device="cuda")
    U.oidn_unet_pack_weights(ws, bs, 9, DTYPE, wbuf)
    nbytes = U.oidn_unet_workspace_bytes(9, W, H, args.max_tile, args.overlap, DTYPE)
    work = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    tiles = U.oidn_plan_tiles(W, H, args.max_tile, args.overlap)
    tw, th = tiles[0][2], tiles[0][3]
    # tiles per launch: the per-kernel events cover the first batch
    nbatch = U.oidn_unet_tile_batch(9, W, H, args.max_tile, args.overlap, DTYPE)

    def step(events=None):
        if events is None:
            U.oidn_unet_forward(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                nbytes, out, DTYPE)
        else:
            U.oidn_unet_forward_timed(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                      U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                      nbytes, out, DTYPE, events)

    nk = 18  # input pass, 16 convs, output pass
    every = max(1, args.events_every)
    inst = [k for k in range(args.steps) if k % every == every - 1] or [args.steps - 1]
    events = {k: [U.oidn_event_create() for _ in range(nk + 1)] for k in inst}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {W}x{H}, {len(tiles)} tile(s) of {tw}x{th}, warmup {args.warmup} done",
          file=sys.stderr, flush=True)

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.steps):
        step(events.get(k))
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # cold Infinity Cache (256 MB): frames timed one by one, each after a
    # 512 MB buffer was written outside its timed interval (not `value`)
    cold = []
    if args.cold_frames > 0:
        flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.cold_frames):
            flush.fill_(1.0)
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del flush

    passes = (standalone_passes(U, torch, W, H, tw, th, DTYPE, d_color, d_albedo, d_normal,
                                args.pass_launches)
              if args.pass_launches > 0 and len(tiles) == 1 else [])

    # per-kernel durations (first tile of each instrumented step)
    dur = np.zeros((len(inst), nk))
    for n, k in enumerate(inst):
        for j in range(nk):
            dur[n, j] = U.oidn_event_elapsed_ms(events[k][j], events[k][j + 1])
    for evs in events.values():
        for e in evs:
            U.oidn_event_destroy(e)
    avg_ms = dur.mean(axis=0)

    # the first pair may run the input pass in its staging (input bit 1), the
    # last the output pass in its epilogue (output field 2)
    def pair_fields(layer):
        sym = U.oidn_unet_layer_kernel(9, layer, tw, th, DTYPE, nbatch)[0]
        if not sym.startswith("conv3x3_pair_"):
            return None
        return [int(f) for f in sym[sym.index("<") + 1:-1].split(", ")]
    first, last = pair_fields(0), pair_fields(U.oidn_unet_layer_count() - 1)
    in_fused = first is not None and (first[3] & 2) != 0
    out_fused = last is not None and last[2] == 2

    def layer_bytes(i, c0, c1, co, level, flags, px):
        """Algorithmic HBM bytes of one layer at 16-bit storage: its sources
        once (an upsampled source at half resolution; the network input as
        the three RGBA images plus the packed tile the input pass writes, or
        the packed tile) and its output once (pooled if the layer pools; the
        last layer's image write plus the alpha read when it runs the output
        pass, else its fp32 RGBA)."""
        st = lambda c: 4 * -(-c // 4)
        lanes = lambda c: 8 * -(-st(c) // 8)         # 16-byte channel groups
        if i == 0:
            b_in = px * (48 + 2 * lanes(c0)) if in_fused else px * 2 * lanes(c0)
        else:
            b_in = (px / 4 if c1 else px) * 2 * st(c0)
        if c1:
            b_in += px * 2 * lanes(c1)
        px_out = px / 4 if flags & U.OIDN_POOL2X2 else px
        if i == U.oidn_unet_layer_count() - 1:
            b_out = px_out * (32 if out_fused else 16)
        else:
            b_out = px_out * 2 * st(co)
        return b_in, b_out

    def roof_frac(flops, nbytes, ms):
        roof = min(PEAK_F16_TFLOPS, flops / nbytes * PEAK_HBM_GBS / 1e3)   # TFLOP/s
        return round(flops / ms / 1e9 / roof, 4), ("mfma" if roof == PEAK_F16_TFLOPS else "hbm")

    layers = []
    groups = {}
    conv_flops = conv_ms = 0.0
    prev_sym = None
    for i in range(U.oidn_unet_layer_count()):
        name, c0, c1, co, level, flags = U.oidn_unet_layer_info(9, i)
        px = (tw >> level) * (th >> level) * nbatch
        # algorithmic work of the method: a decoder conv reads its nearest-2x
        # upsampled source through 2 low-resolution rows per output row (the 3
        # ky taps pre-summed per row parity), so 6 taps for those c0 channels
        flops = 2.0 * px * co * ((6 * c0 + 9 * c1) if c1 else 9 * c0)
        ms = float(avg_ms[i + 1])
        sym, nblocks = U.oidn_unet_layer_kernel(9, i, tw, th, DTYPE, nbatch)
        b_in, b_out = layer_bytes(i, c0, c1, co, level, flags, px)
        conv_flops += flops
        conv_ms += ms
        g = groups.setdefault(sym, {"flops": 0.0, "ms": 0.0, "launches": 0})
        g["flops"] += flops
        g["ms"] += ms
        if sym.startswith("conv3x3_pair") and sym == prev_sym:
            # second layer of a fused pair: its work ran in the previous launch
            prev = layers[-1]
            prev["layer"] += "+" + name
            prev["flops"] += flops
            prev["us"] = round(prev["us"] + ms * 1e3, 2)
            prev["tflops"] = round(prev["flops"] / (prev["us"] / 1e3) / 1e9, 1)
            prev["bytes"] = prev["b_in"] + b_out     # the intermediate stays on chip
            prev["roof_frac"], prev["roof"] = roof_frac(prev["flops"], prev["bytes"],
                                                        prev["us"] / 1e3)
            print(f"  {name:11s}  (fused into the previous launch)", file=sys.stderr)
            prev_sym = None
            continue
        g["launches"] += 1
        prev_sym = sym
        fr, bound = roof_frac(flops, b_in + b_out, ms)
        layers.append({"layer": name, "us": round(ms * 1e3, 2), "flops": flops,
                       "tflops": round(flops / ms / 1e9, 1), "roof": bound, "roof_frac": fr,
                       "bytes": b_in + b_out, "b_in": b_in, "kernel": sym, "blocks": nblocks})
        print(f"  {name:11s} {ms * 1e3:8.1f} us  {flops / ms / 1e9:7.1f} TFLOP/s  {sym} x{nblocks}",
              file=sys.stderr)
    for L in layers:
        L["mb"] = round(L.pop("bytes") / 1e6, 1)
        del L["flops"], L["b_in"]
    px0 = tw * th
    pack_bytes = W * H * 48 + px0 * 16 * 2 if len(tiles) == 1 else None   # 16 lanes fp16 out
    unpack_bytes = W * H * (32 + 16)
    for j, nm, fused, where in ((0, "input pass", in_fused, "first conv's staging"),
                                (nk - 1, "output pass", out_fused, "last conv's epilogue")):
        note = f"  (in the {where})" if fused else ""
        print(f"  {nm:11s} {avg_ms[j] * 1e3:8.1f} us{note}", file=sys.stderr)
    sym, g = max(groups.items(), key=lambda kv: kv[1]["ms"])
    achieved = g["flops"] / g["ms"] / 1e9  # TFLOP/s
    mp = W * H / 1e6
    result = {
        "metric": METRIC,
        "value": round(mp / (ms_per_step / 1e3), 2),
        "unit": "MP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "kernel_timing": {"instrumented_steps": len(inst), "of_steps": args.steps,
                          "note": "HIP events between the launches of every "
                                  f"{every}-th timed step; the other steps run without markers"},
        "config": {"workload": f"UNet denoise {W}x{H}, {len(tiles)} tile(s) of {tw}x{th}, HDR log "
                               f"transfer, 9-channel input, {args.dtype} storage / fp32 accumulate",
                   "width": W, "height": H, "tiles": len(tiles), "tiles_per_launch": nbatch,
                   "max_tile": args.max_tile, "overlap": args.overlap},
        "conv_tflops": round(conv_flops / conv_ms / 1e9, 1),
        "conv_mfma_frac": round(conv_flops / conv_ms / 1e9 / PEAK_F16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": sym, "launches_per_step": g["launches"],
                     "avg_launch_us": round(g["ms"] / g["launches"] * 1e3, 2),
                     "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": recorded_traffic(sym)},
        "elementwise": {
            "input_pass_fused": in_fused,
            "input_pass_us": round(float(avg_ms[0]) * 1e3, 2),
            "input_pass_gbs": (round(pack_bytes / avg_ms[0] / 1e6, 1)
                               if pack_bytes and not in_fused else None),
            "output_pass_fused": out_fused,
            "output_pass_us": round(float(avg_ms[nk - 1]) * 1e3, 2),
            "output_pass_gbs": (round(unpack_bytes / avg_ms[nk - 1] / 1e6, 1)
                                if len(tiles) == 1 and not out_fused else None),
            "peak_gbs": PEAK_HBM_GBS,
            "standalone": passes},
        "layers": layers,
    }
    if cold:
        result["cold_cache"] = {"frames": len(cold), "flush_mb": 512,
                                "ms_median": round(float(np.median(cold)), 4),
                                "ms_p10": round(float(np.percentile(cold, 10)), 4),
                                "ms_p90": round(float(np.percentile(cold, 90)), 4),
                                "note": "each frame timed alone after writing 512 MB; not value"}

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        import threadpoolctl
        t = time.perf_counter()
        O.unet_forward(ws, bs, color, albedo, normal, True, 1.0, args.max_tile, args.overlap,
                       args.dtype)
        dt = time.perf_counter() - t
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
        result["cpu_baseline"] = {"value": round(W * H / 1e6 / dt, 4), "unit": "MP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the same {W}x{H} frame once, end to end (pack, "
                                            f"network, unpack), {args.dtype} storage emulated, float64 "
                                            f"sums; {dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
