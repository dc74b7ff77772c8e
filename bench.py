"""Benchmark: end-to-end 1920x1080 UNet denoise (input pass -> sixteen
3x3 convs -> output pass) on one MI355X, fp16 storage / fp32 accumulate.

Prints one JSON line.  `value` is megapixels of image per second over the
timed steps (inputs resident in HBM).  Per-launch times come from two HIP
events recorded around ONE launch of every second timed step, rotating over
the frame's launches (two markers per instrumented step, so the frame is not
slowed by a marker between every pair of launches); the roofline entry is the
kernel symbol with the largest total time.  `measured_peaks` times the
matrix cores on an MFMA-only stream and HBM on a device copy, for fractions
of measured next to published peaks.  `other_configs` times the single
fp32 conv, the fp16 conv ladder, the network on a 512 x 512 tile and the
3840 x 2160 frame in 1024-pixel tiles.  `cpu_baseline` times the CPU oracle
on one frame of the same workload.
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
    """'void oidn::(anonymous namespace)::conv3x3_f16_mfma<4, 8, 4, false>(...)' -> 'conv3x3_f16_mfma<4, 8, 4, false>'."""
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
        # the 1 GiB calibration copy is the largest device copy of the run
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copy:
            raise SystemExit(f"{d}: no device copy dispatch (run with --copy-calibration)")
        copy = [max(copy)]
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
                     "--steps 3 --warmup 1 --no-cpu-baseline --no-peaks --no-other-configs "
                     "--pass-launches 0 --cold-frames 0 --copy-calibration")
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


PEAK_F32_TFLOPS = 157.3   # MI355X fp32 (matrix) peak, the fp32 path's roof


def cpu_info():
    """Model name, sockets x cores per socket, and the logical CPUs this
    process may run on (lscpu's fields, read from /proc/cpuinfo and the
    scheduler affinity)."""
    model, phys = None, set()
    try:
        cur = {}
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if cur.get("physical id") is not None and cur.get("core id") is not None:
                    phys.add((cur["physical id"], cur["core id"]))
                cur = {}
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            cur[k] = v
            if k == "model name" and model is None:
                model = v
        if cur.get("physical id") is not None and cur.get("core id") is not None:
            phys.add((cur["physical id"], cur["core id"]))
    except OSError:
        pass
    try:
        logical = len(os.sched_getaffinity(0))
    except AttributeError:
        logical = os.cpu_count()
    return {"model": model, "physical_cores": len(phys) or None, "logical_cpus_allowed": logical}


def blas_threads():
    import threadpoolctl
    return max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])


def measured_peaks(U, torch):
    """What this device sustains: an MFMA-only stream (fp16, 16 waves per CU,
    no memory traffic), a 1 GiB device copy (read + write) and a 1 GiB
    streaming read, each the median of 5 timed runs."""
    import numpy as np
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=5):
        fn()
        ts = []
        for _ in range(n):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    blocks, iters = 256 * 4, 4096
    flops = U.oidn_calibrate_mfma(U.OIDN_F16, iters, blocks, sink)
    ms = timed(lambda: U.oidn_calibrate_mfma(U.OIDN_F16, iters, blocks, sink))
    mfma = flops / ms / 1e9
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms_copy = timed(lambda: b.copy_(a))
    ms_read = timed(lambda: U.oidn_calibrate_read(a, COPY_BYTES, sink))
    del a, b
    return {"mfma_f16_tflops": round(mfma, 1), "mfma_f16_frac_of_published": round(mfma / PEAK_F16_TFLOPS, 4),
            "hbm_copy_gbs": round(2 * COPY_BYTES / ms_copy / 1e6, 1),
            "hbm_read_gbs": round(COPY_BYTES / ms_read / 1e6, 1),
            "method": f"MFMA stream: {blocks} workgroups x 4 waves x {iters} x 8 independent "
                      "v_mfma_f32_16x16x32_f16 (oidn_calibrate_mfma); HBM: 1 GiB device copy "
                      "(read + write bytes) and a 1 GiB streaming read (oidn_calibrate_read); medians of 5"}


def unet_flops(U, w, h):
    """Algorithmic FLOPs of the network on a w x h tile, from the library's
    layer table (decoder convs' upsampled channels at 6 taps, as above)."""
    fl = 0.0
    for i in range(U.oidn_unet_layer_count()):
        _, c0, c1, co, level, _ = U.oidn_unet_layer_info(9, i)
        fl += 2.0 * (w >> level) * (h >> level) * co * ((6 * c0 + 9 * c1) if c1 else 9 * c0)
    return fl


def other_configs(U, torch, S, dtype_name):
    """The other workloads, timed on the GPU with events around repeated
    launches (inputs resident): the single fp32 conv (64 x 64, 9 -> 32), the
    fp16 conv ladder at 256 x 256 (five conv + pool stages), the network on
    one packed 512 x 512 tile, and the 3840 x 2160 frame in 1024-pixel tiles
    (overlap 32, 12 tiles, batched)."""
    import numpy as np
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # config 1: fp32 conv
    r = S.rng(0)
    x = S.uniform_activation(r, 64, 64, 9, 12)
    w, b = S.he_normal(r, 32, 9), S.bias(r, 32)
    pk = torch.empty(U.oidn_conv3x3_weights_bytes(9, 0, 32, U.OIDN_F32), dtype=torch.uint8, device="cuda")
    U.oidn_conv3x3_pack_weights(w, b, 9, 0, 32, U.OIDN_F32, pk)
    dx = torch.from_numpy(x).cuda()
    dy = torch.empty((64, 64, 32), dtype=torch.float32, device="cuda")
    ms = timed(lambda: U.oidn_conv3x3(dx, 64, 64, 9, pk, dy, 32, U.OIDN_F32, U.OIDN_F32, U.OIDN_RELU), 200)
    fl = 2.0 * 64 * 64 * 32 * 81
    out["conv_fp32_64x64_9to32"] = {"us": round(ms * 1e3, 2), "tflops": round(fl / ms / 1e9, 3),
                                    "frac_of_fp32_peak": round(fl / ms / 1e9 / PEAK_F32_TFLOPS, 5),
                                    "kernel": U.oidn_conv3x3_kernel(64, 64, 9, 0, 32, U.OIDN_F32,
                                                                    U.OIDN_F32, U.OIDN_RELU)[0]}
    # the same fp32 kernel at a size that fills the GPU: 32 -> 32 at 1920 x 1088
    xb = torch.rand((1088, 1920, 32), dtype=torch.float32, device="cuda")
    wb, bb = S.he_normal(r, 32, 32), S.bias(r, 32)
    pkb = torch.empty(U.oidn_conv3x3_weights_bytes(32, 0, 32, U.OIDN_F32), dtype=torch.uint8, device="cuda")
    U.oidn_conv3x3_pack_weights(wb, bb, 32, 0, 32, U.OIDN_F32, pkb)
    yb = torch.empty((1088, 1920, 32), dtype=torch.float32, device="cuda")
    ms = timed(lambda: U.oidn_conv3x3(xb, 1088, 1920, 32, pkb, yb, 32, U.OIDN_F32, U.OIDN_F32,
                                      U.OIDN_RELU), 20)
    fl = 2.0 * 1088 * 1920 * 32 * 9 * 32
    out["conv_fp32_1088x1920_32to32"] = {"us": round(ms * 1e3, 2), "tflops": round(fl / ms / 1e9, 2),
                                         "frac_of_fp32_peak": round(fl / ms / 1e9 / PEAK_F32_TFLOPS, 4),
                                         "kernel": U.oidn_conv3x3_kernel(1088, 1920, 32, 0, 32, U.OIDN_F32,
                                                                         U.OIDN_F32, U.OIDN_RELU)[0]}
    del xb, yb
    # config 2: fp16 ladder
    r = S.rng(0)
    x = S.relu_normal_activation(r, 256, 256, 32, 32).astype(np.float16)   # round to nearest even
    chans = [32, 48, 64, 80, 96, 96]
    flags = U.OIDN_RELU | U.OIDN_POOL2X2
    bufs = [torch.from_numpy(x).cuda()]
    packs, fl = [], 0.0
    hw = 256
    for i in range(5):
        cin, cout = chans[i], chans[i + 1]
        wt, bb = S.he_normal(r, cout, cin), S.bias(r, cout)
        pkb = torch.empty(U.oidn_conv3x3_weights_bytes(cin, 0, cout, U.OIDN_F16), dtype=torch.uint8,
                          device="cuda")
        U.oidn_conv3x3_pack_weights(wt, bb, cin, 0, cout, U.OIDN_F16, pkb)
        packs.append(pkb)
        bufs.append(torch.empty((hw // 2, hw // 2, cout), dtype=torch.float16, device="cuda"))
        fl += 2.0 * hw * hw * cout * 9 * cin
        hw //= 2

    def ladder():
        s = 256
        for i in range(5):
            U.oidn_conv3x3(bufs[i], s, s, chans[i], packs[i], bufs[i + 1], chans[i + 1], U.OIDN_F16,
                           U.OIDN_F16, flags)
            s //= 2
    ms = timed(ladder, 50)
    out["conv_ladder_f16_256"] = {"us": round(ms * 1e3, 2), "tflops": round(fl / ms / 1e9, 1),
                                  "frac_of_f16_peak": round(fl / ms / 1e9 / PEAK_F16_TFLOPS, 4),
                                  "launches": 5}
    # config 3: network on one packed 512 x 512 tile
    DT = {"f16": U.OIDN_F16, "bf16": U.OIDN_BF16}[dtype_name]
    r = S.rng(0)
    color, albedo, normal = S.images(r, 512, 512)
    ws, bs = S.layer_params(r, U.unet_layer_shapes(9))
    wbuf = torch.empty(U.oidn_unet_weights_bytes(9, DT), dtype=torch.uint8, device="cuda")
    U.oidn_unet_pack_weights(ws, bs, 9, DT, wbuf)
    dev = lambda a: torch.from_numpy(a).cuda()
    packed = torch.empty((512, 512, 12), dtype=torch.float16, device="cuda")
    U.oidn_pack_input(dev(color), dev(albedo), dev(normal), 512, 512, 0, 0, 512, 512, True,
                      U.OIDN_TRANSFER_LOG, 1.0, packed, DT)
    nb = U.oidn_unet_packed_workspace_bytes(9, 512, 512, DT)
    work = torch.empty(nb, dtype=torch.uint8, device="cuda")
    net = torch.empty((512, 512, 4), dtype=torch.float32, device="cuda")
    ms = timed(lambda: U.oidn_unet_forward_packed(wbuf, 9, packed, 512, 512, work, nb, net, DT), 50)
    fl = unet_flops(U, 512, 512)
    out["unet_512_packed"] = {"us": round(ms * 1e3, 2), "mp_s": round(512 * 512 / 1e6 / (ms / 1e3), 1),
                              "conv_tflops": round(fl / ms / 1e9, 1),
                              "frac_of_f16_peak": round(fl / ms / 1e9 / PEAK_F16_TFLOPS, 4)}
    del work
    # config 5: 3840 x 2160 in 1024-pixel tiles
    W5, H5 = 3840, 2160
    r = S.rng(0)
    color, albedo, normal = S.images(r, W5, H5)
    ws, bs = S.layer_params(r, U.unet_layer_shapes(9))
    U.oidn_unet_pack_weights(ws, bs, 9, DT, wbuf)
    nb = U.oidn_unet_workspace_bytes(9, W5, H5, 1024, 32, DT)
    work = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o5 = torch.empty((H5, W5, 4), dtype=torch.float32, device="cuda")
    dc, da, dn = dev(color), dev(albedo), dev(normal)
    ms = timed(lambda: U.oidn_unet_forward(wbuf, 9, dc, da, dn, W5, H5, True, U.OIDN_TRANSFER_LOG,
                                           1.0, 1024, 32, work, nb, o5, DT), 10)
    tiles = U.oidn_plan_tiles(W5, H5, 1024, 32)
    fl = unet_flops(U, tiles[0][2], tiles[0][3]) * len(tiles)
    out["unet_3840x2160_tiled"] = {"ms": round(ms, 4), "mp_s": round(W5 * H5 / 1e6 / (ms / 1e3), 1),
                                   "conv_tflops": round(fl / ms / 1e9, 1),
                                   "tiles": len(tiles), "tile": list(tiles[0][2:4]),
                                   "tiles_per_launch": U.oidn_unet_tile_batch(9, W5, H5, 1024, 32, DT)}
    del work, o5
    return out


def oracle_configs(out_path):
    """The CPU oracle on the other workloads (a reported baseline, not a
    target): wall time and rates on all host threads and, for the single
    conv and the ladder, on one thread.  Writes a markdown summary."""
    import numpy as np
    import threadpoolctl

    import synthetic as S
    from oracle import oracle as O
    rows = []

    def run(name, fn, work, unit, threads=None):
        if threads is None:
            t = time.perf_counter()
            fn()
            dt = time.perf_counter() - t
            used = blas_threads()
        else:
            with threadpoolctl.threadpool_limits(threads):
                t = time.perf_counter()
                fn()
                dt = time.perf_counter() - t
            used = threads
        rows.append((name, used, dt, work / dt, unit))
        print(f"  {name:42s} threads={used:3d} {dt:8.3f} s  {work / dt:10.4g} {unit}", flush=True)

    r = S.rng(0)
    x = S.uniform_activation(r, 64, 64, 9, 12)
    w, b = S.he_normal(r, 32, 9), S.bias(r, 32)
    c1 = lambda: O.conv3x3(x, 9, w, b, True, "f32")
    run("config 1: conv 64x64 9->32 fp32", c1, 2.0 * 64 * 64 * 32 * 81 / 1e9, "GFLOP/s")
    run("config 1: conv 64x64 9->32 fp32", c1, 2.0 * 64 * 64 * 32 * 81 / 1e9, "GFLOP/s", threads=1)
    r = S.rng(0)
    x2 = O.round_to(S.relu_normal_activation(r, 256, 256, 32, 32), "f16")
    chans = [32, 48, 64, 80, 96, 96]
    wl = []
    for i in range(5):
        wt = S.he_normal(r, chans[i + 1], chans[i])
        wl.append((wt, S.bias(r, chans[i + 1])))
    fl2 = sum(2.0 * (256 >> i) ** 2 * chans[i + 1] * 9 * chans[i] for i in range(5))

    def ladder():
        y = x2
        for i in range(5):
            y = O.pool2x2(O.conv3x3(y, chans[i], wl[i][0], wl[i][1], True, "f16"))
    run("config 2: conv ladder 256^2 fp16 storage", ladder, fl2 / 1e9, "GFLOP/s")
    run("config 2: conv ladder 256^2 fp16 storage", ladder, fl2 / 1e9, "GFLOP/s", threads=1)
    r = S.rng(0)
    color, albedo, normal = S.images(r, 512, 512)
    ws, bs = S.layer_params(r, O.unet_layer_shapes(9))
    packed = O.pack_input(color, albedo, normal, 0, 0, 512, 512, True, 1.0, "f16")
    run("config 3: network 512x512 fp16 storage", lambda: O.unet_forward_packed(ws, bs, packed, 9, "f16"),
        512 * 512 / 1e6, "MP/s")
    r = S.rng(0)
    color, albedo, normal = S.images(r, 3840, 2160)
    ws, bs = S.layer_params(r, O.unet_layer_shapes(9))
    run("config 5: 3840x2160, 12 tiles of 1024x784", lambda: O.unet_forward(
        ws, bs, color, albedo, normal, True, 1.0, 1024, 32, "f16"), 3840 * 2160 / 1e6, "MP/s")
    info = cpu_info()
    lines = ["# CPU oracle timings (reported baseline, not a target)", "",
             "Command (repository root, on the GPU box's host):", "", "```",
             f"python bench.py --oracle-configs {os.path.relpath(out_path, ROOT)}", "```", "",
             f"Host: {info['model']}; {info['physical_cores']} physical cores, "
             f"{info['logical_cpus_allowed']} logical CPUs allowed to the process. The oracle is "
             "numpy with float64 sums; `threads` is the BLAS thread count it ran with.", "",
             "| workload | threads | wall s | rate |", "|---|---|---|---|"]
    for name, used, dt, rate, unit in rows:
        lines.append(f"| {name} | {used} | {dt:.3f} | {rate:.4g} {unit} |")
    open(out_path, "w").write("\n".join(lines) + "\n")


def mfma_frames(pmc_dir):
    """Per-dispatch counters of one rocprofv3 --pmc run, cut into frames
    (the launch sequence that starts with the frame's first kernel)."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    by, names = {}, {}
    for r in rows:
        if "oidn::" not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        by.setdefault(d, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        names[d] = kernel_symbol(r["Kernel_Name"])
    order = sorted(by)
    first = names[order[0]]
    starts = [i for i, d in enumerate(order) if names[d] == first]
    period = starts[1] - starts[0] if len(starts) > 1 else len(order)
    frames = [order[s:s + period] for s in starts if s + period <= len(order)]
    return by, names, frames, period


def mfma_rows(pmc_dir):
    """(kernel, MFMA busy, LDS conflict, MFMA GFLOP) per launch of the frame:
    medians over the run's frames."""
    import statistics
    by, names, frames, period = mfma_frames(pmc_dir)
    out = []
    for j in range(period):
        ds = [fr[j] for fr in frames]
        util = statistics.median(by[d]["SQ_VALU_MFMA_BUSY_CYCLES"] / (by[d]["GRBM_GUI_ACTIVE"] / 8 * 1024)
                                 for d in ds)
        conf = statistics.median(by[d]["SQ_LDS_BANK_CONFLICT"] / max(1.0, by[d]["SQ_LDS_IDX_ACTIVE"])
                                 for d in ds)
        gf = statistics.median(by[d]["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / 1e9 for d in ds)
        out.append((names[frames[0][j]], util, conf, gf))
    return out, len(frames)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
                 "SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16")


def mfma_summary(pmc_dir, out_path, base_dir=None, base_rev=None):
    """Per-launch MFMA busy fraction and LDS bank-conflict share of the
    frame's kernels from one rocprofv3 --pmc run (SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE,
    SQ_INSTS_VALU_MFMA_MOPS_F16): MFMA busy = busy cycles / (GPU active
    cycles per XCD x 1024 SIMDs).  With base_dir, the same counters of an
    earlier revision's run (base_rev) in columns beside them."""
    rows, nframes = mfma_rows(pmc_dir)
    base = mfma_rows(base_dir)[0] if base_dir else None
    cmd = (f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d {pmc_dir} -o run -- "
           "python -u bench.py --steps 3 --warmup 1 --no-cpu-baseline --pass-launches 0 --cold-frames 0 "
           "--no-peaks --no-other-configs")
    lines = ["# MFMA utilisation and LDS bank conflicts per launch: UNet denoise 1920x1080, fp16", "",
             "Commands (repository root, one MI355X):", "", "```", cmd]
    if base_dir:
        lines += [f"# the earlier revision, in a checkout of commit {base_rev} (its bench.py has no "
                  "--no-peaks / --no-other-configs):",
                  f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d {base_dir} -o run -- "
                  "python -u bench.py --steps 3 --warmup 1 --no-cpu-baseline --pass-launches 0 --cold-frames 0",
                  f"python bench.py --mfma-summary {pmc_dir} {base_dir} {base_rev}"]
    else:
        lines.append(f"python bench.py --mfma-summary {pmc_dir}")
    lines += ["```", "",
              "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
              "LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (share of the LDS's "
              "active cycles lost to bank conflicts); MFMA work = SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 "
              f"FLOP. Medians over {nframes} frames (counters serialise the kernels).", ""]
    if base:
        lines += [f"| launch | kernel | MFMA busy | LDS conflict | MFMA GFLOP | MFMA busy at {base_rev} "
                  f"| LDS conflict at {base_rev} |", "|---|---|---|---|---|---|---|"]
    else:
        lines += ["| launch | kernel | MFMA busy | LDS conflict | MFMA GFLOP |", "|---|---|---|---|---|"]
    changed = []
    for j, (name, util, conf, gf) in enumerate(rows):
        line = f"| {j} | `{name}` | {util:.3f} | {conf:.3f} | {gf:.2f} |"
        if base and j < len(base):
            # the same launch of the frame, whichever kernel served it then
            line += f" {base[j][1]:.3f} | {base[j][2]:.3f} |"
            if base[j][0] != name:
                changed.append(f"launch {j} ran `{base[j][0]}` at {base_rev}")
        elif base:
            line += " - | - |"
        lines.append(line)
    if changed:
        lines += ["", "Kernels that changed between the two columns: " + "; ".join(changed) + "."]
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=140)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--width", type=int, default=1920)
    ap.add_argument("--height", type=int, default=1080)
    ap.add_argument("--max-tile", type=int, default=0)
    ap.add_argument("--overlap", type=int, default=32)
    ap.add_argument("--cold-frames", type=int, default=20,
                    help="frames timed one by one after an Infinity Cache flush (0: none)")
    ap.add_argument("--dtype", choices=["f16", "bf16"], default="f16",
                    help="16-bit storage of the network (the metric is quoted on f16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / HBM ceilings")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the single conv, ladder, 512^2 and 4K tiled timings")
    ap.add_argument("--pass-launches", type=int, default=10,
                    help="cold-cache launches of each standalone bandwidth-bound pass (0: skip)")
    ap.add_argument("--events-every", type=int, default=2,
                    help="every N-th timed step records two HIP events around one of the frame's "
                         "launches (rotating over them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--mfma-summary", nargs="+", metavar="PMC_DIR",
                    help="write the MFMA-busy / LDS-conflict summary from a rocprofv3 --pmc run "
                         "(optionally followed by an earlier revision's run directory and its "
                         "commit) and exit")
    ap.add_argument("--oracle-configs", metavar="OUT_MD",
                    help="time the CPU oracle on the other workloads, write OUT_MD and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        base = args.mfma_summary[1:3]
        mfma_summary(args.mfma_summary[0], os.path.join(ROOT, "profiles", "conv_kernels_1080p_mfma_util.md"),
                     *(base if len(base) == 2 else []))
        return
    if args.oracle_configs:
        oracle_configs(args.oracle_configs)
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
    # tiles per launch: the per-launch events cover the first batch
    nbatch = U.oidn_unet_tile_batch(9, W, H, args.max_tile, args.overlap, DTYPE)
    nlayers = U.oidn_unet_layer_count()
    syms = [U.oidn_unet_layer_kernel(9, i, tw, th, DTYPE, nbatch) for i in range(nlayers)]
    # the frame's launches: a fused pair's second layer runs in the first's launch
    launches, i = [], 0
    while i < nlayers:
        launches.append(i)
        i += 2 if syms[i][0].startswith("conv3x3_pair") else 1
    nk = nlayers + 2   # events: input pass, layers, output pass

    def step(events=None):
        if events is None:
            U.oidn_unet_forward(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                nbytes, out, DTYPE)
        else:
            U.oidn_unet_forward_timed(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                      U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                      nbytes, out, DTYPE, events)

    every = max(1, args.events_every)
    inst = [k for k in range(args.steps) if k % every == every - 1]
    ev_pool = [U.oidn_event_create() for _ in range(2 * len(inst))]
    plan = {}   # step -> (launch layer, events array)
    for n, k in enumerate(inst):
        li = launches[n % len(launches)]
        arr = [0] * (nk + 1)
        arr[1 + li], arr[2 + li] = ev_pool[2 * n], ev_pool[2 * n + 1]
        plan[k] = (li, arr)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {W}x{H}, {len(tiles)} tile(s) of {tw}x{th}, warmup {args.warmup} done",
          file=sys.stderr, flush=True)

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.steps):
        step(plan[k][1] if k in plan else None)
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

    # per-launch durations: median over the steps that timed that launch
    samples = {li: [] for li in launches}
    for k, (li, arr) in plan.items():
        samples[li].append(U.oidn_event_elapsed_ms(arr[1 + li], arr[2 + li]))
    for e in ev_pool:
        U.oidn_event_destroy(e)
    launch_ms_events = {li: float(np.median(v)) if v else float("nan") for li, v in samples.items()}
    # Each event interval also holds its launch's dispatch gap, which the
    # unmarked frame overlaps with the previous kernel: scale the medians so
    # that they sum to the unmarked step (never up).
    scale = min(1.0, ms_per_step / sum(launch_ms_events.values()))
    launch_ms = {li: v * scale for li, v in launch_ms_events.items()}

    # the first pair may run the input pass in its staging (input bit 1), the
    # last the output pass in its epilogue (output field 2)
    def pair_fields(layer):
        sym = syms[layer][0]
        if not sym.startswith("conv3x3_pair_"):
            return None
        return [int(f) for f in sym[sym.index("<") + 1:-1].split(", ")]
    first, last = pair_fields(0), pair_fields(nlayers - 1)
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
        if i == nlayers - 1:
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
    for i in range(nlayers):
        name, c0, c1, co, level, flags = U.oidn_unet_layer_info(9, i)
        px = (tw >> level) * (th >> level) * nbatch
        # algorithmic work of the method: a decoder conv reads its nearest-2x
        # upsampled source through 2 low-resolution rows per output row (the 3
        # ky taps pre-summed per row parity), so 6 taps for those c0 channels
        flops = 2.0 * px * co * ((6 * c0 + 9 * c1) if c1 else 9 * c0)
        sym, nblocks = syms[i]
        b_in, b_out = layer_bytes(i, c0, c1, co, level, flags, px)
        conv_flops += flops
        if i not in launch_ms:
            # second layer of a fused pair: its work ran in the previous launch
            prev = layers[-1]
            prev["layer"] += "+" + name
            prev["flops"] += flops
            prev["tflops"] = round(prev["flops"] / (prev["us"] / 1e3) / 1e9, 1)
            prev["bytes"] = prev["b_in"] + b_out     # the intermediate stays on chip
            prev["roof_frac"], prev["roof"] = roof_frac(prev["flops"], prev["bytes"],
                                                        prev["us"] / 1e3)
            groups[sym]["flops"] += flops
            print(f"  {name:11s}  (fused into the previous launch)", file=sys.stderr)
            continue
        ms = launch_ms[i]
        conv_ms += ms
        g = groups.setdefault(sym, {"flops": 0.0, "ms": 0.0, "launches": 0})
        g["flops"] += flops
        g["ms"] += ms
        g["launches"] += 1
        fr, bound = roof_frac(flops, b_in + b_out, ms)
        layers.append({"layer": name, "us": round(ms * 1e3, 2),
                       "us_events": round(launch_ms_events[i] * 1e3, 2), "flops": flops,
                       "tflops": round(flops / ms / 1e9, 1), "roof": bound, "roof_frac": fr,
                       "bytes": b_in + b_out, "b_in": b_in, "kernel": sym, "blocks": nblocks,
                       "samples": len(samples[i])})
        print(f"  {name:11s} {ms * 1e3:8.1f} us  {flops / ms / 1e9:7.1f} TFLOP/s  {sym} x{nblocks}",
              file=sys.stderr)
    for L in layers:
        L["mb"] = round(L.pop("bytes") / 1e6, 1)
        del L["flops"], L["b_in"]
    sym, g = max(groups.items(), key=lambda kv: kv[1]["ms"])
    achieved = g["flops"] / g["ms"] / 1e9  # TFLOP/s
    mp = W * H / 1e6
    peaks = None if args.no_peaks else measured_peaks(U, torch)
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
        "kernel_timing": {"method": f"two HIP events around one launch of every {every}-th timed "
                                    "step, rotating over the frame's launches (median per launch, "
                                    "`us_events`); the other steps run without markers. Each "
                                    "interval also holds its launch's dispatch gap, so the medians "
                                    "are scaled to sum to ms_per_step (`us`, used for every rate)",
                          "instrumented_steps": len(inst), "of_steps": args.steps,
                          "launches_per_frame": len(launches),
                          "sum_of_event_medians_ms": round(sum(launch_ms_events.values()), 4),
                          "scale": round(scale, 4)},
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
            "input_pass_fused": in_fused, "output_pass_fused": out_fused,
            "peak_gbs": PEAK_HBM_GBS, "standalone": passes},
        "layers": layers,
    }
    if peaks:
        result["measured_peaks"] = peaks
        result["roofline"]["frac_of_measured"] = round(achieved / peaks["mfma_f16_tflops"], 4)
        result["conv_mfma_frac_of_measured"] = round(conv_flops / conv_ms / 1e9 / peaks["mfma_f16_tflops"], 4)
        for p in passes:
            p["frac_of_measured_copy"] = round(p["gbs"] / peaks["hbm_copy_gbs"], 4)
    if cold:
        result["cold_cache"] = {"frames": len(cold), "flush_mb": 512,
                                "ms_median": round(float(np.median(cold)), 4),
                                "ms_p10": round(float(np.percentile(cold, 10)), 4),
                                "ms_p90": round(float(np.percentile(cold, 90)), 4),
                                "note": "each frame timed alone after writing 512 MB; not value"}
    if not args.no_other_configs:
        del work
        result["other_configs"] = other_configs(U, torch, S, args.dtype)

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        t = time.perf_counter()
        O.unet_forward(ws, bs, color, albedo, normal, True, 1.0, args.max_tile, args.overlap,
                       args.dtype)
        dt = time.perf_counter() - t
        info = cpu_info()
        result["cpu_baseline"] = {"value": round(W * H / 1e6 / dt, 4), "unit": "MP/s",
                                  "cores": blas_threads(), "kind": "oracle",
                                  "cpu_model": info["model"],
                                  "physical_cores": info["physical_cores"],
                                  "logical_cpus_allowed": info["logical_cpus_allowed"],
                                  "sample": f"the same {W}x{H} frame once, end to end (pack, "
                                            f"network, unpack), {args.dtype} storage emulated, float64 "
                                            f"sums on {blas_threads()} BLAS threads; {dt:.1f} s"}
    print(json.dumps(result), flush=True)




if __name__ == "__main__":
    main()
