"""Benchmark: end-to-end 1920x1080 UNet denoise (input pass -> sixteen
3x3 convs -> output pass) on one MI355X, fp16 storage / fp32 accumulate.

Prints one JSON line.  `value` is megapixels of image per second over the
timed steps (inputs resident in HBM).  Per-kernel times come from HIP events
recorded between the launches of every timed step; the roofline entry is the
kernel symbol with the largest total time.  `cpu_baseline` times the CPU
oracle on a bounded 512x512 sample of the same workload.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--width", type=int, default=1920)
    ap.add_argument("--height", type=int, default=1080)
    ap.add_argument("--max-tile", type=int, default=0)
    ap.add_argument("--overlap", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(tiles would shard across GPUs; see the design notes)", file=sys.stderr)
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
    wbuf = torch.empty(U.oidn_unet_weights_bytes(9, U.OIDN_F16), dtype=torch.uint8, device="cuda")
    U.oidn_unet_pack_weights(ws, bs, 9, U.OIDN_F16, wbuf)
    nbytes = U.oidn_unet_workspace_bytes(9, W, H, args.max_tile, args.overlap, U.OIDN_F16)
    work = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    tiles = U.oidn_plan_tiles(W, H, args.max_tile, args.overlap)
    tw, th = tiles[0][2], tiles[0][3]

    def step(events=None):
        if events is None:
            U.oidn_unet_forward(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                nbytes, out, U.OIDN_F16)
        else:
            U.oidn_unet_forward_timed(wbuf, 9, d_color, d_albedo, d_normal, W, H, True,
                                      U.OIDN_TRANSFER_LOG, 1.0, args.max_tile, args.overlap, work,
                                      nbytes, out, U.OIDN_F16, events)

    nk = 18  # input pass, 16 convs, output pass
    events = [[U.oidn_event_create() for _ in range(nk + 1)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {W}x{H}, {len(tiles)} tile(s) of {tw}x{th}, warmup {args.warmup} done",
          file=sys.stderr, flush=True)

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.steps):
        step(events[k])
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-kernel durations (first tile of each step)
    dur = np.zeros((args.steps, nk))
    for k in range(args.steps):
        for j in range(nk):
            dur[k, j] = U.oidn_event_elapsed_ms(events[k][j], events[k][j + 1])
    for evs in events:
        for e in evs:
            U.oidn_event_destroy(e)
    avg_ms = dur.mean(axis=0)

    layers = []
    groups = {}
    conv_flops = conv_ms = 0.0
    for i in range(U.oidn_unet_layer_count()):
        name, c0, c1, co, level, flags = U.oidn_unet_layer_info(9, i)
        px = (tw >> level) * (th >> level)
        flops = 2.0 * px * co * 9 * (c0 + c1)
        ms = float(avg_ms[i + 1])
        sym, nblocks = U.oidn_unet_layer_kernel(9, i, tw, th, U.OIDN_F16)
        g = groups.setdefault(sym, {"flops": 0.0, "ms": 0.0, "launches": 0})
        g["flops"] += flops
        g["ms"] += ms
        g["launches"] += 1
        conv_flops += flops
        conv_ms += ms
        layers.append({"layer": name, "us": round(ms * 1e3, 2),
                       "tflops": round(flops / ms / 1e9, 1), "kernel": sym, "blocks": nblocks})
        print(f"  {name:11s} {ms * 1e3:8.1f} us  {flops / ms / 1e9:7.1f} TFLOP/s  {sym} x{nblocks}",
              file=sys.stderr)
    px0 = tw * th
    pack_bytes = W * H * 48 + px0 * 12 * 2 if len(tiles) == 1 else None
    unpack_bytes = W * H * (32 + 16)
    for j, nm in ((0, "input pass"), (nk - 1, "output pass")):
        print(f"  {nm:11s} {avg_ms[j] * 1e3:8.1f} us", file=sys.stderr)
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
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"UNet denoise {W}x{H}, {len(tiles)} tile(s) of {tw}x{th}, HDR log "
                               "transfer, 9-channel input, fp16 storage / fp32 accumulate",
                   "width": W, "height": H, "tiles": len(tiles), "max_tile": args.max_tile,
                   "overlap": args.overlap},
        "conv_tflops": round(conv_flops / conv_ms / 1e9, 1),
        "conv_mfma_frac": round(conv_flops / conv_ms / 1e9 / PEAK_F16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": sym, "launches_per_step": g["launches"],
                     "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": None},
        "elementwise": {
            "input_pass_us": round(float(avg_ms[0]) * 1e3, 2),
            "input_pass_gbs": round(pack_bytes / avg_ms[0] / 1e6, 1) if pack_bytes else None,
            "output_pass_us": round(float(avg_ms[nk - 1]) * 1e3, 2),
            "output_pass_gbs": round(unpack_bytes / avg_ms[nk - 1] / 1e6, 1) if len(tiles) == 1 else None,
            "peak_gbs": PEAK_HBM_GBS},
        "layers": layers,
    }

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        import threadpoolctl
        cw, ch = 512, 512
        t = time.perf_counter()
        O.unet_forward(ws, bs, color[:ch, :cw], albedo[:ch, :cw], normal[:ch, :cw], True, 1.0, 0,
                       args.overlap, "f16")
        dt = time.perf_counter() - t
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
        result["cpu_baseline"] = {"value": round(cw * ch / 1e6 / dt, 4), "unit": "MP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"one {cw}x{ch} crop of the same frame, end to end "
                                            f"(pack, network, unpack), fp16 storage emulated, "
                                            f"float64 sums; {dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
