"""Benchmark: tiled causal-3D VAE decode at 720p on one MI355X.

One step is one full decode of the LTX-2-shaped plan (the default, ``--workload ltx2``):
- input: seeded latent [1,128,16,22,40], random-init bf16 weights;
- output: [1,3,121,704,1280] fp32 (109,035,520 pixel-frames);
- default tiling: 1x4 patch-halo (mode A); ``--mode overlap`` times the 2x3 overlap-blend decode.
``--workload wan`` times the Wan2.2-TI2V-5B-shaped plan instead: latent [1,48,21,44,80] (padded
with zero channels to 64 for the matrix cores) -> [1,3,81,704,1280] (72,990,720 pixel-frames),
with RMS-norm residual blocks and a mid-block frame attention.

Inputs and weights are resident in HBM before the timed region. Exactly --steps decodes are timed
between two device synchronisations. HIP events recorded by the library on the decode's own stream
give each op's GPU time inside that same timed region, and the conv roofline comes from them.

Output: one JSON line on stdout; progress goes to stderr.

Two helper modes serve the HBM-traffic figure of the conv roofline:
- ``--calibrate-copy MIB`` runs only a plain copy of known size (the library's upsample kernel at
  factor 1), for reading what rocprofv3's FETCH_SIZE / WRITE_SIZE counters report per copied byte;
- ``--traffic-record FETCH WRITE COPY_FETCH COPY_WRITE --out PATH`` turns the four
  ``*_counter_collection.csv`` files of those ``--pmc`` runs into a small JSON record. The bench
  reports the record's traffic only while the conv kernel sources still hash to the digest stored
  in it; otherwise ``traffic`` is null.
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "decoded Mpixel-frames/s (720p VAE decode, 1 GPU) + conv MFMA % of peak"
CSRC = os.path.join(ROOT, "video_diffusion_vae_amd", "csrc")
CONV_SOURCES = sorted(os.path.join("video_diffusion_vae_amd", "csrc", f) for f in os.listdir(CSRC)
                      if f.startswith("conv3d") or f in ("kernels.h", "common.h", "decoder.hip"))
CONV_KERNEL = "conv3d_mfma_kernel"
COPY_KERNEL = "upsample_kernel"
OPERANDS = {
    "f16": "bf16 weights and GroupNorm operands; the 3 upsampling convs and conv_out take fp16 "
           "operands (fp16 hand-off of the fp32 stream, weights exact in fp16); fp32 accumulate",
    "split": "bf16 weights; the upsampling convs up0/up1 and conv_out apply fp32 inputs as bf16 "
             "hi+lo; fp32 accumulate",
    "bf16": "bf16 weights and operands; fp32 accumulate",
}
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "conv3d_mfma_ltx2_720p_decode_merged_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def conv_flops(spec, latent_shape):
    """Algorithmic conv flops of one decode: 2 * 27 * Cin * Cout * output positions per conv."""
    n, t, h, w, c = latent_shape
    total = 0.0
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            total += 2 * 27 * op["cin"] * op["cout"] * n * t * h * w
        elif k in ("res", "res_rms"):
            total += 2 * (2 * 27 * op["c"] * op["c"] * n * t * h * w)
        elif k == "d2s":
            t, h, w = op["st"] * t - (op["st"] - 1), h * op["sh"], w * op["sw"]
        elif k == "nearest":
            h, w = h * op["sh"], w * op["sw"]
        elif k == "s2d":
            t, h, w = (t + op["st"] - 1) // op["st"], h // op["sh"], w // op["sw"]
        elif k == "conv_down":
            t, h, w = (t - 1) // op["st"] + 1, h // op["sh"], w // op["sw"]
            total += 2 * 27 * op["cin"] * op["cout"] * n * t * h * w
    return total


def output_shape(spec, latent_shape):
    """[N, T, H, W, C] of the plan's output for an NDHWC input shape (a decoder's video, an
    encoder's latent)."""
    n, t, h, w, c = latent_shape
    for op in spec["layers"]:
        k = op["op"]
        if k == "conv":
            c = op["cout"]
        elif k == "d2s":
            t, h, w = op["st"] * t - (op["st"] - 1), h * op["sh"], w * op["sw"]
            c //= op["st"] * op["sh"] * op["sw"]
        elif k == "nearest":
            h, w = h * op["sh"], w * op["sw"]
        elif k == "s2d":
            t, h, w = (t + op["st"] - 1) // op["st"], h // op["sh"], w // op["sw"]
            c *= op["st"] * op["sh"] * op["sw"]
        elif k == "conv_down":
            t, h, w, c = (t - 1) // op["st"] + 1, h // op["sh"], w // op["sw"], op["cout"]
    return (n, t, h, w, c)


WORKLOADS = {
    # name: (plan, patch grid of the patch-halo mode, tile grid name of the overlap mode)
    "ltx2": ("LTX2_720P", (1, 4), "2x3"),
    "wan": ("WAN_720P", (1, 4), "2x3"),
    "ltx2_enc": ("LTX2_ENC_720P", (1, 1), "2x3"),    # encode: untiled, or latent-grid tiles
    # the same encoder with bare stride-2 causal convs as its downsamplers
    "ltx2_enc_strided": ("LTX2_ENC_STRIDED_720P", (1, 1), "2x3"),
}
ENCODE_METRIC = "encoded Mpixel-frames/s (720p VAE encode, 1 GPU) + conv MFMA % of peak"


def activations_note(operands):
    if operands == "f16":
        return ("fp32 residual stream; res-block conv1 outputs fp16; norm outputs bf16, or fp16 "
                "where an fp16-operand conv reads them")
    return "fp32 between ops, bf16 norm outputs inside res blocks"


def workload_name(kind, mode, tile_t=0, stride_t=0, clip=0):
    if clip and mode in ("patch", "per_patch"):
        return workload_name(kind, mode) + f"_causal_clips_of_{clip}"
    if kind in ("ltx2_enc", "ltx2_enc_strided"):
        prefix = "ltx2_720p_encode_" + ("strided_" if kind == "ltx2_enc_strided" else "")
        return prefix + ("untiled" if mode == "patch" else "overlap_blend_2x3")
    prefix = {"ltx2": "ltx2_720p", "wan": "wan2.2_ti2v_5b_720p"}[kind]
    if mode == "patch":
        # the 1x4 patch-halo split with one launch per layer over all four patch boxes: on one
        # GPU this computes the untiled decode's tensors
        return prefix + "_decode_1x4_patch_halo_merged_launches"
    if mode == "per_patch":
        return prefix + "_decode_1x4_patch_halo_per_patch_launches"
    return prefix + "_decode_overlap_blend_2x3" + (f"_t{tile_t}s{stride_t}" if tile_t else "")


LAUNCH_NOTE = {
    "patch": "merged: one launch per layer covers the four patch boxes (halos read in place); "
             "equals the untiled decode",
    "per_patch": "per patch: every conv, GroupNorm pass and upsampling launched once per patch "
                 "box, statistics merged across the boxes (four ranks' work, one after another)",
    "overlap": "one overlap tile in flight",
}


def _band(length, parts, i):
    """[start, end) of band i when `length` rows are cut into `parts` bands, the first
    length % parts bands one row longer (the split vae_tile_split makes)."""
    q, r = divmod(length, parts)
    start = i * q + min(i, r)
    return start, start + q + (1 if i < r else 0)


def patch_summary(per_op, steps, patch, latent_box, out_px):
    """Work of one patch of a per-patch decode: its own launches (records with tile == patch) and
    the merges of GroupNorm statistics that every rank would also run (tile == -1)."""
    own = [r for step in per_op for r in step if r["tile"] == patch]
    shared = [r for step in per_op for r in step if r["tile"] == -1]
    own_ms = sum(r["ms"] for r in own) / steps
    shared_ms = sum(r["ms"] for r in shared) / steps
    conv = [r for r in own if r["kind"] == "conv"]
    conv_ms = sum(r["ms"] for r in conv) / steps
    conv_flops = sum(r["flops"] for r in conv) / steps
    tflops = conv_flops / (conv_ms / 1000.0) / 1e12
    layers = {}
    for r in conv:
        L = layers.setdefault(r["layer"], {"ms": 0.0, "flops": 0.0, "n": 0})
        L["ms"] += r["ms"]
        L["flops"] += r["flops"]
        L["n"] += 1
    per_layer = []
    for layer in sorted(layers):
        L = layers[layer]
        tf = L["flops"] / (L["ms"] / 1000.0) / 1e12
        per_layer.append({"layer": layer, "launches_per_step": L["n"] // steps,
                          "ms_per_step": round(L["ms"] / steps, 4), "tflops": round(tf, 1),
                          "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    gn = [r for r in own if r["kind"] == "gn"]
    gn_ms = sum(r["ms"] for r in gn) / steps
    gn_bytes = sum(r["bytes"] for r in gn) / steps
    total = own_ms + shared_ms
    return {
        "patch": patch, "latent_box": latent_box,
        "ms_per_step": round(total, 3), "own_launches_ms": round(own_ms, 3),
        "shared_stat_merges_ms": round(shared_ms, 3),
        "value": round(out_px / (total / 1000.0) / 1e6, 3), "unit": "Mpx-frames/s",
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "kernel": "conv3d_mfma_kernel (this patch's conv launches)",
                     "conv_ms_per_step": round(conv_ms, 3),
                     "conv_tflop_per_step": round(conv_flops / 1e12, 3)},
        "gn": {"ms_per_step": round(gn_ms, 3),
               "gbs": round(gn_bytes / (gn_ms / 1000.0) / 1e9, 1) if gn_ms else None},
        "conv_layers": per_layer,
    }


def run_per_patch(v, dev, spec, params, operands, zd, desc, out, steps, warmup, patch):
    """Times the per-patch decode and returns (per-step op records, wall ms per step)."""
    import torch
    dec = v.upload_decoder(spec, params, dev, operands=operands)
    dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        dec.vae_decode_tiled(zd, desc, out, ws)
    torch.cuda.synchronize(dev)
    dec.set_timing(True)
    per_op = []
    t0 = time.perf_counter()
    for _ in range(steps):
        dec.vae_decode_tiled(zd, desc, out, ws)
        per_op.append(dec.timing())
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    dec.close()
    del ws
    return per_op, ms


def conv_source_digest():
    h = hashlib.sha256()
    for rel in CONV_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _pmc_sum(path, kernel_substr, counter):
    """Sum of one counter over the dispatches whose kernel name contains `kernel_substr`."""
    total, dispatches = 0.0, set()
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_substr in row["Kernel_Name"] and row["Counter_Name"] == counter:
                total += float(row["Counter_Value"])
                dispatches.add(row["Dispatch_Id"])
    return total, len(dispatches)


def write_traffic_record(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, decodes,
                         workload, out):
    """Conv HBM bytes per decode from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    (known copy bytes) / (what the same counter reads for the copy)."""
    copy_bytes = copy_mib * 2**20
    cf, ncf = _pmc_sum(copy_fetch_csv, COPY_KERNEL, "FETCH_SIZE")
    cw, ncw = _pmc_sum(copy_write_csv, COPY_KERNEL, "WRITE_SIZE")
    # the calibration program launches the copy `ncf` times, each moving copy_bytes each way
    fetch_scale = copy_bytes * ncf / (cf * 1024.0)
    write_scale = copy_bytes * ncw / (cw * 1024.0)
    f, nf = _pmc_sum(fetch_csv, CONV_KERNEL, "FETCH_SIZE")
    w, nw = _pmc_sum(write_csv, CONV_KERNEL, "WRITE_SIZE")
    rec = {
        "workload": workload, "kernel": CONV_KERNEL, "decodes": decodes,
        "conv_dispatches_per_decode": nf / decodes,
        "fetch_kib_per_decode_raw": f / decodes, "write_kib_per_decode_raw": w / decodes,
        "copy_bytes": copy_bytes, "copy_dispatches": ncf,
        "copy_fetch_kib_raw": cf / ncf, "copy_write_kib_raw": cw / ncw,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_bytes_per_decode": (f * fetch_scale + w * write_scale) * 1024.0 / decodes,
        "source_sha256": conv_source_digest(),
    }
    assert nf == nw, (nf, nw)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def conv_traffic(workload):
    """HBM bytes of the conv launches of one decode, while the record matches the sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no traffic record"
    if rec.get("workload") != workload:
        return None, "traffic record is for another workload"
    if rec.get("source_sha256") != conv_source_digest():
        return None, "conv sources changed since the counters were taken"
    return rec["hbm_bytes_per_decode"], "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def calibrate_copy(mib, repeats=3):
    """Plain device copy of `mib` MiB (fp32 rows through the library's upsample kernel at factor
    1), `repeats` times; prints what it did as one JSON line."""
    import torch
    import video_diffusion_vae_amd as v
    dev = torch.device("cuda:0")
    n = mib * 2**20 // 4
    rows = n // 1024
    src = torch.ones((1, 1, rows, 1, 1024), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(repeats):
        v.vae_upsample(src, None, v.VAE_UPSAMPLE_NEAREST, 1, 1, 1, dst)
    torch.cuda.synchronize(dev)
    assert bool((dst == 1).all())
    print(json.dumps({"copy_mib": mib, "repeats": repeats, "kernel": COPY_KERNEL}), flush=True)


def standalone_passes(v, dev, reps=5):
    """HBM rates of the streaming passes as standalone library calls at the 720p decode's shapes
    (inside the decode the depth-to-space runs in the conv epilogue, and the merge only in the
    overlap-blend mode). Timed with events on the stream the calls are enqueued on."""
    import torch
    out = {}
    stream = torch.cuda.current_stream(dev)

    def timed(fn, nbytes):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        e.synchronize()
        ms = s.elapsed_time(e) / reps
        gbs = nbytes / (ms / 1000.0) / 1e9
        return {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                "bytes": nbytes}

    # depth-to-space of the largest upsampling conv's output: fp32 [1,61,88,160,1024] -> S3
    x = torch.zeros((1, 61, 88, 160, 1024), dtype=torch.float32, device=dev)
    y = torch.empty((1, 121, 176, 320, 128), dtype=torch.float32, device=dev)
    out["upsample_d2s_f32_s2_to_s3"] = timed(
        lambda: v.vae_upsample(x, None, v.VAE_UPSAMPLE_D2S, 2, 2, 2, y),
        x.numel() * 4 + y.numel() * 4)
    del x
    # GroupNorm apply + SiLU at S3 (fp32 in, bf16 operand out), statistics given
    mr = torch.zeros((1, 32, 2), dtype=torch.float32, device=dev)
    mr[..., 1] = 1.0
    gamma = torch.ones(128, dtype=torch.float32, device=dev)     # per-channel affine, as decoded
    beta = torch.zeros(128, dtype=torch.float32, device=dev)
    yb = torch.empty(y.shape, dtype=torch.bfloat16, device=dev)
    out["gn_apply_silu_f32_to_bf16_s3"] = timed(
        lambda: v.vae_groupnorm_apply(y, None, 32, mr, gamma, beta, True, yb),
        y.numel() * 4 + yb.numel() * 2)
    del y, yb
    torch.cuda.synchronize(dev)
    return out


def cpu_baseline(spec, params, frames=2):
    """The oracle, as it stands, on a bounded sample: the full 720p spatial plan on `frames`
    latent frames (an encoder: the input frames that fold into that many latent frames). `value`
    is the sample's own throughput, the video pixel-frames it produced (or consumed) per second:
    measured, not extrapolated. Per output frame the sample does slightly more conv work than the
    full decode (the first latent frame decodes to one frame), so the figure leans low."""
    import threadpoolctl
    import oracle
    import vae_synth
    encoder = spec.get("kind") == "encoder"
    take = 8 * frames - 7 if encoder else frames       # an encoder's sample: whole latent frames
    z = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1))[:, :take]
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    out = oracle.decode(spec, z, params)
    sample_s = time.perf_counter() - t0
    n, c, t, h, w = spec["input"] if encoder else spec["latent"]
    video = z.shape if encoder else out.shape
    px = video[1] * video[2] * video[3]
    full = (n, t, h, w, c)
    work = conv_flops(spec, z.shape) / px
    work_full = conv_flops(spec, full) / np.prod((output_shape(spec, full) if not encoder
                                                  else full)[1:4])
    what = "encode of video" if encoder else "decode of latent"
    return {
        "value": px / sample_s / 1e6, "unit": "Mpx-frames/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"oracle fp64 {what} [{n},{c},{take},{h},{w}] -> {list(out.shape)} "
                   f"({px / 1e6:.2f} M px-frames) in {sample_s:.1f} s; value = sample "
                   f"px-frames / sample time, not extrapolated (conv work per px-frame "
                   f"{work / work_full:.2f}x the full {t}-frame 720p "
                   f"{'encode' if encoder else 'decode'}'s); os.cpu_count()={os.cpu_count()}"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["patch", "per_patch", "overlap"], default="patch",
                    help="patch: 1x4 patch-halo, one launch per layer; per_patch: the same split "
                         "launched patch by patch; overlap: 2x3 overlap-blend tiles")
    ap.add_argument("--no-quarter", action="store_true",
                    help="skip the per-patch run that measures the interior quarter patch")
    ap.add_argument("--quarter-steps", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="ltx2",
                    help="ltx2: the LTX-2-shaped decode (the headline); wan: the Wan2.2-shaped one")
    ap.add_argument("--operands", choices=["f16", "split", "bf16"], default="f16",
                    help="operands of the convs that read an fp32 activation (up-convs, conv_out)")
    ap.add_argument("--tile-t", type=int, default=0,
                    help="overlap mode: also cut T into clips of this many latent frames")
    ap.add_argument("--stride-t", type=int, default=0,
                    help="overlap mode: latent frames between clip starts (below --tile-t)")
    ap.add_argument("--clip", type=int, default=0,
                    help="patch modes: decode in causal clips of this many latent frames, each "
                         "conv carrying its last two input frames (plans without GroupNorm)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one decode in a HIP graph and time its replays; value "
                         "is then the replayed decode's rate")
    ap.add_argument("--norm-in-conv", action="store_true",
                    help="the convs apply GroupNorm + SiLU while staging their input instead of "
                         "separate normalise passes (VAE_DECODE_NORM_IN_CONV)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=0,
                    help="latent frames of the oracle's sample (default 2 for ltx2, 1 for wan)")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB")
    ap.add_argument("--traffic-record", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"))
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--decodes", type=int, default=1)
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.traffic_record:
        workload = workload_name(args.workload, args.mode)
        write_traffic_record(*args.traffic_record, args.copy_mib, args.decodes, workload,
                             args.out or TRAFFIC_RECORD)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this decode has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import vae_synth
    import video_diffusion_vae_amd as v

    plan_name, patch_grid, tiles = WORKLOADS[args.workload]
    spec = getattr(vae_synth, plan_name)
    encoder = spec.get("kind") == "encoder"
    if args.mode == "overlap" and tiles is None:
        print(f"--workload {args.workload} runs untiled only (--mode patch)", file=sys.stderr)
        sys.exit(2)
    t_setup = time.perf_counter()
    z = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1))
    out_shape = output_shape(spec, z.shape)
    params = vae_synth.decoder_params(spec)
    dev = torch.device("cuda:0")
    dec = v.upload_decoder(spec, params, dev, operands=args.operands,
                           norm_in_conv=args.norm_in_conv)
    if args.mode == "per_patch":
        dec.set_launch(v.VAE_LAUNCH_PER_PATCH)
    if args.clip:
        if args.mode == "overlap":
            print("--clip is for the patch modes (--tile-t cuts overlap tiles in T)",
                  file=sys.stderr)
            sys.exit(2)
        dec.set_clip_frames(args.clip)
    zp = v.pad_latent(z, spec)            # zero channels up to a multiple of 32 (48 -> 64)
    zd = torch.as_tensor(zp).to(device=dev, dtype=torch.bfloat16)
    workload = workload_name(args.workload, args.mode, args.tile_t, args.stride_t, args.clip)
    if args.mode in ("patch", "per_patch"):
        if encoder and args.mode == "per_patch":
            print("--workload ltx2_enc runs untiled or overlap-tiled", file=sys.stderr)
            sys.exit(2)
        desc = v.tiling_desc(v.VAE_TILING_PATCH_HALO, zp.shape, spec.get("scale", (1, 1, 1)),
                             patches=patch_grid)
    else:
        desc = v.tiling_desc(v.VAE_TILING_OVERLAP_BLEND, zp.shape, spec.get("scale", (1, 1, 1)),
                             tile=spec["overlap_tile"], stride=spec["overlap_stride"],
                             tile_t=args.tile_t, stride_t=args.stride_t,
                             down=spec.get("down", (0, 0, 0)))
    ws = torch.empty(dec.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty(out_shape, dtype=torch.float32, device=dev)
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s, workspace "
        f"{ws.numel() / 2**30:.2f} GiB")

    for i in range(args.warmup):
        dec.vae_decode_tiled(zd, desc, out, ws)
    torch.cuda.synchronize(dev)
    log(f"[bench] {args.warmup} warmup steps done")

    graph_ms = None
    if args.graph:
        # the decode enqueues kernels only, so the whole launch sequence (every layer, patch and
        # clip) captures into one graph; timed over the replays alone
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            dec.vae_decode_tiled(zd, desc, out, ws)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dec.vae_decode_tiled(zd, desc, out, ws)
        graph.replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize(dev)
        graph_ms = (time.perf_counter() - t0) * 1000.0 / args.steps
        del graph
        log(f"[bench] {args.steps} graph replays: {graph_ms:.2f} ms/step")

    dec.set_timing(True)
    per_op, step_s, enqueue_s = [], [], []
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        ts = time.perf_counter()
        dec.vae_decode_tiled(zd, desc, out, ws)
        enqueue_s.append(time.perf_counter() - ts)
        per_op.append(dec.timing())          # waits for this step's last event
        step_s.append(time.perf_counter() - ts)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    dec.set_timing(False)
    ms = elapsed * 1000.0 / args.steps
    eager_ms = ms
    if graph_ms is not None:
        ms = graph_ms
    video = z.shape if encoder else out_shape          # pixel-frames of the video side
    px = video[1] * video[2] * video[3]
    value = px / (ms / 1000.0) / 1e6
    log(f"[bench] {args.steps} timed steps: {ms:.2f} ms/step, {value:.1f} Mpx-frames/s")

    kinds = {}
    for step in per_op:
        for r in step:
            k = kinds.setdefault(r["kind"], {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "n": 0})
            k["ms"] += r["ms"]
            k["flops"] += r["flops"]
            k["bytes"] += r["bytes"]
            k["n"] += 1
    summary = {}
    for name, k in kinds.items():
        s = {"ms_per_step": k["ms"] / args.steps, "launch_groups_per_step": k["n"] // args.steps}
        if k["flops"]:
            s["tflops"] = k["flops"] / (k["ms"] / 1000.0) / 1e12
            s["frac_mfma_peak"] = s["tflops"] / PEAK_BF16_TFLOPS
        if k["bytes"] and name != "conv":
            s["gbs"] = k["bytes"] / (k["ms"] / 1000.0) / 1e9
            s["frac_hbm_peak"] = s["gbs"] / PEAK_HBM_GBS
        summary[name] = s
    for r in per_op[-1]:
        if r["kind"] == "conv":
            log(f"  conv layer {r['layer']:2d} tile {r['tile']:2d}: {r['ms']:8.3f} ms "
                f"{r['flops'] / r['ms'] / 1e9:8.1f} TFLOP/s")
    for name, s in summary.items():
        log(f"  {name}: {json.dumps(s)}")

    conv = kinds["conv"]
    achieved = conv["flops"] / (conv["ms"] / 1000.0) / 1e12
    traffic, traffic_note = conv_traffic(workload)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "traffic_unit": "bytes per decode (conv launches)",
                "traffic_note": traffic_note,
                "kernel": "conv3d_mfma_kernel (all conv launches of one decode)",
                "conv_ms_per_step": round(conv["ms"] / args.steps, 3),
                "conv_launches_per_step": conv["n"] // args.steps}
    pct = lambda a, q: float(np.percentile(np.asarray(a) * 1000.0, q))
    timing = {"step_ms_p10": round(pct(step_s, 10), 3), "step_ms_p50": round(pct(step_s, 50), 3),
              "step_ms_p90": round(pct(step_s, 90), 3),
              "host_enqueue_ms_p50": round(pct(enqueue_s, 50), 3)}
    if graph_ms is not None:
        timing["graph_replay_ms_per_step"] = round(graph_ms, 3)
        timing["eager_ms_per_step"] = round(eager_ms, 3)

    passes = standalone_passes(v, dev) if args.workload == "ltx2" else None
    for name, p in (passes or {}).items():
        log(f"  pass {name}: {json.dumps(p)}")

    # The interior quarter patch (patch 1 of the 1x4 split: latent columns [10, 20)) at its real
    # shape: the launches one rank of the split runs, timed inside a per-patch decode.
    quarter = None
    if args.workload in ("ltx2", "wan") and args.mode in ("patch", "per_patch") and \
            not args.no_quarter and not args.clip:
        if args.mode == "per_patch":
            q_ops, q_steps = per_op, args.steps
        else:
            log("[bench] per-patch decode for the quarter-patch figures ...")
            q_ops, q_ms = run_per_patch(v, dev, spec, params, args.operands, zd, desc, out,
                                        args.quarter_steps, 1, 1)
            q_steps = args.quarter_steps
            log(f"[bench] per-patch decode: {q_ms:.2f} ms/step")
        lw = zp.shape[3]
        b0, b1 = _band(lw, 4, 1)
        out_px = out_shape[1] * out_shape[2] * (b1 - b0) * (out_shape[3] // lw)
        quarter = patch_summary(q_ops, q_steps, 1,
                                {"t": [0, zp.shape[1]], "h": [0, zp.shape[2]], "w": [b0, b1]},
                                out_px)
        if args.mode == "patch":
            quarter["per_patch_decode_ms_per_step"] = round(q_ms, 3)
        log(f"[bench] quarter patch: {json.dumps(quarter)}")

    baseline = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on its bounded sample ...")
        frames = args.cpu_frames or (2 if args.workload == "ltx2" else 1)
        baseline = cpu_baseline(spec, params, frames)
        log(f"[bench] cpu baseline: {baseline}")

    line = {
        "metric": ENCODE_METRIC if encoder else METRIC, "value": round(value, 3),
        "unit": "Mpx-frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": ("synthetic (seeded U(-1,1) video, random-init weights)" if encoder
                 else "synthetic (seeded latent, random-init weights)"),
        "config": {"workload": workload,
                   ("input" if encoder else "latent"): list(spec["input" if encoder else "latent"]),
                   "output": [out_shape[0], out_shape[4]] + list(out_shape[1:4]),
                   "parallelism": "none (1 GPU)",
                   "launch": LAUNCH_NOTE[args.mode] + (
                       f"; causal clips of {args.clip} latent frames" if args.clip else "") + (
                       "; replayed from a HIP graph" if args.graph else "") + (
                       "; GroupNorm applied in conv staging" if args.norm_in_conv else ""),
                   "operands": OPERANDS[args.operands],
                   "activations": activations_note(args.operands),
                   "conv_tflop_per_step": round(conv_flops(spec, z.shape) / 1e12, 3)},
        "roofline": roofline, "quarter_patch": quarter, "kernels": summary,
        "standalone_passes": passes, "timing": timing,
        "attention_tflop_per_step": (round(kinds["attn"]["flops"] / args.steps / 1e12, 3)
                                     if "attn" in kinds else None),
        "cpu_baseline": baseline,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
