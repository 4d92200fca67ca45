"""Write sampled oracle outputs of the 720p LTX-2-shaped decode to tests/golden/.

Usage: python tests/golden/make_ltx2_720p_samples.py [whole|overlap|band]

This is the full-size parity reference. The oracle (fp64, CPU) decodes the latent
[1,128,16,22,40] to [1,3,121,704,1280]: fp64 throughout, about 70 TFLOP and 20-40 minutes on
8 cores, peak memory about 35 GB. The script keeps:
- a fixed set of sampled output pixels (all three channels);
- the global min, max, mean and std of the output.
The GPU test decodes the same seeded latent and weights and compares at the sampled pixels.

Modes:
- ``whole``: the untiled decode, which the patch-halo decode must equal;
- ``overlap``: the overlap-blend decode with latent tile 16 and stride 14 (512/448 px);
- ``band``: the untiled decode again, keeping every value of a 16-row band of output frame 60
  (all 1280 columns, so the three seams of the 1x4 width split lie inside it) in
  ``ltx2_720p_whole_band.npz``: a full-T decode compared at every value of a region of a frame
  far past frame 0.

Only ``oracle`` and ``vae_synth`` are used; nothing here touches the GPU path.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle      # noqa: E402
import vae_synth   # noqa: E402

N_RANDOM = 12288
N_SEAM = 4096
BAND = (60, 344, 360)     # output frame, first row, end row of the stored band


def sample_positions(t_out, h_out, w_out, seams):
    g = np.random.Generator(np.random.PCG64(20261202))
    rnd = np.stack([g.integers(0, t_out, N_RANDOM), g.integers(0, h_out, N_RANDOM),
                    g.integers(0, w_out, N_RANDOM)], axis=1)
    cols = np.array(seams)[g.integers(0, len(seams), N_SEAM)]
    seam = np.stack([g.integers(0, t_out, N_SEAM), g.integers(0, h_out, N_SEAM), cols], axis=1)
    corners = np.array([[t, h, w] for t in (0, t_out - 1) for h in (0, h_out - 1)
                        for w in (0, w_out - 1)])
    return np.concatenate([rnd, seam, corners]).astype(np.int32)


def main(mode: str):
    spec = vae_synth.LTX2_720P
    t0 = time.time()
    z = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1))
    params = vae_synth.decoder_params(spec)
    print(f"[golden] inputs ready in {time.time() - t0:.1f}s", flush=True)
    if mode in ("whole", "band"):
        out = oracle.decode(spec, z, params)
    elif mode == "overlap":
        out = oracle.decode_overlap_blend(spec, z, params, spec["overlap_tile"],
                                          spec["overlap_stride"], spec["scale"])
    else:
        raise SystemExit(f"unknown mode {mode!r}")
    print(f"[golden] decode done in {time.time() - t0:.1f}s, shape {out.shape}", flush=True)
    if mode == "band":
        frame, r0, r1 = BAND
        path = os.path.join(HERE, "ltx2_720p_whole_band.npz")
        np.savez_compressed(path, frame=np.int32(frame), rows=np.array([r0, r1], np.int32),
                            values=out[0, frame, r0:r1].astype(np.float64),
                            out_min=out.min(), out_max=out.max(), shape=np.array(out.shape))
        print(f"[golden] wrote {path} in {time.time() - t0:.1f}s", flush=True)
        return
    _, t_out, h_out, w_out, _ = out.shape
    # patch seams of the 1x4 width split and the overlap-tile boundaries (in pixels)
    seams = [319, 320, 639, 640, 959, 960, 447, 448, 511, 512, 895, 896, 1023, 1024]
    pos = sample_positions(t_out, h_out, w_out, seams)
    vals = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :]
    path = os.path.join(HERE, f"ltx2_720p_{mode}_samples.npz")
    np.savez_compressed(path, positions=pos, values=vals.astype(np.float64),
                        out_min=out.min(), out_max=out.max(), out_mean=out.mean(),
                        out_std=out.std(), shape=np.array(out.shape))
    print(f"[golden] wrote {path} ({len(pos)} pixels) in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "whole")
