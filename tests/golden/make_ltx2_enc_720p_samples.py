"""Write sampled oracle outputs of the LTX-2-shaped 720p encode to
tests/golden/ltx2_enc_720p_samples.npz.

Usage: python tests/golden/make_ltx2_enc_720p_samples.py

The oracle (fp64, CPU) encodes the video [1,3,121,704,1280] (U(-1,1), seed 0) with the encoder
plan's random-init weights (affine seed 9: random biases, norm gains and offsets) to the latent
[1,16,22,40,256]. About 51 TFLOP in fp64 (tens of minutes on 8 cores). The script keeps a fixed
set of latent positions (all 256 channels, stored in fp32) and the latent's global min, max,
mean and std; the GPU test encodes the same seeded video and weights untiled and compares at the
sampled positions.

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

N_RANDOM = 384
N_SEAM = 120
AFFINE_SEED = 9


def sample_positions(t, h, w, seams):
    g = np.random.Generator(np.random.PCG64(20261204))
    rnd = np.stack([g.integers(0, t, N_RANDOM), g.integers(0, h, N_RANDOM),
                    g.integers(0, w, N_RANDOM)], axis=1)
    cols = np.array(seams)[g.integers(0, len(seams), N_SEAM)]
    seam = np.stack([g.integers(0, t, N_SEAM), g.integers(0, h, N_SEAM), cols], axis=1)
    corners = np.array([[a, b, c] for a in (0, t - 1) for b in (0, h - 1) for c in (0, w - 1)])
    return np.concatenate([rnd, seam, corners]).astype(np.int32)


def main():
    spec = vae_synth.LTX2_ENC_720P
    t0 = time.time()
    x = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1))
    params = vae_synth.decoder_params(spec, affine_seed=AFFINE_SEED)
    out = oracle.encode(spec, x, params)
    print(f"[golden] encode done in {time.time() - t0:.1f}s, shape {out.shape}", flush=True)
    _, t, h, w, _ = out.shape
    # latent columns at the 1 x 4 band seams (10 columns a band) and the 2 x 3 tile overlaps
    seams = [9, 10, 14, 15, 19, 20, 28, 29, 30, 31]
    pos = sample_positions(t, h, w, seams)
    vals = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :]
    path = os.path.join(HERE, "ltx2_enc_720p_samples.npz")
    np.savez_compressed(path, positions=pos, values=vals.astype(np.float32),
                        out_min=out.min(), out_max=out.max(), out_mean=out.mean(),
                        out_std=out.std(), shape=np.array(out.shape))
    print(f"[golden] wrote {path} ({len(pos)} positions) in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main()
