"""Write sampled oracle outputs of the Wan2.2-shaped 720p decode on six latent frames to
tests/golden/wan_720p_6f_whole_samples.npz.

Usage: python tests/golden/make_wan_720p_samples.py

The oracle (fp64, CPU) decodes the latent [1,48,6,44,80] (seed 0) with the Wan-shaped plan's
random-init weights (affine seed 5: random biases, norm gains and offsets) to [1,21,704,1280,3]:
the full spatial extent, both temporal upsamplings (6 -> 11 -> 21 frames) and the frame
attention over 3520 positions. About 55 TFLOP in fp64 (tens of minutes on 8 cores). The script
keeps a fixed set of sampled output pixels (all three channels) and the global min, max, mean and
std of the output; the GPU test decodes the same seeded latent and weights in 1 x 4 width patches
and compares at the sampled pixels.

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
AFFINE_SEED = 5


def sample_positions(t_out, h_out, w_out, seams):
    g = np.random.Generator(np.random.PCG64(20261203))
    rnd = np.stack([g.integers(0, t_out, N_RANDOM), g.integers(0, h_out, N_RANDOM),
                    g.integers(0, w_out, N_RANDOM)], axis=1)
    cols = np.array(seams)[g.integers(0, len(seams), N_SEAM)]
    seam = np.stack([g.integers(0, t_out, N_SEAM), g.integers(0, h_out, N_SEAM), cols], axis=1)
    corners = np.array([[t, h, w] for t in (0, t_out - 1) for h in (0, h_out - 1)
                        for w in (0, w_out - 1)])
    return np.concatenate([rnd, seam, corners]).astype(np.int32)


def main():
    spec = vae_synth.WAN_720P_6F
    t0 = time.time()
    z = np.ascontiguousarray(vae_synth.latent(spec).transpose(0, 2, 3, 4, 1))
    params = vae_synth.decoder_params(spec, affine_seed=AFFINE_SEED)
    out = oracle.decode(spec, z, params)
    print(f"[golden] decode done in {time.time() - t0:.1f}s, shape {out.shape}", flush=True)
    _, t_out, h_out, w_out, _ = out.shape
    # the seams of the 1 x 4 width patches, in pixels (16 per latent column: 20 columns a patch)
    seams = [319, 320, 639, 640, 959, 960]
    pos = sample_positions(t_out, h_out, w_out, seams)
    vals = out[0, pos[:, 0], pos[:, 1], pos[:, 2], :]
    path = os.path.join(HERE, "wan_720p_6f_whole_samples.npz")
    np.savez_compressed(path, positions=pos, values=vals.astype(np.float64),
                        out_min=out.min(), out_max=out.max(), out_mean=out.mean(),
                        out_std=out.std(), shape=np.array(out.shape))
    print(f"[golden] wrote {path} ({len(pos)} pixels) in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main()
