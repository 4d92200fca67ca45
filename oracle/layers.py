"""Oracle layers: causal Conv3d, GroupNorm, SiLU, upsampling. Channels-last, float64.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from __future__ import annotations

import numpy as np

# Size cap (elements) of the unfolded input built per batch of output frames inside the
# convolution. It bounds memory only: every output element is the same full sum either way.
_COLS_ELEMENTS = 1 << 26


def causal_time_pad(x: np.ndarray, k_t: int = 3) -> np.ndarray:
    """Prepend k_t-1 copies of frame 0 along T.

    Causal temporal padding repeats the first frame, one-sided, along an axis that is never split
    ("Add tiled VAE parallelism & extended model support", commit messages on the LTX-2 decoder
    adapter and on the HunyuanVideo causal decoders).
    """
    x = np.asarray(x, dtype=np.float64)
    return np.concatenate([x[:, :1]] * (k_t - 1) + [x], axis=1)


def conv3d_valid(xp: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """Valid (unpadded) 3-D cross-correlation, stride 1.

    xp: [N, T+kt-1, H+kh-1, W+kw-1, Cin] (already padded); w: [Cout, Cin, kt, kh, kw].
    y[n, t, h, w, o] = b[o] + sum_{c, a, p, q} w[o, c, a, p, q] * xp[n, t+a, h+p, w+q, c].
    Evaluated as one matmul of the unfolded input cols[.., (a, p, q), c] = xp[n, t+a, h+p, w+q, c]
    with the weights laid out as wmat[o, (a, p, q), c] = w[o, c, a, p, q].
    """
    xp = np.asarray(xp, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, tp, hp, wp, cin = xp.shape
    cout, cin2, kt, kh, kw = w.shape
    assert cin == cin2, (cin, cin2)
    t_out, h_out, w_out = tp - kt + 1, hp - kh + 1, wp - kw + 1
    assert t_out >= 1 and h_out >= 1 and w_out >= 1, xp.shape
    wmat = np.ascontiguousarray(w.transpose(0, 2, 3, 4, 1)).reshape(cout, kt * kh * kw * cin)
    y = np.empty((n, t_out, h_out, w_out, cout), dtype=np.float64)
    step = max(1, min(t_out, _COLS_ELEMENTS // (n * h_out * w_out * wmat.shape[1])))
    # buffers reused across frame batches (frame-batch axis first so every batch is contiguous)
    cols = np.empty((step, n, h_out, w_out, kt * kh * kw, cin), dtype=np.float64)
    prod = np.empty((step * n * h_out * w_out, cout), dtype=np.float64)
    for t0 in range(0, t_out, step):
        m = min(step, t_out - t0)
        k = 0
        for a in range(kt):
            for p in range(kh):
                for q in range(kw):
                    cols[:m, :, :, :, k, :] = \
                        xp[:, t0 + a:t0 + a + m, p:p + h_out, q:q + w_out, :].swapaxes(0, 1)
                    k += 1
        rows = m * n * h_out * w_out
        np.matmul(cols[:m].reshape(rows, -1), wmat.T, out=prod[:rows])
        y[:, t0:t0 + m] = prod[:rows].reshape(m, n, h_out, w_out, cout).swapaxes(0, 1)
    if b is not None:
        y += np.asarray(b, dtype=np.float64)
    return y


def causal_conv3d(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """Causal Conv3d, kernel 3x3x3, stride 1, on a whole (unsplit) tensor.

    Temporal: two copies of frame 0 in front, so output frame t sees input frames t-2..t, clamped
    at 0. Spatial: one row/column of zeros on every side; zeros appear only at the true image
    border ("Add tiled VAE parallelism & extended model support", commit message on how the direct
    path pads a patch; the single-conv workload states zero padding 1).
    """
    w = np.asarray(w)
    _, _, kt, kh, kw = w.shape
    xp = causal_time_pad(x, kt)
    xp = np.pad(xp, ((0, 0), (0, 0), (kh // 2, kh // 2), (kw // 2, kw // 2), (0, 0)))
    return conv3d_valid(xp, w, b)


def strided_causal_conv3d(x: np.ndarray, w: np.ndarray, b=None, stride=(2, 2, 2),
                          pad_hw=((1, 1), (1, 1))) -> np.ndarray:
    """Strided causal Conv3d: the bare strided downsampler of an encoder.

    One of the four LTX-2 encoder downsample kinds is a bare strided conv, and Wan's downsampler
    pads (0, 1, 0, 1) and then strides 2 over the result ("Add tiled VAE parallelism & extended
    model support", LTX-2 and Qwen-Image/Wan encoder commit messages). Temporal: kt-1 copies of
    frame 0 in front, then output frame t reads padded frames st*t .. st*t + kt - 1 (input frames
    st*t - (kt-1) .. st*t, clamped at 0), so T frames become (T - 1) // st + 1 (121 -> 61).
    Spatial: zero rows/columns ``pad_hw`` = ((top, bottom), (left, right)), then stride.
    Evaluated as the stride-1 valid correlation of the padded input, kept at every stride-th
    position: y[o] = y1[stride * o].
    """
    w = np.asarray(w)
    _, _, kt, kh, kw = w.shape
    st, sh, sw = stride
    xp = causal_time_pad(x, kt)
    xp = np.pad(xp, ((0, 0), (0, 0), tuple(pad_hw[0]), tuple(pad_hw[1]), (0, 0)))
    y1 = conv3d_valid(xp, w, b)
    return np.ascontiguousarray(y1[:, ::st, ::sh, ::sw])


def group_norm(x: np.ndarray, groups: int, eps: float, gamma=None, beta=None) -> np.ndarray:
    """torch.nn.GroupNorm's definition: per (sample, group), over the group's channels and T, H, W.

    mean = average; var = average of squared deviations from that mean (biased, divide by the
    count, no Bessel correction); y = (x - mean) / sqrt(var + eps) * gamma + beta. The DistVAE
    PatchGroupNorm fix names exactly these two properties: the global mean and the count as divisor
    ("Add tiled VAE parallelism & extended model support", PatchGroupNorm commit message).
    Two passes: the mean first, then the squared deviations about it.
    """
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape[0], x.shape[-1]
    assert c % groups == 0, (c, groups)
    xg = x.reshape(n, -1, groups, c // groups)
    y = np.empty_like(xg)
    for g in range(groups):
        part = xg[:, :, g, :]
        mean = part.mean(axis=(1, 2), keepdims=True)
        dev = part - mean
        var = (dev * dev).mean(axis=(1, 2), keepdims=True)
        y[:, :, g, :] = dev / np.sqrt(var + eps)
    y = y.reshape(x.shape)
    if gamma is not None:
        y *= np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y += np.asarray(beta, dtype=np.float64)
    return y


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def nearest_upsample(x: np.ndarray, sh: int, sw: int) -> np.ndarray:
    """out[t, h, w] = in[t, h // sh, w // sw]."""
    x = np.asarray(x, dtype=np.float64)
    return np.repeat(np.repeat(x, sh, axis=2), sw, axis=3)


def depth_to_space(x: np.ndarray, st: int, sh: int, sw: int, drop: bool = True) -> np.ndarray:
    """Depth-to-space upsampling, then causal drop of the first st-1 frames.

    The upsampler moves channels into space, one input position per output ("Add tiled VAE
    parallelism & extended model support", LTX-2 decoder adapter commit message). The pages do not fix
    the channel order. Here input channel ((dt*sh + dh)*sw + dw)*C + c feeds output channel c at
    (st*t + dt, sh*h + dh, sw*w + dw): the sub-position is slowest and the channel fastest. With
    st > 1 the first st-1 frames are dropped, so T frames become st*T - (st-1) (16 -> 31 -> 61 -> 121
    for the LTX-2-shaped workload). ``drop=False`` keeps them: a later clip of a clip-by-clip
    decode continues the sequence, and only the very first frame of the video is dropped.
    """
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, ck = x.shape
    k = st * sh * sw
    assert ck % k == 0, (ck, k)
    c = ck // k
    y = x.reshape(n, t, h, w, st, sh, sw, c)
    y = y.transpose(0, 1, 4, 2, 5, 3, 6, 7).reshape(n, t * st, h * sh, w * sw, c)
    return np.ascontiguousarray(y[:, st - 1:] if drop else y)


def space_to_depth(x: np.ndarray, st: int, sh: int, sw: int) -> np.ndarray:
    """Space-to-depth downsampling with a causal front pad: the fold of the encoder.

    Most LTX-2 encoder downsamplers fold space into channels after a stride-1 convolution
    ("Add tiled VAE parallelism & extended model support", LTX-2 encoder commit message; the same
    page: a downsampler that folds reads one input position per output one). The pages give
    neither the channel order nor the frame rule. Here, the mirror of ``depth_to_space``: st-1
    copies of frame 0 go in front (T frames become (T + st - 1) / st, so 121 -> 61 -> 31 -> 16),
    and input (st*t + dt, sh*h + dh, sw*w + dw, c) of the padded clip lands in output channel
    ((dt*sh + dh)*sw + dw)*C + c at (t, h, w). ``depth_to_space`` of the result gives ``x`` back.
    """
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, c = x.shape
    assert (t + st - 1) % st == 0 and h % sh == 0 and w % sw == 0, (x.shape, st, sh, sw)
    xp = np.concatenate([np.repeat(x[:, :1], st - 1, axis=1), x], axis=1) if st > 1 else x
    to = xp.shape[1] // st
    y = xp.reshape(n, to, st, h // sh, sh, w // sw, sw, c)
    y = y.transpose(0, 1, 3, 5, 2, 4, 6, 7).reshape(n, to, h // sh, w // sw, st * sh * sw * c)
    return np.ascontiguousarray(y)


def rms_norm(x: np.ndarray, eps: float, gamma=None, beta=None) -> np.ndarray:
    """Per-position RMS normalisation over the channels: y = x / sqrt(mean_c(x^2) + eps) * gamma
    + beta.

    Wan-style decoders normalise with RMS norms that reduce over channels only, so a spatial split
    needs no exchange of statistics ("Add tiled VAE parallelism & extended model support", commit
    messages on the Qwen-Image / Wan adapters and on the HunyuanVideo 1.5 encoder). The pages give
    no formula; this is the plainest reading: the root mean square of the position's channel vector,
    eps inside the root, then the per-channel affine.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s - max) / sum(exp(s - max)) along ``axis``."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


def frame_attention(x: np.ndarray, eps: float, gamma, beta, w_qkv, b_qkv, w_out, b_out) -> np.ndarray:
    """Single-head self-attention over the positions of each frame, with its residual.

    A Wan-style decoder's mid block holds one attention block that takes each frame whole: it
    cannot be applied to a patch, so a patch-split decode gathers the frame around it ("Add tiled
    VAE parallelism & extended model support", commit message on the HunyuanVideo adapters; the Wan
    attention block of "[TRTLLM-14123][feat] add ParallelVAE_TrtllmWan for native Wan VAE",
    Description). The pages give no formula; the plainest reading of a single-head spatial block:
      xn = rms_norm(x); [q | k | v] = xn W_qkv^T + b_qkv  (W_qkv [3C, C]);
      per sample and frame, A = softmax(q k^T / sqrt(C)) over the frame's H*W positions;
      y = (A v) W_out^T + b_out + x.
    """
    x = np.asarray(x, dtype=np.float64)
    n, t, h, w, c = x.shape
    xn = rms_norm(x, eps, gamma, beta).reshape(n, t, h * w, c)
    qkv = xn @ np.asarray(w_qkv, np.float64).T + np.asarray(b_qkv, np.float64)
    q, k, v = qkv[..., :c], qkv[..., c:2 * c], qkv[..., 2 * c:]
    a = softmax((q @ np.swapaxes(k, -1, -2)) / np.sqrt(c), axis=-1)
    o = a @ v
    y = o @ np.asarray(w_out, np.float64).T + np.asarray(b_out, np.float64)
    return y.reshape(n, t, h, w, c) + x
