"""vae_groupnorm_silu_noalloc (the GroupNorm + SiLU entry point that allocates nothing; its scratch
is the library's fixed per-GPU array) against vae_groupnorm_silu with a caller workspace, through
the C ABI. Same kernels, so the outputs must agree bit for bit; both also meet the per-op bound
against the oracle (half a bf16 ulp plus 1e-4 relative, or 1e-4 relative for fp32 outputs)."""
import numpy as np
import pytest

import oracle
import vae_synth
from _util import ndhwc, dev, host, rel_max_abs, bf16_round_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    import torch
    import video_diffusion_vae_amd as v
    assert torch.cuda.is_available()
    return v


# two calls in a row, the second on a smaller input: (N, C, T, H, W), groups, in, out, boxes
CALLS = [
    ((1, 256, 5, 16, 40), 32, "f32", "bf16",
     [(0, 5, 0, 16, 0, 10), (0, 5, 0, 16, 10, 20), (0, 5, 0, 16, 20, 30),
      (0, 5, 0, 16, 30, 40)]),
    ((2, 64, 3, 8, 10), 8, "bf16", "f32", None),
]


def _one(v, shape, groups, idt, odt, boxes, seed):
    import torch
    n, c, t, h, w = shape
    x = ndhwc(vae_synth.normal(shape, [90, seed], scale=1.5, mean=0.3, dtype=idt))
    gamma = vae_synth.normal((c,), [91, seed], scale=0.2, mean=1.0)
    beta = vae_synth.normal((c,), [92, seed], scale=0.1)
    xd = dev(x, idt)
    gd = torch.as_tensor(gamma, device="cuda")
    bd = torch.as_tensor(beta, device="cuda")
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    y_ws = torch.full(xd.shape, 7.0, dtype=tdt, device="cuda")
    y_na = torch.full(xd.shape, -7.0, dtype=tdt, device="cuda")
    v.vae_groupnorm_silu(xd, boxes, groups, 1e-6, gd, bd, True, y_ws)
    torch.cuda.synchronize()
    # the program's own work between the calls
    junk = torch.randn(1 << 20, device="cuda").sum()
    v.vae_groupnorm_silu_noalloc(xd, boxes, groups, 1e-6, gd, bd, True, y_na)
    torch.cuda.synchronize()
    assert torch.isfinite(junk)
    assert torch.equal(y_ws, y_na)
    ref = oracle.silu(oracle.group_norm(x, groups, 1e-6, gamma, beta))
    got = host(y_na)
    if odt == "f32":
        assert rel_max_abs(got, ref) <= 1e-4
    else:
        assert np.all(np.abs(got - ref) <= bf16_round_bound(ref) + 1e-4 * np.abs(ref).max())


def test_noalloc_groupnorm_equals_workspace_call_twice(v):
    """Two calls in a row, the second smaller, each against the workspace call's output."""
    for i, (shape, groups, idt, odt, boxes) in enumerate(CALLS):
        _one(v, shape, groups, idt, odt, boxes, i)
