"""The entry point that allocates nothing (k3moe_layer_noalloc): the layer on the
library's fixed device array, against k3moe_layer on a workspace of its own, on the
same inputs, two calls in a row (the second on a smaller batch, so it runs on what the
first left in the array). Ids bit-exact; y within the layer's bar (rel-L2 1e-5 per row,
max-abs 1e-4 of the row's largest value). Batches whose workspace exceeds the array are
refused before anything runs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import k3gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from mxfp4_routed_expert_amd import device, k3moe  # noqa: E402

REL = 1e-5
ABSF = 1e-4


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def upload(d, seed):
    dense = k3gen.gen_dense(d, seed)
    lay = k3gen.ExpertLayout(d)
    B = lay.blob_bytes
    chunks = ((e0, k3gen.gen_experts(d, seed, e0, min(d.n_experts, e0 + 64)))
              for e0 in range(0, d.n_experts, 64))
    return device.upload_layer(d, dense, chunks, B, lay.offsets)


def both(dev, d, x: np.ndarray):
    T = x.shape[0]
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    out = {}
    for name in ("layer", "noalloc"):
        y = torch.full((T, d.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, d.topk), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, d.topk), float("nan"), dtype=torch.float32, device="cuda")
        if name == "layer":
            ws = device.workspace(d, T)
            k3moe.k3moe_layer(d, T, xd, dev.weights_struct(), y, idx, w, ws)
        else:
            k3moe.k3moe_layer_noalloc(d, T, xd, dev.weights_struct(), y, idx, w)
        torch.cuda.synchronize()
        out[name] = (y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
    return out


def check(out, what):
    (y0, i0, w0), (y1, i1, w1) = out["layer"], out["noalloc"]
    assert np.array_equal(i0, i1), f"{what}: expert ids differ"
    assert np.all(np.isfinite(y1)) and np.all(np.isfinite(w1)), what
    a, b = y1.astype(np.float64), y0.astype(np.float64)
    rel = np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)
    mabs = np.max(np.abs(a - b), axis=1) / np.maximum(np.max(np.abs(b), axis=1), 1e-30)
    wrel = np.max(np.abs(w1.astype(np.float64) - w0) / np.maximum(np.abs(w0), 1e-30))
    say(f"  {what}: max row rel-L2 {rel.max():.3e}, max abs/max|ref| {mabs.max():.3e}, "
        f"bit-identical {np.array_equal(y0, y1)}")
    assert rel.max() <= REL and mabs.max() <= ABSF, what
    assert wrel <= 1e-6, what


@pytest.mark.parametrize("shape", ["tiny", "k3"])
def test_noalloc_matches_layer_two_calls(shape):
    d = k3gen.TINY if shape == "tiny" else k3gen.K3
    seeds = (0, 1) if shape == "tiny" else (1, 1)
    say(f"uploading the {shape} layer")
    dev = upload(d, seeds[0])
    for T in ((64, 5) if shape == "tiny" else (32, 1)):
        assert k3moe.k3moe_workspace_size(d, T) <= k3moe.NOALLOC_SCRATCH_BYTES
        say(f"no-alloc layer {shape} T={T}")
        x = k3gen.gen_x(d, 80 + T, T)
        check(both(dev, d, x), f"{shape} T={T}")
    del dev
    torch.cuda.empty_cache()


def test_noalloc_refuses_a_batch_beyond_its_array():
    d = k3gen.K3
    T = 64  # about 123 MB of workspace
    assert k3moe.k3moe_workspace_size(d, T) > k3moe.NOALLOC_SCRATCH_BYTES
    y = torch.zeros((T, d.hidden), dtype=torch.float32, device="cuda")
    fake = 1 << 20  # never dereferenced: the call is refused on the host
    w = k3moe.k3moe_weights(fake, fake, fake, fake, fake,
                            k3moe.k3moe_experts(*(k3moe.k3moe_mxfp4(fake, fake, 1 << 16, 4096),) * 3))
    rc = k3moe.k3moe_layer_noalloc(d, T, fake, w, y, None, None, check=False)
    assert rc == k3moe.K3MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert not y.any().item()
