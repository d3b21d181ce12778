"""The rate probes of include/segpaged_probe.h on the GPU: the streaming-read
probe reads every byte once (its partial sums add up to the buffer's sum), and
the MFMA probe runs and is deterministic."""
import numpy as np
import pytest
import torch

from sparse_attention_segmentpagetable_amd import probe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("depth", [4, 8, 16])
@pytest.mark.parametrize("n,wgs", [(4, 1), (4 * 1000 + 4, 3), (1 << 20, 64), ((1 << 22) + 36, 257)])
def test_hbm_read_probe_reads_every_chunk_once(n, wgs, depth):
    g = torch.Generator(device="cpu").manual_seed(n)
    x = torch.randn(n, generator=g, dtype=torch.float32)
    out = torch.full((wgs,), float("nan"), dtype=torch.float32, device=DEV)
    probe.hbm_read(x.to(DEV), wgs, out, depth=depth)
    torch.cuda.synchronize()
    got = out.double().sum().item()
    ref = x.double().sum().item()
    # fp32 partial sums: error grows like sqrt(n) ulps of the magnitudes summed
    assert abs(got - ref) <= 1e-5 * float(x.abs().sum()) + 1e-6, (got, ref)
    assert torch.isfinite(out).all()


def test_mfma_probe_runs_and_is_deterministic():
    g = torch.Generator(device="cpu").manual_seed(7)
    seed = torch.randn(probe.SEED_ELEMS, generator=g).to(torch.bfloat16).to(DEV)
    outs = []
    for _ in range(2):
        out = torch.full((2 * 512,), float("nan"), dtype=torch.float32, device=DEV)
        probe.mfma_bf16(seed, 3, 2, out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1])
    assert np.any(outs[0] != 0)
