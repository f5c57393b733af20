"""GPU checks of the streaming-read probe (moe_decode_read_probe): every byte
read exactly once, whatever the size's remainder against the block step."""
import numpy as np
import pytest
import torch

from gpu_cases import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("nbytes", [16, 4096, 16384 + 48, 21233664, (1 << 28) + 48])
def test_read_probe_sums_every_element_once(nbytes):
    import quantized_moe_decode_amd as qmd
    say(f"case read probe {nbytes} bytes of ones")
    data = torch.ones(nbytes // 4, device=DEV)
    part = torch.full((qmd.read_probe_blocks(nbytes) + 3,), -7.0, device=DEV)
    qmd.moe_decode_read_probe(data, part)
    torch.cuda.synchronize()
    n = qmd.read_probe_blocks(nbytes)
    p = part.cpu().numpy().astype(np.float64)
    assert p.sum() - p[n:].sum() == nbytes // 4          # every element once (sums of ones are exact)
    assert np.all(p[n:] == -7.0)                          # nothing written past the grid


def test_read_probe_random_values():
    import quantized_moe_decode_amd as qmd
    say("case read probe random values")
    g = torch.Generator().manual_seed(7)
    host = torch.randn(3 * 65536 + 4, generator=g)
    data = host.to(DEV)
    part = torch.zeros(qmd.read_probe_blocks(data.numel() * 4), device=DEV)
    qmd.moe_decode_read_probe(data, part)
    torch.cuda.synchronize()
    got = part.cpu().double().sum().item()
    want = host.double().sum().item()
    # fp32 summation over at most ~70 sequential additions per term: error <= 70 eps sum|x|
    assert abs(got - want) <= 1e-5 * host.double().abs().sum().item()
