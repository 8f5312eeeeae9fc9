"""The reference copy that bench.py compares the append with (wf_stream_copy): bit-exact, and
nothing written past the requested bytes (needs an MI355X)."""
import pytest
import torch

import chunk_causal_dit_wf_amd as wf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 16 * 1024 * 4 * 2048 + 48, 28753920])
def test_stream_copy_bitexact_and_bounded(nbytes):
    print("case: stream copy", nbytes, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes + 64,), generator=g, dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    wf.wf_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool((dst[nbytes:] == 0xA5).all())
