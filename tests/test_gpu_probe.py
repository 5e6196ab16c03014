"""The streaming-rate probe (dl_stream_probe) moves the bytes it is asked to:
a copy is bit-exact, a read writes one float32 sum per 32 KiB block."""
from __future__ import annotations

import pytest
import torch

from linear_attention_recurrent_gated_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 * 3 + 16 * 7, 1 << 24])
def test_probe_copy_and_read(nbytes):
    print(f"case probe bytes={nbytes}", flush=True)
    n = nbytes // 4
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    x = torch.randint(-8, 9, (n,), device="cuda", generator=g).float()   # sums exact in fp32
    y = torch.full_like(x, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    B.dl_stream_probe(B.DL_PROBE_COPY, x.data_ptr(), y.data_ptr(), nbytes, stream)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    blocks = -(-nbytes // 32768)
    out = torch.full((blocks + 1,), float("nan"), device="cuda")
    B.dl_stream_probe(B.DL_PROBE_READ, x.data_ptr(), out.data_ptr(), nbytes, stream)
    torch.cuda.synchronize()
    pad = torch.zeros(blocks * 8192, device="cuda")
    pad[:n] = x
    assert torch.equal(out[:blocks], pad.view(blocks, 8192).sum(1))
    assert torch.isnan(out[blocks])            # nothing written past the last block
