"""GPU checks of the HBM bandwidth probe (include/gdn_probe.h), the kernels
whose timing gives the access pattern's achievable ceiling: the copy is
bit-exact, the write fills each chunk with its index, and the read kernel's
word per chunk is the XOR of the chunk's 16-byte words (checked with numpy).
37 chunks: more than the XCD count and not a multiple of it, so the id
remap's tail is covered."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_copy_write_read(gdn):
    G = gdn
    ch = G.GDN_PROBE_CHUNK
    n = 37 * ch
    gen = torch.Generator(device="cuda").manual_seed(7)
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda",
                        generator=gen)
    dst = torch.zeros_like(src)
    G.gdn_bandwidth_probe(G.PROBE_COPY, src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)

    G.gdn_bandwidth_probe(G.PROBE_WRITE, None, dst)
    torch.cuda.synchronize()
    want = torch.arange(n // ch, dtype=torch.int32, device="cuda").repeat_interleave(ch // 4)
    assert torch.equal(dst, want)

    sink = torch.zeros(n // ch * 4, dtype=torch.int32, device="cuda")
    G.gdn_bandwidth_probe(G.PROBE_READ, src, sink, n)
    torch.cuda.synchronize()
    words = src.cpu().numpy().view(np.uint32).reshape(n // ch, ch // 16, 4)
    xor = np.bitwise_xor.reduce(words, axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), xor)
