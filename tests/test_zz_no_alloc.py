"""The entry point that allocates nothing (the streaming-read probe with the
library's own scratch array) against the entry point whose scratch the
caller passes in, and both against an emulation of the probe's reads."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _expected(buf_u32, nbytes, grid, waves, depth, pattern):
    """XOR of everything the probe reads: wavefront g reads blocks of 1 KB
    in a window of `depth`; the loop consumes ceil(n / depth) * depth loads,
    the ones past the end re-reading the last block."""
    tw = grid * waves
    n = nbytes // 1024 // tw
    blocks = buf_u32[: nbytes // 4].reshape(-1, 256)
    bx = np.bitwise_xor.reduce(blocks, axis=1)          # XOR of each block
    steps = -(-n // depth) * depth
    k = np.minimum(np.arange(steps), n - 1)
    g = np.arange(tw)[:, None]
    idx = k[None, :] * tw + g if pattern else g * n + k[None, :]
    return int(np.bitwise_xor.reduce(bx[idx.ravel()]))


def test_noalloc_probe_matches_the_probe_with_caller_scratch():
    import torch
    import tree_verification_spec_amd as L
    L.lib()
    dev = torch.device("cuda", 0)
    gen = torch.Generator().manual_seed(81)
    host = torch.randint(-2**31, 2**31 - 1, (20 << 20,), dtype=torch.int32, generator=gen)
    buf = host.to(dev)
    host_u32 = host.numpy().view(np.uint32)
    stream = torch.cuda.Stream(device=dev)
    out = torch.zeros(2, dtype=torch.int32, device=dev)
    # two calls in a row, the second smaller (fewer wavefronts and bytes)
    for nbytes, grid, waves, depth, pattern in ((48 << 20, 96, 8, 8, 1),
                                                (5 << 20, 40, 4, 4, 0)):
        sink = torch.full((grid * waves,), -1, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            L.spec_probe_read_bandwidth(buf.data_ptr(), nbytes, grid, waves, depth, pattern,
                                        sink.data_ptr(), stream.cuda_stream)
            L.spec_probe_read_bandwidth_noalloc(buf.data_ptr(), nbytes, grid, waves, depth,
                                                pattern, out.data_ptr(), stream.cuda_stream)
        stream.synchronize()
        ref = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
        got = int(out[0].cpu().numpy().view(np.uint32))
        want = _expected(host_u32, nbytes, grid, waves, depth, pattern)
        assert ref == want and got == want, (nbytes, grid, waves, hex(ref), hex(got), hex(want))
    # more wavefronts than the scratch array holds are refused before any
    # launch (the read itself would stay inside the 80 MiB buffer)
    with pytest.raises(L.SpecError):
        L.spec_probe_read_bandwidth_noalloc(buf.data_ptr(), 1024 * 4100 * 16, 4100, 16, 8, 1,
                                            out.data_ptr(), stream.cuda_stream)
