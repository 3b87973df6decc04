"""The streaming-read probe (include/ffd_probe.h) reads every 16-byte word of its buffer exactly
once: each work-group's XOR of its chunk equals numpy's XOR over the same chunk."""
import numpy as np
import pytest
import torch

from helpers import DEV
from long_context_decoding_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,groups", [(1, 1), (5, 8), (1000, 7), (4096 * 3 + 5, 64), (1 << 20, 256)])
def test_probe_xor_per_work_group(n16, groups):
    rng = np.random.default_rng(n16 + groups)
    words = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.full((groups, 4), -1, dtype=torch.int32, device=DEV)
    probe.stream_read(src, groups, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    chunk = (n16 + groups - 1) // groups
    for g in range(groups):
        part = words[g * chunk:min((g + 1) * chunk, n16)]
        want = np.bitwise_xor.reduce(part, axis=0) if len(part) else np.zeros(4, np.uint32)
        np.testing.assert_array_equal(got[g], want, err_msg=f"work-group {g}")
