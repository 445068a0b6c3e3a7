"""The read-bandwidth probe returns the sum of the buffer's 64-bit words
modulo 2^64, exactly as the oracle's definition gives it, for sizes from
empty to the 2 GiB buffer the benchmark times: fewer 16-byte pieces than
waves (waves with empty shares), a trailing 8-byte word, shares that end in
a partial round of 16 loads, and many full rounds per wave."""
import numpy as np
import pytest
import torch

from draft_tree_construction_02_amd import _abi as A
from oracle import dartree_oracle as O
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _probe(buf_u8: torch.Tensor) -> int:
    out = A.hbm_read_probe(buf_u8)
    torch.cuda.synchronize()
    return int(out.cpu().numpy().view(np.uint64)[0])


@pytest.mark.parametrize("nbytes", [0, 8, 16, 24, 4096 + 8, 16 * 255, 16 * 257 + 8,
                                    (1 << 20) + 24, 3 * 2048 * 256 * 16 * 8 + 40])
def test_probe_sum_matches_oracle(nbytes):
    print(f"probe {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    raw = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(raw).to(DEV)
    assert _probe(buf) == O.word_sum64(raw)


def test_probe_on_benchmark_size_and_offsets():
    # the 2 GiB buffer of the bandwidth measurement plus one trailing word,
    # then 16-byte-aligned views that start inside it
    n = (2 << 30) + 8
    print(f"probe {n} bytes", flush=True)
    rng = np.random.default_rng(11)
    raw = rng.integers(0, 2 ** 63, n // 8, dtype=np.uint64).view(np.uint8)
    buf = torch.from_numpy(raw).to(DEV)
    assert _probe(buf) == O.word_sum64(raw)
    for off, ln in ((16, 4096), (1 << 30, (1 << 20) + 8)):
        assert _probe(buf[off:off + ln]) == O.word_sum64(raw[off:off + ln])
    # an unaligned start is rejected on the host
    with pytest.raises(A.DartreeError):
        A.hbm_read_probe(buf[8:24])
    del buf
    torch.cuda.empty_cache()
