"""The measurement kernels of the benchmark compute what they claim: the
reader's per-lane XOR of every run it read equals the same XOR formed here,
and the spinning wave reports a shader clock in the GPU's range."""
import numpy as np
import pytest
import torch

import bench

from gpu_helpers import device, log

pytestmark = pytest.mark.gpu


def test_read_runs_checksum_matches_host():
    dev = device()
    calib = bench.Calib()
    g = torch.Generator(device="cpu").manual_seed(5)
    pool = torch.randint(0, 2**31 - 1, (64, 1024), generator=g, dtype=torch.int32)  # 64 runs of 4 KiB
    pool_d = pool.to(dev)
    rng = np.random.default_rng(5)
    lens = [0, 1, 7, 8, 9, 20, 3]               # runs per wave, including an empty wave
    begin = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    runs = rng.integers(0, 64, int(begin[-1]))
    for kib in (4, 2):
        addrs = (pool_d.data_ptr() + runs * 4096).astype(np.int64)
        sink = torch.full((64 * len(lens),), -1, dtype=torch.int32, device=dev)
        calib.read_runs(torch.from_numpy(addrs).to(dev), torch.from_numpy(begin).to(dev), kib,
                        sink, torch.cuda.current_stream(dev))
        torch.cuda.synchronize(dev)
        got = sink.cpu().numpy().view(np.uint32).reshape(len(lens), 64)
        words = pool.numpy().view(np.uint32).reshape(64, 4, 64, 4)  # run, KiB, lane, word
        for w in range(len(lens)):
            want = np.zeros(64, np.uint32)
            for r in runs[begin[w]:begin[w + 1]]:
                for j in range(kib):
                    want ^= np.bitwise_xor.reduce(words[r, j], axis=1)
            assert np.array_equal(got[w], want), (kib, w)


def test_clock_is_in_range():
    dev = device()
    calib = bench.Calib()
    stream = torch.cuda.current_stream(dev)
    mhz = calib.clock(5.0, stream)
    torch.cuda.synchronize(dev)
    log(f"shader clock of an idle wave: {mhz():.0f} MHz")
    assert 300.0 < mhz() < 3500.0
