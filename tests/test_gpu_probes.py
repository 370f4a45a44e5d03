"""The measurement probes (spkv_probe_read, spkv_probe_mfma) compute what they
claim, so that the ceilings the bench reports come from kernels that really
read every byte and really run every MFMA (needs an MI355X).

probe_read: the XOR of all 32-bit words of a seeded buffer (the XOR of the
per-wave sink words), against numpy, for a buffer inside one 32 KB chunk,
one that ends mid-chunk, and two of more chunks than blocks (the grid
strides; a sink of 8 words allows 2 blocks), each with a ragged last chunk.
probe_mfma: per wave, 8 accumulator chains x iters x the sum of all entries
of A.B for the fixed operand pattern; the sum over a product's entries is
sum_k (column sum of A)_k (row sum of B)_k, written from the 32x32x16 operand
placement (A[m][k] in lane m + 32*(k/8), element k%8; B[k][n] in lane
n + 32*(k/8), element k%8).
"""
import sys

import numpy as np
import pytest
import torch

from shared_prefix_paged_amd import runtime as R

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("nbytes,sink_words", [(4096, 4096), (16 * 1000 + 48, 4096),
                                                ((256 << 20) + 16 * 37, 1 << 16), ((1 << 20) + 16 * 5, 8)])
def test_probe_read_xor_matches_numpy(nbytes, sink_words):
    note(f"[probe_read] bytes={nbytes} sink_words={sink_words}")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.zeros(sink_words, dtype=torch.int32, device="cuda:0")
    R.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    assert got == int(np.bitwise_xor.reduce(host))


def test_probe_read_refuses_bad_sizes():
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    with pytest.raises(Exception):
        R.probe_read(torch.zeros(10, dtype=torch.int32, device="cuda:0"), sink)      # 40 bytes
    with pytest.raises(Exception):
        R.probe_read(torch.zeros(16, dtype=torch.int32, device="cuda:0"), sink[:3])  # sink too small


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("waves,iters", [(4, 1), (64, 7)])
def test_probe_mfma_sum_matches_closed_form(waves, iters):
    note(f"[probe_mfma] waves={waves} iters={iters}")
    a = np.zeros((32, 16))
    b = np.zeros((16, 32))
    for lane in range(64):
        for e in range(8):
            k = 8 * (lane // 32) + e
            a[lane % 32, k] = 0.001 * ((lane + e) & 7)
            b[k, lane % 32] = 0.001 * ((lane * 3 + e) & 7)
    a, b = _bf16(a), _bf16(b)
    expect = 8 * iters * float(np.sum(a.sum(axis=0) * b.sum(axis=1)))
    sink = torch.full((waves,), float("nan"), dtype=torch.float32, device="cuda:0")
    R.probe_mfma(waves, iters, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - expect) <= 1e-4 * abs(expect)), (got[:4], expect)
