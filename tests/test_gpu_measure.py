"""GPU: the measurement kernel ada_hbm_read (the streaming-read floor the
decode calls are compared with) reads every 16-byte chunk of its buffer
exactly once: each wavefront's xor of what it read equals the xor of the
chunks its lanes own, computed on the CPU (chunk i goes to thread
i mod (256 * workgroups), wavefront thread / 64)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ada():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import autoregressive_decode_attention_amd as m

    return m


def expected_xor(words: np.ndarray, workgroups: int) -> np.ndarray:
    chunks = words.reshape(-1, 4)
    per_chunk = np.bitwise_xor.reduce(chunks, axis=1)
    threads = 256 * workgroups
    owner = np.arange(len(per_chunk)) % threads // 64
    out = np.zeros(4 * workgroups, dtype=np.uint32)
    np.bitwise_xor.at(out, owner, per_chunk)
    return out


@pytest.mark.parametrize("nbytes,workgroups", [(1 << 20, 256), ((1 << 20) + 16 * 37, 256), (12345 * 16, 7),
                                               (64 << 20, 1024), (16, 3)])
def test_hbm_read_reads_every_chunk_once(ada, nbytes, workgroups):
    print(f"case hbm_read: {nbytes} bytes, {workgroups} workgroups", flush=True)
    g = torch.Generator().manual_seed(nbytes + workgroups)
    words = torch.randint(0, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = words.cuda()
    sink = torch.full((4 * workgroups,), -1, dtype=torch.int32, device="cuda")
    ada.hbm_read(src, sink, workgroups)
    torch.cuda.synchronize()
    want = expected_xor(words.numpy().view(np.uint32), workgroups)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)
