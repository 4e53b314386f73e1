"""The read probe (a plain stream over device memory, the bandwidth reference of the benchmark) reads every
16-byte vector once: each workgroup's XOR of its words matches the same partition done in numpy."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 1000, 4096 * 2048 * 2 + 4096 * 5 + 1234])
def test_read_probe_reads_every_vector_once(n16):
    import torch
    import attention_block_amd as ab
    print(f"[read probe] {n16} vectors", flush=True)
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(ab.READ_PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    ab.read_probe(buf, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    # vector v lies in 64 KB chunk v // 4096, which workgroup (v // 4096) % blocks reads
    G, C = ab.READ_PROBE_BLOCKS, 4096
    vec_xor = np.bitwise_xor.reduce(words.reshape(n16, 4), axis=1)
    nchunk = -(-n16 // C)
    chunks = np.zeros(nchunk * C, dtype=np.uint32)
    chunks[:n16] = vec_xor
    chunk_xor = np.bitwise_xor.reduce(chunks.reshape(nchunk, C), axis=1)
    rounds = -(-nchunk // G)
    padded = np.zeros(rounds * G, dtype=np.uint32)
    padded[:nchunk] = chunk_xor
    want = np.bitwise_xor.reduce(padded.reshape(rounds, G), axis=0)
    assert np.array_equal(got, want)
