"""The read probe (a measurement helper of the library, timed by bench.py
beside the decode kernel) reads exactly the chunks it is given: the words
it stores XOR to the XOR of every 32-bit word of those chunks, for a plain
stream and for a gather at scattered offsets, with more chunks than its
grid has blocks."""
import numpy as np
import pytest
import torch

from sparse_kv_cache_hsa_amd import rkv

pytestmark = pytest.mark.gpu


def xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel()))


@pytest.mark.parametrize("n_chunks", [1, 7, 2048, 5000])
def test_read_probe_stream_reads_every_word(n_chunks):
    chunk = rkv.RKV_READ_PROBE_CHUNK
    g = torch.Generator().manual_seed(n_chunks)
    host = torch.randint(0, 256, (n_chunks * chunk,), generator=g, dtype=torch.uint8)
    print(f"read probe stream: {n_chunks} chunks", flush=True)
    buf = host.cuda()
    sink = torch.zeros(rkv.RKV_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    rkv.rkv_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert xor_words(sink.cpu().numpy()) == xor_words(host.numpy())


@pytest.mark.parametrize("n_chunks", [3, 3000])
def test_read_probe_gather_reads_the_given_chunks(n_chunks):
    chunk = rkv.RKV_READ_PROBE_CHUNK
    total = 4096
    g = torch.Generator().manual_seed(100 + n_chunks)
    host = torch.randint(0, 256, (total * chunk,), generator=g, dtype=torch.uint8)
    pick = torch.randperm(total, generator=g)[:n_chunks]
    print(f"read probe gather: {n_chunks} of {total} chunks", flush=True)
    buf = host.cuda()
    sink = torch.zeros(rkv.RKV_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    rkv.rkv_read_probe(buf, sink, (pick * chunk).to(torch.int64).cuda())
    torch.cuda.synchronize()
    rows = host.view(total, chunk)[pick].numpy()
    assert xor_words(sink.cpu().numpy()) == xor_words(rows)


def test_read_probe_binding_rejects_offsets_outside_the_buffer():
    chunk = rkv.RKV_READ_PROBE_CHUNK
    buf = torch.zeros(4 * chunk, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(rkv.RKV_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    for bad in ([3 * chunk + 16], [-16], [8]):
        with pytest.raises(ValueError):
            rkv.rkv_read_probe(buf, sink, torch.tensor(bad, dtype=torch.int64, device="cuda"))
