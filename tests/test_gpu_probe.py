"""GPU check of the streaming-read probe (nvkv_read_probe), the measurement helper behind the
bench's read ceiling: it must read every 16-byte chunk of its buffer and write nothing else."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MAGIC = 0x9E3779B9 - (1 << 32)          # the probe's fold value, as an int32


def test_read_probe_reads_the_chunk_that_matches():
    import bit_paged_kv_amd as nv
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)       # 4 MiB: 262144 chunks
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for chunk in (0, 123457, (1 << 18) - 1):                        # first, middle and last chunk
        buf.zero_()
        buf[4 * chunk + 2] = MAGIC
        sink.zero_()
        nv.read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == MAGIC, chunk
        buf[4 * chunk + 3] = 1                                      # fold no longer matches
        sink.zero_()
        nv.read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0, chunk
    assert int(buf.count_nonzero().item()) == 2                     # the probe wrote nothing to buf


def test_read_probe_small_buffer():
    import bit_paged_kv_amd as nv
    buf = torch.zeros(4, dtype=torch.int32, device=DEV)             # one chunk, far fewer than the threads
    buf[0] = MAGIC
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    nv.read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == MAGIC
