"""pkv_hbm_read_probe (measurement helper): it reads the whole buffer (the
XOR of what a thread read reaches the sink exactly when it equals the tag)
and refuses misaligned or foreign buffers on the host, before any launch."""
import numpy as np
import pytest
import torch

import paged_kv_cache_406_amd as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16 * 7, 64 << 20])
def test_read_probe_reads_and_reports_only_on_tag(nbytes):
    # a buffer of equal words: every 16-byte group XORs to 0, so every
    # thread's XOR is 0 and tag 0 is stored, any other tag is not
    buf = torch.full((nbytes // 4,), 1.0, dtype=torch.float32, device="cuda")
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    P.pkv_hbm_read_probe(buf, nbytes, sink, tag=0x9E3779B9, stream=s)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
    P.pkv_hbm_read_probe(buf, nbytes, sink, tag=0, stream=s)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_read_probe_xor_of_one_thread():
    # one group of distinct words: a single thread reads it and stores the
    # XOR of its four words when that is the tag
    words = np.array([0x01020304, 0x10203040, 0x0A0B0C0D, 0x77777777], dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    x = int(np.bitwise_xor.reduce(words))
    P.pkv_hbm_read_probe(buf, 16, sink, tag=x, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == x


def test_read_probe_argument_checks():
    buf = torch.zeros(1024, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    host = torch.zeros(1024, dtype=torch.float32)
    with pytest.raises(RuntimeError):
        P.pkv_hbm_read_probe(buf.data_ptr() + 4, 1024, sink)      # misaligned
    with pytest.raises(RuntimeError):
        P.pkv_hbm_read_probe(buf, 1000, sink)                     # not a multiple of 16
    with pytest.raises(RuntimeError):
        # past the allocation (torch's caching allocator serves this tensor
        # from a 2 MiB segment: 64 MiB reaches beyond it)
        P.pkv_hbm_read_probe(buf, 64 << 20, sink)
    with pytest.raises(RuntimeError):
        P.pkv_hbm_read_probe(host, 1024, sink)                    # host memory
