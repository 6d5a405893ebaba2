"""The reference kernels of kvq_probe.h run and leave their sink alone.

They carry no arithmetic the path depends on: the streaming read, the
matrix-core loop and the LDS read loop only give the bench the rates the part
reaches (HBM, fp16 matrix products, LDS reads).  Each writes its sink only when
its fold equals a value that these inputs never produce, so an untouched sink
and a clean launch are what can be checked.
"""

import pytest
import torch

from bit_kv_cache_04_amd import kvq

pytestmark = pytest.mark.gpu


def test_reference_kernels_run():
    dev = torch.device("cuda:0")
    buf = torch.full((1 << 20,), 7, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    print("probes: stream read 4 MiB, mfma 8 x 4, lds 8 x 4", flush=True)
    kvq.kv_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), st)
    kvq.kv_mfma_probe(8, 4, sink.data_ptr(), st)
    kvq.kv_lds_probe(8, 4, sink.data_ptr(), st)
    torch.cuda.synchronize()
    assert torch.equal(sink.cpu(), torch.zeros(4, dtype=torch.int32))
