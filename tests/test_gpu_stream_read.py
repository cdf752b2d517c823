"""The streaming-read measurement primitive (kv_stream_read): it reads the
listed tiles, including ids outside the buffer (which read nothing), leaves
the sink alone for data that do not hash to its value, and rejects bad
arguments before launching."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_stream_read_runs_and_keeps_sink():
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    announce("kv_stream_read 64 MiB")
    dev = torch.device("cuda", 0)
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)   # zeros hash to 0
    n = buf.numel() // 4096
    g = torch.Generator().manual_seed(449)
    ids = torch.randperm(n, generator=g).to(torch.int32)
    ids = torch.cat([ids, torch.tensor([-1, n, n + 5, 2**31 - 1], dtype=torch.int32)]).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for tile in (4096, 16384):
        t = ids if tile == 4096 else (ids // 4).contiguous()
        pk.kv_stream_read(buf, tile, t, sink)
    torch.cuda.synchronize(dev)
    assert sink.item() == 0
    with pytest.raises(pk.PagedKVError):
        pk.kv_stream_read(buf, 1000, ids, sink)
    with pytest.raises(pk.PagedKVError):
        pk.kv_stream_read(buf[:1024], 4096, ids, sink)
