"""The streaming-read reference (moe_bench_stream_read): reads any multiple of
16 bytes (whole and partial workgroups), writes nothing unless its data
reduces to the magic value, and is capturable."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 49152, 49152 * 3 + 160, 75497472])
def test_stream_read_leaves_sink(nbytes):
    from nvfp4_weight_only_moe_amd import binding as B
    src = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda:0")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda:0")
    B.moe_bench_stream_read(src, nbytes, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]


def test_stream_read_in_graph():
    from nvfp4_weight_only_moe_amd import binding as B
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.moe_bench_stream_read(src, src.numel(), sink)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_bench_stream_read(src, src.numel(), sink)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    assert sink.item() == 0
