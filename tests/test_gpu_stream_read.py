"""The yardsticks.  The streaming read (pa_stream_read) reads what it is given:
a one-thread read of a vector whose words XOR to the marker stores the marker
in sink, any other vector leaves sink alone; a large read completes.  The
prefill-loop yardstick (pa_attention_loop_peak) runs in every mode and counts
its flops."""

import pytest
import torch

import paged_kv_cache_424_amd as pa

pytestmark = pytest.mark.gpu

MARK = 0x9e3779b9


def test_stream_read_reads_its_input():
    print("[gpu-case] stream read", flush=True)
    src = torch.tensor([MARK - (1 << 32), 0, 0, 0], dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_stream_read(src, sink, 1, 4, 0)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MARK
    sink.zero_()
    pa.pa_stream_read(src, sink, 1, 16, 1)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MARK
    src = torch.tensor([1, 2, 4, 8], dtype=torch.int32, device="cuda")
    sink.zero_()
    pa.pa_stream_read(src, sink, 1, 1)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    big = torch.zeros((1 << 28) + 48, dtype=torch.uint8, device="cuda")     # grid-stride loop and its tail
    for shape in ((4, 4, 0), (8, 8, 0), (32, 1, 0), (8, 16, 1), (4, 4, 1)):
        pa.pa_stream_read(big, sink, *shape)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_attention_loop_peak_runs_every_mode():
    """The prefill-loop yardstick runs in its three modes, reports the flops of
    its launch (2 workgroups per CU x 4 waves x iterations x 32 MFMAs of
    32x32x16), and the fuller modes are not faster than the emptier ones by
    more than timing noise."""
    src = torch.zeros(2 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rate = {}
    for mode in (0, 1, 2):
        pa.pa_attention_loop_peak(src, sink, 10, mode)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = pa.pa_attention_loop_peak(src, sink, 200, mode)
        e1.record()
        torch.cuda.synchronize()
        assert flops == 2 * cus * 4 * 200 * 32 * 32 * 32 * 16 * 2
        rate[mode] = flops / e0.elapsed_time(e1)
    assert rate[2] <= rate[0] * 1.1
