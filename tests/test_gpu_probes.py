"""The measurement probes on the GPU: kvq_probe_clock reads a plausible shader clock on every
XCD, and kvq_probe_stream_read reads a buffer in each load form without touching the sink."""
import pytest
import torch

from long_context_decode_flash_amd import kvq

pytestmark = pytest.mark.gpu


def test_clock_probe_reads_every_xcd():
    dev = torch.device("cuda:0")
    wg = 256
    out = torch.zeros(3 * wg, dtype=torch.int64, device=dev)
    khz = kvq.clock_counter_khz()
    assert khz > 0
    call = kvq.prepare_clock_probe(out, 2000)
    call()
    torch.cuda.synchronize()
    v = out.view(wg, 3).cpu()
    cycles, ticks, xcd = v[:, 0], v[:, 1], v[:, 2]
    assert bool((ticks >= 2000).all()) and bool((cycles > 0).all())
    mhz = cycles.double() / ticks.double() * khz / 1000.0
    print(f"[clock probe] counter {khz} kHz, shader clock {mhz.min():.0f} .. {mhz.max():.0f} MHz")
    assert bool((mhz > 50).all()) and bool((mhz < 5000).all())
    assert bool((xcd >= 0).all()) and bool((xcd < 8).all())
    assert len(set(xcd.tolist())) == 8  # 256 one-wave workgroups reach every XCD


def test_stream_probe_reads_without_writing():
    dev = torch.device("cuda:0")
    buf = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for mode in (0, 1, 2):
        for wgs in (1, 256, 1024):
            kvq.prepare_stream_probe(buf, mode, wgs, sink)()
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
