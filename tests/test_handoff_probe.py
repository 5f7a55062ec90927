"""The hand-off latency probe (kie_handoff_probe).

Host side (no GPU): every argument error the call rejects before it touches
the device.  GPU: a ping and an all-to-all round complete, idle and beside
streaming, with times and die ids in range; size errors are reported.
"""
import ctypes

import pytest
import torch

from persistent_decode_monokernel_amd import kie

DEV = "cuda:0"
FAKE = 0x10000  # 8- and 16-byte aligned; never dereferenced by the rejected calls


def _call(kind=kie.KIE_PROBE_PING, a=0, b=1, rounds=10, stride=1, depth=3, where=kie.KIE_PROBE_STREAM_NONE,
          buf=FAKE, nbytes=1 << 30, scratch=FAKE, sbytes=kie.KIE_HANDOFF_PROBE_SCRATCH_BYTES, out=True):
    r = kie.kie_handoff_probe_result()
    return kie.lib().kie_handoff_probe(kind, a, b, rounds, stride, depth, where, ctypes.c_void_p(buf), nbytes,
                                       ctypes.c_void_p(scratch), sbytes, None,
                                       ctypes.byref(r) if out else None)


@pytest.mark.parametrize("kw", [
    {"out": False},
    {"scratch": 0},
    {"scratch": FAKE + 4},
    {"kind": 2},
    {"kind": -1},
    {"rounds": 0},
    {"rounds": 100001},
    {"stride": 0},
    {"stride": 3},
    {"stride": 32},
    {"where": 4},
    {"where": -1},
    {"kind": kie.KIE_PROBE_ALL_TO_ALL, "where": kie.KIE_PROBE_STREAM_OTHERS},
    {"where": kie.KIE_PROBE_STREAM_OWN, "depth": 5},
    {"where": kie.KIE_PROBE_STREAM_OWN, "depth": 0},
    {"where": kie.KIE_PROBE_STREAM_OTHERS, "buf": 0},
    {"where": kie.KIE_PROBE_STREAM_OTHERS, "buf": FAKE + 8},
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_argument_errors_before_any_device_call(kw):
    assert _call(**kw) == kie.KIE_ERR_ARG


@pytest.fixture(scope="module")
def bufs():
    buf = torch.ones(1 << 29, dtype=torch.float16, device=DEV)  # 1 GiB
    scratch = torch.zeros(kie.KIE_HANDOFF_PROBE_SCRATCH_BYTES // 8, dtype=torch.int64, device=DEV)
    yield buf, scratch
    del buf, scratch
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_ping_idle_and_beside_streaming(bufs):
    buf, scratch = bufs
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    idle = kie.handoff_probe(kie.KIE_PROBE_PING, rounds=100, wg_a=0, wg_b=1, scratch=scratch)
    print(f"ping idle: {idle.exchange_us:.3f} us, XCDs {idle.xcc_a} {idle.xcc_b}", flush=True)
    assert idle.completed == 1 and idle.grid == min(cus, 1024)
    assert 0.05 < idle.exchange_us < 100
    assert 0 <= idle.xcc_a < 8 and 0 <= idle.xcc_b < 8
    for where in (kie.KIE_PROBE_STREAM_OTHERS, kie.KIE_PROBE_STREAM_OWN,
                  kie.KIE_PROBE_STREAM_OTHERS | kie.KIE_PROBE_STREAM_OWN):
        r = kie.handoff_probe(kie.KIE_PROBE_PING, rounds=100, wg_a=0, wg_b=idle.grid - 1, where=where, depth=3,
                              buf=buf, scratch=scratch)
        print(f"ping, streaming {where}: {r.exchange_us:.3f} us, {r.stream_gbps:.0f} GB/s", flush=True)
        assert r.completed == 1 and 0.05 < r.exchange_us < 1000 and r.stream_gbps > 10


@pytest.mark.gpu
def test_all_to_all_idle_and_beside_streaming(bufs):
    buf, scratch = bufs
    for stride in (1, 2, 16):
        idle = kie.handoff_probe(kie.KIE_PROBE_ALL_TO_ALL, rounds=50, scratch=scratch, stride=stride)
        print(f"all-to-all idle, slot stride {stride}: {idle.exchange_us:.3f} us "
              f"(slowest {idle.exchange_max_us:.3f})", flush=True)
        assert idle.completed == 1 and 0.05 < idle.exchange_us <= idle.exchange_max_us < 1000
    r = kie.handoff_probe(kie.KIE_PROBE_ALL_TO_ALL, rounds=50, where=kie.KIE_PROBE_STREAM_OWN, depth=8,
                          buf=buf, scratch=scratch)
    print(f"all-to-all, own waves stream: {r.exchange_us:.3f} us, {r.stream_gbps:.0f} GB/s", flush=True)
    assert r.completed == 1 and r.exchange_us <= r.exchange_max_us and r.stream_gbps > 10


@pytest.mark.gpu
def test_size_and_range_errors(bufs):
    buf, scratch = bufs
    grid = kie.handoff_probe(kie.KIE_PROBE_PING, rounds=5, scratch=scratch).grid
    with pytest.raises(kie.KieError) as e:
        kie.handoff_probe(kie.KIE_PROBE_PING, rounds=5, wg_a=3, wg_b=3, scratch=scratch)
    assert e.value.status == kie.KIE_ERR_ARG
    with pytest.raises(kie.KieError) as e:
        kie.handoff_probe(kie.KIE_PROBE_PING, rounds=5, wg_a=0, wg_b=grid, scratch=scratch)
    assert e.value.status == kie.KIE_ERR_ARG
    with pytest.raises(kie.KieError) as e:  # a share below one chunk per work-group
        kie.handoff_probe(kie.KIE_PROBE_PING, rounds=5, where=kie.KIE_PROBE_STREAM_OTHERS, depth=3,
                          buf=buf[: 1 << 20], scratch=scratch)
    assert e.value.status == kie.KIE_ERR_CAPACITY
    with pytest.raises(kie.KieError) as e:
        kie.handoff_probe(kie.KIE_PROBE_PING, rounds=5, scratch=scratch[:16])
    assert e.value.status == kie.KIE_ERR_CAPACITY
