"""Host-side helpers of bench.py: the untimed pre-warm loop and the counter-based traffic figure,
which must turn null as soon as the decode sources differ from the ones the counters describe."""
import hashlib

import bench


def test_prewarm_zero_calls_nothing(monkeypatch):
    calls = []
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda: None)
    bench.prewarm(lambda: calls.append(1), 0)
    assert calls == []


def test_prewarm_runs_whole_batches_until_the_deadline(monkeypatch):
    calls, syncs = [], []
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda: syncs.append(1))
    bench.prewarm(lambda: calls.append(1), 5.0)
    assert len(syncs) >= 1 and len(calls) == 64 * len(syncs)


def _sources_sha():
    h = hashlib.sha256()
    for p in bench.DECODE_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def test_traffic_is_split_plus_merge_for_matching_sources(monkeypatch):
    m = dict(bench.MEASURED_TRAFFIC, sha256_prefix=_sources_sha())
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", m)
    want = 1024 * ((m["split"]["fetch_kib"] + m["merge"]["fetch_kib"]) * m["fetch_scale"]
                   + (m["split"]["write_kib"] + m["merge"]["write_kib"]) * m["write_scale"])
    assert bench.measured_traffic() == int(want)


def test_traffic_is_null_once_the_sources_change(monkeypatch):
    m = dict(bench.MEASURED_TRAFFIC, sha256_prefix="0" * 16)
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", m)
    assert bench.measured_traffic() is None


def test_parse_gfx_clock_mhz():
    """The amd-smi clock reading: the mean over the XCDs' gfx clocks of the first GPU, None on
    output it cannot read."""
    import json
    import bench
    def xcd(mhz):
        return {"clk": {"value": mhz, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                "max_clk": {"value": 2400, "unit": "MHz"}}
    clocks = {f"gfx_{i}": xcd(2000 + 10 * i) for i in range(8)}
    clocks["mem_0"] = xcd(1300)                      # not a gfx clock: ignored
    text = json.dumps({"gpu_data": [{"gpu": 0, "clock": clocks}]})
    assert bench.parse_gfx_clock_mhz(text) == 2035.0
    assert bench.parse_gfx_clock_mhz(json.dumps([{"gpu": 0, "clock": clocks}])) == 2035.0
    clocks["gfx_3"]["clk"]["value"] = "N/A"          # an unreadable XCD drops out
    assert bench.parse_gfx_clock_mhz(text.replace('"value": 2030', '"value": "N/A"')) == \
        (sum(2000 + 10 * i for i in range(8)) - 2030) / 7
    assert bench.parse_gfx_clock_mhz("") is None
    assert bench.parse_gfx_clock_mhz("amd-smi: error") is None
    assert bench.parse_gfx_clock_mhz(json.dumps({"gpu_data": []})) is None
