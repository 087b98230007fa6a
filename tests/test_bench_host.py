"""Host-side pieces of bench.py: the committed counter summaries are read back by the same key
the summariser writes, and only while the kernel source they were taken on is unchanged."""
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_summaries_are_read_back(monkeypatch):
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "decode_*_traffic.json")))
    assert files, "no committed counter summary"
    for path in files:
        d = json.load(open(path))
        wl = os.path.basename(path)[len("decode_"):-len("_traffic.json")]
        key = "decode_sources_sha256_16"
        assert key in d and d["bytes_per_launch"] > 0
        monkeypatch.setattr(bench, "decode_source_hash", lambda: d[key])
        assert bench.counter_traffic(wl) == d["bytes_per_launch"]
        monkeypatch.setattr(bench, "decode_source_hash", lambda: "0" * 16)
        assert bench.counter_traffic(wl) is None


def test_settle_stops_on_agreeing_windows(monkeypatch):
    # two consecutive windows within 2% end the settle phase after at least three windows
    times = iter([9.0, 5.0, 4.0, 3.96, 1.0, 1.0])

    class Ev:
        def __init__(self, **_):
            pass

        def record(self):
            pass

        def elapsed_time(self, other):
            return next(times)

    class FakeCuda:
        Event = Ev

        @staticmethod
        def synchronize():
            pass

    import torch
    monkeypatch.setattr(torch, "cuda", FakeCuda)
    monkeypatch.setattr(bench, "attention_only", lambda st, q: None)
    assert bench.settle(None, None, window=10) == 40


def test_summarize_pmc_means_per_dispatch(tmp_path):
    # two dispatches of decode_kernel (counter summed over its two dimensions), one of another kernel
    d = tmp_path / "pmc_x"
    d.mkdir()
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value",
            "1,kvq::decode_kernel<8>,SQ_WAVES,100", "1,kvq::decode_kernel<8>,SQ_WAVES,20",
            "2,kvq::decode_kernel<8>,SQ_WAVES,60", "3,kvq::combine_kernel,SQ_WAVES,7"]
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    assert bench.summarize_pmc([str(d)]) == "pmc_x: SQ_WAVES=90 (dispatches 2)\n"
