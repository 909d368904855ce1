"""Host logic of bench.py (no GPU): the one-GPU guard, the per-launch traffic
summary from two counter runs, and the digest that ties stored counter
readings to the kernel sources."""
import csv
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_source_digest_is_stable_hex():
    d = bench.kernel_source_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", d)
    assert d == bench.kernel_source_digest()


def _counter_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_each_counter_by_the_copy(tmp_path):
    kernel = bench.ROOF["verify"][0]
    kern = f"void nl::{kernel}(nl::FwdArgs2)"
    copy = "void at::native::elementwise_kernel<MulFunctor<float>>(int, F)"
    known = bench.COPY_FLOATS * 4
    # the copy reads half its bytes on FETCH_SIZE (scale 2) and all on WRITE_SIZE (scale 1)
    _counter_csv(str(tmp_path / "f" / "run" / "p_counter_collection.csv"), "FETCH_SIZE",
                 [(kern, 100.0), (kern, 300.0), (copy, known / 2048), (copy, known / 2048 + 7), (copy, 1.0),
                  ("void other(int)", 5e6)])
    _counter_csv(str(tmp_path / "w" / "run" / "p_counter_collection.csv"), "WRITE_SIZE",
                 [(kern, 10.0), (kern, 30.0), (copy, known / 1024)])
    out = tmp_path / "traffic.txt"
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(out), kernel=kernel)
    text = out.read_text()
    # medians of the copy rows set the scales; the kernel rows are averaged
    kf = known / ((known / 2048) * 1024)
    assert re.search(r"hbm read bytes per launch: (\d+)", text).group(1) == f"{200.0 * 1024 * kf:.0f}"
    assert re.search(r"hbm write bytes per launch: (\d+)", text).group(1) == f"{20.0 * 1024:.0f}"
    assert f"kernel source digest: {bench.kernel_source_digest()}" in text
    assert "launches: 2 (fetch run), 2 (write run)" in text


def test_pmc_summary_without_kernel_rows_fails(tmp_path):
    _counter_csv(str(tmp_path / "f" / "p_counter_collection.csv"), "FETCH_SIZE", [("void other(int)", 1.0)])
    _counter_csv(str(tmp_path / "w" / "p_counter_collection.csv"), "WRITE_SIZE", [("void other(int)", 1.0)])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.txt"),
                          kernel=bench.ROOF["draft"][0])


def test_stored_traffic_only_for_the_current_sources(tmp_path):
    path = tmp_path / "traffic.txt"
    digest = bench.kernel_source_digest()
    path.write_text(f"hbm bytes per launch: 38336215\nkernel source digest: {digest}\n")
    assert bench.stored_traffic(digest, str(path)) == 38336215.0
    assert bench.stored_traffic("0" * 16, str(path)) is None
    path.write_text("hbm bytes per launch: 1\n")
    assert bench.stored_traffic(digest, str(path)) is None
    assert bench.stored_traffic(digest, str(tmp_path / "absent.txt")) is None


def test_committed_traffic_summaries_match_their_kernel_names():
    for mode, (kernel, _, _, path) in bench.ROOF.items():
        if not os.path.exists(path):
            pytest.skip(f"no counter summary for the {mode} kernel yet")
        text = open(path).read()
        assert kernel in text
        assert re.search(r"hbm bytes per launch: \d+", text)


def test_roofline_kernels_are_the_forward_instantiations():
    # the names match template instantiations the launchers make
    fwd = open(os.path.join(ROOT, "bit_nested_quantized_amd", "csrc", "nl_fwd.hip")).read()
    staged = open(os.path.join(ROOT, "bit_nested_quantized_amd", "csrc", "nl_kernels.hip")).read()
    assert "void fwd_kernel(const FwdArgs2 a)" in fwd
    assert "launch_fwd_t<BITS, 1, 12, false>" in fwd
    assert "launch_forward_mt<BITS, 1, 4>" in staged
    assert bench.ROOF["verify"][0] == "fwd_kernel<6, 1, 12, false>"
    assert bench.ROOF["draft"][0] == "forward_kernel<0, 1, 4>"


def test_pstats_percentiles():
    st = bench.pstats([float(v) for v in range(1, 101)])
    assert st["us"] == 50.5 and st["samples"] == 100
    assert abs(st["p10"] - 10.9) < 1e-9 and abs(st["p90"] - 90.1) < 1e-9


def test_util_summary_reads_each_pass(tmp_path):
    vk = f"void nl::{bench.ROOF['verify'][0]}(nl::FwdArgs2)"
    dk = f"void nl::{bench.ROOF['draft'][0]}(nl::FwdArgs)"
    _counter_csv(str(tmp_path / "a" / "p_counter_collection.csv"), "VALUBusy", [(vk, 40.0), (vk, 60.0), (dk, 20.0)])
    _counter_csv(str(tmp_path / "b" / "p_counter_collection.csv"), "SQ_WAVES", [(vk, 3072.0), (dk, 2048.0)])
    out = tmp_path / "util.txt"
    bench.util_summary([str(tmp_path / "a"), str(tmp_path / "b")], str(out))
    text = out.read_text()
    assert "VALUBusy: 50 (mean of 2 dispatches)" in text
    assert "VALUBusy: 20 (mean of 1 dispatches)" in text
    assert "SQ_WAVES: 3072" in text and "SQ_WAVES: 2048" in text
