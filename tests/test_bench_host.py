"""Host-side logic of bench.py (CPU only, no GPU call).

* more than one GPU is refused with a message and exit status 2;
* a committed memory-counter summary is used for roofline.traffic only when it
  names the dominant kernel and was taken on the current kernel sources;
* the source digest covers every kernel source file;
* the projection tile width used for the memory-bound passes' byte counts is
  the kernels' own;
* the profiled clock of the dominant kernel is read only for the current
  kernel sources;
* the sampled shader clock is parsed from pp_dpm_sclk's current (starred) line.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, kernel, digest, nbytes=123456789):
    p = tmp_path / "traffic.txt"
    p.write_text("# comment: ignored\n"
                 f"source_digest: {digest}\ntraffic: {kernel} {nbytes}\ntraffic: other_kernel 42\n")
    return str(p)


def test_traffic_read_only_for_matching_kernel_and_sources(tmp_path):
    dig = bench.source_digest()
    assert bench.read_traffic(_summary(tmp_path, "bwd_dw", dig), "bwd_dw") == 123456789
    assert bench.read_traffic(_summary(tmp_path, "bwd_dw", dig), "fwd_proj") is None
    assert bench.read_traffic(_summary(tmp_path, "bwd_dw", "0" * 16), "bwd_dw") is None
    assert bench.read_traffic(str(tmp_path / "missing.txt"), "bwd_dw") is None


def test_digest_covers_kernel_sources():
    src = os.path.join(ROOT, "chunked_kl_loss_row_amd", "csrc")
    names = [n for n in os.listdir(src) if n.endswith((".hip", ".h"))]
    assert len(names) >= 5
    assert len(bench.source_digest()) == 16
    assert bench.source_digest() == bench.source_digest()


def test_projection_tile_width_matches_the_kernels():
    import re
    src = open(os.path.join(ROOT, "chunked_kl_loss_row_amd", "csrc", "kd_internal.h")).read()
    m = re.search(r"constexpr int kProjBN = (\d+);", src)
    assert m and int(m.group(1)) == bench.PROJ_TILE_V


def test_clock_read_only_for_current_sources(tmp_path):
    p = tmp_path / "sq.txt"
    dig = bench.source_digest()
    p.write_text(f"# header\nsource_digest: {dig}\n# kernel dur_ms cycles clk_GHz\n  bwd_dw 2.5 4.7e6 1.932 2.4e6\n")
    assert bench.read_clock(str(p), "bwd_dw") == 1.932
    assert bench.read_clock(str(p), "bwd_dh") is None
    p.write_text("source_digest: 0000000000000000\n  bwd_dw 2.5 4.7e6 1.932 2.4e6\n")
    assert bench.read_clock(str(p), "bwd_dw") is None


def test_sclk_parse():
    assert bench.parse_sclk("0: 500Mhz\n1: 1795Mhz *\n2: 2400Mhz\n") == 1795.0
    assert bench.parse_sclk("0: 500Mhz *\n1: 2400Mhz\n") == 500.0
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.parse_sclk("") is None
    with bench.ClockSampler() as c:   # no GPU here: no sysfs entry, or an idle reading
        pass
    assert c.summary() is None or c.summary()["samples"] >= 1
    assert c.power_summary() is None or c.power_summary()["samples"] >= 1
    assert c.temp_summary() is None or c.temp_summary()["samples"] >= 1


def test_hwmon_sampling(tmp_path):
    # a card directory laid out as the amdgpu driver does: the sampler finds
    # power1_input / power1_cap and the temperature labelled "junction"
    dev = tmp_path / "card0" / "device"
    h = dev / "hwmon" / "hwmon3"
    h.mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1734Mhz *\n2: 2400Mhz\n")
    (h / "power1_input").write_text("1398000000\n")
    (h / "power1_cap").write_text("1400000000\n")
    (h / "temp1_label").write_text("edge\n")
    (h / "temp1_input").write_text("40000\n")
    (h / "temp2_label").write_text("junction\n")
    (h / "temp2_input").write_text("81000\n")
    c = bench.ClockSampler()
    c.path = str(dev / "pp_dpm_sclk")
    c.hwmon = c._find_hwmon(c.path)
    assert c.hwmon == (str(h / "power1_input"), str(h / "power1_cap"), str(h / "temp2_input"))
    with c:
        pass
    assert c.summary()["mean"] == 1734.0
    p = c.power_summary()
    assert p["mean"] == 1398.0 and p["cap"] == 1400.0
    assert c.temp_summary()["mean"] == 81.0
