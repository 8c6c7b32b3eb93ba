"""bench.py's readers of the profiles/ summaries (host only): a summary counts
only when it was taken on the current kernel source, and the MFMA-busy
fraction is the counted busy cycles over 1024 SIMDs x 2.4 GHz x the kernel time."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _write(tmp_path, sha, extra):
    p = tmp_path / "summary.txt"
    p.write_text("# comment: ignored\nkernel_source_sha256_16: %s\n%s" % (sha, extra))
    return str(p)


SQ = ("mfma_busy_cycles_per_launch: 1.2288e+10\nmfma_busy_frac_of_busy_cycles: 0.5\n"
      "mfma_insts_per_wave_block: 12.0\nvalu_insts_per_wave_block: 64.0\nwave_blocks_per_launch: 1000\n")


def test_stale_summary_is_ignored(tmp_path):
    p = _write(tmp_path, "0000000000000000", "hbm_bytes_per_launch: 1e9\n" + SQ)
    assert bench.read_traffic(p) is None
    assert bench.mfma_busy(10.0, p) is None


def test_missing_summary_is_none(tmp_path):
    assert bench.read_summary(str(tmp_path / "absent.txt")) is None
    assert bench.mfma_busy(10.0, str(tmp_path / "absent.txt")) is None


def test_current_summary_is_read(tmp_path):
    p = _write(tmp_path, bench.source_hash(), "hbm_bytes_per_launch: 2.5e9   (note)\n" + SQ)
    assert bench.read_traffic(p) == 2.5e9
    mb = bench.mfma_busy(10.0, p)
    # 1.2288e10 busy cycles over 1024 SIMDs x 2.4e9 Hz x 10 ms = 0.5
    assert mb["frac"] == pytest.approx(1.2288e10 / (1024 * 2.4e9 * 10e-3))
    assert mb["frac"] == pytest.approx(0.5)
    assert mb["wave_blocks_per_launch"] == 1000


def test_committed_summaries_parse():
    """Every summary under profiles/ with a source hash has the keys bench.py reads."""
    for name in os.listdir(os.path.join(bench.ROOT, "profiles")):
        path = os.path.join(bench.ROOT, "profiles", name)
        with open(path) as f:
            text = f.read()
        if "kernel_source_sha256_16:" not in text:
            continue
        if name.endswith("_sq_counters.txt"):
            assert "mfma_busy_cycles_per_launch:" in text and "wave_blocks_per_launch:" in text
        else:
            assert "hbm_bytes_per_launch:" in text
