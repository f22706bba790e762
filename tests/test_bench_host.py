"""CPU tests of bench.py's host-side figures: the algorithmic byte counts the
roofline divides by (each a closed form over the buffers the call must
touch), the least-squares line of the rows sweep, and the rule that HBM
traffic from a counter summary is reported only while the kernel sources
match the hash the summary was taken with."""
import os

import pytest

import bench

MB = 1 << 20


def test_forward_bytes_closed_form():
    # 16384 x 4096, E4M3, gain: read x (128 MiB) and gamma (8 KiB), write
    # codes (64 MiB), scales (2 MiB) and rho (64 KiB)
    assert bench.algorithmic_bytes(16384, 4096, 0) == 128 * MB + 8192 + 64 * MB + 2 * MB + 65536
    assert bench.algorithmic_bytes(16384, 4096, 0) == 203497472
    # E2M1 packs two codes per byte; no gain, no rho
    assert bench.algorithmic_bytes(16384, 4096, 1) == 128 * MB + 8192 + 32 * MB + 2 * MB + 65536
    assert bench.algorithmic_bytes(256, 768, 0, gamma=False, with_rrms=False) == \
        256 * 768 * 2 + 256 * 768 + 256 * 24
    # the 32x-smaller scale tensor is 1/32 of the code bytes at E4M3
    r, d = 8192, 2048
    assert bench.algorithmic_bytes(r, d, 0) - bench.algorithmic_bytes(r, d, 0, with_rrms=False) \
        == 4 * r


def test_two_pass_bytes_exceed_the_fused_pass():
    # RMSNorm writes a bf16 y that the cast reads back: 4 B per element more
    for elem in (0, 1):
        fused = bench.algorithmic_bytes(16384, 4096, elem)
        assert bench.two_pass_bytes(16384, 4096, elem) - fused == 4 * 16384 * 4096
    # 7.03 against 3.03 bytes per element at E4M3
    n = 16384 * 4096
    assert abs(bench.two_pass_bytes(16384, 4096, 0) / n - 7.03) < 0.01
    assert abs(bench.algorithmic_bytes(16384, 4096, 0) / n - 3.03) < 0.01


def test_backward_bytes_closed_form():
    # read x, dy, write dx (6 B per element), read rho; the gain adds gamma
    # (bf16) and dgamma (fp32)
    assert bench.bwd_bytes(16384, 4096, gain=False) == 6 * 16384 * 4096 + 4 * 16384
    assert bench.bwd_bytes(16384, 4096) == 6 * 16384 * 4096 + 4 * 16384 + 6 * 4096


def test_fit_line_recovers_an_exact_line():
    xs = [1.0e8, 2.0e8, 4.0e8, 8.0e8]
    a, b = bench.fit_line(xs, [1.5 + x / 6.4e9 for x in xs])
    assert a == pytest.approx(1.5, rel=1e-9)
    assert b == pytest.approx(1 / 6.4e9, rel=1e-9)


def test_traffic_only_for_matching_kernel_sources(tmp_path, monkeypatch):
    summary = tmp_path / "pmc.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    assert bench.read_traffic() is None                    # no summary
    summary.write_text("kernel_source_hash: %s\nhbm_bytes_per_launch: 203877472\n"
                       % bench.kernel_hash())
    assert bench.read_traffic() == 203877472.0
    summary.write_text("kernel_source_hash: 0000000000000000\nhbm_bytes_per_launch: 1\n")
    assert bench.read_traffic() is None                    # stale: sources changed


def test_kernel_hash_covers_the_headline_sources():
    for rel in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, rel)), rel
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_hash()
