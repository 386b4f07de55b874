"""Host logic of bench.py (CPU only): the one-GPU guard, the roofline point,
the stored-traffic lookup and its source check, and the algorithmic bytes of
the timed step."""
import os
import subprocess
import sys

import pytest

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_roofline_entry_is_bytes_over_time():
    e = bench.roofline_entry("k", 8e9, 1e6)  # 8 GB in one second
    assert e["achieved"] == 8.0 and e["unit"] == "GB/s" and e["bound"] == "hbm"
    assert e["peak"] == bench.HBM_PEAK_GBS and e["frac"] == round(8.0 / bench.HBM_PEAK_GBS, 4)
    assert e["algorithmic_bytes"] == 8_000_000_000 and e["traffic"] is None and e["launches"] == 1
    e = bench.roofline_entry("k", 16_005_922_816, 5000.0, traffic=1.0)
    assert abs(e["achieved"] - 16_005_922_816 / 5e-3 / 1e9) < 0.05 and e["traffic"] == 1.0


def _traffic_file(tmp_path, sha, layout="tiled16"):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "kq_chain_kernel.w.traffic.md").write_text(
        "# summary\n\n"
        f"- source_sha256: `{sha}`\n"
        f"- weight_layout: `{layout}`\n"
        "- traffic_bytes_chain_m16: `17257130728`\n"
        "- traffic_bytes_lm_head_m1: `511644148`\n")


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    sha = bench.source_digest()
    _traffic_file(tmp_path, sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: sha)
    assert bench.stored_traffic("w", 16, "tiled16", "chain") == 17257130728.0
    assert bench.stored_traffic("w", 1, "tiled16", "lm_head") == 511644148.0
    assert bench.stored_traffic("w", 1, "tiled16", "chain") is None      # not measured
    assert bench.stored_traffic("w", 16, "rows", "chain") is None        # other layout
    assert bench.stored_traffic("other", 16, "tiled16", "chain") is None  # no summary
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.stored_traffic("w", 16, "tiled16", "chain") is None     # sources changed


def test_source_digest_covers_the_kernel_sources():
    d = bench.source_digest()
    assert len(d) == 64 and int(d, 16) >= 0
    assert d == bench.source_digest()


def test_step_algorithmic_bytes():
    """The chain's algorithmic bytes at M = 16: every stack weight once, the
    activations once per phase (4 M K bytes), the logits (4 M N per matrix)."""
    mats = synthetic.stack_matrices(synthetic.LAYERS)
    w = sum(g.weight_bytes for g in mats)
    assert w == 15_649_800_192
    phases = []
    for layer in range(synthetic.LAYERS):
        base = 7 * layer
        for idx in ((0, 1, 2), (3,), (4, 5), (6,)):
            phases.append(mats[base + idx[0]])
    m = 16
    x = sum(4 * m * g.k for g in phases)
    lg = sum(4 * m * g.n for g in mats)
    assert w + x + lg == 16_005_922_816


def test_host_cpu_model_is_named():
    name = bench.host_cpu_model()
    assert isinstance(name, str) and name and "\n" not in name
