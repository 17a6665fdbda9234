"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte accounting
of the step, and the rule that counter-measured HBM traffic is reported only for the
kernel source it was measured on."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_step_bytes_follow_the_formats():
    # bf16 is 2 bytes; a code is half a byte; an E4M3 scale is one byte per 16 elements
    assert bench.BYTES_PER_ELEM["amax"] == 2
    assert bench.BYTES_PER_ELEM["fake_quant"] == 2 + 2
    assert bench.BYTES_PER_ELEM["quantize_pack"] == 2 + 0.5 + 1 / 16
    assert bench.BYTES_PER_ELEM["dequant_unpack"] == 0.5 + 1 / 16 + 2
    # the step: amax + fake-quant, amax + quantize-pack, dequant-unpack
    assert bench.STEP_BYTES_PER_ELEM == 13.125


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    csrc = tmp_path / "fp4_block_fake_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("kernel a\n")
    (csrc / "b.hpp").write_text("header b\n")
    (csrc / "notes.txt").write_text("not a source\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def write_traffic(root, src_hash, hbm="12345"):
    (root / "profiles" / "traffic_k_x_w.txt").write_text(
        "# comment: ignored\nsource_sha256_16: %s\nbytes_past_l2_per_launch: %s\n" % (src_hash, hbm))


def test_source_hash_covers_every_kernel_source(fake_root):
    h0 = bench.kernel_source_hash()
    (fake_root / "fp4_block_fake_amd" / "csrc" / "notes.txt").write_text("changed\n")
    assert bench.kernel_source_hash() == h0
    (fake_root / "fp4_block_fake_amd" / "csrc" / "b.hpp").write_text("header b, changed\n")
    h1 = bench.kernel_source_hash()
    assert h1 != h0
    os.rename(fake_root / "fp4_block_fake_amd" / "csrc" / "b.hpp", fake_root / "fp4_block_fake_amd" / "csrc" / "c.hpp")
    assert bench.kernel_source_hash() != h1


def test_source_hash_follows_code_not_comments(fake_root):
    src = fake_root / "fp4_block_fake_amd" / "csrc" / "a.hip"
    src.write_text("int k(int a) {\n    return a + 1;   // one more\n}\n")
    h0 = bench.kernel_source_hash()
    src.write_text("/* the kernel */\nint k(int a) {\n\n  return a + 1;   // one more than a\n}\n")
    assert bench.kernel_source_hash() == h0                       # comments and spacing only
    src.write_text("int k(int a) {\n    return a + 2;   // one more\n}\n")
    assert bench.kernel_source_hash() != h0                       # the code changed


def test_traffic_only_for_the_source_it_was_measured_on(fake_root):
    assert bench.read_traffic("k_x", "w") is None                 # never measured
    write_traffic(fake_root, bench.kernel_source_hash())
    assert bench.read_traffic("k_x", "w") == 12345.0
    (fake_root / "fp4_block_fake_amd" / "csrc" / "a.hip").write_text("kernel a, changed\n")
    assert bench.read_traffic("k_x", "w") is None                 # the kernel changed since
    write_traffic(fake_root, bench.kernel_source_hash(), hbm="n/a")
    assert bench.read_traffic("k_x", "w") is None                 # unreadable figure



def test_oracle_runner_threads_give_the_single_threaded_bytes():
    """The CPU-baseline runner shards rows over threads; amax and codes must not change."""
    import numpy as np

    import synth
    x = synth.c5_weight(rows=40)
    one, four = bench.OracleRunner(1), bench.OracleRunner(4)
    assert one.amax(x) == four.amax(x)
    a = one.amax(x)
    p1, p4 = one.quantize(x, a), four.quantize(x, a)
    assert len(p1) == 1 and len(p4) == 4
    assert np.array_equal(p1[0][0], np.concatenate([p[0] for p in p4]))
    assert np.array_equal(p1[0][1], np.concatenate([p[1] for p in p4]))
    sibs = [s[:32] for s in synth.c3_siblings()]
    assert one.amax(*sibs) == four.amax(*sibs)


def test_host_info_names_the_cpus():
    info = bench.host_info()
    assert info["nproc"] >= 1 and info["usable_cpus"] >= 1
