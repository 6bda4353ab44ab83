"""bench.py's command line on the CPU: it runs on one GPU only and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr, r.stderr
    assert not r.stdout.strip().startswith("{")


def test_kernel_source_hash_covers_every_kernel_source():
    """Every HIP source and header of the library enters kernel_source_hash,
    so a profile can never outlive a change to any kernel."""
    import glob
    import os
    import bench
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "long_sequence_block_amd", "csrc")
    on_disk = {os.path.basename(p) for p in glob.glob(os.path.join(csrc, "*.hip")) +
               glob.glob(os.path.join(csrc, "*.h"))}
    assert set(bench.KERNEL_SOURCES) == on_disk
