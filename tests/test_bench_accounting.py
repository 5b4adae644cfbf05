"""bench.py's algorithmic byte accounting and its one-GPU contract, on the CPU.

Every GB/s figure and roofline fraction that bench.py reports divides these
byte counts by a measured time, so they are pinned here against values worked
out by hand from the byte formulas (the state read and written once in fp32,
each input and output of the step moved once at its I/O width):

  large-batch decode (B=256, T=1, Hk=16, Hv=32, Dk=Dv=128, bf16, a mask):
      record 8*256*32*128*128 + 4*256 + 256*2*(2*16*128 + 3*32*128 + 2*32)
           = 1073741824 + 1024 + 8421376 = 1082164224
      replay (one accepted position)
           = 1073741824 + 4*256 + 256*2*32*(128 + 128 + 1) = 1077953536
  4096-step prefill (B=1, Hk=16, Hv=32, Dk=Dv=128, bf16, no mask):
      record 8*32*128*128 + 4096*2*16448 = 138936320
      GQA expansion of q or k in fp32: 4*4096*128*(16 + 32) = 100663296
  RMSNorm of 4096 x 2048 fp32 tokens with a bf16 weight: 8*4096*2048 + 2*2048 = 67112960
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (module level: only definitions, no GPU work)


def test_large_batch_decode_record_and_replay_bytes():
    assert bench.record_bytes(256, 1, 16, 32, 128, 128, 2, 256, True) == 1082164224
    assert bench.replay_bytes(256, 1, 32, 128, 128, 2, 1, 256, True) == 1077953536


def test_prefill_record_and_expand_bytes():
    assert bench.record_bytes(1, 4096, 16, 32, 128, 128, 2, 4096, False) == 138936320
    assert bench.expand_bytes(4096, 16, 32, 128, 4) == 100663296


def test_rms_norm_and_capture_bytes():
    assert bench.rms_norm_bytes(4096, 2048) == 67112960
    # the fused capture writes, per active step, the keys of every value head and the gates
    assert bench.capture_bytes(32, 128, 2, 256) == 256 * 2 * 32 * 129


def test_masked_steps_move_no_step_bytes():
    """Inactive steps move no step inputs or outputs: only the state and the mask words."""
    full = bench.record_bytes(2, 8, 1, 2, 32, 16, 2, 16, True)
    none = bench.record_bytes(2, 8, 1, 2, 32, 16, 2, 0, True)
    assert none == 8 * 2 * 2 * 16 * 32 + 4 * 2 * 8
    assert full - none == 16 * 2 * (2 * 32 + 3 * 2 * 16 + 2 * 2)
    # a replay reads the mask only up to the accepted count
    assert bench.replay_bytes(2, 8, 2, 32, 16, 2, 3, 0, True) == 8 * 2 * 2 * 16 * 32 + 4 * 2 * 3
    assert bench.replay_bytes(2, 8, 2, 32, 16, 2, 99, 0, True) == 8 * 2 * 2 * 16 * 32 + 4 * 2 * 8


def test_every_timed_kernel_has_its_sources():
    for kernel in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(kernel)) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("p,expect", [(0, 1.0), (50, 3.0), (100, 5.0)])
def test_percentile_helper(p, expect):
    assert bench._pct([5.0, 1.0, 3.0, 2.0, 4.0], p) == expect
