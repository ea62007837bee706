"""Host-only checks of the build and measurement bookkeeping.

* every translation unit under level_dsl_amd/csrc is in the build list, so
  no kernel family is left out of libmxgemm.so;
* every kernel and launch source is in bench.py's source hash, so a change
  to any of them makes the committed HBM-traffic figures read as stale
  (bench.py then reports `traffic` as null) instead of silently reused.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from level_dsl_amd import build  # noqa: E402

CSRC = os.path.join(ROOT, "level_dsl_amd", "csrc")


def test_every_translation_unit_is_built():
    units = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    assert sorted(build.SRCS) == units


def test_traffic_hash_covers_every_kernel_source():
    import bench
    srcs = sorted("level_dsl_amd/csrc/" + f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    assert sorted(bench.KERNEL_SOURCES) == srcs


def test_traffic_hash_is_well_formed():
    import bench
    h = bench.kernel_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
