"""The device tables' per-workgroup index layout, on the CPU.

The multi-tensor AdamW table and the gather/flatten copy tables store one
descriptor index per workgroup, XCD-major within each launch (internal.hpp,
xcd_major_index). tests/host_table_index.cpp compiles that helper with g++ and
checks, for table sizes around the launch boundaries (up to two launches), that
the entry each workgroup reads holds its own value and lies inside the index.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_partition_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_table_index_layout(tmp_path):
    exe = str(tmp_path / "table_index")
    b = subprocess.run(["g++", "-O2", "-std=c++17", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__",
                        f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
                        os.path.join(ROOT, "tests", "host_table_index.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-2000:])
