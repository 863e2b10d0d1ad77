import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive host checks that take tens of seconds")


@pytest.fixture(scope="session")
def ora():
    import oracle

    oracle.lib()
    return oracle


# Library pin for the Philox4x32-10 generator: the rocRAND header's host-side
# engine.  engine(seed, subsequence, offset) produces the block at counter
# (offset/4, subsequence) with key = seed.
ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


@pytest.fixture(scope="session")
def rocrand_philox():
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(hdr) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ not available")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "p.cpp"), os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(ROCRAND_PROBE)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    src, "-o", exe], check=True, capture_output=True)

    def run(cases):
        inp = "".join(f"{s} {sub} {off}\n" for s, sub, off in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]

    yield run
    shutil.rmtree(d)


