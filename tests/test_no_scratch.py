"""No kernel of libqc uses scratch (private) memory.

Kernels that need more registers than a lane has spill to scratch memory;
spilled builds of the 65,536-element encoders gave results on the GPU that
differ from what their source computes (the same source, run on the CPU,
matched the oracle bit for bit), so the library is laid out to keep every
kernel inside the register file.  This test reads the kernel descriptors of
the gfx950 code objects inside the built libqc.so (this repository's own
build) and checks every kernel's private segment size is zero."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "embedding_communication_codecs_amd", "libqc.so")
LLVM = "/opt/rocm/llvm/bin"


def kernel_private_sizes(lib_path):
    """{kernel symbol: private segment bytes} over the library's gfx950 code objects."""
    out = {}
    d = tempfile.mkdtemp()
    try:
        copy = os.path.join(d, "lib.so")
        shutil.copy(lib_path, copy)
        subprocess.run([os.path.join(LLVM, "llvm-objdump"), "--offloading", copy], check=True, capture_output=True,
                       cwd=d)
        for f in sorted(os.listdir(d)):
            if "amdgcn" not in f or "gfx950" not in f:
                continue
            notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", os.path.join(d, f)], check=True,
                                   capture_output=True, text=True).stdout
            # each kernel's metadata map lists .name and .private_segment_fixed_size
            for block in re.split(r"\n\s+- \.", notes):
                name = re.search(r"\.name:\s+(\S+)", block)
                priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
                if name and priv:
                    out[name.group(1)] = int(priv.group(1))
    finally:
        shutil.rmtree(d)
    return out


@pytest.mark.skipif(not os.path.exists(LIB), reason="libqc.so is not built")
@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "llvm-readelf")), reason="ROCm LLVM tools not found")
def test_no_kernel_uses_scratch_memory():
    sizes = kernel_private_sizes(LIB)
    assert len(sizes) > 200, f"found only {len(sizes)} kernels"
    spilled = {k: v for k, v in sizes.items() if v != 0}
    assert not spilled, f"{len(spilled)} kernels use scratch memory, e.g. {sorted(spilled.items())[:5]}"
