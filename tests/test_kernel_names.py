"""Every kernel the host side of libhda.so launches exists, under the same
mangled name, in the gfx950 code objects embedded in it (CPU only).

The host and device compilations of a HIP source each mangle a kernel's
name; a template argument of an unnamed type (an anonymous enum, a lambda)
gets a compiler-made name that can differ between the two, and the runtime
then finds no device function for the host's handle and aborts at the first
launch.  This reads the host's kernel handles from the library's symbol
table and the device kernels (their .kd descriptors) from the offload
bundles in its .hip_fatbin section, and compares the two sets; likewise the
device array hda_decode_noalloc finds through its host stand-in.
"""

import os
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "load_balanced_split_step_amd", "libhda.so")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _nm(path):
    out = subprocess.run(["nm", path], capture_output=True, text=True, check=True).stdout
    return [line.split()[-1] for line in out.splitlines() if line.split()]


def _device_symbols(fatbin, tmp):
    """(kernel names, all symbol names) of the gfx950 code objects."""
    names, syms = set(), set()
    for start in range(0, len(fatbin), 8):
        if not fatbin.startswith(MAGIC, start):
            continue
        p = start + len(MAGIC)
        (n,) = struct.unpack_from("<Q", fatbin, p)
        p += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            p += 24
            triple = fatbin[p:p + tlen].decode()
            p += tlen
            if "gfx950" in triple:
                co = os.path.join(tmp, f"co_{start}.o")
                with open(co, "wb") as f:
                    f.write(fatbin[start + off:start + off + size])
                all_syms = _nm(co)
                names |= {s[:-3] for s in all_syms if s.endswith(".kd")}
                syms |= set(all_syms)
    return names, syms


@pytest.mark.skipif(not (shutil.which("nm") and shutil.which("objcopy")),
                    reason="binutils nm / objcopy not available")
def test_host_kernel_handles_have_device_kernels():
    if not os.path.exists(LIB):
        pytest.skip("libhda.so is not built")
    with tempfile.TemporaryDirectory() as tmp:
        fb = os.path.join(tmp, "fatbin.bin")
        subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fb}", LIB, os.path.join(tmp, "x")],
                       check=True, capture_output=True)
        with open(fb, "rb") as f:
            dev, dev_syms = _device_symbols(f.read(), tmp)
    host_syms = _nm(LIB)
    host = {s for s in host_syms if s.startswith("_Z") and "_kernel" in s and "__device_stub__" not in s}
    # the device array hda_decode_noalloc looks up by its host stand-in
    scratch = [s for s in host_syms if s.endswith("7scratchE")]
    assert len(scratch) == 1 and scratch[0] in dev_syms, scratch
    assert dev, "no gfx950 kernels found in the library"
    assert host, "no kernel handles found in the library"
    missing = sorted(host - dev)
    assert not missing, f"{len(missing)} host kernel handles without a device kernel: {missing[:3]}"
