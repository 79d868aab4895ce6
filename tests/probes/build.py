"""Build the layout-probe library the GPU primitive tests load.

The probes (``probe.hip``) are two one-wave kernels that record the
matrix-core fragment layouts and the DPP row shift the library's kernels are
written against.  They are test code: they are compiled here, beside the
tests, into ``tests/probes/libtq_probe.so``, never into ``libtq.so``.
``__graft_entry__.build()`` calls ``build()`` so that the library exists
before any GPU run.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libtq_probe.so")

if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def build():
    from kv_cache_vector_quantize_amd import build as pkg_build
    tmp = LIB + ".tmp"
    cmd = [pkg_build.HIPCC, *pkg_build.COMMON_FLAGS, "-shared", os.path.join(HERE, "probe.hip"),
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probe.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
