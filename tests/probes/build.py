"""Build the test probes under tests/probes (hipcc, gfx950) next to their sources."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from sparse_attention_indexer_quant_amd import build as lib_build  # noqa: E402

LIBRARY = os.path.join(HERE, "libmfma_probe.so")


def build() -> str:
    src = os.path.join(HERE, "mfma_precision.hip")
    tmp = LIBRARY + ".tmp"
    cmd = [lib_build.hipcc()] + lib_build.common_flags() + ["-shared", "-o", tmp, src]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{proc.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
