"""Identity of the compiled kernels: a hash of the kernel sources and build
flags.  Counter measurements (profiles/traffic.json) record it, and the
benchmark only reports traffic measured on kernels with the same hash."""
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(HERE, "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]
