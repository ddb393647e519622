"""Identity of the compiled kernels: a hash of the device sources (the .hip
files and the headers they include) and the build flags.  Counter
measurements (profiles/traffic.json) record it with the configuration name,
and the benchmark only reports traffic measured on the same kernel with the
same hash.  Host-only sources (.cpp: argument checks, the planner) do not
change a kernel and are left out."""
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_src_hash(pkg_dir: str = HERE) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(pkg_dir, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".cpp"):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(pkg_dir, "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]
