"""Hash of the sources the HIP library is built from.

``build.py`` compiles this hash into the library and the binding compares it
with the hash of the sources next to the library when it loads, so a library
built from other sources is refused instead of silently tested.  Plain
Python with no imports from the package (both load it by path)."""

import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def source_files():
    csrc = os.path.join(HERE, "csrc")
    names = sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp", ".cpp", ".h")))
    return ([os.path.join(csrc, n) for n in names]
            + [os.path.join(ROOT, "include", "nvfp4.h"), os.path.join(HERE, "build.py")])


def source_hash():
    """sha256 over the names and bytes of every source, in a fixed order."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()
