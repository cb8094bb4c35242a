"""Build the HIP library once per test session if it is not there yet (the
build itself is a cross-compile and needs no GPU)."""
import os
import threading

_lock = threading.Lock()


def ensure_built():
    from paged_mla_decode_02_amd import LIB_PATH
    with _lock:
        if not os.path.exists(LIB_PATH):
            from paged_mla_decode_02_amd.build import build
            build()
    return LIB_PATH
