"""Peak probes (streaming read, streaming copy, MFMA loops) that the benchmark measures the
device's achievable HBM and matrix-core rates with; a library of their own, not libdsa."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa_peaks.so")


def build() -> str:
    """hipcc for gfx950 with libdsa's device flags; always recompiles."""
    import subprocess
    from ..build import CFLAGS, hipcc
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + CFLAGS + ["-shared", os.path.join(HERE, "peaks.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for peaks.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.dsa_peak_stream_read.restype = ctypes.c_int
    L.dsa_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.dsa_peak_stream_copy.restype = ctypes.c_int
    L.dsa_peak_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.dsa_peak_mfma.restype = ctypes.c_int
    L.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L
