"""The HIP runtime that torch loaded, for tests that need to know where an
allocation ends (hipMemGetAddressRange)."""
import ctypes


def _runtime():
    # the copy of libamdhip64 already mapped into this process (torch's own)
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in path:
                return ctypes.CDLL(path)
    raise RuntimeError("libamdhip64 is not loaded")


def alloc_range(ptr):
    """(base, size) of the hipMalloc block that holds device address ptr."""
    L = _runtime()
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    rc = L.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(ptr))
    if rc != 0:
        raise RuntimeError("hipMemGetAddressRange failed: %d" % rc)
    return base.value, size.value
