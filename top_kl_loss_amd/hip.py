"""Minimal ctypes access to the HIP runtime of the process.

The binding loads libkdtopk.so after torch, so the library, torch and this
module all use the one runtime torch loaded (soname libamdhip64.so.7).  The
benchmark uses it for what torch does not expose: events recorded by the
library's launch log around single kernel launches, device attributes and
hipMemGetInfo.
"""
from __future__ import annotations

import ctypes

_hip = None


def runtime():
    """The HIP runtime of the process (the one torch and libkdtopk.so use)."""
    global _hip
    if _hip is not None:
        return _hip
    from . import load_library
    load_library()  # loads torch's runtime first, then the library
    h = ctypes.CDLL("libamdhip64.so.7")
    vp = ctypes.c_void_p
    h.hipDeviceSynchronize.restype = ctypes.c_int
    h.hipSetDevice.argtypes = [ctypes.c_int]
    h.hipStreamSynchronize.argtypes = [vp]
    h.hipStreamCreate.argtypes = [ctypes.POINTER(vp)]
    h.hipStreamDestroy.argtypes = [vp]
    h.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
    h.hipEventRecord.argtypes = [vp, vp]
    h.hipEventSynchronize.argtypes = [vp]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
    h.hipEventDestroy.argtypes = [vp]
    h.hipGetErrorString.argtypes = [ctypes.c_int]
    h.hipGetErrorString.restype = ctypes.c_char_p
    h.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    h.hipMemGetInfo.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    _hip = h
    return h


def check(err):
    if err != 0:
        msg = runtime().hipGetErrorString(err).decode()
        raise RuntimeError(f"HIP error {err}: {msg}")


# hipDeviceAttribute_t values of the runtime's header
ATTR_CLOCK_RATE_KHZ = 5        # hipDeviceAttributeClockRate
ATTR_MULTIPROCESSOR_COUNT = 63  # hipDeviceAttributeMultiprocessorCount


def device_attribute(attr: int, device: int = 0) -> int:
    v = ctypes.c_int(0)
    check(runtime().hipDeviceGetAttribute(ctypes.byref(v), int(attr), int(device)))
    return v.value


def mem_get_info():
    """(free, total) bytes of the current device."""
    free, total = ctypes.c_size_t(0), ctypes.c_size_t(0)
    check(runtime().hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)))
    return free.value, total.value


def set_device(index: int):
    check(runtime().hipSetDevice(int(index)))


def synchronize(stream=None):
    """Wait for `stream` (a raw handle; None: the whole device)."""
    if stream is None:
        check(runtime().hipDeviceSynchronize())
    else:
        check(runtime().hipStreamSynchronize(stream))


class Stream:
    """A default-priority stream created through the runtime (raw handle in
    ``value``; torch.cuda.ExternalStream can wrap it)."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        check(runtime().hipStreamCreate(ctypes.byref(self.handle)))

    @property
    def value(self):
        return self.handle.value

    def synchronize(self):
        synchronize(self.handle)

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipStreamDestroy(self.handle)


class Event:
    """A timing event (raw handle in ``value``), for the launch log."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        check(runtime().hipEventCreate(ctypes.byref(self.handle)))

    @property
    def value(self):
        return self.handle.value

    def record(self, stream=None):
        check(runtime().hipEventRecord(self.handle, stream))

    def synchronize(self):
        check(runtime().hipEventSynchronize(self.handle))

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float(0.0)
        check(runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle,
                                            end.handle))
        return ms.value

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)
