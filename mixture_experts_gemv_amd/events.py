"""HIP events through ctypes, for moe_forward_timed and stream-level timing.

torch.cuda.Event does not expose its hipEvent_t handle, which the C ABI's
timed entry point takes; these are plain handles from libamdhip64."""

from __future__ import annotations

import ctypes


class HipEvents:
    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                self.close()
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(e.value)

    def record(self, i: int, stream: int) -> None:
        rc = self.hip.hipEventRecord(self.ev[i], stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []
