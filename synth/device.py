"""Device twin of the host generator: fills GPU buffers with the same bf16 K/V values.

Loads synth/libloopvq_synth.so (built by synth/build_device.py).  torch supplies
device memory and the stream.  Input generation only.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import gen
from .workloads import Workload

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopvq_synth.so")


class synth_kv_args(ctypes.Structure):
    _fields_ = [("key", ctypes.c_uint64), ("table", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("inv_sqrt_d", ctypes.c_double), ("rho", ctypes.c_double),
                ("innov", ctypes.c_double), ("T4", ctypes.c_int32), ("L", ctypes.c_int32), ("B", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("n_ctx", ctypes.c_int32), ("d", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("b0", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("h0", ctypes.c_int32), ("nh", ctypes.c_int32), ("n0", ctypes.c_int32), ("nn", ctypes.c_int32),
                ("t0", ctypes.c_int32), ("nt", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("s_loop", ctypes.c_int64), ("s_b", ctypes.c_int64), ("s_h", ctypes.c_int64),
                ("s_n", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run synth/build_device.py")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_kv.argtypes = [ctypes.POINTER(synth_kv_args), ctypes.c_void_p]
        L.synth_kv.restype = ctypes.c_int
        _lib = L
    return _lib


class DeviceGen:
    """Holds the device-side tables of one workload (normal quantiles, scales, rotation signs)."""

    def __init__(self, wl: Workload, device="cuda"):
        import torch
        self.wl = wl
        self.table = torch.from_numpy(np.array(gen.normal_table(), copy=True)).to(device)
        self.scales_np = gen.scales(wl)
        self.scales = torch.from_numpy(np.ascontiguousarray(self.scales_np)).to(device)
        self.signs = (torch.from_numpy(gen.rotation_signs(wl)).to(device) if wl.rotate_keys else None)
        self.key = int(gen.stream_key(wl, gen.S_DATA))

    def kv(self, out, *, kind, layer, b0, nb, h0, nh, n0, nn, t0, nt, s_loop, s_b, s_h, s_n, stream=None):
        """Write cache values of (sequences b0.., heads h0.., tokens n0.., loops t0..) into `out`.

        out[(t - t0)*s_loop + (b - b0)*s_b + (h - h0)*s_h + (n - n0)*s_n + ch] (bf16 bits).
        """
        import torch
        wl = self.wl
        a = synth_kv_args(key=self.key, table=self.table.data_ptr(), scales=self.scales.data_ptr(),
                          signs=self.signs.data_ptr() if self.signs is not None else None,
                          inv_sqrt_d=gen.inv_sqrt_d(wl), rho=gen.AR_RHO, innov=gen.AR_INNOV,
                          T4=gen.loops_padded(wl.loops), L=wl.layers, B=wl.batch, Hkv=wl.kv_heads,
                          n_ctx=wl.context, d=wl.head_dim, kind=kind, layer=layer, b0=b0, nb=nb, h0=h0, nh=nh,
                          n0=n0, nn=nn, t0=t0, nt=nt, out=out.data_ptr(), s_loop=s_loop, s_b=s_b, s_h=s_h, s_n=s_n)
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        rc = _load().synth_kv(ctypes.byref(a), st)
        if rc != 0:
            raise RuntimeError(f"synth_kv failed ({rc})")
