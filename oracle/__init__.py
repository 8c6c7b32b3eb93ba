"""Reference oracle for windowed-RoPE attention (ATFlash idea).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path
(``rope_frequency_windowed_amd``) never does and shares no code with it.

Two independent pieces live here:

* ``atf_oracle.c`` -- plain fp64 C loops that follow the definition step by
  step (window table, RoPE rotation, per-pair windowed score, two-pass softmax,
  weighted sum of values, skipped-term count).  Wrapped by :func:`attention`,
  :func:`window_table` and :func:`skipped_closed_form`.
* ``dense_ref.py`` -- the textbook dense RoPE softmax attention in NumPy fp64,
  used to pin the oracle's special cases (alpha = inf, short sequences, ...).

Source page for the method: "ATFlash: RoPE-Frequenzen kuerzen
Attention-Arbeit um bis zu 57 Prozent" (sudo-ai.de), section "Was ATFlash
anders macht" (per-pair windows proportional to the wavelength, slow pairs keep
distant keys reachable) and section "Die Zahlen - und ihre Grenze" (online
softmax unchanged).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "atf_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
W_INF = np.iinfo(np.int64).max
LAYOUTS = {"neox": 0, "gptj": 1}

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle (gcc, fp64, no FMA contraction) into ``out``."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.orc_window_table.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, i64p]
    lib.orc_window_table.restype = ctypes.c_int
    lib.orc_attention_rows.argtypes = [
        f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, i64p, ctypes.c_int64, f32p, f64p, u64p]
    lib.orc_attention_rows.restype = ctypes.c_int
    lib.orc_skipped_closed_form.argtypes = [
        ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int, u64p]
    lib.orc_skipped_closed_form.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB_PATH)
    return _lib


class Oracle:
    """The oracle bound to one compiled copy of ``atf_oracle.c``."""

    W_INF = W_INF

    def __init__(self, lib_path: str | None = None):
        self._path = lib_path

    @property
    def lib(self):
        if self._path is None:
            return _load()
        if not hasattr(self, "_lib"):
            self._lib = _bind(self._path)
        return self._lib

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def window_table(self, d: int, base: float, alpha: float) -> np.ndarray:
        """W_p for p < d/2 as int64; ``W_INF`` marks an uncut pair."""
        W = np.zeros(d // 2, dtype=np.int64)
        rc = self.lib.orc_window_table(d, base, alpha, W.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        if rc != 0:
            raise ValueError("bad window-table arguments")
        return W

    @staticmethod
    def _as_f32(x) -> np.ndarray:
        if hasattr(x, "detach"):  # torch tensor (any dtype, any device)
            x = x.detach().to("cpu").float().contiguous().numpy()
        return np.ascontiguousarray(x, dtype=np.float32)

    def attention(self, q, k, v, *, base: float, alpha: float, causal: bool = True,
                  q_pos0: int = 0, k_pos0: int = 0, rows=None, q_shape=None, layout: str = "neox"):
        """Windowed-RoPE attention in fp64.

        q: [B, Hq, Sq, d]; k, v: [B, Hkv, Sk, d] (any float dtype; values are used
        exactly).  Query i sits at ``q_pos0 + i``, key j at ``k_pos0 + j``.
        ``rows``: optional int array [n, 3] of (b, h_q, i); default all rows.
        ``q_shape``: if given as (B, Hq, Sq, d), ``q`` holds only the listed
        rows' query vectors, [n, d] (for sampled rows of huge inputs).
        ``layout``: "neox" (pair p = dims p and p + d/2) or "gptj" (pair p =
        dims 2p and 2p + 1).
        Returns (out, skipped): out is [n, d] fp64 when ``rows`` is given, else
        [B, Hq, Sq, d]; skipped is the number of dropped (row, key, pair) terms.
        """
        if layout not in LAYOUTS:
            raise ValueError("layout must be one of %s" % sorted(LAYOUTS))
        q32, k32, v32 = self._as_f32(q), self._as_f32(k), self._as_f32(v)
        compact = q_shape is not None
        if compact and rows is None:
            raise ValueError("compact query rows need `rows`")
        B, Hq, Sq, d = q_shape if compact else q32.shape
        Bk, Hkv, Sk, dk = k32.shape
        if Bk != B or dk != d or v32.shape != k32.shape:
            raise ValueError("shape mismatch")
        full = rows is None
        if full:
            bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Sq), indexing="ij")
            rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.zeros((rows.shape[0], d), dtype=np.float64)
        skipped = ctypes.c_uint64(0)
        f32p = ctypes.POINTER(ctypes.c_float)
        if compact and q32.shape != (rows.shape[0], d):
            raise ValueError("compact q must be [n_rows, d]")
        rc = self.lib.orc_attention_rows(
            None if compact else q32.ctypes.data_as(f32p), k32.ctypes.data_as(f32p),
            v32.ctypes.data_as(f32p),
            B, Hq, Hkv, Sq, Sk, d, LAYOUTS[layout], float(base), float(alpha), 1 if causal else 0,
            int(q_pos0), int(k_pos0),
            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.shape[0],
            q32.ctypes.data_as(f32p) if compact else None,
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ctypes.byref(skipped))
        if rc != 0:
            raise ValueError("bad oracle arguments")
        if full:
            out = out.reshape(B, Hq, Sq, d)
        return out, int(skipped.value)

    def skipped_closed_form(self, S: int, d: int, base: float, alpha: float, decode: bool = False) -> int:
        """Dropped pair terms for ONE (b, h_q): causal prefill of S tokens, or one
        decode query placed after S cached keys."""
        out = ctypes.c_uint64(0)
        rc = self.lib.orc_skipped_closed_form(int(S), int(d), float(base), float(alpha),
                                             1 if decode else 0, ctypes.byref(out))
        if rc != 0:
            raise ValueError("bad closed-form arguments")
        return int(out.value)


_default = Oracle()
window_table = _default.window_table
attention = _default.attention
skipped_closed_form = _default.skipped_closed_form
num_threads = _default.num_threads
