"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers. The GPU path does not import this
package, and this package imports nothing from the GPU path.

The arithmetic lives in ``fa_oracle.c`` (plain C, double precision); this
module builds it with gcc and marshals arrays through ctypes. See the header
of ``fa_oracle.c`` for the definition it follows and the passages it cites.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_SRC_BWD = os.path.join(_HERE, "fa_oracle_bwd.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_BWD = os.path.join(_HERE, "liboracle_bwd.so")
_lib = None
_lib_bwd = None


def build(src=_SRC, out=_LIB, extra_flags=()):
    """Compile the forward oracle (or a variant of its source) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", *extra_flags,
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_bwd(src=_SRC_BWD, out=_LIB_BWD, extra_flags=()):
    """Compile the backward oracle (or a variant of its source) into a shared library."""
    return build(src, out, extra_flags)


def build_all():
    build()
    build_bwd()


def _bind(lib):
    fn = lib.fa_oracle_fwd_masked
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5 + [
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int]
    return lib


def load(path=None):
    """Load the built oracle, building it first if it is missing."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


MAX_THREADS = 16  # the CPU share of one GPU on the test machines


def default_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def _as_f32(x):
    """dtype-rounded tensor/array -> contiguous fp32 numpy (exact for fp16/bf16)."""
    if hasattr(x, "detach"):  # torch tensor, possibly bf16
        import torch
        x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def attention_fwd(q, k, v, causal, scale, rows=None, tile_n=0, nthreads=None, lib=None,
                  window_left=-1, window_right=-1, key_lens=None):
    """fp64 attention forward on the CPU.

    q       : ``[B, H, Nq, d]``; k, v: ``[B, H, Nk, d]`` (torch or numpy; values
              already in the storage dtype). ``scale`` is applied to Q.K^T
              before the softmax. A causal row i sees keys j <= i (top-left
              alignment when Nq != Nk).
    rows    : optional sorted list of query rows to evaluate (all by default).
    tile_n  : 0 for the two-pass definition, > 0 for the online order.
    window_left, window_right, key_lens : the masks of ``fa_oracle_fwd_masked``
              (-1 = unbounded; key_lens a length-B sequence or None). A row
              with no visible key gets O = 0 and lse = -inf.
    Returns ``(o, lse)`` as float64 numpy arrays of shape ``[B, H, R, d]`` and
    ``[B, H, R]``, where ``R`` is ``len(rows)`` or ``Nq``; lse is natural-log.
    """
    lib = lib or load()
    qf, kf, vf = _as_f32(q), _as_f32(k), _as_f32(v)
    B, H, N, d = qf.shape
    Nk = kf.shape[2]
    assert kf.shape == (B, H, Nk, d) and vf.shape == kf.shape
    if rows is None:
        R, rows_arr, rows_ptr = N, None, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R, rows_ptr = rows_arr.size, rows_arr.ctypes.data
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    kl = None if key_lens is None else np.ascontiguousarray(np.asarray(key_lens, dtype=np.int64))
    if kl is not None:
        assert kl.shape == (B,)
    rc = lib.fa_oracle_fwd_masked(qf.ctypes.data, kf.ctypes.data, vf.ctypes.data, B, H, N, Nk, d,
                           1 if causal else 0, int(window_left), int(window_right),
                           None if kl is None else kl.ctypes.data, float(scale), rows_ptr,
                           0 if rows_arr is None else R, int(tile_n), o.ctypes.data,
                           lse.ctypes.data, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd failed with status {rc}")
    return o, lse


def _bind_bwd(lib):
    fn = lib.fa_oracle_bwd_masked
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 5 + [
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    return lib


def load_bwd(path=None):
    """Load the built backward oracle, building it first if it is missing."""
    global _lib_bwd
    if path is not None:
        return _bind_bwd(ctypes.CDLL(path))
    if _lib_bwd is None:
        if not os.path.exists(_LIB_BWD):
            build_bwd()
        _lib_bwd = _bind_bwd(ctypes.CDLL(_LIB_BWD))
    return _lib_bwd


def attention_bwd(q, k, v, dout, causal, scale, nthreads=None, lib=None, window_left=-1,
                  window_right=-1, key_lens=None):
    """fp64 gradients of sum(dout * O) for O = attention(q, k, v) on the CPU.

    q, dout : ``[B, H, Nq, d]``; k, v: ``[B, H, Nk, d]`` (values in the storage
              dtype). window_left, window_right, key_lens: the masks of
              ``attention_fwd``. Returns ``(dq, dk, dv)`` as float64 numpy
              arrays. See the header of ``fa_oracle_bwd.c`` for the definition.
    """
    lib = lib or load_bwd()
    qf, kf, vf, df = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, H, Nq, d = qf.shape
    Nk = kf.shape[2]
    assert kf.shape == (B, H, Nk, d) and vf.shape == kf.shape and df.shape == qf.shape
    dq = np.empty((B, H, Nq, d), dtype=np.float64)
    dk = np.empty((B, H, Nk, d), dtype=np.float64)
    dv = np.empty((B, H, Nk, d), dtype=np.float64)
    kl = None if key_lens is None else np.ascontiguousarray(np.asarray(key_lens, dtype=np.int64))
    if kl is not None:
        assert kl.shape == (B,)
    rc = lib.fa_oracle_bwd_masked(qf.ctypes.data, kf.ctypes.data, vf.ctypes.data, df.ctypes.data, B,
                                  H, Nq, Nk, d, 1 if causal else 0, int(window_left),
                                  int(window_right), None if kl is None else kl.ctypes.data,
                                  float(scale), dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                  int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd failed with status {rc}")
    return dq, dk, dv
