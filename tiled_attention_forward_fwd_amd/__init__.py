"""Python binding of libfa, the gfx950 attention library (forward and backward).

Argument marshalling only: every step of the forward and backward passes runs
in the HIP kernels of ``libfa.so``. PyTorch provides device memory, the
stream and the workspaces some entry points take. There is no fallback: if
the library is missing or fails to load, the functions here raise.

    o, lse = fwd(q, k, v, causal=False, scale=None)
    dq, dk, dv = bwd(q, k, v, o, lse, dout, causal=False, scale=None)

q is ``[B, H, Nq, d]`` and k, v are ``[B, H, Nk, d]``; Nq may differ from Nk
(a causal row i sees keys j <= i). d is any multiple of 8 up to 128 (fp32:
64 or 128); float16, bfloat16, or float32 (forward only). ``fwd``
also takes padding lengths and sliding windows (``key_lens``,
``window_left``, ``window_right``) and picks the split-key launch for small
grids (``splits``). The C entry points are exposed under their own names
(those in ``EXPORTED``) for callers that manage their own buffers.
"""

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1

# Entry points declared in include/fa.h.
EXPORTED = ("fa_fwd", "fa_fwd_qk", "fa_fwd_split_qk", "fa_fwd_split_qk_noalloc", "fa_split_count",
            "fa_split_workspace_bytes",
            "fa_fwd_masked", "fa_fwd_split_masked", "fa_fwd_f32", "fa_f32_workspace_bytes", "fa_bwd", "fa_bwd_qk", "fa_bwd_masked",
            "fa_status_string", "fa_tile_counts",
            "fa_tile_counts_qk", "fa_tile_counts_masked", "fa_plan", "fa_plan_qk", "fa_plan_masked")


class FaPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("threads", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("workgroups", ctypes.c_int64),
                ("pairs_visited", ctypes.c_int64), ("mfma_flops", ctypes.c_double),
                ("algo_flops", ctypes.c_double), ("algo_bytes", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class FaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libfa status {status}: {message}")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """Load libfa.so (built by ``tiled_attention_forward_fwd_amd.build``)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libfa.so not found at {path}; build it with "
                          "`python -m tiled_attention_forward_fwd_amd.build`")
    import torch  # noqa: F401  (load torch's HIP runtime first so both share it)
    lib = ctypes.CDLL(path)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_qk.restype = ctypes.c_int
    lib.fa_fwd_qk.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_split_qk.restype = ctypes.c_int
    lib.fa_fwd_split_qk.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.fa_fwd_split_qk_noalloc.restype = ctypes.c_int
    lib.fa_fwd_split_qk_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_masked.restype = ctypes.c_int
    lib.fa_fwd_masked.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 8 + [
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_split_masked.restype = ctypes.c_int
    lib.fa_fwd_split_masked.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 8 + [
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p]
    lib.fa_tile_counts_masked.restype = ctypes.c_int
    lib.fa_tile_counts_masked.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.fa_plan_masked.restype = ctypes.c_int
    lib.fa_plan_masked.argtypes = [ctypes.c_int] * 8 + [ctypes.c_void_p, ctypes.c_int,
                                                        ctypes.POINTER(FaPlan)]
    lib.fa_fwd_f32.restype = ctypes.c_int
    lib.fa_fwd_f32.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.fa_f32_workspace_bytes.restype = ctypes.c_int64
    lib.fa_f32_workspace_bytes.argtypes = [ctypes.c_int] * 4
    lib.fa_split_count.restype = ctypes.c_int
    lib.fa_split_count.argtypes = [ctypes.c_int] * 6
    lib.fa_split_workspace_bytes.restype = ctypes.c_int64
    lib.fa_split_workspace_bytes.argtypes = [ctypes.c_int] * 5
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_bwd_masked.restype = ctypes.c_int
    lib.fa_bwd_masked.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 8 + [
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_bwd_qk.restype = ctypes.c_int
    lib.fa_bwd_qk.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_tile_counts.restype = ctypes.c_int
    lib.fa_tile_counts.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int64)]
    lib.fa_tile_counts_qk.restype = ctypes.c_int
    lib.fa_tile_counts_qk.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
    lib.fa_plan.restype = ctypes.c_int
    lib.fa_plan.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(FaPlan)]
    lib.fa_plan_qk.restype = ctypes.c_int
    lib.fa_plan_qk.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(FaPlan)]
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def _check(rc):
    if rc != FA_OK:
        raise FaError(rc, fa_status_string(rc))


def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_fwd(q, k, v, o, lse, int(B), int(H), int(N), int(d), int(causal),
                                 float(scale), int(dtype), stream)


def fa_fwd_qk(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_fwd_qk(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk), int(d),
                                    int(causal), float(scale), int(dtype), stream)


def fa_fwd_split_qk(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, n_splits, workspace,
                    workspace_bytes, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_fwd_split_qk(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk), int(d),
                                          int(causal), float(scale), int(dtype), int(n_splits),
                                          workspace, int(workspace_bytes), stream)


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # FA_NOALLOC_SCRATCH_BYTES of include/fa.h


def fa_fwd_split_qk_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, n_splits, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status.
    The split partials go to the library's static scratch (no allocation)."""
    return load_library().fa_fwd_split_qk_noalloc(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk),
                                                  int(d), int(causal), float(scale), int(dtype),
                                                  int(n_splits), stream)


def fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, d, causal, window_left, window_right, key_lens,
                  scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints; key_lens a device
    pointer or None); returns the status."""
    return load_library().fa_fwd_masked(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk), int(d),
                                        int(causal), int(window_left), int(window_right), key_lens,
                                        float(scale), int(dtype), stream)


def fa_fwd_split_masked(q, k, v, o, lse, B, H, Nq, Nk, d, causal, window_left, window_right,
                        key_lens, scale, dtype, n_splits, workspace, workspace_bytes, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_fwd_split_masked(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk),
                                              int(d), int(causal), int(window_left),
                                              int(window_right), key_lens, float(scale), int(dtype),
                                              int(n_splits), workspace, int(workspace_bytes), stream)


def fa_tile_counts_masked(Nq, Nk, block_m, block_n, causal, window_left, window_right, key_len):
    """fa_tile_counts for one batch under padding and window masks."""
    out = (ctypes.c_int64 * 4)()
    _check(load_library().fa_tile_counts_masked(int(Nq), int(Nk), int(block_m), int(block_n),
                                                int(causal), int(window_left), int(window_right),
                                                int(key_len), out))
    return tuple(out)


def fa_plan_masked(B, H, Nq, Nk, d, causal, window_left, window_right, key_lens, dtype):
    """The plan of fa_fwd_masked; key_lens is a host sequence of B ints or None."""
    plan = FaPlan()
    arr = None if key_lens is None else (ctypes.c_int32 * int(B))(*[int(x) for x in key_lens])
    _check(load_library().fa_plan_masked(int(B), int(H), int(Nq), int(Nk), int(d), int(causal),
                                         int(window_left), int(window_right),
                                         None if arr is None else ctypes.addressof(arr), int(dtype),
                                         ctypes.byref(plan)))
    return plan.as_dict()


def fa_fwd_f32(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, workspace, workspace_bytes, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_fwd_f32(q, k, v, o, lse, int(B), int(H), int(Nq), int(Nk), int(d),
                                     int(causal), float(scale), workspace, int(workspace_bytes), stream)


def fa_f32_workspace_bytes(B, H, Nk, d):
    return int(load_library().fa_f32_workspace_bytes(int(B), int(H), int(Nk), int(d)))


def fa_split_count(B, H, Nq, Nk, d, causal):
    return int(load_library().fa_split_count(int(B), int(H), int(Nq), int(Nk), int(d), int(causal)))


def fa_split_workspace_bytes(B, H, Nq, d, n_splits):
    return int(load_library().fa_split_workspace_bytes(int(B), int(H), int(Nq), int(d), int(n_splits)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H), int(N),
                                 int(d), int(causal), float(scale), int(dtype), stream)


def fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H), int(Nq),
                                    int(Nk), int(d), int(causal), float(scale), int(dtype), stream)


def fa_bwd_masked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, window_left,
                  window_right, key_lens, scale, dtype, stream):
    """Direct call of the C entry point with raw pointers (ints); returns the status."""
    return load_library().fa_bwd_masked(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H),
                                        int(Nq), int(Nk), int(d), int(causal), int(window_left),
                                        int(window_right), key_lens, float(scale), int(dtype), stream)


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, stream=None, window_left=-1, window_right=-1,
        key_lens=None):
    """Attention backward on the GPU: returns ``(dq, dk, dv)``.

    q, o, dout : CUDA (HIP) tensors ``[B, H, Nq, d]``; k, v ``[B, H, Nk, d]``;
                 contiguous, one of float16/bfloat16; ``o`` and ``lse``
                 (``[B, H, Nq]`` float32) from ``fwd`` with the same causal
                 flag, scale and masks. The D = rowsum(dO * O) scratch is
                 allocated with torch.
    window_left, window_right, key_lens : the masks of ``fwd``.
    """
    import torch
    ts = (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout))
    for name, t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] GPU tensor")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in dtype")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must match q in shape")
    if k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3] or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    code = dtype_code(q.dtype)
    if scale is None:
        scale = default_scale(d)
    sobj = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device), torch.cuda.stream(sobj):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
        kl_ptr = None
        if key_lens is not None:
            key_lens = _device_key_lens(key_lens, B, q.device)
            kl_ptr = key_lens.data_ptr()
        rc = fa_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                           B, H, N, Nk, d, causal, window_left, window_right, kl_ptr, scale, code,
                           sobj.cuda_stream)
    _check(rc)
    return dq, dk, dv


def fa_tile_counts_qk(Nq, Nk, block_m, block_n, causal):
    """fa_tile_counts for Nq query rows against Nk keys."""
    out = (ctypes.c_int64 * 4)()
    _check(load_library().fa_tile_counts_qk(int(Nq), int(Nk), int(block_m), int(block_n),
                                            int(causal), out))
    return tuple(out)


def fa_plan_qk(B, H, Nq, Nk, d, causal, dtype):
    plan = FaPlan()
    _check(load_library().fa_plan_qk(int(B), int(H), int(Nq), int(Nk), int(d), int(causal),
                                     int(dtype), ctypes.byref(plan)))
    return plan.as_dict()


def fa_tile_counts(N, block_m, block_n, causal):
    """(all pairs, visited, visited without mask, visited with mask) for one head."""
    out = (ctypes.c_int64 * 4)()
    _check(load_library().fa_tile_counts(int(N), int(block_m), int(block_n), int(causal), out))
    return tuple(out)


def fa_plan(B, H, N, d, causal, dtype):
    plan = FaPlan()
    _check(load_library().fa_plan(int(B), int(H), int(N), int(d), int(causal), int(dtype),
                                  ctypes.byref(plan)))
    return plan.as_dict()


def _launch_stream(stream, device):
    """The torch stream object the kernels go on (torch's current stream when
    `stream` is None; a raw hipStream_t handle is wrapped). Every temporary a
    call allocates (outputs, workspaces, the delta scratch, the device copy of
    key_lens) is allocated and filled while this stream is current, so the
    caching allocator orders its reuse after the kernels that read it."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _device_key_lens(key_lens, B, device):
    import torch
    if not torch.is_tensor(key_lens):
        key_lens = torch.tensor([int(x) for x in key_lens], dtype=torch.int32, device=device)
    if (key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.shape != (B,)
            or not key_lens.is_contiguous()):
        raise ValueError("key_lens must be a contiguous int32 [B] GPU tensor")
    return key_lens


def dtype_code(torch_dtype):
    import torch
    if torch_dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if torch_dtype == torch.float16:
        return FA_DTYPE_F16
    raise TypeError(f"unsupported dtype {torch_dtype}; libfa takes float16 or bfloat16")


def default_scale(d):
    """1/sqrt(d) rounded to fp32, the value passed to the kernel."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(d)))


def _fwd_f32(q, k, v, causal, scale, out, lse, stream, workspace, splits, window_left, window_right,
             key_lens):
    import torch
    if splits not in (None, 1) or key_lens is not None or window_left != -1 or window_right != -1:
        raise ValueError("float32 inputs take neither key splits nor masks")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    sobj = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device), torch.cuda.stream(sobj):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
        if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor like q")
        if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        need = fa_f32_workspace_bytes(B, H, Nk, d)
        if workspace is None:
            workspace = torch.empty(max(need, 16) // 2, device=q.device, dtype=torch.bfloat16)
        ws_bytes = workspace.numel() * workspace.element_size()
        if ws_bytes < need or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes")
        rc = fa_fwd_f32(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                        N, Nk, d, causal, scale, workspace.data_ptr(), ws_bytes, sobj.cuda_stream)
    _check(rc)
    return out, lse


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None, splits=None,
        workspace=None, window_left=-1, window_right=-1, key_lens=None):
    """Attention forward on the GPU: returns ``(o, lse)``.

    q       : CUDA (HIP) tensor ``[B, H, Nq, d]``; k, v: ``[B, H, Nk, d]``;
              contiguous, float16, bfloat16 or float32, all the same dtype.
              A causal row i sees keys j <= i. float32 runs ``fa_fwd_f32``
              (split-bf16 products; no masks or key splits) with a workspace
              from torch unless ``workspace`` is given.
    scale   : defaults to 1/sqrt(d) in fp32.
    out/lse : optional preallocated outputs (``[B, H, Nq, d]`` dtype and
              ``[B, H, Nq]`` float32).
    splits  : key chunks of the split-key path (``fa_fwd_split_qk``). None
              takes ``fa_split_count``'s suggestion, which is 1 (the direct
              entry point, which runs its key-split kernel on small grids of
              up to 2048 keys) unless the grid is too small to fill the GPU
              over longer key ranges; the workspace is then allocated with
              torch unless given.
    window_left, window_right, key_lens : the masks of ``fa_fwd_masked``
              (-1 = unbounded; key_lens a length-B int32 GPU tensor or a
              sequence, copied to the GPU). A row that sees no key gets O = 0
              and lse = -inf.
    The kernels are enqueued on ``stream`` (default: torch's current stream).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    if k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3] or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must have the same dtype")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if q.dtype == torch.float32:
        return _fwd_f32(q, k, v, causal, scale, out, lse, stream, workspace, splits, window_left,
                        window_right, key_lens)
    code = dtype_code(q.dtype)
    if scale is None:
        scale = default_scale(d)
    if splits is None:
        splits = fa_split_count(B, H, N, Nk, d, causal) or 1
    masked = key_lens is not None or window_left != -1 or window_right != -1
    sobj = _launch_stream(stream, q.device)
    handle = sobj.cuda_stream
    with torch.cuda.device(q.device), torch.cuda.stream(sobj):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
        if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor like q")
        if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        kl_ptr = None
        if key_lens is not None:
            key_lens = _device_key_lens(key_lens, B, q.device)
            kl_ptr = key_lens.data_ptr()
        if masked:
            if splits == 1:
                rc = fa_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, N, Nk, d, causal, window_left, window_right,
                                   kl_ptr, scale, code, handle)
            else:
                need = fa_split_workspace_bytes(B, H, N, d, splits)
                if workspace is None:
                    workspace = torch.empty(need // 4, device=q.device, dtype=torch.float32)
                if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
                    raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes")
                rc = fa_fwd_split_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), B, H, N, Nk, d, causal, window_left,
                                         window_right, kl_ptr, scale, code, splits,
                                         workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), handle)
        elif splits == 1:
            rc = fa_fwd_qk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, N, Nk, d, causal, scale, code, handle)
        else:
            need = fa_split_workspace_bytes(B, H, N, d, splits)
            if workspace is None:
                workspace = torch.empty(need // 4, device=q.device, dtype=torch.float32)
            if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
                raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes")
            rc = fa_fwd_split_qk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, H, N, Nk, d, causal, scale, code, splits,
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 handle)
    _check(rc)
    return out, lse
