"""Python binding of libfa355, the gfx950 attention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa355.so``.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing or cannot be loaded, every
call raises.

Raw C-ABI functions (same names and argument order as include/fa355.h):
    fa_fwd(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype) -> int
    fa_fwd_splitkv_workspace(B, H, N, d, num_splits) -> int (bytes or status)
    fa_fwd_splitkv(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype,
                   num_splits, workspace, workspace_bytes) -> int
    fa_fwd_blocksparse(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype,
                       block_mask, mask_heads) -> int
    fa_bwd_workspace(B, H, N, d) -> int (bytes or status)
    fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, scale, causal, stream, dtype,
           workspace, workspace_bytes) -> int
    fa_strerror(status) -> str
    fa_version() -> int
where Q, K, V, O, L and stream are integer addresses.

Tensor front end:
    fwd(q, k, v, scale=None, causal=False, out=None, lse=None) -> (O, L)
    fwd_splitkv(q, k, v, num_splits, scale=None, causal=False, out=None,
                lse=None, workspace=None) -> (O, L, workspace)
    fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False, out=None,
                    lse=None) -> (O, L)
    bwd(q, k, v, o, do, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
        workspace=None) -> (dQ, dK, dV)
"""

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa355.so")

FA_BF16 = 0
FA_F32 = 1
FA_F16 = 2

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_UNSUPPORTED_D = -3
FA_ERR_DTYPE = -4
FA_ERR_SCALE = -5
FA_ERR_ALIGN = -6
FA_ERR_ALIAS = -7
FA_ERR_HIP = -8
FA_ERR_ARG = -9
FA_ERR_SPLITS = -10
FA_ERR_WORKSPACE = -11
FA_ERR_SCRATCH = -12
# Size of the library's own split workspace (fa_fwd_splitkv_noalloc).
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_lib = None


class FaError(RuntimeError):
    """A non-zero status returned by libfa355."""

    def __init__(self, status):
        super().__init__(f"fa_fwd failed ({status}): {fa_strerror(status)}")
        self.status = status


def load(path=LIB_PATH):
    """Load libfa355.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m io_aware_softmax_06_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, vp, ctypes.c_int]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_splitkv_workspace.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.fa_fwd_splitkv_workspace.restype = i64
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                   ctypes.c_float, ctypes.c_int, vp, ctypes.c_int,
                                   ctypes.c_int, vp, i64]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                           ctypes.c_float, ctypes.c_int, vp, ctypes.c_int,
                                           ctypes.c_int]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                       ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp, i64]
    lib.fa_fwd_blocksparse.restype = ctypes.c_int
    lib.fa_bwd_workspace.argtypes = [i64, i64, i64, i64]
    lib.fa_bwd_workspace.restype = i64
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp, i64]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_strerror.argtypes = [ctypes.c_int]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def fa_fwd(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype):
    """Direct call of the C entry point; returns its status code."""
    return load().fa_fwd(Q, K, V, O, L, B, H, N, d, float(scale), int(causal), stream, dtype)


def fa_fwd_splitkv_workspace(B, H, N, d, num_splits):
    """Workspace bytes of fa_fwd_splitkv, or a negative status."""
    return load().fa_fwd_splitkv_workspace(B, H, N, d, int(num_splits))


def fa_fwd_splitkv(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype, num_splits,
                   workspace, workspace_bytes):
    """Direct call of the C entry point; returns its status code."""
    return load().fa_fwd_splitkv(Q, K, V, O, L, B, H, N, d, float(scale), int(causal), stream,
                                 dtype, int(num_splits), workspace, workspace_bytes)


def fa_fwd_splitkv_noalloc(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype, num_splits):
    """Direct call of the C entry point; returns its status code."""
    return load().fa_fwd_splitkv_noalloc(Q, K, V, O, L, B, H, N, d, float(scale), int(causal),
                                         stream, dtype, int(num_splits))


def fa_fwd_blocksparse(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype, block_mask,
                       mask_heads):
    """Direct call of the C entry point; returns its status code."""
    return load().fa_fwd_blocksparse(Q, K, V, O, L, B, H, N, d, float(scale), int(causal),
                                     stream, dtype, block_mask, int(mask_heads))


def fa_bwd_workspace(B, H, N, d):
    """Workspace bytes of fa_bwd, or a negative status."""
    return load().fa_bwd_workspace(B, H, N, d)


def fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, scale, causal, stream, dtype, workspace,
           workspace_bytes):
    """Direct call of the C entry point; returns its status code."""
    return load().fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, float(scale), int(causal),
                         stream, dtype, workspace, workspace_bytes)


def fa_strerror(status):
    return load().fa_strerror(int(status)).decode()


def fa_version():
    return load().fa_version()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _on_device(dev):
    """Context making ``dev`` the current HIP device: the library launches
    on the calling thread's current device, which must hold the tensors."""
    import torch
    return torch.cuda.device(dev)


def _prepare(q, k, v, scale, out, lse, stream):
    import torch
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k and v must share shape, dtype and device")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
          or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return (B, H, N, d), scale, out, lse, stream


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """Attention forward on [B, H, N, d] device tensors; returns (O, L).

    O has q's dtype and shape; L is float32 [B, H, N].  Runs on ``stream``
    (default: torch's current stream) and does not synchronise.
    """
    (B, H, N, d), scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    with _on_device(q.device):
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, d, scale, 1 if causal else 0, stream.cuda_stream, _dtype_code(q))
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def fwd_splitkv(q, k, v, num_splits, scale=None, causal=False, out=None, lse=None,
                workspace=None, stream=None):
    """Key-range split forward; returns (O, L, workspace).

    Same result as ``fwd`` up to float rounding.  ``workspace`` is a uint8
    device tensor of at least ``fa_fwd_splitkv_workspace(...)`` bytes
    (allocated here when None); after the call it holds the per-range
    partials O_s float32 [num_splits, B, H, N, d] followed by L_s float32
    [num_splits, B, H, N].
    """
    import torch
    (B, H, N, d), scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    need = fa_fwd_splitkv_workspace(B, H, N, d, num_splits)
    if need < 0:
        raise FaError(need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(q.device):
        rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, H, N, d, scale, 1 if causal else 0,
                            stream.cuda_stream, _dtype_code(q), num_splits,
                            workspace.data_ptr(), ws_bytes)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse, workspace


def fwd_splitkv_noalloc(q, k, v, num_splits, scale=None, causal=False, out=None, lse=None,
                        stream=None):
    """Key-range split forward on the library's own scratch buffer; returns (O, L).

    The library allocates nothing for the partials: they go to its fixed
    per-device scratch of NOALLOC_SCRATCH_BYTES (FaError FA_ERR_SCRATCH when
    the call needs more).  Calls that may overlap on one device race on it.
    (O and L are still allocated here when not given.)
    """
    (B, H, N, d), scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    with _on_device(q.device):
        rc = fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, N, d, scale, 1 if causal else 0,
                                    stream.cuda_stream, _dtype_code(q), num_splits)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def split_partials(workspace, num_splits, B, H, N, d):
    """Views (O_s [S, B, H, N, d], L_s [S, B, H, N]) of a split workspace."""
    import torch
    rows = B * H * N
    f = workspace[: num_splits * rows * (d + 1) * 4].view(torch.float32)
    o = f[: num_splits * rows * d].view(num_splits, B, H, N, d)
    l = f[num_splits * rows * d:].view(num_splits, B, H, N)
    return o, l


MASK_BLOCK = 64


def fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False, out=None, lse=None,
                    stream=None):
    """Block-sparse attention forward; returns (O, L).

    ``block_mask`` is a uint8 device tensor [nb, nb], [H, nb, nb] or
    [B, H, nb, nb] with nb = ceil(N / 64): entry [i, j] nonzero lets the
    queries of 64-row block i see the keys of 64-key block j.
    """
    import torch
    (B, H, N, d), scale, out, lse, stream = _prepare(q, k, v, scale, out, lse, stream)
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    m = block_mask
    if m.dtype != torch.uint8 or m.device != q.device or not m.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 tensor on q's device")
    if m.dim() == 2 and m.shape == (nb, nb):
        mask_heads = 1
    elif m.dim() == 3 and m.shape == (H, nb, nb):
        mask_heads = H
    elif m.dim() == 4 and m.shape == (B, H, nb, nb):
        mask_heads = B * H
    else:
        raise ValueError(f"block_mask must be [{nb}, {nb}], [H, {nb}, {nb}] or [B, H, {nb}, {nb}]")
    with _on_device(q.device):
        rc = fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, d, scale, 1 if causal else 0,
                                stream.cuda_stream, _dtype_code(q), m.data_ptr(), mask_heads)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def bwd(q, k, v, o, do, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Attention backward; returns (dQ, dK, dV) with q's dtype and shape.

    ``o`` and ``lse`` are the forward's outputs for the same q, k, v, scale
    and mask; ``do`` is the gradient of the loss with respect to o.  The
    workspace (uint8, at least ``fa_bwd_workspace(...)`` bytes) receives the
    row sums D = rowsum(do * o); it is allocated here when None.
    """
    import torch
    (B, H, N, d), scale, _, _, stream = _prepare(q, k, v, scale, o, lse, stream)
    if do.shape != q.shape or do.dtype != q.dtype or do.device != q.device or not do.is_contiguous():
        raise ValueError("do must be a contiguous tensor like q")
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_like(q)
        elif g.shape != q.shape or g.dtype != q.dtype or g.device != q.device or not g.is_contiguous():
            raise ValueError("dq, dk and dv must be contiguous tensors like q")
        grads.append(g)
    need = fa_bwd_workspace(B, H, N, d)
    if need < 0:
        raise FaError(need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(q.device):
        rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                    lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                    grads[2].data_ptr(), B, H, N, d, scale, 1 if causal else 0,
                    stream.cuda_stream, _dtype_code(q), workspace.data_ptr(), ws_bytes)
    if rc != FA_OK:
        raise FaError(rc)
    return tuple(grads)
