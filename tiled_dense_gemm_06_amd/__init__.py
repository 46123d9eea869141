"""tlg: C = ReLU(A . B) on MI355X (gfx950), fp16 in, fp32 accumulation, fp16 out.

The operation is the quick-start ``matmul_relu`` of the TileLang article
(aiwiki.ai/wiki/tilelang, "Programming model"). All computation happens in
the hand-written gfx950 kernels of ``libtlg.so`` behind the C ABI in
``include/tlg.h``; this module only passes PyTorch device pointers, leading
dimensions and the current stream to it. There is no CPU fallback: without
the built library every call raises.
"""
from __future__ import annotations

from . import _native
from ._native import (  # noqa: F401  (re-exported C-ABI names)
    TLG_VARIANT_AUTO, TLG_VARIANT_FILL_ZERO, TLG_VARIANT_NAIVE, TLG_VARIANT_NOOP, TLG_VARIANT_PINGPONG,
    TLG_VARIANT_SPLITK, TLG_VARIANT_TILED_DMA, TLG_VARIANT_TILED_GENERAL, TLG_VARIANT_TILED_PIPE, TlgError,
    tlg_arch_supported, tlg_check_args, tlg_plan, tlg_plan_config_name, tlg_status_string,
    tlg_version, tlg_workspace_bytes,
)

__all__ = ["gemm_relu", "gemm_relu_grouped", "gemm_relu_mx", "gemm_relu_mx_grouped", "Handle", "handle_for", "plan",
           "plan_mx"]


class Handle:
    """A tlg handle bound to one GPU (tlg_create / tlg_destroy)."""

    def __init__(self, device=None):
        import torch

        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else
                                   torch.device(device).index or 0)
        with torch.cuda.device(self.device):
            self.ptr = _native.tlg_create()

    def close(self):
        if getattr(self, "ptr", None):
            _native.tlg_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_handles: dict[int, Handle] = {}


def handle_for(device) -> Handle:
    """The module's cached handle for a CUDA/HIP device (created on first use)."""
    idx = device.index if device.index is not None else 0
    h = _handles.get(idx)
    if h is None:
        h = Handle(device)
        _handles[idx] = h
    return h


def _ld(t) -> int:
    """Leading dimension (elements) of a row-major 2-D tensor."""
    rows, cols = t.shape
    if rows <= 1 or t.numel() == 0:
        return max(1, cols)
    return t.stride(0)


def _check(t, name):
    import torch

    if t.dtype != torch.float16:
        raise TypeError(f"{name} must be float16, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.numel() == 0:
        return  # no element is read or written; an empty tensor's strides carry no layout
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its rows (row-major)")
    if t.shape[0] > 1 and t.stride(0) < max(1, t.shape[1]):
        raise ValueError(f"{name} rows overlap")


def _out_for(out, M, N, device):
    import torch

    if out is None:
        return torch.empty((M, N), dtype=torch.float16, device=device)
    _check(out, "out")
    if tuple(out.shape) != (M, N) or out.device != device:
        raise ValueError("out has the wrong shape or device")
    return out


def gemm_relu(A, B, out=None, *, trans_b: bool = False, variant: int = TLG_VARIANT_AUTO, config: int = -1,
              splits: int = 0, stream=None, handle=None):
    """C = ReLU(A @ B) for fp16 row-major A (M, K) and B (K, N); returns C (M, N).

    With ``trans_b`` B is given transposed, as an (N, K) row-major tensor, and
    C = ReLU(A @ B.T). ``out`` may be a preallocated fp16 (M, N) tensor (a
    padded row view is fine: only its M x N window is written). The work is
    enqueued on ``stream`` (default: the current stream of A's device) and is
    asynchronous. ``variant``/``config``/``splits`` force a kernel family, tile
    configuration and split count (tests and measurements; with ``trans_b``
    the families are the direct-to-LDS and pipelined ones, without splits).
    """
    import torch

    _check(A, "A")
    _check(B, "B")
    M, K = A.shape
    if trans_b:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    out = _out_for(out, M, N, A.device)
    h = handle if handle is not None else handle_for(A.device)
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        if trans_b:
            st = _native.tlg_gemm_relu_bt_variant(h.ptr, variant, config, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(),
                                                  _ld(B), out.data_ptr(), _ld(out), s.cuda_stream)
        else:
            st = _native.tlg_gemm_relu_variant(h.ptr, variant, config, splits, M, N, K, A.data_ptr(), _ld(A),
                                               B.data_ptr(), _ld(B), out.data_ptr(), _ld(out), s.cuda_stream)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_gemm_relu_bt" if trans_b else "tlg_gemm_relu")
    return out


def gemm_relu_grouped(As, Bs, outs=None, *, trans_b: bool = False, config: int = -1, stream=None, handle=None):
    """C_i = ReLU(A_i @ B_i) (or A_i @ B_i.T with ``trans_b``) for up to 16
    problems in one launch; returns the list of C_i."""
    import torch

    if len(As) != len(Bs) or (outs is not None and len(outs) != len(As)):
        raise ValueError("As, Bs and outs differ in length")
    if len(As) > _native.TLG_GROUP_MAX:
        raise ValueError(f"at most {_native.TLG_GROUP_MAX} problems per call")
    if not As:
        return []
    dev = As[0].device
    descs, res = [], []
    for i, (A, B) in enumerate(zip(As, Bs)):
        _check(A, "A")
        _check(B, "B")
        if A.device != dev or B.device != dev:
            raise ValueError("all operands must be on one device")
        M, K = A.shape
        N, K2 = B.shape if trans_b else (B.shape[1], B.shape[0])
        if K != K2:
            raise ValueError(f"problem {i}: inner dimensions differ: {K} vs {K2}")
        C = _out_for(None if outs is None else outs[i], M, N, dev)
        res.append(C)
        descs.append((M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), C.data_ptr(), _ld(C)))
    h = handle if handle is not None else handle_for(dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.tlg_gemm_relu_grouped_variant(h.ptr, config, descs, 1 if trans_b else 0, s.cuda_stream)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_gemm_relu_grouped")
    return res


def plan(M, N, K, lda=None, ldb=None, ldc=None, *, aligned: bool = True, variant: int = TLG_VARIANT_AUTO,
         config: int = -1, splits: int = 0, trans_b: bool = False) -> dict:
    """What gemm_relu would launch for a problem (host logic only, no GPU).

    Pointers are stand-ins: 16-byte aligned when ``aligned`` else 2-byte aligned.
    """
    lda = max(1, K) if lda is None else lda
    ldb = (max(1, K) if trans_b else max(1, N)) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    base = 1 << 20 if aligned else (1 << 20) + 2
    if trans_b:
        st, info = _native.tlg_plan_bt(M, N, K, base, lda, base, ldb, base, ldc, variant, config)
    else:
        st, info = _native.tlg_plan(M, N, K, base, lda, base, ldb, base, ldc, variant, config, splits)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_plan_bt" if trans_b else "tlg_plan")
    d = info.as_dict()
    d["variant_name"] = _native.VARIANT_NAMES.get(info.variant, "?")
    d["config_name"] = _native.tlg_plan_config_name(info.variant, info.config)
    return d


def _mx_format(fmt) -> int:
    f = _native.MX_FORMATS.get(fmt, fmt) if isinstance(fmt, str) else int(fmt)
    if f not in _native.MX_FORMATS.values():
        raise ValueError(f"unknown block-scaled format {fmt!r} (e4m3, e5m2 or e2m1)")
    return f


def _mx_ld(t, what, per_byte) -> int:
    """Leading dimension in codes of a row-major 2-D uint8 tensor of packed codes."""
    import torch

    if t.dtype != torch.uint8 or t.dim() != 2:
        raise TypeError(f"{what} must be a 2-D uint8 tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on a GPU")
    if t.numel() and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} must have unit stride along its rows (row-major)")
    rows, cols = t.shape
    ld = max(1, cols) if rows <= 1 or t.numel() == 0 else t.stride(0)
    return ld * per_byte


def gemm_relu_mx(fmt, A, SA, Bt, SB, out=None, *, config: int = -1, stream=None, handle=None):
    """Block-scaled C = ReLU(A . Bt^T) (fp16 out) for element codes A (M, K)
    and Bt (N, K) (``fmt`` "e4m3", "e5m2", or "e2m1" with two codes per byte,
    so the uint8 tensors are (M, K/2) and (N, K/2)) and E8M0 scale bytes SA
    (M, K/32), SB (N, K/32), all uint8 on the GPU. ``config`` forces a tile
    configuration (0: 256 x 256, 1: 128 x 128)."""
    import torch

    f = _mx_format(fmt)
    per = 2 if f == _native.TLG_MX_E2M1 else 1
    lda, ldb = _mx_ld(A, "A", per), _mx_ld(Bt, "Bt", per)
    ldsa, ldsb = _mx_ld(SA, "SA", 1), _mx_ld(SB, "SB", 1)
    M, K = A.shape[0], A.shape[1] * per
    N = Bt.shape[0]
    if Bt.shape[1] * per != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Bt.shape[1] * per}")
    if tuple(SA.shape) != (M, K // 32) or tuple(SB.shape) != (N, K // 32):
        raise ValueError("scale tensors must be (M, K/32) and (N, K/32)")
    out = _out_for(out, M, N, A.device)
    h = handle if handle is not None else handle_for(A.device)
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        st = _native.tlg_gemm_relu_mx_variant(h.ptr, config, f, M, N, K, A.data_ptr(), lda, SA.data_ptr(), ldsa,
                                              Bt.data_ptr(), ldb, SB.data_ptr(), ldsb, out.data_ptr(), _ld(out),
                                              s.cuda_stream)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_gemm_relu_mx")
    return out


def gemm_relu_mx_grouped(fmt, As, SAs, Bts, SBs, outs=None, *, config: int = -1, stream=None, handle=None):
    """Up to 16 block-scaled problems (arguments as gemm_relu_mx, one format)
    in one launch; returns the list of fp16 C_i."""
    import torch

    f = _mx_format(fmt)
    per = 2 if f == _native.TLG_MX_E2M1 else 1
    n = len(As)
    if not (len(SAs) == len(Bts) == len(SBs) == n) or (outs is not None and len(outs) != n):
        raise ValueError("As, SAs, Bts, SBs and outs differ in length")
    if n > _native.TLG_GROUP_MAX:
        raise ValueError(f"at most {_native.TLG_GROUP_MAX} problems per call")
    if n == 0:
        return []
    dev = As[0].device
    descs, res = [], []
    for i in range(n):
        A, SA, Bt, SB = As[i], SAs[i], Bts[i], SBs[i]
        if any(t.device != dev for t in (A, SA, Bt, SB)):
            raise ValueError("all operands must be on one device")
        lda, ldb = _mx_ld(A, "A", per), _mx_ld(Bt, "Bt", per)
        ldsa, ldsb = _mx_ld(SA, "SA", 1), _mx_ld(SB, "SB", 1)
        M, K, N = A.shape[0], A.shape[1] * per, Bt.shape[0]
        if Bt.shape[1] * per != K:
            raise ValueError(f"problem {i}: inner dimensions differ")
        if tuple(SA.shape) != (M, K // 32) or tuple(SB.shape) != (N, K // 32):
            raise ValueError(f"problem {i}: scale tensors must be (M, K/32) and (N, K/32)")
        C = _out_for(None if outs is None else outs[i], M, N, dev)
        res.append(C)
        descs.append((M, N, K, A.data_ptr(), lda, SA.data_ptr(), ldsa, Bt.data_ptr(), ldb, SB.data_ptr(), ldsb,
                      C.data_ptr(), _ld(C)))
    h = handle if handle is not None else handle_for(dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = _native.tlg_gemm_relu_mx_grouped_variant(h.ptr, config, f, descs, s.cuda_stream)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_gemm_relu_mx_grouped")
    return res


def plan_mx(fmt, M, N, K, *, config: int = -1, lda=None, ldb=None, ldsa=None, ldsb=None, ldc=None,
            aligned: bool = True) -> dict:
    """What gemm_relu_mx would launch (host logic only). Pointers are stand-ins,
    16-byte aligned when ``aligned`` else only 2-byte aligned."""
    f = _mx_format(fmt)
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldsa = max(1, K // 32) if ldsa is None else ldsa
    ldsb = max(1, K // 32) if ldsb is None else ldsb
    ldc = max(1, N) if ldc is None else ldc
    base = 1 << 20 if aligned else (1 << 20) + 2
    st, info = _native.tlg_plan_mx(f, M, N, K, base, lda, 1 << 20, ldsa, base, ldb, 1 << 20, ldsb, base, ldc, config)
    if st != _native.TLG_SUCCESS:
        raise TlgError(st, "tlg_plan_mx")
    d = info.as_dict()
    d["variant_name"] = _native.VARIANT_NAMES.get(info.variant, "?")
    d["config_name"] = _native.tlg_plan_mx_config_name(info.config) if info.variant == TLG_VARIANT_TILED_DMA else ""
    return d
