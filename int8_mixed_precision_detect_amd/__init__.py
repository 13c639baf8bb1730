"""LLM.int8() mixed-precision linear layer for MI355X (gfx950).

A thin binding over libi8mm's C ABI (include/i8mm.h): it checks tensor
dtypes, devices and contiguity, allocates outputs and the workspace with
torch, and passes raw device pointers and torch's current HIP stream.  All
arithmetic happens in the library's HIP kernels; there is no CPU path.

The method (Hugging Face LLM.int8() summary, section "LLM.int8() の核心アイデア"):
outlier hidden dims (columns of X with some |x| >= threshold) are multiplied
in fp16, the rest is absmax-quantized to int8 (per row of X, per output
channel of W) and multiplied with int32 accumulation, then dequantized and
summed with the fp16 part.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import NOALLOC_SCRATCH_BYTES, I8mmError, WsLayout, check, lib

__all__ = [
    "I8mmError", "quantize_weight", "linear_forward", "linear_forward_fp16w", "weight_rowsum",
    "linear_forward_zeropoint", "linear_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "workspace_layout", "workspace_size", "alloc_workspace", "init_workspace", "shared_workspace",
    "linear_status",
    "find_outliers", "quantize_rows", "outlier_weights", "gemm_s32", "profile_enable",
    "profile_read", "set_split_override", "set_tile_override", "set_row_prep",
    "Int8Linear",
]

DEFAULT_THRESHOLD = 6.0


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_weight(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp16 W [N,K] -> (CB int8 [N,K], SCB fp32 [N]) with W ~= CB*SCB/127."""
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    CB = torch.empty((N, K), dtype=torch.int8, device=W.device)
    SCB = torch.empty((N,), dtype=torch.float32, device=W.device)
    check("int8_quantize_weight",
          lib().int8_quantize_weight(_ptr(W), N, K, _ptr(CB), _ptr(SCB), _stream(W)))
    return CB, SCB


def workspace_layout(T: int, N: int, K: int, max_outliers: Optional[int] = None) -> dict:
    mo = K if max_outliers is None else max_outliers
    L = WsLayout()
    check("int8_linear_workspace_layout",
          lib().int8_linear_workspace_layout(T, N, K, mo, ctypes.byref(L)))
    return {f: getattr(L, f) for f, _ in WsLayout._fields_}


def workspace_size(T: int, N: int, K: int, max_outliers: Optional[int] = None) -> int:
    return workspace_layout(T, N, K, max_outliers)["total"]


def alloc_workspace(T: int, N: int, K: int, max_outliers: Optional[int] = None,
                    device="cuda") -> torch.Tensor:
    """A uint8 device buffer big enough for a forward call of this shape,
    initialized (``int8_linear_workspace_init``) on the current stream."""
    mo = K if max_outliers is None else max_outliers
    ws = torch.empty(max(workspace_size(T, N, K, mo), 256), dtype=torch.uint8, device=device)
    init_workspace(ws, T, N, K, mo)
    return ws


# One workspace per (device, stream), shared by every Int8Linear: calls on
# one stream never overlap, the mask sits at the same place for every shape
# and forwards leave it zero, so layers of different shapes take turns on it.
# It grows to the largest call seen and is initialized when (re)allocated.
_SHARED_WS: dict = {}


def shared_workspace(T: int, N: int, K: int, max_outliers: Optional[int] = None,
                     device=None) -> torch.Tensor:
    """The workspace of the current stream on `device`, at least large enough
    for this shape (see ``Int8Linear``)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    stream = torch.cuda.current_stream(device)
    key = (device.index, stream.cuda_stream)
    need = max(workspace_size(T, N, K, max_outliers), 256)
    ws = _SHARED_WS.get(key)
    if ws is None or ws.numel() < need:
        _SHARED_WS.pop(key, None)
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        with torch.cuda.stream(stream):
            init_workspace(ws, T, N, K, max_outliers)
        _SHARED_WS[key] = ws
    return ws


def init_workspace(ws: torch.Tensor, T: int, N: int, K: int,
                   max_outliers: Optional[int] = None) -> None:
    """Zero the head of a workspace (counts and mask) before its first
    forward; forwards, of any shape, leave it ready for the next one."""
    mo = K if max_outliers is None else max_outliers
    check("int8_linear_workspace_init",
          lib().int8_linear_workspace_init(_ptr(ws), T, N, K, mo, _stream(ws)))


def linear_forward(X: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor,
                   bias: Optional[torch.Tensor] = None, threshold: float = DEFAULT_THRESHOLD,
                   max_outliers: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, check_overflow: bool = False) -> torch.Tensor:
    """Y fp16 [T,N] = the LLM.int8() product of X fp16 [T,K] with (CB, SCB), plus bias.

    max_outliers (default K, always enough) sizes the outlier list and the
    Wo / Xo regions of the workspace.  If X has more outlier columns than
    that, Y is undefined and the workspace's status says so
    (``linear_status``); with ``check_overflow=True`` this call reads the
    status (a synchronization) and raises ``I8mmError`` in that case."""
    _need(X, "X", torch.float16, 2)
    _need(CB, "CB", torch.int8, 2)
    _need(SCB, "SCB", torch.float32, 1)
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape[0] != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} CB {tuple(CB.shape)} "
                         f"SCB {tuple(SCB.shape)}")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must have N elements")
    mo = K if max_outliers is None else max_outliers
    if workspace is None:
        workspace = alloc_workspace(T, N, K, mo, X.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (T, N):
            raise ValueError("out must be [T, N]")
    check("int8_linear_forward",
          lib().int8_linear_forward(_ptr(X), T, K, _ptr(CB), _ptr(SCB), N, _ptr(bias),
                                    float(threshold), _ptr(out), _ptr(workspace),
                                    workspace.numel(), mo, _stream(X)))
    if check_overflow:
        code, _ = linear_status(workspace)
        check("int8_linear_forward", code)
    return out


def linear_forward_noalloc(X: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor,
                           bias: Optional[torch.Tensor] = None,
                           threshold: float = DEFAULT_THRESHOLD, max_outliers: int = 256,
                           out: Optional[torch.Tensor] = None,
                           status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """linear_forward on the library's per-GPU scratch array instead of a
    workspace (int8_linear_forward_noalloc): the call allocates nothing when
    `out` is given.  `status` (int32 [4] on the device, optional) receives
    [outlier columns found, overflow flag, 0, 0].  Calls that overlap on one
    GPU race; max_outliers bounds the scratch use (I8MM_ERR_WORKSPACE past
    NOALLOC_SCRATCH_BYTES)."""
    _need(X, "X", torch.float16, 2)
    _need(CB, "CB", torch.int8, 2)
    _need(SCB, "SCB", torch.float32, 1)
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape[0] != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} CB {tuple(CB.shape)} "
                         f"SCB {tuple(SCB.shape)}")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (T, N):
            raise ValueError("out must be [T, N]")
    if status is not None:
        _need(status, "status", torch.int32, 1)
        if status.numel() < 4:
            raise ValueError("status must hold 4 int32")
    check("int8_linear_forward_noalloc",
          lib().int8_linear_forward_noalloc(_ptr(X), T, K, _ptr(CB), _ptr(SCB), N, _ptr(bias),
                                            float(threshold), _ptr(out), int(max_outliers),
                                            _ptr(status), _stream(X)))
    return out


def linear_forward_fp16w(X: torch.Tensor, W: torch.Tensor, bias: Optional[torch.Tensor] = None,
                         threshold: float = DEFAULT_THRESHOLD, max_outliers: Optional[int] = None,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None,
                         CB: Optional[torch.Tensor] = None, SCB: Optional[torch.Tensor] = None):
    """The layer with the fp16 weight W [N,K] kept: W is quantized on every call
    (into CB/SCB, allocated when not given) and the outlier weight dims are
    W[:, O] itself.  Returns (Y, CB, SCB)."""
    _need(X, "X", torch.float16, 2)
    _need(W, "W", torch.float16, 2)
    T, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} W {tuple(W.shape)}")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must have N elements")
    if CB is None:
        CB = torch.empty((N, K), dtype=torch.int8, device=X.device)
    if SCB is None:
        SCB = torch.empty((N,), dtype=torch.float32, device=X.device)
    _need(CB, "CB", torch.int8, 2)
    _need(SCB, "SCB", torch.float32, 1)
    if tuple(CB.shape) != (N, K) or SCB.shape[0] != N:
        raise ValueError("CB must be [N, K] and SCB [N]")
    mo = K if max_outliers is None else max_outliers
    if workspace is None:
        workspace = alloc_workspace(T, N, K, mo, X.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (T, N):
            raise ValueError("out must be [T, N]")
    check("int8_linear_forward_fp16w",
          lib().int8_linear_forward_fp16w(_ptr(X), T, K, _ptr(W), N, _ptr(bias), float(threshold),
                                          _ptr(CB), _ptr(SCB), _ptr(out), _ptr(workspace),
                                          workspace.numel(), mo, _stream(X)))
    return out, CB, SCB


def weight_rowsum(CB: torch.Tensor) -> torch.Tensor:
    """int32 [N] row sums of CB (once per weight, for the zero-point layer)."""
    _need(CB, "CB", torch.int8, 2)
    N, K = CB.shape
    out = torch.empty((N,), dtype=torch.int32, device=CB.device)
    check("int8_weight_rowsum", lib().int8_weight_rowsum(_ptr(CB), N, K, _ptr(out), _stream(CB)))
    return out


def linear_forward_zeropoint(X: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor,
                             rsum: torch.Tensor, bias: Optional[torch.Tensor] = None,
                             threshold: float = DEFAULT_THRESHOLD,
                             max_outliers: Optional[int] = None,
                             workspace: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer with zero-point (asymmetric) row quantization of X; rsum from
    ``weight_rowsum(CB)``."""
    _need(X, "X", torch.float16, 2)
    _need(CB, "CB", torch.int8, 2)
    _need(SCB, "SCB", torch.float32, 1)
    _need(rsum, "rsum", torch.int32, 1)
    T, K = X.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape[0] != N or rsum.shape[0] != N:
        raise ValueError("shape mismatch")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias must have N elements")
    mo = K if max_outliers is None else max_outliers
    if workspace is None:
        workspace = alloc_workspace(T, N, K, mo, X.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    else:
        _need(out, "out", torch.float16, 2)
        if tuple(out.shape) != (T, N):
            raise ValueError("out must be [T, N]")
    check("int8_linear_forward_zeropoint",
          lib().int8_linear_forward_zeropoint(_ptr(X), T, K, _ptr(CB), _ptr(SCB), _ptr(rsum), N,
                                              _ptr(bias), float(threshold), _ptr(out),
                                              _ptr(workspace), workspace.numel(), mo, _stream(X)))
    return out


def linear_status(workspace: torch.Tensor) -> Tuple[int, int]:
    """(status code, n_outliers) of the last forward call on this workspace (syncs)."""
    n = ctypes.c_int32(0)
    code = lib().int8_linear_status(_ptr(workspace), ctypes.byref(n), _stream(workspace))
    return code, n.value


def find_outliers(X: torch.Tensor, threshold: float = DEFAULT_THRESHOLD,
                  max_outliers: Optional[int] = None):
    """Step 1 alone: (O int32 [max_outliers], counts int32 [4], mask uint32-as-int32)."""
    _need(X, "X", torch.float16, 2)
    T, K = X.shape
    mo = K if max_outliers is None else max_outliers
    O = torch.empty(max(mo, 1), dtype=torch.int32, device=X.device)
    counts = torch.empty(4, dtype=torch.int32, device=X.device)
    mask = torch.empty(max((K + 31) // 32, 1), dtype=torch.int32, device=X.device)
    check("int8_find_outliers",
          lib().int8_find_outliers(_ptr(X), T, K, float(threshold), _ptr(O), _ptr(counts),
                                   _ptr(mask), mo, _stream(X)))
    return O, counts, mask


def quantize_rows(X: torch.Tensor, mask: torch.Tensor, max_outliers: int,
                  ldq: Optional[int] = None, ldo: Optional[int] = None):
    """Step 2, activation side, for an outlier bit mask (uint32 words, int32 tensor):
    (Xq int8 [T,ldq], sx fp32 [T], Xo fp16 [T,ldo])."""
    _need(X, "X", torch.float16, 2)
    T, K = X.shape
    ldq = ((K + 63) // 64) * 64 if ldq is None else ldq
    ldo = max(((max_outliers + 31) // 32) * 32, 32) if ldo is None else ldo
    Xq = torch.empty((T, ldq), dtype=torch.int8, device=X.device)
    sx = torch.empty(T, dtype=torch.float32, device=X.device)
    Xo = torch.empty((T, ldo), dtype=torch.float16, device=X.device)
    check("int8_quantize_rows",
          lib().int8_quantize_rows(_ptr(X), T, K, _ptr(mask), max_outliers, _ptr(Xq), ldq,
                                   _ptr(sx), _ptr(Xo), ldo, _stream(X)))
    return Xq, sx, Xo


def outlier_weights(CB: torch.Tensor, SCB: torch.Tensor, mask: torch.Tensor,
                    max_outliers: int, ldo: Optional[int] = None) -> torch.Tensor:
    """Step 2, weight side: Wo fp16 [N, ldo] = fp16(CB[:, O] * SCB / 127), zero-padded."""
    _need(CB, "CB", torch.int8, 2)
    N, K = CB.shape
    ldo = max(((max_outliers + 31) // 32) * 32, 32) if ldo is None else ldo
    Wo = torch.empty((N, ldo), dtype=torch.float16, device=CB.device)
    check("int8_outlier_weights",
          lib().int8_outlier_weights(_ptr(CB), _ptr(SCB), N, K, _ptr(mask), max_outliers,
                                     _ptr(Wo), ldo, _stream(CB)))
    return Wo


def gemm_s32(A: torch.Tensor, B: torch.Tensor, K: Optional[int] = None) -> torch.Tensor:
    """C int32 [T,N] = A int8 [T,>=K] . B int8 [N,>=K]^T over the first K columns."""
    _need(A, "A", torch.int8, 2)
    _need(B, "B", torch.int8, 2)
    T, N = A.shape[0], B.shape[0]
    K = A.shape[1] if K is None else K
    C = torch.empty((T, N), dtype=torch.int32, device=A.device)
    check("int8_gemm_s32",
          lib().int8_gemm_s32(_ptr(A), A.shape[1], _ptr(B), B.shape[1], _ptr(C), T, N, K,
                              _stream(A)))
    return C


def set_tile_override(cfg: int = -1) -> None:
    """Output tile of the product at T > 32 (0: 320 x 256, 1: 256 x 256,
    2: 192 x 256, 3: 320 x 128); -1 = the library's choice.  Process-wide; size workspaces
    under the same setting."""
    check("i8mm_set_tile_override", lib().i8mm_set_tile_override(int(cfg)))


def set_row_prep(enable: bool = True) -> None:
    """Forwards of one to eight tokens of the absmax layer take steps 1-2
    from one launch of a workgroup per row (the default) or from the
    detection and step-2 launches.
    Process-wide; the workspace holds the same values either way, and Y too
    for outlier sets of up to 128 columns."""
    check("i8mm_set_row_prep", lib().i8mm_set_row_prep(1 if enable else 0))


def set_split_override(splits: int = 0) -> None:
    """Workgroups per output tile of the product at T > 32 (split K); 0 = the
    library's choice.  Process-wide; size workspaces under the same setting."""
    check("i8mm_set_split_override", lib().i8mm_set_split_override(int(splits)))


def profile_enable(on: bool = True) -> None:
    check("i8mm_profile_enable", lib().i8mm_profile_enable(1 if on else 0))


def profile_read():
    """(ms per stage summed [detect, quantize, product, whole], calls timed)."""
    ms = (ctypes.c_double * 4)()
    calls = (ctypes.c_int64 * 4)()
    check("i8mm_profile_read", lib().i8mm_profile_read(ms, calls))
    return list(ms), int(calls[3])


class Int8Linear(torch.nn.Module):
    """``torch.nn.Linear`` in LLM.int8() form: the interface of the pages'
    ``Linear8bitLt(in_features, out_features, bias, has_fp16_weights,
    threshold)`` ("transformers への統合" and "accelerate を使ったゼロメモリモデル
    構築" sections of the Hugging Face summary).

    Life cycle, as there: build it, load an fp16 ``nn.Linear`` state dict
    (``weight``, ``bias``), move it to the GPU -- the move quantizes the weight
    into ``CB`` (int8 [out, in]) and ``SCB`` (fp32 [out]).  With
    ``has_fp16_weights=False`` the fp16 weight is dropped then; the state dict
    holds ``CB``, ``SCB`` and ``bias`` and loads back without quantizing again
    (the int8 form persists).  With ``has_fp16_weights=True`` the fp16 weight
    stays and every call quantizes it (``linear_forward_fp16w``).  Inputs are
    fp16 ``[..., in_features]``; the product runs on the GPU only.

    Memory: a module holds CB, SCB and bias (about half the fp16 weight);
    the intermediate results of a call go to one workspace per (device,
    stream) shared by all modules (``shared_workspace``), sized for the
    largest call, with room for every column to be an outlier.  ``.half()``
    and ``.to(dtype)`` leave CB int8 and SCB fp32."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 has_fp16_weights: bool = False, threshold: float = DEFAULT_THRESHOLD,
                 device=None):
        super().__init__()
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.has_fp16_weights = bool(has_fp16_weights)
        self.threshold = float(threshold)
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=torch.float16, device=device),
            requires_grad=False)
        if bias:
            self.bias = torch.nn.Parameter(
                torch.zeros(out_features, dtype=torch.float16, device=device), requires_grad=False)
        else:
            self.register_parameter("bias", None)
        # the int8 form (persistent once made); scratch CB/SCB of the fp16 form
        self.register_buffer("CB", None)
        self.register_buffer("SCB", None)
        self._cb_scratch = None
        self._scb_scratch = None

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, has_fp16_weights: bool = False,
                    threshold: float = DEFAULT_THRESHOLD) -> "Int8Linear":
        m = cls(linear.in_features, linear.out_features, linear.bias is not None,
                has_fp16_weights, threshold, device=linear.weight.device)
        m.load_state_dict({k: v.to(torch.float16) for k, v in linear.state_dict().items()})
        return m

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, has_fp16_weights={self.has_fp16_weights}, "
                f"threshold={self.threshold}, quantized={self.CB is not None}")

    def _quantize_if_on_gpu(self) -> None:
        w = self.weight
        if w is None or not w.is_cuda:
            return
        if self.has_fp16_weights:
            return  # quantized on every call
        self.CB, self.SCB = quantize_weight(w.detach().to(torch.float16).contiguous())
        self.weight = None  # the int8 form replaces it

    def _apply(self, fn, recurse=True):
        # CB (int8) and SCB (fp32) keep their dtypes under .half() / .to(dtype):
        # they follow the module's device only (a cast would lose the scales)
        cb, scb = self.CB, self.SCB
        self._buffers["CB"], self._buffers["SCB"] = None, None
        super()._apply(fn, recurse)
        if cb is not None:
            dev = fn(torch.empty(0, device=cb.device)).device
            self._buffers["CB"] = cb.to(dev)
            self._buffers["SCB"] = scb.to(device=dev, dtype=torch.float32)
        self._cb_scratch, self._scb_scratch = None, None
        self._quantize_if_on_gpu()
        return self

    def _load_from_state_dict(self, state_dict, prefix, local_metadata, strict, missing_keys,
                              unexpected_keys, error_msgs):
        cb, scb = state_dict.get(prefix + "CB"), state_dict.get(prefix + "SCB")
        if cb is not None and scb is not None:
            # the int8 form: no fp16 weight to load
            dev = self.bias.device if self.bias is not None else cb.device
            self.CB = cb.to(device=dev, dtype=torch.int8).contiguous()
            self.SCB = scb.to(device=dev, dtype=torch.float32).contiguous()
            self.weight = None
            if self.bias is not None and prefix + "bias" in state_dict:
                with torch.no_grad():
                    self.bias.copy_(state_dict[prefix + "bias"].to(torch.float16))
            elif self.bias is not None:
                missing_keys.append(prefix + "bias")
            return
        if self.weight is None and prefix + "weight" in state_dict:
            self.weight = torch.nn.Parameter(
                torch.empty((self.out_features, self.in_features), dtype=torch.float16,
                            device=self.CB.device if self.CB is not None else None),
                requires_grad=False)
            self.CB, self.SCB = None, None
        super()._load_from_state_dict(state_dict, prefix, local_metadata, strict, missing_keys,
                                      unexpected_keys, error_msgs)
        self._quantize_if_on_gpu()

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not x.is_cuda:
            raise RuntimeError("Int8Linear runs on the GPU only; move the module and the input")
        lead = x.shape[:-1]
        X = x.reshape(-1, self.in_features).to(torch.float16).contiguous()
        T = X.shape[0]
        ws = shared_workspace(T, self.out_features, self.in_features, None, X.device)
        bias = None if self.bias is None else self.bias.to(torch.float16).contiguous()
        if self.has_fp16_weights:
            if self.weight is None or not self.weight.is_cuda:
                raise RuntimeError("the fp16 weight must be on the GPU")
            Y, self._cb_scratch, self._scb_scratch = linear_forward_fp16w(
                X, self.weight.to(torch.float16).contiguous(), bias, self.threshold,
                workspace=ws, CB=self._cb_scratch, SCB=self._scb_scratch)
        else:
            if self.CB is None:
                raise RuntimeError("the weight is not quantized yet; move the module to the GPU")
            Y = linear_forward(X, self.CB, self.SCB, bias, self.threshold, workspace=ws)
        return Y.reshape(*lead, self.out_features)
