"""Thin ctypes binding over libmshard.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module only checks
tensor dtypes/devices, allocates outputs with ``torch.empty`` and passes raw
device pointers plus the current HIP stream.  If the library is not built the
import fails loudly; there is no fallback.

Entry points mirror the C ABI in include/mshard.h:
  mlp_shard_fwd, mlp_shard_bwd, vocab_ce_shard_fwd, ce_combine,
  vocab_ce_shard_bwd, attn_shard_fwd, attn_shard_bwd, fingerprint, plus the
  workspace-size queries, the allocation-free vocab_ce_shard_fwd_noalloc and
  device_info.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmshard.so")

MS_OK, MS_ERR_NULL, MS_ERR_SHAPE, MS_ERR_ALIGN, MS_ERR_ALIAS, MS_ERR_WORKSPACE, MS_ERR_ENUM, MS_ERR_HIP = range(8)
STATUS_NAMES = ["MS_OK", "MS_ERR_NULL", "MS_ERR_SHAPE", "MS_ERR_ALIGN", "MS_ERR_ALIAS", "MS_ERR_WORKSPACE",
                "MS_ERR_ENUM", "MS_ERR_HIP"]
GELU = {"erf": 0, "tanh": 1}

EXPORTED = ("mlp_shard_workspace_bytes", "mlp_shard_fwd_workspace_bytes", "mlp_shard_fwd", "mlp_shard_bwd",
            "vocab_ce_workspace_bytes",
            "vocab_ce_shard_fwd", "ce_combine_workspace_bytes", "ce_combine", "vocab_ce_bwd_workspace_bytes",
            "vocab_ce_shard_bwd", "attn_shard_workspace_bytes", "attn_shard_fwd", "attn_shard_bwd",
            "ms_fingerprint_words", "ms_fingerprint", "ms_arm_kernel_events",
            "ms_last_error", "ms_version", "ms_device_info", "vocab_ce_shard_fwd_noalloc")

# ms_kernel ids: the single GEMM launches ms_arm_kernel_events can bracket
KERNELS = {"ce_gemm": 0, "fwd_h": 1, "fwd_z": 2, "bwd_dh": 3, "bwd_db": 4, "bwd_da": 5, "bwd_dx": 6,
           "ce_bwd_l": 7, "ce_bwd_dx": 8, "ce_bwd_de": 9, "attn_qkv": 10, "attn_core_fwd": 11, "attn_out": 12,
           "attn_bwd_do": 13, "attn_bwd_dwo": 14, "attn_core_bwd": 15, "attn_bwd_dwqkv": 16, "attn_bwd_dx": 17}


class MshardError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{func}: {name}: {msg}")
        self.status = status


_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m megatron_tensor_transformer_mlp_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "mlp_shard_workspace_bytes": (_sz, [_i64, _i64, _i64]),
        "mlp_shard_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64]),
        "mlp_shard_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp,
                                         _sz, _vp]),
        "mlp_shard_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp,
                                         _vp, _vp, _vp, _sz, _vp]),
        "vocab_ce_workspace_bytes": (_sz, [_i64, _i64, _i64]),
        "vocab_ce_shard_fwd": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
        "ce_combine_workspace_bytes": (_sz, [_i32, _i64]),
        "ce_combine": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz, _vp]),
        "vocab_ce_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64]),
        "vocab_ce_shard_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, ctypes.c_float, _i64, _i64, _i64,
                                              _i64, _vp, _vp, _vp, _sz, _vp]),
        "attn_shard_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
        "attn_shard_fwd": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp,
                                          _sz, _vp]),
        "attn_shard_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i32, _vp,
                                          _vp, _vp, _vp, _sz, _vp]),
        "ms_fingerprint_words": (_sz, [_sz, _sz]),
        "ms_fingerprint": (ctypes.c_int, [_vp, _sz, _sz, _vp, _vp]),
        "ms_arm_kernel_events": (ctypes.c_int, [ctypes.c_int, _vp, _vp]),
        "ms_last_error": (ctypes.c_char_p, []),
        "ms_version": (ctypes.c_char_p, []),
        "ms_device_info": (ctypes.c_int, [_i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
        "vocab_ce_shard_fwd_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def version() -> str:
    return LIB.ms_version().decode()


def device_info(device: int = 0) -> dict:
    """Compute units and peak shader clock (kHz) of a HIP device, from the runtime."""
    cus, khz = _i32(0), _i32(0)
    _check(LIB.ms_device_info(device, ctypes.byref(cus), ctypes.byref(khz)), "ms_device_info")
    return {"compute_units": cus.value, "clock_khz": khz.value}


def arm_kernel_events(kernel: str, before: Optional[torch.cuda.Event], after: Optional[torch.cuda.Event]) -> None:
    """Have the next call (on this thread) of the entry point that launches `kernel`
    record `before`/`after` on its stream around that one GEMM launch; None, None
    disarms.  The events must already exist on the device (record them once)."""
    if (before is None) != (after is None):
        raise ValueError("give both events or neither")
    handles = (None, None) if before is None else (before.cuda_event, after.cuda_event)
    if before is not None and not (handles[0] and handles[1]):
        raise ValueError("events have no device handle yet; record them once first")
    _check(LIB.ms_arm_kernel_events(KERNELS[kernel], *handles), "ms_arm_kernel_events")


def _check(status: int, func: str) -> None:
    if status != MS_OK:
        raise MshardError(status, func, LIB.ms_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# Device type every tensor must have (HIP devices are "cuda" in PyTorch-ROCm).
_DEVICE_TYPE = "cuda"


def _dev(t: torch.Tensor, name: str, dtype, shape) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _outs(out, specs, device):
    """Caller-supplied outputs: the library writes every byte of each one, so each
    must have exactly the shape and dtype it would have been allocated with, be
    contiguous and sit on the inputs' device.  ``specs`` holds (name, dtype, shape,
    optional); an optional output may be None."""
    if len(out) != len(specs):
        raise ValueError(f"out must hold {len(specs)} tensors ({', '.join(n for n, *_ in specs)})")
    for t, (name, dtype, shape, optional) in zip(out, specs):
        if t is None:
            if not optional:
                raise ValueError(f"out: {name} is required")
            continue
        _dev(t, name, dtype, shape)
        if t.device != device:
            raise ValueError(f"out: {name} is on {t.device}, the inputs on {device}")
    return out


def _same_device(device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, X on {device}: every tensor must be on one device")


def _on(device):
    """The library launches on the current device: make it the tensors' one."""
    return torch.cuda.device(device) if device.type == "cuda" else contextlib.nullcontext()


def _gelu(gelu: str) -> int:
    if gelu not in GELU:
        raise ValueError(f"gelu must be one of {sorted(GELU)} (got {gelu!r})")
    return GELU[gelu]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def mlp_shard_workspace_bytes(T: int, h: int, f_i: int) -> int:
    return int(LIB.mlp_shard_workspace_bytes(T, h, f_i))


def mlp_shard_fwd_workspace_bytes(T: int, h: int, f_i: int) -> int:
    return int(LIB.mlp_shard_fwd_workspace_bytes(T, h, f_i))


def vocab_ce_workspace_bytes(T: int, h: int, v_i: int) -> int:
    return int(LIB.vocab_ce_workspace_bytes(T, h, v_i))


def vocab_ce_bwd_workspace_bytes(T: int, h: int, v_i: int) -> int:
    return int(LIB.vocab_ce_bwd_workspace_bytes(T, h, v_i))


def ce_combine_workspace_bytes(t: int, T: int) -> int:
    return int(LIB.ce_combine_workspace_bytes(t, T))


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return given
    if given is not None:
        if (not isinstance(given, torch.Tensor) or given.device != device or not given.is_contiguous()
                or given.numel() * given.element_size() < nbytes):
            raise ValueError(f"workspace must be a contiguous tensor of >= {nbytes} bytes on {device}")
        return given
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mlp_shard_fwd(X: torch.Tensor, A_i: torch.Tensor, B_i: torch.Tensor, b1_i: Optional[torch.Tensor] = None,
                  gelu: str = "erf", out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                  workspace: Optional[torch.Tensor] = None):
    """(H_i, Y_i, Z_i) = forward of one rank's MLP shard (bf16 H, Y; fp32 partial Z).

    A workspace is allocated when the launch plan needs one and none is given
    (mlp_shard_fwd_workspace_bytes; the backward's workspace is large enough)."""
    T, h = X.shape
    f_i = A_i.shape[1]
    bf = torch.bfloat16
    _dev(X, "X", bf, (T, h)); _dev(A_i, "A_i", bf, (h, f_i)); _dev(B_i, "B_i", bf, (f_i, h))
    if b1_i is not None:
        _dev(b1_i, "b1_i", bf, (f_i,))
    _same_device(X.device, A_i=A_i, B_i=B_i, b1_i=b1_i)
    if out is None:
        H = torch.empty((T, f_i), dtype=bf, device=X.device)
        Y = torch.empty((T, f_i), dtype=bf, device=X.device)
        Z = torch.empty((T, h), dtype=torch.float32, device=X.device)
    else:
        H, Y, Z = _outs(out, (("H", bf, (T, f_i), False), ("Y", bf, (T, f_i), False),
                              ("Z", torch.float32, (T, h), False)), X.device)
    nbytes = mlp_shard_fwd_workspace_bytes(T, h, f_i)
    ws = _workspace(nbytes, X.device, workspace) if nbytes else None
    with _on(X.device):
        st = LIB.mlp_shard_fwd(_ptr(X), _ptr(A_i), _ptr(b1_i), _ptr(B_i), T, h, f_i, _gelu(gelu),
                               _ptr(H), _ptr(Y), _ptr(Z), _ptr(ws), nbytes, _stream(X.device))
    _check(st, "mlp_shard_fwd")
    return H, Y, Z


def mlp_shard_bwd(X, A_i, B_i, H_i, Y_i, dZ, gelu: str = "erf", want_db1: bool = False,
                  workspace: Optional[torch.Tensor] = None, out=None):
    """(dX_i fp32, dA_i bf16, dB_i bf16, db1_i bf16 or None) = backward of one rank's MLP shard."""
    T, h = X.shape
    f_i = A_i.shape[1]
    bf = torch.bfloat16
    for t, n, s in ((X, "X", (T, h)), (A_i, "A_i", (h, f_i)), (B_i, "B_i", (f_i, h)), (H_i, "H_i", (T, f_i)),
                    (Y_i, "Y_i", (T, f_i)), (dZ, "dZ", (T, h))):
        _dev(t, n, bf, s)
    _same_device(X.device, A_i=A_i, B_i=B_i, H_i=H_i, Y_i=Y_i, dZ=dZ)
    if out is None:
        dX = torch.empty((T, h), dtype=torch.float32, device=X.device)
        dA = torch.empty((h, f_i), dtype=bf, device=X.device)
        dB = torch.empty((f_i, h), dtype=bf, device=X.device)
        db1 = torch.empty((f_i,), dtype=bf, device=X.device) if want_db1 else None
    else:
        dX, dA, dB, db1 = _outs(out, (("dX", torch.float32, (T, h), False), ("dA", bf, (h, f_i), False),
                                      ("dB", bf, (f_i, h), False), ("db1", bf, (f_i,), True)), X.device)
    nbytes = mlp_shard_workspace_bytes(T, h, f_i)
    ws = _workspace(nbytes, X.device, workspace)
    with _on(X.device):
        st = LIB.mlp_shard_bwd(_ptr(X), _ptr(A_i), _ptr(B_i), _ptr(H_i), _ptr(Y_i), _ptr(dZ), T, h, f_i, _gelu(gelu),
                               _ptr(dX), _ptr(dA), _ptr(dB), _ptr(db1), _ptr(ws), nbytes, _stream(X.device))
    _check(st, "mlp_shard_bwd")
    return dX, dA, dB, db1


def vocab_ce_shard_fwd(X, E_i, target, vocab_start: int, workspace: Optional[torch.Tensor] = None, out=None):
    """(m_i, s_i, z_i) fp32 [T] = this rank's fused logits-GEMM + CE partials."""
    T, h = X.shape
    v_i = E_i.shape[1]
    _dev(X, "X", torch.bfloat16, (T, h)); _dev(E_i, "E_i", torch.bfloat16, (h, v_i))
    _dev(target, "target", torch.int64, (T,))
    _same_device(X.device, E_i=E_i, target=target)
    if out is None:
        m, s, z = (torch.empty((T,), dtype=torch.float32, device=X.device) for _ in range(3))
    else:
        m, s, z = _outs(out, tuple((n, torch.float32, (T,), False) for n in ("m", "s", "z")), X.device)
    nbytes = vocab_ce_workspace_bytes(T, h, v_i)
    ws = _workspace(nbytes, X.device, workspace)
    with _on(X.device):
        st = LIB.vocab_ce_shard_fwd(_ptr(X), _ptr(E_i), _ptr(target), T, h, v_i, int(vocab_start), _ptr(m), _ptr(s),
                                    _ptr(z), _ptr(ws), nbytes, _stream(X.device))
    _check(st, "vocab_ce_shard_fwd")
    return m, s, z


def vocab_ce_shard_fwd_noalloc(X, E_i, target, vocab_start: int, out):
    """vocab_ce_shard_fwd through the library's allocation-free entry point: the caller
    passes the outputs (m, s, z) fp32 [T] and no workspace; nothing is allocated."""
    T, h = X.shape
    v_i = E_i.shape[1]
    _dev(X, "X", torch.bfloat16, (T, h)); _dev(E_i, "E_i", torch.bfloat16, (h, v_i))
    _dev(target, "target", torch.int64, (T,))
    _same_device(X.device, E_i=E_i, target=target)
    m, s, z = _outs(out, tuple((n, torch.float32, (T,), False) for n in ("m", "s", "z")), X.device)
    with _on(X.device):
        st = LIB.vocab_ce_shard_fwd_noalloc(_ptr(X), _ptr(E_i), _ptr(target), T, h, v_i, int(vocab_start), _ptr(m),
                                            _ptr(s), _ptr(z), _stream(X.device))
    _check(st, "vocab_ce_shard_fwd_noalloc")
    return m, s, z


def ce_combine(m: torch.Tensor, s: torch.Tensor, z: torch.Tensor, want_mean: bool = True, out=None):
    """(loss [T] fp32, mean [1] fp32 or None) from [t, T] shard partials in rank order."""
    t, T = m.shape
    for x, n in ((m, "m"), (s, "s"), (z, "z")):
        _dev(x, n, torch.float32, (t, T))
    _same_device(m.device, s=s, z=z)
    if out is None:
        loss = torch.empty((T,), dtype=torch.float32, device=m.device)
        mean = torch.empty((1,), dtype=torch.float32, device=m.device) if want_mean else None
    else:
        loss, mean = _outs(out, (("loss", torch.float32, (T,), False), ("mean", torch.float32, (1,), True)),
                           m.device)
    with _on(m.device):
        st = LIB.ce_combine(_ptr(m), _ptr(s), _ptr(z), t, T, _ptr(loss), _ptr(mean), None, 0, _stream(m.device))
    _check(st, "ce_combine")
    return loss, mean


def vocab_ce_shard_bwd(X, E_i, target, m, s, vocab_start: int, dloss: Optional[torch.Tensor] = None,
                       grad_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None, out=None):
    """(dX_i fp32 [T, h], dE_i bf16 [h, v_i]) = backward of this rank's fused logits GEMM + CE.

    m, s: fp32 [t, T], every rank's forward partials in rank order.  The objective is
    sum_t coef[t] * loss[t] with coef = grad_scale * dloss (grad_scale alone without
    dloss); grad_scale defaults to 1/T, the gradient of the mean loss."""
    T, h = X.shape
    v_i = E_i.shape[1]
    t = m.shape[0]
    _dev(X, "X", torch.bfloat16, (T, h)); _dev(E_i, "E_i", torch.bfloat16, (h, v_i))
    _dev(target, "target", torch.int64, (T,))
    _dev(m, "m", torch.float32, (t, T)); _dev(s, "s", torch.float32, (t, T))
    if dloss is not None:
        _dev(dloss, "dloss", torch.float32, (T,))
    _same_device(X.device, E_i=E_i, target=target, m=m, s=s, dloss=dloss)
    scale = 1.0 / T if grad_scale is None else float(grad_scale)
    if out is None:
        dX = torch.empty((T, h), dtype=torch.float32, device=X.device)
        dE = torch.empty((h, v_i), dtype=torch.bfloat16, device=X.device)
    else:
        dX, dE = _outs(out, (("dX", torch.float32, (T, h), False), ("dE", torch.bfloat16, (h, v_i), False)),
                       X.device)
    nbytes = vocab_ce_bwd_workspace_bytes(T, h, v_i)
    ws = _workspace(nbytes, X.device, workspace)
    with _on(X.device):
        st = LIB.vocab_ce_shard_bwd(_ptr(X), _ptr(E_i), _ptr(target), _ptr(m), _ptr(s), t, _ptr(dloss), scale, T, h,
                                    v_i, int(vocab_start), _ptr(dX), _ptr(dE), _ptr(ws), nbytes, _stream(X.device))
    _check(st, "vocab_ce_shard_bwd")
    return dX, dE


def fingerprint_words(nbytes: int, chunk_bytes: int) -> int:
    return int(LIB.ms_fingerprint_words(nbytes, chunk_bytes))


def fingerprint(t: torch.Tensor, chunk_bytes: int = 1 << 16) -> torch.Tensor:
    """Device int64 tensor [1 + chunks]: XXH64 of the tensor's bytes as a whole
    (element 0) and per chunk of ``chunk_bytes`` (elements 1 ..), computed by the
    library on the current stream.  The tensor must be contiguous on a HIP device."""
    if not isinstance(t, torch.Tensor) or t.device.type != _DEVICE_TYPE:
        raise ValueError("fingerprint needs a tensor on a HIP device")
    if not t.is_contiguous():
        raise ValueError("fingerprint needs a contiguous tensor")
    nbytes = t.numel() * t.element_size()
    words = fingerprint_words(nbytes, chunk_bytes)
    if words == 0:
        raise ValueError(f"chunk_bytes {chunk_bytes} must be a positive multiple of 8")
    out = torch.empty(words, dtype=torch.int64, device=t.device)
    ptr = t.data_ptr() if nbytes else out.data_ptr()  # zero bytes: the address is never read
    with _on(t.device):
        _check(LIB.ms_fingerprint(ptr, nbytes, chunk_bytes, out.data_ptr(), _stream(t.device)), "ms_fingerprint")
    return out


def attn_shard_workspace_bytes(b: int, s: int, h: int, n: int, d: int) -> int:
    return int(LIB.attn_shard_workspace_bytes(b, s, h, n, d))


def attn_shard_fwd(X, Wqkv_i, Wo_i, b: int, s: int, n: int, d: int, causal: bool = True, out=None):
    """(QKV bf16 [T, 3nd], O bf16 [T, nd], lse fp32 [n, T], Z_i fp32 [T, h]) = forward of one
    rank's self-attention shard over b sequences of s tokens (T = b*s), n heads of size d."""
    T, h = X.shape
    nd = n * d
    if T != b * s:
        raise ValueError(f"X has {T} rows, expected b*s = {b * s}")
    bf = torch.bfloat16
    _dev(X, "X", bf, (T, h)); _dev(Wqkv_i, "Wqkv_i", bf, (h, 3 * nd)); _dev(Wo_i, "Wo_i", bf, (nd, h))
    _same_device(X.device, Wqkv_i=Wqkv_i, Wo_i=Wo_i)
    if out is None:
        QKV = torch.empty((T, 3 * nd), dtype=bf, device=X.device)
        O = torch.empty((T, nd), dtype=bf, device=X.device)
        lse = torch.empty((n, T), dtype=torch.float32, device=X.device)
        Z = torch.empty((T, h), dtype=torch.float32, device=X.device)
    else:
        QKV, O, lse, Z = _outs(out, (("QKV", bf, (T, 3 * nd), False), ("O", bf, (T, nd), False),
                                     ("lse", torch.float32, (n, T), False), ("Z", torch.float32, (T, h), False)),
                               X.device)
    with _on(X.device):
        st = LIB.attn_shard_fwd(_ptr(X), _ptr(Wqkv_i), _ptr(Wo_i), b, s, h, n, d, int(bool(causal)), _ptr(QKV), _ptr(O),
                                _ptr(lse), _ptr(Z), None, 0, _stream(X.device))
    _check(st, "attn_shard_fwd")
    return QKV, O, lse, Z


def attn_shard_bwd(X, Wqkv_i, Wo_i, QKV, O, lse, dZ, b: int, s: int, n: int, d: int, causal: bool = True,
                   workspace: Optional[torch.Tensor] = None, out=None):
    """(dX_i fp32 [T, h], dWqkv_i bf16 [h, 3nd], dWo_i bf16 [nd, h]) = backward of attn_shard_fwd."""
    T, h = X.shape
    nd = n * d
    if T != b * s:
        raise ValueError(f"X has {T} rows, expected b*s = {b * s}")
    bf = torch.bfloat16
    for t, nm, shp, dt in ((X, "X", (T, h), bf), (Wqkv_i, "Wqkv_i", (h, 3 * nd), bf), (Wo_i, "Wo_i", (nd, h), bf),
                           (QKV, "QKV", (T, 3 * nd), bf), (O, "O", (T, nd), bf), (lse, "lse", (n, T), torch.float32),
                           (dZ, "dZ", (T, h), bf)):
        _dev(t, nm, dt, shp)
    _same_device(X.device, Wqkv_i=Wqkv_i, Wo_i=Wo_i, QKV=QKV, O=O, lse=lse, dZ=dZ)
    if out is None:
        dX = torch.empty((T, h), dtype=torch.float32, device=X.device)
        dWqkv = torch.empty((h, 3 * nd), dtype=bf, device=X.device)
        dWo = torch.empty((nd, h), dtype=bf, device=X.device)
    else:
        dX, dWqkv, dWo = _outs(out, (("dX", torch.float32, (T, h), False), ("dWqkv", bf, (h, 3 * nd), False),
                                     ("dWo", bf, (nd, h), False)), X.device)
    nbytes = attn_shard_workspace_bytes(b, s, h, n, d)
    ws = _workspace(nbytes, X.device, workspace)
    with _on(X.device):
        st = LIB.attn_shard_bwd(_ptr(X), _ptr(Wqkv_i), _ptr(Wo_i), _ptr(QKV), _ptr(O), _ptr(lse), _ptr(dZ), b, s, h, n,
                                d, int(bool(causal)), _ptr(dX), _ptr(dWqkv), _ptr(dWo), _ptr(ws), nbytes,
                                _stream(X.device))
    _check(st, "attn_shard_bwd")
    return dX, dWqkv, dWo
