"""Alternating attention for MI355X: Python binding of libvga.so.

Thin argument marshalling over the C ABI declared in ``include/vga.h``:
every step of the attention path runs in the library's HIP kernels; torch is
used only for device memory and the current stream.  The functions keep the
C names without the ``vga_`` prefix:

* ``frame_attn(q, k, v, frames)``  -> vga_frame_attn
* ``global_attn(q, k, v, frames)`` -> vga_global_attn
* ``sga_attn(q, k, v, frames, sga)`` -> vga_sga_attn (+ workspace)
* ``sga_attn_noalloc(q, k, v, frames, sga)`` -> vga_sga_attn_noalloc (no
  workspace argument: the library's static scratch, 64 MiB per GPU)
* ``sga_select(k, v, frames, sga)`` -> vga_sga_select (the selection,
  compaction and dropped mean alone; returns the workspace)
* ``sga_workspace_layout(frames, sga)`` -> vga_sga_workspace_layout
* ``register_attn(q, k, v, frames)`` -> vga_register_attn (+ workspace)
* ``register_workspace_layout(frames)`` -> vga_register_workspace_layout
* ``frame_attn_rows / global_attn_rows / sga_attn_rows(q_rows, k, v, frames,
  row_begin, ...)`` -> the ``vga_*_attn_rows`` row-range calls
* ``qkv_proj(x, w, b, frames)`` -> vga_qkv_proj (returns q, k, v)
* ``out_proj(o, w, b, frames)`` -> vga_out_proj
* ``layer_schedule(num_global, num_early, sga)`` -> vga_layer_schedule
* ``layer_schedule_sga(num_global, num_early, per_slot)`` -> vga_layer_schedule_sga
* ``layer_schedule_register(num_global, num_early, register_every, sga)``
  -> vga_layer_schedule_register

q, k, v: contiguous [N*L, H, 64] tensors (float32 or bfloat16) on one GPU.
The library must be built (``python alternating_attention_amd/_build.py`` or
``__graft_entry__.build()``);
importing this module without it raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# VGA_LIB_PATH loads another build of the same library (the CPU tests use it
# for the build whose host code carries AddressSanitizer and UBSan)
LIB_PATH = os.environ.get("VGA_LIB_PATH") or os.path.join(_HERE, "libvga.so")

VGA_OK = 0
STATUS_NAMES = ["VGA_OK", "VGA_ERR_NULL", "VGA_ERR_SHAPE", "VGA_ERR_DTYPE",
                "VGA_ERR_PARAM", "VGA_ERR_ALIGN", "VGA_ERR_ALIAS",
                "VGA_ERR_WORKSPACE", "VGA_ERR_UNSUPPORTED", "VGA_ERR_HIP"]
VGA_F32, VGA_BF16 = 0, 1
MODE_FRAME, MODE_GLOBAL, MODE_SGA, MODE_REGISTER = 0, 1, 2, 3

# every symbol include/vga.h declares
EXPORTS = ["vga_frame_attn", "vga_global_attn", "vga_sga_workspace_layout",
           "vga_sga_attn", "vga_register_workspace_layout", "vga_register_attn",
           "vga_layer_schedule", "vga_layer_schedule_register", "vga_layer_schedule_sga",
           "vga_frame_attn_rows", "vga_global_attn_rows", "vga_sga_attn_rows",
           "vga_sga_select", "vga_sga_attn_noalloc",
           "vga_qkv_proj", "vga_out_proj",
           "vga_status_string", "vga_last_error", "vga_abi_version"]


class VgaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s: %s" % (name, detail))


class CFrames(ctypes.Structure):
    _fields_ = [("num_frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("num_special", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class CSga(ctypes.Structure):
    _fields_ = [("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
                ("phase_h", ctypes.c_int32), ("phase_w", ctypes.c_int32),
                ("diagonal", ctypes.c_int32), ("mean_fill", ctypes.c_int32)]


class CLayer(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("sga", CSga)]


class CLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("keep_idx", "keep_mask", "kmean", "vmean", "kc", "vc", "partials", "total")] + \
               [(n, ctypes.c_int64) for n in
                ("kept_per_frame", "num_kept", "num_dropped", "partial_blocks")]


class CRegLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("qs", "ks", "vs", "os", "total")] + \
               [("num_special_rows", ctypes.c_int64)]


@dataclass(frozen=True)
class Frames:
    """N frames of a gh x gw patch grid plus S special tokens, H heads of 64."""
    num_frames: int
    grid_h: int
    grid_w: int
    num_special: int
    num_heads: int
    head_dim: int = 64
    scale: float = 0.0       # <= 0: 1/sqrt(head_dim)

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w + self.num_special

    @property
    def tokens(self) -> int:
        return self.num_frames * self.tokens_per_frame

    def c(self, dtype_code: int, tokens_per_frame: int | None = None) -> CFrames:
        ints = (self.num_frames,
                self.tokens_per_frame if tokens_per_frame is None else tokens_per_frame,
                self.grid_h, self.grid_w, self.num_special, self.num_heads, self.head_dim,
                dtype_code)
        # ctypes would wrap larger values silently
        if any(not -(1 << 31) <= int(x) < (1 << 31) for x in ints):
            raise ValueError("frame descriptor field outside int32: %r" % (ints,))
        return CFrames(*ints, self.scale)


@dataclass(frozen=True)
class Sga:
    """Subsampled Global Attention parameters (phase -1: (stride-1)//2;
    mean_fill 0 off, 1 / True count-weighted, 2 unit weight)."""
    stride_h: int = 2
    stride_w: int = 2
    phase_h: int = -1
    phase_w: int = -1
    diagonal: bool = True
    mean_fill: int = 1

    def c(self) -> CSga:
        return CSga(self.stride_h, self.stride_w, self.phase_h, self.phase_w,
                    int(self.diagonal), int(self.mean_fill))

    @classmethod
    def from_c(cls, cs: CSga) -> "Sga":
        return cls(int(cs.stride_h), int(cs.stride_w), int(cs.phase_h), int(cs.phase_w),
                   bool(cs.diagonal), int(cs.mean_fill))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libvga.so is not built (%s); run "
                          "python alternating_attention_amd/_build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    for name in ("vga_frame_attn", "vga_global_attn"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(CFrames), vp, vp, vp, vp, vp]
    lib.vga_sga_workspace_layout.restype = ctypes.c_int
    lib.vga_sga_workspace_layout.argtypes = [ctypes.POINTER(CFrames), ctypes.POINTER(CSga),
                                             ctypes.POINTER(CLayout)]
    lib.vga_sga_attn.restype = ctypes.c_int
    lib.vga_sga_attn.argtypes = [ctypes.POINTER(CFrames), ctypes.POINTER(CSga), vp, vp, vp,
                                 vp, vp, ctypes.c_size_t, vp]
    lib.vga_sga_attn_noalloc.restype = ctypes.c_int
    lib.vga_sga_attn_noalloc.argtypes = [ctypes.POINTER(CFrames), ctypes.POINTER(CSga), vp, vp,
                                         vp, vp, vp]
    lib.vga_sga_select.restype = ctypes.c_int
    lib.vga_sga_select.argtypes = [ctypes.POINTER(CFrames), ctypes.POINTER(CSga), vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.vga_layer_schedule.restype = ctypes.c_int
    lib.vga_layer_schedule.argtypes = [i32, i32, ctypes.POINTER(CSga), ctypes.POINTER(CLayer)]
    lib.vga_layer_schedule_sga.restype = ctypes.c_int
    lib.vga_layer_schedule_sga.argtypes = [i32, i32, ctypes.POINTER(CSga), ctypes.POINTER(CLayer)]
    lib.vga_layer_schedule_register.restype = ctypes.c_int
    lib.vga_layer_schedule_register.argtypes = [i32, i32, i32, ctypes.POINTER(CSga),
                                                ctypes.POINTER(CLayer)]
    lib.vga_register_workspace_layout.restype = ctypes.c_int
    lib.vga_register_workspace_layout.argtypes = [ctypes.POINTER(CFrames),
                                                  ctypes.POINTER(CRegLayout)]
    lib.vga_register_attn.restype = ctypes.c_int
    lib.vga_register_attn.argtypes = [ctypes.POINTER(CFrames), vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    i64 = ctypes.c_int64
    for name in ("vga_frame_attn_rows", "vga_global_attn_rows"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(CFrames), i64, i64, vp, vp, vp, vp, vp]
    lib.vga_sga_attn_rows.restype = ctypes.c_int
    lib.vga_sga_attn_rows.argtypes = [ctypes.POINTER(CFrames), ctypes.POINTER(CSga), i64, i64,
                                      vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.vga_qkv_proj.restype = ctypes.c_int
    lib.vga_qkv_proj.argtypes = [ctypes.POINTER(CFrames), vp, vp, vp, vp, vp, vp, vp]
    lib.vga_out_proj.restype = ctypes.c_int
    lib.vga_out_proj.argtypes = [ctypes.POINTER(CFrames), vp, vp, vp, vp, vp]
    lib.vga_status_string.restype = ctypes.c_char_p
    lib.vga_status_string.argtypes = [ctypes.c_int]
    lib.vga_last_error.restype = ctypes.c_char_p
    lib.vga_last_error.argtypes = []
    lib.vga_abi_version.restype = i32
    lib.vga_abi_version.argtypes = []
    return lib


lib = _load()


def _check(status: int):
    if status != VGA_OK:
        raise VgaError(status, lib.vga_last_error().decode())


def abi_version() -> int:
    return int(lib.vga_abi_version())


def status_string(status: int) -> str:
    return lib.vga_status_string(status).decode()


def last_error() -> str:
    return lib.vga_last_error().decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return VGA_F32
    if t.dtype == torch.bfloat16:
        return VGA_BF16
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % t.dtype)


def _check_tokens(frames: Frames, **tensors):
    """Every tensor a contiguous GPU [N*L, H, D] array, one dtype and device."""
    first = next(iter(tensors.values()))
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dtype != first.dtype or t.shape != first.shape or t.device != first.device:
            raise ValueError("%s must share dtype, shape and device" % ", ".join(tensors))
    expect = (frames.tokens, frames.num_heads, frames.head_dim)
    if tuple(first.shape) != expect:
        raise ValueError("%s shape %s != [N*L, H, D] = %s"
                         % ("/".join(tensors), tuple(first.shape), expect))


def _prepare(q, k, v, frames: Frames, out):
    import torch
    _check_tokens(frames, q=q, k=k, v=v)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous tensor like q")
    return out


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def frame_attn(q, k, v, frames: Frames, out=None):
    """Frame attention: each token attends to the L tokens of its own frame."""
    out = _prepare(q, k, v, frames, out)
    cf = frames.c(_dtype_code(q))
    _check(lib.vga_frame_attn(ctypes.byref(cf), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              out.data_ptr(), _stream(q.device)))
    return out


def global_attn(q, k, v, frames: Frames, out=None):
    """Exact global attention over all N*L tokens."""
    out = _prepare(q, k, v, frames, out)
    cf = frames.c(_dtype_code(q))
    _check(lib.vga_global_attn(ctypes.byref(cf), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               out.data_ptr(), _stream(q.device)))
    return out


def sga_workspace_layout(frames: Frames, sga: Sga, dtype_code: int = VGA_BF16) -> CLayout:
    cf = frames.c(dtype_code)
    cs = sga.c()
    lay = CLayout()
    _check(lib.vga_sga_workspace_layout(ctypes.byref(cf), ctypes.byref(cs), ctypes.byref(lay)))
    return lay


def sga_attn(q, k, v, frames: Frames, sga: Sga, out=None, workspace=None):
    """Subsampled Global Attention.  Returns (out, workspace); the workspace
    (uint8 GPU tensor) holds keep_idx, keep_mask, kmean, vmean, Kc, Vc at the
    offsets of ``sga_workspace_layout``."""
    import torch
    out = _prepare(q, k, v, frames, out)
    code = _dtype_code(q)
    lay = sga_workspace_layout(frames, sga, code)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(int(lay.total), dtype=torch.uint8, device=q.device)
    cf = frames.c(code)
    cs = sga.c()
    _check(lib.vga_sga_attn(ctypes.byref(cf), ctypes.byref(cs), q.data_ptr(), k.data_ptr(),
                            v.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), _stream(q.device)))
    return out, workspace


def sga_attn_noalloc(q, k, v, frames: Frames, sga: Sga, out=None):
    """Subsampled Global Attention with the library's static scratch as the
    workspace (nothing allocated by the call; calls that overlap on one GPU
    race).  Returns out."""
    out = _prepare(q, k, v, frames, out)
    cf = frames.c(_dtype_code(q))
    cs = sga.c()
    _check(lib.vga_sga_attn_noalloc(ctypes.byref(cf), ctypes.byref(cs), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    _stream(q.device)))
    return out


def sga_select(k, v, frames: Frames, sga: Sga, workspace=None):
    """The SGA key selection, compaction and dropped mean alone (what
    sga_attn does before its attention).  Returns the workspace, whose
    sections ``workspace_views`` reads."""
    import torch
    _check_tokens(frames, k=k, v=v)
    code = _dtype_code(k)
    lay = sga_workspace_layout(frames, sga, code)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(int(lay.total), dtype=torch.uint8, device=k.device)
    cf = frames.c(code)
    cs = sga.c()
    _check(lib.vga_sga_select(ctypes.byref(cf), ctypes.byref(cs), k.data_ptr(), v.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(k.device)))
    return workspace


def workspace_views(workspace, frames: Frames, sga: Sga, dtype_code: int = VGA_BF16):
    """Views of the SGA workspace sections (after a vga_sga_attn or
    vga_sga_select call)."""
    import torch
    lay = sga_workspace_layout(frames, sga, dtype_code)
    H, D = frames.num_heads, frames.head_dim
    nk, T = int(lay.num_kept), frames.tokens

    def sect(off, count, dt):
        nbytes = count * torch.tensor([], dtype=dt).element_size()
        return workspace[off:off + nbytes].view(dt)

    et = torch.float32 if dtype_code == VGA_F32 else torch.bfloat16
    return dict(
        keep_idx=sect(lay.keep_idx, nk, torch.int32),
        keep_mask=sect(lay.keep_mask, T, torch.uint8),
        kmean=sect(lay.kmean, H * D, torch.float32).view(H, D),
        vmean=sect(lay.vmean, H * D, torch.float32).view(H, D),
        kc=sect(lay.kc, nk * H * D, et).view(nk, H, D),
        vc=sect(lay.vc, nk * H * D, et).view(nk, H, D),
        layout=lay,
    )


def register_workspace_layout(frames: Frames, dtype_code: int = VGA_BF16) -> CRegLayout:
    cf = frames.c(dtype_code)
    lay = CRegLayout()
    _check(lib.vga_register_workspace_layout(ctypes.byref(cf), ctypes.byref(lay)))
    return lay


def register_attn(q, k, v, frames: Frames, out=None, workspace=None):
    """Register attention: special tokens attend over the special tokens of
    all frames, patch tokens over their own frame.  Returns (out, workspace)."""
    import torch
    out = _prepare(q, k, v, frames, out)
    code = _dtype_code(q)
    lay = register_workspace_layout(frames, code)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(max(int(lay.total), 1), dtype=torch.uint8, device=q.device)
    cf = frames.c(code)
    _check(lib.vga_register_attn(ctypes.byref(cf), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 _stream(q.device)))
    return out, workspace


def _prepare_rows(q_rows, k, v, frames: Frames, out):
    import torch
    for name, t in (("q_rows", q_rows), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dtype != k.dtype or t.device != k.device:
            raise ValueError("q_rows, k, v must share dtype and device")
    expect = (frames.tokens, frames.num_heads, frames.head_dim)
    if tuple(k.shape) != expect or tuple(v.shape) != expect:
        raise ValueError("k/v shape must be [N*L, H, D] = %s" % (expect,))
    if q_rows.dim() != 3 or tuple(q_rows.shape[1:]) != expect[1:]:
        raise ValueError("q_rows shape must be [R, H, D]")
    if out is None:
        out = torch.empty_like(q_rows)
    elif (out.shape != q_rows.shape or out.dtype != q_rows.dtype or not out.is_contiguous()
          or out.device != q_rows.device):
        raise ValueError("out must be a contiguous tensor like q_rows")
    return out


def frame_attn_rows(q_rows, k, v, frames: Frames, row_begin: int, out=None):
    """Frame attention for query rows [row_begin, row_begin + len(q_rows))
    (whole frames) against the full K/V."""
    out = _prepare_rows(q_rows, k, v, frames, out)
    cf = frames.c(_dtype_code(k))
    r1 = row_begin + q_rows.shape[0]
    _check(lib.vga_frame_attn_rows(ctypes.byref(cf), row_begin, r1, q_rows.data_ptr(),
                                   k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   _stream(k.device)))
    return out


def global_attn_rows(q_rows, k, v, frames: Frames, row_begin: int, out=None):
    """Exact global attention for query rows [row_begin, row_begin +
    len(q_rows)) against all N*L keys."""
    out = _prepare_rows(q_rows, k, v, frames, out)
    cf = frames.c(_dtype_code(k))
    r1 = row_begin + q_rows.shape[0]
    _check(lib.vga_global_attn_rows(ctypes.byref(cf), row_begin, r1, q_rows.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    _stream(k.device)))
    return out


def sga_attn_rows(q_rows, k, v, frames: Frames, sga: Sga, row_begin: int, out=None,
                  workspace=None):
    """SGA for query rows [row_begin, row_begin + len(q_rows)); selection and
    mean over all tokens.  Returns (out, workspace)."""
    import torch
    out = _prepare_rows(q_rows, k, v, frames, out)
    code = _dtype_code(k)
    lay = sga_workspace_layout(frames, sga, code)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(int(lay.total), dtype=torch.uint8, device=k.device)
    cf = frames.c(code)
    cs = sga.c()
    r1 = row_begin + q_rows.shape[0]
    _check(lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(cs), row_begin, r1,
                                 q_rows.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 _stream(k.device)))
    return out, workspace


def _plan(arr, n):
    """(mode, Sga or None) per slot: the SGA parameters only for SGA slots."""
    return [(int(arr[i].mode), Sga.from_c(arr[i].sga) if arr[i].mode == MODE_SGA else None)
            for i in range(n)]


def layer_schedule(num_global: int, num_early: int, sga: Sga | None):
    """Per-global-slot list of (mode, Sga or None) of the training-free
    pipeline; each entry can be passed to ``attention`` as it stands."""
    arr = (CLayer * max(num_global, 1))()
    cs = sga.c() if sga is not None else None
    _check(lib.vga_layer_schedule(num_global, num_early,
                                  ctypes.byref(cs) if cs is not None else None, arr))
    return _plan(arr, num_global)


def layer_schedule_sga(num_global: int, num_early: int, per_slot):
    """Per-slot SGA schedule: FRAME for the first num_early slots, then SGA
    with per_slot[i] (a list of num_global - num_early Sga) for slot
    num_early + i."""
    n = num_global - num_early
    arr = (CLayer * max(num_global, 1))()
    sg = (CSga * max(len(per_slot), 1))(*[p.c() for p in per_slot])
    if len(per_slot) != max(n, 0):
        raise ValueError("need %d per-slot SGA parameters, got %d" % (max(n, 0), len(per_slot)))
    _check(lib.vga_layer_schedule_sga(num_global, num_early, sg, arr))
    return _plan(arr, num_global)


def layer_schedule_register(num_global: int, num_early: int, register_every: int,
                            sga: Sga | None):
    """As layer_schedule, with every register_every-th slot (outside the early
    ones) running register attention."""
    arr = (CLayer * max(num_global, 1))()
    cs = sga.c() if sga is not None else None
    _check(lib.vga_layer_schedule_register(num_global, num_early, register_every,
                                           ctypes.byref(cs) if cs is not None else None, arr))
    return _plan(arr, num_global)


def _prepare_linear(x, w, b, frames: Frames, n_out: int):
    C = frames.num_heads * frames.head_dim
    for name, t, shape in (("x", x, (frames.tokens, C)), ("w", w, (n_out * C, C))):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
        if t.dtype != x.dtype or t.device != x.device:
            raise ValueError("x and w must share dtype and device")
        if t.numel() != shape[0] * shape[1]:
            raise ValueError("%s must hold %d x %d elements" % (name, shape[0], shape[1]))
    if b is not None and (not b.is_cuda or not b.is_contiguous() or b.dtype != x.dtype
                          or b.numel() != n_out * C):
        raise ValueError("b must be a contiguous GPU tensor of %d elements like x" % (n_out * C))
    return C


def qkv_proj(x, w, b, frames: Frames, out=None):
    """QKV projection y = x w^T + b: x [T, C] (C = 64 H), w [3C, C], b [3C]
    or None.  Returns (q, k, v), each [T, H, 64] (out: a tuple of three such
    tensors to write into)."""
    import torch
    _prepare_linear(x, w, b, frames, 3)
    shape = (frames.tokens, frames.num_heads, frames.head_dim)
    if out is None:
        out = tuple(torch.empty(shape, dtype=x.dtype, device=x.device) for _ in range(3))
    for t in out:
        if tuple(t.shape) != shape or t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError("q, k, v outputs must be contiguous [T, H, 64] like x")
    cf = frames.c(_dtype_code(x))
    _check(lib.vga_qkv_proj(ctypes.byref(cf), x.data_ptr(), w.data_ptr(),
                            None if b is None else b.data_ptr(), out[0].data_ptr(),
                            out[1].data_ptr(), out[2].data_ptr(), _stream(x.device)))
    return out


def out_proj(o, w, b, frames: Frames, out=None):
    """Output projection y = o w^T + b: o [T, H, 64] (read as [T, C]),
    w [C, C], b [C] or None.  Returns y [T, C]."""
    import torch
    C = _prepare_linear(o, w, b, frames, 1)
    if out is None:
        out = torch.empty((frames.tokens, C), dtype=o.dtype, device=o.device)
    elif out.numel() != frames.tokens * C or out.dtype != o.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, C] tensor like o")
    cf = frames.c(_dtype_code(o))
    _check(lib.vga_out_proj(ctypes.byref(cf), o.data_ptr(), w.data_ptr(),
                            None if b is None else b.data_ptr(), out.data_ptr(),
                            _stream(o.device)))
    return out


def attention(mode: int, q, k, v, frames: Frames, sga: Sga | None = None, out=None,
              workspace=None):
    """Run one layer of a schedule: ``mode`` and ``sga`` as one entry of
    ``layer_schedule*`` returns them.  Returns the output tensor; the SGA
    and register workspaces are allocated here unless passed."""
    if mode == MODE_SGA and sga is None:
        raise ValueError("an SGA layer needs its Sga parameters")
    if mode == MODE_FRAME:
        return frame_attn(q, k, v, frames, out)
    if mode == MODE_GLOBAL:
        return global_attn(q, k, v, frames, out)
    if mode == MODE_SGA:
        return sga_attn(q, k, v, frames, sga, out, workspace)[0]
    if mode == MODE_REGISTER:
        return register_attn(q, k, v, frames, out)[0]
    raise ValueError("unknown mode %r" % mode)
