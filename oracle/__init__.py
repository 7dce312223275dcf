"""fp64 CPU oracle for alternating attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  It shares no code with the HIP library
(``alternating_attention_amd``) and never imports it.

Two independent implementations of the same definitions live here:

* ``vga_oracle.c`` (plain C, fp64, OpenMP over (row, head)), loaded with
  ctypes -- explicit column lists and a max-shifted softmax per row;
* ``brute.py`` (numpy, fp64) -- the whole logit matrix with a mask and an
  augmented mean column, for tiny inputs.

What is computed follows the pages:

* "VGGT CVPR25 Best Paper" notes, section "Alternating-Attention": frame-wise
  self-attention, then global self-attention over every token of every frame.
* "AVGGT: Rethinking Global Attention for Accelerating VGGT", technical summary,
  section 3 (Methodology): early global layers become frame attention; the
  rest run Subsampled Global Attention (all queries kept; K/V on a strided
  patch grid; the diagonal kept; dropped columns replaced by one global mean;
  one shared softmax over the three parts).
* "VGGT-Omega" notes, section 2 (Register Attention) and architecture section
  2.3: in a register-attention layer only the per-frame register and camera
  tokens exchange information across frames; image tokens stay in their frame.
* The projections around an attention layer (QKV before, output after), which
  the pages do not spell out, read as plain nn.Linear-style layers
  y = x W^T + b (``linear``, ``qkv_proj``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vga_oracle.c")
# VGA_ORACLE_LIB loads another build of vga_oracle.c (the sanitizer build
# of build_sanitized, in the CPU tests)
_LIB_PATH = os.environ.get("VGA_ORACLE_LIB") or os.path.join(_HERE, "libvga_oracle.so")

MODE_FRAME, MODE_GLOBAL, MODE_SGA, MODE_REGISTER = 0, 1, 2, 3
_F32, _BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile vga_oracle.c with gcc into libvga_oracle.so (in-tree)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out: str) -> str:
    """vga_oracle.c with gcc's AddressSanitizer and UBSan into `out`; the
    loading process must preload gcc's libasan (sanitizer_runtime())."""
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def sanitizer_runtime() -> str:
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, dbl, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.vgao_select.restype = i64
    lib.vgao_select.argtypes = [i32] * 8 + [vp, vp]
    lib.vgao_dropped_mean.restype = i64
    lib.vgao_dropped_mean.argtypes = [i32] * 7 + [vp, vp] + [i32] * 4 + [vp, vp]
    lib.vgao_attention.restype = ctypes.c_int
    lib.vgao_attention.argtypes = ([i32] * 8 + [dbl, vp, vp, vp] + [i32] * 6
                                   + [vp, i64, vp, i32])
    lib.vgao_schedule.restype = ctypes.c_int
    lib.vgao_schedule.argtypes = [i32, i32, i32, vp]
    lib.vgao_schedule_register.restype = ctypes.c_int
    lib.vgao_schedule_register.argtypes = [i32, i32, i32, i32, vp]
    lib.vgao_max_threads.restype = i32
    lib.vgao_max_threads.argtypes = []
    lib.vgao_linear.restype = ctypes.c_int
    lib.vgao_linear.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, i32]
    lib.vgao_qkv_proj.restype = ctypes.c_int
    lib.vgao_qkv_proj.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, i32]
    _lib = lib
    return lib


def _elements(x: np.ndarray):
    """(contiguous array, dtype code): float32 as is, bf16 as raw uint16 bits."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), _F32
    if x.dtype in (np.uint16, np.int16):
        return np.ascontiguousarray(x).view(np.uint16), _BF16
    raise TypeError("oracle inputs are float32 or bf16 bits (uint16), got %s" % x.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def select(N, L, gh, gw, sh, sw, oh, ow):
    """SGA key selection: (keep_idx int64[N*kpf], keep_mask uint8[N*L])."""
    lib = _load()
    T = N * L
    idx = np.empty(T, dtype=np.int64)
    mask = np.empty(T, dtype=np.uint8)
    n = lib.vgao_select(N, L, gh, gw, sh, sw, oh, ow, _ptr(idx), _ptr(mask))
    return idx[:n].copy(), mask


def dropped_mean(k, v, N, L, gh, gw, sh, sw, oh, ow):
    """(kmean [H,d] fp64, vmean [H,d] fp64, |D|) over the SGA-dropped tokens."""
    lib = _load()
    kk, dt = _elements(k)
    vv, dt2 = _elements(v)
    assert dt == dt2 and kk.shape == vv.shape and kk.ndim == 3
    _, H, d = kk.shape
    km = np.zeros((H, d))
    vm = np.zeros((H, d))
    nd = lib.vgao_dropped_mean(N, L, gh, gw, H, d, dt, _ptr(kk), _ptr(vv),
                               sh, sw, oh, ow, _ptr(km), _ptr(vm))
    return km, vm, int(nd)


def attention(mode, q, k, v, N, L, gh, gw, scale, sga=None, rows=None, threads=0):
    """fp64 attention output [len(rows) or T, H, d] for mode
    FRAME/GLOBAL/SGA/REGISTER.

    q, k, v: [T, H, d] float32, or bf16 given as uint16 bits.
    sga: dict(stride_h, stride_w, phase_h, phase_w, diagonal, mean_fill);
    mean_fill 1 is count-weighted, 2 unit-weight."""
    lib = _load()
    qq, dt = _elements(q)
    kk, dtk = _elements(k)
    vv, dtv = _elements(v)
    assert dt == dtk == dtv and qq.shape == kk.shape == vv.shape and qq.ndim == 3
    T, H, d = qq.shape
    assert T == N * L
    s = sga or {}
    if mode == MODE_SGA and not sga:
        raise ValueError("SGA mode needs sga parameters")
    if rows is None:
        rr, nrows, rp = None, T, None
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows, rp = rr.shape[0], _ptr(rr)
    out = np.empty((nrows, H, d), dtype=np.float64)
    rc = lib.vgao_attention(mode, N, L, gh, gw, H, d, dt, float(scale),
                            _ptr(qq), _ptr(kk), _ptr(vv),
                            s.get("stride_h", 1), s.get("stride_w", 1),
                            s.get("phase_h", 0), s.get("phase_w", 0),
                            s.get("diagonal", 0), s.get("mean_fill", 0),
                            rp, nrows, _ptr(out), threads)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def linear(x, w, b=None, threads=0):
    """fp64 y = x W^T + b for x [M, K], w [N, K] (output feature n in row n)
    and b [N] or None, all float32 or all bf16 bits: the projections around
    an attention layer, read as plain nn.Linear-style layers."""
    lib = _load()
    xx, dt = _elements(x)
    ww, dtw = _elements(w)
    assert xx.ndim == 2 and ww.ndim == 2 and xx.shape[1] == ww.shape[1] and dt == dtw
    bp = None
    if b is not None:
        bb, dtb = _elements(b)
        assert dtb == dt and bb.shape == (ww.shape[0],)
        bp = _ptr(bb)
    M, K = xx.shape
    N = ww.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    if lib.vgao_linear(M, K, N, dt, _ptr(xx), _ptr(ww), bp, _ptr(y), threads) != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def qkv_proj(x, w, b, H, threads=0):
    """(q, k, v), each fp64 [M, H, 64], of the QKV projection: y = x W^T + b
    with x [M, 64H], w [3*64H, 64H] and b [3*64H] or None; output features
    [0, C), [C, 2C) and [2C, 3C) (C = 64H) are q, k and v."""
    lib = _load()
    xx, dt = _elements(x)
    ww, dtw = _elements(w)
    C = 64 * H
    assert xx.ndim == 2 and xx.shape[1] == C and ww.shape == (3 * C, C) and dt == dtw
    bp = None
    if b is not None:
        bb, dtb = _elements(b)
        assert dtb == dt and bb.shape == (3 * C,)
        bp = _ptr(bb)
    M = xx.shape[0]
    q, k, v = (np.empty((M, H, 64), dtype=np.float64) for _ in range(3))
    if lib.vgao_qkv_proj(M, H, dt, _ptr(xx), _ptr(ww), bp, _ptr(q), _ptr(k), _ptr(v),
                         threads) != 0:
        raise ValueError("oracle rejected the arguments")
    return q, k, v


def schedule(num_global, num_early, use_sga):
    """Per-global-slot modes (MODE_FRAME / MODE_GLOBAL / MODE_SGA)."""
    lib = _load()
    out = np.empty(max(num_global, 0), dtype=np.int32)
    if lib.vgao_schedule(num_global, num_early, int(bool(use_sga)), _ptr(out)) != 0:
        raise ValueError("num_early must lie in [0, num_global]")
    return out


def schedule_register(num_global, num_early, register_every, use_sga):
    """As schedule(), with every register_every-th slot (counted from slot 0,
    outside the early ones) running MODE_REGISTER."""
    lib = _load()
    out = np.empty(max(num_global, 0), dtype=np.int32)
    if lib.vgao_schedule_register(num_global, num_early, register_every,
                                  int(bool(use_sga)), _ptr(out)) != 0:
        raise ValueError("bad schedule arguments")
    return out


def max_threads() -> int:
    return int(_load().vgao_max_threads())


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to float64 (bf16 is the top half of fp32)."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
