"""Host-side checks of libvga.so (CPU only: no kernel is launched).

* the library loads and exports every function include/vga.h declares;
* argument validation rejects bad calls with the documented status before
  anything would be enqueued (fake, never-dereferenced device pointers);
* the SGA workspace layout reports the closed-form kept counts, and the
  register-attention layout the special-row sections;
* the layer schedules (with and without register attention) match the
  oracle's.
"""
import ctypes
import os
import re

import pytest

from tests.oracle_pins import kept_per_frame_closed_form

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def vga():
    import alternating_attention_amd as vga
    return vga


def _declared():
    hdr = open(os.path.join(ROOT, "include", "vga.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(vga_[a-z_]+)\s*\(", hdr)))


def test_exports_every_declared_symbol(vga):
    declared = _declared()
    assert declared == sorted(vga.EXPORTS)
    raw = ctypes.CDLL(vga.LIB_PATH)
    for name in declared:
        assert getattr(raw, name) is not None, name


def test_abi_version_and_strings(vga):
    assert vga.abi_version() == 6
    for code, name in enumerate(vga.STATUS_NAMES):
        assert vga.status_string(code) == name


def _frames(vga, **kw):
    f = dict(num_frames=2, grid_h=8, grid_w=8, num_special=5, num_heads=2)
    f.update(kw)
    return vga.Frames(**f)


FAKE = 0x7F0000000000  # 16-byte aligned; never dereferenced by validation


def _call_global(vga, cf, q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000,
                 o=FAKE + 0x3000000):
    return vga.lib.vga_global_attn(ctypes.byref(cf), q, k, v, o, None)


def test_validation_statuses(vga):
    f = _frames(vga)
    ok = f.c(vga.VGA_BF16)
    # NULL pointers
    assert vga.lib.vga_global_attn(None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert _call_global(vga, ok, q=None) == 1
    assert "non-NULL" in vga.last_error()
    # L inconsistent with grid + specials
    assert _call_global(vga, f.c(vga.VGA_BF16, tokens_per_frame=70)) == 2
    # dtype
    bad = f.c(vga.VGA_BF16)
    bad.dtype = 7
    assert _call_global(vga, bad) == 3
    # head_dim
    bad = f.c(vga.VGA_BF16)
    bad.head_dim = 128
    assert _call_global(vga, bad) == 8
    # alignment
    assert _call_global(vga, ok, k=FAKE + 8) == 5
    # o aliases q
    assert _call_global(vga, ok, o=FAKE + 64) == 6
    # too large: T*H*64 >= 2^31
    big = vga.Frames(num_frames=20000, grid_h=37, grid_w=37, num_special=5, num_heads=16)
    assert _call_global(vga, big.c(vga.VGA_BF16)) == 2
    # head counts above the supported maximum: 64 in bf16, 32 in fp32
    assert _call_global(vga, _frames(vga, num_heads=65).c(vga.VGA_BF16)) == 8
    assert _call_global(vga, _frames(vga, num_heads=33).c(vga.VGA_F32)) == 8
    # frame attention shares the checks
    assert vga.lib.vga_frame_attn(ctypes.byref(ok), None, FAKE, FAKE, FAKE, None) == 1


def test_huge_shapes_rejected_before_overflow(vga):
    # N = L = 2^30 with 64 heads: T*H*64 = 2^72 would wrap to 0 in 64 bits;
    # the token count is checked on its own first, so the call is refused
    f = vga.Frames(1 << 30, 1, 1 << 30, 0, 64)
    cf = f.c(vga.VGA_BF16)
    assert vga.lib.vga_global_attn(ctypes.byref(cf), FAKE, FAKE + 0x1000000, FAKE + 0x2000000,
                                   FAKE + 0x3000000, None) == 2
    assert "exceeds 2^31" in vga.last_error()
    with pytest.raises(ValueError):
        vga.Frames(1 << 31, 1, 1, 0, 1).c(vga.VGA_BF16)   # would wrap to -2^31
    f = vga.Frames(1 << 16, 1, 1 << 15, 0, 1)     # T = 2^31 exactly
    assert vga.lib.vga_frame_attn(ctypes.byref(f.c(vga.VGA_BF16)), FAKE, FAKE + 0x1000000,
                                  FAKE + 0x2000000, FAKE + 0x3000000, None) == 2


def test_sga_validation(vga):
    f = _frames(vga)
    cf = f.c(vga.VGA_BF16)

    def call(sga, ws=FAKE + 0x4000000, nbytes=1 << 30, o=FAKE + 0x3000000):
        cs = sga.c()
        return vga.lib.vga_sga_attn(ctypes.byref(cf), ctypes.byref(cs), FAKE,
                                    FAKE + 0x1000000, FAKE + 0x2000000, o, ws, nbytes, None)

    assert call(vga.Sga(stride_h=0)) == 4                  # stride < 1
    assert call(vga.Sga(stride_h=9)) == 4                  # stride > grid
    assert call(vga.Sga(stride_h=2, phase_h=2)) == 4       # phase >= stride
    assert call(vga.Sga(diagonal=2)) == 4
    assert call(vga.Sga(mean_fill=3)) == 4
    assert call(vga.Sga(mean_fill=-1)) == 4
    assert call(vga.Sga(), ws=None) == 7
    assert call(vga.Sga(), nbytes=100) == 7
    assert call(vga.Sga(), ws=FAKE + 0x4000008) == 5
    assert call(vga.Sga(), ws=FAKE + 0x3000000 + 256) == 6  # o overlaps workspace
    assert vga.lib.vga_sga_attn(ctypes.byref(cf), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                None) == 1


def test_select_validation(vga):
    # every rejected call returns before any launch (fake device pointers)
    f = _frames(vga)
    cf = f.c(vga.VGA_BF16)

    def call(sga, k=FAKE + 0x1000000, v=FAKE + 0x2000000, ws=FAKE + 0x4000000,
             nbytes=1 << 30):
        cs = sga.c()
        return vga.lib.vga_sga_select(ctypes.byref(cf), ctypes.byref(cs), k, v, ws, nbytes, None)

    assert call(vga.Sga(stride_h=0)) == 4
    assert call(vga.Sga(mean_fill=3)) == 4
    assert call(vga.Sga(), k=None) == 1
    assert call(vga.Sga(), v=None) == 1
    assert call(vga.Sga(), k=FAKE + 0x1000004) == 5
    assert call(vga.Sga(), ws=None) == 7
    assert call(vga.Sga(), nbytes=100) == 7
    assert call(vga.Sga(), ws=FAKE + 0x4000008) == 5
    assert call(vga.Sga(), ws=FAKE + 0x2000000 + 256) == 6  # v overlaps the workspace
    assert vga.lib.vga_sga_select(ctypes.byref(cf), None, FAKE, FAKE, FAKE, 1, None) == 1
    bad = f.c(vga.VGA_BF16)
    bad.head_dim = 32
    assert vga.lib.vga_sga_select(ctypes.byref(bad), ctypes.byref(vga.Sga().c()),
                                  FAKE, FAKE, FAKE, 1 << 30, None) == 8


def test_rows_validation(vga):
    f = _frames(vga)                 # T = 138, L = 69
    cf = f.c(vga.VGA_BF16)
    Q, K, V, O = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000

    def glob(r0, r1, q=Q, o=O):
        return vga.lib.vga_global_attn_rows(ctypes.byref(cf), r0, r1, q, K, V, o, None)

    def frame(r0, r1):
        return vga.lib.vga_frame_attn_rows(ctypes.byref(cf), r0, r1, Q, K, V, O, None)

    assert glob(-1, 10) == 2
    assert glob(20, 10) == 2
    assert glob(0, 139) == 2
    assert glob(5, 5) == 0                  # empty range: nothing to enqueue
    assert glob(0, 10, q=None) == 1
    assert glob(0, 10, o=Q + 16) == 6       # o overlaps the q rows
    assert glob(0, 10, o=K + 4096) == 6     # o overlaps k
    assert frame(0, 70) == 2                # not whole frames
    assert frame(1, 69) == 2
    assert frame(69, 69) == 0
    cs = vga.Sga().c()
    assert vga.lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(cs), 0, 200, Q, K, V, O,
                                     FAKE + 0x4000000, 1 << 30, None) == 2
    assert vga.lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(cs), 0, 10, Q, K, V, O,
                                     None, 1 << 30, None) == 7
    assert vga.lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(cs), 3, 3, Q, K, V, O,
                                     FAKE + 0x4000000, 1 << 30, None) == 0
    # an empty range reads no pointer
    assert glob(7, 7, q=None, o=None) == 0
    assert vga.lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(cs), 3, 3, None, None,
                                     None, None, None, 0, None) == 0
    bad = vga.Sga(stride_h=0).c()
    assert vga.lib.vga_sga_attn_rows(ctypes.byref(cf), ctypes.byref(bad), 3, 3, None, None,
                                     None, None, None, 0, None) == 4


def test_projection_validation(vga):
    f = _frames(vga, num_heads=2)           # C = 128, T = 138
    cf = f.c(vga.VGA_BF16)
    X, W, B = FAKE, FAKE + 0x1000000, FAKE + 0x2000000
    Q, K, V = FAKE + 0x3000000, FAKE + 0x4000000, FAKE + 0x5000000

    def qkv(x=X, w=W, b=B, q=Q, k=K, v=V, shape=cf):
        return vga.lib.vga_qkv_proj(ctypes.byref(shape), x, w, b, q, k, v, None)

    def outp(o=X, w=W, b=B, y=Q):
        return vga.lib.vga_out_proj(ctypes.byref(cf), o, w, b, y, None)

    assert qkv(x=None) == 1 and qkv(w=None) == 1 and qkv(v=None) == 1
    assert outp(y=None) == 1
    assert vga.lib.vga_qkv_proj(None, X, W, B, Q, K, V, None) == 1
    assert qkv(x=X + 8) == 5 and qkv(k=K + 4) == 5
    assert qkv(b=B + 1) == 5                 # bias must be element-aligned
    assert qkv(q=X + 256) == 6               # q overlaps x
    assert qkv(k=W + 0x100) == 6             # k overlaps w
    assert qkv(v=Q + 0x1000) == 6            # v overlaps q
    assert qkv(q=B) == 6                     # q overlaps the bias
    assert outp(y=X) == 6
    bad = f.c(vga.VGA_BF16)
    bad.dtype = 5
    assert qkv(shape=bad) == 3
    bad = f.c(vga.VGA_BF16, tokens_per_frame=70)
    assert qkv(shape=bad) == 2


def test_register_layout_and_validation(vga):
    f = _frames(vga, num_heads=3)
    lay = vga.register_workspace_layout(f, vga.VGA_BF16)
    rows = f.num_frames * f.num_special
    sect = (rows * 3 * 64 * 2 + 255) // 256 * 256
    assert lay.num_special_rows == rows
    assert [lay.qs, lay.ks, lay.vs, lay.os, lay.total] == [0, sect, 2 * sect, 3 * sect, 4 * sect]
    lay32 = vga.register_workspace_layout(f, vga.VGA_F32)
    assert lay32.total == 4 * ((rows * 3 * 64 * 4 + 255) // 256 * 256)
    assert vga.register_workspace_layout(_frames(vga, num_special=0)).total == 0
    cf = f.c(vga.VGA_BF16)

    def call(ws=FAKE + 0x4000000, nbytes=1 << 30, o=FAKE + 0x3000000):
        return vga.lib.vga_register_attn(ctypes.byref(cf), FAKE, FAKE + 0x1000000,
                                         FAKE + 0x2000000, o, ws, nbytes, None)

    assert call(ws=None) == 7
    assert call(nbytes=lay.total - 1) == 7
    assert call(ws=FAKE + 0x4000004) == 5
    assert call(o=FAKE + 0x4000000 - 64) == 6   # o runs into the workspace
    assert vga.lib.vga_register_attn(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 1


@pytest.mark.parametrize("gh,gw,S,sh,sw,oh,ow", [
    (8, 8, 5, 2, 2, 0, 0), (37, 37, 5, 2, 2, 0, 0), (37, 37, 5, 3, 3, 1, 1),
    (37, 37, 5, 3, 3, -1, -1), (5, 7, 2, 3, 2, 2, 1), (6, 4, 0, 1, 1, 0, 0),
    (1, 1, 0, 1, 1, 0, 0), (9, 3, 4, 4, 3, 3, 2)])
def test_workspace_layout_counts(vga, gh, gw, S, sh, sw, oh, ow):
    N = 3
    f = vga.Frames(num_frames=N, grid_h=gh, grid_w=gw, num_special=S, num_heads=4)
    lay = vga.sga_workspace_layout(f, vga.Sga(sh, sw, oh, ow))
    rh = (sh - 1) // 2 if oh == -1 else oh
    rw = (sw - 1) // 2 if ow == -1 else ow
    kpf = kept_per_frame_closed_form(gh, gw, S, sh, sw, rh, rw)
    assert lay.kept_per_frame == kpf
    assert lay.num_kept == N * kpf
    assert lay.num_dropped == f.tokens - N * kpf
    offs = [lay.keep_idx, lay.keep_mask, lay.kmean, lay.vmean, lay.kc, lay.vc, lay.partials]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and lay.total >= lay.partials + 8 * 4 * 64 * lay.partial_blocks


def test_kept_counts_of_the_workloads(vga):
    # 8x8 + 5 at 2x2 -> 21 per frame; 37x37 + 5 at 2x2 -> 366; at 3x3 phase 1 -> 149
    for (g, s, ph, kpf) in [(8, 2, 0, 21), (37, 2, 0, 366), (37, 3, 1, 149)]:
        f = vga.Frames(num_frames=2, grid_h=g, grid_w=g, num_special=5, num_heads=16)
        lay = vga.sga_workspace_layout(f, vga.Sga(s, s, ph, ph))
        assert lay.kept_per_frame == kpf


def test_layer_schedule(vga):
    sch = vga.layer_schedule(24, 8, vga.Sga(3, 3, -1, -1))
    assert [m for m, _ in sch] == [vga.MODE_FRAME] * 8 + [vga.MODE_SGA] * 16
    assert all(s.phase_h == 1 and s.phase_w == 1 and s.diagonal == 1 for m, s in sch[8:])
    sch = vga.layer_schedule(6, 2, None)
    assert [m for m, _ in sch] == [vga.MODE_FRAME] * 2 + [vga.MODE_GLOBAL] * 4
    with pytest.raises(vga.VgaError) as ei:
        vga.layer_schedule(4, 5, None)
    assert ei.value.status == 4
    with pytest.raises(vga.VgaError):
        vga.layer_schedule(4, 1, vga.Sga(stride_h=0))
    assert vga.lib.vga_layer_schedule(3, 1, None, None) == 1
    assert vga.layer_schedule(0, 0, None) == []
    # entries go to attention() as they stand: Sga parameters on SGA slots only
    sch = vga.layer_schedule(4, 1, vga.Sga(2, 2, 0, 0, True, 2))
    assert sch[0] == (vga.MODE_FRAME, None)
    assert all(e == (vga.MODE_SGA, vga.Sga(2, 2, 0, 0, True, 2)) for e in sch[1:])
    assert all(p is None for _, p in vga.layer_schedule(3, 1, None))


def test_attention_dispatch_refuses_sga_without_parameters(vga):
    with pytest.raises(ValueError):
        vga.attention(vga.MODE_SGA, None, None, None, vga.Frames(1, 2, 2, 0, 1))
    with pytest.raises(ValueError):
        vga.attention(7, None, None, None, vga.Frames(1, 2, 2, 0, 1))


def test_layer_schedule_per_slot_sga(vga):
    import oracle
    ramp = [vga.Sga(2, 2, 0, 0)] * 8 + [vga.Sga(3, 3, -1, -1, False, 2)] * 8
    sch = vga.layer_schedule_sga(24, 8, ramp)
    assert [m for m, _ in sch] == list(oracle.schedule(24, 8, True))
    assert all((s.stride_h, s.phase_h, s.diagonal, s.mean_fill) == (2, 0, 1, 1) for _, s in sch[8:16])
    assert all((s.stride_w, s.phase_w, s.diagonal, s.mean_fill) == (3, 1, 0, 2) for _, s in sch[16:])
    assert [m for m, _ in vga.layer_schedule_sga(3, 3, [])] == [vga.MODE_FRAME] * 3
    with pytest.raises(ValueError):
        vga.layer_schedule_sga(4, 1, [vga.Sga()] * 2)       # needs 3 entries
    # a bad slot anywhere is refused before anything is written
    out = (vga.CLayer * 4)()
    for l in out:
        l.mode = 77
    bad = (vga.CSga * 3)(vga.Sga().c(), vga.Sga(stride_h=0).c(), vga.Sga().c())
    assert vga.lib.vga_layer_schedule_sga(4, 1, bad, out) == 4
    assert [l.mode for l in out] == [77] * 4
    assert vga.lib.vga_layer_schedule_sga(4, 5, bad, out) == 4
    assert vga.lib.vga_layer_schedule_sga(4, 1, None, out) == 1
    assert vga.lib.vga_layer_schedule_sga(4, 1, bad, None) == 1
    assert vga.lib.vga_layer_schedule_sga(2, 2, None, out) == 0


def test_schedule_matches_oracle(vga):
    import oracle
    for G, E, use in [(24, 8, True), (12, 0, False), (5, 5, True)]:
        mine = [m for m, _ in vga.layer_schedule(G, E, vga.Sga() if use else None)]
        assert mine == list(oracle.schedule(G, E, use))
    for G, E, R, use in [(24, 0, 4, False), (24, 8, 4, True), (10, 3, 3, True), (7, 2, 0, False),
                         (5, 0, 1, True)]:
        mine = [m for m, _ in vga.layer_schedule_register(G, E, R, vga.Sga() if use else None)]
        assert mine == list(oracle.schedule_register(G, E, R, use))
    with pytest.raises(vga.VgaError) as ei:
        vga.layer_schedule_register(4, 0, -1, None)
    assert ei.value.status == 4


def test_sga_noalloc_refuses_beyond_scratch(vga):
    # the workspace of 100 frames at stride 2x2 (about 150 MB) exceeds the
    # 64 MiB static scratch: refused before any device call (so this runs
    # without a GPU), with the sizes in the message
    big = vga.Frames(num_frames=100, grid_h=37, grid_w=37, num_special=5, num_heads=16)
    cf, cs = big.c(vga.VGA_BF16), vga.Sga(2, 2, 0, 0).c()
    lay = vga.sga_workspace_layout(big, vga.Sga(2, 2, 0, 0))
    assert lay.total > 64 << 20
    st = vga.lib.vga_sga_attn_noalloc(ctypes.byref(cf), ctypes.byref(cs), None, None, None,
                                      None, None)
    assert st == 7, vga.last_error()
    assert "static scratch holds 67108864" in vga.last_error()
    # a bad stride is still a parameter error, as for vga_sga_attn
    bad = vga.Sga(0, 2, 0, 0).c()
    assert vga.lib.vga_sga_attn_noalloc(ctypes.byref(cf), ctypes.byref(bad), None, None, None,
                                        None, None) == 4
