"""vga_sga_attn_noalloc (the SGA call whose workspace is the library's
static scratch) against vga_sga_attn with a caller workspace, through the C
ABI: the same kernels on the same inputs, so the outputs must be equal bit
for bit -- inside the parity bar of the attention calls (bf16 max-abs
1.5e-2, fp32 1e-5) a fortiori.  Two calls in a row, the second with a
smaller input, in each element type: the second call reuses the scratch the
first one filled.
"""
import ctypes

import pytest

from vga_inputs import tiny_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import alternating_attention_amd as vga
    return vga


def noalloc(vga, q, k, v, frames, sga):
    out = torch.empty_like(q)
    code = vga.VGA_F32 if q.dtype == torch.float32 else vga.VGA_BF16
    cf, cs = frames.c(code), sga.c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = vga.lib.vga_sga_attn_noalloc(ctypes.byref(cf), ctypes.byref(cs), q.data_ptr(),
                                      k.data_ptr(), v.data_ptr(), out.data_ptr(), stream)
    assert st == 0, vga.last_error()
    return out


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_noalloc_equals_sga_attn_two_calls(vga, dt):
    cases = [
        (vga.Frames(6, 20, 20, 5, 4), vga.Sga(2, 2, 0, 0), 11),            # T = 2,430
        (vga.Frames(2, 9, 8, 2, 2), vga.Sga(3, 3, -1, -1, True, 2), 12),   # T = 148, smaller
    ]
    for frames, sga, seed in cases:
        print("case noalloc %s T=%d H=%d %s" % (dt, frames.tokens, frames.num_heads, sga),
              flush=True)
        q, k, v = (torch.from_numpy(a).cuda().to(dt).contiguous()
                   for a in tiny_qkv(frames.tokens, frames.num_heads, 64, seed=seed))
        ref, _ = vga.sga_attn(q, k, v, frames, sga)
        got = noalloc(vga, q, k, v, frames, sga)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), float((got.float() - ref.float()).abs().max())
        # the Python binding reaches the same entry point
        again = vga.sga_attn_noalloc(q, k, v, frames, sga)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
