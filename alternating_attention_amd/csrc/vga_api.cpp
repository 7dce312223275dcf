// vga_api.cpp -- the C ABI of libvga.so: argument checks, the SGA
// workspace layout, the layer schedule and the kernel dispatch.  Every check
// runs before anything is enqueued, so a failing call leaves the stream
// untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/vga.h"
#include "vga_internal.h"

namespace {

thread_local char g_last_error[512] = "";

vga_status fail(vga_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = getenv("VGA_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

size_t elem_size(int32_t dtype) { return dtype == VGA_F32 ? 4 : 2; }

struct Checked {
  int64_t T;
  size_t bytes;   // bytes of one [T, H, 64] tensor
  float scale;
};

vga_status check_shape(const vga_frames* s, Checked* c) {
  if (!s) return fail(VGA_ERR_NULL, "shape descriptor is NULL");
  if (s->dtype != VGA_F32 && s->dtype != VGA_BF16)
    return fail(VGA_ERR_DTYPE, "dtype %d is neither VGA_F32 nor VGA_BF16", s->dtype);
  if (s->head_dim != vga::kHeadDim)
    return fail(VGA_ERR_UNSUPPORTED, "head_dim %d is not 64", s->head_dim);
  if (s->num_frames < 1 || s->num_heads < 1 || s->grid_h < 0 || s->grid_w < 0 ||
      s->num_special < 0)
    return fail(VGA_ERR_SHAPE, "need N >= 1, H >= 1, grid >= 0, S >= 0 (N=%d H=%d %dx%d S=%d)",
                s->num_frames, s->num_heads, s->grid_h, s->grid_w, s->num_special);
  const int64_t patches = (int64_t)s->grid_h * s->grid_w;
  if (s->tokens_per_frame < 1 || patches + s->num_special != s->tokens_per_frame)
    return fail(VGA_ERR_SHAPE, "tokens_per_frame %d != grid %dx%d + %d specials",
                s->tokens_per_frame, s->grid_h, s->grid_w, s->num_special);
  const int64_t T = (int64_t)s->num_frames * s->tokens_per_frame;
  const int64_t elems = T * s->num_heads * vga::kHeadDim;
  if (elems >= ((int64_t)1 << 31))
    return fail(VGA_ERR_SHAPE, "T*H*64 = %lld exceeds 2^31 elements", (long long)elems);
  if (s->num_heads > 64 / (s->dtype == VGA_F32 ? 2 : 1))
    return fail(VGA_ERR_UNSUPPORTED, "num_heads %d above the supported maximum", s->num_heads);
  if (!(s->scale == s->scale) || isinf(s->scale))
    return fail(VGA_ERR_PARAM, "scale is not finite");
  c->T = T;
  c->bytes = (size_t)elems * elem_size(s->dtype);
  c->scale = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  return VGA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

vga_status check_tensors(const Checked& c, const void* q, const void* k, const void* v,
                         const void* o) {
  if (!q || !k || !v || !o) return fail(VGA_ERR_NULL, "q, k, v and o must be non-NULL");
  const void* ptrs[4] = {q, k, v, o};
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16) return fail(VGA_ERR_ALIGN, "tensor %p is not 16-byte aligned", p);
  if (overlaps(o, c.bytes, q, c.bytes) || overlaps(o, c.bytes, k, c.bytes) ||
      overlaps(o, c.bytes, v, c.bytes))
    return fail(VGA_ERR_ALIAS, "o overlaps q, k or v");
  return VGA_OK;
}

vga_status resolve_sga(const vga_frames* s, const vga_sga* in, vga_sga* out) {
  if (!in) return fail(VGA_ERR_NULL, "SGA parameters are NULL");
  vga_sga r = *in;
  const int32_t gh = s ? s->grid_h : 0, gw = s ? s->grid_w : 0;
  if (r.stride_h < 1 || r.stride_w < 1)
    return fail(VGA_ERR_PARAM, "SGA strides must be >= 1 (%d x %d)", r.stride_h, r.stride_w);
  if (s && (r.stride_h > (gh > 0 ? gh : 1) || r.stride_w > (gw > 0 ? gw : 1)))
    return fail(VGA_ERR_PARAM, "SGA stride %dx%d exceeds the %dx%d grid", r.stride_h,
                r.stride_w, gh, gw);
  if (r.phase_h == -1) r.phase_h = (r.stride_h - 1) / 2;
  if (r.phase_w == -1) r.phase_w = (r.stride_w - 1) / 2;
  if (r.phase_h < 0 || r.phase_h >= r.stride_h || r.phase_w < 0 || r.phase_w >= r.stride_w)
    return fail(VGA_ERR_PARAM, "SGA phase (%d,%d) outside [0, stride)", r.phase_h, r.phase_w);
  if ((r.diagonal != 0 && r.diagonal != 1) || (r.mean_fill != 0 && r.mean_fill != 1))
    return fail(VGA_ERR_PARAM, "diagonal and mean_fill must be 0 or 1");
  *out = r;
  return VGA_OK;
}

vga::SgaGrid make_grid(const vga_frames* s, const vga_sga& r) {
  vga::SgaGrid g;
  g.L = s->tokens_per_frame;
  g.gh = s->grid_h;
  g.gw = s->grid_w;
  g.sh = r.stride_h;
  g.sw = r.stride_w;
  g.oh = r.phase_h;
  g.ow = r.phase_w;
  g.nh = g.gh > g.oh ? (g.gh - g.oh + g.sh - 1) / g.sh : 0;
  g.nw = g.gw > g.ow ? (g.gw - g.ow + g.sw - 1) / g.sw : 0;
  if (g.gh == 0 || g.gw == 0) g.nh = g.nw = 0;
  g.kpf = g.nh * g.nw + (g.L - g.gh * g.gw);
  return g;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

void fill_layout(const vga_frames* s, const Checked& c, const vga::SgaGrid& g,
                 vga_sga_ws_layout* w) {
  const int64_t nk = (int64_t)s->num_frames * g.kpf;
  const uint64_t row = (uint64_t)s->num_heads * vga::kHeadDim;
  const int32_t blocks = vga::gather_blocks(c.T);
  uint64_t off = 0;
  w->keep_idx = off;  off = align256(off + sizeof(int32_t) * (uint64_t)nk);
  w->keep_mask = off; off = align256(off + (uint64_t)c.T);
  w->kmean = off;     off = align256(off + sizeof(float) * row);
  w->vmean = off;     off = align256(off + sizeof(float) * row);
  w->kc = off;        off = align256(off + elem_size(s->dtype) * row * (uint64_t)nk);
  w->vc = off;        off = align256(off + elem_size(s->dtype) * row * (uint64_t)nk);
  w->partials = off;  off = align256(off + sizeof(float) * 2 * row * (uint64_t)blocks);
  w->total = off;
  w->kept_per_frame = g.kpf;
  w->num_kept = nk;
  w->num_dropped = c.T - nk;
  w->partial_blocks = blocks;
}

vga_status finish(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess)
    return fail(VGA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
      return fail(VGA_ERR_HIP, "%s: execution failed: %s", what, hipGetErrorString(e));
  }
  return VGA_OK;
}

vga::FlashParams base_params(const vga_frames* s, const Checked& c, const void* q,
                             const void* k, const void* v, void* o) {
  vga::FlashParams p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.num_q = c.T;
  p.num_keys = c.T;
  p.H = s->num_heads;
  p.L = s->tokens_per_frame;
  p.num_frames = s->num_frames;
  p.scale = c.scale;
  return p;
}

vga_status dense_attn(vga::KeyRange kr, const vga_frames* s, const void* q, const void* k,
                      const void* v, void* o, void* stream, const char* what) {
  Checked c;
  vga_status st = check_shape(s, &c);
  if (st != VGA_OK) return st;
  st = check_tensors(c, q, k, v, o);
  if (st != VGA_OK) return st;
  const vga::FlashParams p = base_params(s, c, q, k, v, o);
  hipStream_t hs = (hipStream_t)stream;
  const hipError_t e = s->dtype == VGA_BF16 ? vga::launch_flash_bf16(kr, p, hs)
                                            : vga::launch_flash_f32(kr, p, hs);
  return finish(e, hs, what);
}

}  // namespace

extern "C" {

vga_status vga_frame_attn(const vga_frames* shape, const void* q, const void* k,
                          const void* v, void* o, void* stream) {
  return dense_attn(vga::KeyRange::kFrame, shape, q, k, v, o, stream, "vga_frame_attn");
}

vga_status vga_global_attn(const vga_frames* shape, const void* q, const void* k,
                           const void* v, void* o, void* stream) {
  return dense_attn(vga::KeyRange::kGlobal, shape, q, k, v, o, stream, "vga_global_attn");
}

vga_status vga_sga_workspace_layout(const vga_frames* shape, const vga_sga* sga,
                                    vga_sga_ws_layout* out) {
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  vga_sga r;
  st = resolve_sga(shape, sga, &r);
  if (st != VGA_OK) return st;
  if (!out) return fail(VGA_ERR_NULL, "layout output is NULL");
  fill_layout(shape, c, make_grid(shape, r), out);
  return VGA_OK;
}

vga_status vga_sga_attn(const vga_frames* shape, const vga_sga* sga, const void* q,
                        const void* k, const void* v, void* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  vga_sga r;
  st = resolve_sga(shape, sga, &r);
  if (st != VGA_OK) return st;
  st = check_tensors(c, q, k, v, o);
  if (st != VGA_OK) return st;
  const vga::SgaGrid g = make_grid(shape, r);
  vga_sga_ws_layout w;
  fill_layout(shape, c, g, &w);
  if (!workspace) return fail(VGA_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace % 16) return fail(VGA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < w.total)
    return fail(VGA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %llu", workspace_bytes,
                (unsigned long long)w.total);
  if (overlaps(o, c.bytes, workspace, w.total))
    return fail(VGA_ERR_ALIAS, "o overlaps the workspace");
  if (overlaps(q, c.bytes, workspace, w.total) || overlaps(k, c.bytes, workspace, w.total) ||
      overlaps(v, c.bytes, workspace, w.total))
    return fail(VGA_ERR_ALIAS, "an input overlaps the workspace");

  char* ws = (char*)workspace;
  hipStream_t hs = (hipStream_t)stream;
  vga::GatherParams gp;
  memset(&gp, 0, sizeof gp);
  gp.k = k;
  gp.v = v;
  gp.kc = ws + w.kc;
  gp.vc = ws + w.vc;
  gp.keep_idx = (int32_t*)(ws + w.keep_idx);
  gp.keep_mask = (uint8_t*)(ws + w.keep_mask);
  gp.partials = (float*)(ws + w.partials);
  gp.kmean = (float*)(ws + w.kmean);
  gp.vmean = (float*)(ws + w.vmean);
  gp.T = c.T;
  gp.H = shape->num_heads;
  gp.blocks = (int32_t)w.partial_blocks;
  gp.num_dropped = w.num_dropped;
  gp.grid = g;
  hipError_t e = vga::launch_sga_gather(shape->dtype == VGA_BF16, gp, hs);
  if (e != hipSuccess) return finish(e, hs, "vga_sga_attn (gather)");

  vga::FlashParams p = base_params(shape, c, q, ws + w.kc, ws + w.vc, o);
  p.num_keys = w.num_kept;
  p.k_full = k;
  p.v_full = v;
  p.kmean = gp.kmean;
  p.vmean = gp.vmean;
  p.use_diag = r.diagonal;
  p.use_mean = r.mean_fill && w.num_dropped > 0;
  p.log_ndrop = w.num_dropped > 0 ? (float)log((double)w.num_dropped) : 0.f;
  p.grid = g;
  e = shape->dtype == VGA_BF16 ? vga::launch_flash_bf16(vga::KeyRange::kSga, p, hs)
                               : vga::launch_flash_f32(vga::KeyRange::kSga, p, hs);
  return finish(e, hs, "vga_sga_attn");
}

vga_status vga_layer_schedule(int32_t num_global_layers, int32_t num_early_to_frame,
                              const vga_sga* sga, vga_layer* out) {
  if (num_global_layers < 0 || num_early_to_frame < 0 ||
      num_early_to_frame > num_global_layers)
    return fail(VGA_ERR_PARAM, "need 0 <= num_early (%d) <= num_global (%d)",
                num_early_to_frame, num_global_layers);
  if (num_global_layers > 0 && !out) return fail(VGA_ERR_NULL, "schedule output is NULL");
  vga_sga r;
  memset(&r, 0, sizeof r);
  if (sga) {
    const vga_status st = resolve_sga(nullptr, sga, &r);
    if (st != VGA_OK) return st;
  }
  for (int32_t g = 0; g < num_global_layers; ++g) {
    vga_layer l;
    memset(&l, 0, sizeof l);
    if (g < num_early_to_frame) {
      l.mode = VGA_MODE_FRAME;
    } else if (sga) {
      l.mode = VGA_MODE_SGA;
      l.sga = r;
    } else {
      l.mode = VGA_MODE_GLOBAL;
    }
    out[g] = l;
  }
  return VGA_OK;
}

const char* vga_status_string(vga_status s) {
  switch (s) {
    case VGA_OK: return "VGA_OK";
    case VGA_ERR_NULL: return "VGA_ERR_NULL";
    case VGA_ERR_SHAPE: return "VGA_ERR_SHAPE";
    case VGA_ERR_DTYPE: return "VGA_ERR_DTYPE";
    case VGA_ERR_PARAM: return "VGA_ERR_PARAM";
    case VGA_ERR_ALIGN: return "VGA_ERR_ALIGN";
    case VGA_ERR_ALIAS: return "VGA_ERR_ALIAS";
    case VGA_ERR_WORKSPACE: return "VGA_ERR_WORKSPACE";
    case VGA_ERR_UNSUPPORTED: return "VGA_ERR_UNSUPPORTED";
    case VGA_ERR_HIP: return "VGA_ERR_HIP";
  }
  return "VGA_ERR_UNKNOWN";
}

const char* vga_last_error(void) { return g_last_error; }

int32_t vga_abi_version(void) { return VGA_ABI_VERSION; }

}  // extern "C"
