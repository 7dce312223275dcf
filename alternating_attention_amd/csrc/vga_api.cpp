// vga_api.cpp -- the C ABI of libvga.so: argument checks, the SGA and
// register-attention workspace layouts, the layer schedules and the kernel
// dispatch.  Every check runs before anything is enqueued, so a failing call
// leaves the stream untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/vga.h"
#include "vga_internal.h"

// The workspace of vga_sga_attn_noalloc: one static array per GPU, held
// from the first call on that GPU until the process ends.  Host code never
// passes this name to a kernel or a copy (on the host it only stands for
// the device symbol); it uses the device address that hipGetSymbolAddress
// returns for the current device (scratch_for below).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

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
  if (s->num_heads > 64 / (s->dtype == VGA_F32 ? 2 : 1))
    return fail(VGA_ERR_UNSUPPORTED, "num_heads %d above the supported maximum", s->num_heads);
  // T < 2^31 first, so that T*H*64 (H <= 64) cannot overflow
  const int64_t T = (int64_t)s->num_frames * s->tokens_per_frame;
  if (T >= ((int64_t)1 << 31))
    return fail(VGA_ERR_SHAPE, "T = %lld tokens exceeds 2^31", (long long)T);
  const int64_t elems = T * s->num_heads * vga::kHeadDim;
  if (elems >= ((int64_t)1 << 31))
    return fail(VGA_ERR_SHAPE, "T*H*64 = %lld exceeds 2^31 elements", (long long)elems);
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
  if (r.diagonal != 0 && r.diagonal != 1)
    return fail(VGA_ERR_PARAM, "diagonal must be 0 or 1");
  if (r.mean_fill < 0 || r.mean_fill > 2)
    return fail(VGA_ERR_PARAM, "mean_fill must be 0, 1 (count-weighted) or 2 (unit weight)");
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

hipError_t launch_flash(const vga_frames* s, vga::KeyRange kr, const vga::FlashParams& p,
                        hipStream_t hs) {
  return s->dtype == VGA_BF16 ? vga::launch_flash_bf16(kr, p, hs)
                              : vga::launch_flash_f32(kr, p, hs);
}

// Rows [r0, r1) of the query side: q_rows/o_rows hold those rows, k/v all
// T rows.  Checks the range, NULLs, alignment and overlaps.
vga_status check_rows(const vga_frames* s, const Checked& c, int64_t r0, int64_t r1,
                      bool whole_frames, const void* q, const void* k, const void* v,
                      const void* o) {
  if (r0 < 0 || r1 < r0 || r1 > c.T)
    return fail(VGA_ERR_SHAPE, "row range [%lld, %lld) outside [0, %lld]", (long long)r0,
                (long long)r1, (long long)c.T);
  if (whole_frames && (r0 % s->tokens_per_frame || r1 % s->tokens_per_frame))
    return fail(VGA_ERR_SHAPE, "row range [%lld, %lld) is not whole frames of %d tokens",
                (long long)r0, (long long)r1, s->tokens_per_frame);
  if (r1 == r0) return VGA_OK;  // nothing is read or written
  if (!q || !k || !v || !o) return fail(VGA_ERR_NULL, "q, k, v and o must be non-NULL");
  const void* ptrs[4] = {q, k, v, o};
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16) return fail(VGA_ERR_ALIGN, "tensor %p is not 16-byte aligned", p);
  const size_t rb = c.bytes / (size_t)c.T * (size_t)(r1 - r0);
  if (overlaps(o, rb, q, rb) || overlaps(o, rb, k, c.bytes) || overlaps(o, rb, v, c.bytes))
    return fail(VGA_ERR_ALIAS, "o overlaps q, k or v");
  return VGA_OK;
}

size_t row_bytes(const vga_frames* s) {
  return (size_t)s->num_heads * vga::kHeadDim * elem_size(s->dtype);
}

vga_status dense_attn(vga::KeyRange kr, const vga_frames* s, int64_t r0, int64_t r1,
                      bool ranged, const void* q, const void* k, const void* v, void* o,
                      void* stream, const char* what) {
  Checked c;
  vga_status st = check_shape(s, &c);
  if (st != VGA_OK) return st;
  if (!ranged) {
    r0 = 0;
    r1 = c.T;
  }
  st = check_rows(s, c, r0, r1, kr == vga::KeyRange::kFrame, q, k, v, o);
  if (st != VGA_OK) return st;
  if (r1 == r0) return VGA_OK;
  vga::FlashParams p = base_params(s, c, q, k, v, o);
  p.num_q = r1 - r0;
  if (kr == vga::KeyRange::kFrame) {
    // whole frames: the shard is a frame-attention problem of its own
    p.k = (const char*)k + (size_t)r0 * row_bytes(s);
    p.v = (const char*)v + (size_t)r0 * row_bytes(s);
    p.num_keys = r1 - r0;
    p.num_frames = (int32_t)((r1 - r0) / s->tokens_per_frame);
  }
  hipStream_t hs = (hipStream_t)stream;
  return finish(launch_flash(s, kr, p, hs), hs, what);
}

// The SGA workspace: present, 16-byte aligned and large enough.
vga_status check_workspace(const vga_sga_ws_layout& w, const void* workspace,
                           size_t workspace_bytes) {
  if (!workspace) return fail(VGA_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace % 16) return fail(VGA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < w.total)
    return fail(VGA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %llu", workspace_bytes,
                (unsigned long long)w.total);
  return VGA_OK;
}

// Launch the SGA selection, gather and mean over all T tokens into the
// workspace (its layout w); returns the gather parameters for the attention.
hipError_t launch_select(const vga_frames* shape, const Checked& c, const vga::SgaGrid& g,
                         const vga_sga_ws_layout& w, const void* k, const void* v,
                         void* workspace, hipStream_t hs, vga::GatherParams* out) {
  char* ws = (char*)workspace;
  vga::GatherParams& gp = *out;
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
  return vga::launch_sga_gather(shape->dtype == VGA_BF16, gp, hs);
}

// SGA on query rows [r0, r1): selection, gather and mean over all T tokens,
// then the shared-softmax attention for the rows.
vga_status sga_run(const vga_frames* shape, const vga_sga* sga, int64_t r0, int64_t r1,
                   bool ranged, const void* q, const void* k, const void* v, void* o,
                   void* workspace, size_t workspace_bytes, void* stream, const char* what) {
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  vga_sga r;
  st = resolve_sga(shape, sga, &r);
  if (st != VGA_OK) return st;
  if (!ranged) {
    r0 = 0;
    r1 = c.T;
  }
  st = check_rows(shape, c, r0, r1, false, q, k, v, o);
  if (st != VGA_OK || r1 == r0) return st;
  const vga::SgaGrid g = make_grid(shape, r);
  vga_sga_ws_layout w;
  fill_layout(shape, c, g, &w);
  st = check_workspace(w, workspace, workspace_bytes);
  if (st != VGA_OK) return st;
  const size_t rb = row_bytes(shape) * (size_t)(r1 - r0);
  if (overlaps(o, rb, workspace, w.total))
    return fail(VGA_ERR_ALIAS, "o overlaps the workspace");
  if (overlaps(q, rb, workspace, w.total) || overlaps(k, c.bytes, workspace, w.total) ||
      overlaps(v, c.bytes, workspace, w.total))
    return fail(VGA_ERR_ALIAS, "an input overlaps the workspace");

  char* ws = (char*)workspace;
  hipStream_t hs = (hipStream_t)stream;
  vga::GatherParams gp;
  hipError_t e = launch_select(shape, c, g, w, k, v, workspace, hs, &gp);
  if (e != hipSuccess) return finish(e, hs, what);

  vga::FlashParams p = base_params(shape, c, q, ws + w.kc, ws + w.vc, o);
  p.num_q = r1 - r0;
  p.num_keys = w.num_kept;
  p.row0 = r0;
  p.k_full = (const char*)k + (size_t)r0 * row_bytes(shape);  // row 0 of the shard
  p.v_full = (const char*)v + (size_t)r0 * row_bytes(shape);
  p.kmean = gp.kmean;
  p.vmean = gp.vmean;
  p.use_diag = r.diagonal;
  p.use_mean = r.mean_fill != 0 && w.num_dropped > 0;
  p.log_ndrop = (r.mean_fill == 1 && w.num_dropped > 0) ? (float)log((double)w.num_dropped)
                                                        : 0.f;
  p.grid = g;
  return finish(launch_flash(shape, vga::KeyRange::kSga, p, hs), hs, what);
}

void fill_register_layout(const vga_frames* s, vga_register_ws_layout* w) {
  const int64_t rows = (int64_t)s->num_frames * s->num_special;
  const uint64_t sect = align256((uint64_t)rows * row_bytes(s));
  w->qs = 0;
  w->ks = sect;
  w->vs = 2 * sect;
  w->os = 3 * sect;
  w->total = 4 * sect;
  w->num_special_rows = rows;
}

vga_status schedule(int32_t num_global_layers, int32_t num_early_to_frame,
                    int32_t register_every, const vga_sga* sga, vga_layer* out) {
  if (num_global_layers < 0 || num_early_to_frame < 0 ||
      num_early_to_frame > num_global_layers)
    return fail(VGA_ERR_PARAM, "need 0 <= num_early (%d) <= num_global (%d)",
                num_early_to_frame, num_global_layers);
  if (register_every < 0)
    return fail(VGA_ERR_PARAM, "register_every %d is negative", register_every);
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
    } else if (register_every > 0 && g % register_every == register_every - 1) {
      l.mode = VGA_MODE_REGISTER;
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

// y = x w^T + b with the columns split over outputs[0..n_out): shared by
// the QKV projection (3 outputs of [T, C]) and the output projection (1).
vga_status linear_run(const vga_frames* s, const void* x, const void* w, const void* b,
                      void* const* outs, int n_out, void* stream, const char* what) {
  Checked c;
  vga_status st = check_shape(s, &c);
  if (st != VGA_OK) return st;
  if (!x || !w) return fail(VGA_ERR_NULL, "%s: x and w must be non-NULL", what);
  for (int i = 0; i < n_out; ++i)
    if (!outs[i]) return fail(VGA_ERR_NULL, "%s: outputs must be non-NULL", what);
  const size_t es = elem_size(s->dtype);
  const int64_t C = (int64_t)s->num_heads * vga::kHeadDim;
  const size_t x_bytes = c.bytes;                     // [T, C]
  const size_t w_bytes = (size_t)n_out * C * C * es;  // [n_out * C, C]
  const size_t b_bytes = (size_t)n_out * C * es;
  const void* aligned[2] = {x, w};
  for (const void* p : aligned)
    if ((uintptr_t)p % 16) return fail(VGA_ERR_ALIGN, "%s: %p is not 16-byte aligned", what, p);
  for (int i = 0; i < n_out; ++i)
    if ((uintptr_t)outs[i] % 16)
      return fail(VGA_ERR_ALIGN, "%s: output %p is not 16-byte aligned", what, outs[i]);
  if (b && (uintptr_t)b % es)
    return fail(VGA_ERR_ALIGN, "%s: bias %p is not aligned to its element", what, b);
  for (int i = 0; i < n_out; ++i) {
    if (overlaps(outs[i], c.bytes, x, x_bytes) || overlaps(outs[i], c.bytes, w, w_bytes) ||
        (b && overlaps(outs[i], c.bytes, b, b_bytes)))
      return fail(VGA_ERR_ALIAS, "%s: an output overlaps an input", what);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], c.bytes, outs[j], c.bytes))
        return fail(VGA_ERR_ALIAS, "%s: two outputs overlap", what);
  }
  vga::LinearParams p;
  memset(&p, 0, sizeof p);
  p.x = x;
  p.w = w;
  p.b = b;
  for (int i = 0; i < n_out; ++i) p.y[i] = outs[i];
  p.M = c.T;
  p.K = C;
  p.N = n_out * C;
  p.C = C;
  hipStream_t hs = (hipStream_t)stream;
  return finish(vga::launch_linear(s->dtype == VGA_BF16, p, hs), hs, what);
}

// The device address of `scratch` on the device that runs `stream` (the
// current device for the null stream), taken once per device with that
// device current and kept.  The table is shared by all threads.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

vga_status scratch_for(hipStream_t hs, void** out) {
  int dev = 0;
  hipError_t e = hs ? hipStreamGetDevice(hs, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(VGA_ERR_HIP, "vga_sga_attn_noalloc: device of the stream: %s",
                hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VGA_ERR_UNSUPPORTED, "vga_sga_attn_noalloc: device %d beyond the first %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e != hipSuccess)
      return fail(VGA_ERR_HIP, "vga_sga_attn_noalloc: select device %d: %s", dev,
                  hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !ptr)
      return fail(VGA_ERR_HIP, "vga_sga_attn_noalloc: scratch address on device %d: %s", dev,
                  hipGetErrorString(e));
    if (back != hipSuccess)
      return fail(VGA_ERR_HIP, "vga_sga_attn_noalloc: restore device %d: %s", cur,
                  hipGetErrorString(back));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VGA_OK;
}

}  // namespace

extern "C" {

vga_status vga_qkv_proj(const vga_frames* shape, const void* x, const void* w_qkv,
                        const void* b_qkv, void* q, void* k, void* v, void* stream) {
  void* outs[3] = {q, k, v};
  return linear_run(shape, x, w_qkv, b_qkv, outs, 3, stream, "vga_qkv_proj");
}

vga_status vga_out_proj(const vga_frames* shape, const void* o, const void* w_o,
                        const void* b_o, void* y, void* stream) {
  void* outs[1] = {y};
  return linear_run(shape, o, w_o, b_o, outs, 1, stream, "vga_out_proj");
}

vga_status vga_frame_attn(const vga_frames* shape, const void* q, const void* k,
                          const void* v, void* o, void* stream) {
  return dense_attn(vga::KeyRange::kFrame, shape, 0, 0, false, q, k, v, o, stream,
                    "vga_frame_attn");
}

vga_status vga_global_attn(const vga_frames* shape, const void* q, const void* k,
                           const void* v, void* o, void* stream) {
  return dense_attn(vga::KeyRange::kGlobal, shape, 0, 0, false, q, k, v, o, stream,
                    "vga_global_attn");
}

vga_status vga_frame_attn_rows(const vga_frames* shape, int64_t row_begin, int64_t row_end,
                               const void* q_rows, const void* k, const void* v,
                               void* o_rows, void* stream) {
  return dense_attn(vga::KeyRange::kFrame, shape, row_begin, row_end, true, q_rows, k, v,
                    o_rows, stream, "vga_frame_attn_rows");
}

vga_status vga_global_attn_rows(const vga_frames* shape, int64_t row_begin, int64_t row_end,
                                const void* q_rows, const void* k, const void* v,
                                void* o_rows, void* stream) {
  return dense_attn(vga::KeyRange::kGlobal, shape, row_begin, row_end, true, q_rows, k, v,
                    o_rows, stream, "vga_global_attn_rows");
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
  return sga_run(shape, sga, 0, 0, false, q, k, v, o, workspace, workspace_bytes, stream,
                 "vga_sga_attn");
}

vga_status vga_sga_attn_noalloc(const vga_frames* shape, const vga_sga* sga, const void* q,
                                const void* k, const void* v, void* o, void* stream) {
  // the size check needs no device: a call beyond the scratch fails here
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  vga_sga r;
  st = resolve_sga(shape, sga, &r);
  if (st != VGA_OK) return st;
  vga_sga_ws_layout w;
  fill_layout(shape, c, make_grid(shape, r), &w);
  if (w.total > kScratchBytes)
    return fail(VGA_ERR_WORKSPACE,
                "vga_sga_attn_noalloc: needs %llu bytes of workspace, the static scratch holds "
                "%llu; use vga_sga_attn with a caller workspace",
                (unsigned long long)w.total, (unsigned long long)kScratchBytes);
  void* ws = nullptr;
  st = scratch_for((hipStream_t)stream, &ws);
  if (st != VGA_OK) return st;
  return sga_run(shape, sga, 0, 0, false, q, k, v, o, ws, kScratchBytes, stream,
                 "vga_sga_attn_noalloc");
}

vga_status vga_sga_select(const vga_frames* shape, const vga_sga* sga, const void* k,
                          const void* v, void* workspace, size_t workspace_bytes,
                          void* stream) {
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  vga_sga r;
  st = resolve_sga(shape, sga, &r);
  if (st != VGA_OK) return st;
  if (!k || !v) return fail(VGA_ERR_NULL, "k and v must be non-NULL");
  if ((uintptr_t)k % 16 || (uintptr_t)v % 16)
    return fail(VGA_ERR_ALIGN, "k and v must be 16-byte aligned");
  const vga::SgaGrid g = make_grid(shape, r);
  vga_sga_ws_layout w;
  fill_layout(shape, c, g, &w);
  st = check_workspace(w, workspace, workspace_bytes);
  if (st != VGA_OK) return st;
  if (overlaps(k, c.bytes, workspace, w.total) || overlaps(v, c.bytes, workspace, w.total))
    return fail(VGA_ERR_ALIAS, "an input overlaps the workspace");
  hipStream_t hs = (hipStream_t)stream;
  vga::GatherParams gp;
  return finish(launch_select(shape, c, g, w, k, v, workspace, hs, &gp), hs, "vga_sga_select");
}

vga_status vga_sga_attn_rows(const vga_frames* shape, const vga_sga* sga, int64_t row_begin,
                             int64_t row_end, const void* q_rows, const void* k,
                             const void* v, void* o_rows, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return sga_run(shape, sga, row_begin, row_end, true, q_rows, k, v, o_rows, workspace,
                 workspace_bytes, stream, "vga_sga_attn_rows");
}

vga_status vga_register_workspace_layout(const vga_frames* shape,
                                         vga_register_ws_layout* out) {
  Checked c;
  const vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  if (!out) return fail(VGA_ERR_NULL, "layout output is NULL");
  fill_register_layout(shape, out);
  return VGA_OK;
}

vga_status vga_register_attn(const vga_frames* shape, const void* q, const void* k,
                             const void* v, void* o, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Checked c;
  vga_status st = check_shape(shape, &c);
  if (st != VGA_OK) return st;
  st = check_tensors(c, q, k, v, o);
  if (st != VGA_OK) return st;
  vga_register_ws_layout w;
  fill_register_layout(shape, &w);
  if (w.total > 0) {
    if (!workspace) return fail(VGA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % 16)
      return fail(VGA_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < w.total)
      return fail(VGA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %llu", workspace_bytes,
                  (unsigned long long)w.total);
    if (overlaps(o, c.bytes, workspace, w.total))
      return fail(VGA_ERR_ALIAS, "o overlaps the workspace");
    if (overlaps(q, c.bytes, workspace, w.total) || overlaps(k, c.bytes, workspace, w.total) ||
        overlaps(v, c.bytes, workspace, w.total))
      return fail(VGA_ERR_ALIAS, "an input overlaps the workspace");
  }
  hipStream_t hs = (hipStream_t)stream;
  // 1. every row as frame attention (patch rows are final)
  vga::FlashParams p = base_params(shape, c, q, k, v, o);
  hipError_t e = launch_flash(shape, vga::KeyRange::kFrame, p, hs);
  if (e != hipSuccess || w.num_special_rows == 0) return finish(e, hs, "vga_register_attn");
  // 2. the special rows: pack, attend over all special tokens, unpack over O
  char* ws = (char*)workspace;
  vga::SpecialRowsParams sp;
  memset(&sp, 0, sizeof sp);
  sp.src[0] = q;
  sp.src[1] = k;
  sp.src[2] = v;
  sp.dst[0] = ws + w.qs;
  sp.dst[1] = ws + w.ks;
  sp.dst[2] = ws + w.vs;
  sp.ntensors = 3;
  sp.row_chunks = (int32_t)(row_bytes(shape) / 16);
  sp.rows = w.num_special_rows;
  sp.L = shape->tokens_per_frame;
  sp.patches = shape->grid_h * shape->grid_w;
  sp.S = shape->num_special;
  sp.to_compact = 1;
  e = vga::launch_special_rows(sp, hs);
  if (e != hipSuccess) return finish(e, hs, "vga_register_attn (pack)");
  vga::FlashParams pg = base_params(shape, c, ws + w.qs, ws + w.ks, ws + w.vs, ws + w.os);
  pg.num_q = w.num_special_rows;
  pg.num_keys = w.num_special_rows;
  e = launch_flash(shape, vga::KeyRange::kGlobal, pg, hs);
  if (e != hipSuccess) return finish(e, hs, "vga_register_attn (special rows)");
  sp.src[0] = ws + w.os;
  sp.dst[0] = o;
  sp.ntensors = 1;
  sp.to_compact = 0;
  return finish(vga::launch_special_rows(sp, hs), hs, "vga_register_attn (unpack)");
}

vga_status vga_layer_schedule(int32_t num_global_layers, int32_t num_early_to_frame,
                              const vga_sga* sga, vga_layer* out) {
  return schedule(num_global_layers, num_early_to_frame, 0, sga, out);
}

vga_status vga_layer_schedule_register(int32_t num_global_layers,
                                       int32_t num_early_to_frame,
                                       int32_t register_every, const vga_sga* sga,
                                       vga_layer* out) {
  return schedule(num_global_layers, num_early_to_frame, register_every, sga, out);
}

vga_status vga_layer_schedule_sga(int32_t num_global_layers, int32_t num_early_to_frame,
                                  const vga_sga* per_slot_sga, vga_layer* out) {
  if (num_global_layers < 0 || num_early_to_frame < 0 ||
      num_early_to_frame > num_global_layers)
    return fail(VGA_ERR_PARAM, "need 0 <= num_early (%d) <= num_global (%d)",
                num_early_to_frame, num_global_layers);
  const int32_t n_sga = num_global_layers - num_early_to_frame;
  if (n_sga > 0 && !per_slot_sga) return fail(VGA_ERR_NULL, "per-slot SGA parameters are NULL");
  if (num_global_layers > 0 && !out) return fail(VGA_ERR_NULL, "schedule output is NULL");
  // every slot's parameters are checked before anything is written
  for (int32_t i = 0; i < n_sga; ++i) {
    vga_sga r;
    const vga_status st = resolve_sga(nullptr, &per_slot_sga[i], &r);
    if (st != VGA_OK) return st;
  }
  for (int32_t g = 0; g < num_global_layers; ++g) {
    vga_layer l;
    memset(&l, 0, sizeof l);
    if (g < num_early_to_frame) {
      l.mode = VGA_MODE_FRAME;
    } else {
      l.mode = VGA_MODE_SGA;
      resolve_sga(nullptr, &per_slot_sga[g - num_early_to_frame], &l.sga);
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
