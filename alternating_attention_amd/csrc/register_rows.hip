// register_rows.hip -- row moves of register attention ("VGGT-Omega"
// notes, section 2, Register Attention): the cross-frame exchange of a
// register-attention layer involves only the per-frame special tokens
// (camera and registers), so their Q/K/V rows are packed into compact
// [N*S, H, 64] tensors, attended globally by the flash kernel, and the
// outputs are written back over the frame-attention result.
//
// Both directions are plain HBM copies of whole rows in 16-byte chunks;
// consecutive lanes take consecutive chunks of a row, so each row moves as
// one contiguous run.
#include "vga_internal.h"

namespace vga {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;

__global__ void __launch_bounds__(kCopyThreads) special_rows_kernel(SpecialRowsParams p) {
  const int64_t per_tensor = p.rows * p.row_chunks;
  const int64_t total = per_tensor * p.ntensors;
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < total; i += stride) {
    const int tsel = (int)(i / per_tensor);
    const int64_t w = i - tsel * per_tensor;
    const int64_t j = w / p.row_chunks;         // compact row
    const int64_t c = w - j * p.row_chunks;     // chunk inside the row
    const int64_t f = j / p.S;
    const int64_t t = f * p.L + p.patches + (j - f * p.S);  // token of row j
    const int64_t src_row = p.to_compact ? t : j;
    const int64_t dst_row = p.to_compact ? j : t;
    const u32x4* src = (const u32x4*)(tsel == 0 ? p.src[0] : tsel == 1 ? p.src[1] : p.src[2]);
    u32x4* dst = (u32x4*)(tsel == 0 ? p.dst[0] : tsel == 1 ? p.dst[1] : p.dst[2]);
    dst[dst_row * p.row_chunks + c] = src[src_row * p.row_chunks + c];
  }
}

}  // namespace

hipError_t launch_special_rows(const SpecialRowsParams& p, hipStream_t s) {
  const int64_t total = p.rows * p.row_chunks * p.ntensors;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(special_rows_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace vga
