// vga_internal.h -- declarations shared by the host API and the kernel
// translation units of libvga.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vga {

constexpr int kHeadDim = 64;

enum class KeyRange : int { kFrame = 0, kGlobal = 1, kSga = 2 };

// Closed-form SGA selection on the patch grid of one frame.  Patch (r, c)
// is kept iff r % sh == oh and c % sw == ow; special tokens (u >= gh*gw)
// are always kept.  Kept tokens of a frame are ranked in ascending token
// order: patches first (row-major lattice), then the specials.
struct SgaGrid {
  int32_t L, gh, gw, sh, sw, oh, ow;
  int32_t nh, nw;   // lattice rows/cols: ceil((gh-oh)/sh), ceil((gw-ow)/sw)
  int32_t kpf;      // kept per frame: nh*nw + (L - gh*gw)
};

// Arguments of the flash-attention kernels.  Q/O rows are [T, H, 64]; the
// key source K/V is [num_keys, H, 64] (the full K/V for frame and global
// attention, the compacted kept rows for SGA).
struct FlashParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t num_q;        // T
  int64_t num_keys;     // T (frame/global) or N*kpf (SGA)
  int32_t H;
  int32_t L;            // tokens per frame
  int32_t num_frames;
  float scale;          // softmax scale
  // SGA extras
  const void* k_full;   // K/V of every token (diagonal column)
  const void* v_full;
  const float* kmean;   // [H, 64]
  const float* vmean;   // [H, 64]
  int32_t use_diag;
  int32_t use_mean;
  float log_ndrop;      // ln |D| (count-weighted mean column), else 0
  SgaGrid grid;
  int64_t row0;         // token index of query row 0 (row-range calls)
};

struct GatherParams {
  const void* k;
  const void* v;
  void* kc;
  void* vc;
  int32_t* keep_idx;
  uint8_t* keep_mask;
  float* partials;      // [blocks, 2, H, 64]
  float* kmean;
  float* vmean;
  int64_t T;
  int32_t H;
  int32_t blocks;
  int64_t num_dropped;
  SgaGrid grid;
};

// Copy of the special-token rows between [T, H, 64] tensors and compact
// [N*S, H, 64] ones (register attention).  Compact row j is token
// (j / S) * L + patches + j % S.  to_compact: src full -> dst compact, else
// src compact -> dst full.  Up to three tensors per launch.
struct SpecialRowsParams {
  const void* src[3];
  void* dst[3];
  int32_t ntensors;
  int32_t row_chunks;   // 16-byte chunks per row (H * 64 * elem / 16)
  int64_t rows;         // N * S
  int32_t L, patches, S;
  int32_t to_compact;
};

// Arguments of the projection kernels: Y = X W^T + b, X [M, K], W [N, K],
// b [N] or NULL, Y columns split over up to three [M, C] tensors (column n
// goes to y[n / C] at column n % C).
struct LinearParams {
  const void* x;
  const void* w;
  const void* b;
  void* y[3];
  int64_t M;
  int64_t K;
  int64_t N;
  int64_t C;
};

// Launchers (return the HIP status of the launch).
hipError_t launch_flash_bf16(KeyRange kr, const FlashParams& p, hipStream_t s);
hipError_t launch_flash_f32(KeyRange kr, const FlashParams& p, hipStream_t s);
hipError_t launch_sga_gather(bool bf16, const GatherParams& p, hipStream_t s);
hipError_t launch_special_rows(const SpecialRowsParams& p, hipStream_t s);
hipError_t launch_linear(bool bf16, const LinearParams& p, hipStream_t s);

// Number of partial-sum blocks of the gather for T tokens.
int32_t gather_blocks(int64_t T);

}  // namespace vga
