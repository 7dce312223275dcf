// sga_gather.hip -- key/value subsampling of Subsampled Global Attention
// ("AVGGT: Rethinking Global Attention for Accelerating VGGT", technical
// summary section 3, step two: uniform grid sampling of K/V on the patch
// grid, and one global mean vector standing for every dropped column).
//
// sga_gather_kernel reads K and V once, row by row, and
//  - writes keep_mask[t] and, for kept tokens, keep_idx[rank] = t;
//  - copies each kept row of K and V to its compacted slot Kc/Vc[rank];
//  - sums each dropped row into per-thread fp32 partials, which the block
//    combines in a fixed order into partials[block] (no float atomics).
// The kept rank comes from the closed form of the strided lattice: kept
// patch (r, c) of frame f has rank f*kpf + ((r-oh)/sh)*nw + (c-ow)/sw and
// special token u has rank f*kpf + nh*nw + (u - gh*gw).
// sga_reduce_kernel sums the block partials in a fixed order and divides by
// |D|, giving kmean and vmean [H, 64] in fp32.  Both kernels are HBM-bound
// streaming passes; rows are read as 16-byte chunks, fully coalesced.
#include "vga_internal.h"

namespace vga {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kUnroll = 8;        // tokens in flight per thread
constexpr int kMaxSlots = 4;      // chunks per thread when a row pair > 256 chunks

struct Rank {
  bool kept;
  int64_t rank;
};

__device__ __forceinline__ Rank sga_rank(const SgaGrid& g, int64_t t) {
  const int64_t f = t / g.L;
  const int32_t u = (int32_t)(t - f * g.L);
  Rank r;
  if (u >= g.gh * g.gw) {
    r.kept = true;
    r.rank = f * g.kpf + (int64_t)g.nh * g.nw + (u - g.gh * g.gw);
    return r;
  }
  const int32_t row = u / g.gw, col = u - row * g.gw;
  r.kept = (row % g.sh == g.oh) && (col % g.sw == g.ow);
  r.rank = f * g.kpf + (int64_t)((row - g.oh) / g.sh) * g.nw + (col - g.ow) / g.sw;
  return r;
}

// Accumulate a 16-byte chunk (8 bf16 or 4 fp32) into acc[0..8).
template <bool BF16>
__device__ __forceinline__ void add_chunk(float* acc, const u32x4& w) {
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(w[e] << 16);
      acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kGatherThreads) sga_gather_kernel(GatherParams p) {
  constexpr int kEpc = BF16 ? 8 : 4;          // elements per 16-byte chunk
  const int C = p.H * 64;                     // elements per row
  const int W = C / kEpc;                     // chunks per row
  const int P = 2 * W;                        // chunk slots per token (K, V)
  const int G = P >= kGatherThreads ? 1 : kGatherThreads / P;  // tokens / step
  const int NS = (G * P + kGatherThreads - 1) / kGatherThreads; // slots/thread
  const int64_t tpb = (p.T + p.blocks - 1) / p.blocks;
  const int64_t t_begin = (int64_t)blockIdx.x * tpb;
  const int64_t t_end = min(t_begin + tpb, p.T);

  const u32x4* kg = (const u32x4*)p.k;
  const u32x4* vg = (const u32x4*)p.v;
  u32x4* kc = (u32x4*)p.kc;
  u32x4* vc = (u32x4*)p.vc;

  float acc[kMaxSlots][8];
  int grp[kMaxSlots], slot[kMaxSlots];
  bool active[kMaxSlots];
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) {
    const int vt = threadIdx.x + kGatherThreads * i;
    active[i] = i < NS && vt < G * P;
    grp[i] = vt / P;
    slot[i] = vt - grp[i] * P;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  for (int64_t t0 = t_begin; t0 < t_end; t0 += (int64_t)G * kUnroll) {
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) {
      if (!active[i]) continue;
      const bool is_v = slot[i] >= W;
      const int ch = is_v ? slot[i] - W : slot[i];
      const u32x4* src = is_v ? vg : kg;
      u32x4 w[kUnroll];
      int64_t tok[kUnroll];
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        tok[uu] = t0 + (int64_t)G * uu + grp[i];
        if (tok[uu] < t_end) w[uu] = src[tok[uu] * W + ch];
      }
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        if (tok[uu] >= t_end) continue;
        const Rank r = sga_rank(p.grid, tok[uu]);
        if (r.kept) {
          (is_v ? vc : kc)[r.rank * W + ch] = w[uu];
        } else {
          add_chunk<BF16>(acc[i], w[uu]);
        }
        if (slot[i] == 0) {
          p.keep_mask[tok[uu]] = (uint8_t)r.kept;
          if (r.kept) p.keep_idx[r.rank] = (int32_t)tok[uu];
        }
      }
    }
  }

  // Block partial: [2][C] = sum over the G token groups, in group order.
  float* out = p.partials + (size_t)blockIdx.x * 2 * C;
  if (G == 1) {
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) {
      if (!active[i]) continue;
#pragma unroll
      for (int e = 0; e < kEpc; ++e) out[slot[i] * kEpc + e] = acc[i][e];
    }
    return;
  }
  extern __shared__ float red[];  // [G][P][kEpc]
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) {
    if (!active[i]) continue;
#pragma unroll
    for (int e = 0; e < kEpc; ++e) red[((size_t)grp[i] * P + slot[i]) * kEpc + e] = acc[i][e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < P * kEpc; c += kGatherThreads) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += red[(size_t)g * P * kEpc + c];
    out[c] = s;
  }
}

constexpr int kReduceCols = 64;
constexpr int kReduceGroups = 4;

__global__ void __launch_bounds__(kReduceCols * kReduceGroups) sga_reduce_kernel(GatherParams p) {
  const int C = p.H * 64;
  const int col = blockIdx.x * kReduceCols + (threadIdx.x % kReduceCols);
  const int grp = threadIdx.x / kReduceCols;
  __shared__ float part[kReduceGroups][kReduceCols];
  float s = 0.f;
  if (col < 2 * C)
    for (int b = grp; b < p.blocks; b += kReduceGroups)
      s += p.partials[(size_t)b * 2 * C + col];
  part[grp][threadIdx.x % kReduceCols] = s;
  __syncthreads();
  if (grp == 0 && col < 2 * C) {
    const int c = threadIdx.x;
    const float total = (part[0][c] + part[1][c]) + (part[2][c] + part[3][c]);
    const float mean = p.num_dropped > 0 ? total / (float)p.num_dropped : 0.f;
    if (col < C)
      p.kmean[col] = mean;
    else
      p.vmean[col - C] = mean;
  }
}

}  // namespace

int32_t gather_blocks(int64_t T) {
  int64_t b = (T + 127) / 128;
  if (b < 1) b = 1;
  if (b > 1024) b = 1024;
  return (int32_t)b;
}

hipError_t launch_sga_gather(bool bf16, const GatherParams& p, hipStream_t s) {
  const int C = p.H * 64;
  const int P = 2 * C / (bf16 ? 8 : 4);
  const int G = P >= kGatherThreads ? 1 : kGatherThreads / P;
  const size_t shmem = G > 1 ? (size_t)G * P * (bf16 ? 8 : 4) * sizeof(float) : 0;
  if (p.T > 0) {
    if (bf16)
      hipLaunchKernelGGL(sga_gather_kernel<true>, dim3(p.blocks), dim3(kGatherThreads), shmem, s, p);
    else
      hipLaunchKernelGGL(sga_gather_kernel<false>, dim3(p.blocks), dim3(kGatherThreads), shmem, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rblocks = (2 * C + kReduceCols - 1) / kReduceCols;
  hipLaunchKernelGGL(sga_reduce_kernel, dim3(rblocks), dim3(kReduceCols * kReduceGroups), 0, s, p);
  return hipGetLastError();
}

}  // namespace vga
