// sga_gather.hip -- key/value subsampling of Subsampled Global Attention
// ("AVGGT: Rethinking Global Attention for Accelerating VGGT", technical
// summary section 3, step two: uniform grid sampling of K/V on the patch
// grid, and one global mean vector standing for every dropped column).
//
// sga_gather_kernel reads K and V once, row by row.  Each block owns a
// contiguous token range:
//  1. one thread per token evaluates the closed-form selection -- kept patch
//     (r, c) of frame f has rank f*kpf + ((r-oh)/sh)*nw + (c-ow)/sw, special
//     token u has rank f*kpf + nh*nw + (u - gh*gw) -- writes keep_mask[t]
//     and keep_idx[rank] = t, and leaves the rank (or -1) in LDS;
//  2. all threads stream the rows as 16-byte chunks (fully coalesced; K and
//     V are read once, so with non-temporal loads that do not displace
//     cached lines): kept rows are copied to Kc/Vc[rank], dropped rows are
//     summed into per-thread fp32 partials, combined in a fixed order into
//     partials[block] (no float atomics).
// sga_reduce_kernel sums the block partials in a fixed order and divides by
// |D|, giving kmean and vmean [H, 64] in fp32.  Both are HBM-bound streaming
// passes.
#include "vga_internal.h"

namespace vga {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kUnroll = 16;         // tokens in flight per thread
constexpr int kMaxTokensPerBlock = 2048;

// Rank of token t among the kept tokens, or -1 when it is dropped.
__device__ __forceinline__ int32_t sga_rank(const SgaGrid& g, int32_t t) {
  const int32_t f = t / g.L;
  const int32_t u = t - f * g.L;
  const int32_t patches = g.gh * g.gw;
  if (u >= patches) return f * g.kpf + g.nh * g.nw + (u - patches);
  const int32_t row = u / g.gw, col = u - row * g.gw;
  if (row % g.sh != g.oh || col % g.sw != g.ow) return -1;
  return f * g.kpf + ((row - g.oh) / g.sh) * g.nw + (col - g.ow) / g.sw;
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
  __shared__ int32_t rank_of[kMaxTokensPerBlock];
  extern __shared__ float red[];              // [G][P][kEpc] when G > 1

  const int C = p.H * 64;                     // elements per row
  const int W = C / kEpc;                     // chunks per row
  const int P = 2 * W;                        // chunk slots per token (K, V)
  const int G = P >= kGatherThreads ? 1 : kGatherThreads / P;  // tokens / step
  const int NS = (G * P + kGatherThreads - 1) / kGatherThreads; // slots/thread
  const int32_t T = (int32_t)p.T;
  const int32_t tpb = (T + p.blocks - 1) / p.blocks;
  const int32_t t_begin = blockIdx.x * tpb;
  const int32_t t_end = min(t_begin + tpb, T);

  // 1. selection of this block's tokens
  for (int32_t t = t_begin + threadIdx.x; t < t_end; t += kGatherThreads) {
    const int32_t r = sga_rank(p.grid, t);
    rank_of[t - t_begin] = r;
    p.keep_mask[t] = (uint8_t)(r >= 0);
    if (r >= 0) p.keep_idx[r] = t;
  }
  __syncthreads();

  // 2. stream the rows: chunk slot vt = threadIdx.x + 256*i covers token
  //    group vt / P and chunk vt % P (K chunks first, then V chunks)
  const u32x4* kg = (const u32x4*)p.k;
  const u32x4* vg = (const u32x4*)p.v;
  u32x4* kc = (u32x4*)p.kc;
  u32x4* vc = (u32x4*)p.vc;
  float* out = p.partials + (size_t)blockIdx.x * 2 * C;
  for (int i = 0; i < NS; ++i) {
    const int vt = threadIdx.x + kGatherThreads * i;
    if (vt >= G * P) break;
    const int grp = vt / P, slot = vt - (vt / P) * P;
    const bool is_v = slot >= W;
    const int ch = is_v ? slot - W : slot;
    const u32x4* src = (is_v ? vg : kg) + ch;
    u32x4* dst = (is_v ? vc : kc) + ch;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    int32_t tok = t_begin + grp;
    // full groups of kUnroll tokens: all loads in flight before any use
    for (; tok + G * (kUnroll - 1) < t_end; tok += G * kUnroll) {
      u32x4 w[kUnroll];
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu)
        w[uu] = __builtin_nontemporal_load(&src[(size_t)(tok + G * uu) * W]);
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int32_t r = rank_of[tok + G * uu - t_begin];
        if (r >= 0)
          dst[(size_t)r * W] = w[uu];
        else
          add_chunk<BF16>(acc, w[uu]);
      }
    }
    for (; tok < t_end; tok += G) {
      const u32x4 w = __builtin_nontemporal_load(&src[(size_t)tok * W]);
      const int32_t r = rank_of[tok - t_begin];
      if (r >= 0)
        dst[(size_t)r * W] = w;
      else
        add_chunk<BF16>(acc, w);
    }
    if (G == 1) {
#pragma unroll
      for (int e = 0; e < kEpc; ++e) out[slot * kEpc + e] = acc[e];
    } else {
#pragma unroll
      for (int e = 0; e < kEpc; ++e) red[((size_t)grp * P + slot) * kEpc + e] = acc[e];
    }
  }
  if (G == 1) return;

  // block partial [2][C]: sum over the G token groups in group order
  __syncthreads();
  for (int c = threadIdx.x; c < P * kEpc; c += kGatherThreads) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += red[(size_t)g * P * kEpc + c];
    out[c] = s;
  }
}

// Fixed-order reduction of the block partials: thread (quad q, group g)
// sums 4 adjacent columns over blocks b = g, g + 128, ...; the 128 group
// sums are then added pairwise in a fixed tree.  Eight quads per workgroup
// spread the partials over 2C/32 workgroups.
constexpr int kReduceQuads = 8;
constexpr int kReduceGroups = 128;

__global__ void __launch_bounds__(kReduceQuads * kReduceGroups) sga_reduce_kernel(GatherParams p) {
  __shared__ f32x4 part[kReduceGroups][kReduceQuads];
  const int C = p.H * 64;
  const int nq = 2 * C / 4;
  const int qd = threadIdx.x % kReduceQuads;
  const int g = threadIdx.x / kReduceQuads;
  const int quad = blockIdx.x * kReduceQuads + qd;
  f32x4 s = 0.f;
  if (quad < nq) {
    const f32x4* src = (const f32x4*)p.partials + quad;
    int b = g;
    for (; b + 3 * kReduceGroups < p.blocks; b += 4 * kReduceGroups) {
      const f32x4 a0 = src[(size_t)b * nq];
      const f32x4 a1 = src[(size_t)(b + kReduceGroups) * nq];
      const f32x4 a2 = src[(size_t)(b + 2 * kReduceGroups) * nq];
      const f32x4 a3 = src[(size_t)(b + 3 * kReduceGroups) * nq];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; b < p.blocks; b += kReduceGroups) s += src[(size_t)b * nq];
  }
  part[g][qd] = s;
  __syncthreads();
  for (int w = kReduceGroups / 2; w >= 1; w /= 2) {
    if (g < w) part[g][qd] += part[g + w][qd];
    __syncthreads();
  }
  if (g == 0 && quad < nq) {
    const f32x4 total = part[0][qd];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = 4 * quad + e;
      const float mean = p.num_dropped > 0 ? total[e] / (float)p.num_dropped : 0.f;
      if (col < C)
        p.kmean[col] = mean;
      else
        p.vmean[col - C] = mean;
    }
  }
}

}  // namespace

int32_t gather_blocks(int64_t T) {
  // enough blocks to fill the chip, few enough that each block's token
  // ranks fit in LDS
  int64_t b = (T + 127) / 128;
  if (b < 1) b = 1;
  if (b > 1024) b = 1024;
  while ((T + b - 1) / b > kMaxTokensPerBlock) b *= 2;
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
  const int nq = 2 * C / 4;
  const int rblocks = (nq + kReduceQuads - 1) / kReduceQuads;
  hipLaunchKernelGGL(sga_reduce_kernel, dim3(rblocks), dim3(kReduceQuads * kReduceGroups), 0, s, p);
  return hipGetLastError();
}

}  // namespace vga
