// proj_gemm.hip -- the linear projections around an attention layer for
// gfx950 (MI355X): the QKV projection that produces Q, K, V and the output
// projection after attention ("VGGT CVPR25 Best Paper" notes, section
// "Alternating-Attention": each frame and global block is a self-attention
// layer over the tokens; the pages leave the projections themselves open,
// read here as nn.Linear-style layers).
//
//   Y[m][n] = sum_k X[m][k] * W[n][k] + b[n]
//
// X is [M, K] (M tokens, K = 64*H features), W is [N, K] row-major (row n
// holds output feature n), b is [N] or absent.  The output columns go to up
// to three [M, C] tensors: column n lands in tensor n / C at column n % C
// (the QKV projection writes q, k and v; the output projection one tensor).
//
// bf16 path (MFMA).  A workgroup of 8 waves owns a 256 (tokens) x 256
// (features) output tile and walks K in 64-wide steps through two LDS
// stages, filled by global_load_lds_dwordx4 while the other stage is
// computed.  A stage holds 256 W rows and 256 X rows of 128 bytes each,
// their 16-byte granules permuted within the row (XOR swizzle) instead of
// padded, so the DMA moves no padding.  The product is taken transposed,
// Y^T = W X^T, with v_mfma_f32_32x32x16_bf16: both operands are then rows
// with K contiguous, read from LDS with one pattern, and each lane ends with
// 16 features of one token.  Each wave owns 128 features x 64 tokens (8
// accumulators); the operand reads of the next 16-wide k step are pinned
// between the MFMAs of the current one, so no MFMA waits on a read just
// issued.  The tile's bias is read into LDS once; the epilogue adds it in
// fp32, rounds to bf16 (RNE), stages the tile in LDS and writes whole rows
// with 16-byte stores.
//
// fp32 path: one thread per output, fp32 dot products in K order.
#include <stdint.h>

#include "vga_internal.h"

namespace vga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kThreads = 512;     // 8 waves
constexpr int kBM = 256;          // tokens per tile
constexpr int kBN = 256;          // output features per tile
constexpr int kBK = 64;           // K per stage
constexpr int kRow = 128;         // LDS bytes per row of 64 bf16, 16-byte slots swizzled
constexpr int kOpTile = 256 * kRow;              // 32768: one operand
constexpr int kStage = 2 * kOpTile;              // 65536: W tile, then X tile
constexpr int kDmaPerWave = kStage / 1024 / 8;   // 8
constexpr int kOutRow = 2 * kBN + 16;            // LDS bytes per staged output row
constexpr int kLds = kBM * kOutRow > 2 * kStage ? kBM * kOutRow : 2 * kStage;

// Granule g (k = 8g .. 8g+7) of row r sits in slot g ^ swz(r): any 16
// consecutive rows (two per 256-byte bank line) and any 8 consecutive rows
// use distinct bank groups for one granule.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

__global__ void __launch_bounds__(kThreads, 1) linear_bf16_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ __attribute__((aligned(16))) uint16_t bias_s[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const uint32_t n_tiles = (uint32_t)((p.N + kBN - 1) / kBN);
  // Workgroup b runs on XCD b mod 8; each XCD takes one contiguous range of
  // tiles (bl), in grouped order: 8 token tiles x every feature tile, token
  // tile fastest, so that the ~32 tiles an XCD runs at once cover 8 token
  // tiles x 4 feature tiles and share their X and W rows in its L2.
  const uint32_t nb = gridDim.x, x8 = blockIdx.x % 8u, per = nb / 8u, rem = nb % 8u;
  const uint32_t bl = x8 * per + min(x8, rem) + blockIdx.x / 8u;
  const uint32_t m_tiles = (uint32_t)((p.M + kBM - 1) / kBM);
  const uint32_t grp = bl / (8u * n_tiles), first_m = grp * 8u;
  const uint32_t gsz = min(m_tiles - first_m, 8u);
  const uint32_t in_grp = bl - grp * 8u * n_tiles;
  const int64_t m0 = (int64_t)(first_m + in_grp % gsz) * kBM;
  const int64_t n0 = (int64_t)(in_grp / gsz) * kBN;
  const int64_t K = p.K;
  const int nk = (int)(K / kBK);

  // DMA plan: instruction j = 8 * s + wave (s < 8) of a stage fills LDS
  // bytes [1024 j, 1024 j + 1024), lane by lane: W rows for j < 32, X rows
  // after.  Lane l writes slot l % 8 of row 8 (j % 32) + l / 8 of its
  // operand, i.e. loads global granule (l % 8) ^ swz(row) of that row.  Rows
  // past the matrix load its last row (their results are never stored).
  // The base pointer of an instruction is wave-uniform and the lane only
  // adds a 32-bit offset (every operand is below 4 GiB).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t src_off[kDmaPerWave];
  const char* src_base[kDmaPerWave];
#pragma unroll
  for (int s = 0; s < kDmaPerWave; ++s) {
    // a value in SGPRs: the DMA asm clobbers memory, so the kernel argument
    // would otherwise be read again after every instruction
    src_base[s] = s < 4 ? (const char*)p.w : (const char*)p.x;
    asm volatile("" : "+s"(src_base[s]));
    const int j = 8 * s + wave_u;
    const int r = 8 * (j % 32) + lane / 8;      // row within the operand tile
    const int g = (lane % 8) ^ swz(r & 31);
    const int64_t row = s < 4 ? min(n0 + r, p.N - 1) : min(m0 + r, p.M - 1);
    src_off[s] = (uint32_t)(row * K * 2 + g * 16);
  }
  auto issue = [&](int kstep, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kDmaPerWave; ++s) {
      const char* base = src_base[s] + (int64_t)kstep * kBK * 2;
      // Issued from asm, as in the attention kernel: the compiler's wait
      // model would otherwise hold every later LDS read until this DMA
      // lands.  Completion is awaited before each barrier.  The instruction
      // writes LDS only and has no destination registers.
      const uint32_t ldsa = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)&lds[stage * kStage + 1024 * (8 * s + wave_u)]);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(src_off[s]), "s"(base), "s"(ldsa)
                   : "memory", "m0");
    }
  };

  // operand reads: A = W rows (features), B = X rows (tokens), each lane
  // row l32 of a 32-row block, granule 2c + hf (k = 16c + 8hf + [0, 8)) of
  // k step c, found in slot (2c + hf) ^ swz(l32) (swz only sees l32)
  const int wn = (wave & 1) * 128;   // this wave's features within the tile
  const int wm = (wave >> 1) * 64;   // this wave's tokens within the tile
  const int sw = swz(l32);
  int a_off[4], b_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a_off[c] = (wn + l32) * kRow + 16 * ((2 * c + hf) ^ sw);
    b_off[c] = kOpTile + (wm + l32) * kRow + 16 * ((2 * c + hf) ^ sw);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    acc[nb][0] = 0.f;
    acc[nb][1] = 0.f;
  }

  issue(0, 0);
  // this tile's bias (zero past N or without a bias), read once, element
  // by element: the bias need only be aligned to its 2-byte element
  if (tid < kBN / 8) {
    u32x4 bw = {0u, 0u, 0u, 0u};
    const int64_t n = n0 + 8 * tid;
    if (p.b && n < p.N) {
      const uint16_t* bs = (const uint16_t*)p.b + n;   // N is a multiple of 64
#pragma unroll
      for (int e = 0; e < 4; ++e) bw[e] = (uint32_t)bs[2 * e] | ((uint32_t)bs[2 * e + 1] << 16);
    }
    *(__attribute__((address_space(3))) u32x4*)&bias_s[8 * tid] = bw;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int st = s & 1;
    if (s + 1 < nk) issue(s + 1, st ^ 1);  // its stage was last read in step s-1
    const char* base = &lds[st * kStage];
    bf16x8 a[2][4], b[2][2];
    auto load = [&](int c, int buf) __attribute__((always_inline)) {
      // in the order of first use: b0, a0, b1, a1, a2, a3
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        if (i == 0 || i == 2) {
          const int mb = i / 2;
          b[buf][mb] = __builtin_bit_cast(
              bf16x8, *(const lds_u32x4*)(base + b_off[c] + mb * 32 * kRow));
        } else {
          const int nb = i == 1 ? 0 : i - 2;
          a[buf][nb] = __builtin_bit_cast(
              bf16x8, *(const lds_u32x4*)(base + a_off[c] + nb * 32 * kRow));
        }
      }
    };
    load(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 1 < 4) load(c + 1, (c + 1) & 1);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 1][nb], b[c & 1][mb],
                                                                acc[nb][mb], 0, 0, 0);
      // one operand read of the next k step, then one MFMA, six times; then
      // the last two MFMAs
      if (c + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the next stage has landed
    __syncthreads();                     // and every wave is done with this one
  }

  // ---- epilogue: bias, bf16, staged in LDS as [token][feature] rows
  char* out_tile = &lds[0];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = wm + 32 * mb + l32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = wn + 32 * nb + 8 * g + 4 * hf;  // 4 consecutive features
        const u32x2 bb = *(const __attribute__((address_space(3))) u32x2*)&bias_s[n];
        const float bias[4] = {__uint_as_float(bb[0] << 16), __uint_as_float(bb[0] & 0xffff0000u),
                               __uint_as_float(bb[1] << 16), __uint_as_float(bb[1] & 0xffff0000u)};
        u32x2 w2;
        w2[0] = pack_bf16(acc[nb][mb][4 * g + 0] + bias[0], acc[nb][mb][4 * g + 1] + bias[1]);
        w2[1] = pack_bf16(acc[nb][mb][4 * g + 2] + bias[2], acc[nb][mb][4 * g + 3] + bias[3]);
        *(__attribute__((address_space(3))) u32x2*)(out_tile + m * kOutRow + n * 2) = w2;
      }
    }
  __syncthreads();
  // 256 rows x 32 granules of 16 bytes; granule (row, j) holds features
  // n0 + 8j .. n0 + 8j + 7 of token m0 + row
#pragma unroll 4
  for (int i = tid; i < kBM * (kBN / 8); i += kThreads) {
    const int row = i >> 5, j = i & 31;
    const int64_t m = m0 + row, n = n0 + 8 * j;
    if (m >= p.M || n >= p.N) continue;
    const int which = n >= 2 * p.C ? 2 : n >= p.C ? 1 : 0;
    const int64_t col = n - which * p.C;
    char* dst = (char*)p.y[which] + (m * p.C + col) * 2;
    *(u32x4*)dst = *(const __attribute__((address_space(3))) u32x4*)(out_tile + row * kOutRow + j * 16);
  }
}

__global__ void __launch_bounds__(256) linear_f32_kernel(LinearParams p) {
  const int64_t total = p.M * p.N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t m = i / p.N, n = i - m * p.N;
    const float* xr = (const float*)p.x + m * p.K;
    const float* wr = (const float*)p.w + n * p.K;
    float acc = 0.f;
    for (int64_t k = 0; k < p.K; ++k) acc = __builtin_fmaf(xr[k], wr[k], acc);
    if (p.b) acc += ((const float*)p.b)[n];
    const int which = n >= 2 * p.C ? 2 : n >= p.C ? 1 : 0;
    ((float*)p.y[which])[m * p.C + (n - which * p.C)] = acc;
  }
}

}  // namespace

hipError_t launch_linear(bool bf16, const LinearParams& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  if (bf16) {
    const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN);
    hipLaunchKernelGGL(linear_bf16_kernel, dim3((uint32_t)tiles), dim3(kThreads), 0, s, p);
  } else {
    int64_t blocks = (p.M * p.N + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(linear_f32_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace vga
