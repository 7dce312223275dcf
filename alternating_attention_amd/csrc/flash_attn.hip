// flash_attn.hip -- attention over frames of tokens for gfx950 (MI355X).
//
// One kernel core serves the three attention modes of an alternating-
// attention trunk ("VGGT CVPR25 Best Paper" notes, "Alternating-Attention";
// "AVGGT: Rethinking Global Attention for Accelerating VGGT", section 3):
//   kFrame  -- the keys of a query are the L tokens of its own frame;
//   kGlobal -- the keys are all T tokens; the T x T score matrix only ever
//              exists one 64-key tile at a time in registers;
//   kSga    -- the keys are the compacted kept rows (Kc, Vc), and the
//              softmax state of each query starts from its diagonal column
//              (own token, when dropped) and the count-weighted mean column,
//              so the three parts share one softmax.
//
// bf16 path (MFMA).  A workgroup of 4 waves owns 256 queries of one head;
// each wave owns 64 queries as two 32-query blocks.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys index the
// accumulator rows and queries its columns, so every lane holds 16 scores of
// ONE query.  Row statistics therefore stay in the lane (plus its partner
// lane l^32); the probabilities P^T feed O^T = V^T P^T directly as the B
// operand without touching LDS.  K rows are stored in LDS in a permuted
// order (bits 2 and 3 of the row index swapped) so that accumulator
// register r of lane half h holds key 16*(r/8) + 8*h + r%8 -- exactly the
// B-operand k-slot order of the PV product.  V is stored transposed (V^T,
// keys contiguous) so the PV A operand is one 16-byte LDS read.  Both LDS
// tiles use XOR-swizzled 16-byte chunks to avoid bank conflicts.
//
// Softmax: the MFMA produces exact fp32 dot products of the bf16 rows; one
// FMA per score turns them into log2 units and subtracts the row's
// reference max m.  The reference max is updated lazily: a tile whose probabilities sum above
// 2^16 in a lane (or the first tile) takes a wave-uniform slow path that
// raises m to the tile max and rescales O and l; otherwise P = exp2(S)
// directly.  P is rounded to bf16 (RNE) for the PV MFMA; l, O accumulate in
// fp32.
//
// fp32 path: a plain VALU kernel (one lane per query and head, exact online
// softmax in fp32), used for fp32 inputs.
#include "vga_internal.h"

namespace vga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // 4 waves
constexpr int kQPerWave = 64;
constexpr int kBQ = 4 * kQPerWave;     // queries per workgroup
constexpr int kBK = 64;                // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSum = 65536.f;  // lazy-rescale trigger (2^16)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (RNE) and pack them (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// LDS row of key (within a 32-key sub-tile) swaps bits 2 and 3.
__device__ __forceinline__ int perm_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Element offset of 16-byte chunk j of K row i in a [64][64] bf16 tile.
__device__ __forceinline__ int k_off(int row, int j) { return row * 64 + ((j ^ (row & 7)) << 3); }
// Element offset of key-chunk kc (8 keys) of V^T row d in a [64][64] tile.
__device__ __forceinline__ int v_off(int d, int kc) {
  return d * 64 + ((kc ^ ((d ^ (d >> 3)) & 7)) << 3);
}

struct TileRange {
  int64_t q_begin, q_end;    // query rows of this workgroup
  int64_t k_begin, k_end;    // key rows
  int32_t head;
};

template <KeyRange KR>
__device__ __forceinline__ TileRange tile_range(const FlashParams& p) {
  TileRange t;
  const int64_t b = blockIdx.x;
  if constexpr (KR == KeyRange::kFrame) {
    const int64_t qtpf = (p.L + kBQ - 1) / kBQ;
    const int64_t per_head = qtpf * p.num_frames;
    t.head = (int32_t)(b / per_head);
    const int64_t rem = b % per_head;
    const int64_t f = rem / qtpf, qt = rem % qtpf;
    t.q_begin = f * p.L + qt * kBQ;
    t.q_end = min(t.q_begin + kBQ, (f + 1) * (int64_t)p.L);
    t.k_begin = f * p.L;
    t.k_end = (f + 1) * (int64_t)p.L;
  } else {
    const int64_t nqt = (p.num_q + kBQ - 1) / kBQ;
    t.head = (int32_t)(b / nqt);
    t.q_begin = (b % nqt) * kBQ;
    t.q_end = min(t.q_begin + kBQ, p.num_q);
    t.k_begin = 0;
    t.k_end = p.num_keys;
  }
  return t;
}

// Is token t kept as a K/V column by the SGA grid sampling?
__device__ __forceinline__ bool sga_kept(const SgaGrid& g, int64_t t) {
  const int32_t u = (int32_t)(t % g.L);
  if (u >= g.gh * g.gw) return true;
  const int32_t r = u / g.gw, c = u - r * g.gw;
  return (r % g.sh == g.oh) && (c % g.sw == g.ow);
}

template <KeyRange KR>
__global__ void __launch_bounds__(kThreads, 2) flash_bf16_kernel(FlashParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kBK * 64];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][64 * kBK];

  const TileRange tr = tile_range<KR>(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half: k-group of the MFMA operands
  const int H = p.H;
  const int head = tr.head;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v;
  const float qscale = p.scale * kLog2e;

  // ---- Q block of this wave into registers (B operand of S^T = K Q^T):
  // lane holds query l32 of block qb, dims 16c + 8*hf + [0, 8), as stored.
  bf16x8 qreg[2][4];
  int64_t qrow[2];
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t row = tr.q_begin + wave * kQPerWave + qb * 32 + l32;
    qvalid[qb] = row < tr.q_end;
    qrow[qb] = qvalid[qb] ? row : tr.q_end - 1;
    const uint16_t* src = qg + ((size_t)qrow[qb] * H + head) * 64 + 8 * hf;
#pragma unroll
    for (int c = 0; c < 4; ++c) qreg[qb][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * c));
  }

  // ---- softmax state.  Lane (l32, hf) of block qb holds, for its query:
  // o[qb][db] register r = O^T[d][q] with d = 32*db + 8*(r/4) + 4*hf + r%4;
  // lsum = this lane's share of the row sum; m = reference max (log2 units).
  f32x16 o[2][2];
  float lsum[2], m[2];
  bool mset[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    o[qb][0] = 0.f;
    o[qb][1] = 0.f;
    lsum[qb] = 0.f;
    m[qb] = 0.f;
    mset[qb] = false;
  }

  if constexpr (KR == KeyRange::kSga) {
    // Diagonal and mean columns start the shared softmax of each query.
    const uint16_t* kf = (const uint16_t*)p.k_full;
    const uint16_t* vf = (const uint16_t*)p.v_full;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t row = qrow[qb];
      const bool diag = p.use_diag && !sga_kept(p.grid, row);
      const uint16_t* qs = qg + ((size_t)row * H + head) * 64 + 8 * hf;
      const uint16_t* ks = kf + ((size_t)row * H + head) * 64 + 8 * hf;
      const float* kms = p.kmean + head * 64 + 8 * hf;
      float dk = 0.f, dm = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 wq = *(const u32x4*)(qs + 16 * c);
        const u32x4 wk = *(const u32x4*)(ks + 16 * c);
        const f32x4 m0 = *(const f32x4*)(kms + 16 * c);
        const f32x4 m1 = *(const f32x4*)(kms + 16 * c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float qa = bf16_lo(wq[e]), qb2 = bf16_hi(wq[e]);
          dk += qa * bf16_lo(wk[e]) + qb2 * bf16_hi(wk[e]);
          const float ma = e < 2 ? m0[2 * e] : m1[2 * e - 4];
          const float mb = e < 2 ? m0[2 * e + 1] : m1[2 * e - 3];
          dm += qa * ma + qb2 * mb;
        }
      }
      dk += __shfl_xor(dk, 32);
      dm += __shfl_xor(dm, 32);
      const float zd = dk * qscale;
      const float zm = dm * qscale + p.log_ndrop * kLog2e;
      if (diag || p.use_mean) {
        float m0v = diag ? zd : zm;
        if (diag && p.use_mean) m0v = fmaxf(zd, zm);
        const float wd = diag ? exp2f(zd - m0v) : 0.f;
        const float wm = p.use_mean ? exp2f(zm - m0v) : 0.f;
        m[qb] = m0v;
        mset[qb] = true;
        lsum[qb] = hf == 0 ? wd + wm : 0.f;
        const uint16_t* vs = vf + ((size_t)row * H + head) * 64;
        const float* vms = p.vmean + head * 64;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hf;
            const u32x2 wv = *(const u32x2*)(vs + d0);
            const f32x4 mv = *(const f32x4*)(vms + d0);
            o[qb][db][4 * g + 0] = wd * bf16_lo(wv[0]) + wm * mv[0];
            o[qb][db][4 * g + 1] = wd * bf16_hi(wv[0]) + wm * mv[1];
            o[qb][db][4 * g + 2] = wd * bf16_lo(wv[1]) + wm * mv[2];
            o[qb][db][4 * g + 3] = wd * bf16_hi(wv[1]) + wm * mv[3];
          }
      }
    }
  }

  // ---- K/V tile staging: global -> registers -> LDS (double buffered).
  const int ld_j = tid & 7;    // 16-byte chunk (8 dims) of a row
  const int ld_i = tid >> 3;   // 0..31
  u32x4 kst[2], vst[2];
  auto load_tile = [&](int64_t key0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t kk = key0 + 32 * rr + perm_row(ld_i);
      kst[rr] = kk < tr.k_end
                    ? *(const u32x4*)(kg + ((size_t)kk * H + head) * 64 + 8 * ld_j)
                    : u32x4{0u, 0u, 0u, 0u};
      const int64_t kv = key0 + 2 * ld_i + rr;
      vst[rr] = kv < tr.k_end
                    ? *(const u32x4*)(vg + ((size_t)kv * H + head) * 64 + 8 * ld_j)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 32 * rr + ld_i;
      *(u32x4*)&lds_k[st][k_off(row, ld_j)] = kst[rr];
    }
    // V^T: dims 8*ld_j + e, keys 2*ld_i and 2*ld_i + 1 packed in one word
    const int key = 2 * ld_i;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * ld_j + e;
      const uint32_t a = vst[0][e >> 1], b = vst[1][e >> 1];
      const uint32_t w = (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                                 : __builtin_amdgcn_perm(b, a, 0x05040100u);
      *(uint32_t*)&lds_v[st][v_off(d, key >> 3) + (key & 7)] = w;
    }
  };

  const int64_t ntiles = (tr.k_end - tr.k_begin + kBK - 1) / kBK;

  load_tile(tr.k_begin);
  store_tile(0);
  __syncthreads();

  for (int64_t t = 0; t < ntiles; ++t) {
    const int st = (int)(t & 1);
    const int64_t key0 = tr.k_begin + t * kBK;
    if (t + 1 < ntiles) load_tile(key0 + kBK);

    // ---- S^T = scale*log2(e) * K Q^T - m for block qb and 32-key sub-tile
    // sb, with the keys past the end of the range masked to -inf.
    auto scores = [&](int qb, int sb) {
      const int row = 32 * sb + l32;
      f32x16 acc = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *(const u32x4*)&lds_k[st][k_off(row, 2 * c + hf)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], acc, 0, 0, 0);
      }
      const float nm = -m[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(acc[r], qscale, nm);
      if (key0 + kBK > tr.k_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = key0 + 32 * sb + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (key >= tr.k_end) acc[r] = -INFINITY;
        }
      }
      return acc;
    };
    // P = exp2(S - delta) rounded to bf16 into the PV operand; returns the
    // lane's fp32 sum of the rounded P (the values the PV product uses).
    const bf16x2 kOnes = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    u32x4 pk[2][2][2];  // [qb][sb][k-chunk] bf16 P^T operands
    auto exp_pack = [&](int qb, int sb, const f32x16& sv, float delta) {
      float acc = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sv[8 * c2 + 2 * e] - delta);
          const float p1 = __builtin_amdgcn_exp2f(sv[8 * c2 + 2 * e + 1] - delta);
          const uint32_t pp = pack_bf16(p0, p1);
          pk[qb][sb][c2][e] = pp;
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes, acc, false);
        }
      return acc;
    };

    // ---- fast path: P = exp2(S) against the current reference max
    float lt[2] = {0.f, 0.f};
    bool slow = (t == 0);
    if (!slow) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) lt[qb] += exp_pack(qb, sb, scores(qb, sb), 0.f);
      slow = __any(!(lt[0] <= kRescaleSum && lt[1] <= kRescaleSum));
    }
    // ---- slow path (first tile, or a tile far above the reference max):
    // recompute S, raise m to the tile max, rescale O and l.
    if (slow) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sv[2] = {scores(qb, 0), scores(qb, 1)};
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[sb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float delta = mset[qb] ? fmaxf(mx, 0.f) : mx;
        const float factor = mset[qb] ? exp2f(-delta) : 1.f;
        m[qb] += delta;
        mset[qb] = true;
        lsum[qb] *= factor;
        o[qb][0] *= factor;
        o[qb][1] *= factor;
        lt[qb] = exp_pack(qb, 0, sv[0], delta) + exp_pack(qb, 1, sv[1], delta);
      }
    }
    lsum[0] += lt[0];
    lsum[1] += lt[1];

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + l32;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, *(const u32x4*)&lds_v[st][v_off(d, 4 * sb + 2 * c2 + hf)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                va, __builtin_bit_cast(bf16x8, pk[qb][sb][c2]), o[qb][db], 0, 0, 0);
        }
    }

    if (t + 1 < ntiles) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- normalise and store O (bf16, RNE)
  uint16_t* __restrict__ og = (uint16_t*)p.o;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.f / l;
    if (qvalid[qb]) {
      uint16_t* dst = og + ((size_t)qrow[qb] * H + head) * 64;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * hf;
          u32x2 w;
          w[0] = pack_bf16(o[qb][db][4 * g + 0] * inv, o[qb][db][4 * g + 1] * inv);
          w[1] = pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          *(u32x2*)(dst + d0) = w;
        }
    }
  }
}

// ----------------------------------------------------------------- fp32 path
constexpr int kF32Threads = 64;

template <KeyRange KR>
__global__ void __launch_bounds__(kF32Threads) flash_f32_kernel(FlashParams p) {
  const int64_t b = blockIdx.x;
  int32_t head;
  int64_t q_begin, q_end, k_begin, k_end;
  if constexpr (KR == KeyRange::kFrame) {
    const int64_t qtpf = (p.L + kF32Threads - 1) / kF32Threads;
    const int64_t per_head = qtpf * p.num_frames;
    head = (int32_t)(b / per_head);
    const int64_t rem = b % per_head;
    const int64_t f = rem / qtpf, qt = rem % qtpf;
    q_begin = f * p.L + qt * kF32Threads;
    q_end = min(q_begin + kF32Threads, (f + 1) * (int64_t)p.L);
    k_begin = f * p.L;
    k_end = (f + 1) * (int64_t)p.L;
  } else {
    const int64_t nqt = (p.num_q + kF32Threads - 1) / kF32Threads;
    head = (int32_t)(b / nqt);
    q_begin = (b % nqt) * kF32Threads;
    q_end = min(q_begin + kF32Threads, p.num_q);
    k_begin = 0;
    k_end = p.num_keys;
  }
  const int64_t row = q_begin + threadIdx.x;
  if (row >= q_end) return;
  const int H = p.H;
  const float* qg = (const float*)p.q;
  const float* kg = (const float*)p.k;
  const float* vg = (const float*)p.v;
  float q[64], acc[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    q[e] = qg[((size_t)row * H + head) * 64 + e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // online softmax in natural-log units; one column at a time
  auto add_column = [&](float z, const float* vrow, float vmul) {
    if (z > m) {
      const float corr = expf(m - z);  // 0 on the first column
      l *= corr;
#pragma unroll
      for (int e = 0; e < 64; ++e) acc[e] *= corr;
      m = z;
    }
    const float w = expf(z - m);
    l += w;
#pragma unroll
    for (int e = 0; e < 64; ++e) acc[e] += w * (vrow[e] * vmul);
  };
  if constexpr (KR == KeyRange::kSga) {
    const float* kf = (const float*)p.k_full;
    const float* vf = (const float*)p.v_full;
    if (p.use_diag && !sga_kept(p.grid, row)) {
      const float* kr = kf + ((size_t)row * H + head) * 64;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e) dot += q[e] * kr[e];
      add_column(dot * p.scale, vf + ((size_t)row * H + head) * 64, 1.f);
    }
    if (p.use_mean) {
      const float* km = p.kmean + head * 64;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e) dot += q[e] * km[e];
      add_column(dot * p.scale + p.log_ndrop, p.vmean + head * 64, 1.f);
    }
  }
  for (int64_t j = k_begin; j < k_end; ++j) {
    const float* kr = kg + ((size_t)j * H + head) * 64;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) dot += q[e] * kr[e];
    add_column(dot * p.scale, vg + ((size_t)j * H + head) * 64, 1.f);
  }
  float* og = (float*)p.o + ((size_t)row * H + head) * 64;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < 64; ++e) og[e] = acc[e] * inv;
}

template <typename KernelT>
int64_t blocks_for(KeyRange kr, const FlashParams& p, int rows_per_block) {
  if (kr == KeyRange::kFrame)
    return (int64_t)p.H * p.num_frames * ((p.L + rows_per_block - 1) / rows_per_block);
  return (int64_t)p.H * ((p.num_q + rows_per_block - 1) / rows_per_block);
}

}  // namespace

hipError_t launch_flash_bf16(KeyRange kr, const FlashParams& p, hipStream_t s) {
  const int64_t nb = blocks_for<void>(kr, p, kBQ);
  if (nb <= 0) return hipSuccess;
  const dim3 grid((uint32_t)nb), block(kThreads);
  switch (kr) {
    case KeyRange::kFrame: hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kFrame>, grid, block, 0, s, p); break;
    case KeyRange::kGlobal: hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kGlobal>, grid, block, 0, s, p); break;
    case KeyRange::kSga: hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kSga>, grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_flash_f32(KeyRange kr, const FlashParams& p, hipStream_t s) {
  const int64_t nb = blocks_for<void>(kr, p, kF32Threads);
  if (nb <= 0) return hipSuccess;
  const dim3 grid((uint32_t)nb), block(kF32Threads);
  switch (kr) {
    case KeyRange::kFrame: hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kFrame>, grid, block, 0, s, p); break;
    case KeyRange::kGlobal: hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kGlobal>, grid, block, 0, s, p); break;
    case KeyRange::kSga: hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kSga>, grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace vga
