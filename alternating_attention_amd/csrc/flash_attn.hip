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
// B-operand k-slot order of the PV product.  V stays in its natural layout;
// the PV A operand (V^T) comes from ds_read_b64_tr_b16 transposed reads.
// K/V tiles move global -> LDS with global_load_lds_dwordx4 (no registers),
// double buffered: tile t+1 loads while tile t is computed.
//
// Softmax: the MFMA produces exact fp32 dot products of the bf16 rows; one
// FMA per score turns them into log2 units and subtracts the row's
// reference max m.  m is updated lazily: the first tile, or a tile whose
// probabilities sum above 2^16 in a lane, takes a wave-uniform slow path
// that recomputes S, raises m to the tile max and rescales O and l (the
// textbook online softmax); every other tile uses P = exp2(S - m) as is.
// P is rounded to bf16 (RNE) for the PV MFMA; l (summed from the rounded P)
// and O accumulate in fp32.
//
// fp32 path: a plain VALU kernel (one lane per query and head, exact online
// softmax in fp32), used for fp32 inputs.
#include <type_traits>

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


struct TileRange {
  int64_t q_begin, q_end;    // query rows of this workgroup
  int64_t k_begin, k_end;    // key rows
  int32_t head;
};

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8), each with its own L2.  Logical tile order gives every XCD one
// contiguous range, so the query tiles that share a frame's or a head's K/V
// run on the same XCD at about the same time.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nblocks) {
  constexpr int64_t kXcds = 8;
  const int64_t q = nblocks / kXcds, r = nblocks % kXcds;
  const int64_t x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

template <KeyRange KR>
__device__ __forceinline__ TileRange tile_range(const FlashParams& p) {
  TileRange t;
  const int64_t b = xcd_remap(blockIdx.x, gridDim.x);
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

// LDS tiles.  K: 64 rows of 128 bytes padded to 144 (row i of a 32-key
// sub-tile holds key perm_row(i)); V: 64 rows (natural key order) padded to
// 160 bytes.  The padding spreads the rows that one LDS read touches over
// distinct banks, and keeps every read address a per-lane base plus an
// immediate.  Both tiles are filled by global_load_lds_dwordx4 (global ->
// LDS without registers), 1 KB (64 x 16 bytes) per instruction; granules
// that fall in the padding load a harmless in-range duplicate.
constexpr int kKRow = 144, kVRow = 160;
constexpr int kKTile = kBK * kKRow, kVTile = kBK * kVRow;     // 9216, 10240
constexpr int kStage = kKTile + kVTile;                        // 19456
constexpr int kKInstr = kKTile / 1024, kVInstr = kVTile / 1024;  // 9, 10
constexpr int kDmaSlots = (kKInstr + kVInstr + 3) / 4;         // per wave: 5
constexpr int kStages = 2;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <KeyRange KR>
__global__ void __launch_bounds__(kThreads, 2) flash_bf16_kernel(FlashParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStage];

  const TileRange tr = tile_range<KR>(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half: k-group of the MFMA operands
  const int H = p.H;
  const int head = tr.head;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
  const float qscale = p.scale * kLog2e;
  const int64_t row_bytes = (int64_t)H * 128;

  // ---- Q block of this wave into registers (B operand of S^T = K Q^T):
  // lane holds query l32 of block qb (clamped into range), dims
  // 16c + 8*hf + [0, 8), as stored.
  bf16x8 qreg[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t row = min(tr.q_begin + wave * kQPerWave + qb * 32 + l32, tr.q_end - 1);
    const uint16_t* src = qg + ((size_t)row * H + head) * 64 + 8 * hf;
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
      const int64_t row = min(tr.q_begin + wave * kQPerWave + qb * 32 + l32, tr.q_end - 1);
      const bool diag = p.use_diag && !sga_kept(p.grid, p.row0 + row);
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

  // ---- DMA plan: wave w issues the tile's 1 KB instructions w, w+4, ...
  // (0..8: K, 9..18: V).  A lane's granule: key offset within the tile and
  // byte offset within the row.
  auto dma_granule = [&](int i, int& key, uint32_t& col) {
    if (i < kKInstr) {
      const int g = i * 64 + lane, row = g / 9, gc = g % 9;
      key = (row & 32) + perm_row(row & 31);
      col = gc < 8 ? gc * 16 : 0;
    } else {
      const int g = (i - kKInstr) * 64 + lane, row = g / 10, gc = g % 10;
      key = row;
      col = gc < 8 ? gc * 16 : 0;
    }
  };
  uint32_t dma_off[kDmaSlots];
#pragma unroll
  for (int s = 0; s < kDmaSlots; ++s) {
    int key;
    uint32_t col;
    dma_granule(4 * s + wave, key, col);
    dma_off[s] = (uint32_t)key * (uint32_t)row_bytes + col;
  }
  const char* kbytes = (const char*)p.k + (int64_t)head * 128;
  const char* vbytes = (const char*)p.v + (int64_t)head * 128;
  // Issue the DMA of the tile at key0 into `stage`; with clamp (ragged last
  // tile) keys past the range load the last key instead.
  auto issue = [&](int64_t key0, int stage, auto clamp_tag) {
    constexpr bool clamp = decltype(clamp_tag)::value;
#pragma unroll
    for (int s = 0; s < kDmaSlots; ++s) {
      const int i = 4 * s + wave;
      if (i >= kKInstr + kVInstr) continue;
      const bool isk = i < kKInstr;
      const char* base = isk ? kbytes : vbytes;
      const char* src;
      if constexpr (clamp) {
        int kk;
        uint32_t col;
        dma_granule(i, kk, col);
        int64_t key = key0 + kk;
        key = key < tr.k_end ? key : tr.k_end - 1;
        src = base + key * row_bytes + col;
      } else {
        src = base + key0 * row_bytes + dma_off[s];
      }
      char* dst = lds + stage * kStage + (isk ? i * 1024 : kKTile + (i - kKInstr) * 1024);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  // per-lane LDS read bases: K operand (row l32 of a sub-tile, granule hf)
  // and the V^T transposed read (16-lane group g reads 4 keys x 16 dims).
  const int kread = l32 * kKRow + hf * 16;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vread = kKTile + (8 * hf + (j16 >> 2)) * kVRow + (16 * (g16 & 1) + 4 * (j16 & 3)) * 2;

  const int64_t nkeys = tr.k_end - tr.k_begin;
  const int64_t nfull = nkeys / kBK;
  const int64_t ntiles = (nkeys + kBK - 1) / kBK;
  const bf16x2 kOnes = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // One key tile.  Full tiles run without any masking; a ragged last tile
  // (tail) runs the same body with its out-of-range keys masked to -inf.
  auto tile_step = [&](int64_t t, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    const int st = (int)(t & 1);
    const int64_t key0 = tr.k_begin + t * kBK;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA landed
    __syncthreads();                     // ... and every other wave's
    if (t + 1 < ntiles) {
      if (t + 1 == nfull)
        issue(key0 + kBK, st ^ 1, std::true_type{});
      else
        issue(key0 + kBK, st ^ 1, std::false_type{});
    }
    const char* sk = lds + st * kStage + kread;
    const char* sv = lds + st * kStage + vread;

    // ---- S^T = scale*log2(e) * K Q^T - m for block qb and 32-key sub-tile
    // sb; keys past the end of the range (tail tile only) get -inf.
    auto scores = [&](int qb, int sb) {
      f32x16 acc = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(sk + sb * 32 * kKRow + c * 32));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], acc, 0, 0, 0);
      }
      const float nm = -m[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = __builtin_fmaf(acc[r], qscale, nm);
      if constexpr (tail) {
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
    u32x4 pk[2][2][2];  // [qb][sb][k-chunk] bf16 P^T operands
    auto exp_pack = [&](int qb, int sb, const f32x16& sv2, float delta) {
      float acc = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sv2[8 * c2 + 2 * e] - delta);
          const float p1 = __builtin_amdgcn_exp2f(sv2[8 * c2 + 2 * e + 1] - delta);
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
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) lt[qb] += exp_pack(qb, sb, scores(qb, sb), 0.f);
      slow = __any(!(lt[0] <= kRescaleSum && lt[1] <= kRescaleSum));
    }
    // ---- slow path (first tile, or a tile far above the reference max):
    // recompute S, raise m to the tile max, rescale O and l.
    if (slow) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sv2[2] = {scores(qb, 0), scores(qb, 1)};
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv2[sb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float delta = mset[qb] ? fmaxf(mx, 0.f) : mx;
        const float factor = mset[qb] ? exp2f(-delta) : 1.f;
        m[qb] += delta;
        mset[qb] = true;
        lsum[qb] *= factor;
        o[qb][0] *= factor;
        o[qb][1] *= factor;
        lt[qb] = exp_pack(qb, 0, sv2[0], delta) + exp_pack(qb, 1, sv2[1], delta);
      }
    }
    lsum[0] += lt[0];
    lsum[1] += lt[1];

    // ---- O^T += V^T P^T; the V^T operand comes from two transposed reads
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const char* a = sv + (32 * sb + 16 * c2) * kVRow + db * 64;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 4 * kVRow));
          const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                va, __builtin_bit_cast(bf16x8, pk[qb][sb][c2]), o[qb][db], 0, 0, 0);
        }
  };
  if (nfull == 0)
    issue(tr.k_begin, 0, std::true_type{});
  else
    issue(tr.k_begin, 0, std::false_type{});
  for (int64_t t = 0; t < nfull; ++t) tile_step(t, std::false_type{});
  if (ntiles > nfull) tile_step(nfull, std::true_type{});

  // ---- normalise and store O (bf16, RNE)
  uint16_t* __restrict__ og = (uint16_t*)p.o;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.f / l;
    const int64_t row = tr.q_begin + wave * kQPerWave + qb * 32 + l32;
    if (row < tr.q_end) {
      uint16_t* dst = og + ((size_t)row * H + head) * 64;
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
    if (p.use_diag && !sga_kept(p.grid, p.row0 + row)) {
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
