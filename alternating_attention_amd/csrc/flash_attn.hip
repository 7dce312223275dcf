// flash_attn.hip -- attention over frames of tokens for gfx950 (MI355X).
//
// One kernel core serves the three attention modes of an alternating-
// attention trunk ("VGGT CVPR25 Best Paper" notes, "Alternating-Attention";
// "AVGGT: Rethinking Global Attention for Accelerating VGGT", section 3):
//   kFrame  -- the keys of a query are the L tokens of its own frame;
//   kGlobal -- the keys are all T tokens; the T x T score matrix only ever
//              exists one 32-key sub-tile at a time in registers;
//   kSga    -- the keys are the compacted kept rows (Kc, Vc); after the
//              key loop each query's diagonal column (own token, when
//              dropped) and the mean column (count-weighted or unit weight)
//              are merged into its softmax state, so the three parts share
//              one softmax.
//
// bf16 path (MFMA).  A workgroup of 8 waves (two per SIMD) owns 512 queries
// of one head; each wave owns 64 queries as two 32-query blocks.  Scores are
// computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys
// index the accumulator rows and queries its columns, so every lane holds
// 16 scores of ONE query.  Row statistics therefore stay in the lane (plus
// its partner lane l^32); the probabilities P^T feed O^T = V^T P^T directly
// as the B operand without touching LDS.  K rows are stored in LDS in a
// permuted order (bits 2 and 3 of the row index swapped) so that accumulator
// register r of lane half h holds key 16*(r/8) + 8*h + r%8 -- exactly the
// B-operand k-slot order of the PV product.  V stays in its natural layout;
// the PV A operand (V^T) comes from ds_read_b64_tr_b16 transposed reads.
// K/V tiles of 128 keys move global -> LDS with global_load_lds_dwordx4 (no
// registers) through a ring of three stages (114 KB: one workgroup per CU);
// a ragged last tile is taken first (softmax sums do not depend on the key
// order), so every later tile is full and needs no masking; the ragged tile
// runs the same pipelined steps with its keys past the end masked.
//
// Software pipeline over 32-key sub-tiles j: step j issues the QK^T MFMAs
// of sub-tile j+1 and the PV MFMAs of sub-tile j-1 while the VALU computes
// the softmax of sub-tile j; the three are independent, and sched barriers
// interleave them one MFMA to one pair of scores, so the matrix core and
// the VALU of one wave run side by side (a second wave per SIMD fills the
// gaps).  Each tile (four steps) costs one barrier, before its fourth step:
// tile t+1 must have landed before its first QK, and tile t+2 then loads
// into the stage of tile t-1, whose last reader (the PV of its last
// sub-tile, in the first step of tile t) ran before that barrier.
//
// Softmax: the MFMA produces exact fp32 dot products of the bf16 rows; one
// FMA per score turns them into log2 units and subtracts the row's
// reference max m.  m is updated lazily: the first sub-tile, or a sub-tile
// whose probabilities sum above 2^16 in a lane, takes a wave-uniform slow
// path that (re)computes its scores, raises m to the sub-tile max and
// rescales O and l (the textbook online softmax); every other sub-tile uses
// P = exp2(S - m) as is.  P is rounded to bf16 (RNE) for the PV MFMA; l
// (summed from the rounded P) and O accumulate in fp32.
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

constexpr int kThreads = 512;          // 8 waves
constexpr int kQPerWave = 64;
constexpr int kBQ = 8 * kQPerWave;     // queries per workgroup
constexpr int kBK = 128;               // keys per LDS tile (4 sub-tiles of 32)
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

// LDS tiles.  K: 128 rows of 128 bytes padded to 144 (row i of a 32-key
// sub-tile holds key perm_row(i)); V: 128 rows (natural key order) padded to
// 160 bytes.  The padding spreads the rows that one LDS read touches over
// distinct banks, and keeps every read address a per-lane base plus an
// immediate.  Both tiles are filled by global_load_lds_dwordx4 (global ->
// LDS without registers), 1 KB (64 x 16 bytes) per instruction; granules
// that fall in the padding load a harmless in-range duplicate.
constexpr int kKRow = 144, kVRow = 160;
constexpr int kKTile = kBK * kKRow, kVTile = kBK * kVRow;     // 18432, 20480
constexpr int kStage = kKTile + kVTile;                        // 38912
constexpr int kKInstr = kKTile / 1024, kVInstr = kVTile / 1024;  // 18, 20
constexpr int kDmaSlots = (kKInstr + kVInstr + 7) / 8;         // per wave: 5
constexpr int kStages = 3;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <KeyRange KR>
__global__ void __launch_bounds__(kThreads, 1) flash_bf16_kernel(FlashParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kStages][kStage];

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
    for (int c = 0; c < 4; ++c)
      qreg[qb][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * c));
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

  // ---- DMA plan: wave w issues the tile's 1 KB instructions w, w+8, ...
  // (0..17: K, 18..37: V).  A lane's granule: key offset within the tile and
  // byte offset within the row.
  auto dma_granule = [&](int i, int& key, uint32_t& col) {
    if (i < kKInstr) {
      const int g = i * 64 + lane, row = g / 9, gc = g % 9;
      key = (row & ~31) + perm_row(row & 31);
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
    dma_granule(8 * s + wave, key, col);
    dma_off[s] = (uint32_t)key * (uint32_t)row_bytes + col;
  }
  const char* kbytes = (const char*)p.k + (int64_t)head * 128;
  const char* vbytes = (const char*)p.v + (int64_t)head * 128;
  // Issue the DMA of the tile at key0 into `stage`; with clamp (the ragged
  // tile) keys past the range load the last key instead.
  auto issue = [&](int64_t key0, int stage, auto clamp_tag) __attribute__((always_inline)) {
    constexpr bool clamp = decltype(clamp_tag)::value;
#pragma unroll
    for (int s = 0; s < kDmaSlots; ++s) {
      const int i = 8 * s + wave;
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
      char* dst = &lds[stage][isk ? i * 1024 : kKTile + (i - kKInstr) * 1024];
      // Issued from asm: the compiler then does not make every later LDS
      // read wait for this DMA (it cannot tell that the reads hit another
      // stage).  Completion is awaited explicitly before each barrier.  The
      // instruction writes LDS only and has no destination registers, so no
      // register can be reused while it is in flight; its address
      // registers are read at issue (as for the builtin form).
      const uint32_t ldsa = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "s"(ldsa)
                   : "memory", "m0");
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

  // ---- building blocks on one 32-key sub-tile (sb of the tile in stage st)
  // S^T (raw dot products) of both query blocks
  auto qk = [&](int st, int sb, f32x16 (&S)[2]) __attribute__((always_inline)) {
    const char* sk = &lds[st][0] + kread + sb * 32 * kKRow;
    S[0] = 0.f;
    S[1] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(sk + c * 32));
      S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[0][c], S[0], 0, 0, 0);
      S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[1][c], S[1], 0, 0, 0);
    }
  };
  // O^T += V^T P^T; the V^T operand comes from two transposed reads
  auto pv = [&](int st, int sb, const u32x4 (&P)[2][2]) __attribute__((always_inline)) {
    const char* sv = &lds[st][0] + vread + sb * 32 * kVRow;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const char* a = sv + 16 * c2 * kVRow + db * 64;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 4 * kVRow));
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              va, __builtin_bit_cast(bf16x8, P[qb][c2]), o[qb][db], 0, 0, 0);
      }
  };
  // P = exp2(qscale*S - m - delta) rounded to bf16 into the PV operand;
  // returns the lane's fp32 sum of the rounded P.  Tail: keys at or past the
  // end of the range get P = 0.
  auto exp_pack = [&](int qb, const f32x16& S, float delta, u32x4 (&P)[2], int64_t key0,
                      auto tail_tag) __attribute__((always_inline)) {
    constexpr bool tail = decltype(tail_tag)::value;
    const float nm = -(m[qb] + delta);
    float acc = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float z0 = __builtin_fmaf(S[8 * c2 + 2 * e], qscale, nm);
        float z1 = __builtin_fmaf(S[8 * c2 + 2 * e + 1], qscale, nm);
        if constexpr (tail) {
          const int64_t k0 = key0 + 16 * c2 + 8 * hf + 2 * e;
          if (k0 >= tr.k_end) z0 = -INFINITY;
          if (k0 + 1 >= tr.k_end) z1 = -INFINITY;
        }
        const uint32_t pp = pack_bf16(__builtin_amdgcn_exp2f(z0), __builtin_amdgcn_exp2f(z1));
        P[c2][e] = pp;
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes, acc, false);
      }
    return acc;
  };
  // Softmax of one sub-tile: the fast path uses the reference max m as is;
  // the first sub-tile, or one whose probabilities sum above 2^16 in a lane,
  // raises m to the sub-tile max (and rescales O and l) and redoes P.
  auto softmax = [&](const f32x16 (&S)[2], u32x4 (&P)[2][2], bool first, int64_t key0,
                     auto tail_tag) __attribute__((always_inline)) {
    float lt[2] = {0.f, 0.f};
    bool slow = first;
    if (!slow) {
      lt[0] = exp_pack(0, S[0], 0.f, P[0], key0, tail_tag);
      lt[1] = exp_pack(1, S[1], 0.f, P[1], key0, tail_tag);
      slow = __any(!(lt[0] <= kRescaleSum && lt[1] <= kRescaleSum));
    }
    if (slow) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float rmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = S[qb][r];
          if constexpr (decltype(tail_tag)::value) {
            const int64_t key = key0 + 16 * (r >> 3) + 8 * hf + (r & 7);
            if (key >= tr.k_end) x = -INFINITY;
          }
          rmax = fmaxf(rmax, x);
        }
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
        const float mx = rmax == -INFINITY ? -INFINITY : __builtin_fmaf(rmax, qscale, -m[qb]);
        // a fully masked sub-tile (tail) leaves the state unchanged
        const float delta = mx == -INFINITY ? 0.f : (mset[qb] ? fmaxf(mx, 0.f) : mx);
        const float factor = mset[qb] ? exp2f(-delta) : 1.f;
        m[qb] += delta;
        mset[qb] = mset[qb] || mx != -INFINITY;
        lsum[qb] *= factor;
        o[qb][0] *= factor;
        o[qb][1] *= factor;
        lt[qb] = exp_pack(qb, S[qb], 0.f, P[qb], key0, tail_tag);
      }
    }
    lsum[0] += lt[0];
    lsum[1] += lt[1];
  };

  // Steady-state step, fast path, unit by unit: QK of the next sub-tile
  // (K at stK/sbK) and PV of the previous one (V at stV/sbV, operand Pp)
  // on the matrix core, each MFMA followed by one pair of this sub-tile's
  // softmax (scores Sc -> Pc); the sched barriers pin that order.  Returns
  // the lane sums of the rounded P in lt.  Tail: the sub-tile's keys start
  // at key0 and those at or past the end of the range get P = 0.
  auto step_fast = [&](int stK, int sbK, int stV, int sbV, const f32x16 (&Sc)[2],
                       u32x4 (&Pc)[2][2], f32x16 (&Sn)[2], const u32x4 (&Pp)[2][2],
                       float (&lt)[2], int64_t key0, auto tail_tag) __attribute__((always_inline)) {
    constexpr bool tail = decltype(tail_tag)::value;
    const char* sk = &lds[stK][0] + kread + sbK * 32 * kKRow;
    const char* sv = &lds[stV][0] + vread + sbV * 32 * kVRow;
    // PV units first (they free Pp), then the QK units (they fill Sn); the
    // operand of each MFMA pair is read from LDS two units ahead
    bf16x8 va[2][2], ka[4];
    auto load_v = [&](int db, int c2) __attribute__((always_inline)) {
      const char* a = sv + 16 * c2 * kVRow + db * 64;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 4 * kVRow));
      va[db][c2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto load_k = [&](int c) __attribute__((always_inline)) {
      ka[c] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(sk + c * 32));
    };
    const float nm0 = -m[0], nm1 = -m[1];
    lt[0] = 0.f;
    lt[1] = 0.f;
    auto pair = [&](int u) __attribute__((always_inline)) {
      const int qb = u >> 3, c2 = (u >> 2) & 1, e = u & 3;
      const float nm = qb ? nm1 : nm0;
      float z0 = __builtin_fmaf(Sc[qb][8 * c2 + 2 * e], qscale, nm);
      float z1 = __builtin_fmaf(Sc[qb][8 * c2 + 2 * e + 1], qscale, nm);
      if constexpr (tail) {
        const int64_t k0 = key0 + 16 * c2 + 8 * hf + 2 * e;
        if (k0 >= tr.k_end) z0 = -INFINITY;
        if (k0 + 1 >= tr.k_end) z1 = -INFINITY;
      }
      const uint32_t pp = pack_bf16(__builtin_amdgcn_exp2f(z0), __builtin_amdgcn_exp2f(z1));
      Pc[qb][c2][e] = pp;
      lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes, lt[qb],
                                               false);
    };
    load_v(0, 0);
    load_v(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // PV unit: operand (db, c2) for query block qb
      const int db = u >> 2, c2 = (u >> 1) & 1, qb = u & 1;
      if (u == 1) load_v(1, 0);
      if (u == 3) load_v(1, 1);
      if (u == 5) load_k(0);
      if (u == 6) load_k(1);
      pair(u);
      o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va[db][c2], __builtin_bit_cast(bf16x8, Pp[qb][c2]), o[qb][db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 8; u < 16; ++u) {
      // QK unit: k-step c for query block qb
      const int w = u - 8, c = w >> 1, qb = w & 1;
      if (w == 1) load_k(2);
      if (w == 3) load_k(3);
      pair(u);
      Sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qreg[qb][c],
                                                       c == 0 ? f32x16(0.f) : Sn[qb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the rare exact redo after a fast step: raise m to the sub-tile max
  // (O and l rescaled) and recompute P
  // (tail: only the keys before the end of the range count; the sub-tile
  // is never the first, so m is set and a fully masked one changes nothing)
  auto redo_exact = [&](const f32x16 (&S)[2], u32x4 (&P)[2][2], float (&lt)[2], int64_t key0,
                        auto tail_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float rmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = S[qb][r];
        if constexpr (decltype(tail_tag)::value) {
          if (key0 + 16 * (r >> 3) + 8 * hf + (r & 7) >= tr.k_end) x = -INFINITY;
        }
        rmax = fmaxf(rmax, x);
      }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      const float mx = __builtin_fmaf(rmax, qscale, -m[qb]);
      const float delta = mset[qb] ? fmaxf(mx, 0.f) : mx;
      const float factor = mset[qb] ? exp2f(-delta) : 1.f;
      m[qb] += delta;
      mset[qb] = true;
      lsum[qb] *= factor;
      o[qb][0] *= factor;
      o[qb][1] *= factor;
      lt[qb] = exp_pack(qb, S[qb], 0.f, P[qb], key0, tail_tag);
    }
  };

  // ---- software pipeline over 32-key sub-tiles j (four per LDS tile): step
  // j runs QK of sub-tile j+1 and PV of sub-tile j-1 on the matrix core
  // while the VALU computes the softmax of sub-tile j.  Three LDS stages:
  // tile t+2 loads into the stage of tile t-1, whose last reader (the PV of
  // its last sub-tile) ran before the barrier that precedes the load.
  f32x16 Sa[2], Sb[2];
  u32x4 Pa[2][2], Pb[2][2];
  // Tile order: the ragged tail first (if any), then the full tiles; the
  // softmax sums do not depend on the key order.
  const bool has_tail = ntiles > nfull;
  auto tile_key0 = [&](int64_t i) __attribute__((always_inline)) {
    return has_tail ? (i == 0 ? tr.k_begin + nfull * kBK : tr.k_begin + (i - 1) * kBK)
                    : tr.k_begin + i * kBK;
  };
  auto issue_tile = [&](int64_t i, int st) __attribute__((always_inline)) {
    if (has_tail && i == 0)
      issue(tile_key0(0), st, std::true_type{});
    else
      issue(tile_key0(i), st, std::false_type{});
  };
  issue_tile(0, 0);
  if (ntiles > 1) issue_tile(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // fast pipeline step: QK -> Sn (stage stK, sub sbK), PV of Pp (stage stV,
  // sub sbV), softmax Sc -> Pc of the full sub-tile in stage stC, sub sbC
  // (tail: the same with the sub-tile's keys starting at key0 masked at the
  // end of the range)
  auto step_m = [&](int stK, int sbK, int stV, int sbV, int stC, int sbC, const f32x16 (&Sc)[2],
                    u32x4 (&Pc)[2][2], f32x16 (&Sn)[2], const u32x4 (&Pp)[2][2], int64_t key0,
                    auto tail_tag) __attribute__((always_inline)) {
    float lt[2];
    step_fast(stK, sbK, stV, sbV, Sc, Pc, Sn, Pp, lt, key0, tail_tag);
    if (__any(!(lt[0] <= kRescaleSum && lt[1] <= kRescaleSum))) {
      // rare: recompute this sub-tile's scores (its tile is still in LDS)
      f32x16 Sr[2];
      qk(stC, sbC, Sr);
      redo_exact(Sr, Pc, lt, key0, tail_tag);
    }
    lsum[0] += lt[0];
    lsum[1] += lt[1];
  };
  auto step = [&](int stK, int sbK, int stV, int sbV, int stC, int sbC, const f32x16 (&Sc)[2],
                  u32x4 (&Pc)[2][2], f32x16 (&Sn)[2], const u32x4 (&Pp)[2][2])
      __attribute__((always_inline)) {
    step_m(stK, sbK, stV, sbV, stC, sbC, Sc, Pc, Sn, Pp, 0, std::false_type{});
  };
  // tile t+1 must have landed before its first QK; tile t+2 then loads into
  // the stage of tile t-1
  auto advance = [&](int64_t t, int st_prev) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (t + 2 < ntiles) issue_tile(t + 2, st_prev);
  };
  // ---- tile 0 (the ragged tail when there is one): steps 0..3
  const int64_t key00 = tile_key0(0);
  const int st1 = ntiles > 1 ? 1 : 0;  // QK target of step 3 (a dummy re-read if no tile 1)
  qk(0, 0, Sa);
  if (has_tail) {
    qk(0, 1, Sb);
    softmax(Sa, Pa, true, key00, std::true_type{});
    step_m(0, 2, 0, 0, 0, 1, Sb, Pb, Sa, Pa, key00 + 32, std::true_type{});
    step_m(0, 3, 0, 1, 0, 2, Sa, Pa, Sb, Pb, key00 + 64, std::true_type{});
    if (ntiles > 1) advance(0, kStages - 1);
    step_m(st1, 0, 0, 2, 0, 3, Sb, Pb, Sa, Pa, key00 + 96, std::true_type{});
  } else {
    qk(0, 1, Sb);
    softmax(Sa, Pa, true, key00, std::false_type{});
    step(0, 2, 0, 0, 0, 1, Sb, Pb, Sa, Pa);
    step(0, 3, 0, 1, 0, 2, Sa, Pa, Sb, Pb);
    if (ntiles > 1) advance(0, kStages - 1);
    step(st1, 0, 0, 2, 0, 3, Sb, Pb, Sa, Pa);
  }
  // ---- full tiles 1 .. ntiles-1: steps 4t .. 4t+3
  int st = 0;
  for (int64_t t = 1; t < ntiles; ++t) {
    const int st_prev = st;
    st = st == kStages - 1 ? 0 : st + 1;
    const int st_next = st == kStages - 1 ? 0 : st + 1;
    const bool has_next = t + 1 < ntiles;
    step(st, 1, st_prev, 3, st, 0, Sa, Pa, Sb, Pb);  // QK(t,1) | PV(t-1,3) | softmax(t,0)
    step(st, 2, st, 0, st, 1, Sb, Pb, Sa, Pa);       // QK(t,2) | PV(t,0)   | softmax(t,1)
    step(st, 3, st, 1, st, 2, Sa, Pa, Sb, Pb);       // QK(t,3) | PV(t,1)   | softmax(t,2)
    if (has_next) advance(t, st_prev);
    // QK(t+1,0) | PV(t,2) | softmax(t,3); the QK re-reads this tile when t is last
    step(has_next ? st_next : st, 0, st, 2, st, 3, Sb, Pb, Sa, Pa);
  }
  pv(st, 3, Pb);  // drain

  // This wave's first query row, recomputed here: the value from the Q load
  // would otherwise be kept, in registers or scratch, across the loop.
  int64_t row0 = tr.q_begin + wave * kQPerWave + l32;
  asm volatile("" : "+v"(row0));

  if constexpr (KR == KeyRange::kSga) {
    // The diagonal and mean columns join each query's shared softmax here,
    // merged into (m, l, O) after the compacted keys (the softmax sums do not
    // depend on the column order).
    const uint16_t* kf = (const uint16_t*)p.k_full;
    const uint16_t* vf = (const uint16_t*)p.v_full;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t row = min(row0 + qb * 32, tr.q_end - 1);
      const bool diag = p.use_diag && !sga_kept(p.grid, p.row0 + row);
      const uint16_t* ks = kf + ((size_t)row * H + head) * 64 + 8 * hf;
      const float* kms = p.kmean + head * 64 + 8 * hf;
      float dk = 0.f, dm = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 wq = __builtin_bit_cast(u32x4, qreg[qb][c]);  // dims 16c + 8hf + [0, 8)
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
        float mn = mset[qb] ? m[qb] : -INFINITY;
        if (diag) mn = fmaxf(mn, zd);
        if (p.use_mean) mn = fmaxf(mn, zm);
        const float f = mset[qb] ? exp2f(m[qb] - mn) : 0.f;
        const float wd = diag ? exp2f(zd - mn) : 0.f;
        const float wm = p.use_mean ? exp2f(zm - mn) : 0.f;
        lsum[qb] = lsum[qb] * f + (hf == 0 ? wd + wm : 0.f);
        const uint16_t* vs = vf + ((size_t)row * H + head) * 64;
        const float* vms = p.vmean + head * 64;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hf;
            const u32x2 wv = *(const u32x2*)(vs + d0);
            const f32x4 mv = *(const f32x4*)(vms + d0);
            o[qb][db][4 * g + 0] = o[qb][db][4 * g + 0] * f + wd * bf16_lo(wv[0]) + wm * mv[0];
            o[qb][db][4 * g + 1] = o[qb][db][4 * g + 1] * f + wd * bf16_hi(wv[0]) + wm * mv[1];
            o[qb][db][4 * g + 2] = o[qb][db][4 * g + 2] * f + wd * bf16_lo(wv[1]) + wm * mv[2];
            o[qb][db][4 * g + 3] = o[qb][db][4 * g + 3] * f + wd * bf16_hi(wv[1]) + wm * mv[3];
          }
      }
    }
  }

  // ---- normalise and store O (bf16, RNE)
  uint16_t* __restrict__ og = (uint16_t*)p.o;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.f / l;
    const int64_t row = row0 + qb * 32;
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

int64_t blocks_for(KeyRange kr, const FlashParams& p, int rows_per_block) {
  if (kr == KeyRange::kFrame)
    return (int64_t)p.H * p.num_frames * ((p.L + rows_per_block - 1) / rows_per_block);
  return (int64_t)p.H * ((p.num_q + rows_per_block - 1) / rows_per_block);
}

}  // namespace

hipError_t launch_flash_bf16(KeyRange kr, const FlashParams& p, hipStream_t s) {
  const int64_t nb = blocks_for(kr, p, kBQ);
  if (nb <= 0) return hipSuccess;
  const dim3 grid((uint32_t)nb), block(kThreads);
  switch (kr) {
    case KeyRange::kFrame:
      hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kFrame>, grid, block, 0, s, p);
      break;
    case KeyRange::kGlobal:
      hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kGlobal>, grid, block, 0, s, p);
      break;
    case KeyRange::kSga:
      hipLaunchKernelGGL(flash_bf16_kernel<KeyRange::kSga>, grid, block, 0, s, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_flash_f32(KeyRange kr, const FlashParams& p, hipStream_t s) {
  const int64_t nb = blocks_for(kr, p, kF32Threads);
  if (nb <= 0) return hipSuccess;
  const dim3 grid((uint32_t)nb), block(kF32Threads);
  switch (kr) {
    case KeyRange::kFrame:
      hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kFrame>, grid, block, 0, s, p);
      break;
    case KeyRange::kGlobal:
      hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kGlobal>, grid, block, 0, s, p);
      break;
    case KeyRange::kSga:
      hipLaunchKernelGGL(flash_f32_kernel<KeyRange::kSga>, grid, block, 0, s, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace vga
