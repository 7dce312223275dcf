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
// of one head; each wave owns 64 queries as two 32-query blocks (a ragged
// frame workgroup spreads its blocks over the SIMDs instead, and waves skip
// the products of blocks they lack).  Scores are
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
// registers) through a ring of three stages (102 KB: one workgroup per CU);
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
// reference max m, the exact max of the first sub-tile (online softmax with
// the reference fixed early: the sums need m only as a common shift, and the
// first sub-tile's max keeps every later P = exp2(S - m) finite unless a
// score exceeds it by 128 in log2 units).  P is rounded to bf16 (RNE) for
// the PV MFMA; O accumulates in fp32, and so do the row sums of the rounded
// P, on the matrix core (a 16x16x32 MFMA against a 0/1 operand; see rowsum).
// The step keeps no per-step max test: after the key loop every wave checks
// that its row sums and output accumulators are finite, and if any wave of
// the workgroup finds otherwise, all redo their rows with the exact online
// softmax one sub-tile at a time (max update, rescale of O and l), where
// every P is at most 1.
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (RNE) and pack them (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// The same conversion (v_cvt_pk_bf16_f32 rounds to nearest even, S0 into
// the low half) as one instruction placed where it stands, right after the
// exps that produce its operands, with the one wait state their results
// need.  Left to itself the compiler gathers four such conversions into a
// group once all four pairs exist, which serialises the step's end.
__device__ __forceinline__ uint32_t pack_bf16_now(float lo, float hi) {
  uint32_t r;
  asm("s_nop 0\n\tv_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
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

// A workgroup-uniform 64-bit value, stated as such: the 64-bit divisions
// that derive the tile bounds run on the VALU, and without this the results
// would stay in vector registers for the whole kernel.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8), each with its own L2.  Logical tile order gives every XCD one
// contiguous range, so the query tiles that share a frame's or a head's K/V
// run on the same XCD at about the same time.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
  constexpr uint32_t kXcds = 8;
  const uint32_t q = nblocks / kXcds, r = nblocks % kXcds;
  const uint32_t x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

// The workgroup's tile range.  Block, frame and tile counts are below 2^31
// (T < 2^31), so the index arithmetic runs in 32 bits: 64-bit divisions
// here cost about 2 % of a frame-attention workgroup.
template <KeyRange KR>
__device__ __forceinline__ TileRange tile_range(const FlashParams& p) {
  TileRange t;
  const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
  if constexpr (KR == KeyRange::kFrame) {
    const uint32_t qtpf = ((uint32_t)p.L + kBQ - 1) / kBQ;
    const uint32_t per_head = qtpf * (uint32_t)p.num_frames;
    const uint32_t head = b / per_head, rem = b - head * per_head;
    const uint32_t f = rem / qtpf, qt = rem - f * qtpf;
    t.head = (int32_t)head;
    t.k_begin = (int64_t)f * p.L;
    t.k_end = t.k_begin + p.L;
    t.q_begin = t.k_begin + (int64_t)qt * kBQ;
    t.q_end = min(t.q_begin + kBQ, t.k_end);
  } else {
    const uint32_t nqt = (uint32_t)((p.num_q + kBQ - 1) / kBQ);
    const uint32_t head = b / nqt;
    t.head = (int32_t)head;
    t.q_begin = (int64_t)(b - head * nqt) * kBQ;
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

// LDS tiles (the LDS has 64 four-byte banks).
//  K: 128 rows of 128 bytes padded to 144 (row i of a 32-key sub-tile holds
//     key perm_row(i)).  The padding puts the 16 rows that one pass of a
//     ds_read_b128 touches on distinct banks.
//  V: 128 rows of 128 bytes in natural key order, the two 64-byte halves of
//     a row swapped when bit 1 of its index is set.  A transposed read
//     (ds_read_b64_tr_b16) takes 64 bytes from each of four consecutive
//     rows per pass; without the swap rows r and r+2 would share banks (with
//     160-byte padded rows, 2 of the read's 4 LDS cycles were conflicts).
// Every read address is a per-lane base plus an immediate.  Both tiles are
// filled by global_load_lds_dwordx4 (global -> LDS without registers), 1 KB
// (64 x 16 bytes) per instruction; granules that fall in K's padding load a
// harmless in-range duplicate.
constexpr int kKRow = 144, kVRow = 128;
constexpr int kKTile = kBK * kKRow, kVTile = kBK * kVRow;     // 18432, 16384
constexpr int kStage = kKTile + kVTile;                        // 34816
constexpr int kKInstr = kKTile / 1024, kVInstr = kVTile / 1024;  // 18, 16
constexpr int kDmaSlots = (kKInstr + kVInstr + 7) / 8;         // per wave: 5
constexpr int kStages = 3;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <KeyRange KR>
__global__ void __launch_bounds__(kThreads, 1) flash_bf16_kernel(FlashParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kStages][kStage];
  __shared__ int fallback;  // set when some wave's rows need the exact loop

  TileRange tr = tile_range<KR>(p);
  tr.q_begin = uniform64(tr.q_begin);
  tr.q_end = uniform64(tr.q_end);
  tr.k_begin = uniform64(tr.k_begin);
  tr.k_end = uniform64(tr.k_end);
  tr.head = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)tr.head);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform: the DMA slot choices below become scalar branches
  const int wave = (int)__builtin_amdgcn_readfirstlane((uint32_t)tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half: k-group of the MFMA operands
  const int H = p.H;
  const int head = tr.head;
  const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
  const float qscale = p.scale * kLog2e;
  const int64_t row_bytes = (int64_t)H * 128;

  // ---- this wave's query blocks (32 rows each, at most two).  In a full
  // workgroup wave w has rows 64w .. 64w+63.  In frame attention a ragged
  // workgroup (nb < 16 blocks: a 1,374-token frame's last 350 rows are 11)
  // spreads its blocks over the four SIMDs as evenly as possible: SIMD s
  // (waves s and s+4) takes nb/4 blocks, or one more for s < nb%4, wave s
  // up to two of them, and blocks are numbered in wave order.  A workgroup
  // lasts as long as its busiest SIMD's products, and the key loop skips
  // the products of absent blocks (a wave with one block runs the
  // one-block step, a wave with none only its share of the tile DMA and the
  // barriers).  Global and SGA attention, whose only ragged workgroup is a
  // head's last, keep two blocks per wave.
  int64_t wq_begin = tr.q_begin + wave * kQPerWave;   // this wave's rows
  int64_t wq_end = tr.q_end;                           // (stores stop here)
  int nblk = 2;
  if constexpr (KR == KeyRange::kFrame) {
    const int nb = (int)((tr.q_end - tr.q_begin + 31) >> 5);  // 1 .. 16
    int first_blk = 0;
    for (int w = 0; w <= wave; ++w) {
      const int cs = (nb >> 2) + ((w & 3) < (nb & 3) ? 1 : 0);
      const int n0 = cs < 2 ? cs : 2;
      const int nw = w < 4 ? n0 : cs - n0;
      if (w < wave)
        first_blk += nw;
      else
        nblk = nw;
    }
    wq_begin = tr.q_begin + 32 * first_blk;
    wq_end = min(wq_begin + 32 * nblk, tr.q_end);
  }

  // ---- Q block of this wave into registers (B operand of S^T = K Q^T):
  // lane holds query l32 of block qb (clamped into the workgroup's rows),
  // dims 16c + 8*hf + [0, 8), as stored.
  bf16x8 qreg[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t row = min(wq_begin + qb * 32 + l32, tr.q_end - 1);
    const uint16_t* src = qg + ((size_t)row * H + head) * 64 + 8 * hf;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qreg[qb][c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * c));
  }

  // ---- softmax state.  Lane (l32, hf) of block qb holds, for its query:
  // o[qb][db] register r = O^T[d][q] with d = 32*db + 8*(r/4) + 4*hf + r%4;
  // m = reference max (log2 units).  Row sums: in the main loop, lrs[qb]
  // (a 16x16 MFMA accumulator, see rowsum below); in the exact fallback
  // loop, lsum[qb] = this lane's share of the row sum.
  f32x16 o[2][2];
  float lsum[2], m[2];
  bool mset[2];
  f32x4 lrs[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    o[qb][0] = 0.f;
    o[qb][1] = 0.f;
    lsum[qb] = 0.f;
    m[qb] = 0.f;
    mset[qb] = false;
    lrs[qb] = 0.f;
  }
  if (tid == 0) fallback = 0;  // published by the first barrier below

  // ---- DMA plan: wave w issues the tile's 1 KB instructions w, w+8, ...
  // (0..17: K, 18..33: V).  A lane's granule: key offset within the tile and
  // byte offset within the row.
  auto dma_granule = [&](int i, int& key, uint32_t& col) {
    if (i < kKInstr) {
      const int g = i * 64 + lane, row = g / 9, gc = g % 9;
      key = (row & ~31) + perm_row(row & 31);
      col = gc < 8 ? gc * 16 : 0;
    } else {
      const int g = (i - kKInstr) * 64 + lane, row = g >> 3;
      key = row;
      col = (uint32_t)(((g & 7) ^ (row & 2 ? 4 : 0)) * 16);
    }
  };
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
        // the lane's granule, recomputed per tile (a few integer ops; kept
        // in registers across the loop it would cost ten of them)
        int kk;
        uint32_t col;
        dma_granule(i, kk, col);
        src = base + key0 * row_bytes + ((uint32_t)kk * (uint32_t)row_bytes + col);
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
  // and the V^T transposed read (16-lane group g reads 4 keys x 16 dims),
  // one base per 32-dim half db.  The lane's rows all have bit 1 equal to
  // bit 3 of j16, which decides whether its row halves are swapped.
  const int kread = l32 * kKRow + hf * 16;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vlane = kKTile + (8 * hf + (j16 >> 2)) * kVRow + 32 * (g16 & 1) + 8 * (j16 & 3);
  const int vswap = (j16 & 8) ? 64 : 0;
  const int vread[2] = {vlane + vswap, vlane + 64 - vswap};

  // keys of the sub-tile at key0 that lie before the end of the range, as a
  // uniform count in [0, 32]: a key at offset j of the sub-tile is masked
  // iff j >= valid(key0)
  auto valid = [&](int64_t key0) __attribute__((always_inline)) {
    const int64_t n = tr.k_end - key0;
    return (int)__builtin_amdgcn_readfirstlane((uint32_t)(n < 0 ? 0 : n > 32 ? 32 : n));
  };
  const int64_t nkeys = tr.k_end - tr.k_begin;
  // tile counts (uniform; below 2^24 since keys number below 2^31)
  const int32_t nfull = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(nkeys / kBK));
  const int32_t ntiles =
      (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)((nkeys + kBK - 1) / kBK));
  const bf16x2 kOnes = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // Row sums on the matrix core: D += A B with v_mfma_f32_16x16x32_bf16,
  // B = one P operand register set as it stands (lane L gives column L%16,
  // k-group L/16), A = 0/1 selecting k-groups {0, 2} for rows 0-7 and
  // {1, 3} for rows 8-15.  Lane L of a P operand holds query L%32, so
  // k-groups 0 and 2 are query j = L%16 and groups 1 and 3 query 16 + j:
  // rows 0-7 of column j sum the 16 probabilities of query j, rows 8-15
  // those of query 16 + j.  Accumulator lane L (rows 4*(L/16)..+3 of column
  // L%16) thus holds the running sum of query L (L < 16), L - 16 (L < 48) or
  // L - 32.  This keeps the row sum off the VALU, whose dot2 form competes
  // with the MFMA issue far more than its instruction count suggests.
  bf16x8 rs_sel;
  {
    const uint32_t w = (((g16 & 1) == 0) == (j16 < 8)) ? 0x3f803f80u : 0u;
    const u32x4 wv = {w, w, w, w};
    rs_sel = __builtin_bit_cast(bf16x8, wv);
  }
  auto rowsum = [&](int qb, const u32x4& P) __attribute__((always_inline)) {
    lrs[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rs_sel, __builtin_bit_cast(bf16x8, P),
                                                     lrs[qb], 0, 0, 0);
  };

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
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const char* a = &lds[st][0] + vread[db] + sb * 32 * kVRow + 16 * c2 * kVRow;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 4 * kVRow));
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              va, __builtin_bit_cast(bf16x8, P[qb][c2]), o[qb][db], 0, 0, 0);
      }
  };
  // P = exp2(qscale*S - m) rounded to bf16 into the PV operand.  Tail: keys
  // at or past the end of the range get P = 0.  With_sum: also returns the
  // lane's fp32 sum of the rounded P (exact fallback loop only).
  auto exp_pack = [&](int qb, const f32x16& S, u32x4 (&P)[2], int64_t key0, auto tail_tag,
                      auto sum_tag) __attribute__((always_inline)) {
    constexpr bool tail = decltype(tail_tag)::value;
    constexpr bool with_sum = decltype(sum_tag)::value;
    const float nm = -m[qb];
    float acc = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float z0 = __builtin_fmaf(S[8 * c2 + 2 * e], qscale, nm);
        float z1 = __builtin_fmaf(S[8 * c2 + 2 * e + 1], qscale, nm);
        if constexpr (tail) {
          const int j = 16 * c2 + 8 * hf + 2 * e, lim = valid(key0);
          if (j >= lim) z0 = -INFINITY;
          if (j + 1 >= lim) z1 = -INFINITY;
        }
        const uint32_t pp = pack_bf16(__builtin_amdgcn_exp2f(z0), __builtin_amdgcn_exp2f(z1));
        P[c2][e] = pp;
        if constexpr (with_sum)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes, acc, false);
      }
    return acc;
  };
  // The sub-tile's max over its keys (tail: keys before the end of the
  // range only), across both lane halves, in raw dot-product units.
  auto subtile_max = [&](const f32x16& S, int64_t key0, auto tail_tag)
      __attribute__((always_inline)) {
    float rmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = S[r];
      if constexpr (decltype(tail_tag)::value) {
        if (16 * (r >> 3) + 8 * hf + (r & 7) >= valid(key0)) x = -INFINITY;
      }
      rmax = fmaxf(rmax, x);
    }
    return fmaxf(rmax, __shfl_xor(rmax, 32));
  };
  // Exact online-softmax update of one sub-tile (the textbook form): raise
  // m to the sub-tile max, rescale O and l, then P and its row sum.  A fully
  // masked sub-tile (tail) leaves the state unchanged.
  auto softmax_exact = [&](const f32x16 (&S)[2], u32x4 (&P)[2][2], int64_t key0, auto tail_tag)
      __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float rmax = subtile_max(S[qb], key0, tail_tag);
      const float mx = rmax == -INFINITY ? -INFINITY : __builtin_fmaf(rmax, qscale, -m[qb]);
      const float delta = mx == -INFINITY ? 0.f : (mset[qb] ? fmaxf(mx, 0.f) : mx);
      const float factor = mset[qb] ? exp2f(-delta) : 1.f;
      m[qb] += delta;
      mset[qb] = mset[qb] || mx != -INFINITY;
      lsum[qb] *= factor;
      o[qb][0] *= factor;
      o[qb][1] *= factor;
      lsum[qb] += exp_pack(qb, S[qb], P[qb], key0, tail_tag, std::true_type{});
    }
  };

  // ---- the pipeline's state: one score tile S[qb] and one probability
  // operand set P[qb] per query block, the K operands of one sub-tile (ka)
  // and the V operands of one (va)
  f32x16 S[2];
  u32x4 P[2][2];
  bf16x8 ka[4], va[2][2];
  auto load_k = [&](int st, int sb, int c) __attribute__((always_inline)) {
    ka[c] = __builtin_bit_cast(
        bf16x8, *(const lds_u32x4*)(&lds[st][0] + kread + sb * 32 * kKRow + c * 32));
  };
  // V^T operand (db, c2) of a sub-tile: two transposed reads
  auto load_v = [&](int st, int sb, int db, int c2) __attribute__((always_inline)) {
    const char* a = &lds[st][0] + vread[db] + sb * 32 * kVRow + 16 * c2 * kVRow;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a + 4 * kVRow));
    va[db][c2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Step j (the softmax of sub-tile j), sixteen units of one MFMA and one
  // pair of scores each, pinned in that order by sched barriers:
  //   units  0-3   QK(j, block 1)        | softmax(j, block 0), pairs 0-3
  //   units  4-7   PV(j-1, block 1)      | softmax(j, block 0), pairs 4-7
  //   units  8-11  QK(j+1, block 0)      | softmax(j, block 1), pairs 0-3
  //   units 12-15  PV(j, block 0)        | softmax(j, block 1), pairs 4-7
  // so every MFMA's operands were produced at least four units earlier and
  // each block needs one score tile and one probability set: block 0's S
  // is consumed (units 0-7) before QK(j+1) refills it (8-11), block 1's P
  // is consumed by PV(j-1) (4-7) before the softmax rewrites it (8-15).
  // The K operands of sub-tile j+1 (at stK/sbK) load in units 4-7, after
  // QK(j, block 1) last read ka; the V operands of sub-tile j (at stV/sbV)
  // in units 8-11, after PV(j-1) last read va.  The row sums of each P set
  // go to the matrix core beside its PV products.  First (sub-tile 0): no
  // PV(j-1), and block 1's reference max is taken at unit 8, once its
  // scores exist.  Tail: keys at or past the end of the range get P = 0.
  auto step = [&](int stK, int sbK, int stV, int sbV, int64_t key0, auto first_tag,
                  auto tail_tag, auto nb_tag) __attribute__((always_inline)) {
    constexpr bool first = decltype(first_tag)::value;
    constexpr bool tail = decltype(tail_tag)::value;
    constexpr bool two = decltype(nb_tag)::value == 2;  // else block 0 only
    const int lim = tail ? valid(key0) : 32;
    // softmax of pair w (operand half w/4, register pair w%4) of block qb:
    // z = scale*S - m (log2 units), P = exp2(z) as bf16
    auto pair = [&](int qb, int w) __attribute__((always_inline)) {
      const int c2 = w >> 2, e = w & 3;
      const float nm = -m[qb];
      float z0 = __builtin_fmaf(S[qb][8 * c2 + 2 * e], qscale, nm);
      float z1 = __builtin_fmaf(S[qb][8 * c2 + 2 * e + 1], qscale, nm);
      if constexpr (tail) {
        const int j = 16 * c2 + 8 * hf + 2 * e;
        if (j >= lim) z0 = -INFINITY;
        if (j + 1 >= lim) z1 = -INFINITY;
      }
      P[qb][c2][e] = pack_bf16_now(__builtin_amdgcn_exp2f(z0), __builtin_amdgcn_exp2f(z1));
    };
    // The two waves of a SIMD (w and w+4) take turns at the higher issue
    // priority, step by step.  Left to the arbiter, the older wave runs
    // ahead and waits about a quarter of each tile at the barrier.
    if ((sbV & 1) == (wave >> 2))
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u >= 4 && u < 8) load_k(stK, sbK, u - 4);
      // V operands in the order the PV units use them: (db, c2) = (0,0),
      // (1,0), (0,1), (1,1), so consecutive PV MFMAs alternate accumulators
      if (u >= 8 && u < 12) load_v(stV, sbV, (u - 8) & 1, (u - 8) >> 1);
      if (two && first && u == 8) {
        m[1] = subtile_max(S[1], key0, tail_tag) * qscale;
        mset[1] = true;
      }
      if (two || u < 8) pair(u >> 3, u & 7);
      if (u < 4) {
        if constexpr (two)
          S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[u], qreg[1][u],
                                                         u == 0 ? f32x16(0.f) : S[1], 0, 0, 0);
      } else if (u < 8) {
        if constexpr (two && !first) {
          const int db = (u - 4) & 1, c2 = (u - 4) >> 1;
          o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              va[db][c2], __builtin_bit_cast(bf16x8, P[1][c2]), o[1][db], 0, 0, 0);
          if (db == 0) rowsum(1, P[1][c2]);
        }
      } else if (u < 12) {
        const int c = u - 8;
        S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qreg[0][c],
                                                       c == 0 ? f32x16(0.f) : S[0], 0, 0, 0);
      } else {
        const int db = (u - 12) & 1, c2 = (u - 12) >> 1;
        o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            va[db][c2], __builtin_bit_cast(bf16x8, P[0][c2]), o[0][db], 0, 0, 0);
        if (db == 0) rowsum(0, P[0][c2]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop over 32-key sub-tiles j, four per LDS tile.  Three LDS
  // stages: tile t+2 loads into the stage of tile t-1 at the barrier before
  // step 4t+3 (the first step that reads tile t+1); tile t-1's last reader
  // (the V loads of step 4t-1) ran before it.  The reference max m is the
  // exact max of the first sub-tile; later sub-tiles use P = exp2(S - m) as
  // is, which stays finite unless a score exceeds m by 128 (log2 units) --
  // checked after the loop.
  // Tile order: the ragged tail first (if any), then the full tiles; the
  // softmax sums do not depend on the key order.
  const bool has_tail = ntiles > nfull;
  auto tile_key0 = [&](int32_t i) __attribute__((always_inline)) {
    return has_tail ? (i == 0 ? tr.k_begin + (int64_t)nfull * kBK
                              : tr.k_begin + (int64_t)(i - 1) * kBK)
                    : tr.k_begin + (int64_t)i * kBK;
  };
  auto issue_tile = [&](int32_t i, int st) __attribute__((always_inline)) {
    if (has_tail && i == 0)
      issue(tile_key0(0), st, std::true_type{});
    else
      issue(tile_key0(i), st, std::false_type{});
  };
  issue_tile(0, 0);
  if (ntiles > 1) issue_tile(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  auto advance = [&](int32_t t, int st_prev) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (t + 2 < ntiles) issue_tile(t + 2, st_prev);
  };
  constexpr std::true_type yes{};
  constexpr std::false_type no{};
  constexpr std::integral_constant<int, 2> kTwo{};
  constexpr std::integral_constant<int, 1> kOne{};
  // The key loop of a wave with NB query blocks (NB_TAG: kTwo or kOne), expanded in place for each
  // block count so that every expansion compiles as the kernel's own
  // straight-line code (wrapped in a lambda, the compiler schedules the
  // global and SGA loops differently, and measurably slower).
#define VGA_KEY_LOOP(NB_TAG)                                                                       \
  do {                                                                                             \
    /* ---- tile 0 (the ragged tail when there is one): steps 0..3.  Before */                     \
    /* step 0: K operands and block 0's scores of sub-tile 0, and block 0's */                     \
    /* reference max (sub-tile 0 holds at least one key). */                                       \
    const int64_t key00 = tile_key0(0);                                                            \
    const int st1 = ntiles > 1 ? 1 : 0;  /* K source of step 3 (a dummy re-read if no tile 1) */   \
  _Pragma("unroll")                                                                                \
    for (int c = 0; c < 4; ++c) load_k(0, 0, c);                                                   \
  _Pragma("unroll")                                                                                \
    for (int c = 0; c < 4; ++c)                                                                    \
      S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qreg[0][c], c == 0 ? f32x16(0.f) : S[0], \
                                                     0, 0, 0);                                     \
    if (has_tail) {                                                                                \
      m[0] = subtile_max(S[0], key00, yes) * qscale;                                               \
      mset[0] = true;                                                                              \
      step(0, 1, 0, 0, key00, yes, yes, NB_TAG);                                                   \
      step(0, 2, 0, 1, key00 + 32, no, yes, NB_TAG);                                               \
      step(0, 3, 0, 2, key00 + 64, no, yes, NB_TAG);                                               \
      if (ntiles > 1) advance(0, kStages - 1);                                                     \
      step(st1, 0, 0, 3, key00 + 96, no, yes, NB_TAG);                                             \
    } else {                                                                                       \
      m[0] = subtile_max(S[0], key00, no) * qscale;                                                \
      mset[0] = true;                                                                              \
      step(0, 1, 0, 0, 0, yes, no, NB_TAG);                                                        \
      step(0, 2, 0, 1, 0, no, no, NB_TAG);                                                         \
      step(0, 3, 0, 2, 0, no, no, NB_TAG);                                                         \
      if (ntiles > 1) advance(0, kStages - 1);                                                     \
      step(st1, 0, 0, 3, 0, no, no, NB_TAG);                                                       \
    }                                                                                              \
    /* ---- full tiles 1 .. ntiles-1: steps 4t .. 4t+3 */                                          \
    int st = 0;                                                                                    \
    for (int32_t t = 1; t < ntiles; ++t) {                                                         \
      const int st_prev = st;                                                                      \
      st = st == kStages - 1 ? 0 : st + 1;                                                         \
      const int st_next = st == kStages - 1 ? 0 : st + 1;                                          \
      const bool has_next = t + 1 < ntiles;                                                        \
      step(st, 1, st, 0, 0, no, no, NB_TAG);                                                       \
      step(st, 2, st, 1, 0, no, no, NB_TAG);                                                       \
      step(st, 3, st, 2, 0, no, no, NB_TAG);                                                       \
      if (has_next) advance(t, st_prev);                                                           \
      /* K of sub-tile 4t+4 (tile t+1); a dummy re-read of this tile when t is last */             \
      step(has_next ? st_next : st, 0, st, 3, 0, no, no, NB_TAG);                                  \
    }                                                                                              \
    /* drain: PV and row sums of the last sub-tile's block 1 */                                    \
    if constexpr (decltype(NB_TAG)::value == 2) {                                                  \
  _Pragma("unroll")                                                                                \
      for (int c2 = 0; c2 < 2; ++c2) {                                                             \
  _Pragma("unroll")                                                                                \
        for (int db = 0; db < 2; ++db)                                                             \
          o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                                      \
              va[db][c2], __builtin_bit_cast(bf16x8, P[1][c2]), o[1][db], 0, 0, 0);                \
        rowsum(1, P[1][c2]);                                                                       \
      }                                                                                            \
    }                                                                                              \
  } while (0)
  if constexpr (KR == KeyRange::kFrame) {
    // A wave without query blocks takes part in the tile DMA and the
    // barriers exactly as the key loop does: advance() after tile 0's third
    // step and after each later tile's third step but the last's.
    if (nblk == 2) {
      VGA_KEY_LOOP(kTwo);
    } else if (nblk == 1) {
      VGA_KEY_LOOP(kOne);
    } else {
      if (ntiles > 1) advance(0, kStages - 1);
      int st = 0;
      for (int32_t t = 1; t < ntiles; ++t) {
        const int st_prev = st;
        st = st == kStages - 1 ? 0 : st + 1;
        if (t + 1 < ntiles) advance(t, st_prev);
      }
    }
  } else {
    VGA_KEY_LOOP(kTwo);
  }
#undef VGA_KEY_LOOP

  // Row sums into the lane of their query (lane L holds query L % 32):
  // accumulator lane L % 32 (< 16) or L % 32 + 16 (>= 16) has it.
  const int rs_src = l32 < 16 ? l32 : l32 + 16;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float full = __shfl(lrs[qb][0], rs_src);
    lsum[qb] = hf == 0 ? full : 0.f;
  }

  // ---- the check: every row sum and output accumulator finite (x * 0 is
  // NaN exactly for x non-finite); otherwise a score exceeded m by 128 or
  // more somewhere in the workgroup, and every wave redoes its rows with
  // the exact online softmax (P <= 1 throughout).
  {
    float nf = lsum[0] * 0.f + lsum[1] * 0.f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) nf = __builtin_fmaf(o[qb][db][r], 0.f, nf);
    if (__any(nf != nf) && lane == 0) fallback = 1;
  }
  __syncthreads();
  if (fallback) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      o[qb][0] = 0.f;
      o[qb][1] = 0.f;
      lsum[qb] = 0.f;
      m[qb] = 0.f;
      mset[qb] = false;
    }
    // one tile at a time through stage 0, each sub-tile exact
    for (int32_t t = 0; t < ntiles; ++t) {
      __syncthreads();  // every wave is done with stage 0
      issue_tile(t, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int64_t key0 = tile_key0(t);
      for (int sb = 0; sb < 4; ++sb) {
        f32x16 Sx[2];
        u32x4 Px[2][2];
        qk(0, sb, Sx);
        if (has_tail && t == 0)
          softmax_exact(Sx, Px, key0 + 32 * sb, std::true_type{});
        else
          softmax_exact(Sx, Px, 0, std::false_type{});
        pv(0, sb, Px);
      }
    }
  }

  // This wave's first query row, recomputed here: the value from the Q load
  // would otherwise be kept, in registers or scratch, across the loop.
  int64_t row0 = wq_begin + l32;
  asm volatile("" : "+v"(row0));

  if constexpr (KR == KeyRange::kSga) {
    // The diagonal and mean columns join each query's shared softmax here,
    // merged into (m, l, O) after the compacted keys (the softmax sums do not
    // depend on the column order).  Every load of the merge -- the query's
    // own K and V rows and the mean columns -- is issued first, so the merge
    // waits for memory once (the rows are in range: row < T; the mean
    // columns always exist, zero when nothing is dropped).
    const uint16_t* kf = (const uint16_t*)p.k_full;
    const uint16_t* vf = (const uint16_t*)p.v_full;
    const float* kms = p.kmean + head * 64 + 8 * hf;
    const float* vms = p.vmean + head * 64;
    u32x4 wk[2][4];
    u32x2 wv[2][2][4];
    f32x4 km[4][2], vm[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t row = min(row0 + qb * 32, tr.q_end - 1);
      const uint16_t* ks = kf + ((size_t)row * H + head) * 64 + 8 * hf;
      const uint16_t* vs = vf + ((size_t)row * H + head) * 64;
#pragma unroll
      for (int c = 0; c < 4; ++c) wk[qb][c] = *(const u32x4*)(ks + 16 * c);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) wv[qb][db][g] = *(const u32x2*)(vs + 32 * db + 8 * g + 4 * hf);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      km[c][0] = *(const f32x4*)(kms + 16 * c);
      km[c][1] = *(const f32x4*)(kms + 16 * c + 4);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) vm[db][g] = *(const f32x4*)(vms + 32 * db + 8 * g + 4 * hf);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t row = min(row0 + qb * 32, tr.q_end - 1);
      const bool diag = p.use_diag && !sga_kept(p.grid, p.row0 + row);
      float dk = 0.f, dm = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 wq = __builtin_bit_cast(u32x4, qreg[qb][c]);  // dims 16c + 8hf + [0, 8)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float qa = bf16_lo(wq[e]), qb2 = bf16_hi(wq[e]);
          dk += qa * bf16_lo(wk[qb][c][e]) + qb2 * bf16_hi(wk[qb][c][e]);
          const float ma = e < 2 ? km[c][0][2 * e] : km[c][1][2 * e - 4];
          const float mb = e < 2 ? km[c][0][2 * e + 1] : km[c][1][2 * e - 3];
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
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2 w = wv[qb][db][g];
            const f32x4 mv = vm[db][g];
            o[qb][db][4 * g + 0] = o[qb][db][4 * g + 0] * f + wd * bf16_lo(w[0]) + wm * mv[0];
            o[qb][db][4 * g + 1] = o[qb][db][4 * g + 1] * f + wd * bf16_hi(w[0]) + wm * mv[1];
            o[qb][db][4 * g + 2] = o[qb][db][4 * g + 2] * f + wd * bf16_lo(w[1]) + wm * mv[2];
            o[qb][db][4 * g + 3] = o[qb][db][4 * g + 3] * f + wd * bf16_hi(w[1]) + wm * mv[3];
          }
      }
    }
  }

  // ---- normalise and store O (bf16, RNE)
  uint16_t* __restrict__ og = (uint16_t*)p.o;
  if constexpr (KR == KeyRange::kFrame) {
    // Frame attention (short workgroups, where the epilogue weighs): the
    // wave stages its 64 rows in LDS and writes whole 128-byte rows with
    // 16-byte stores, 8 lanes per row.  Each wave has its own 8 KB in the
    // ring's stages 1-2, which no wave reads after the key loop (the exact
    // fallback uses stage 0 only); 16-byte slot g of staged row r sits at
    // slot g ^ ((r >> 1) & 7).  LDS operations of one wave complete in
    // order, so the reads see the writes without a barrier.
    char* stg = &lds[1][0] + wave * 8192;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l = lsum[qb] + __shfl_xor(lsum[qb], 32);
      const float inv = 1.f / l;
      const int r = qb * 32 + l32;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack_bf16(o[qb][db][4 * g + 0] * inv, o[qb][db][4 * g + 1] * inv);
          w[1] = pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          const int slot = (4 * db + g) ^ ((r >> 1) & 7);
          *(__attribute__((address_space(3))) u32x2*)(stg + r * 128 + slot * 16 + 8 * hf) = w;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 8 * k + (lane >> 3), g = lane & 7;
      const u32x4 w = *(const lds_u32x4*)(stg + r * 128 + ((g ^ ((r >> 1) & 7)) * 16));
      const int64_t row = wq_begin + r;
      if (row < wq_end) *(u32x4*)(og + ((size_t)row * H + head) * 64 + 8 * g) = w;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.f / l;
    const int64_t row = row0 + qb * 32;
    if (row < wq_end) {
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
