// Big-tile grouped GEMMs: gate/up + SwiGLU and down over the big tiles of
// the schedule (and, in the same launch, its small tiles), for bf16, 4-bit
// block and MXFP4 weights.
//
// Where a group has a hundred rows or more the layer is bound by the matrix
// cores, not by weight bytes.  A block owns 256 weight rows x up to 128 token
// rows (items of 128, 64, 32 or 16 token rows, by the tile) and walks K in
// super-stages of 128:
//  * the token rows (operand B, shared by the block's waves) are copied from
//    global memory straight into LDS with global_load_lds_dwordx4, into a ring
//    of stages, in a row-major layout whose 16-byte chunks are
//    XOR-swizzled by row so that fragment reads avoid bank conflicts;
//  * each wave owns 64 weight rows (bf16, MX: four waves) or 32 (4-bit: eight
//    waves, two per SIMD) as operand A and loads them from global memory
//    directly into registers in the MFMA fragment layout, into a ring of
//    register tiles; 4-bit codes are dequantised in registers right before
//    the MFMAs that use them, so every weight byte is read and decoded once
//    per block and never passes through LDS;
//  * the loads of super-stage S + ring - 1 are issued while S is computed;
//  * v_mfma_f32_16x16x32_bf16 accumulates (weight rows) x (token rows) per
//    wave.
// 4-bit: the decode is about two VALU instructions per weight, and one wave
// per SIMD issues VALU instructions well below the SIMD's rate, hence two
// waves per SIMD; the weight fragments of step k + 1 are decoded alongside
// the MFMAs of step k.  The K order inside a super-stage is permuted so
// that each lane's 16-byte load is one whole 32-code block (one scale, one
// min); the token fragments are read from LDS in the same order, which
// leaves the dot products unchanged.
// MXFP4 weights (E2M1, one E8M0 scale per 32) against MXFP8 token rows take
// the same loop with one scaled FP4 x FP8 MFMA (16x16x128) per fragment pair
// and super-stage: a lane's 16-byte weight load is its whole 32-element block,
// nothing is decoded, and the token rows are 128 bytes per super-stage in LDS.
// The item's scales (MX: E8M0 bytes of its weight and token rows; 4-bit: the
// fp16 scales and mins of its weight rows) are copied into LDS once, in
// 16-byte chunks, before the loop: read per super-stage from global memory,
// each row's scale lines were touched over the whole item, fell out of L2 and
// held the load issue back.
//
// The shared expert and every routed expert go through the same launch; the
// grouping itself is the point of the pages' "concatenated-expert" fix
// ("~2.7s fixed per-request TTFT ... concatenated-expert GEMM", section "The
// fix") and of "the lever is M>1" ("MoE Decode Partition and Submit Floor",
// M2 update).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBN = 256;                 // weight rows per block (4 waves x 64; 4-bit: 8 x 32)
constexpr int kSK = 128;                 // K per super-stage
// Super-stages resident (LDS stages and A register tiles), one block per CU:
// bf16 and 4-bit a ring of three (4-bit: with the item's scales, the three
// 32 KB token stages of a 128-row item fill the LDS), MX four.
#ifndef MOE_BIG_RING_Q4
#define MOE_BIG_RING_Q4 3
#endif
#ifndef MOE_BIG_RING_MX
#define MOE_BIG_RING_MX 4
#endif
// 4-bit items of at most 32 token rows (short tiles) do a sixteenth or an
// eighth of a 128-row item's MFMAs per weight byte: the registers of their
// accumulators go to a deeper ring.
#ifndef MOE_BIG_RING_SHORT
#define MOE_BIG_RING_SHORT 4
#endif
template <int WF, int BM>
constexpr int ring() {
  return WF == kQ4 ? (BM <= 32 ? MOE_BIG_RING_SHORT : MOE_BIG_RING_Q4) : WF == kMX4 ? MOE_BIG_RING_MX : 3;
}
static_assert(MOE_BIG_RING_Q4 == 3, "ring depth: three 32 KB token stages and the item's scales fill the LDS");
static_assert(MOE_BIG_RING_MX >= 3 && MOE_BIG_RING_MX <= 4, "ring depth");
static_assert(MOE_BIG_RING_SHORT >= 2 && MOE_BIG_RING_SHORT <= 4, "ring depth");
// Waves per block: 4-bit eight (two per SIMD; the 4-bit decode is VALU-bound,
// and one wave per SIMD issues VALU instructions at well under the SIMD's
// rate), the other formats four.  Each wave owns 256 / (16 x waves)
// fragments of 16 weight rows.
template <int WF> constexpr int big_waves() { return WF == kQ4 ? 8 : 4; }
template <int WF> constexpr int big_threads() { return kWave * big_waves<WF>(); }
template <int WF> constexpr int frags() { return kBN / 16 / big_waves<WF>(); }
// Token rows per block: kBigTileRows for the big-tile list, kTileRows for the
// small-tile list.  Bytes of one token row per super-stage (bf16: 256, E4M3:
// 128), 16-byte chunks per row, rows per 1 KB DMA instruction; B stage bytes
// (MX: the rows, then 4 scale bytes per row), and DMA instructions per wave
// per stage for the rows.
template <int WF> constexpr int b_row_bytes() { return WF == kMX4 ? kSK : kSK * 2; }
template <int WF> constexpr int b_row_chunks() { return b_row_bytes<WF>() / 16; }
template <int WF> constexpr int b_rows_per_dma() { return 1024 / b_row_bytes<WF>(); }
template <int WF, int BM> constexpr int b_data_bytes() { return BM * b_row_bytes<WF>(); }
template <int WF, int BM> constexpr int b_stage_bytes() { return b_data_bytes<WF, BM>(); }
// MX item scales in LDS (K <= kMxMaxK, K % 512 == 0): the 256 weight rows'
// bytes, then the token rows', each row K / 32 bytes, copied in 16-byte
// chunks (256 K / 512 and BM K / 512 of them) spread over the block's lanes.
constexpr int kMxMaxK = 2048;
constexpr int kMxScaleBytes = kBN * (kMxMaxK / 32) + kBigTileRows * (kMxMaxK / 32);
// 4-bit item scales and mins in LDS (K <= kQ4MaxK, K % 256 == 0): the 256
// weight rows' fp16 scales, then their fp16 mins, K / 32 of each per row; K
// 16-byte DMA chunks per array, spread over the block's lanes.
constexpr int kQ4MaxK = 2048;
constexpr int kQ4ArrayBytes = kBN * (kQ4MaxK / 32) * 2;
constexpr int kQ4ScaleBytes = 2 * kQ4ArrayBytes;
// 1 KB DMA instructions per stage (all waves), per wave (at least one: with
// fewer instructions than waves, wave w repeats instruction w % total, the
// same bytes to the same place).
template <int WF, int BM> constexpr int b_dma_total() { return b_data_bytes<WF, BM>() / 1024; }
template <int WF, int BM> constexpr int b_dma_per_wave() {
  return b_dma_total<WF, BM>() >= big_waves<WF>() ? b_dma_total<WF, BM>() / big_waves<WF>() : 1;
}
// Chunk slot of a row's 16-byte chunk c in LDS: XOR-swizzled by row so that
// the 16 rows of a fragment read spread over the banks (256-byte rows: all
// 16 slots; 128-byte rows: two rows per 256 bytes, 8 slots each).
template <int WF> __device__ __forceinline__ int b_swz(int row) {
  return WF == kMX4 ? (row >> 1) & 7 : row % 16;
}
static_assert(kBigTileRows == 128 && kTileRows == 64, "tile heights the B loader and fragments are laid out for");
// Item heights: 128 (big tiles), 64, 32 and 16 (small tiles, by their rows;
// MX: 32 at least, one 1 KB DMA of token rows per wave).
template <int WF, int BM>
constexpr bool item_height_ok() {
  return (BM == 128 || BM == 64 || BM == 32 || (BM == 16 && WF != kMX4)) && b_dma_per_wave<WF, BM>() >= 1;
}

// Down items of two 256-column blocks (4-bit and MX; the bf16 kernel has no
// registers to spare for a store inside its loop).
template <int WF, bool kGU>
constexpr bool kTwoBlocks() { return !kGU && WF != kBF16; }

struct Bp {
  const void* act;          // x [T][K] (gate/up, gathered by row_token) or h [R][K] (down), bf16 (MX: E4M3)
  const uint8_t* act_scale; // MX: E8M0 bytes [rows][K / 32] of act
  const int32_t* row_token;
  const int32_t* sched;
  const void* w;
  const void* w_scale;
  const void* w_min;
  void* out;                // h [R][N] or y [R][N], bf16 (MX: fp32)
  int K, N, T, R;
  int ncb;                  // 256-column weight blocks per item (down: 2 when they fit, else 1)
};

typedef __attribute__((address_space(3))) void lds_void;

// A-operand loads are opaque to the compiler so that they stay where they are
// issued (two super-stages ahead of their use) instead of being sunk next to
// it; completion is awaited with explicit s_waitcnt vmcnt.
__device__ __forceinline__ u32x4 gload16(const void* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}
// Same loads at a 32-bit byte offset from a uniform base (scalar base + vector offset).
__device__ __forceinline__ u32x4 gload16(const void* base, uint32_t off) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(r) : "v"(off), "s"(base) : "memory");
  return r;
}


// Vector-memory loads each thread issues per super-stage (LDS DMA + A).
template <int WF, int BM>
constexpr int loads_per_stage() {
  return b_dma_per_wave<WF, BM>() + (WF == kQ4 || WF == kMX4 ? frags<WF>() : 16);
}

// One wave's A operand for one super-stage: 4 fragments of 16 weight rows.
//   4-bit: lane (r, q) holds the 16 bytes of block q of the super-stage
//          (codes k = 32q .. 32q+31); the scales and mins are in LDS;
//   bf16:  lane (r, q) holds, for step kk, elements k = 32kk + 8q .. +7.
//   MX:    lane (r, q) holds the 16 bytes of block q (elements k = 32q .. 32q+31);
//          the scale bytes are in LDS.
template <int WF>
struct ATile {
  u32x4 v[frags<WF>()][WF == kQ4 || WF == kMX4 ? 1 : 4];
};

// Part g (0..7) of one super-stage's A loads (the loads are spread over the
// eight parts the compute loop issues).  4-bit and MX: the codes of fragment
// g / (8 / F) when g is a multiple of 8 / F (F fragments per wave); bf16:
// fragment g / 2, steps 2 (g % 2) and 2 (g % 2) + 1.
template <int WF, class Row>
__device__ __forceinline__ void load_a_part(const Bp& p, ATile<WF>& a, const Row (&arow)[frags<WF>()], Row roff,
                                            int S, int q, int g) {
  if constexpr (WF == kMX4 || WF == kQ4) {
    // 32-bit offsets (the launcher checks that the weights fit)
    static_assert(sizeof(Row) == 4, "4-bit and MX weights use 32-bit offsets");
    constexpr int PPF = 8 / frags<WF>();  // parts per fragment
    const int b = g / PPF;
    if (g % PPF == 0) a.v[b][0] = gload16(p.w, (arow[b] + roff) * (uint32_t)(p.K / 2) + S * (kSK / 2) + 16 * q);
  } else {
    const int b = g / 2;
#pragma unroll
    for (int kk = 2 * (g % 2); kk < 2 * (g % 2) + 2; ++kk)
      a.v[b][kk] = gload16((const uint16_t*)p.w + (arow[b] + roff) * p.K + S * kSK + 32 * kk + 8 * q);
  }
}

// Make every later use of a tile's registers depend on the preceding wait.
template <int WF>
__device__ __forceinline__ void tie(ATile<WF>& a) {
#pragma unroll
  for (int b = 0; b < frags<WF>(); ++b) {
#pragma unroll
    for (int i = 0; i < (WF == kQ4 || WF == kMX4 ? 1 : 4); ++i) asm volatile("" : "+v"(a.v[b][i]));
  }
}

// DMA instruction i of wave `wave` for the token rows of one stage: which
// 1 KB of the stage it writes.
template <int WF, int BM>
__device__ __forceinline__ int b_dma_index(int wave, int i) {
  return (b_dma_per_wave<WF, BM>() * wave + i) % b_dma_total<WF, BM>();
}

// B operand of one super-stage -> LDS, DMA instruction i of the wave: it
// writes the 1 KB at d = b_dma_index KB of the stage: rows
// RPD d + lane / (64 / RPD), chunk slot lane % (64 / RPD), which holds the
// row's chunk slot ^ b_swz(row).
template <int WF, int BM, class Src>
__device__ __forceinline__ void load_b_part(uint8_t* stage, const void* act,
                                            const Src (&src)[b_dma_per_wave<WF, BM>()], int S, int wave, int i) {
  const uint8_t* g;
  if constexpr (sizeof(Src) == 4)
    g = (const uint8_t*)act + (src[i] + (uint32_t)S * b_row_bytes<WF>());  // 32-bit byte offset
  else
    g = (const uint8_t*)src[i] + (size_t)S * b_row_bytes<WF>();
  __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(stage + b_dma_index<WF, BM>(wave, i) * 1024), 16, 0, 0);
}

// MX: one 16-byte chunk of item scales -> LDS (lane-consecutive destinations).
__device__ __forceinline__ void load_scale_chunk(uint8_t* dst, const uint8_t* src) {
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst, 16, 0, 0);
}

// Barrier between super-stages.  __syncthreads() would also fence the
// pending LDS DMA (the loads two super-stages ahead) and so drain the ring;
// here each wave waits only for its own LDS reads (the slot they read is
// refilled after the barrier), and the DMA data of the next super-stage is
// covered by the explicit vmcnt wait before the barrier.  The memory clobbers
// keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk (16 bytes = 8 K) of a token row that lane group q reads for step kk.
// MX: kk = 0 / 1 are the two halves of the FP8 operand (K 16q .. 16q+15 and
// 64+16q .. 64+16q+15 of the super-stage: chunks q and 4 + q).
template <int WF>
__device__ __forceinline__ int b_chunk(int q, int kk) {
  return WF == kQ4 ? 4 * q + kk : WF == kMX4 ? 4 * kk + q : 4 * kk + q;
}

// A fragment of step kk for weight block b.  4-bit: the dword holds codes
// 8kk .. 8kk+7 of the lane's block, two per byte (even code in the low nibble).
template <int WF>
__device__ __forceinline__ u32x4 a_frag(const ATile<WF>& a, const Q4Block (&qs)[frags<WF>()], int b, int kk) {
  if constexpr (WF == kQ4) {
    return q4_decode8(a.v[b][0][kk], qs[b]);  // codes 8kk .. 8kk+7 of the lane's block
  } else {
    return a.v[b][kk];
  }
}

// One super-stage of MFMAs, software-pipelined in groups of 4 token blocks
// (NG = BM / 64 groups per step kk): the B fragments of the next group are
// read from LDS before the 16 MFMAs of the current group are issued, and the
// A fragments of the next step are decoded alongside them, so neither the LDS
// latency nor the decode stalls the matrix pipe.  The 8 parts of the global
// loads of a later super-stage (issue_part(p)) are spread evenly over the
// groups, so that the memory pipeline fills while the MFMAs run instead of in
// one burst.  sched_barrier pins that order.
// Item scales of one super-stage in LDS.  MX: a[b] = this lane's byte for
// weight fragment b (its row, block 4 S + q), b = token block 0's (row lr),
// token block c's at b + c * bstep.  4-bit: s[b], m[b] = the fp16 bits of
// the scale and min of weight fragment b's block 4 S + q (read from LDS one
// super-stage ahead).
struct ItemSc {
  const uint8_t* a[4];
  const uint8_t* b;
  int bstep;
  uint32_t s[4], m[4];
};

template <int WF, int BM, class IssuePart>
__device__ __forceinline__ void compute(const ATile<WF>& a, const uint8_t* st, f32x4 (&acc)[frags<WF>()][BM / 16], int lr,
                                        int q, IssuePart&& issue_part, const ItemSc& sc = ItemSc{}) {
  constexpr int NG = BM / 64, G = 4 * NG, PPG = G > 0 ? 8 / G : 0;  // groups per step, groups, load parts per group
  constexpr int F = frags<WF>();
  if constexpr (WF == kMX4) {
    // One scaled MFMA per (weight block, token block), in groups of GW token
    // blocks; the next group's two FP8 halves and scale bytes are read from
    // LDS before the current group's 4 GW MFMAs are issued (one wave per
    // SIMD: nothing else would cover the LDS latency).
    constexpr int GW = BM / 16 < 4 ? BM / 16 : 4, MG = BM / 16 / GW, MPPG = 8 / MG;
    // Row 16c + lr of the stage: the swizzle depends on lr alone, so the LDS
    // addresses of a token block differ from block 0's by a constant.
    const uint8_t* h0 = st + lr * b_row_bytes<WF>() + 16 * (b_chunk<WF>(q, 0) ^ b_swz<WF>(lr));
    const uint8_t* h1 = st + lr * b_row_bytes<WF>() + 16 * (b_chunk<WF>(q, 1) ^ b_swz<WF>(lr));
    uint32_t as[F];
#pragma unroll
    for (int b = 0; b < F; ++b) as[b] = *sc.a[b];
    struct BG {
      u32x4 b0[GW], b1[GW];
      uint32_t bs[GW];
    };
    auto read_group = [&](BG& o, int g) {
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int c = GW * g + i;
        o.b0[i] = *reinterpret_cast<const u32x4*>(h0 + c * 16 * b_row_bytes<WF>());
        o.b1[i] = *reinterpret_cast<const u32x4*>(h1 + c * 16 * b_row_bytes<WF>());
        o.bs[i] = sc.b[c * sc.bstep];
      }
    };
    BG cur, nxt;
    read_group(cur, 0);
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < MG) read_group(nxt, g + 1);
#pragma unroll
      for (int pp = 0; pp < MPPG; ++pp) issue_part(g * MPPG + pp);
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int b = 0; b < F; ++b)
          acc[b][GW * g + i] =
              mfma_mx4_mx8_16x16x128(a.v[b][0], as[b], cur.b0[i], cur.b1[i], cur.bs[i], acc[b][GW * g + i]);
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < MG) cur = nxt;
    }
    return;
  }
  Q4Block qs[F];
  if constexpr (WF == kQ4) {
#pragma unroll
    for (int b = 0; b < F; ++b) qs[b] = q4_block(sc.s[b], sc.m[b]);
    // 4-bit, every item height: the F NC MFMAs of step kk go out together
    // with the decode of the wave's weight fragments of step kk + 1 and the
    // LDS reads of its token fragments, so the decode (about two VALU
    // instructions per weight) and the LDS latency overlap the matrix pipe;
    // the other wave on the SIMD fills the gaps (the compiler's order within
    // a step measured as good as one pinned with sched_group_barrier).
    constexpr int NC = BM / 16;
    auto bfr = [&](int kk, int c) {
      return *reinterpret_cast<const u32x4*>(st + (16 * c + lr) * (kSK * 2) + 16 * (b_chunk<WF>(q, kk) ^ lr));
    };
    u32x4 af[F], bf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) bf[c] = bfr(0, c);
#pragma unroll
    for (int b = 0; b < F; ++b) af[b] = a_frag<WF>(a, qs, b, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      issue_part(2 * kk);
      issue_part(2 * kk + 1);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 an[F], bn[NC];
      if (kk < 3) {
#pragma unroll
        for (int c = 0; c < NC; ++c) bn[c] = bfr(kk + 1, c);
#pragma unroll
        for (int b = 0; b < F; ++b) an[b] = a_frag<WF>(a, qs, b, kk + 1);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int b = 0; b < F; ++b) acc[b][c] = mfma_bf16_16x16x32(af[b], bf[c], acc[b][c]);
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) {
#pragma unroll
        for (int c = 0; c < NC; ++c) bf[c] = bn[c];
#pragma unroll
        for (int b = 0; b < F; ++b) af[b] = an[b];
      }
    }
    return;
  } else {
  if constexpr (BM < 64) {
    // Short bf16 items (one or two token blocks): per step kk, two parts of
    // the later loads, the NC token fragments, the four weight fragments and
    // 4 NC MFMAs.
    constexpr int NC = BM / 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      issue_part(2 * kk);
      issue_part(2 * kk + 1);
      u32x4 af[4], bf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        bf[c] = *reinterpret_cast<const u32x4*>(st + (16 * c + lr) * (kSK * 2) + 16 * (b_chunk<WF>(q, kk) ^ lr));
#pragma unroll
      for (int b = 0; b < 4; ++b) af[b] = a_frag<WF>(a, qs, b, kk);
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b][c] = mfma_bf16_16x16x32(af[b], bf[c], acc[b][c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }

  // token row 16c + lr, chunk slot b_chunk ^ lr (the row's low 4 bits are lr)
  auto bfrag = [&](int kk, int c) {
    return *reinterpret_cast<const u32x4*>(st + (16 * c + lr) * (kSK * 2) + 16 * (b_chunk<WF>(q, kk) ^ lr));
  };
  u32x4 af[4], bf[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) af[b] = a_frag<WF>(a, qs, b, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) bf[i] = bfrag(0, i);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int kk = g / NG, c0 = 4 * (g % NG);
    const bool next_a = g % NG == NG - 1 && kk < 3;
    u32x4 nb[4], na[4];
    if (g < G - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) nb[i] = bfrag((g + 1) / NG, 4 * ((g + 1) % NG) + i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) issue_part(g * PPG + pp);
    if (next_a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) na[b] = a_frag<WF>(a, qs, b, kk + 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b][c0 + i] = mfma_bf16_16x16x32(af[b], bf[i], acc[b][c0 + i]);
    __builtin_amdgcn_sched_barrier(0);
    if (g < G - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bf[i] = nb[i];
    }
    if (next_a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) af[b] = na[b];
    }
  }
  }  // bf16
}

__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }

// One item: weight columns [n0, n0 + 256 ncb) (gate/up: 128 gate/up pairs,
// ncb = 1) of group `group` against token rows [row0, row0 + rows)
// (rows <= BM).  With ncb = 2 (down) the item walks K once per 256-column
// block, the ring running on from the first block into the second, so the
// second block's first loads are in flight while the first block's results
// are stored.
template <int WF, bool kGU, int BM>
__device__ __forceinline__ void gemm_item(const Bp& p, uint8_t* lds, int group, int row0, int rows, int n0) {
  constexpr int kBStage = b_stage_bytes<WF, BM>(), NC = BM / 16, NB = b_dma_per_wave<WF, BM>();
  constexpr int kRPD = b_rows_per_dma<WF>(), kLPR = kWave / kRPD;  // rows per DMA, lanes per row
  constexpr int kEB = WF == kMX4 ? 1 : 2;                            // bytes per token element
  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);  // uniform: keep it in a scalar register
  const int lr = lane % 16, q = lane / 16;

  static_assert(item_height_ok<WF, BM>(), "item height");
  constexpr int kRing = ring<WF, BM>(), kAhead = kRing - 1;
  static_assert(kRing * kBStage <= ring<WF, kBigTileRows>() * b_stage_bytes<WF, kBigTileRows>(), "ring fits the LDS");
  constexpr bool k32 = WF == kQ4 || WF == kMX4;  // 32-bit offsets
  using Row = typename std::conditional<k32, uint32_t, size_t>::type;
  using Src = typename std::conditional<k32, uint32_t, const uint8_t*>::type;
  // This wave's F weight fragments, as rows of the item's 256 (lw): gate/up:
  // the first F / 2 are gate rows (item rows < 128: gate columns n0 + lw),
  // the rest the up rows of the same columns (lw - 128); down: columns n0 + lw.
  constexpr int F = frags<WF>();
  const int ncb = kTwoBlocks<WF, kGU>() ? p.ncb : 1;
  auto local_row = [&](int b) {
    return kGU ? (b < F / 2 ? 0 : 128) + 8 * F * wave + 16 * (b % (F / 2)) + lr : 16 * F * wave + 16 * b + lr;
  };
  Row arow[F];
#pragma unroll
  for (int b = 0; b < F; ++b) {
    const int lw = local_row(b);
    if constexpr (kGU)
      arow[b] = (Row)group * 2 * p.N + (lw < 128 ? n0 + lw : p.N + n0 + lw - 128);
    else
      arow[b] = (Row)group * p.N + n0 + lw;
  }
  // B sources of this lane's DMA chunks (rows past the tile repeat row 0).
  Src bsrc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int rr = kRPD * b_dma_index<WF, BM>(wave, i) + lane / kLPR;
    const int r = rr < rows ? row0 + rr : row0;
    const int chunk = (lane % kLPR) ^ b_swz<WF>(rr);
    if constexpr (k32) {
      const uint32_t src_row = kGU ? (uint32_t)min(max(p.row_token[r], 0), p.T - 1) : (uint32_t)r;
      bsrc[i] = src_row * (uint32_t)p.K * kEB + 16 * chunk;
    } else {
      const size_t src_row = kGU ? (size_t)min(max(p.row_token[r], 0), p.T - 1) : (size_t)r;
      bsrc[i] = (const uint8_t*)p.act + src_row * (size_t)p.K * kEB + 16 * chunk;
    }
  }
  // MX: the item's scale bytes -> LDS after the ring (weight rows, then token
  // rows; K / 32 bytes per row, 16-byte chunks, lane-consecutive), issued
  // before the first super-stage's loads, so the first wait covers them.
  uint8_t* const asc_lds = lds + ring<WF, kBigTileRows>() * b_stage_bytes<WF, kBigTileRows>();
  uint8_t* const bsc_lds = asc_lds + kBN * (kMxMaxK / 32);
  const int kpr = p.K / 32;
  if constexpr (WF == kMX4) {
    // weight rows: 256 ncb cpr chunks (a multiple of 64), instruction i of
    // wave w copies chunks c0 .. c0 + 63, c0 = 64 (na w + i) mod ca (later waves
    // repeat the first ones when there are fewer chunks than lanes); token
    // rows: BM cpr chunks, lanes past the last one repeat it into the padding
    constexpr int NW = big_waves<WF>();
    const int cpr = p.K / 512, ca = 256 * ncb * cpr, cb = BM * cpr;
    const int na = (ca + kWave * NW - 1) / (kWave * NW), nb = max(1, cb / (kWave * NW));
#pragma unroll
    for (int i = 0; i < (kBN * (kMxMaxK / 512) + kWave * NW - 1) / (kWave * NW); ++i) {
      if (i < na) {
        const int c0 = ((wave * na + i) * kWave) % ca, ci = c0 + lane;
        const int lw = ci / cpr, part = ci % cpr;
        const uint32_t grow = kGU ? (uint32_t)group * 2 * p.N + (lw < 128 ? n0 + lw : p.N + n0 + lw - 128)
                                  : (uint32_t)group * p.N + n0 + lw;
        load_scale_chunk(asc_lds + c0 * 16, (const uint8_t*)p.w_scale + grow * (uint32_t)kpr + 16 * part);
      }
    }
#pragma unroll
    for (int i = 0; i < (kBigTileRows * (kMxMaxK / 512) + kWave * NW - 1) / (kWave * NW); ++i) {
      if (i < nb) {
        const int ci = min((wave * nb + i) * kWave + lane, cb - 1);
        const int rr = ci / cpr, part = ci % cpr;
        const int r = rr < rows ? row0 + rr : row0;
        const uint32_t src_row = kGU ? (uint32_t)min(max(p.row_token[r], 0), p.T - 1) : (uint32_t)r;
        load_scale_chunk(bsc_lds + (wave * nb + i) * 1024, p.act_scale + src_row * (uint32_t)kpr + 16 * part);
      }
    }
  }
  // 4-bit: the item's fp16 scales and mins -> LDS after the ring (the 256
  // weight rows in item order, K / 32 values per row; 16-byte chunks,
  // lane-consecutive), issued before the first super-stage's loads, so the
  // first wait covers them.  Read per super-stage from global memory instead,
  // each row's 128-byte lines of scales and mins were touched once per
  // super-stage over the whole item and fell out of L2 in between.  The
  // chunks of a row sit XOR-swizzled by the row (when the chunks per row are
  // a power of two), so that the 16 rows of a fragment read one block's
  // values from different banks.
  uint16_t* const qsc_lds = reinterpret_cast<uint16_t*>(lds + ring<WF, kBigTileRows>() * b_stage_bytes<WF, kBigTileRows>());
  uint16_t* const qmn_lds = qsc_lds + kQ4ArrayBytes / 2;
  if constexpr (WF == kQ4) {
    // ncb K chunks per array (256 ncb rows); instruction i of wave w copies
    // chunks c0 .. c0 + 63, c0 = 64 (n w + i) mod (ncb K) (with fewer chunks
    // than lanes in the block, the later waves repeat the first ones: the
    // same bytes to the same place)
    constexpr int NW = big_waves<WF>();
    const int cpr = p.K / 256, chunks = ncb * p.K, n = (chunks + kWave * NW - 1) / (kWave * NW);
    const int sw = (cpr & (cpr - 1)) == 0 ? cpr - 1 : 0;
#pragma unroll
    for (int i = 0; i < (kQ4MaxK + kWave * NW - 1) / (kWave * NW); ++i) {
      if (i < n) {
        const int c0 = ((wave * n + i) * kWave) % chunks, ci = c0 + lane;  // < 256 ncb cpr
        const int lw = ci / cpr, part = (ci % cpr) ^ (lw & sw);
        const uint32_t grow = kGU ? (uint32_t)group * 2 * p.N + (lw < 128 ? n0 + lw : p.N + n0 + lw - 128)
                                  : (uint32_t)group * p.N + n0 + lw;
        const uint32_t off = grow * (uint32_t)(kpr * 2) + 16 * part;
        load_scale_chunk((uint8_t*)qsc_lds + c0 * 16, (const uint8_t*)p.w_scale + off);
        load_scale_chunk((uint8_t*)qmn_lds + c0 * 16, (const uint8_t*)p.w_min + off);
      }
    }
  }
  // This lane's item scales of super-stage S (column block S / nSK, K block
  // 4 (S % nSK) + q): weight fragment b's row; MX also token block 0's row
  // (lr), token block c at + 16 c kpr.
  const int nSK = p.K / kSK;
  auto item_sc = [&](int S0) {
    ItemSc sc{};
    const int cbk = S0 / nSK, S = S0 - cbk * nSK;
#pragma unroll
    for (int b = 0; b < F; ++b) {
      const int lw = local_row(b) + 256 * cbk;
      if constexpr (WF == kMX4) sc.a[b] = asc_lds + lw * kpr + 4 * S + q;
      if constexpr (WF == kQ4) {
        const int cpr = p.K / 256, sw = (cpr & (cpr - 1)) == 0 ? cpr - 1 : 0, blk = 4 * S + q;
        const int i = lw * kpr + (((blk >> 3) ^ (lw & sw)) << 3) + (blk & 7);
        sc.s[b] = qsc_lds[i];
        sc.m[b] = qmn_lds[i];
      }
    }
    if constexpr (WF == kMX4) {
      sc.b = bsc_lds + lr * kpr + 4 * S + q;
      sc.bstep = 16 * kpr;
    }
    return sc;
  };

  f32x4 acc[F][NC];
#pragma unroll
  for (int b = 0; b < F; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Results of column block cbk: fragment b's D[i][j] (i: weight row, j:
  // token) is in lane j + 16 * (i / 4), register i % 4.
  auto store = [&](int cbk) {
  #pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int tr = 16 * c + lr;
      if (tr >= rows) continue;
      const int r = row0 + tr;
      if constexpr (kGU) {
  #pragma unroll
        for (int b = 0; b < F / 2; ++b) {
          const int col = n0 + 256 * cbk + local_row(b) - lr + 4 * q;  // gate fragment b, up fragment b + F / 2
          float v[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu_fast(acc[b][c][i]) * acc[b + F / 2][c][i];
          if constexpr (WF == kMX4) {
            *reinterpret_cast<f32x4*>((float*)p.out + (size_t)r * p.N + col) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
          }
        }
      } else if constexpr (WF == kMX4) {
  #pragma unroll
        for (int b = 0; b < F; ++b) {
          const int col = n0 + 256 * cbk + local_row(b) - lr + 4 * q;
          *reinterpret_cast<f32x4*>((float*)p.out + (size_t)r * p.N + col) = acc[b][c];
        }
      } else {
  #pragma unroll
        for (int b = 0; b < F; ++b) {
          const int col = n0 + 256 * cbk + local_row(b) - lr + 4 * q;
          u32x2 o = {pack_bf16x2(acc[b][c][0], acc[b][c][1]), pack_bf16x2(acc[b][c][2], acc[b][c][3])};
          *reinterpret_cast<u32x2*>((uint16_t*)p.out + (size_t)r * p.N + col) = o;
        }
      }
    }
  };

  // Ring of kRing super-stages.  step(S, j) computes S from slot j while
  // issuing the loads of S + kAhead (clamped to the last super-stage, so that
  // every step issues the same number of loads and the wait below is a
  // constant) into slot (j + kAhead) % kRing, which S - 1 used and the barrier
  // closing S - 1 freed; it then waits until only the loads issued after
  // those of S + 1 are outstanding (none with a ring of two).
  ATile<WF> at[kRing];
  const int nS = ncb * nSK;
  constexpr int L = loads_per_stage<WF, BM>();
  // Part g (0..7) of the loads of super-stage S (column block S / nSK) into slot j.
  auto part = [&](int S, int j, int g) {
    const int cbk = S / nSK, sk = S - cbk * nSK;
    if (g < NB) load_b_part<WF, BM>(lds + j * kBStage, p.act, bsrc, sk, wave, g);
    load_a_part<WF>(p, at[j], arow, (Row)(256 * cbk), sk, q, g);
  };
  auto issue = [&](int S, int j) {
#pragma unroll
    for (int g = 0; g < 8; ++g) part(S, j, g);
  };
  issue(0, 0);
  if constexpr (kAhead > 1) issue(min(1, nS - 1), 1);
  if constexpr (kAhead > 2) issue(min(2, nS - 1), 2);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L * (kAhead - 1)) : "memory");  // super-stage 0 landed
  tie<WF>(at[0]);
  stage_barrier();
  // item scales: MX pointers into LDS; 4-bit values, read one super-stage ahead
  ItemSc isc = item_sc(0);
  auto step = [&](int S, auto slot) {
    constexpr int j = decltype(slot)::value;
    const int S2 = min(S + kAhead, nS - 1);
    const ItemSc cur = isc;
    isc = item_sc(min(S + 1, nS - 1));
    compute<WF, BM>(at[j], lds + j * kBStage, acc, lr, q, [&](int g) { part(S2, (j + kAhead) % kRing, g); },
                    cur);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L * (kAhead - 1)) : "memory");  // super-stage S + 1 landed
    tie<WF>(at[(j + 1) % kRing]);
    stage_barrier();
    if constexpr (kTwoBlocks<WF, kGU>()) {
      if (S + 1 < nS && S + 1 == nSK) {  // the first of two column blocks is done
        store(0);
#pragma unroll
        for (int b = 0; b < F; ++b)
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // Whole rounds of the ring, then the remaining super-stages (fewer than
  // kRing; nested, so that every path through the waits is one the ring takes).
  int S = 0;
  for (; S + kRing <= nS; S += kRing) {
    step(S, std::integral_constant<int, 0>{});
    step(S + 1, std::integral_constant<int, 1>{});
    if constexpr (kRing > 2) step(S + 2, std::integral_constant<int, 2 % kRing>{});
    if constexpr (kRing > 3) step(S + 3, std::integral_constant<int, 3 % kRing>{});
  }
  if (S < nS) {
    step(S, std::integral_constant<int, 0>{});
    if constexpr (kRing > 2)
      if (S + 1 < nS) {
        step(S + 1, std::integral_constant<int, 1>{});
        if constexpr (kRing > 3)
          if (S + 2 < nS) step(S + 2, std::integral_constant<int, 2 % kRing>{});
      }
  }
  // Drain the last (clamped) refills.  Their registers are tied after the wait
  // so that the compiler keeps them reserved until the loads have landed.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < kRing; ++j) tie<WF>(at[j]);
  store(ncb - 1);
}

// Waves per SIMD (blocks per CU): bf16 one (three-deep ring, operand
// prefetch), 4-bit two (see the top of the file).  MX: one -- its 64 x 128
// fp32 accumulators per wave, two register slots of FP4 weights and the FP8
// token fragments (8 registers each) do not fit in half the register file.
template <int WF>
constexpr int big_waves_per_simd() { return big_waves<WF>() / 4; }

// One block per item.  Items of the big-tile list (128-row tiles) and, for
// 4-bit weights, of the small-tile list (<= 64 rows) share the launch: block b
// runs on XCD b % 8, and each XCD takes a contiguous run of the big items
// first and then a contiguous run of the small items, so the small items fill
// the CUs that the last big items leave idle, and the column blocks of one
// row tile (which read the same token rows) share an L2.
template <int WF, bool kGU, bool kSmall>
__global__ __launch_bounds__(big_threads<WF>()) __attribute__((amdgpu_waves_per_eu(big_waves_per_simd<WF>())))
void big_gemm_kernel(Bp p) {
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[ring<WF, kBigTileRows>() * b_stage_bytes<WF, kBigTileRows>() +
              (WF == kMX4 ? kMxScaleBytes : WF == kQ4 ? kQ4ScaleBytes : 0)];
  const int cols = kGU ? kBN / 2 : kBN * p.ncb;  // output columns per item
  const int per_tile = p.N / cols;
  const int big_items = p.sched[kSchedBig] * per_tile;
  const int small_items = kSmall ? p.sched[kSchedSmall] * per_tile : 0;
  const int big_px = (big_items + kXcds - 1) / kXcds, small_px = (small_items + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  if (slot < big_px) {
    const int item = xcd * big_px + slot;
    if (item >= big_items) return;
    const int32_t* tile = p.sched + p.sched[kSchedBigStart] + (size_t)(item / per_tile) * kTileInts;
    gemm_item<WF, kGU, kBigTileRows>(p, lds, tile[0], tile[1], tile[2], (item % per_tile) * cols);
  } else if (kSmall && slot < big_px + small_px) {
    const int item = xcd * small_px + (slot - big_px);
    if (item >= small_items) return;
    const int32_t* tile = p.sched + kSchedHeader + (size_t)(item / per_tile) * kTileInts;
    const int rows = tile[2], n0 = (item % per_tile) * cols;
    // item height by the tile's rows (uniform over the block)
    if (WF != kMX4 && rows <= 16)
      gemm_item<WF, kGU, WF == kMX4 ? 32 : 16>(p, lds, tile[0], tile[1], rows, n0);
    else if (rows <= 32)
      gemm_item<WF, kGU, 32>(p, lds, tile[0], tile[1], rows, n0);
    else
      gemm_item<WF, kGU, kTileRows>(p, lds, tile[0], tile[1], rows, n0);
  }
}

// bf16: one wave per SIMD (the accumulators, 64 x 128 per wave, and the
// three-deep A register ring need more than half the register file); 4-bit:
// two (see the top of the file).  A spill would add scratch loads to the
// vmcnt accounting of the ring: the build's assembly check rejects it.
template <bool kGU>
hipError_t launch(const GemmArgs& a, bool with_small, hipStream_t stream) {
  if (a.wfmt != kBF16 && a.wfmt != kQ4 && a.wfmt != kMX4) return hipErrorInvalidValue;
  if (!with_small) return hipErrorInvalidValue;  // the small tiles always run in the same launch
  const bool mx = a.wfmt == kMX4;
  if (mx && (a.K % 512 != 0 || a.K > kMxMaxK)) return hipErrorInvalidValue;
  if (a.wfmt == kQ4 && (a.K % 256 != 0 || a.K > kQ4MaxK)) return hipErrorInvalidValue;
  // down items of long calls take two 256-column blocks where N allows and
  // their scales fit the item's LDS copy (short K: the per-item prologue and
  // epilogue weigh most there); shorter calls keep one, for enough items to
  // spread evenly over the CUs
  const int max_k = mx ? kMxMaxK : kQ4MaxK;
  const int ncb = !kGU && a.wfmt != kBF16 && a.T >= kBigTileMinTokens && a.N % (2 * kBN) == 0 && 2 * a.K <= max_k
                      ? 2 : 1;
  const int cols = kGU ? kBN / 2 : kBN * ncb;
  if (a.N % cols != 0 || a.K % kSK != 0) return hipErrorInvalidValue;
  Bp p{mx ? (const void*)a.act_q : a.act, mx ? (const uint8_t*)a.act_scale : nullptr, a.row_token, a.sched, a.w,
       a.w_scale, a.w_min, a.out, a.K, a.N, a.T, a.R, ncb};
  // grid: per XCD, slots for an upper bound of each list's items (big tiles
  // hold >= kBigPartMin rows)
  const int64_t per_tile = a.N / cols;
  const int64_t big_px = (((int64_t)a.R / kBigPartMin + 1) * per_tile + kXcds - 1) / kXcds;
  const int64_t small_px = with_small ? ((int64_t)sched_small_cap(a.R, a.G) * per_tile + kXcds - 1) / kXcds : 0;
  const int64_t blocks = (big_px + small_px) * kXcds;
  if (blocks > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  if (mx)
    hipLaunchKernelGGL((big_gemm_kernel<kMX4, kGU, true>), dim3(blocks), dim3(big_threads<kMX4>()), 0, stream, p);
  else if (a.wfmt == kQ4)
    hipLaunchKernelGGL((big_gemm_kernel<kQ4, kGU, true>), dim3(blocks), dim3(big_threads<kQ4>()), 0, stream, p);
  else
    hipLaunchKernelGGL((big_gemm_kernel<kBF16, kGU, true>), dim3(blocks), dim3(big_threads<kBF16>()), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_big_gate_up(const GemmArgs& a, bool with_small, hipStream_t stream) {
  return launch<true>(a, with_small, stream);
}
hipError_t launch_big_down(const GemmArgs& a, bool with_small, hipStream_t stream) {
  return launch<false>(a, with_small, stream);
}

}  // namespace moe
