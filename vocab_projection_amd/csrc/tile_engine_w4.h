// tile_engine_w4.h - the 256x256 MFMA tile of C = A . B^T with one wave per
// SIMD (gfx950), for bf16 operands: K-contiguous ones in rows of 128 bytes
// (KRow128), or any layout of the eight-wave engine through Pair.
//
// A block of 256 threads: four wave64s in a 2x2 grid, one per SIMD, each
// owning a 128x128 sub-tile of fp32 accumulators (8 x 8 MFMA tiles of
// 16 x 16, all 256 accumulation registers).  Against the eight-wave engine
// (tile_engine.h, 128x64 per wave) a K step takes 16 fragment reads from LDS
// for 64 MFMAs instead of 12 for 32: a third fewer reads per MFMA, and half
// the waves issuing them.  K advances in stages of 64 elements (128 bytes per
// row, two MFMA K steps) held in two LDS buffers of 64 KiB.  Global memory
// goes to LDS by LDS-DMA (no staging registers), one stage ahead of the
// MFMAs, spread over the MFMA stream so that no copy burst stalls it; one
// barrier per stage separates a buffer's last reads from its next copies and
// its copies' completion from its first reads (the schedule is set out above
// run_tiles).  The copy stream runs across the block's tiles (persistent
// blocks), so a tile's epilogue overlaps the next tile's first copies.  Rows
// past an operand's extent and K past its end read as zeros through the
// buffer descriptors' range checks.
#pragma once

#include <type_traits>

#include "tile_engine.h"

namespace lce {
namespace w4 {

constexpr int kThreads = 256;
constexpr int kWaves = 4;                        // 2 along M x 2 along N
constexpr int kWaveM = 128;
constexpr int kWaveN = 128;
constexpr int kMI = kWaveM / kMfma;              // 8
constexpr int kNI = kWaveN / kMfma;              // 8
constexpr int kStageK = 64;                      // bf16 K elements per stage
constexpr int kRowBytes = kStageK * 2;           // 128
constexpr int kOpBytes = kTile * kRowBytes;      // one operand's stage: 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;        // A and B: 64 KiB
constexpr int kLdsBytes = 2 * kStageBytes;       // two stage buffers
constexpr int kStagingBytes = 32 * 1024;         // epilogue staging after them (GEMMs only)
constexpr int kLoads = kOpBytes / 16 / kThreads; // 16-byte loads per thread per operand per stage
static_assert(kLoads == 8 && kLdsBytes + kStagingBytes <= 160 * 1024, "stage geometry");

// Accumulators of one wave, with the wave shape the epilogues read.
// The epilogues read it element by element through read(), which moves one
// accumulator register to a VGPR where it is used: left to itself the compiler
// copies all 256 out at the end of the loop and spills them.
struct Acc {
  static constexpr int MI = kMI, NI = kNI, WaveM = kWaveM, WaveN = kWaveN;
  f32x4_t c[kMI][kNI];
  __device__ __forceinline__ static float read(const f32x4_t& v, int e) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v[e]));
    return r;
  }
};

// The MFMAs accumulate in place in accumulation registers, written as inline
// assembly with a tied operand: through the builtin, the register allocator
// does not keep an accumulator in one place when all 256 accumulation
// registers are in use, and copies every accumulator around each stage.  The
// first MFMA of a tile adds to the constant 0, so no accumulator is cleared by
// a VALU write (which would need wait states before an MFMA reads it).  The
// hazards the compiler does not see in inline assembly are covered by hand:
// an accumulator is read back only after at least 32 wait states
// (end_of_tile), and consecutive MFMAs on one accumulator are 32 MFMAs apart.
__device__ __forceinline__ void mfma_acc(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void end_of_tile() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Rows of a stage in LDS are 128 bytes (8 chunks of 16); chunk c of row r sits
// at c ^ swz(r).  A fragment read takes one chunk of 16 consecutive rows per
// 16 lanes; with the swizzle those land on 16 distinct 16-byte bank groups of
// the 256-byte bank period, and so do the 16 lanes of a stage write (two
// whole rows).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Operand sides.  A side fills its operand's half of a stage buffer (kOpBytes
// at dst) with copy i = 0..7 of this wave for stage kt of the tile it is
// pointed at, and reads the fragment of 16-row (or 16-column) sub-tile mi for
// K step ks of a stage at src:
//   init(op, mn0, wave, lane, sub0)   per-lane offsets; sub0 = the wave's first
//                                     row (column) in the tile
//   retarget_if(op, mn0, yes)         point the copies at the tile at mn0 if
//                                     yes (branch-free)
//   copy(dst, kt, wave, live, i)      a dead copy (live == false) reads zeros
//   frag(src, ks, mi)

// K-contiguous bf16 operand kept as 256 rows of 128 bytes (both K steps of a
// stage in one row).  Copy i of wave w fills rows 8 c .. 8 c + 7, c = 8 w + i;
// lane l fills physical chunk l % 8 of row 8 c + l / 8, i.e. reads the row's
// logical chunk (l % 8) ^ swz(row).  A fragment read: lane l reads row l % 16
// of the sub-tile, logical chunk 4 ks + l / 16.
struct KRow128 {
  u32x4_t rsrc;
  int64_t k_ext_bytes;
  uint32_t voff[kLoads];  // per copy: row * row_bytes + logical chunk * 16
  uint32_t kb[2];         // logical chunk bytes of even and odd copies
  uint32_t off[2];        // per K step: this lane's fragment offset in sub-tile 0

  __device__ __forceinline__ void retarget(const Operand<__bf16>& op, int64_t mn0) {
    rsrc = make_rsrc(op.base + mn0 * op.ld, (op.mn_ext - mn0) * op.ld * 2);
  }
  __device__ __forceinline__ void retarget_if(const Operand<__bf16>& op, int64_t mn0, bool yes) {
    const u32x4_t r = make_rsrc(op.base + mn0 * op.ld, (op.mn_ext - mn0) * op.ld * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) rsrc[q] = yes ? r[q] : rsrc[q];
  }
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t mn0, int wave, int lane,
                                       int sub0) {
    const int64_t row_bytes = op.ld * 2;
    k_ext_bytes = op.k_ext * 2;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = kLoads * wave + i;
      const int row = 8 * c + (lane >> 3);
      const int lc = (lane & 7) ^ swz(row);
      voff[i] = (uint32_t)(row * row_bytes + lc * 16);
      if (i < 2) kb[i] = (uint32_t)(lc * 16);  // swz(row) depends on c only through c & 1
    }
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      off[ks] = (uint32_t)((sub0 + j) * kRowBytes + (((4 * ks + g) ^ swz(j)) * 16));
    retarget(op, mn0);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live, int i) const {
    const int64_t k0 = kt * kRowBytes;
    const bool ok = live && k0 + kb[i & 1] < k_ext_bytes;
    // (the stage offset is uniform; readfirstlane keeps it in an SGPR)
    dma16(rsrc, dst + (kLoads * wave + i) * 1024, ok ? voff[i] : kOutOfRange,
          __builtin_amdgcn_readfirstlane(live ? (uint32_t)k0 : 0u));
  }
  __device__ __forceinline__ u32x4_t frag(const char* src, int ks, int mi) const {
    return *reinterpret_cast<const u32x4_t*>(src + off[ks] + mi * kMfma * kRowBytes);
  }
};

// An operand side of the eight-wave engine (tile_engine.h), built for four
// copies per wave: its stages are one MFMA K step (kOperandBytes = 16 KiB), so
// stage kt here is its stages 2 kt and 2 kt + 1, one after the other.  Copies
// 0..3 of a wave fill the first, 4..7 the second.
constexpr int kCopiesPerSub = kLoads / 2;
template <typename S>
struct Pair {
  S s;
  int64_t mn0;  // the tile the copies point at
  static_assert(2 * kOperandBytes == kOpBytes, "two stages of the eight-wave engine per stage");
  __device__ __forceinline__ void retarget_if(const Operand<__bf16>& op, int64_t next, bool yes) {
    mn0 = yes ? next : mn0;
    s.retarget(op, mn0);
  }
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t first, int wave, int lane,
                                       int sub0) {
    mn0 = first;
    s.init(op, first, wave, lane, sub0);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live, int i) const {
    const int h = i / kCopiesPerSub;
    s.copy_at(dst + h * kOperandBytes, 2 * kt + h, wave, live, i % kCopiesPerSub);
  }
  __device__ __forceinline__ u32x4_t frag(const char* src, int ks, int mi) const {
    return s.frag(src + ks * kOperandBytes, mi);
  }
};

// The eight-wave engine's layouts with four copies per wave: K-contiguous
// gradient strip in blocks (split placement), MN-contiguous bf16 (descriptor
// computed per stage), and the blocked MN-contiguous gradient strip.
using KSplitBlk = Pair<SideK<__bf16, true, true, kCopiesPerSub>>;
using MN = Pair<SideMNb16<false, kCopiesPerSub>>;
using MNBlk = Pair<SideMNb16Blk<kCopiesPerSub>>;

// Until every copy and LDS access of this wave is done (vmcnt(0) lgkmcnt(0)).
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Half h of K step ks: the MFMAs of sub-tiles mi in [4 h, 4 h + 4) for every
// ni, ni-major, each followed (per the caller's plan) by one fragment read and
// at most one stage copy (after MFMAs 1, 1 + Gap, ...), in program order
// (scheduling fences keep it).
//   h = 0: reads a[4..8) of this K step (their registers were freed by the
//          last half);
//   h = 1: reads a[0..4) of the next K step (free since half 0) and each b[ni]
//          of the next K step right after its last MFMA here.
template <int H, bool First, int Gap = 4, typename SA, typename SB, typename CopyFn>
__device__ __forceinline__ void half_step(Acc& acc, u32x4_t (&a)[kMI], u32x4_t (&b)[kNI],
                                          const SA& sa, const SB& sb, const char* a_src,
                                          const char* b_src, int ks_read, int n_copies,
                                          CopyFn&& copy_fn) {
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int ni = t / 4, mi = 4 * H + t % 4;
    if constexpr (First)
      mfma_first(acc.c[mi][ni], a[mi], b[ni]);
    else
      mfma_acc(acc.c[mi][ni], a[mi], b[ni]);
    if constexpr (H == 0) {
      if (t < 4) a[4 + t] = sa.frag(a_src, ks_read, 4 + t);
    } else {
      if (t % 4 == 3) b[ni] = sb.frag(b_src, ks_read, ni);
      else if (t < 5) a[t < 3 ? t : t - 1] = sa.frag(a_src, ks_read, t < 3 ? t : t - 1);
    }
    if (t % Gap == 1 && t / Gap < n_copies) copy_fn(t / Gap);
    sched_fence();
  }
}

// Every tile of this block: pre(m0, n0) (loads that the epilogue needs, which
// then complete under the tile's stages), C[m0:m0+256, n0:n0+256] = sum_k
// A[m, k] B[n, k] over k < k_len, then epi(acc, m0, n0, staging), where
// staging is the kStagingBytes of LDS past the two stage buffers.  Needs at
// least two K stages per tile (the copy stream runs at most one tile ahead).
//
// Stage q lives in buffer q % 2 and has two K steps; with the MFMAs at stage q:
//   half 0 of step 0:  reads a[4..8) of step 0; B's copies of stage q + 1
//                      into the other buffer, one per four MFMAs (A's were
//                      issued before) - unless Late;
//   half 1 of step 0:  reads a[0..4) and b of step 1;
//   half 0 of step 1:  reads a[4..8) of step 1 (the last reads of buffer q);
//   wait for every copy (stage q + 1's) and read; barrier;
//   half 1 of step 1:  reads a[0..4) and b of stage q + 1's step 0 from the
//                      other buffer; A's copies of stage q + 2 into buffer q,
//                      one per four MFMAs, or with Late both operands'
//                      copies, one per two MFMAs.
// Late gives B's copies a whole stage of lead instead of half of one: the
// gradient strip with many tiles per block gains from it (1%), with two
// tiles per block it loses (3%), and dW (MN-contiguous operands, a
// descriptor computed per copy) loses 6%.  A buffer is written
// only after the barrier that follows its last reads, and read only after
// the barrier that follows its copies' completion.  The epilogue's loads and
// stores are waited for with the copies at the next barrier.
template <typename SA, typename SB, bool Late = false, typename Pre, typename Epi>
__device__ __forceinline__ void run_tiles(const Operand<__bf16>& A, const Operand<__bf16>& B,
                                          int64_t k_len, const TileGrid& grid, char* lds,
                                          Pre&& pre, Epi&& epi) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t lds0 = lds_addr(lds);
  char* const staging = lds + kLdsBytes;
  const int64_t nk = (k_len + kStageK - 1) / kStageK;
  const int64_t tiles = grid.count();
  if (tiles == 0) return;

  int64_t m0, n0, next_m0, next_n0;
  grid.coords(0, &m0, &n0);
  next_m0 = m0;
  next_n0 = n0;
  if (tiles > 1) grid.coords(1, &next_m0, &next_n0);

  SA sa;
  SB sb;
  sa.init(A, m0, wave, lane, wm * kWaveM);
  sb.init(B, n0, wave, lane, wn * kWaveN);

  // copy stream: stage ck of the block's tile ct; copy i < 8 is A's, else
  // B's.  Branch-free, so that a stage is one basic block: a branch in the
  // loop made the register allocator shuttle accumulators between AGPRs and
  // VGPRs.
  int64_t ct = 0, ck = 0;
  auto advance = [&]() {
    const bool wrap = ++ck == nk;
    ck = wrap ? 0 : ck;
    ct += wrap ? 1 : 0;
    // the stream is at most one tile ahead of the MFMAs: tile ct is the next one
    sa.retarget_if(A, next_m0, wrap);
    sb.retarget_if(B, next_n0, wrap);
  };
  auto copy_one = [&](uint32_t buf_addr, int i) {
    if (i < kLoads)
      sa.copy(buf_addr, ck, wave, ct < tiles, i);
    else
      sb.copy(buf_addr + kOpBytes, ck, wave, ct < tiles, i - kLoads);
  };

  // stage 0 into buffer 0; stage 1 (Late), or A's half of it, into buffer 1
  constexpr int kAhead = Late ? 2 * kLoads : kLoads;  // copies of stage 1
#pragma unroll
  for (int i = 0; i < 2 * kLoads; ++i) copy_one(lds0, i);
  advance();
#pragma unroll
  for (int i = 0; i < kAhead; ++i) copy_one(lds0 + kStageBytes, i);
  if constexpr (Late) advance();
  __builtin_amdgcn_s_waitcnt((kAhead & 15) | ((kAhead >> 4) << 14) | (7 << 4));  // stage 0 landed
  block_barrier();

  Acc acc;
  u32x4_t a[kMI], b[kNI];
#pragma unroll
  for (int i = 0; i < kMI / 2; ++i) a[i] = sa.frag(lds, 0, i);
#pragma unroll
  for (int i = 0; i < kNI; ++i) b[i] = sb.frag(lds + kOpBytes, 0, i);
  uint32_t buf = 0;

  for (int64_t t = 0; t < tiles; ++t) {
    // one stage; the first of a tile starts the accumulators from 0
    auto stage = [&](auto first) {
      constexpr bool kFirst = decltype(first)::value;
      const char* const cur = lds + buf * kStageBytes;
      const char* const nxt = lds + (buf ^ 1) * kStageBytes;
      const uint32_t cur_addr = lds0 + buf * kStageBytes;
      const uint32_t nxt_addr = lds0 + (buf ^ 1) * kStageBytes;
      auto copy_b = [&](int i) { copy_one(nxt_addr, kLoads + i); };
      auto copy_a = [&](int i) { copy_one(cur_addr, i); };  // i >= kLoads: B's (Late)
      auto none = [&](int) {};
      half_step<0, kFirst>(acc, a, b, sa, sb, cur, cur + kOpBytes, 0, Late ? 0 : kLoads, copy_b);
      if constexpr (!Late) advance();
      half_step<1, kFirst>(acc, a, b, sa, sb, cur, cur + kOpBytes, 1, 0, none);
      half_step<0, false>(acc, a, b, sa, sb, cur, cur + kOpBytes, 1, 0, none);
      wait_all();
      block_barrier();
      half_step<1, false, Late ? 2 : 4>(acc, a, b, sa, sb, nxt, nxt + kOpBytes, 0,
                                        Late ? 2 * kLoads : kLoads, copy_a);
      if constexpr (Late) advance();
      buf ^= 1;
    };
    pre(m0, n0);
    stage(std::true_type{});
    for (int64_t kt = 1; kt < nk; ++kt) stage(std::false_type{});
    end_of_tile();
    epi(acc, m0, n0, staging);
    m0 = next_m0;
    n0 = next_n0;
    if (t + 2 < tiles) grid.coords(t + 2, &next_m0, &next_n0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // nothing in flight when the block ends
}

}  // namespace w4
}  // namespace lce
