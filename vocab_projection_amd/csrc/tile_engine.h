// tile_engine.h - one 256x256 MFMA tile of C = A . B^T on gfx950 (CDNA4).
//
// A block of 512 threads (eight wave64s in a 2x4 grid, two per SIMD, each
// owning a 128x64 sub-tile of fp32 accumulators as 8 x 4 MFMA tiles of
// 16 x 16) walks K in stages of 64 bytes per row (32 bf16 or 16 f32
// elements).  Two waves per SIMD let one
// wave's MFMAs run while the other waits on an LDS read or on the texture
// unit; LDS read bandwidth (about 240 B/clk per CU with eight waves, half
// that with four) covers the 1.5x fragment reads this layout costs.  Stages
// are copied from global memory straight into LDS with buffer_load ... lds
// (no register staging) into a ring of kStages buffers, so a stage is copied
// kStages - 1 stages before it is read.
// The copies of a stage are spread over the MFMAs of the stage before: two
// wave-wide copies per half stage of 16 MFMAs, after MFMAs 0 and 4 (0 and 8
// where both operands are MN-contiguous).  The texture unit takes many cycles
// per 1 KiB copy and is shared by the CU's waves, so copies issued in a
// burst stall every wave's MFMA issue at once; spread out, they hide behind
// the MFMAs.  The lead given by the ring is what lets them be spread.
// Fragments are read back from LDS as 16-byte K-runs that feed
// v_mfma_f32_16x16x32_bf16 (bf16: one MFMA takes a whole stage's K) or four
// v_mfma_f32_16x16x4_f32 (f32), half a stage ahead of their MFMAs.  Under
// the part's power limit the 16x16x32 form delivers more FLOP per joule than
// 32x32x16: it reads and writes a quarter of the accumulator bytes per MFMA
// for half the FLOP.
//
// Operands may be stored K-contiguous (element (mn, k) at row mn, column k)
// or MN-contiguous (element (mn, k) at row k, column mn):
//  - a K-contiguous stage is kept as 256 rows of four 16-byte chunks, the
//    chunk index XOR-swizzled by the row, and read with ds_read_b128;
//  - an MN-contiguous bf16 stage is kept as 32 k-rows of 512 bytes (chunk
//    index swizzled by the k-row) and read with ds_read_b64_tr_b16, which
//    hands each lane four K values of one column; two such reads make a
//    fragment.  f32 stages (16 k-rows of 1 KiB) are read one float at a time.
// The MN-contiguous swizzles and the split K-contiguous placement (below) keep
// every fragment read free of LDS bank conflicts (64 four-byte banks, 256
// bytes per cycle); the row-major K-contiguous placement, kept for the f32
// gradient strip beside a transposed operand, costs a 2-way conflict.
//
// The bf16 gradient strip (the A operand of dH and dW) is kept in 1 KiB blocks
// of 16 tokens x 64 bytes (BlockedG), so that a copy of either GEMM moves one
// contiguous kilobyte and the gradient epilogue stores whole blocks from
// registers.
//
// Loads go through buffer resources whose record count ends at the last
// valid row, so rows past the operand's extent read as zeros and nothing is
// read out of bounds; the tile needs no masking in its inner loop.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

constexpr int kTile = 256;                 // block tile along M and along N
constexpr int kWaves = 8;                  // waves per block, 2 along M x kWaves / 2 along N
constexpr int kWaveM = 128;                // wave sub-tile along M
constexpr int kWaveN = kTile / (kWaves / 2);  // wave sub-tile along N
constexpr int kMfma = 16;                  // MFMA tile edge (16 x 16 outputs)
constexpr int kMI = kWaveM / kMfma;        // MFMA tiles of a wave along M
constexpr int kNI = kWaveN / kMfma;        // MFMA tiles of a wave along N
constexpr int kThreads = 64 * kWaves;
constexpr int kStageRowBytes = 64;         // K bytes per row per stage (one 16x16x32 bf16 MFMA)
constexpr int kChunks = kStageRowBytes / 16;  // 16-byte chunks per row per stage
constexpr int kOperandBytes = kTile * kStageRowBytes;   // per operand per stage
constexpr int kStageBytes = 2 * kOperandBytes;          // A and B
constexpr int kStages = 3;                 // ring of stages in LDS
constexpr int kRingBytes = kStages * kStageBytes;
constexpr int kStagingBytes = 64 * 1024;   // epilogue staging, after the ring
constexpr int kLdsBytes = kRingBytes + kStagingBytes;
constexpr int kCopiesPerWave = kOperandBytes / 1024 / kWaves;  // 1 KiB per wave-wide copy
constexpr int kRowsPerCopy = 1024 / kStageRowBytes;       // K-contiguous rows per copy
static_assert(kStageRowBytes == 64 && kChunks == 4, "a stage is one 16-byte run per lane group");
static_assert(kStages >= 3 && kLdsBytes <= 160 * 1024, "ring and staging fit in LDS");
constexpr uint32_t kOutOfRange = 0x80000000u;           // voffset that reads zeros
constexpr int kRsrcWord3 = 0x00020000;                  // raw buffer, gfx9 family

// Swizzle of a K-contiguous stage: physical chunk = logical chunk ^ swz_k(row)
// (a function of row bits 1..3 only).
__device__ __forceinline__ int swz_k(int r) {
  return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
}
// Swizzle of an MN-contiguous bf16 stage: physical chunk = chunk ^ swz_mn(k-row).
// A transposed fragment read covers, per 32 lanes, the same two chunks of the
// k-rows {0..3, 8..11} (+ 4, + 16): XOR-ing the 32-byte window index with
// (k & 3) | ((k >> 3) & 1) << 2 puts those eight k-rows in eight different
// 32-byte windows of the 256-byte bank period.
__device__ __forceinline__ int swz_mn(int k) {
  return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
}

// Record count of a descriptor for `bytes` bytes, capped at 2^31 so that the
// out-of-range offset kOutOfRange (2^31) is always past the end.  Every tile
// addresses at most 256 rows of at most 8 MiB (the host limits H <= 2^20 and
// strip <= 2^21), i.e. offsets below 2^31, so the cap never hides valid data.
__device__ __forceinline__ uint32_t record_count(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= (int64_t)kOutOfRange ? kOutOfRange : (uint32_t)bytes);
}

// Raw buffer descriptor for the byte range [base, base + bytes): 48-bit base,
// stride 0, record count, gfx9 raw-buffer word 3.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, record_count(bytes),
                 (uint32_t)kRsrcWord3};
}

// The same range as a compiler-visible buffer resource (for loads and stores
// whose completion the compiler tracks).  Only the VGPR offset (plus the
// immediate) is range-checked against the record count, so callers put every
// row- and column-dependent part of an address there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buffer(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)record_count(bytes), kRsrcWord3);
}

// LDS byte address of a pointer into the block's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (one
// wave-wide 1 KiB copy).  Issued as inline assembly so that the compiler does
// not treat later LDS reads as waiting on it: completion is tracked by hand
// with s_waitcnt vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(u32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// Barrier of the block that also publishes this wave's LDS accesses: the
// hardware barrier does not wait for them, so LDS writes (and reads) still in
// flight are waited for first (lgkmcnt(0)); without it a wave past the barrier
// could read staging rows before another wave's writes had landed.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Operand in global memory.  K-contiguous: mn_ext rows of ld elements, of
// which the first k_ext are used.  MN-contiguous: k_ext rows of ld elements,
// of which the first mn_ext are used.
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;
  int64_t mn_ext;
  int64_t k_ext;
};

// ---------------------------------------------------------------------------
// Stage copies (global -> LDS) and fragment reads (LDS -> registers).
// ---------------------------------------------------------------------------
// Operand layouts in LDS: MN-contiguous (the copy descriptor recomputed per
// stage, or followed by adds), K-contiguous row-major, and K-contiguous with
// the split sub-tile placement below.
enum : int {
  kMN = 0, kKRow = 1, kKSplit = 2, kMNStep = 3,
  // a bf16 gradient strip kept in blocks (see BlockedG below): the split
  // K-contiguous LDS layout, and a blocked transposed one
  kKSplitBlk = 5, kMNBlkStep = 6
};
__host__ __device__ constexpr bool is_mn(int l) { return l == kMN || l == kMNStep || l == kMNBlkStep; }

// A gradient strip in blocks: element (t, v) of an operand with row length ld
// (elements) lives in block (t / 16, v / kBlkCols) of 16 rows x 64 bytes
// (1 KiB), blocks of one 16-row band side by side along v, bands ld * elt * 16
// bytes apart; inside a block the rows are 64 bytes apart.  A 64-byte K stage
// of 16 rows - a K-contiguous copy, or the accumulators of two 16 x 16 MFMA
// tiles of one wave - is then one contiguous kilobyte.
struct BlockedG {
  static constexpr int kBlkBytes = 1024;
  static constexpr int kBlkRows = 16;
  static constexpr int kRowBytes = 64;
  // bytes between 16-row bands of an operand whose rows hold ld elements of elt bytes
  __host__ __device__ static constexpr int64_t band_bytes(int64_t ld, int64_t elt) {
    return ld * elt * kBlkRows;
  }
};
template <typename T, int L> struct Side;

// Buffer descriptor of an MN-contiguous operand's current stage (kElt-byte
// elements), the record count stopping at the operand's last byte.  Step =
// false recomputes it from the stage index at each copy; Step = true follows
// it with two adds per stage.  (Which is faster depends on the kernel:
// following measured 3% faster where both operands are MN-contiguous, 2%
// slower for dH.)
template <bool Step, int kElt>
struct MNDesc {
  static constexpr int kStageRows = kStageRowBytes / kElt;  // k-rows per stage
  int64_t row_bytes;
  const char* base;  // element (mn0, first k-row of the current stage; of stage 0 if !Step)
  int64_t bytes;     // bytes from base to the operand's last byte
  __device__ __forceinline__ void retarget(const void* p, int64_t b) {
    base = reinterpret_cast<const char*>(p);
    bytes = b;
  }
  __device__ __forceinline__ void step() {
    if constexpr (Step) {
      base += kStageRows * row_bytes;
      bytes -= kStageRows * row_bytes;
    }
  }
  __device__ __forceinline__ u32x4_t rsrc(int64_t kt) const {
    if constexpr (Step) {
      return make_rsrc(base, bytes);
    } else {
      const int64_t k0 = kt * kStageRows * row_bytes;
      return make_rsrc(base + k0, bytes - k0);
    }
  }
};

// K-contiguous operand.  A stage is 16 blocks of 1 KiB, each 16 row slots of
// 64 bytes (four 16-byte chunks, chunk index XOR-swizzled by swz_k(slot)).
// Row-major (kKRow): block b, slot s holds row 16 b + s.  Split (kKSplit):
// each 32-row group of the tile (two 16-row MFMA sub-tiles h = 0, 1) takes
// two blocks b = 0, 1, and block b, slot 8 h + s holds row 16 h + 8 b + s of
// the group.  A fragment read (lane l: row l % 16 of a sub-tile, chunk
// l / 16) then takes 8 slots from each of two blocks, which measured free of
// LDS bank conflicts, while 16 slots of one block cost a 2-way conflict on
// every read.  The split placement pays where both operands are
// K-contiguous (the strip kernels, 1% faster); with a transposed operand
// beside it (dH) the row-major one measured 3% faster.  Copy i of wave w
// fills block c = c w + i (c = CPW): lane l reads physical chunk
// l % kChunks of the row in slot l / kChunks, 64 contiguous bytes per 4 lanes.
// CPW is the number of copies per wave (16 / waves per block).
template <typename T, bool Split, bool Blk = false, int CPW = kCopiesPerWave>
struct SideK {
  u32x4_t rsrc;
  uint32_t voff[CPW];
  uint32_t kbyte;        // byte column of this lane's logical chunk
  int64_t k_ext_bytes;
  uint32_t frag_off[2];  // byte offset of this lane's fragment, even and odd sub-tile of pair 0

  // Point the copies at the tile whose first row is mn0 (a multiple of 16).
  __device__ __forceinline__ void retarget(const Operand<T>& op, int64_t mn0) {
    if constexpr (Blk) {
      const int64_t band = BlockedG::band_bytes(op.ld, sizeof(T));
      rsrc = make_rsrc(reinterpret_cast<const char*>(op.base) + (mn0 / 16) * band,
                       ((op.mn_ext + 15) / 16 - mn0 / 16) * band);
    } else {
      rsrc = make_rsrc(op.base + mn0 * op.ld, (op.mn_ext - mn0) * op.ld * (int64_t)sizeof(T));
    }
  }
  __device__ __forceinline__ void step() {}  // stages differ by the scalar offset only
  // Per-lane copy and fragment offsets (the same for every tile).
  __device__ __forceinline__ void init_lanes(const Operand<T>& op, int wave, int lane, int sub0) {
    const int64_t row_bytes = op.ld * (int64_t)sizeof(T);
    k_ext_bytes = op.k_ext * (int64_t)sizeof(T);
    const int slot = lane / kChunks;  // row slot within a copy's block
    static_assert(kRowsPerCopy == 16, "a copy fills one block of 16 slots");
    kbyte = (uint32_t)(((lane % kChunks) ^ swz_k(slot)) * 16);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = CPW * wave + i;  // block
      const int row = Split ? 32 * (c >> 1) + 16 * (slot >> 3) + 8 * (c & 1) + (slot & 7)
                            : 16 * c + slot;
      if constexpr (Blk)
        voff[i] = (uint32_t)((row / 16) * BlockedG::band_bytes(op.ld, sizeof(T)) +
                             (row % 16) * BlockedG::kRowBytes) + kbyte;
      else
        voff[i] = (uint32_t)(row * row_bytes) + kbyte;
    }
    // fragment: row j = lane % 16 of the sub-tile, logical chunk lane / 16
    // (K elements 8 (lane / 16) .. + 8 of bf16, 4 (lane / 16) .. + 4 of f32).
    // Split: sub-tile h of a pair has row j in block j / 8, slot 8 h + j % 8.
    // sub0 is a multiple of 32 rows.
    const int j = lane & 15;
#pragma unroll
    for (int h = 0; h < (Split ? 2 : 1); ++h) {
      const int fslot = Split ? 8 * h + (j & 7) : j;  // slot from the pair's first block
      frag_off[h] = (uint32_t)(sub0 * kStageRowBytes + (Split ? (j >> 3) * 1024 : 0) +
                               fslot * kStageRowBytes + (((lane >> 4) ^ swz_k(fslot)) * 16));
    }
  }
  __device__ __forceinline__ void init(const Operand<T>& op, int64_t mn0, int wave, int lane,
                                       int sub0) {
    init_lanes(op, wave, lane, sub0);
    retarget(op, mn0);
  }
  // Copy stage kt (K bytes [kt, kt + 1) * kStageRowBytes) to LDS address dst;
  // a dead copy (live == false) reads zeros.  In blocks, stage kt is block
  // column kt of the band.
  // Copy i (< CPW) of this wave.
  __device__ __forceinline__ void copy_one(uint32_t dst, int64_t kt, int wave, bool live,
                                          int i) const {
    const int64_t k0 = kt * kStageRowBytes;
    const uint32_t soff = live ? (uint32_t)(Blk ? kt * BlockedG::kBlkBytes : k0) : 0u;
    const bool ok = live && k0 + kbyte < k_ext_bytes;
    dma16(rsrc, dst + (CPW * wave + i) * 1024, ok ? voff[i] : kOutOfRange, soff);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live) const {
#pragma unroll
    for (int i = 0; i < CPW; ++i) copy_one(dst, kt, wave, live, i);
  }
  // The same, for a caller that never steps the side (stages differ only by kt).
  __device__ __forceinline__ void copy_at(uint32_t dst, int64_t kt, int wave, bool live,
                                         int i) const {
    copy_one(dst, kt, wave, live, i);
  }
  // Fragment of 16-row sub-tile mi of the stage at src (pair mi / 2 is the
  // 32-row group's 2 KiB).
  __device__ __forceinline__ u32x4_t frag(const char* src, int mi) const {
    if constexpr (Split)
      return *reinterpret_cast<const u32x4_t*>(src + frag_off[mi & 1] +
                                               (mi >> 1) * 2 * kMfma * kStageRowBytes);
    else
      return *reinterpret_cast<const u32x4_t*>(src + frag_off[0] + mi * kMfma * kStageRowBytes);
  }
};

template <typename T> struct Side<T, kKRow> : SideK<T, false> {};
template <typename T> struct Side<T, kKSplit> : SideK<T, true> {};
template <> struct Side<__bf16, kKSplitBlk> : SideK<__bf16, true, true> {};

// MN-contiguous bf16 operand: a stage is kStageRowBytes / 2 k-rows x 256 mn.
// Copy i of wave w covers k-rows 2 (c w + i) and +1 (c = CPW, copies per
// wave); lane l fills physical chunk l % 32 of k-row 2 (c w + i) + l / 32.
template <bool Step, int CPW = kCopiesPerWave>
struct SideMNb16 {
  MNDesc<Step, 2> d;
  uint32_t voff[CPW];
  uint32_t frag_off[kMI];  // per mi: byte offset of this lane's first transposed read

  __device__ __forceinline__ void retarget(const Operand<__bf16>& op, int64_t mn0) {
    d.retarget(op.base + mn0, op.k_ext * op.ld * 2 - mn0 * 2);
  }
  __device__ __forceinline__ void step() { d.step(); }
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t mn0, int wave, int lane,
                                       int sub0) {
    init_lanes(op, wave, lane, sub0);
    retarget(op, mn0);
  }
  __device__ __forceinline__ void init_lanes(const Operand<__bf16>& op, int wave, int lane,
                                             int sub0) {
    const int64_t row_bytes = op.ld * 2;
    d.row_bytes = row_bytes;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int kr = 2 * (CPW * wave + i) + (lane >> 5);
      const int c = (lane & 31) ^ swz_mn(kr);
      voff[i] = (uint32_t)(kr * row_bytes + c * 16);
    }
    // ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
    // i % 4 of the 8-byte runs addressed by lanes i / 4 + 4 r (r = 0..3).
    // Lane jj of group g addresses k-row 8 g + jj / 4 (+ 4 for the second
    // read) and the 4 columns 4 (jj % 4) of its 16-column sub-tile, so lane i
    // of the group gets K values 8 g .. 8 g + 7 of column i, as the MFMA
    // operand expects.  swz_mn(kr + 4) == swz_mn(kr), so one offset serves
    // both reads.
    const int g = lane >> 4, jj = lane & 15;
    const int kr = 8 * g + (jj >> 2);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      const int col = sub0 + mi * kMfma + 4 * (jj & 3);
      const int c = (col >> 3) ^ swz_mn(kr);
      frag_off[mi] = (uint32_t)(kr * 512 + c * 16 + (col & 7) * 2);
    }
  }
  __device__ __forceinline__ void copy_one(uint32_t dst, int64_t kt, int wave, bool live,
                                          int i) const {
    dma16(d.rsrc(kt), dst + (CPW * wave + i) * 1024, live ? voff[i] : kOutOfRange, 0);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live) const {
#pragma unroll
    for (int i = 0; i < CPW; ++i) copy_one(dst, kt, wave, live, i);
  }
  __device__ __forceinline__ void copy_at(uint32_t dst, int64_t kt, int wave, bool live,
                                         int i) const {
    static_assert(!Step, "a stepped descriptor depends on the stages copied before");
    copy_one(dst, kt, wave, live, i);
  }
  __device__ __forceinline__ u32x4_t frag(const char* src, int mi) const {
    const char* p = src + frag_off[mi];
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p + 4 * 512));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
};

// MN-contiguous bf16 operand kept in blocks (BlockedG: k-rows are the 16-row
// bands' rows, mn runs along a band).  A stage (32 k-rows = two bands, 256 mn
// = eight block columns) is kept in LDS as the same 16 blocks of 1 KiB, block
// (column cb, band b) at (2 cb + b) KiB, so every copy moves one whole block
// (1 KiB contiguous in memory).  Inside a block, row r's 16-byte chunk c sits
// at chunk c ^ (2 (r >> 3 & 1)): a transposed fragment read takes 32 bytes of
// each of the rows {0..3, 8..11} of a band per 32 lanes (+ 4 for its second
// read), and rows r and r + 8 of one 64-byte window then land on opposite
// halves of it, which keeps the reads free of bank conflicts.  The descriptor
// follows the stages by adds (copy_one), or is computed from the stage
// (copy_at, with the side never stepped).
template <int CPW = kCopiesPerWave>
struct SideMNb16Blk {
  const char* base;  // stage's first band, at the tile's first block column
  int64_t bytes;     // from base to the operand's last band's end
  int64_t band;      // bytes between bands
  uint32_t voff[CPW];
  uint32_t frag_off[kMI];

  __device__ __forceinline__ static int chunk_swz(int r) { return ((r >> 3) & 1) << 1; }

  __device__ __forceinline__ void retarget(const Operand<__bf16>& op, int64_t mn0) {
    band = BlockedG::band_bytes(op.ld, 2);
    const int64_t col = (mn0 / 32) * BlockedG::kBlkBytes;  // mn0 is a multiple of 256
    base = reinterpret_cast<const char*>(op.base) + col;
    bytes = ((op.k_ext + 15) / 16) * band - col;
  }
  __device__ __forceinline__ void step() {
    base += 2 * band;
    bytes -= 2 * band;
  }
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t mn0, int wave, int lane,
                                       int sub0) {
    init_lanes(op, wave, lane, sub0);
    retarget(op, mn0);
  }
  __device__ __forceinline__ void init_lanes(const Operand<__bf16>& op, int wave, int lane,
                                             int sub0) {
    const int64_t bb = BlockedG::band_bytes(op.ld, 2);
    // lane l fills LDS slot l of its copy's block: row l / 4, physical chunk
    // l % 4, i.e. the block's logical chunk (l % 4) ^ chunk_swz(row)
    const int r = lane >> 2;
    const int lchunk = (lane & 3) ^ chunk_swz(r);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int bi = CPW * wave + i;  // LDS block: column bi / 2, band bi % 2
      voff[i] = (uint32_t)((bi & 1) * bb + (bi >> 1) * BlockedG::kBlkBytes +
                           r * BlockedG::kRowBytes + lchunk * 16);
    }
    // ds_read_b64_tr_b16: lane jj of group g addresses k-row 8 g + jj / 4 (and
    // + 4 for the second read) and the 4 columns 4 (jj % 4) of the sub-tile
    const int g = lane >> 4, jj = lane & 15;
    const int kr = 8 * g + (jj >> 2);
    const int rb = kr & 15, bnd = kr >> 4;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      const int col = sub0 + mi * kMfma + 4 * (jj & 3);
      const int cb = col >> 5, cc = col & 31;
      frag_off[mi] = (uint32_t)((2 * cb + bnd) * BlockedG::kBlkBytes + rb * BlockedG::kRowBytes +
                                (((cc >> 3) ^ chunk_swz(rb)) * 16) + (cc & 7) * 2);
    }
  }
  __device__ __forceinline__ void copy_one(uint32_t dst, int64_t, int wave, bool live,
                                          int i) const {
    dma16(make_rsrc(base, bytes), dst + (CPW * wave + i) * 1024, live ? voff[i] : kOutOfRange,
          0);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live) const {
#pragma unroll
    for (int i = 0; i < CPW; ++i) copy_one(dst, kt, wave, live, i);
  }
  // Stage kt (two bands) of the tile, from its first stage.
  __device__ __forceinline__ void copy_at(uint32_t dst, int64_t kt, int wave, bool live,
                                         int i) const {
    const int64_t o = kt * 2 * band;
    dma16(make_rsrc(base + o, bytes - o), dst + (CPW * wave + i) * 1024,
          live ? voff[i] : kOutOfRange, 0);
  }
  // The second read is 4 k-rows further: 4 block rows, the same swizzle.
  __device__ __forceinline__ u32x4_t frag(const char* src, int mi) const {
    const char* p = src + frag_off[mi];
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p + 4 * BlockedG::kRowBytes));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
};

// MN-contiguous f32 operand: a stage is kStageRowBytes / 4 k-rows of 256
// floats (1 KiB), one k-row per copy, no swizzle; fragments are read one float
// at a time.
template <bool Step>
struct SideMNf32 {
  MNDesc<Step, 4> d;
  uint32_t voff[kCopiesPerWave];
  uint32_t frag_off;

  __device__ __forceinline__ void retarget(const Operand<float>& op, int64_t mn0) {
    d.retarget(op.base + mn0, op.k_ext * op.ld * 4 - mn0 * 4);
  }
  __device__ __forceinline__ void step() { d.step(); }
  __device__ __forceinline__ void init(const Operand<float>& op, int64_t mn0, int wave, int lane,
                                       int sub0) {
    init_lanes(op, wave, lane, sub0);
    retarget(op, mn0);
  }
  __device__ __forceinline__ void init_lanes(const Operand<float>& op, int wave, int lane,
                                             int sub0) {
    const int64_t row_bytes = op.ld * 4;
    d.row_bytes = row_bytes;
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) {
      const int kr = kCopiesPerWave * wave + i;
      voff[i] = (uint32_t)(kr * row_bytes + lane * 16);
    }
    // column lane % 16 of the sub-tile, k-rows 4 (lane / 16) .. + 4
    frag_off = (uint32_t)((sub0 + (lane & 15)) * 4 + (lane >> 4) * 4 * 1024);
  }
  __device__ __forceinline__ void copy_one(uint32_t dst, int64_t kt, int wave, bool live,
                                          int i) const {
    dma16(d.rsrc(kt), dst + (kCopiesPerWave * wave + i) * 1024, live ? voff[i] : kOutOfRange, 0);
  }
  __device__ __forceinline__ void copy(uint32_t dst, int64_t kt, int wave, bool live) const {
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) copy_one(dst, kt, wave, live, i);
  }
  // Lane group h (= lane / 16) takes k-rows 4 h + q, q = 0..3.
  __device__ __forceinline__ u32x4_t frag(const char* src, int mi) const {
    const char* p = src + frag_off + mi * kMfma * 4;
    u32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint32_t*>(p + q * 1024);
    return v;
  }
};

template <> struct Side<__bf16, kMN> : SideMNb16<false> {};
template <> struct Side<__bf16, kMNStep> : SideMNb16<true> {};
template <> struct Side<float, kMN> : SideMNf32<false> {};
template <> struct Side<float, kMNStep> : SideMNf32<true> {};
template <> struct Side<__bf16, kMNBlkStep> : SideMNb16Blk<> {};

// ---------------------------------------------------------------------------
// MFMA on one 16-byte fragment pair.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

// A and B use the same K assignment (lane group h = lane / 16 holds K
// elements 8 h .. 8 h + 7 of a bf16 stage), so every product pairs equal K.
template <>
struct Mfma<__bf16> {
  __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  // Float q of lane group h's fragment is K element 4 h + q of the stage;
  // MFMA q of the four takes those (one K value per lane group), for A and B
  // alike.  Each element is copied to a scalar before the bit cast: a bit
  // cast of a vector-element lvalue reads element 0 whatever the index.
  __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ua = a[q];
      const uint32_t ub = b[q];
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ua),
                                               __builtin_bit_cast(float, ub), c, 0, 0, 0);
    }
    return c;
  }
};

// Accumulators of one wave: kMI x kNI MFMA tiles of 16 x 16.
// Element (mi, ni, e) of lane l sits at tile row
//   wm*kWaveM + mi*16 + (l/16)*4 + e   and column  wn*kWaveN + ni*16 + l%16.
struct Acc {
  static constexpr int MI = kMI, NI = kNI, WaveM = kWaveM, WaveN = kWaveN;
  f32x4_t c[kMI][kNI];
  __device__ __forceinline__ static float read(const f32x4_t& v, int e) { return v[e]; }
};

__device__ __forceinline__ int acc_row(int mi, int e, int lane) {
  return mi * kMfma + (lane >> 4) * 4 + e;
}

// Fragments of one stage: a[mi] for the kMI sub-tiles of A, b[ni] for the kNI
// of B.  A stage's MFMAs run in two halves (sub-tiles mi < kMI / 2, then the
// rest), so each register is refilled from the next stage as soon as its
// last MFMA of this stage has issued.
template <typename T, int AK, int BK>
struct Frags {
  u32x4_t a[kMI], b[kNI];
  // What the first half of a stage needs: a[0 .. kMI / 2) and all of b.
  __device__ __forceinline__ void read_first(const Side<T, AK>& sa, const Side<T, BK>& sb,
                                             const char* stage) {
#pragma unroll
    for (int i = 0; i < kMI / 2; ++i) a[i] = sa.frag(stage, i);
#pragma unroll
    for (int i = 0; i < kNI; ++i) b[i] = sb.frag(stage + kOperandBytes, i);
  }
};

// Wait until at most N of this wave's copies are still in flight and its own
// LDS reads are done (vmcnt(N) lgkmcnt(0), gfx9 encoding).  Copies complete in
// issue order.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// x, hidden from the optimiser: values computed from it are recomputed where
// they are written instead of being hoisted and kept live.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Keeps the instruction scheduler from moving anything across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------
// Tile order and the persistent tile loop.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;  // blocks are dispatched to the 8 XCDs round-robin

// Tiles of an M x N output, ordered in groups of group_m M-tiles: within a
// group N advances after every group_m tiles, so that consecutive tiles share
// operand rows.  Groups are dealt out in bands of kXcds groups, one group of a
// band to each XCD (block b runs on XCD b % 8): the XCDs then walk N in step,
// so an operand panel along N that one XCD reads is read by the others at
// about the same time and comes from the shared MALL rather than HBM again.
// (Without bands, an output many groups tall puts each XCD on its own stretch
// of N.)  The M-tiles past the last full band form one partial band, whose
// group order is split into kXcds contiguous ranges, one per XCD.  Either way
// the tiles resident on one XCD at the same time are neighbours and share its
// L2.  Block `block` of the `blocks` that work on this output takes the tiles
// of virtual blocks block, block + G, block + 2G, ... (G = blocks; G is the
// tile count or a multiple of 8, and the first block of the output sits at a
// multiple of 8 in the grid, so that every virtual block maps to the XCD of
// its block).  Virtual block v is the (v / 8)-th tile of XCD v % 8; each XCD
// has total / 8 tiles, one more for the first total % 8, which is exactly its
// share of [0, total), so the order is a bijection.
struct TileGrid {
  int64_t m_tiles, n_tiles, group_m;
  int64_t block, blocks;
  bool bands;  // deal groups out in bands; false: the whole order is one partial band

  __host__ __device__ __forceinline__ int64_t total() const { return m_tiles * n_tiles; }
  // Tiles taken by this block (zero if it is past the last tile).
  __host__ __device__ __forceinline__ int64_t count() const {
    return (total() - block + blocks - 1) / blocks;
  }
  // First row and column of this block's i-th tile.
  __host__ __device__ __forceinline__ void coords(int64_t i, int64_t* m0, int64_t* n0) const {
    const int64_t b = block + i * blocks;
    const int64_t x = b % kXcds, j = b / kXcds;
    const int64_t band_m = kXcds * group_m;
    const int64_t full = bands ? m_tiles / band_m : 0;  // full bands
    const int64_t per_xcd = group_m * n_tiles;    // one group: an XCD's share of a band
    int64_t m, n;
    if (j < full * per_xcd) {
      const int64_t band = j / per_xcd, local = j - band * per_xcd;
      m = band * band_m + x * group_m + local % group_m;
      n = local / group_m;
    } else {
      const int64_t m_base = full * band_m, rem = m_tiles - m_base;
      const int64_t tot = rem * n_tiles, q = tot / kXcds, r = tot % kXcds;
      const int64_t t = x * q + (x < r ? x : r) + (j - full * per_xcd);
      const int64_t g = t / per_xcd;
      const int64_t first_m = g * group_m;
      const int64_t gm = rem - first_m < group_m ? rem - first_m : group_m;
      const int64_t local = t - g * per_xcd;
      m = m_base + first_m + local % gm;
      n = local / gm;
    }
    *m0 = m * kTile;
    *n0 = n * kTile;
  }
};

// Copies of one operand for a stream of stages that runs across this block's
// tiles: the stage `kt` of tile `ti`, in ring buffer `buf`.
template <typename T, int KC>
struct Cursor {
  Side<T, KC> side;
  int64_t kt, ti;
  uint32_t buf;
  // Copy i of the current stage (the operand's half of the ring buffer at off).
  __device__ __forceinline__ void copy_one(uint32_t lds0, uint32_t off, int wave, int64_t tiles,
                                           int i) const {
    side.copy_one(lds0 + buf * kStageBytes + off, kt, wave, ti < tiles, i);
  }
  __device__ __forceinline__ void copy(uint32_t lds0, uint32_t off, int wave, int64_t tiles) const {
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) copy_one(lds0, off, wave, tiles, i);
  }
  // On to the next stage; the stream enters the next tile (first row next_mn0)
  // after the last stage of a tile.
  __device__ __forceinline__ void advance(const Operand<T>& op, int64_t nk, int64_t next_mn0) {
    buf = buf + 1 == kStages ? 0u : buf + 1;
    if (++kt == nk) {
      kt = 0;
      ++ti;
      side.retarget(op, next_mn0);
    } else {
      side.step();
    }
  }
};

// Half H of a stage: the MFMAs of sub-tiles mi in [H kMI / 2, (H + 1) kMI / 2)
// for every ni, ni-major (so b[ni] sees its last MFMA of the stage early in
// the second half), with the fragment reads that refill registers:
//   H = 0: a[kMI / 2 ..) of this stage (src = this stage);
//   H = 1: a[0 .. kMI / 2) and each b[ni], right after its last use, of the
//          next stage (src = next stage);
// and, with Copy, the kCopiesPerWave copies of one operand's current stage,
// one after MFMAs 0 and 4, or 0 and 8 where both operands are MN-contiguous
// (each measured fastest for its kernels among the placements tried).  Spreading the
// copies keeps the MFMA pipe fed while the texture unit works through them;
// issued in a burst, they would hold every wave of the CU at once.
template <int H, bool Reads, bool Copy, typename T, int AK, int BK, typename C>
__device__ __forceinline__ void half_stage(const Side<T, AK>& sa, const Side<T, BK>& sb,
                                           Frags<T, AK, BK>& f, const char* src, const C& cur,
                                           uint32_t lds0, uint32_t off, int wave, int64_t tiles,
                                           Acc& acc) {
  constexpr int kHalf = kMI / 2;  // sub-tiles along M per half
  constexpr int kMfmas = kHalf * kNI;
  // MFMAs between copies: front-loaded (every 4th) unless both operands are
  // MN-contiguous (spread over the whole half stage)
  constexpr int kCopyGap = is_mn(AK) && is_mn(BK) ? kMfmas / kCopiesPerWave : 4;
  static_assert(kHalf == 4 && kCopyGap * kCopiesPerWave <= kMfmas, "copies fit in a half stage");
#pragma unroll
  for (int t = 0; t < kHalf * kNI; ++t) {
    const int ni = t / kHalf, mi = H * kHalf + t % kHalf;
    acc.c[mi][ni] = Mfma<T>::run(f.a[mi], f.b[ni], acc.c[mi][ni]);
    if constexpr (Reads) {
      if constexpr (H == 0) {
        if (t < kHalf) f.a[kHalf + t] = sa.frag(src, kHalf + t);
      } else {
        if (t % kHalf == kHalf - 1) f.b[ni] = sb.frag(src + kOperandBytes, ni);
        else if (t < 5) f.a[t < 3 ? t : t - 1] = sa.frag(src, t < 3 ? t : t - 1);
      }
    }
    if constexpr (Copy) {
      if (t % kCopyGap == 0 && t / kCopyGap < kCopiesPerWave)
        cur.copy_one(lds0, off, wave, tiles, t / kCopyGap);
    }
    // The order above is pinned where an operand is read with transposing
    // reads (measured faster); with both operands K-contiguous the compiler's
    // own interleaving, with two waves per SIMD, measured faster still.
    if constexpr (is_mn(AK) || is_mn(BK)) sched_fence();
  }
}

// Every tile of this block: C[m0:m0+256, n0:n0+256] = sum_k A[m, k] B[n, k]
// over k in [0, k_len), then epi(acc, m0, n0, staging) with the tile in acc
// and kStagingBytes of LDS after the ring free for the epilogue.
//
// All tiles of the block form one stream of stages (a tile is nk stages of
// one MFMA K step; stage s lives in ring buffer s % kStages).  The copies run
// ahead of the MFMAs by the depth of the ring, across tile boundaries, so the
// first stages of the next tile land while a tile's epilogue runs.  With the
// MFMAs at stage s:
//   half A: MFMAs of sub-tiles mi < kMI / 2, reads of the other a[] of stage
//           s (its last reads), B copies of stage s + kStages - 1 (into the
//           buffer freed at the previous barrier);
//   wait until stage s + 1 has landed and this wave's reads are done; barrier
//           (every wave is past its last read of buffer s % kStages);
//   half B: MFMAs of sub-tiles mi >= kMI / 2, reads of a[0 .. kMI / 2) and b[]
//           of stage s + 1, A copies of stage s + kStages (into buffer
//           s % kStages).
// Every stage issues one stage of copies, so the waits are constants; past the
// block's last stage the copies are dead (they read zeros into buffers that
// are not read again).  The last stage of a tile is peeled off, so the loop
// body has no branch.  A cursor enters the next tile while the MFMAs are
// still in this one if nk > kStages; with fewer stages per tile, launch one
// tile per block (the copies past it are dead).
//
// The epilogue's stores (and loads) share vmcnt with the copies.  A counted
// wait vmcnt(n), n = copies issued after the awaited ones, is safe: loads
// complete in issue order among themselves, so while an awaited copy is
// outstanding so is every later copy, and the count cannot drop to n.  Any
// other operation in flight (a store, an uncounted load) only makes the wait
// stricter: stores may complete out of order with respect to loads, so they
// cannot be counted in n.  The first wait after an epilogue (half a stage
// into the next tile) therefore also waits for the epilogue's stores to be
// acknowledged.
// ABlk: A is a bf16 gradient strip kept in blocks (BlockedG).
template <typename T, bool AK, bool BK, bool ABlk = false, typename Epi>
__device__ __forceinline__ void run_tiles(const Operand<T>& A, const Operand<T>& B, int64_t k_len,
                                          const TileGrid& grid, char* lds, Epi&& epi) {
  constexpr int64_t kStageK = kStageRowBytes / sizeof(T);
  constexpr int kPerStage = 2 * kCopiesPerWave;  // copies per wave per stage
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const uint32_t lds0 = lds_addr(lds);
  char* const staging = lds + kRingBytes;
  const int64_t nk = (k_len + kStageK - 1) / kStageK;
  const int64_t tiles = grid.count();
  if (tiles == 0) return;  // more blocks than tiles for this output

  int64_t m0, n0, next_m0, next_n0;  // this tile, and the next one
  grid.coords(0, &m0, &n0);
  next_m0 = m0;
  next_n0 = n0;
  if (tiles > 1) grid.coords(1, &next_m0, &next_n0);

  // K-contiguous operands take the split placement when both are (strip
  // kernels), the row-major one beside a transposed operand.
  // MN-contiguous descriptors follow by adds where both operands are (dW).
  // A gradient strip in blocks (ABlk) takes the split placement (conflict-free
  // fragment reads) when K-contiguous, the blocked transposed stage otherwise;
  // with blocks, a split copy still reads two 512-byte runs, and measured
  // faster than the row-major placement beside dH's transposed W (0.6% per
  // step, same box).
  constexpr int LA0 = !AK ? (BK ? kMN : kMNStep) : (BK ? kKSplit : kKRow);
  constexpr int LA = !ABlk ? LA0 : (AK ? kKSplitBlk : kMNBlkStep);
  constexpr int LB = !BK ? (AK ? kMN : kMNStep) : (AK ? kKSplit : kKRow);
  Cursor<T, LA> ca{{}, 0, 0, 0u};
  Cursor<T, LB> cb{{}, 0, 0, 0u};
  ca.side.init(A, m0, wave, lane, wm * kWaveM);
  cb.side.init(B, n0, wave, lane, wn * kWaveN);
  const Side<T, LA>& sa = ca.side;  // fragment offsets do not depend on the tile
  const Side<T, LB>& sb = cb.side;

  // Stages 0 .. kStages - 2 whole, and the A copies of stage kStages - 1.
#pragma unroll
  for (int s = 0; s + 1 < kStages; ++s) {
    ca.copy(lds0, 0, wave, tiles);
    ca.advance(A, nk, next_m0);
    cb.copy(lds0, kOperandBytes, wave, tiles);
    cb.advance(B, nk, next_n0);
  }
  ca.copy(lds0, 0, wave, tiles);
  ca.advance(A, nk, next_m0);
  wait_copies<(kStages - 2) * kPerStage + kCopiesPerWave>();
  block_barrier();

  Acc acc;
  Frags<T, LA, LB> f;
  uint32_t buf = 0;  // ring buffer of the stage the MFMAs are at
  for (int64_t i = 0; i < tiles; ++i) {
    {
      // per-lane offsets again, so that none of them is live across an epilogue
      const int l = opaque(lane);
      ca.side.init_lanes(A, wave, l, wm * kWaveM);
      cb.side.init_lanes(B, wave, l, wn * kWaveN);
    }
#pragma unroll
    for (int r = 0; r < kMI; ++r)
#pragma unroll
      for (int c = 0; c < kNI; ++c) acc.c[r][c] = f32x4_t{};
    f.read_first(sa, sb, lds + buf * kStageBytes);
    sched_fence();
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
      const uint32_t next = buf + 1 == kStages ? 0u : buf + 1;
      half_stage<0, true, true>(sa, sb, f, lds + buf * kStageBytes, cb, lds0, kOperandBytes,
                                wave, tiles, acc);
      cb.advance(B, nk, next_n0);
      wait_copies<(kStages - 2) * kPerStage>();
      block_barrier();
      half_stage<1, true, true>(sa, sb, f, lds + next * kStageBytes, ca, lds0, 0, wave, tiles,
                                acc);
      ca.advance(A, nk, next_m0);
      buf = next;
    }
    {
      const uint32_t next = buf + 1 == kStages ? 0u : buf + 1;
      half_stage<0, true, true>(sa, sb, f, lds + buf * kStageBytes, cb, lds0, kOperandBytes,
                                wave, tiles, acc);
      cb.advance(B, nk, next_n0);
      wait_copies<(kStages - 2) * kPerStage>();
      block_barrier();
      half_stage<1, false, true>(sa, sb, f, lds, ca, lds0, 0, wave, tiles, acc);
      ca.advance(A, nk, next_m0);
      buf = next;
    }
    epi(acc, m0, n0, staging);
    m0 = next_m0;
    n0 = next_n0;
    if (i + 2 < tiles) grid.coords(i + 2, &next_m0, &next_n0);
  }
  wait_copies<0>();  // no copy may still be writing LDS when the block exits
}

}  // namespace lce
