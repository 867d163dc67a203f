// lce_kernels.hip - gfx950 kernels of the strip-wise linear cross-entropy.
//
// Forward, per vocabulary strip W_s = W[v0 : v0 + v_len]:
//   strip_lse   Z^T = W_s . h^T on MFMA; the epilogue reduces each token's
//               column of the 256 x 256 tile to a partial (max, sum of exp)
//               per 128 vocabulary rows and captures the target logit.  The
//               logits never leave registers.
//   fold        merges the partials of the strip into the running per-token
//               (max, sum) - the state fold of Ring-DTP (second page, 3.2).
// and once per pass: state_init before the first strip, finalize after the
// last (lse = max + log(sum), row loss = lse - target logit, reduction).
//
// Backward, per strip: strip_grad recomputes Z^T and writes
// G = scale * (softmax - onehot) as the input element type into the strip
// buffer [N, ldG] (bf16: in blocks of 16 tokens); gemm_dh forms
// dH (+)= G . W_s and gemm_dw forms dW_s = G^T . h, both accumulating in
// fp32 (one shared launch where that is shorter).
//
// The bf16 GEMMs with at least 16 K stages of 64 run on the one-wave-per-SIMD
// engine (tile_engine_w4.h), the rest on the eight-wave engine
// (tile_engine.h).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "lce_kernels.h"
#include "tile_engine.h"
#include "tile_engine_w4.h"

namespace lce {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 gradient strips are kept in blocks (BlockedG); f32 ones row-major
// [N, ldg].
template <typename T> constexpr bool kGBlocked = false;
template <> constexpr bool kGBlocked<__bf16> = true;

// ---------------------------------------------------------------------------
// Forward strip: MFMA M = vocabulary rows of the strip, N = tokens, K = H.
// ---------------------------------------------------------------------------
// The combination of x over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (one
// token's four row groups), in every lane, by row swaps on the VALU: after
// v_permlane16_swap of two copies of x, lane by lane one copy holds x of the
// even and the other x of the odd row of a row pair, and after
// v_permlane32_swap x of the lower and of the upper half, so op of the two is
// the xor-16 and then the xor-32 combination (the same operands, in either
// order, as exchanges through ds_bpermute, without their LDS round trips).
// The swap's results are copied to scalars before the bit casts:
// __builtin_bit_cast of an element of the returned vector read element 0
// for either index.
__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }

template <typename Op>
__device__ __forceinline__ float combine_row_groups(float x, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t p0 = p[0], p1 = p[1];
  x = op(as_float(p0), as_float(p1));
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t q0 = q[0], q1 = q[1];
  return op(as_float(q0), as_float(q1));
}

// The token of column block ni of a tile that this lane's values belong to.
template <typename AccT>
__device__ __forceinline__ int64_t lse_token(int64_t n0, int ni) {
  const int tid = (int)threadIdx.x;
  return n0 + (__builtin_amdgcn_readfirstlane(tid >> 6) >> 1) * AccT::WaveN + ni * kMfma + (tid & 15);
}

// The targets of this lane's tokens of a tile, read at the token clamped to
// N - 1 (the caller drops tokens past N): an unconditional load goes straight
// to its register, where a guarded one was followed by a select that waited
// for it.
template <typename T, typename AccT>
__device__ __forceinline__ void lse_targets(const StripArgs<T>& a, int64_t n0,
                                            int32_t (&tgt)[AccT::NI]) {
#pragma unroll
  for (int ni = 0; ni < AccT::NI; ++ni) {
    const int64_t tok = lse_token<AccT>(n0, ni);
    tgt[ni] = a.targets[tok < a.N ? tok : a.N - 1];
  }
}

// Per token of the tile and per 128 strip rows of a wave: (max, sum of
// exp(z - max)) to partials, and the target logit to z_target.  A token's
// 128 rows of a wave sit in the four lanes l % 16 + 16 h (h = 0..3), 32
// values each.  tgt: the tokens' targets, loaded before the tile's stages
// (pre), or null to load them here, all before the first use.
template <typename T, typename AccT>
__device__ __forceinline__ void lse_epilogue(const StripArgs<T>& a, AccT& acc, int64_t m0,
                                             int64_t n0, const int32_t* pre_tgt = nullptr) {
  constexpr int kMI = AccT::MI, kNI = AccT::NI, kWaveM = AccT::WaveM;
  // lane values recomputed per tile rather than hoisted and kept live
  const int tid = opaque((int)threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1;
  const int64_t vrow0 = m0 + wm * kWaveM;             // first strip row of this wave
  const int64_t rows_left = a.v_len - vrow0;
  if (rows_left <= 0) return;                          // wave-uniform
  const int nrows = rows_left < kWaveM ? (int)rows_left : kWaveM;
  const bool full = nrows == kWaveM;
  const int64_t blk = vrow0 / kWaveM;
  const int r_lane = (lane >> 4) * 4;  // acc_row(mi, e, lane) - acc_row(mi, e, 0)

  int32_t tgt[kNI];
  if (pre_tgt) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) tgt[ni] = pre_tgt[ni];
  } else {
    lse_targets<T, AccT>(a, n0, tgt);
  }

  // One 16-token column block (ni) at a time, so that only its 32 values per
  // lane are held in VGPRs.
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t tok = lse_token<AccT>(n0, ni);
    float v[4 * kMI];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[mi * 4 + e] = AccT::read(acc.c[mi][ni], e);
    if (!full) {
      // rows past the strip's end: -inf adds nothing to the max or the sum
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[mi * 4 + e] = r_lane >= nrows - acc_row(mi, e, 0) ? -INFINITY : v[mi * 4 + e];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4 * kMI; ++q) mx = fmaxf(mx, v[q]);
    mx = combine_row_groups(mx, [](float x, float y) { return fmaxf(x, y); });
    const float mscaled = mx * kLog2e;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 4 * kMI; ++q) sum += fast_exp2(__builtin_fmaf(v[q], kLog2e, -mscaled));
    sum = combine_row_groups(sum, [](float x, float y) { return x + y; });

    // Target logit: at most one (row, token) pair of the whole strip matches.
    const int32_t t = tok < a.N ? tgt[ni] : a.ignore_index;
    const int64_t local = (int64_t)t - (a.v_begin + vrow0);
    const bool hit = t != a.ignore_index && local >= 0 && local < nrows;
    if (__any(hit)) {
      const int d = hit ? (int)local - r_lane : -1;  // acc_row(mi, e, 0) of the target, if here
      float zt = 0.f;
      bool mine = false;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool eq = d == acc_row(mi, e, 0);
          zt = eq ? v[mi * 4 + e] : zt;
          mine = mine || eq;
        }
      if (mine) a.z_target[tok] = zt;
    }
    if (lane < 16 && tok < a.N) a.partials[blk * a.N + tok] = float2{mx, sum};
    sched_fence();
  }
}

// The forward strip on the one-wave-per-SIMD engine (bf16).
__global__ __launch_bounds__(w4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void strip_lse_kernel_w4(StripArgs<__bf16> a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<__bf16> A{a.weight_strip, a.H, a.v_len, a.H};
  const Operand<__bf16> B{a.hidden, a.H, a.N, a.H};
  const TileGrid grid{a.m_tiles, a.n_tiles, a.group_m, blockIdx.x, gridDim.x, true};
  int32_t tgt[w4::kNI];  // loaded at a tile's start, used by its epilogue
  w4::run_tiles<w4::KRow128, w4::KRow128>(
      A, B, a.H, grid, lds,
      [&](int64_t, int64_t n0) { lse_targets<__bf16, w4::Acc>(a, n0, tgt); },
      [&](w4::Acc& acc, int64_t m0, int64_t n0, char*) { lse_epilogue(a, acc, m0, n0, tgt); });
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void strip_lse_kernel(StripArgs<T> a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<T> A{a.weight_strip, a.H, a.v_len, a.H};
  const Operand<T> B{a.hidden, a.H, a.N, a.H};
  const TileGrid grid{a.m_tiles, a.n_tiles, a.group_m, blockIdx.x, gridDim.x, true};
  run_tiles<T, true, true>(A, B, a.H, grid, lds,
                           [&](Acc& acc, int64_t m0, int64_t n0, char*) {
                             lse_epilogue(a, acc, m0, n0);
                           });
}

// ---------------------------------------------------------------------------
// Backward strip: same tile, epilogue writes G[tok, v] = scale*(p - onehot).
// ---------------------------------------------------------------------------
// Four consecutive gradient values of one token row, packed in the strip's
// element type (8 bytes of bf16, rounded to nearest even, or 16 bytes of f32).
template <typename T> struct GPack;
template <> struct GPack<__bf16> {
  typedef u32x2_t type;
  __device__ __forceinline__ static type pack(float a, float b, float c, float d) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t lo{(__bf16)a, (__bf16)b};
    const bf16x2_t hi{(__bf16)c, (__bf16)d};
    return type{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  }
};
template <> struct GPack<float> {
  typedef u32x4_t type;
  __device__ __forceinline__ static type pack(float a, float b, float c, float d) {
    return type{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  }
};

// f32 gradient strips leave through LDS in passes of kTok tokens: the waves
// holding those tokens write their G values as token rows, then every thread
// stores whole 16-byte runs of a row, so a wave writes 1024 contiguous bytes
// of G per instruction.  (bf16 strips use the packed path below.)
template <typename T> struct GradStage {
  static constexpr int kTok = 32;                               // tokens per pass
  static constexpr int kRowBytes = kTile * (int)sizeof(T);      // 256 vocabulary columns
  static constexpr int kStride = kRowBytes + 16;                // padded LDS row
  static constexpr int kRunsPerRow = kRowBytes / 16;
  static constexpr int kRowsPerSweep = kThreads / kRunsPerRow;
  static constexpr int kSweeps = kTok / kRowsPerSweep;
  static_assert(kTok * kStride <= kStagingBytes, "staging fits in LDS");
};

// Where a tile's G goes: the element (token n0, vocabulary row m0) of the tile
// at `tile`, rows `ld` elements apart, `bytes` valid bytes from there (rows
// past them are dropped by the buffer's range check).
template <typename T>
struct GradDst {
  T* tile;
  int64_t ld;
  int64_t bytes;
};

// The tile's place in the strip buffer G [N, ldg].
template <typename T>
__device__ __forceinline__ GradDst<T> strip_dst(const StripArgs<T>& a, int64_t m0, int64_t n0) {
  return GradDst<T>{a.g_strip + n0 * a.ldg + m0, a.ldg,
                    (a.N - n0) * a.ldg * (int64_t)sizeof(T) - m0 * (int64_t)sizeof(T)};
}

template <typename T>
__device__ __forceinline__ void grad_epilogue(const StripArgs<T>& a, Acc& acc, int64_t m0,
                                              int64_t n0, char* lds, const GradDst<T>& dst) {
  typedef GradStage<T> S;
  const int tid = opaque((int)threadIdx.x);  // recomputed per tile, not kept live
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t vrow0 = m0 + wm * kWaveM;
  const bool full = vrow0 + kWaveM <= a.v_len;  // no strip rows past v_len in this wave
  const float scale_all = a.ctrl->grad_scale;
  // G rows of the tile: byte offset (tok - n0) * ld * elt + (col - m0) * elt;
  // rows past the destination's valid bytes are out of range.
  const int64_t row_bytes = dst.ld * (int64_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t gbuf = make_buffer(dst.tile, dst.bytes);
  static_assert(S::kTok <= kWaveN && kWaveN % S::kTok == 0, "a pass lies in one wave column");
  constexpr int kNiPerPass = S::kTok / kMfma;

  // G for every element, in place (all waves at once).
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t tok = n0 + wn * kWaveN + ni * kMfma + (lane & 15);
    const bool tok_ok = tok < a.N;
    const int32_t t = tok_ok ? a.targets[tok] : a.ignore_index;
    const float sc = t != a.ignore_index ? scale_all : 0.f;
    const float lse2 = (tok_ok ? a.lse[tok] : 0.f) * kLog2e;
    const int64_t tl64 = (int64_t)t - (a.v_begin + vrow0);  // target row in this wave
    const bool hit = t != a.ignore_index && tl64 >= 0 && tl64 < kWaveM;
    const int tl = hit ? (int)tl64 : -1;
    const bool any_hit = __any(hit);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = acc_row(mi, e, lane);
        float g = sc * fast_exp2(__builtin_fmaf(acc.c[mi][ni][e], kLog2e, -lse2));
        if (!full) g = (vrow0 + r < a.v_len) ? g : 0.f;
        if (any_hit) g = (r == tl) ? g - sc : g;
        acc.c[mi][ni][e] = g;
      }
  }

#pragma unroll
  for (int pass = 0; pass < kTile / S::kTok; ++pass) {
    block_barrier();  // staging free: the previous pass (or tile) is done with it
    const int tok_base = pass * S::kTok;  // first token of the pass within the tile
    if (wn == tok_base / kWaveN) {
#pragma unroll
      for (int nj = 0; nj < kNiPerPass; ++nj) {
        const int ni = (tok_base % kWaveN) / kMfma + nj;
        const int tok_local = wn * kWaveN + ni * kMfma + (lane & 15);
        char* lrow = lds + (tok_local - tok_base) * S::kStride +
                     (wm * kWaveM + (lane >> 4) * 4) * (int)sizeof(T);
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi) {
          const f32x4_t& c = acc.c[mi][ni];
          *reinterpret_cast<typename GPack<T>::type*>(lrow + mi * kMfma * (int)sizeof(T)) =
              GPack<T>::pack(c[0], c[1], c[2], c[3]);
        }
      }
    }
    block_barrier();
    const int run = tid % S::kRunsPerRow;
#pragma unroll
    for (int i = 0; i < S::kSweeps; ++i) {
      const int row = tid / S::kRunsPerRow + S::kRowsPerSweep * i;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + row * S::kStride + run * 16);
      const uint32_t off = (uint32_t)((tok_base + row) * row_bytes) + run * 16;
      __builtin_amdgcn_raw_buffer_store_b128(v, gbuf, off, 0, 0);
    }
  }
}

// bf16 strips: G leaves in two passes through the 64 KiB staging area, pass
// p holding the MFMA column blocks ni = 2 p, 2 p + 1 of every wave: 32 tokens
// per wave column, (kWaves / 2) x 32 = 128 tokens, as 128 rows of 512 bytes
// whose 16-byte chunks are XOR-swizzled by the row, so that neither the
// MFMA-layout writes nor the row reads pile onto a few banks.  Every wave
// computes its part of a pass straight into staging (per element one FMA,
// one exp2 and half a pack: the token's |scale| is folded into the exponent,
// its sign applied to the packed bits), so the accumulators of a column block
// die in its pass and no packed copy of G is held: the kernel stays within
// its registers.  (A spill would bring scratch loads, and their waits drain
// every copy and store in flight.)  Targets and lse are loaded before any
// store, so waiting for them never waits for this tile's stores.
__device__ __forceinline__ void grad_epilogue(const StripArgs<__bf16>& a, Acc& acc, int64_t m0,
                                              int64_t n0, char* lds, const GradDst<__bf16>& dst) {
  constexpr int kRowBytes = kTile * 2;        // 256 bf16 vocabulary columns
  constexpr int kNiPass = 2;                  // column blocks per wave per pass
  constexpr int kPassTok = kWaves / 2 * kNiPass * kMfma;  // 128 tokens per pass
  static_assert(kPassTok * kRowBytes <= kStagingBytes, "staging fits in LDS");
  static_assert(kNI % kNiPass == 0, "whole passes");
  const int tid = opaque((int)threadIdx.x);  // recomputed per tile, not kept live
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t vrow0 = m0 + wm * kWaveM;
  const bool full = vrow0 + kWaveM <= a.v_len;  // no strip rows past v_len in this wave
  // strip rows of this wave below v_len (only used when !full, then < kWaveM)
  const int rows_left = full ? kWaveM : (int)max<int64_t>(a.v_len - vrow0, 0);
  const int r_lane = (lane >> 4) * 4;  // acc_row(mi, e, lane) - acc_row(mi, e, 0)
  const float scale_all = a.ctrl->grad_scale;
  const float abs_scale = fabsf(scale_all);
  const uint32_t sign = scale_all < 0.f ? 0x80008000u : 0u;
  const float log2_scale = __builtin_amdgcn_logf(abs_scale);  // -inf for a zero scale

  float c[kNI];   // |scale| * exp(z - lse) = exp2(z log2e + c); an ignored token gets c = -inf
  int tl[kNI];    // target row in this wave, or -1
  bool any_hit[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t tok = n0 + wn * kWaveN + ni * kMfma + (lane & 15);
    const bool tok_ok = tok < a.N;
    const int32_t t = tok_ok ? a.targets[tok] : a.ignore_index;
    const bool valid = t != a.ignore_index;
    const float lse2 = (tok_ok ? a.lse[tok] : 0.f) * kLog2e;
    c[ni] = valid ? log2_scale - lse2 : -INFINITY;
    const int64_t tl64 = (int64_t)t - (a.v_begin + vrow0);
    const bool hit = valid && tl64 >= 0 && tl64 < kWaveM;
    tl[ni] = hit ? (int)tl64 : -1;
    any_hit[ni] = __any(hit);
  }

  // G rows of the tile: byte offset (tok - n0) * ld * 2 + (col - m0) * 2;
  // rows past the destination's valid bytes are out of range.
  const int64_t row_bytes = dst.ld * 2;
  const __amdgpu_buffer_rsrc_t gbuf = make_buffer(dst.tile, dst.bytes);
#pragma unroll
  for (int pass = 0; pass < kNI / kNiPass; ++pass) {
    block_barrier();  // staging free: the previous pass (or tile) is done with it
#pragma unroll
    for (int nj = 0; nj < kNiPass; ++nj) {
      const int ni = pass * kNiPass + nj;
      float v[4 * kMI];
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[mi * 4 + e] = fast_exp2(__builtin_fmaf(acc.c[mi][ni][e], kLog2e, c[ni]));
      // Row tests against the lane's row offset: acc_row(mi, e, lane) =
      // acc_row(mi, e, 0) + r_lane, so each compares one VGPR with a constant.
      if (!full) {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[mi * 4 + e] = r_lane < rows_left - acc_row(mi, e, 0) ? v[mi * 4 + e] : 0.f;
      }
      if (any_hit[ni]) {
        const int d = tl[ni] - r_lane;  // the target's row minus the lane's offset
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[mi * 4 + e] = d == acc_row(mi, e, 0) ? v[mi * 4 + e] - abs_scale : v[mi * 4 + e];
      }
      // staging row of this lane's token: wave column wn, block nj, lane % 16
      const int row = wn * kNiPass * kMfma + nj * kMfma + (lane & 15);
      // its 4 rows acc_row(mi, 0..3, lane) are columns wm*128 + mi*16 + r_lane:
      // byte 2 (...) = 16-byte chunk wm*16 + 2 mi + (lane >> 5), half (lane >> 4) & 1
      char* lrow = lds + row * kRowBytes + ((lane >> 4) & 1) * 8;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi) {
        const float* w = &v[mi * 4];
        const u32x2_t pk = GPack<__bf16>::pack(w[0], w[1], w[2], w[3]);
        const int chunk = wm * 16 + mi * 2 + (lane >> 5);
        *reinterpret_cast<u32x2_t*>(lrow + ((chunk ^ (row & 31)) * 16)) =
            u32x2_t{pk[0] ^ sign, pk[1] ^ sign};
      }
      sched_fence();  // one column block at a time: its 32 values, then the next
    }
    block_barrier();
    const int run = tid & 31;  // 16-byte run of a row
#pragma unroll
    for (int i = 0; i < kPassTok * 32 / kThreads; ++i) {
      const int row = (tid >> 5) + (kThreads / 32) * i;
      const u32x4_t val =
          *reinterpret_cast<const u32x4_t*>(lds + row * kRowBytes + ((run ^ (row & 31)) * 16));
      // staging row -> token: wave column row / 32, block row / 16 % 2, lane row % 16
      const int tok = (row >> 5) * kWaveN + (pass * kNiPass + ((row >> 4) & 1)) * kMfma + (row & 15);
      const uint32_t off = (uint32_t)(tok * row_bytes) + run * 16;
      __builtin_amdgcn_raw_buffer_store_b128(val, gbuf, off, 0, 0);
    }
    sched_fence();
  }
}

// bf16 strips in the strip buffer: G is kept in blocks (BlockedG, 16 tokens x
// 32 vocabulary rows per kilobyte), so every wave stores its gradient values
// straight from registers, one whole block per store instruction, with no LDS
// staging and no barrier.  Per element one FMA, one exp2 and half a packed
// bf16 conversion (the token's |scale| folded into the exponent, its sign
// applied to the packed bits).  Two MFMA tiles mi = 2 p, 2 p + 1 of a column
// block ni form block (token band, vocabulary column p) of the wave: lane
// group g holds vocabulary rows 4 g .. + 3 of each; one permlane16 swap per
// packed dword gives every lane 16 contiguous bytes of a block row (groups 0
// and 2 the first tile's halves, groups 1 and 3 the second's).  Targets and
// lse are loaded before any store.
// What the gradient epilogue reads per token of a tile (targets, lse) and the
// gradient scale: loaded before the tile's stages, so that the epilogue does
// not wait on them (nor on the copies in flight that such a wait would drain).
template <typename AccT>
struct GradInputs {
  int32_t tgt[AccT::NI];
  float lse[AccT::NI];
  float scale;
};

// (Read at the token clamped to N - 1, as in lse_targets; the epilogue drops
// tokens past N.)
template <typename AccT>
__device__ __forceinline__ void grad_inputs(const StripArgs<__bf16>& a, int64_t n0,
                                            GradInputs<AccT>& in) {
#pragma unroll
  for (int ni = 0; ni < AccT::NI; ++ni) {
    const int64_t tok = lse_token<AccT>(n0, ni);
    const int64_t tc = tok < a.N ? tok : a.N - 1;
    in.tgt[ni] = a.targets[tc];
    in.lse[ni] = a.lse[tc];
  }
  in.scale = a.ctrl->grad_scale;
}

template <typename AccT>
__device__ __forceinline__ void grad_epilogue_blocked(const StripArgs<__bf16>& a, AccT& acc,
                                                      int64_t m0, int64_t n0,
                                                      const GradInputs<AccT>* pre = nullptr) {
  constexpr int kMI = AccT::MI, kNI = AccT::NI, kWaveM = AccT::WaveM, kWaveN = AccT::WaveN;
  const int tid = opaque((int)threadIdx.x);  // recomputed per tile, not kept live
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t vrow0 = m0 + wm * kWaveM;
  const bool full = vrow0 + kWaveM <= a.v_len;
  const int rows_left = full ? kWaveM : (int)max<int64_t>(a.v_len - vrow0, 0);
  const int r_lane = (lane >> 4) * 4;
  GradInputs<AccT> in;
  if (pre)
    in = *pre;
  else
    grad_inputs<AccT>(a, n0, in);
  const float scale_all = in.scale;
  const float abs_scale = fabsf(scale_all);
  const uint32_t sign = scale_all < 0.f ? 0x80008000u : 0u;
  const float log2_scale = __builtin_amdgcn_logf(abs_scale);

  float c[kNI];
  int tl[kNI];
  bool any_hit[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const bool tok_ok = lse_token<AccT>(n0, ni) < a.N;
    const int32_t t = tok_ok ? in.tgt[ni] : a.ignore_index;
    const bool valid = t != a.ignore_index;
    const float lse2 = (tok_ok ? in.lse[ni] : 0.f) * kLog2e;
    c[ni] = valid ? log2_scale - lse2 : -INFINITY;
    const int64_t tl64 = (int64_t)t - (a.v_begin + vrow0);
    const bool hit = valid && tl64 >= 0 && tl64 < kWaveM;
    tl[ni] = hit ? (int)tl64 : -1;
    any_hit[ni] = __any(hit);
  }

  // blocks from the tile's first one: band n0 / 16, block column m0 / 32;
  // bands past the strip buffer's last (tokens past round_up(N, 16)) are
  // out of range
  const int64_t band = BlockedG::band_bytes(a.ldg, 2);
  const int64_t col0 = (m0 / 32) * BlockedG::kBlkBytes;
  const __amdgpu_buffer_rsrc_t gbuf =
      make_buffer(reinterpret_cast<char*>(a.g_strip) + (n0 / 16) * band + col0,
                  ((a.N + 15) / 16 - n0 / 16) * band - col0);
  const int g = lane >> 4;
  // byte offset of this lane's 16 bytes in the wave's first block (bands are
  // below 2^26 bytes apart: ldg <= 2^21)
  const uint32_t band32 = (uint32_t)band;
  const uint32_t off0 = (uint32_t)(wn * (kWaveN / 16)) * band32 +
                        (uint32_t)(wm * (kWaveM / 32) * BlockedG::kBlkBytes) +
                        (uint32_t)((lane & 15) * BlockedG::kRowBytes + (((g & 1) << 1) | (g >> 1)) * 16);
  // One 16-token column block at a time: its 32 values per lane, the row and
  // target tests as wave-uniform branches over all of them (selects per
  // element would triple the VALU work), then four packed block stores.
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    float v[4 * kMI];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[mi * 4 + e] = fast_exp2(__builtin_fmaf(AccT::read(acc.c[mi][ni], e), kLog2e, c[ni]));
    if (!full) {
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[mi * 4 + e] = r_lane < rows_left - acc_row(mi, e, 0) ? v[mi * 4 + e] : 0.f;
    }
    if (any_hit[ni]) {
      const int d = tl[ni] - r_lane;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[mi * 4 + e] = d == acc_row(mi, e, 0) ? v[mi * 4 + e] - abs_scale : v[mi * 4 + e];
    }
#pragma unroll
    for (int p = 0; p < kMI / 2; ++p) {
      const u32x2_t q0 = GPack<__bf16>::pack(v[8 * p], v[8 * p + 1], v[8 * p + 2], v[8 * p + 3]);
      const u32x2_t q1 =
          GPack<__bf16>::pack(v[8 * p + 4], v[8 * p + 5], v[8 * p + 6], v[8 * p + 7]);
      const auto x = __builtin_amdgcn_permlane16_swap(q0[0] ^ sign, q1[0] ^ sign, false, false);
      const auto y = __builtin_amdgcn_permlane16_swap(q0[1] ^ sign, q1[1] ^ sign, false, false);
      const u32x4_t val{x[0], y[0], x[1], y[1]};
      const uint32_t off = off0 + (uint32_t)ni * band32 + (uint32_t)(p * BlockedG::kBlkBytes);
      __builtin_amdgcn_raw_buffer_store_b128(val, gbuf, off, 0, 0);
    }
    sched_fence();  // one column block at a time: its 32 values, then the next
  }
}

// The backward strip on the one-wave-per-SIMD engine (bf16, blocked G).
template <bool Late>
__global__ __launch_bounds__(w4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void strip_grad_kernel_w4(StripArgs<__bf16> a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<__bf16> A{a.weight_strip, a.H, a.v_len, a.H};
  const Operand<__bf16> B{a.hidden, a.H, a.N, a.H};
  const TileGrid grid{a.m_tiles, a.n_tiles, a.group_m, blockIdx.x, gridDim.x, true};
  GradInputs<w4::Acc> in;  // loaded at a tile's start, used by its epilogue
  w4::run_tiles<w4::KRow128, w4::KRow128, Late>(
      A, B, a.H, grid, lds, [&](int64_t, int64_t n0) { grad_inputs<w4::Acc>(a, n0, in); },
      [&](w4::Acc& acc, int64_t m0, int64_t n0, char*) {
        grad_epilogue_blocked(a, acc, m0, n0, &in);
      });
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void strip_grad_kernel(StripArgs<T> a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<T> A{a.weight_strip, a.H, a.v_len, a.H};
  const Operand<T> B{a.hidden, a.H, a.N, a.H};
  const TileGrid grid{a.m_tiles, a.n_tiles, a.group_m, blockIdx.x, gridDim.x, true};
  run_tiles<T, true, true>(A, B, a.H, grid, lds,
                           [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
                             if constexpr (kGBlocked<T>)
                               grad_epilogue_blocked(a, acc, m0, n0);
                             else
                               grad_epilogue(a, acc, m0, n0, staging, strip_dst(a, m0, n0));
                           });
}

// ---------------------------------------------------------------------------
// Plain fp32-output GEMM tile: C[m, n] (+)= sum_k A[m, k] B[n, k].
//
// The epilogue goes through the LDS staging area in four passes of 64 rows
// (1 KiB each, unpadded: the 16-byte chunk index is XOR-swizzled by row bits
// 2..3, so the four rows of an MFMA-layout write never share banks): the
// waves that hold those rows write them, then all threads move whole 16-byte
// runs of each row, so that every wave reads and writes 1 KiB of one row of C
// per instruction.  With Accum a pass issues half of its loads of C before
// the staging writes, so that their latency hides behind them.
// ---------------------------------------------------------------------------
// Tile order of the fp32-output GEMMs: bands of groups (see TileGrid) or one
// contiguous range of the group order per XCD.
constexpr bool kGemmBands = false;

constexpr int kEpiRows = 64;                        // rows of C per pass
constexpr int kEpiRowBytes = kTile * 4;             // one row of C in LDS
static_assert(kEpiRows * kEpiRowBytes <= kStagingBytes, "epilogue staging fits in LDS");

// Byte offset in the staging area of 16-byte chunk `chunk` of row `row`.
__device__ __forceinline__ int epi_offset(int row, int chunk) {
  return row * kEpiRowBytes + ((chunk ^ (((row >> 2) & 3) << 2)) * 16);
}

template <typename T, bool Accum>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs<T>& g, Acc& acc, int64_t m0,
                                              int64_t n0, char* lds) {
  const int tid = opaque((int)threadIdx.x);  // recomputed per tile, not kept live
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // C from (m0, n0): byte offset (row - m0) * ldc * 4 + (col - n0) * 4.  Rows
  // past m fall past the record count; 16-byte runs past n get an
  // out-of-range offset (n is a multiple of 4, so runs are never split).
  const uint32_t ldc4 = (uint32_t)(g.ldc * 4);
  const __amdgpu_buffer_rsrc_t cbuf =
      make_buffer(g.c + m0 * g.ldc + n0, (g.m - m0) * g.ldc * 4 - n0 * 4);
  const int run = tid & 63;                         // 16-byte run of a row (4 columns)
  const bool run_ok = n0 + 4 * run < g.n;
  constexpr int kRowsPerThread = kEpiRows / kWaves;  // every wave one row at a time

#pragma unroll
  for (int pass = 0; pass < kTile / kEpiRows; ++pass) {
    const int row0 = pass * kEpiRows;
    // rows of this thread: row0 + wave + kWaves i; byte offsets from the tile's row 0
    const uint32_t off0 = run_ok ? (uint32_t)(row0 + wave) * ldc4 + run * 16 : kOutOfRange;
    const uint32_t step = run_ok ? kWaves * ldc4 : 0u;
    constexpr int kEarly = kRowsPerThread / 2;  // C rows loaded before the staging writes
    u32x4_t old[kRowsPerThread];
    if constexpr (Accum) {
#pragma unroll
      for (int i = 0; i < kEarly; ++i)
        old[i] = __builtin_amdgcn_raw_buffer_load_b128(cbuf, off0 + i * step, 0, 0);
    }
    block_barrier();  // staging free: the previous pass (or tile) is done with it
    constexpr int kPassesPerWave = kWaveM / kEpiRows;
    if (wm == pass / kPassesPerWave) {
      // rows kEpiRows (pass % kPassesPerWave) .. + kEpiRows of this wave's kWaveM
#pragma unroll
      for (int h = 0; h < kEpiRows / kMfma; ++h) {
        const int mi = (kEpiRows / kMfma) * (pass % kPassesPerWave) + h;
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          const int col = wn * kWaveN + ni * kMfma + (lane & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = h * kMfma + acc_row(0, e, lane);
            *reinterpret_cast<float*>(lds + epi_offset(row, col >> 2) + (col & 3) * 4) =
                acc.c[mi][ni][e];
          }
        }
      }
    }
    block_barrier();
    f32x4_t v[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int row = wave + kWaves * i;
      v[i] = *reinterpret_cast<const f32x4_t*>(lds + epi_offset(row, run));
    }
    if constexpr (Accum) {
#pragma unroll
      for (int i = kEarly; i < kRowsPerThread; ++i)
        old[i] = __builtin_amdgcn_raw_buffer_load_b128(cbuf, off0 + i * step, 0, 0);
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) v[i] += __builtin_bit_cast(f32x4_t, old[i]);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[i]), cbuf, off0 + i * step,
                                             0, 0);
    sched_fence();  // one pass at a time: keeps the live registers to one pass's rows
  }
}

template <typename T, bool AK, bool BK, bool Accum>
__global__ __launch_bounds__(kThreads, 1) void gemm_f32out_kernel(GemmArgs<T> g) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<T> A{g.a, g.lda, g.a_mn_ext, g.a_k_ext};
  const Operand<T> B{g.b, g.ldb, g.b_mn_ext, g.b_k_ext};
  const TileGrid grid{g.m_tiles, g.n_tiles, g.group_m, blockIdx.x, gridDim.x, kGemmBands};
  run_tiles<T, AK, BK, kGBlocked<T>>(A, B, g.k_len, grid, lds,
                       [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
                         gemm_epilogue<T, Accum>(g, acc, m0, n0, staging);
                       });
}

// The fp32-output epilogue of the one-wave-per-SIMD engine: rows of C move
// through the kStagingBytes after its stage buffers in eight passes of 32
// rows, pass p taking the 16 rows of MFMA sub-tile p from each half of the
// tile (tile rows 16 p .. 16 p + 15 and 128 + 16 p ..), so that every wave
// writes its share of every pass; then all four waves move whole rows, 1 KiB
// of C per instruction.  Staging row r holds tile row (r / 16) 128 + 16 p +
// r % 16.
constexpr int kEpi4Rows = w4::kStagingBytes / kEpiRowBytes;  // 32

template <typename T, bool Accum>
__device__ __forceinline__ void gemm_epilogue_w4(const GemmArgs<T>& g, w4::Acc& acc, int64_t m0,
                                                 int64_t n0, char* lds) {
  const int tid = opaque((int)threadIdx.x);  // recomputed per tile, not kept live
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t ldc4 = (uint32_t)(g.ldc * 4);
  const __amdgpu_buffer_rsrc_t cbuf =
      make_buffer(g.c + m0 * g.ldc + n0, (g.m - m0) * g.ldc * 4 - n0 * 4);
  const int run = tid & 63;
  const bool run_ok = n0 + 4 * run < g.n;
  constexpr int kRowsPerThread = kEpi4Rows / w4::kWaves;  // 8: staging rows wave + 4 i
  static_assert(kEpi4Rows == 2 * kMfma && w4::kMI * kMfma == w4::kWaveM, "pass geometry");

#pragma unroll
  for (int pass = 0; pass < w4::kMI; ++pass) {
    // staging row wave + 4 i is tile row (i / 4) 128 + 16 pass + wave + 4 (i % 4)
    auto row_off = [&](int i) -> uint32_t {
      const int row = (i / 4) * w4::kWaveM + kMfma * pass + wave + 4 * (i % 4);
      return run_ok ? (uint32_t)row * ldc4 + run * 16 : kOutOfRange;
    };
    constexpr int kEarly = kRowsPerThread / 2;
    u32x4_t old[kRowsPerThread];
    if constexpr (Accum) {
#pragma unroll
      for (int i = 0; i < kEarly; ++i)
        old[i] = __builtin_amdgcn_raw_buffer_load_b128(cbuf, row_off(i), 0, 0);
    }
    block_barrier();  // staging free: the previous pass (or tile) is done with it
#pragma unroll
    for (int ni = 0; ni < w4::kNI; ++ni) {
      const int col = wn * w4::kWaveN + ni * kMfma + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm * kMfma + acc_row(0, e, lane);
        *reinterpret_cast<float*>(lds + epi_offset(row, col >> 2) + (col & 3) * 4) =
            w4::Acc::read(acc.c[pass][ni], e);
      }
    }
    block_barrier();
    f32x4_t v[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int row = wave + w4::kWaves * i;
      v[i] = *reinterpret_cast<const f32x4_t*>(lds + epi_offset(row, run));
    }
    if constexpr (Accum) {
#pragma unroll
      for (int i = kEarly; i < kRowsPerThread; ++i)
        old[i] = __builtin_amdgcn_raw_buffer_load_b128(cbuf, row_off(i), 0, 0);
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) v[i] += __builtin_bit_cast(f32x4_t, old[i]);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[i]), cbuf, row_off(i),
                                             0, 0);
    sched_fence();
  }
}

// dH (AK: K-contiguous blocked G, MN-contiguous W_s) and dW (blocked G and
// h, both MN-contiguous) on the one-wave-per-SIMD engine.
template <bool AK, bool Accum>
__global__ __launch_bounds__(w4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_f32out_kernel_w4(GemmArgs<__bf16> g) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const Operand<__bf16> A{g.a, g.lda, g.a_mn_ext, g.a_k_ext};
  const Operand<__bf16> B{g.b, g.ldb, g.b_mn_ext, g.b_k_ext};
  const TileGrid grid{g.m_tiles, g.n_tiles, g.group_m, blockIdx.x, gridDim.x, kGemmBands};
  using SA = typename std::conditional<AK, w4::KSplitBlk, w4::MNBlk>::type;
  w4::run_tiles<SA, w4::MN>(A, B, g.k_len, grid, lds, [](int64_t, int64_t) {},
                            [&](w4::Acc& acc, int64_t m0, int64_t n0, char* staging) {
                              gemm_epilogue_w4<__bf16, Accum>(g, acc, m0, n0, staging);
                            });
}

// dH and dW sharing one launch (see gemm_dh_dw_kernel below) on the
// one-wave-per-SIMD engine.
template <bool AccumDh, bool AccumDw>
__global__ __launch_bounds__(w4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_dh_dw_kernel_w4(GemmArgs<__bf16> dh, GemmArgs<__bf16> dw, int64_t split) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int64_t b = blockIdx.x;
  if (b < split) {
    const Operand<__bf16> A{dh.a, dh.lda, dh.a_mn_ext, dh.a_k_ext};
    const Operand<__bf16> B{dh.b, dh.ldb, dh.b_mn_ext, dh.b_k_ext};
    const TileGrid grid{dh.m_tiles, dh.n_tiles, dh.group_m, b, split, kGemmBands};
    w4::run_tiles<w4::KSplitBlk, w4::MN>(
        A, B, dh.k_len, grid, lds, [](int64_t, int64_t) {}, [&](w4::Acc& acc, int64_t m0, int64_t n0, char* staging) {
          gemm_epilogue_w4<__bf16, AccumDh>(dh, acc, m0, n0, staging);
        });
  } else {
    const Operand<__bf16> A{dw.a, dw.lda, dw.a_mn_ext, dw.a_k_ext};
    const Operand<__bf16> B{dw.b, dw.ldb, dw.b_mn_ext, dw.b_k_ext};
    const TileGrid grid{dw.m_tiles, dw.n_tiles, dw.group_m, b - split, gridDim.x - split,
                        kGemmBands};
    w4::run_tiles<w4::MNBlk, w4::MN>(
        A, B, dw.k_len, grid, lds, [](int64_t, int64_t) {}, [&](w4::Acc& acc, int64_t m0, int64_t n0, char* staging) {
          gemm_epilogue_w4<__bf16, AccumDw>(dw, acc, m0, n0, staging);
        });
  }
}

// dH and dW of one strip in one launch: blocks [0, split) form dH
// (K-contiguous G, MN-contiguous W_s), the rest dW (MN-contiguous G and h).
// Both read G and write disjoint outputs, so the compute units can be shared
// out by work when one of them alone has too few tiles to fill them.
template <typename T, bool AccumDh, bool AccumDw>
__global__ __launch_bounds__(kThreads, 1) void gemm_dh_dw_kernel(GemmArgs<T> dh, GemmArgs<T> dw,
                                                                 int64_t split) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int64_t b = blockIdx.x;
  if (b < split) {
    const Operand<T> A{dh.a, dh.lda, dh.a_mn_ext, dh.a_k_ext};
    const Operand<T> B{dh.b, dh.ldb, dh.b_mn_ext, dh.b_k_ext};
    const TileGrid grid{dh.m_tiles, dh.n_tiles, dh.group_m, b, split, kGemmBands};
    run_tiles<T, true, false, kGBlocked<T>>(A, B, dh.k_len, grid, lds,
                                            [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
                                              gemm_epilogue<T, AccumDh>(dh, acc, m0, n0, staging);
                                            });
  } else {
    const Operand<T> A{dw.a, dw.lda, dw.a_mn_ext, dw.a_k_ext};
    const Operand<T> B{dw.b, dw.ldb, dw.b_mn_ext, dw.b_k_ext};
    const TileGrid grid{dw.m_tiles, dw.n_tiles, dw.group_m, b - split, gridDim.x - split,
                        kGemmBands};
    run_tiles<T, false, false, kGBlocked<T>>(A, B, dw.k_len, grid, lds,
                                             [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
                                               gemm_epilogue<T, AccumDw>(dw, acc, m0, n0, staging);
                                             });
  }
}

// ---------------------------------------------------------------------------
// Backward without a strip buffer: each (token tile i, vocabulary tile j)
// pair is recomputed, its G tile formed and multiplied at once into the rows
// of dH and dW it feeds, so G never exists beyond one tile per block.
// ---------------------------------------------------------------------------
// Block b = r * C + c takes the pairs (i, j) with i in token group r and j in
// vocabulary group c, i-major.  Per pair:
//   Z^T = W_j . h_i^T (K = H), G = scale (softmax - onehot) into the block's
//   own 256 x 256 tile of g_scratch;
//   dh (with do_dh): dh_dst[c][rows of i] (+)= G . W_j   (K = rows of j)
//   dw (with do_dw): dw_dst[r][rows of j] (+)= G^T . h_i (K = rows of i)
// dh_dst[c] is written only by blocks of vocabulary group c and token rows of
// their own token group, so each output row has one writer and a fixed order
// of additions (over j for dH, over i for dW): no atomics, and results that do
// not depend on timing.  The first pair that touches a row overwrites it.
template <typename T>
struct FusedArgs {
  const T* hidden;         // [N, H]
  const T* weight;         // [V, H]
  const int32_t* targets;  // [N]
  const float* lse;        // [N]
  const Control* ctrl;
  int64_t N, H, V;
  int32_t ignore_index;
  T* g_scratch;            // [gridDim.x][256][256]
  float* dh_dst;           // [C][N][H] (dH itself when C == 1)
  float* dw_dst;           // [R][V][H] (dW itself when R == 1)
  int64_t C, tok_per_r, voc_per_c;  // groups: tiles per token group / vocabulary group
  int do_dh, do_dw;
};

// C[0:m, 0:n] (+)= A . B^T for one block, its 256 x 256 output tiles walked
// along n.  The persistent tile loop runs its copy stream one tile ahead, which
// needs more K stages per tile than the ring holds; shorter K goes one tile
// per call.
template <typename T, bool AK, bool BK>
__device__ __forceinline__ void block_gemm_rows(const Operand<T>& A, Operand<T> B, int64_t k_len,
                                                GemmArgs<T> g, bool accum, char* lds) {
  constexpr int64_t kStageK = kStageRowBytes / sizeof(T);
  const int64_t n_tiles = (g.n + kTile - 1) / kTile;
  auto epi = [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
    if (accum)
      gemm_epilogue<T, true>(g, acc, m0, n0, staging);
    else
      gemm_epilogue<T, false>(g, acc, m0, n0, staging);
  };
  if ((k_len + kStageK - 1) / kStageK > kStages) {
    const TileGrid grid{1, n_tiles, 1, 0, 1, false};
    run_tiles<T, AK, BK>(A, B, k_len, grid, lds, epi);
    return;
  }
  const TileGrid one{1, 1, 1, 0, 1, false};
  for (int64_t t = 0; t < n_tiles; ++t) {
    // B is MN-contiguous here: column block t starts t * 256 elements along a row
    Operand<T> Bt{B.base + t * kTile, B.ld, B.mn_ext - t * kTile, B.k_ext};
    GemmArgs<T> gt = g;
    gt.c = g.c + t * kTile;
    gt.n = g.n - t * kTile;
    auto epi_t = [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
      if (accum)
        gemm_epilogue<T, true>(gt, acc, m0, n0, staging);
      else
        gemm_epilogue<T, false>(gt, acc, m0, n0, staging);
    };
    run_tiles<T, AK, BK>(A, Bt, k_len, one, lds, epi_t);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void fused_bwd_kernel(FusedArgs<T> f) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int64_t b = blockIdx.x;
  const int64_t c = b % f.C, r = b / f.C;
  const int64_t tok_tiles = (f.N + kTile - 1) / kTile, voc_tiles = (f.V + kTile - 1) / kTile;
  const int64_t i_lo = r * f.tok_per_r, i_hi = min(tok_tiles, i_lo + f.tok_per_r);
  const int64_t j_lo = c * f.voc_per_c, j_hi = min(voc_tiles, j_lo + f.voc_per_c);
  T* const gt = f.g_scratch + b * (int64_t)kTile * kTile;
  // this block's copy of each output (the output itself when not split)
  float* const dh = f.do_dh ? f.dh_dst + c * f.N * f.H : nullptr;
  float* const dw = f.do_dw ? f.dw_dst + r * f.V * f.H : nullptr;
  for (int64_t i = i_lo; i < i_hi; ++i) {
    const int64_t t0 = i * kTile, nt = min<int64_t>(kTile, f.N - t0);
    for (int64_t j = j_lo; j < j_hi; ++j) {
      const int64_t v0 = j * kTile, nv = min<int64_t>(kTile, f.V - v0);
      // the pair's logits, recomputed, and its G tile
      StripArgs<T> a{};
      a.hidden = f.hidden + t0 * f.H;
      a.weight_strip = f.weight + v0 * f.H;
      a.targets = f.targets + t0;
      a.N = nt;
      a.H = f.H;
      a.v_begin = v0;
      a.v_len = nv;
      a.ignore_index = f.ignore_index;
      a.lse = f.lse + t0;
      a.ctrl = f.ctrl;
      const Operand<T> Wj{a.weight_strip, f.H, nv, f.H};
      const Operand<T> hi{a.hidden, f.H, nt, f.H};
      const GradDst<T> dst{gt, kTile, nt * kTile * (int64_t)sizeof(T)};
      run_tiles<T, true, true>(Wj, hi, f.H, TileGrid{1, 1, 1, 0, 1, false}, lds,
                               [&](Acc& acc, int64_t m0, int64_t n0, char* staging) {
                                 grad_epilogue(a, acc, m0, n0, staging, dst);
                               });
      // G's stores complete and are visible to the block's copies that follow
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      block_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (f.do_dh) {
        // dH rows of tile i (+)= G[nt, nv] . W_j[nv, H]: A = G K-contiguous, B = W_j
        // MN-contiguous (row = vocabulary row, the contraction index)
        const Operand<T> A{gt, kTile, nt, nv};
        const Operand<T> B{a.weight_strip, f.H, f.H, nv};
        GemmArgs<T> g{};
        g.c = dh + t0 * f.H; g.ldc = f.H; g.m = nt; g.n = f.H;
        block_gemm_rows<T, true, false>(A, B, nv, g, j > j_lo, lds);
      }
      if (f.do_dw) {
        // dW rows of tile j (+)= G^T[nv, nt] . h_i[nt, H]: both MN-contiguous (row =
        // token, the contraction index); G's pad columns are zero
        const int64_t cols = (nv + 7) / 8 * 8;
        const Operand<T> A{gt, kTile, cols, nt};
        const Operand<T> B{a.hidden, f.H, f.H, nt};
        GemmArgs<T> g{};
        g.c = dw + v0 * f.H; g.ldc = f.H; g.m = nv; g.n = f.H;
        block_gemm_rows<T, false, false>(A, B, nt, g, i > i_lo, lds);
      }
      // every copy of G has landed before the next pair's epilogue rewrites it
      block_barrier();
    }
  }
}

// out[k] = sum_p parts[p][k] over p = 0 .. P - 1 in that order (fixed order:
// the result does not depend on timing).  count is a multiple of 4.
__global__ void sum_parts_kernel(const float* __restrict__ parts, int64_t P, int64_t count,
                                 float* __restrict__ out) {
  const int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (q >= count) return;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(parts + q);
  for (int64_t p = 1; p < P; ++p) acc += *reinterpret_cast<const f32x4_t*>(parts + p * count + q);
  *reinterpret_cast<f32x4_t*>(out + q) = acc;
}

// ---------------------------------------------------------------------------
// Small per-token kernels.
// ---------------------------------------------------------------------------
__global__ void state_init_kernel(float* m, float* s, float* zt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    m[i] = -INFINITY;
    s[i] = 0.f;
    zt[i] = __builtin_nanf("");
  }
}

// Merge (m, s) with (mp, sp): both describe sum_v exp(z_v) as s * e^m.
__device__ __forceinline__ void lse_merge(float& m, float& s, float mp, float sp) {
  const float mn = fmaxf(m, mp);
  if (mn == -INFINITY) return;  // nothing seen on either side
  s = s * fast_exp2((m - mn) * kLog2e) + sp * fast_exp2((mp - mn) * kLog2e);
  m = mn;
}

// Fold partials [n_blocks, n] into the running state (m, s) [n]: a block of
// kFoldWays waves takes 64 consecutive tokens (one per lane, so every load is
// 512 contiguous bytes); wave w merges the partial blocks w, w + kFoldWays,
// ... of its tokens, then wave 0 merges the kFoldWays results in wave order
// and the state.  The order of merges is fixed, so results do not depend on
// timing.  Spreading the blocks over waves keeps enough loads in flight when
// there are few tokens and many blocks (a whole vocabulary in one fold).
constexpr int kFoldWays = 16;

__global__ __launch_bounds__(64 * kFoldWays) void fold_kernel(const float2* __restrict__ partials,
                                                              int64_t n_blocks, float* m, float* s,
                                                              int64_t n) {
  __shared__ float2 part[kFoldWays][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  float mm = -INFINITY, ss = 0.f;
  if (i < n) {
    int64_t b = w;
    for (; b + 3 * kFoldWays < n_blocks; b += 4 * kFoldWays) {
      float2 p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = partials[(b + u * kFoldWays) * n + i];
#pragma unroll
      for (int u = 0; u < 4; ++u) lse_merge(mm, ss, p[u].x, p[u].y);
    }
    for (; b < n_blocks; b += kFoldWays) {
      const float2 p = partials[b * n + i];
      lse_merge(mm, ss, p.x, p.y);
    }
  }
  part[w][lane] = float2{mm, ss};
  __syncthreads();
  if (w == 0 && i < n) {
    mm = m[i];
    ss = s[i];
#pragma unroll
    for (int k = 0; k < kFoldWays; ++k) lse_merge(mm, ss, part[k][lane].x, part[k][lane].y);
    m[i] = mm;
    s[i] = ss;
  }
}

// The running state as three rows [3, n] (max, sum, target logit), out and in.
__global__ void state_export_kernel(const float* __restrict__ m, const float* __restrict__ s,
                                    const float* __restrict__ zt, float* __restrict__ state,
                                    int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    state[i] = m[i];
    state[n + i] = s[i];
    state[2 * n + i] = zt[i];
  }
}

__global__ void state_merge_kernel(const float* __restrict__ state, float* m, float* s, float* zt,
                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float mm = m[i], ss = s[i];
    lse_merge(mm, ss, state[i], state[n + i]);
    m[i] = mm;
    s[i] = ss;
    const float z = zt[i];
    if (z != z) zt[i] = state[2 * n + i];  // NaN: the target was not folded on this side
  }
}

constexpr int kReduceThreads = 1024;

// One block: lse, row loss, n_valid and the reduced loss (fixed-order sums).
__global__ __launch_bounds__(kReduceThreads) void finalize_kernel(
    const float* __restrict__ m, const float* __restrict__ s, const float* __restrict__ zt,
    const int32_t* __restrict__ targets, int64_t n, int32_t ignore_index, int reduction,
    float* lse, float* row_loss, float* loss) {
  __shared__ double part_sum[kReduceThreads];
  __shared__ long long part_cnt[kReduceThreads];
  double acc = 0.0;
  long long cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += kReduceThreads) {
    const float l = m[i] + logf(s[i]);
    lse[i] = l;
    const bool valid = targets[i] != ignore_index;
    const float rl = valid ? l - zt[i] : 0.f;
    if (row_loss) row_loss[i] = rl;
    acc += (double)rl;
    cnt += valid ? 1 : 0;
  }
  part_sum[threadIdx.x] = acc;
  part_cnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = kReduceThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      part_sum[threadIdx.x] += part_sum[threadIdx.x + w];
      part_cnt[threadIdx.x] += part_cnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tot = part_sum[0];
    const long long nv = part_cnt[0];
    loss[0] = reduction == 0 ? (float)(tot / (double)nv) : (float)tot;
  }
}

// One block: count non-ignored rows and form the gradient scale.
__global__ __launch_bounds__(kReduceThreads) void grad_scale_kernel(
    const int32_t* __restrict__ targets, int64_t n, int32_t ignore_index, int reduction,
    const float* __restrict__ grad_out, Control* ctrl) {
  __shared__ long long part_cnt[kReduceThreads];
  long long cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += kReduceThreads) cnt += targets[i] != ignore_index;
  part_cnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = kReduceThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part_cnt[threadIdx.x] += part_cnt[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long nv = part_cnt[0];
    const float go = grad_out[0];
    ctrl->n_valid = nv;
    ctrl->grad_scale = reduction == 0 ? (nv > 0 ? (float)((double)go / (double)nv) : 0.f) : go;
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
static hipError_t set_lds(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

// M-tiles per group of the tile order: 8 vocabulary tiles of a strip (their
// W rows stay in L2 while token tiles stream past).
constexpr int64_t kStripGroupM = 8;
// Output GEMMs: 4 M-tiles per group, all N-tiles of those rows.
constexpr int64_t kGemmGroupM = 4;

// Compute units of the current device, rounded down to a multiple of the XCD
// count (queried once per device).
static int64_t persistent_blocks() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* slot = dev < 64 ? &cache[dev] : nullptr;
  int n = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = kXcds;
    n = n / kXcds * kXcds;
    if (n <= 0) n = kXcds;
    if (slot) slot->store(n, std::memory_order_relaxed);
  }
  return n;
}

// Blocks for `tiles` tiles of `nk` stages each: one per compute unit, each
// looping over its tiles, when a tile has more stages than the ring holds
// (so the copy stream is never more than one tile ahead); else one per tile.
static int64_t grid_blocks(int64_t tiles, int64_t nk) {
  if (nk <= kStages) return tiles;
  const int64_t p = persistent_blocks();
  return tiles < p ? tiles : p;
}

// A grid of one block per tile can only be launched up to 2^31 - 1 blocks.
static bool grid_ok(int64_t blocks) { return blocks >= 1 && blocks <= 0x7fffffffLL; }

template <typename T>
static int64_t stages_of(int64_t k_len) {
  constexpr int64_t kStageK = kStageRowBytes / sizeof(T);
  return (k_len + kStageK - 1) / kStageK;
}

// A strip kernel on the one-wave-per-SIMD engine, in persistent blocks (its
// copy stream needs at least two K stages per tile).  The gradient strip
// takes the late copy schedule (both operands' copies of a stage in the last
// half step two stages ahead) when its blocks have at least 8 tiles: at
// 131072 tokens, 64 tiles per block, it was 0.7-1.2% faster on four boxes;
// at 4096 tokens, 2 tiles per block, 2.5-4% slower.  The forward keeps the
// default schedule (with the late one: within noise at 131072 tokens, up to
// 2.4% slower at 4096 with 37 tiles per block).
static hipError_t launch_w4(void (*early)(StripArgs<__bf16>), void (*late)(StripArgs<__bf16>),
                            const StripArgs<__bf16>& a, hipStream_t st) {
  if (cdiv(a.H, w4::kStageK) < 2) return hipErrorInvalidValue;
  const int64_t tiles = a.m_tiles * a.n_tiles;
  const int64_t p = persistent_blocks();
  const int64_t blocks = tiles < p ? tiles : p;
  if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
  void (*kernel)(StripArgs<__bf16>) = late && tiles >= 8 * blocks ? late : early;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, w4::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(w4::kThreads), w4::kLdsBytes, st, a);
  return hipGetLastError();
}

// bf16 strip kernels of at least 12 K stages (H >= 768), and output GEMMs of
// at least 16, run on the one-wave-per-SIMD engine; shorter ones, and fp32,
// on the eight-wave engine.  With a single wave on a SIMD nothing covers a
// tile's epilogue, which the MFMAs of 12 stages amortise and those of 8 do
// not: at H = 512 the one-wave forward took 11% longer than the eight-wave
// one; with the one-wave strip kernels the step was 1.6% faster at H = 768,
// 0.5% at 1024 and 2.6% at 1536 (32768 tokens), and at H = 2048 the forward
// 4% faster at 131072 tokens.  The output GEMMs' read-modify-write epilogue
// weighs more per tile, and they keep 16.
constexpr int64_t kW4MinStagesStrip = 12;
constexpr int64_t kW4MinStages = 16;

template <typename T>
static bool use_w4(const StripArgs<T>& a) {
  if constexpr (std::is_same<T, __bf16>::value)
    return cdiv(a.H, w4::kStageK) >= kW4MinStagesStrip;
  else
    return false;
}

template <typename T>
hipError_t launch_strip_lse(StripArgs<T> a, hipStream_t st) {
  a.m_tiles = cdiv(a.v_len, kTile);
  a.n_tiles = cdiv(a.N, kTile);
  a.group_m = kStripGroupM;
  if constexpr (std::is_same<T, __bf16>::value)
    if (use_w4(a)) return launch_w4(strip_lse_kernel_w4, nullptr, a, st);
  const int64_t blocks = grid_blocks(a.m_tiles * a.n_tiles, stages_of<T>(a.H));
  if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
  hipError_t e = set_lds<T>(reinterpret_cast<const void*>(&strip_lse_kernel<T>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(strip_lse_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_strip_grad(StripArgs<T> a, hipStream_t st) {
  a.m_tiles = cdiv(a.v_len, kTile);
  a.n_tiles = cdiv(a.N, kTile);
  a.group_m = kStripGroupM;
  if constexpr (std::is_same<T, __bf16>::value)
    if (use_w4(a))
      return launch_w4(strip_grad_kernel_w4<false>, strip_grad_kernel_w4<true>, a, st);
  const int64_t blocks = grid_blocks(a.m_tiles * a.n_tiles, stages_of<T>(a.H));
  if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
  hipError_t e = set_lds<T>(reinterpret_cast<const void*>(&strip_grad_kernel<T>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(strip_grad_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes, st, a);
  return hipGetLastError();
}

template <typename T, bool AK, bool BK, bool Accum>
static hipError_t launch_gemm(GemmArgs<T> g, hipStream_t st) {
  g.m_tiles = cdiv(g.m, kTile);
  g.n_tiles = cdiv(g.n, kTile);
  g.group_m = kGemmGroupM;
  if constexpr (std::is_same<T, __bf16>::value && !BK) {
    // dH and dW on the one-wave-per-SIMD engine from 16 K stages on.  dW is
    // 5-6% faster there at 131072 tokens.  dH alone measures 0.7-1.1% slower
    // (its read-modify-write epilogue, whose stores the next tile's first
    // barrier waits for, costs more than its faster main loop saves), but
    // the whole step is 0.7% faster with it there (the kernels after it run
    // faster), so the step decides.
    if (cdiv(g.k_len, w4::kStageK) >= kW4MinStages) {
      const int64_t tiles = g.m_tiles * g.n_tiles;
      const int64_t p = persistent_blocks();
      const int64_t blocks = tiles < p ? tiles : p;
      if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
      constexpr int kLds = w4::kLdsBytes + w4::kStagingBytes;
      const void* k = reinterpret_cast<const void*>(&gemm_f32out_kernel_w4<AK, Accum>);
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_f32out_kernel_w4<AK, Accum>), dim3((unsigned)blocks),
                         dim3(w4::kThreads), kLds, st, g);
      return hipGetLastError();
    }
  }
  const int64_t blocks = grid_blocks(g.m_tiles * g.n_tiles, stages_of<T>(g.k_len));
  if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
  hipError_t e =
      set_lds<T>(reinterpret_cast<const void*>(&gemm_f32out_kernel<T, AK, BK, Accum>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_f32out_kernel<T, AK, BK, Accum>), dim3((unsigned)blocks),
                     dim3(kThreads), kLdsBytes, st, g);
  return hipGetLastError();
}

// dH[N, H] (+)= G[N, :v_len] . W_s[v_len, H]: M = tokens, N = H, K = strip rows.
template <typename T>
static GemmArgs<T> dh_args(const T* g_strip, int64_t ldg, const T* w_strip, int64_t v_len,
                           int64_t n_tok, int64_t h, float* d_hidden) {
  GemmArgs<T> g{};
  g.a = g_strip; g.lda = ldg; g.a_mn_ext = n_tok; g.a_k_ext = v_len;   // K-contiguous
  g.b = w_strip; g.ldb = h;   g.b_mn_ext = h;     g.b_k_ext = v_len;   // MN-contiguous
  g.k_len = v_len;
  g.c = d_hidden; g.ldc = h; g.m = n_tok; g.n = h;
  g.m_tiles = cdiv(g.m, kTile);
  g.n_tiles = cdiv(g.n, kTile);
  g.group_m = kGemmGroupM;
  return g;
}

// dW_s[v_len, H] = G[:, :v_len]^T . h: M = strip rows, N = H, K = tokens.
template <typename T>
static GemmArgs<T> dw_args(const T* g_strip, int64_t ldg, const T* hidden, int64_t v_len,
                           int64_t n_tok, int64_t h, float* d_weight_strip) {
  GemmArgs<T> g{};
  const int64_t cols = cdiv(v_len, 8) * 8;  // chunk-aligned; the pad columns of G are zero
  g.a = g_strip; g.lda = ldg; g.a_mn_ext = cols; g.a_k_ext = n_tok;    // MN-contiguous
  g.b = hidden;  g.ldb = h;   g.b_mn_ext = h;    g.b_k_ext = n_tok;    // MN-contiguous
  g.k_len = n_tok;
  g.c = d_weight_strip; g.ldc = h; g.m = v_len; g.n = h;
  g.m_tiles = cdiv(g.m, kTile);
  g.n_tiles = cdiv(g.n, kTile);
  g.group_m = kGemmGroupM;
  return g;
}

template <typename T>
hipError_t launch_dh(const T* g_strip, int64_t ldg, const T* w_strip, int64_t v_len, int64_t n_tok,
                     int64_t h, float* d_hidden, int accumulate, hipStream_t st) {
  const GemmArgs<T> g = dh_args(g_strip, ldg, w_strip, v_len, n_tok, h, d_hidden);
  return accumulate ? launch_gemm<T, true, false, true>(g, st)
                    : launch_gemm<T, true, false, false>(g, st);
}

template <typename T>
hipError_t launch_dw(const T* g_strip, int64_t ldg, const T* hidden, int64_t v_len, int64_t n_tok,
                     int64_t h, float* d_weight_strip, int accumulate, hipStream_t st) {
  const GemmArgs<T> g = dw_args(g_strip, ldg, hidden, v_len, n_tok, h, d_weight_strip);
  return accumulate ? launch_gemm<T, false, false, true>(g, st)
                    : launch_gemm<T, false, false, false>(g, st);
}

template <typename T, bool AccumDh, bool AccumDw>
static hipError_t launch_dh_dw_shared(const GemmArgs<T>& dh, const GemmArgs<T>& dw, int64_t split,
                                      int64_t blocks, hipStream_t st) {
  if constexpr (std::is_same<T, __bf16>::value) {
    // on the one-wave-per-SIMD engine when both GEMMs have 16 K stages or more
    if (cdiv(dh.k_len, w4::kStageK) >= kW4MinStages &&
        cdiv(dw.k_len, w4::kStageK) >= kW4MinStages) {
      constexpr int kLds = w4::kLdsBytes + w4::kStagingBytes;
      const void* k = reinterpret_cast<const void*>(&gemm_dh_dw_kernel_w4<AccumDh, AccumDw>);
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_dh_dw_kernel_w4<AccumDh, AccumDw>), dim3((unsigned)blocks),
                         dim3(w4::kThreads), kLds, st, dh, dw, split);
      return hipGetLastError();
    }
  }
  hipError_t e =
      set_lds<T>(reinterpret_cast<const void*>(&gemm_dh_dw_kernel<T, AccumDh, AccumDw>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_dh_dw_kernel<T, AccumDh, AccumDw>), dim3((unsigned)blocks),
                     dim3(kThreads), kLdsBytes, st, dh, dw, split);
  return hipGetLastError();
}

// Stages each compute unit runs (the longest block) when `blocks` blocks share
// `tiles` tiles of `nk` stages.
static int64_t stage_load(int64_t tiles, int64_t nk, int64_t blocks) {
  return cdiv(tiles, blocks) * nk;
}

// Blocks of a shared dH + dW launch that work on dH, or 0 for two launches:
// the split (a multiple of 8) that minimises the longest block's stage count,
// taken only when both GEMMs are persistent (more stages per tile than the
// ring holds) and the shared launch is strictly shorter than two launches.
template <typename T>
int64_t dh_dw_split(int64_t v_len, int64_t n_tok, int64_t h) {
  const int64_t t_dh = cdiv(n_tok, kTile) * cdiv(h, kTile), nk_dh = stages_of<T>(v_len);
  const int64_t t_dw = cdiv(v_len, kTile) * cdiv(h, kTile), nk_dw = stages_of<T>(n_tok);
  const int64_t p = persistent_blocks();
  int64_t best_split = 0, best = stage_load(t_dh, nk_dh, p) + stage_load(t_dw, nk_dw, p);
  if (nk_dh > kStages && nk_dw > kStages) {
    for (int64_t split = kXcds; split < p; split += kXcds) {
      const int64_t a = stage_load(t_dh, nk_dh, split), b = stage_load(t_dw, nk_dw, p - split);
      const int64_t c = a > b ? a : b;
      if (c < best) { best = c; best_split = split; }
    }
  }
  return best_split;
}

template <typename T>
hipError_t launch_dh_dw(const T* g_strip, int64_t ldg, const T* w_strip, const T* hidden,
                        int64_t v_len, int64_t n_tok, int64_t h, float* d_hidden, int acc_dh,
                        float* d_weight_strip, int acc_dw, hipStream_t st) {
  const int64_t best_split = dh_dw_split<T>(v_len, n_tok, h);
  if (best_split == 0) {
    hipError_t e = launch_dh(g_strip, ldg, w_strip, v_len, n_tok, h, d_hidden, acc_dh, st);
    if (e != hipSuccess) return e;
    return launch_dw(g_strip, ldg, hidden, v_len, n_tok, h, d_weight_strip, acc_dw, st);
  }
  const GemmArgs<T> dh = dh_args(g_strip, ldg, w_strip, v_len, n_tok, h, d_hidden);
  const GemmArgs<T> dw = dw_args(g_strip, ldg, hidden, v_len, n_tok, h, d_weight_strip);
  const int64_t p = persistent_blocks();
  if (acc_dh)
    return acc_dw ? launch_dh_dw_shared<T, true, true>(dh, dw, best_split, p, st)
                  : launch_dh_dw_shared<T, true, false>(dh, dw, best_split, p, st);
  return acc_dw ? launch_dh_dw_shared<T, false, true>(dh, dw, best_split, p, st)
                : launch_dh_dw_shared<T, false, false>(dh, dw, best_split, p, st);
}

template <typename T>
hipError_t launch_fused_bwd(const FusedLaunch<T>& L, hipStream_t st) {
  FusedArgs<T> f{};
  f.hidden = L.hidden; f.weight = L.weight; f.targets = L.targets; f.lse = L.lse;
  f.ctrl = L.ctrl; f.N = L.N; f.H = L.H; f.V = L.V; f.ignore_index = L.ignore_index;
  f.g_scratch = L.g_scratch;
  f.dh_dst = L.dh_dst; f.dw_dst = L.dw_dst;
  f.C = L.C; f.tok_per_r = L.tok_per_r; f.voc_per_c = L.voc_per_c;
  f.do_dh = L.do_dh; f.do_dw = L.do_dw;
  const int64_t blocks = L.C * L.R;
  if (!grid_ok(blocks)) return hipErrorInvalidConfiguration;
  hipError_t e = set_lds<T>(reinterpret_cast<const void*>(&fused_bwd_kernel<T>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fused_bwd_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), kLdsBytes, st, f);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, int64_t P, int64_t count, float* out,
                            hipStream_t st) {
  const int64_t threads = cdiv(count, 4);
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, st, parts,
                     P, count, out);
  return hipGetLastError();
}

hipError_t launch_state_init(float* m, float* s, float* zt, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, m, s, zt, n);
  return hipGetLastError();
}

hipError_t launch_fold(const float2* partials, int64_t n_blocks, float* m, float* s, int64_t n,
                       hipStream_t st) {
  hipLaunchKernelGGL(fold_kernel, dim3((unsigned)cdiv(n, 64)), dim3(64 * kFoldWays), 0, st,
                     partials, n_blocks, m, s, n);
  return hipGetLastError();
}

hipError_t launch_state_export(const float* m, const float* s, const float* zt, float* state,
                               int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(state_export_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, m, s, zt,
                     state, n);
  return hipGetLastError();
}

hipError_t launch_state_merge(const float* state, float* m, float* s, float* zt, int64_t n,
                              hipStream_t st) {
  hipLaunchKernelGGL(state_merge_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, state, m,
                     s, zt, n);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* m, const float* s, const float* zt, const int32_t* targets,
                           int64_t n, int32_t ignore_index, int reduction, float* lse,
                           float* row_loss, float* loss, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kReduceThreads), 0, st, m, s, zt, targets, n,
                     ignore_index, reduction, lse, row_loss, loss);
  return hipGetLastError();
}

hipError_t launch_grad_scale(const int32_t* targets, int64_t n, int32_t ignore_index,
                             int reduction, const float* grad_out, Control* ctrl, hipStream_t st) {
  hipLaunchKernelGGL(grad_scale_kernel, dim3(1), dim3(kReduceThreads), 0, st, targets, n,
                     ignore_index, reduction, grad_out, ctrl);
  return hipGetLastError();
}

template hipError_t launch_strip_lse<__bf16>(StripArgs<__bf16>, hipStream_t);
template hipError_t launch_strip_lse<float>(StripArgs<float>, hipStream_t);
template hipError_t launch_strip_grad<__bf16>(StripArgs<__bf16>, hipStream_t);
template hipError_t launch_strip_grad<float>(StripArgs<float>, hipStream_t);
template hipError_t launch_dh<__bf16>(const __bf16*, int64_t, const __bf16*, int64_t, int64_t,
                                      int64_t, float*, int, hipStream_t);
template hipError_t launch_dh<float>(const float*, int64_t, const float*, int64_t, int64_t,
                                     int64_t, float*, int, hipStream_t);
template hipError_t launch_dw<__bf16>(const __bf16*, int64_t, const __bf16*, int64_t, int64_t,
                                      int64_t, float*, int, hipStream_t);
template hipError_t launch_dh_dw<__bf16>(const __bf16*, int64_t, const __bf16*, const __bf16*,
                                         int64_t, int64_t, int64_t, float*, int, float*, int,
                                         hipStream_t);
template hipError_t launch_dh_dw<float>(const float*, int64_t, const float*, const float*, int64_t,
                                        int64_t, int64_t, float*, int, float*, int, hipStream_t);
template hipError_t launch_dw<float>(const float*, int64_t, const float*, int64_t, int64_t,
                                     int64_t, float*, int, hipStream_t);
template int64_t dh_dw_split<__bf16>(int64_t, int64_t, int64_t);
template hipError_t launch_fused_bwd<__bf16>(const FusedLaunch<__bf16>&, hipStream_t);
template hipError_t launch_fused_bwd<float>(const FusedLaunch<float>&, hipStream_t);
template int64_t dh_dw_split<float>(int64_t, int64_t, int64_t);

}  // namespace lce
