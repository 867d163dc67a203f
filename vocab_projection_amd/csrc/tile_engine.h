// tile_engine.h - one 256x256 MFMA tile of C = A . B^T on gfx950 (CDNA4).
//
// A block of 256 threads (four wave64s in a 2x2 grid, each owning a 128x128
// sub-tile) walks K in stages of 128 bytes per row: 64 bf16 or 32 f32
// elements.  Each stage of both operands is staged in LDS (64 KiB), double
// buffered (128 KiB of the 160 KiB per CU), and read back as 16-byte
// fragments that feed v_mfma_f32_32x32x16_bf16 (bf16) or four
// v_mfma_f32_32x32x2f32 (f32), accumulating in fp32.
//
// Operands may be stored K-contiguous (element (mn, k) at base[mn*ld + k]) or
// MN-contiguous (element (mn, k) at base[k*ld + mn]).  Either way the LDS
// copy is K-contiguous: 256 rows of eight 16-byte chunks, the chunk index
// XOR-swizzled by the row so that both the fragment reads (32 rows, same
// chunk) and the stores of the transposing loader (8 rows apart) hit distinct
// banks.  MN-contiguous stages are transposed in registers on the way to LDS.
//
// Out-of-range rows and K positions are loaded as zeros, so the tile needs
// no masking in its inner loop; epilogues mask what they write.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kTile = 256;           // block tile along M and along N
constexpr int kWaveTile = 128;       // wave sub-tile along M and along N
constexpr int kThreads = 256;        // four waves
constexpr int kChunks = 8;           // 16-byte K chunks per row per stage
constexpr int kRowBytes = kChunks * 16;
constexpr int kOperandBytes = kTile * kRowBytes;    // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kOperandBytes;       // A and B
constexpr int kLdsBytes = 2 * kStageBytes;           // double buffered: 128 KiB

template <typename T> struct Elem;
template <> struct Elem<__bf16> { static constexpr int kPerChunk = 8; };
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };

// Physical chunk of logical chunk c in LDS row r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ uint32_t lds_off(int r, int c) {
  return (uint32_t)(r * kRowBytes + swz(r, c) * 16);
}

// ---------------------------------------------------------------------------
// Stage loaders: global -> registers (load), registers -> LDS (store).
// ---------------------------------------------------------------------------

// K-contiguous operand.  Thread t copies chunk (t & 7) of rows (t >> 3) + 32 i.
template <typename T>
struct LoadK {
  u32x4_t v[8];
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int64_t mn0,
                                       int64_t mn_ext, int64_t k0, int64_t k_ext, int tid) {
    const int c = tid & 7;
    const int64_t k = k0 + (int64_t)c * Elem<T>::kPerChunk;
    const bool kok = k < k_ext;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t mn = mn0 + (tid >> 3) + 32 * i;
      if (kok && mn < mn_ext) {
        v[i] = *reinterpret_cast<const u32x4_t*>(base + mn * ld + k);
      } else {
        v[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(r, c)) = v[i];
    }
  }
};

// MN-contiguous operand.
template <typename T> struct LoadMN;

// bf16: thread t loads an 8 (k) x 8 (mn) block: mn chunk (t & 31), k rows
// 8 (t >> 5) .. +8, and transposes it so that each LDS row (one mn) receives
// 8 consecutive k values.  mn_ext must be a multiple of 8.
template <>
struct LoadMN<__bf16> {
  u32x4_t v[8];
  __device__ __forceinline__ void load(const __bf16* __restrict__ base, int64_t ld, int64_t mn0,
                                       int64_t mn_ext, int64_t k0, int64_t k_ext, int tid) {
    const int64_t mn = mn0 + (int64_t)(tid & 31) * 8;
    const bool mok = mn < mn_ext;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t k = k0 + (tid >> 5) * 8 + r;
      if (mok && k < k_ext) {
        v[r] = *reinterpret_cast<const u32x4_t*>(base + k * ld + mn);
      } else {
        v[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int mb = tid & 31;
    const int kc = tid >> 5;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      // element m of k-row r sits in dword m/2 of v[r], low half if m is even
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = v[2 * j][m >> 1];
        const uint32_t y = v[2 * j + 1][m >> 1];
        o[j] = (m & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      *reinterpret_cast<u32x4_t*>(lds + lds_off(mb * 8 + m, kc)) = o;
    }
  }
};

// f32: thread t loads two 4 (k) x 4 (mn) blocks: mn chunk (t & 63), k chunks
// (t >> 6) and (t >> 6) + 4.  mn_ext must be a multiple of 4.
template <>
struct LoadMN<float> {
  u32x4_t v[8];
  __device__ __forceinline__ void load(const float* __restrict__ base, int64_t ld, int64_t mn0,
                                       int64_t mn_ext, int64_t k0, int64_t k_ext, int tid) {
    const int64_t mn = mn0 + (int64_t)(tid & 63) * 4;
    const bool mok = mn < mn_ext;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t k = k0 + ((tid >> 6) + 4 * b) * 4 + r;
        if (mok && k < k_ext) {
          v[4 * b + r] = *reinterpret_cast<const u32x4_t*>(base + k * ld + mn);
        } else {
          v[4 * b + r] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int mb = tid & 63;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kc = (tid >> 6) + 4 * b;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4_t o{v[4 * b + 0][m], v[4 * b + 1][m], v[4 * b + 2][m], v[4 * b + 3][m]};
        *reinterpret_cast<u32x4_t*>(lds + lds_off(mb * 4 + m, kc)) = o;
      }
    }
  }
};

template <typename T, bool KContig> struct Loader;
template <typename T> struct Loader<T, true> { typedef LoadK<T> type; };
template <typename T> struct Loader<T, false> { typedef LoadMN<T> type; };

// Operand in global memory.  For a K-contiguous operand, mn_ext bounds the
// rows and k_ext the columns; for an MN-contiguous one, the reverse.
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;
  int64_t mn_ext;
  int64_t k_ext;
};

// ---------------------------------------------------------------------------
// MFMA on one 16-byte fragment pair.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <>
struct Mfma<__bf16> {
  __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  // The four floats of a fragment are four successive K steps of 32x32x2; the
  // two lane halves supply the two K values of each step.  A and B use the
  // same assignment, so every product pairs equal K.
  __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    // Copy each element to a scalar before the bit cast: a bit cast of a
    // vector-element lvalue reads element 0 whatever the index.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ua = a[q];
      const uint32_t ub = b[q];
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, ua),
                                               __builtin_bit_cast(float, ub), c, 0, 0, 0);
    }
    return c;
  }
};

// Accumulators of one wave: 4 x 4 MFMA tiles of 32 x 32.
// Element (mi, ni, e) of lane l sits at tile row
//   wm*128 + mi*32 + (e/4)*8 + (l/32)*4 + e%4   and column  wn*128 + ni*32 + l%32.
struct Acc {
  f32x16_t c[4][4];
};

__device__ __forceinline__ int acc_row(int mi, int e, int lane) {
  return mi * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}

// C[m0:m0+256, n0:n0+256] = sum_k A[m, k] B[n, k] over k in [0, k_len).
template <typename T, bool AK, bool BK>
__device__ __forceinline__ void tile_mainloop(const Operand<T>& A, const Operand<T>& B,
                                              int64_t m0, int64_t n0, int64_t k_len, char* lds,
                                              Acc& acc) {
  constexpr int kPer = Elem<T>::kPerChunk;
  constexpr int64_t kStageK = (int64_t)kChunks * kPer;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.c[i][j] = f32x16_t{};

  typename Loader<T, AK>::type la;
  typename Loader<T, BK>::type lb;
  const int64_t nk = (k_len + kStageK - 1) / kStageK;

  la.load(A.base, A.ld, m0, A.mn_ext, 0, A.k_ext, tid);
  lb.load(B.base, B.ld, n0, B.mn_ext, 0, B.k_ext, tid);
  la.store(lds, tid);
  lb.store(lds + kOperandBytes, tid);
  __syncthreads();

  const int frow_a = wm * kWaveTile + (lane & 31);
  const int frow_b = wn * kWaveTile + (lane & 31);
  const int fhalf = lane >> 5;

  for (int64_t kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * kStageBytes;
    char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k0 = (kt + 1) * kStageK;
      la.load(A.base, A.ld, m0, A.mn_ext, k0, A.k_ext, tid);
      lb.load(B.base, B.ld, n0, B.mn_ext, k0, B.k_ext, tid);
    }
#pragma unroll
    for (int ks = 0; ks < kChunks / 2; ++ks) {
      const int ch = 2 * ks + fhalf;
      u32x4_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = *reinterpret_cast<const u32x4_t*>(cur + lds_off(frow_a + 32 * i, ch));
        fb[i] = *reinterpret_cast<const u32x4_t*>(cur + kOperandBytes + lds_off(frow_b + 32 * i, ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc.c[i][j] = Mfma<T>::run(fa[i], fb[j], acc.c[i][j]);
    }
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + kOperandBytes, tid);
    }
    __syncthreads();
  }
}

}  // namespace lce
