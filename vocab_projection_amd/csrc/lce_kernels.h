// lce_kernels.h - internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

// Scalars kept at the head of the workspace.
struct Control {
  float grad_scale;   // d loss / d row_loss of a non-ignored row
  float pad0;
  long long n_valid;  // non-ignored rows
};

// One vocabulary strip against all tokens.
template <typename T>
struct StripArgs {
  const T* hidden;        // [N, H]
  const T* weight_strip;  // [v_len, H], row 0 = vocabulary row v_begin
  const int32_t* targets; // [N]
  int64_t N, H;
  int64_t v_begin, v_len;
  int32_t ignore_index;
  int64_t m_tiles, n_tiles, group_m;  // tile order, set by the launcher
  // forward
  float2* partials;       // [ceil(v_len / 128), N]
  float* z_target;        // [N]
  // backward
  const float* lse;       // [N]
  const Control* ctrl;
  T* g_strip;             // [N, ldg]
  int64_t ldg;
};

template <typename T>
struct GemmArgs {
  const T* a; int64_t lda, a_mn_ext, a_k_ext;
  const T* b; int64_t ldb, b_mn_ext, b_k_ext;
  int64_t k_len;
  float* c; int64_t ldc, m, n;
  int64_t m_tiles, n_tiles, group_m;  // tile order, set by the launcher
};

template <typename T> hipError_t launch_strip_lse(StripArgs<T> a, hipStream_t st);
template <typename T> hipError_t launch_strip_grad(StripArgs<T> a, hipStream_t st);
template <typename T>
hipError_t launch_dh(const T* g_strip, int64_t ldg, const T* w_strip, int64_t v_len, int64_t n_tok,
                     int64_t h, float* d_hidden, int accumulate, hipStream_t st);
template <typename T>
hipError_t launch_dw(const T* g_strip, int64_t ldg, const T* hidden, int64_t v_len, int64_t n_tok,
                     int64_t h, float* d_weight_strip, int accumulate, hipStream_t st);
// Both of the above; in one launch that shares the compute units between them
// when that is shorter than two launches.
template <typename T>
hipError_t launch_dh_dw(const T* g_strip, int64_t ldg, const T* w_strip, const T* hidden,
                        int64_t v_len, int64_t n_tok, int64_t h, float* d_hidden, int acc_dh,
                        float* d_weight_strip, int acc_dw, hipStream_t st);

// Blocks of the shared launch that work on dH, or 0 when launch_dh_dw issues
// two launches (dH, then dW) for a strip of v_len rows.
template <typename T> int64_t dh_dw_split(int64_t v_len, int64_t n_tok, int64_t h);

// The backward without a strip buffer (fused_bwd_kernel): a grid of C x R
// blocks, block r * C + c taking token tiles [r tok_per_r, + tok_per_r) and
// vocabulary tiles [c voc_per_c, + voc_per_c); dH partials per vocabulary
// group at dh_dst + c N H, dW partials per token group at dw_dst + r V H.
template <typename T>
struct FusedLaunch {
  const T* hidden;
  const T* weight;
  const int32_t* targets;
  const float* lse;
  const Control* ctrl;
  int64_t N, H, V;
  int32_t ignore_index;
  T* g_scratch;  // C R blocks x 256 x 256 elements
  float* dh_dst;
  float* dw_dst;
  int64_t C, R, tok_per_r, voc_per_c;
  int do_dh, do_dw;
};
template <typename T> hipError_t launch_fused_bwd(const FusedLaunch<T>& L, hipStream_t st);
// out[k] = sum over p of parts[p * count + k], p in order; count % 4 == 0.
hipError_t launch_sum_parts(const float* parts, int64_t P, int64_t count, float* out,
                            hipStream_t st);

hipError_t launch_state_init(float* m, float* s, float* zt, int64_t n, hipStream_t st);
hipError_t launch_fold(const float2* partials, int64_t n_blocks, float* m, float* s, int64_t n,
                       hipStream_t st);
hipError_t launch_state_export(const float* m, const float* s, const float* zt, float* state,
                               int64_t n, hipStream_t st);
hipError_t launch_state_merge(const float* state, float* m, float* s, float* zt, int64_t n,
                              hipStream_t st);
hipError_t launch_finalize(const float* m, const float* s, const float* zt, const int32_t* targets,
                           int64_t n, int32_t ignore_index, int reduction, float* lse,
                           float* row_loss, float* loss, hipStream_t st);
hipError_t launch_grad_scale(const int32_t* targets, int64_t n, int32_t ignore_index,
                             int reduction, const float* grad_out, Control* ctrl, hipStream_t st);

}  // namespace lce
