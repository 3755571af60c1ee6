// Internal interface between the C ABI (sc_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sc {

constexpr int kRowBlock = 512;  // threads per workgroup of the row kernels

// Everything a row kernel needs, passed by value.
struct RowParams {
  const void* logits;
  int in_dtype;          // 0 fp32, 1 bf16
  int vector;            // 1: 16-byte vector path; 0: scalar path
  int64_t n_rows, vocab, row_stride;
  const int32_t* head_ids;
  const float* head_probs;
  int32_t k;
  const int32_t* sampled;
  const float* rollout_logp;
  const int32_t* resp_idx;
  const float* advantages;
  int32_t n_responses;
  float temperature;
  float c;               // log2(e) / T
  const int64_t* n_valid;
  float* row_stats;
  int32_t* row_idx;
  float* head_logp;
  float* coef;
  void* row_out;
  int out_dtype;
  int64_t out_stride;
  int row_mode;
  uint32_t* dev_status;
  // LDS layout (bytes into dynamic shared memory)
  int hs, hshift, bm_wpt, ke;
  int off_bitmap, off_hkey, off_hval, off_headz, off_headp, off_hout;
  int off_entvec, off_entval, off_entperm;
  size_t lds_bytes;
};

hipError_t launch_row(const RowParams& P, int kind, int grid, hipStream_t s);
hipError_t launch_group_norm(const float* r, int n_groups, int G, int mode,
                             float eps, float* adv, hipStream_t s);
hipError_t launch_count_valid(const int32_t* resp, int64_t n, int64_t* out,
                              int acc, hipStream_t s);
hipError_t launch_batch_sums(const float* st, const int32_t* resp, int64_t n,
                             const int64_t* n_valid, double* batch, int acc,
                             hipStream_t s);

}  // namespace sc
