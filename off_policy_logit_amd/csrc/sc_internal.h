// Internal interface between the C ABI (sc_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sc {

// Launch shape of each row kernel (compile-time; overridable for sweeps):
// threads per workgroup, 16-byte vectors per thread per tile, and the
// occupancy target (waves per SIMD, which caps VGPRs at 512 / value).  The
// grid has one workgroup per row.
#ifndef SC_STATS_BLOCK
#define SC_STATS_BLOCK 256
#endif
#ifndef SC_STATS_TILE
#define SC_STATS_TILE 4
#endif
#ifndef SC_STATS_WAVES
#define SC_STATS_WAVES 3
#endif
#ifndef SC_CENTER_BLOCK
#define SC_CENTER_BLOCK 256
#endif
#ifndef SC_CENTER_TILE
#define SC_CENTER_TILE 4
#endif
#ifndef SC_CENTER_WAVES
#define SC_CENTER_WAVES 3
#endif
#ifndef SC_FUSED_BLOCK
#define SC_FUSED_BLOCK 256
#endif
#ifndef SC_FUSED_TILE
#define SC_FUSED_TILE 8
#endif
#ifndef SC_FUSED_WAVES
#define SC_FUSED_WAVES 2
#endif
constexpr int kKindBlock[3] = {SC_STATS_BLOCK, SC_CENTER_BLOCK, SC_FUSED_BLOCK};

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
  double c64;            // log2(e) / T
  float c_hi, c_lo;      // c64 = c_hi + c_lo (c_hi = c64 rounded to fp32)
  const int64_t* n_valid;
  float* row_stats;
  int32_t* row_idx;
  float* head_logp;
  float* coef;
  void* row_out;
  int out_dtype;
  int64_t out_stride;
  int row_mode;
  int is_mode;           // sc_is_mode
  float is_lo, is_hi;    // MIS interval / TIS cap
  int centering;         // 0: centering term dropped
  uint32_t* dev_status;
  // LDS layout (bytes into dynamic shared memory)
  int hs, hshift, bm_wpt, ke;
  int off_bitmap, off_hkey, off_hval, off_headz, off_headp, off_headlp, off_hout;
  int off_lval, off_lvec, off_lslot;
  size_t lds_bytes;
};

hipError_t launch_row(const RowParams& P, int kind, int grid, hipStream_t s);

// Fused LM-head statistics (sc_logprobs_lmhead / sc_lmhead_logits): tile of
// 256 vocabulary ids x 256 rows, k stages of 64, at most 256 vocabulary splits.
constexpr int kLmTileV = 256;
constexpr int kLmTileP = 256;
constexpr int kLmKStage = 64;
constexpr int kLmMaxSplits = 256;

struct LmParams {
  const uint16_t* x;     // hidden states, bf16 [n_rows, d], row stride xs
  int64_t xs;
  const uint16_t* w;     // vocabulary projection, bf16 [vocab, d], row stride ws
  int64_t ws;
  int64_t n_rows, vocab;
  int d;
  float c;               // log2(e) / T (fp32)
  double c64;            // log2(e) / T
  float c_hi, c_lo;      // c64 = c_hi + c_lo (c_hi = c64 rounded to fp32)
  int splits, n_chunks, n_ptiles;
  int order;             // 0: row tiles vary fastest over the grid, 1: XCD groups
  int lm_pt, lm_sp;      // order 1: row tiles x splits per XCD group (lm_sp divides splits)
  const int32_t* head_ids;
  int32_t k;
  const int32_t* sampled;
  const int32_t* resp_idx;
  // workspace
  long long* skey;       // [n_rows, k] sorted (id << 32 | slot)
  int32_t* scount;       // [n_rows] keys to use (0: padding or data error)
  int32_t* sa;           // [n_rows] sampled id, -1 when nothing is captured
  uint32_t* sflags;      // [n_rows] data-error bits found by the stage kernel
  float4* state;         // [splits, n_rows] (max, tail sum, entropy sum, argmax)
  float* za;             // [n_rows] logit of the sampled id
  float* head_raw;       // [n_rows, k] logits of the recorded ids
  // dLogits recomputation (sc_lmhead_dlogits / sc_lmhead_backward)
  const float* head_probs;
  const float* advantages;
  int32_t n_responses;
  const int64_t* n_valid;
  float temperature;
  int centering;
  const float* stats_in;     // row statistics from sc_logprobs_lmhead + sc_center
  const int32_t* idx_in;     // row_idx (a_slot in column 1)
  const float* head_logp_in;
  uint16_t* dz;              // bf16 [n_rows, dzs]
  int64_t dzs;
  int64_t dz_cols;           // columns [vocab, dz_cols) of dz are written as 0
  uint16_t* dzt;             // optional transpose: bf16 [vocab, dzts], columns
  int64_t dzts;              //   [n_rows, dzt_cols) written as 0
  int64_t dzt_cols;
  // outputs of the store mode (logits check, or C = A B^T of the backward)
  float* out;            // fp32 [n_rows, os], or
  uint16_t* out16;       // bf16 [n_rows, os]
  int64_t os;
  int out_accum;         // fp32 out: add to it
  int out_vec;           // 16-byte aligned rows: vector stores
  float* row_stats;
  int32_t* row_idx;
  float* head_logp;
  uint32_t* dev_status;
};

// Static workspace of sc_logprobs_lmhead_static (bytes per GPU).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
// Its device address on the current device (looked up once per device).
hipError_t static_scratch(void** ptr);

// mode 0: statistics (stage, main, finalize); 1: fp32 logits; 2: bf16 dLogits
// (main, then the recorded / sampled ids).
hipError_t launch_lmhead(const LmParams& P, int mode, hipStream_t s);

// bf16 transpose: dst [cols, rpad] (row stride ds) = src [rows, cols]^T (row
// stride ss); dst columns [rows, rpad) are written as 0.
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t rows, int64_t cols, int64_t ss,
                                 uint16_t* dst, int64_t rpad, int64_t ds, hipStream_t s);

// Rollout-side record (sc_record): top-k of the rollout softmax per row.
struct RecParams {
  const void* logits;
  int in_dtype;          // 0 fp32, 1 bf16
  int vector;            // 1: 16-byte vector path
  int64_t n_rows, vocab, row_stride;
  float c;               // log2(e) / T (fp32)
  double c64;            // log2(e) / T
  int32_t k;
  const int32_t* sampled;
  int32_t* head_ids;
  float* head_probs;
  float* sampled_logp;
  uint32_t* dev_status;
  int cap;               // per-wave candidate buffer (set by the launcher)
};
size_t record_lds_bytes(int k);
hipError_t launch_record(RecParams P, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_group_norm(const float* r, int n_groups, int G, int mode,
                             float eps, float* adv, hipStream_t s);
hipError_t launch_count_valid(const int32_t* resp, int64_t n, int64_t* out,
                              int acc, hipStream_t s);
hipError_t launch_batch_sums(const float* st, const int32_t* resp, int64_t n,
                             const int64_t* n_valid, double* batch, int acc,
                             hipStream_t s);

}  // namespace sc
