// C ABI of the SC library: argument validation (before any HIP call), LDS
// layout, grid sizing and kernel dispatch.  See include/sc.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "sc.h"
#include "sc_internal.h"

namespace {

constexpr int64_t kMaxI32 = 2147483647;
constexpr int kMaxK = 1024;
static_assert(sc::kStaticScratchBytes == (size_t)SC_STATIC_SCRATCH_BYTES,
              "the static workspace size is declared twice");
constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per compute unit

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dtype) { return dtype == SC_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == SC_F32 || d == SC_BF16; }

// c = log2(e) / T (float64, > 0) as an fp32 pair hi + lo with hi < c, so
// that lo > 0: the kernels form z c as fma(z, lo, fma(z, hi, -E)), and for a
// masked logit z = -inf that is -inf only when both products are -inf (with
// lo < 0 the inner -inf meets +inf: NaN).  Rounded to nearest, lo is negative
// for T = 0.6 ... 0.9, for instance.
void split_scale(double c64, float& hi, float& lo) {
  hi = (float)c64;
  if ((double)hi >= c64) hi = std::nextafter(hi, 0.f);
  lo = (float)(c64 - (double)hi);
}

// log2(e) / T as fp32, as float64 and as an fp32 pair (hi + lo).
void set_lm_temperature(sc::LmParams& P, float temperature) {
  P.c64 = 1.4426950408889634 / (double)temperature;
  P.c = (float)P.c64;
  split_scale(P.c64, P.c_hi, P.c_lo);
}

// Shared row-kernel argument checks; fills the geometry part of RowParams.
int check_rows(sc::RowParams& P, const void* logits, bool logits_needed, int logits_dtype,
               int64_t n_rows, int64_t vocab, int64_t row_stride,
               const int32_t* head_ids, int32_t k, const int32_t* sampled,
               float temperature, float* row_stats, int32_t* row_idx) {
  if (!dtype_ok(logits_dtype)) return SC_ERR_ARG;
  if (n_rows < 0 || n_rows > kMaxI32) return SC_ERR_ARG;
  if (vocab < 1 || vocab > kMaxI32 - 64) return SC_ERR_ARG;
  if (row_stride < vocab) return SC_ERR_ARG;
  if (k < 1 || k > kMaxK || (int64_t)k > vocab) return SC_ERR_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SC_ERR_ARG;
  if (!head_ids || !sampled || !row_stats || !row_idx) return SC_ERR_ARG;
  if (logits_needed && !logits) return SC_ERR_ARG;
  if (logits && !aligned(logits, esize(logits_dtype))) return SC_ERR_ARG;
  if (!aligned(head_ids, 4) || !aligned(sampled, 4) || !aligned(row_stats, 4) ||
      !aligned(row_idx, 4))
    return SC_ERR_ARG;
  P.logits = logits;
  P.in_dtype = logits_dtype;
  P.n_rows = n_rows;
  P.vocab = vocab;
  P.row_stride = row_stride;
  P.head_ids = head_ids;
  P.k = k;
  P.sampled = sampled;
  P.temperature = temperature;
  P.c64 = 1.4426950408889634 / (double)temperature;
  split_scale(P.c64, P.c_hi, P.c_lo);
  P.row_stats = row_stats;
  P.row_idx = row_idx;
  return SC_OK;
}

// LDS layout of a row kernel; needs P.vector, P.vocab, P.k set.
int layout(sc::RowParams& P, int kind) {
  const int B = sc::kKindBlock[kind];
  const int64_t N = P.vector ? 16 / (int64_t)esize(P.in_dtype) : 1;
  const int64_t n_full = P.vocab / N;
  const int64_t jmax = (n_full + B - 1) / B;
  P.bm_wpt = (int)std::max<int64_t>(1, (jmax + 31) / 32);
  int hs = 2, hbits = 1;
  while (hs < 2 * P.k) { hs <<= 1; ++hbits; }
  P.hs = hs;
  P.hshift = 32 - hbits;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = (off + bytes + 15) & ~size_t(15); return (int)o; };
  P.off_bitmap = take((size_t)P.bm_wpt * B * 4);
  P.off_hkey = take((size_t)hs * 4);
  P.off_hval = take((size_t)hs * 4);
  P.off_headz = take((size_t)P.k * 4);
  P.off_headp = take((size_t)P.k * 8);
  P.off_headlp = take((size_t)P.k * 8);
  P.off_hout = take((size_t)P.k * 4);
  // marked-vector list: at most k vectors holding recorded ids, the sampled
  // id's vector and the partial last vector
  P.ke = P.k + 2;
  P.off_lval = take((size_t)P.ke * N * 4);
  P.off_lvec = take((size_t)P.ke * 4);
  P.off_lslot = take((size_t)P.ke * N * 2);   // recorded-id slot of each listed element
  P.lds_bytes = off;
  return off <= kMaxLds ? SC_OK : SC_ERR_UNSUPPORTED;
}

bool vector_ok(const void* p, int dtype, int64_t stride) {
  return p == nullptr || (aligned(p, 16) && ((size_t)stride * esize(dtype)) % 16 == 0);
}

int run_rows(sc::RowParams& P, int kind, void* stream) {
  int st = layout(P, kind);
  if (st != SC_OK) return st;
  if (P.n_rows == 0) return SC_OK;
  // One workgroup per row: rows take different times (padding rows return
  // at once, marked-vector lists differ), and the hardware dispatches the
  // next workgroup to whichever slot frees up.  A persistent grid with rows
  // assigned in turn was 2.5% (fused) to 4% (statistics only) slower.
  hipError_t e = sc::launch_row(P, kind, (int)P.n_rows, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int check_center(sc::RowParams& P, const float* head_probs, const float* rollout_logp,
                 const int32_t* resp_idx, const float* advantages, int32_t n_responses,
                 const int64_t* n_valid, float* coef, void* row_out, int out_dtype,
                 int64_t out_stride, int row_mode, int is_mode, float is_lo, float is_hi,
                 int centering, uint32_t* dev_status) {
  if (!head_probs || !resp_idx || !advantages) return SC_ERR_ARG;
  if (is_mode < SC_IS_NONE || is_mode > SC_IS_MIS) return SC_ERR_ARG;
  if (is_mode != SC_IS_NONE) {
    if (!rollout_logp) return SC_ERR_ARG;
    if (!(std::isfinite(is_lo) && std::isfinite(is_hi) && is_lo >= 0.f && is_hi > 0.f &&
          is_lo <= is_hi))
      return SC_ERR_ARG;
  }
  if (n_responses < 0) return SC_ERR_ARG;
  if (row_mode < SC_ROW_DLOGITS || row_mode > SC_ROW_CORRECTION) return SC_ERR_ARG;
  if (row_out) {
    if (!dtype_ok(out_dtype) || out_stride < P.vocab) return SC_ERR_ARG;
    if (!aligned(row_out, esize(out_dtype))) return SC_ERR_ARG;
    if (row_mode == SC_ROW_DLOGITS && !n_valid) return SC_ERR_ARG;
  }
  if (!aligned(head_probs, 4) || !aligned(resp_idx, 4) || !aligned(advantages, 4) ||
      (rollout_logp && !aligned(rollout_logp, 4)) || (coef && !aligned(coef, 4)) ||
      (n_valid && !aligned(n_valid, 8)) || (dev_status && !aligned(dev_status, 4)))
    return SC_ERR_ARG;
  P.head_probs = head_probs;
  P.rollout_logp = rollout_logp;
  P.resp_idx = resp_idx;
  P.advantages = advantages;
  P.n_responses = n_responses;
  P.n_valid = n_valid;
  P.coef = coef;
  P.row_out = row_out;
  P.out_dtype = row_out ? out_dtype : SC_F32;
  P.out_stride = row_out ? out_stride : 0;
  P.row_mode = row_mode;
  P.is_mode = is_mode;
  P.is_lo = is_lo;
  P.is_hi = is_hi;
  P.centering = centering ? 1 : 0;
  P.dev_status = dev_status;
  P.vector = (vector_ok(P.logits, P.in_dtype, P.row_stride) &&
              vector_ok(row_out, P.out_dtype, P.out_stride)) ? 1 : 0;
  return SC_OK;
}

}  // namespace

extern "C" {

int sc_logprobs(const void* logits, int logits_dtype, int64_t n_rows, int64_t vocab,
                int64_t row_stride, const int32_t* head_ids, int32_t k,
                const int32_t* sampled, const int32_t* resp_idx, float temperature,
                float* row_stats, int32_t* row_idx, float* head_logp,
                uint32_t* dev_status, void* stream) {
  sc::RowParams P{};
  int st = check_rows(P, logits, true, logits_dtype, n_rows, vocab, row_stride, head_ids, k,
                      sampled, temperature, row_stats, row_idx);
  if (st != SC_OK) return st;
  if ((resp_idx && !aligned(resp_idx, 4)) || (head_logp && !aligned(head_logp, 4)) ||
      (dev_status && !aligned(dev_status, 4)))
    return SC_ERR_ARG;
  P.resp_idx = resp_idx;
  P.head_logp = head_logp;
  P.dev_status = dev_status;
  P.out_dtype = SC_F32;
  P.vector = vector_ok(logits, logits_dtype, row_stride) ? 1 : 0;
  return run_rows(P, 0, stream);
}

int sc_center(const void* logits, int logits_dtype, int64_t n_rows, int64_t vocab,
              int64_t row_stride, const int32_t* head_ids, const float* head_probs,
              int32_t k, const int32_t* sampled, const float* rollout_logp,
              const int32_t* resp_idx, const float* advantages, int32_t n_responses,
              float temperature, const int64_t* n_valid, float* row_stats,
              int32_t* row_idx, const float* head_logp, float* coef, void* row_out,
              int out_dtype, int64_t out_stride, int row_mode, int is_mode, float is_lo,
              float is_hi, int centering, uint32_t* dev_status, void* stream) {
  sc::RowParams P{};
  int st = check_rows(P, logits, row_out != nullptr, logits_dtype, n_rows, vocab, row_stride,
                      head_ids, k, sampled, temperature, row_stats, row_idx);
  if (st != SC_OK) return st;
  if (!head_logp || !aligned(head_logp, 4)) return SC_ERR_ARG;
  st = check_center(P, head_probs, rollout_logp, resp_idx, advantages, n_responses, n_valid,
                    coef, row_out, out_dtype, out_stride, row_mode, is_mode, is_lo,
                    is_hi, centering, dev_status);
  if (st != SC_OK) return st;
  P.head_logp = const_cast<float*>(head_logp);
  return run_rows(P, 1, stream);
}

int sc_correct(const void* logits, int logits_dtype, int64_t n_rows, int64_t vocab,
               int64_t row_stride, const int32_t* head_ids, const float* head_probs,
               int32_t k, const int32_t* sampled, const float* rollout_logp,
               const int32_t* resp_idx, const float* advantages, int32_t n_responses,
               float temperature, const int64_t* n_valid, float* row_stats,
               int32_t* row_idx, float* head_logp, float* coef, void* row_out,
               int out_dtype, int64_t out_stride, int row_mode, int is_mode, float is_lo,
               float is_hi, int centering, uint32_t* dev_status, void* stream) {
  sc::RowParams P{};
  int st = check_rows(P, logits, true, logits_dtype, n_rows, vocab, row_stride, head_ids, k,
                      sampled, temperature, row_stats, row_idx);
  if (st != SC_OK) return st;
  if (head_logp && !aligned(head_logp, 4)) return SC_ERR_ARG;
  st = check_center(P, head_probs, rollout_logp, resp_idx, advantages, n_responses, n_valid,
                    coef, row_out, out_dtype, out_stride, row_mode, is_mode, is_lo,
                    is_hi, centering, dev_status);
  if (st != SC_OK) return st;
  P.head_logp = head_logp;
  return run_rows(P, 2, stream);
}

int sc_group_norm(const float* rewards, int32_t n_groups, int32_t group_size, int32_t mode,
                  float eps, float* advantages, void* stream) {
  if (!rewards || !advantages || n_groups < 0 || group_size < 1 || group_size > 4096)
    return SC_ERR_ARG;
  if (mode < 0 || mode > 2 || !(std::isfinite(eps) && eps >= 0.f)) return SC_ERR_ARG;
  if ((int64_t)n_groups * group_size > kMaxI32) return SC_ERR_ARG;
  if (!aligned(rewards, 4) || !aligned(advantages, 4)) return SC_ERR_ARG;
  if (n_groups == 0) return SC_OK;
  hipError_t e = sc::launch_group_norm(rewards, n_groups, group_size, mode, eps, advantages,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int sc_count_valid(const int32_t* resp_idx, int64_t n_rows, int64_t* out, int32_t accumulate,
                   void* stream) {
  if (!out || n_rows < 0 || n_rows > kMaxI32 || (n_rows > 0 && !resp_idx)) return SC_ERR_ARG;
  if (!aligned(out, 8) || (resp_idx && !aligned(resp_idx, 4))) return SC_ERR_ARG;
  hipError_t e = sc::launch_count_valid(resp_idx, n_rows, out, accumulate ? 1 : 0,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int sc_batch_sums(const float* row_stats, const int32_t* resp_idx, int64_t n_rows,
                  const int64_t* n_valid, double* batch, int32_t accumulate, void* stream) {
  if (!batch || !n_valid || n_rows < 0 || n_rows > kMaxI32) return SC_ERR_ARG;
  if (n_rows > 0 && (!row_stats || !resp_idx)) return SC_ERR_ARG;
  if (!aligned(batch, 8) || !aligned(n_valid, 8) || (row_stats && !aligned(row_stats, 4)) ||
      (resp_idx && !aligned(resp_idx, 4)))
    return SC_ERR_ARG;
  hipError_t e = sc::launch_batch_sums(row_stats, resp_idx, n_rows, n_valid, batch,
                                       accumulate ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int sc_reference_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > ((int64_t)1 << 40)) return SC_ERR_ARG;
  if (bytes > 0 && (!src || !dst || !aligned(src, 16) || !aligned(dst, 16))) return SC_ERR_ARG;
  if (bytes == 0) return SC_OK;
  hipError_t e = sc::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Fused LM-head statistics
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kLmMaxStride = 4194303;  // tile offsets stay below 2^31 bytes

int lm_splits(int64_t vocab) {
  const int64_t chunks = (vocab + sc::kLmTileV - 1) / sc::kLmTileV;
  return (int)std::min<int64_t>(sc::kLmMaxSplits, chunks);
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// Grid order of the MFMA tile loop (needs P.splits): share the larger
// operand's tiles.  With row tiles as the larger side, the 32 concurrent
// workgroups of an XCD take lm_pt row tiles x lm_sp splits, lm_sp dividing
// the split count: 8 when it can, every split when there are at most 32,
// else the largest divisor below 8.
void lm_order(sc::LmParams& P, int64_t rows, int64_t vocab) {
  P.order = rows > vocab ? 1 : 0;
  int sp = 1;
  if (P.splits % 8 == 0) {
    sp = 8;
  } else if (P.splits <= 32) {
    sp = P.splits;
  } else {
    for (int q = 7; q >= 1; --q)
      if (P.splits % q == 0) { sp = q; break; }
  }
  P.lm_sp = sp;
  P.lm_pt = std::max(1, 32 / sp);
}

// Workspace layout; returns its size and, when P is given, points P's
// workspace arrays into `base`.
size_t lm_workspace(int64_t n, int64_t vocab, int k, sc::LmParams* P, char* base) {
  const int S = lm_splits(vocab);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  const size_t skey = take((size_t)n * k * 8);
  const size_t head_raw = take((size_t)n * k * 4);
  const size_t state = take((size_t)S * n * 16);
  const size_t za = take((size_t)n * 4);
  const size_t scount = take((size_t)n * 4);
  const size_t sa = take((size_t)n * 4);
  const size_t sflags = take((size_t)n * 4);
  if (P && base) {
    P->skey = reinterpret_cast<long long*>(base + skey);
    P->head_raw = reinterpret_cast<float*>(base + head_raw);
    P->state = reinterpret_cast<float4*>(base + state);
    P->za = reinterpret_cast<float*>(base + za);
    P->scount = reinterpret_cast<int32_t*>(base + scount);
    P->sa = reinterpret_cast<int32_t*>(base + sa);
    P->sflags = reinterpret_cast<uint32_t*>(base + sflags);
  }
  return off;
}

// Checks shared by the two LM-head entry points; fills the GEMM geometry.
int check_lm(sc::LmParams& P, const void* hidden, int64_t n_rows, int32_t d,
             int64_t hidden_stride, const void* weight, int64_t vocab, int64_t weight_stride) {
  if (!hidden || !weight) return SC_ERR_ARG;
  if (n_rows < 0 || n_rows > kMaxI32) return SC_ERR_ARG;
  if (vocab < 1 || vocab > kMaxI32 - sc::kLmTileV) return SC_ERR_ARG;
  if (d < 1 || hidden_stride < d || weight_stride < d) return SC_ERR_ARG;
  if (hidden_stride > kLmMaxStride || weight_stride > kLmMaxStride) return SC_ERR_ARG;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || hidden_stride % 8 || weight_stride % 8)
    return SC_ERR_ARG;
  if (d % sc::kLmKStage) return SC_ERR_UNSUPPORTED;
  P.x = static_cast<const uint16_t*>(hidden);
  P.xs = hidden_stride;
  P.w = static_cast<const uint16_t*>(weight);
  P.ws = weight_stride;
  P.n_rows = n_rows;
  P.vocab = vocab;
  P.d = d;
  P.splits = lm_splits(vocab);
  lm_order(P, n_rows, vocab);
  P.n_chunks = (int)((vocab + sc::kLmTileV - 1) / sc::kLmTileV);
  P.n_ptiles = (int)((n_rows + sc::kLmTileP - 1) / sc::kLmTileP);
  return SC_OK;
}

}  // namespace

int64_t sc_lmhead_workspace_size(int64_t n_rows, int64_t vocab, int32_t k) {
  if (n_rows < 0 || n_rows > kMaxI32 || vocab < 1 || vocab > kMaxI32 - sc::kLmTileV)
    return SC_ERR_ARG;
  if (k < 1 || k > kMaxK || (int64_t)k > vocab) return SC_ERR_ARG;
  return (int64_t)lm_workspace(n_rows, vocab, k, nullptr, nullptr);
}

namespace {

// Argument checks of the LM-head statistics entry points (no HIP call).
int check_lmhead_stats(sc::LmParams& P, const void* hidden, int64_t n_rows, int32_t d,
                       int64_t hidden_stride, const void* weight, int64_t vocab,
                       int64_t weight_stride, const int32_t* head_ids, int32_t k,
                       const int32_t* sampled, const int32_t* resp_idx, float temperature,
                       float* row_stats, int32_t* row_idx, float* head_logp,
                       uint32_t* dev_status) {
  int st = check_lm(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride);
  if (st != SC_OK) return st;
  if (k < 1 || k > kMaxK || (int64_t)k > vocab) return SC_ERR_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SC_ERR_ARG;
  if (!head_ids || !sampled || !row_stats || !row_idx) return SC_ERR_ARG;
  if (!aligned(head_ids, 4) || !aligned(sampled, 4) || !aligned(row_stats, 4) ||
      !aligned(row_idx, 4) || (head_logp && !aligned(head_logp, 4)) ||
      (resp_idx && !aligned(resp_idx, 4)) || (dev_status && !aligned(dev_status, 4)))
    return SC_ERR_ARG;
  set_lm_temperature(P, temperature);
  P.head_ids = head_ids;
  P.k = k;
  P.sampled = sampled;
  P.resp_idx = resp_idx;
  P.row_stats = row_stats;
  P.row_idx = row_idx;
  P.head_logp = head_logp;
  P.dev_status = dev_status;
  return SC_OK;
}

}  // namespace

int sc_logprobs_lmhead(const void* hidden, int64_t n_rows, int32_t d, int64_t hidden_stride,
                       const void* weight, int64_t vocab, int64_t weight_stride,
                       const int32_t* head_ids, int32_t k, const int32_t* sampled,
                       const int32_t* resp_idx, float temperature, float* row_stats,
                       int32_t* row_idx, float* head_logp, void* workspace,
                       int64_t workspace_bytes, uint32_t* dev_status, void* stream) {
  sc::LmParams P{};
  int st = check_lmhead_stats(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride,
                              head_ids, k, sampled, resp_idx, temperature, row_stats, row_idx,
                              head_logp, dev_status);
  if (st != SC_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return SC_ERR_ARG;
  const size_t need = lm_workspace(n_rows, vocab, k, nullptr, nullptr);
  if (workspace_bytes < 0 || (size_t)workspace_bytes < need) return SC_ERR_ARG;
  lm_workspace(n_rows, vocab, k, &P, static_cast<char*>(workspace));
  if (n_rows == 0) return SC_OK;
  hipError_t e = sc::launch_lmhead(P, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int sc_logprobs_lmhead_static(const void* hidden, int64_t n_rows, int32_t d,
                              int64_t hidden_stride, const void* weight, int64_t vocab,
                              int64_t weight_stride, const int32_t* head_ids, int32_t k,
                              const int32_t* sampled, const int32_t* resp_idx,
                              float temperature, float* row_stats, int32_t* row_idx,
                              float* head_logp, uint32_t* dev_status, void* stream) {
  sc::LmParams P{};
  int st = check_lmhead_stats(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride,
                              head_ids, k, sampled, resp_idx, temperature, row_stats, row_idx,
                              head_logp, dev_status);
  if (st != SC_OK) return st;
  if (lm_workspace(n_rows, vocab, k, nullptr, nullptr) > sc::kStaticScratchBytes)
    return SC_ERR_TOO_LARGE;
  if (n_rows == 0) return SC_OK;
  void* ws = nullptr;
  if (sc::static_scratch(&ws) != hipSuccess) return SC_ERR_HIP;
  lm_workspace(n_rows, vocab, k, &P, static_cast<char*>(ws));
  hipError_t e = sc::launch_lmhead(P, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int sc_lmhead_logits(const void* hidden, int64_t n_rows, int32_t d, int64_t hidden_stride,
                     const void* weight, int64_t vocab, int64_t weight_stride, float* logits,
                     int64_t logits_stride, void* stream) {
  sc::LmParams P{};
  int st = check_lm(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride);
  if (st != SC_OK) return st;
  if (!logits || !aligned(logits, 4) || logits_stride < vocab) return SC_ERR_ARG;
  P.out = logits;
  P.os = logits_stride;
  P.out_vec = (logits_stride % 4 == 0) && aligned(logits, 16);
  set_lm_temperature(P, 1.f);
  if (n_rows == 0) return SC_OK;
  hipError_t e = sc::launch_lmhead(P, 1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

// ---------------------------------------------------------------------------
// LM-head backward: dLogits recomputed from the forward statistics
// ---------------------------------------------------------------------------
namespace {

int64_t pad64(int64_t x) { return (x + 63) / 64 * 64; }

// Backward workspace: W^T [d, Vp], the chunk's dLogits [chunk, Vp] and their
// transpose [V, chunk_p], the chunk's hidden states transposed [d, chunk_p]
// (Vp, chunk_p: multiples of 64, zero padded, so every GEMM's k extent is a
// whole number of 64-wide stages).
struct BwdLayout {
  int64_t vp, cp;
  size_t wt, dz, dzt, xt, total;
};
// True when the backward's workspace for these sizes would exceed 2^62 bytes
// (its size arithmetic stays far from wrapping below that).
bool bwd_too_large(int64_t chunk, int64_t vocab, int64_t d) {
  const long double vp = (long double)pad64(vocab), cp = (long double)pad64(chunk);
  const long double bytes = 2.0L * ((long double)d * vp + (long double)chunk * vp +
                                    (long double)vocab * cp + (long double)d * cp);
  return bytes > 4611686018427387904.0L;
}

BwdLayout bwd_layout(int64_t chunk, int64_t vocab, int64_t d) {
  BwdLayout L{};
  L.vp = pad64(vocab);
  L.cp = pad64(chunk);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  L.wt = take((size_t)d * L.vp * 2);
  L.dz = take((size_t)chunk * L.vp * 2);
  L.dzt = take((size_t)vocab * L.cp * 2);
  L.xt = take((size_t)d * L.cp * 2);
  L.total = off;
  return L;
}

// C [n, os] = A [m, k] B [n, k]^T through the LM-head MFMA loop (A is its
// vocabulary operand, B its row operand); k a multiple of 64.
hipError_t gemm_nt(const uint16_t* A, int64_t m, int64_t as, const uint16_t* B, int64_t n,
                   int64_t bs, int64_t k, float* out, uint16_t* out16, int64_t os, int accum,
                   hipStream_t s) {
  sc::LmParams G{};
  G.x = B;
  G.xs = bs;
  G.w = A;
  G.ws = as;
  G.n_rows = n;
  G.vocab = m;
  G.d = (int)k;
  G.splits = lm_splits(m);
  lm_order(G, n, m);
  G.n_chunks = (int)((m + sc::kLmTileV - 1) / sc::kLmTileV);
  G.n_ptiles = (int)((n + sc::kLmTileP - 1) / sc::kLmTileP);
  G.out = out;
  G.out16 = out16;
  G.os = os;
  G.out_accum = accum;
  G.out_vec = (os % 4 == 0) && aligned(out16 ? (const void*)out16 : (const void*)out, 16);
  return sc::launch_lmhead(G, 1, s);
}

int check_lm_dz(sc::LmParams& P, const int32_t* head_ids, const float* head_probs, int32_t k,
                const int32_t* sampled, const int32_t* resp_idx, const float* advantages,
                int32_t n_responses, float temperature, const int64_t* n_valid,
                const float* row_stats, const int32_t* row_idx, const float* head_logp,
                int centering) {
  if (k < 1 || k > kMaxK || (int64_t)k > P.vocab) return SC_ERR_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SC_ERR_ARG;
  if (!head_ids || !head_probs || !sampled || !advantages || !n_valid || !row_stats ||
      !row_idx || !head_logp || n_responses < 0)
    return SC_ERR_ARG;
  if (!aligned(head_ids, 4) || !aligned(head_probs, 4) || !aligned(sampled, 4) ||
      !aligned(advantages, 4) || !aligned(n_valid, 8) || !aligned(row_stats, 4) ||
      !aligned(row_idx, 4) || !aligned(head_logp, 4) || (resp_idx && !aligned(resp_idx, 4)))
    return SC_ERR_ARG;
  set_lm_temperature(P, temperature);
  P.temperature = temperature;
  P.head_ids = head_ids;
  P.head_probs = head_probs;
  P.k = k;
  P.sampled = sampled;
  P.resp_idx = resp_idx;
  P.advantages = advantages;
  P.n_responses = n_responses;
  P.n_valid = n_valid;
  P.stats_in = row_stats;
  P.idx_in = row_idx;
  P.head_logp_in = head_logp;
  P.centering = centering ? 1 : 0;
  return SC_OK;
}

// Row slice [r0, r0 + rows) of a dLogits problem.
sc::LmParams lm_slice(const sc::LmParams& P, int64_t r0, int64_t rows) {
  sc::LmParams Q = P;
  Q.x = P.x + r0 * P.xs;
  Q.n_rows = rows;
  Q.n_ptiles = (int)((rows + sc::kLmTileP - 1) / sc::kLmTileP);
  Q.head_ids = P.head_ids + r0 * P.k;
  Q.head_probs = P.head_probs + r0 * P.k;
  Q.sampled = P.sampled + r0;
  Q.resp_idx = P.resp_idx ? P.resp_idx + r0 : nullptr;
  Q.stats_in = P.stats_in + r0 * SC_NSTATS;
  Q.idx_in = P.idx_in + r0 * 2;
  Q.head_logp_in = P.head_logp_in + r0 * P.k;
  return Q;
}

}  // namespace

int sc_lmhead_dlogits(const void* hidden, int64_t n_rows, int32_t d, int64_t hidden_stride,
                      const void* weight, int64_t vocab, int64_t weight_stride,
                      const int32_t* head_ids, const float* head_probs, int32_t k,
                      const int32_t* sampled, const int32_t* resp_idx, const float* advantages,
                      int32_t n_responses, float temperature, const int64_t* n_valid,
                      const float* row_stats, const int32_t* row_idx, const float* head_logp,
                      int centering, void* dlogits, int64_t dlogits_stride, void* stream) {
  sc::LmParams P{};
  int st = check_lm(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride);
  if (st != SC_OK) return st;
  st = check_lm_dz(P, head_ids, head_probs, k, sampled, resp_idx, advantages, n_responses,
                   temperature, n_valid, row_stats, row_idx, head_logp, centering);
  if (st != SC_OK) return st;
  if (!dlogits || !aligned(dlogits, 8) || dlogits_stride < vocab || dlogits_stride % 4)
    return SC_ERR_ARG;
  P.dz = static_cast<uint16_t*>(dlogits);
  P.dzs = dlogits_stride;
  P.dz_cols = vocab;
  if (n_rows == 0) return SC_OK;
  hipError_t e = sc::launch_lmhead(P, 2, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

int64_t sc_lmhead_backward_workspace_size(int64_t chunk_rows, int64_t vocab, int32_t d) {
  if (chunk_rows < 1 || chunk_rows > kMaxI32 || vocab < 1 || vocab > kMaxI32 - sc::kLmTileV ||
      d < 1)
    return SC_ERR_ARG;
  if (bwd_too_large(chunk_rows, vocab, d)) return SC_ERR_UNSUPPORTED;
  return (int64_t)bwd_layout(chunk_rows, vocab, d).total;
}

int sc_lmhead_backward(const void* hidden, int64_t n_rows, int32_t d, int64_t hidden_stride,
                       const void* weight, int64_t vocab, int64_t weight_stride,
                       const int32_t* head_ids, const float* head_probs, int32_t k,
                       const int32_t* sampled, const int32_t* resp_idx, const float* advantages,
                       int32_t n_responses, float temperature, const int64_t* n_valid,
                       const float* row_stats, const int32_t* row_idx, const float* head_logp,
                       int centering, void* d_hidden, int dh_dtype, int64_t dh_stride,
                       float* d_weight, int64_t dw_stride, int accumulate, int64_t chunk_rows,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  sc::LmParams P{};
  int st = check_lm(P, hidden, n_rows, d, hidden_stride, weight, vocab, weight_stride);
  if (st != SC_OK) return st;
  st = check_lm_dz(P, head_ids, head_probs, k, sampled, resp_idx, advantages, n_responses,
                   temperature, n_valid, row_stats, row_idx, head_logp, centering);
  if (st != SC_OK) return st;
  if (!d_hidden || !dtype_ok(dh_dtype) || dh_stride < d || !aligned(d_hidden, esize(dh_dtype)))
    return SC_ERR_ARG;
  if (!d_weight || dw_stride < d || !aligned(d_weight, 4)) return SC_ERR_ARG;
  if (chunk_rows < 1 || chunk_rows > kMaxI32 || !workspace || !aligned(workspace, 256))
    return SC_ERR_ARG;
  if (bwd_too_large(chunk_rows, vocab, d)) return SC_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout(chunk_rows, vocab, d);
  if (L.cp > kLmMaxStride || L.vp > kLmMaxStride) return SC_ERR_UNSUPPORTED;
  if (workspace_bytes < 0 || (size_t)workspace_bytes < L.total) return SC_ERR_ARG;
  if (n_rows == 0) return SC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.wt);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  uint16_t* dzt = reinterpret_cast<uint16_t*>(ws + L.dzt);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + L.xt);
  P.dz = dz;
  P.dzs = L.vp;
  P.dz_cols = L.vp;
  // W^T [d, Vp], ids past the vocabulary zero
  hipError_t e = sc::launch_transpose_bf16(P.w, vocab, d, weight_stride, wt, L.vp, L.vp, s);
  if (e != hipSuccess) return SC_ERR_HIP;
  for (int64_t r0 = 0; r0 < n_rows; r0 += chunk_rows) {
    const int64_t rows = std::min<int64_t>(chunk_rows, n_rows - r0);
    const sc::LmParams Q = lm_slice(P, r0, rows);
    // the chunk's dLogits [rows, Vp] (columns >= V zero) and their transpose
    // [V, rows_p] from the same kernel, the hidden states' transpose
    // [d, rows_p] (rows_p = rows rounded up to 64, columns >= rows zero)
    const int64_t rp = pad64(rows);
    sc::LmParams Qd = Q;
    Qd.dzt = dzt;
    Qd.dzts = L.cp;
    Qd.dzt_cols = rp;
    if ((e = sc::launch_lmhead(Qd, 2, s)) != hipSuccess) return SC_ERR_HIP;
    if ((e = sc::launch_transpose_bf16(Q.x, rows, d, hidden_stride, xt, rp, L.cp, s)) !=
        hipSuccess)
      return SC_ERR_HIP;
    // dW [V, d] (+)= dZ^T X:  C[v][j] = sum_r dZ^T[v][r] X^T[j][r], r < rows_p
    e = gemm_nt(xt, d, L.cp, dzt, vocab, L.cp, rp, d_weight, nullptr, dw_stride,
                (accumulate || r0 > 0) ? 1 : 0, s);
    if (e != hipSuccess) return SC_ERR_HIP;
    // dHidden rows [rows, d] = dZ W:  C[r][j] = sum_v dZ[r][v] W^T[j][v]
    char* dh = static_cast<char*>(d_hidden) + r0 * dh_stride * (int64_t)esize(dh_dtype);
    e = gemm_nt(wt, d, L.vp, dz, rows, L.vp, L.vp,
                dh_dtype == SC_BF16 ? nullptr : reinterpret_cast<float*>(dh),
                dh_dtype == SC_BF16 ? reinterpret_cast<uint16_t*>(dh) : nullptr, dh_stride, 0,
                s);
    if (e != hipSuccess) return SC_ERR_HIP;
  }
  return SC_OK;
}

int sc_record(const void* logits, int logits_dtype, int64_t n_rows, int64_t vocab,
              int64_t row_stride, float temperature, int32_t k, const int32_t* sampled,
              int32_t* head_ids, float* head_probs, float* sampled_logp,
              uint32_t* dev_status, void* stream) {
  if (!dtype_ok(logits_dtype)) return SC_ERR_ARG;
  if (n_rows < 0 || n_rows > kMaxI32) return SC_ERR_ARG;
  if (vocab < 1 || vocab > kMaxI32 - 64 || row_stride < vocab) return SC_ERR_ARG;
  if (k < 1 || k > kMaxK || (int64_t)k > vocab) return SC_ERR_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SC_ERR_ARG;
  if (!logits || !head_ids || !head_probs) return SC_ERR_ARG;
  if (!aligned(logits, esize(logits_dtype)) || !aligned(head_ids, 4) ||
      !aligned(head_probs, 4) || (sampled && !aligned(sampled, 4)) ||
      (sampled_logp && !aligned(sampled_logp, 4)) || (dev_status && !aligned(dev_status, 4)))
    return SC_ERR_ARG;
  if (sampled_logp && !sampled) return SC_ERR_ARG;
  sc::RecParams P{};
  P.logits = logits;
  P.in_dtype = logits_dtype;
  P.vector = vector_ok(logits, logits_dtype, row_stride) ? 1 : 0;
  P.n_rows = n_rows;
  P.vocab = vocab;
  P.row_stride = row_stride;
  P.c64 = 1.4426950408889634 / (double)temperature;
  P.c = (float)P.c64;
  P.k = k;
  P.sampled = sampled;
  P.head_ids = head_ids;
  P.head_probs = head_probs;
  P.sampled_logp = sampled_logp;
  P.dev_status = dev_status;
  if (sc::record_lds_bytes(k) > kMaxLds) return SC_ERR_UNSUPPORTED;
  if (n_rows == 0) return SC_OK;
  hipError_t e = sc::launch_record(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SC_OK : SC_ERR_HIP;
}

const char* sc_status_string(int status) {
  switch (status) {
    case SC_OK: return "SC_OK";
    case SC_ERR_ARG: return "SC_ERR_ARG: invalid argument";
    case SC_ERR_UNSUPPORTED: return "SC_ERR_UNSUPPORTED: outside what the library supports";
    case SC_ERR_HIP: return "SC_ERR_HIP: HIP runtime call or kernel launch failed";
    case SC_ERR_TOO_LARGE:
      return "SC_ERR_TOO_LARGE: the request needs more than the static workspace of "
             "sc_logprobs_lmhead_static (SC_STATIC_SCRATCH_BYTES per GPU)";
    default: return "unknown sc_status";
  }
}

int sc_version(void) { return 101; }

}  // extern "C"
