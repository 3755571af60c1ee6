// Host harness: the library's C ABI (sc_api.cpp) and its row and LM-head
// kernels built for the CPU (emulated, see hip/hip_runtime.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
//   harness abi                      argument checks and workspace arithmetic
//   harness rows CASES SEED [OUT]    seeded random shapes through sc_logprobs,
//                                    sc_correct and sc_center; with OUT, each
//                                    case's sc_correct inputs and outputs
//   harness lmhead OUT N V D K CHUNK the LM-head entry points on one seeded
//                                    problem; inputs and outputs written to OUT
//                                    for a comparison with the oracle
//   harness record OUT CASES SEED    seeded random shapes through sc_record;
//                                    inputs and outputs written to OUT
//   harness replay N V D CHUNK       sc_lmhead_backward alone (bounds only)
//
// Every mode ends with "HARNESS OK" when no entry point failed and no buffer
// access fell outside its resource; a sanitizer finding aborts the process.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <random>
#include <string>

#include "sc.h"
#include "sc_internal.h"

static int failures = 0;

#define EXPECT(call, want)                                                         \
  do {                                                                             \
    const int got_ = (call);                                                       \
    if (got_ != (want)) {                                                          \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call,  \
              got_, (int)(want));                                                  \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Argument checks: every rejection happens before a launch, and the size
// arithmetic of the workspaces holds at the extremes.
// ---------------------------------------------------------------------------
static void abi_checks() {
  alignas(256) static unsigned char buf[1 << 16];
  void* p = buf;
  int32_t* ip = reinterpret_cast<int32_t*>(buf);
  float* fp = reinterpret_cast<float*>(buf);
  int64_t* lp = reinterpret_cast<int64_t*>(buf);
  void* odd = buf + 1;
  // sc_logprobs
  EXPECT(sc_logprobs(p, SC_BF16, 0, 100, 100, ip, 4, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_OK);
  EXPECT(sc_logprobs(nullptr, SC_BF16, 3, 100, 100, ip, 4, ip, nullptr, 1.f, fp, ip, fp,
                     nullptr, nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, 7, 3, 100, 100, ip, 4, ip, nullptr, 1.f, fp, ip, fp, nullptr, nullptr),
         SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, 100, 99, ip, 4, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, 100, 100, ip, 0, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, 100, 100, ip, 1025, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, 100, 100, ip, 4, ip, nullptr, 0.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, 100, 100, ip, 4, ip, nullptr, NAN, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(odd, SC_BF16, 3, 100, 100, ip, 4, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, -1, 100, 100, ip, 4, ip, nullptr, 1.f, fp, ip, fp, nullptr,
                     nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_BF16, 3, (int64_t)1 << 40, (int64_t)1 << 40, ip, 4, ip, nullptr, 1.f,
                     fp, ip, fp, nullptr, nullptr), SC_ERR_ARG);
  EXPECT(sc_logprobs(p, SC_F32, 3, (1 << 30), (1 << 30), ip, 4, ip, nullptr, 1.f, fp, ip, fp,
                     nullptr, nullptr), SC_ERR_UNSUPPORTED);          // LDS bitmap too large
  // sc_center / sc_correct
  EXPECT(sc_center(nullptr, SC_BF16, 0, 100, 100, ip, fp, 4, ip, nullptr, ip, fp, 2, 1.f, lp,
                   fp, ip, fp, fp, nullptr, SC_BF16, 100, SC_ROW_DLOGITS, SC_IS_NONE, 0.5f, 2.f,
                   1, nullptr, nullptr), SC_OK);              // no row: logits not needed
  EXPECT(sc_center(nullptr, SC_BF16, 3, 100, 100, ip, fp, 4, ip, nullptr, ip, fp, 2, 1.f, lp,
                   fp, ip, fp, fp, p, SC_BF16, 100, SC_ROW_DLOGITS, SC_IS_NONE, 0.5f, 2.f, 1,
                   nullptr, nullptr), SC_ERR_ARG);            // a row needs the logits
  EXPECT(sc_correct(p, SC_BF16, 3, 100, 100, ip, fp, 4, ip, nullptr, ip, fp, 2, 1.f, nullptr,
                    fp, ip, fp, fp, p, SC_BF16, 100, SC_ROW_DLOGITS, SC_IS_NONE, 0.5f, 2.f, 1,
                    nullptr, nullptr), SC_ERR_ARG);           // dLogits need n_valid
  EXPECT(sc_correct(p, SC_BF16, 3, 100, 100, ip, fp, 4, ip, nullptr, ip, fp, 2, 1.f, lp, fp, ip,
                    fp, fp, p, SC_BF16, 100, 9, SC_IS_NONE, 0.5f, 2.f, 1, nullptr, nullptr),
         SC_ERR_ARG);
  EXPECT(sc_correct(p, SC_BF16, 3, 100, 100, ip, fp, 4, ip, nullptr, ip, fp, 2, 1.f, lp, fp, ip,
                    fp, fp, p, SC_BF16, 100, SC_ROW_DLOGITS, SC_IS_MIS, 0.5f, 2.f, 1, nullptr,
                    nullptr), SC_ERR_ARG);                    // MIS needs rollout log p
  EXPECT(sc_correct(p, SC_BF16, 3, 100, 100, ip, fp, 4, ip, fp, ip, fp, 2, 1.f, lp, fp, ip, fp,
                    fp, p, SC_BF16, 100, SC_ROW_DLOGITS, SC_IS_MIS, 3.f, 2.f, 1, nullptr,
                    nullptr), SC_ERR_ARG);                    // lo > hi
  // small kernels
  EXPECT(sc_group_norm(fp, 0, 4, 0, 1e-6f, fp, nullptr), SC_OK);
  EXPECT(sc_group_norm(fp, 4, 0, 0, 1e-6f, fp, nullptr), SC_ERR_ARG);
  EXPECT(sc_group_norm(fp, 1 << 20, 1 << 20, 0, 1e-6f, fp, nullptr), SC_ERR_ARG);
  EXPECT(sc_count_valid(ip, -1, lp, 0, nullptr), SC_ERR_ARG);
  EXPECT(sc_batch_sums(fp, ip, 5, nullptr, reinterpret_cast<double*>(buf), 0, nullptr),
         SC_ERR_ARG);
  // LM-head workspace sizes: monotone, and no overflow at the largest sizes
  const int64_t w1 = sc_lmhead_workspace_size(1000, 248320, 128);
  const int64_t w2 = sc_lmhead_workspace_size(2000, 248320, 128);
  if (!(w1 > 0 && w2 > w1)) { fprintf(stderr, "lmhead workspace sizes %lld %lld\n",
                                      (long long)w1, (long long)w2); ++failures; }
  EXPECT((int)(sc_lmhead_workspace_size(2147483647, 2147483647 - 256, 1024) > 0), 1);
  EXPECT((int)sc_lmhead_workspace_size(-1, 100, 4), SC_ERR_ARG);
  EXPECT((int)(sc_lmhead_backward_workspace_size(8192, 248320, 4096) > 0), 1);
  EXPECT((int)sc_lmhead_backward_workspace_size(2147483647, 2147483647 - 256, 4096),
         SC_ERR_UNSUPPORTED);                                 // beyond 2^62 bytes
  EXPECT(sc_logprobs_lmhead(p, 300, 256, 256, p, 1000, 256, ip, 16, ip, nullptr, 1.f, fp, ip,
                            nullptr, p, 100, nullptr, nullptr), SC_ERR_ARG);   // workspace short
  EXPECT(sc_logprobs_lmhead(p, 300, 200, 200, p, 1000, 200, ip, 16, ip, nullptr, 1.f, fp, ip,
                            nullptr, p, 1 << 30, nullptr, nullptr), SC_ERR_UNSUPPORTED);
  EXPECT(sc_logprobs_lmhead_static(p, 11882, 4096, 4096, p, 248320, 4096, ip, 128, ip, nullptr,
                                   1.f, fp, ip, nullptr, nullptr, nullptr), SC_ERR_TOO_LARGE);
  EXPECT(sc_logprobs_lmhead_static(p, 0, 4096, 4096, p, 248320, 4096, ip, 128, ip, nullptr, 1.f,
                                   fp, ip, nullptr, nullptr, nullptr), SC_OK);
  EXPECT(sc_lmhead_backward(p, 10, 64, 64, p, 100, 64, ip, fp, 4, ip, ip, fp, 1, 1.f, lp, fp, ip,
                            fp, 1, p, SC_F32, 64, fp, 64, 0, 0, p, 1 << 30, nullptr),
         SC_ERR_ARG);                                          // chunk_rows 0
  EXPECT(sc_reference_copy(p, p, 24, nullptr), SC_ERR_ARG);
  EXPECT(sc_reference_copy(odd, p, 16, nullptr), SC_ERR_ARG);
  printf("abi checks done, %d failures\n", failures);
}

// ---------------------------------------------------------------------------
// Row kernels: seeded random shapes (bounds, barriers, sanitizers).
// ---------------------------------------------------------------------------
// With `out`, each case's sc_correct inputs and outputs are appended to that
// file (before sc_center writes its own) for a comparison with the oracle.
static void rows(int cases, uint64_t seed0, const char* out = nullptr) {
  FILE* rec = out ? fopen(out, "wb") : nullptr;
  if (out && !rec) { ++failures; return; }
  for (int c = 0; c < cases; ++c) {
    std::mt19937_64 g(seed0 * 1000003 + c);
    auto U = [&](int lo, int hi) { return lo + (int)(g() % (uint64_t)(hi - lo + 1)); };
    const int n = U(1, 5);
    const int V = (g() % 4 == 0) ? U(1, 40) : U(41, 9000);
    const int K = std::min(V, (g() % 5 == 0) ? U(200, 1024) : U(1, 160));
    const int dtype = g() % 2 ? SC_BF16 : SC_F32;
    const int out_dtype = g() % 2 ? SC_BF16 : SC_F32;
    const int mode = U(0, 2);
    const int pad = g() % 3 == 0 ? U(1, 9) : 0;
    const int64_t stride = V + pad;
    const float T = (g() % 3 == 0) ? 0.7f : 1.f;
    const float scales[5] = {0.1f, 1.f, 3.f, 8.f, 30.f};
    std::normal_distribution<float> nd(0.f, scales[U(0, 4)]);
    std::vector<float> zf((size_t)n * stride, 0.f);
    for (int r = 0; r < n; ++r)
      for (int v = 0; v < V; ++v) zf[(size_t)r * stride + v] = nd(g);
    std::vector<int32_t> ids((size_t)n * K), sampled(n), resp(n);
    std::vector<float> q((size_t)n * K), rlp(n);
    for (int r = 0; r < n; ++r) {
      std::vector<int> perm(V);
      std::iota(perm.begin(), perm.end(), 0);
      if (g() % 2) {  // consecutive ids (sharing vectors)
        const int s0 = U(0, V - K);
        for (int k = 0; k < K; ++k) perm[k] = s0 + k;
        std::shuffle(perm.begin(), perm.begin() + K, g);
      } else {
        for (int k = 0; k < K; ++k) std::swap(perm[k], perm[k + g() % (V - k)]);
      }
      for (int k = 0; k < K; ++k) {
        ids[(size_t)r * K + k] = perm[k];
        q[(size_t)r * K + k] = (g() % 4 == 0 ? 1.0f : 0.9f) / K;
      }
      sampled[r] = (g() % 2) ? ids[(size_t)r * K + (g() % K)] : (int)(g() % V);
      resp[r] = (g() % 5 == 0) ? -1 : r;
      rlp[r] = -0.5f;
      const int err = U(0, 12);  // data errors and special rows
      if (err == 0) ids[(size_t)r * K] = V;
      if (err == 1 && K > 1) ids[(size_t)r * K + 1] = ids[(size_t)r * K];
      if (err == 2) sampled[r] = -3;
      if (err == 3) zf[(size_t)r * stride + U(0, V - 1)] = -INFINITY;
      if (err == 4) for (int v = 0; v < V; v += 3) zf[(size_t)r * stride + v] = -INFINITY;
      if (err == 5) zf[(size_t)r * stride + U(0, V - 1)] = NAN;
      if (err == 6) for (int v = 0; v < V; ++v) zf[(size_t)r * stride + v] = 1.5f;
    }
    std::vector<uint16_t> zb(zf.size());
    for (size_t i = 0; i < zf.size(); ++i) zb[i] = to_bf16(zf[i]);
    std::vector<float> adv(n);
    for (auto& a : adv) a = nd(g);
    int64_t nv = n;
    std::vector<float> stats((size_t)n * SC_NSTATS), hl((size_t)n * K), coef((size_t)n * K);
    std::vector<int32_t> idx((size_t)n * 2);
    std::vector<uint16_t> out16((size_t)n * stride);
    std::vector<float> out32((size_t)n * stride);
    void* logits = dtype == SC_BF16 ? (void*)zb.data() : (void*)zf.data();
    void* outp = out_dtype == SC_BF16 ? (void*)out16.data() : (void*)out32.data();
    uint32_t status = 0;
    EXPECT(sc_logprobs(logits, dtype, n, V, stride, ids.data(), K, sampled.data(), resp.data(), T,
                       stats.data(), idx.data(), hl.data(), &status, nullptr), SC_OK);
    EXPECT(sc_correct(logits, dtype, n, V, stride, ids.data(), q.data(), K, sampled.data(),
                      rlp.data(), resp.data(), adv.data(), n, T, &nv, stats.data(), idx.data(),
                      hl.data(), coef.data(), outp, out_dtype, stride, mode, SC_IS_NONE, 0.5f,
                      2.f, 1, &status, nullptr), SC_OK);
    if (rec) {
      const int32_t hdr[7] = {n, V, K, (int32_t)stride, dtype, out_dtype, mode};
      fwrite(hdr, 4, 7, rec);
      fwrite(&T, 4, 1, rec);
      fwrite(zf.data(), 4, zf.size(), rec);           // the fp32 logits (bf16 input: rounded below)
      fwrite(ids.data(), 4, ids.size(), rec);
      fwrite(q.data(), 4, q.size(), rec);
      fwrite(sampled.data(), 4, n, rec);
      fwrite(resp.data(), 4, n, rec);
      fwrite(rlp.data(), 4, n, rec);
      fwrite(adv.data(), 4, n, rec);
      fwrite(&nv, 8, 1, rec);
      fwrite(stats.data(), 4, stats.size(), rec);
      fwrite(idx.data(), 4, idx.size(), rec);
      fwrite(hl.data(), 4, hl.size(), rec);
      fwrite(coef.data(), 4, coef.size(), rec);
      if (out_dtype == SC_BF16) fwrite(out16.data(), 2, out16.size(), rec);
      else fwrite(out32.data(), 4, out32.size(), rec);
    }
    EXPECT(sc_center(logits, dtype, n, V, stride, ids.data(), q.data(), K, sampled.data(),
                     rlp.data(), resp.data(), adv.data(), n, T, &nv, stats.data(), idx.data(),
                     hl.data(), coef.data(), outp, out_dtype, stride, mode, SC_IS_NONE, 0.5f, 2.f,
                     1, &status, nullptr), SC_OK);
    // the centering alone: with the logits (read at the recorded and sampled
    // ids only) and without them
    EXPECT(sc_center(logits, dtype, n, V, stride, ids.data(), q.data(), K, sampled.data(),
                     rlp.data(), resp.data(), adv.data(), n, T, &nv, stats.data(), idx.data(),
                     hl.data(), coef.data(), nullptr, out_dtype, stride, mode, SC_IS_NONE, 0.5f,
                     2.f, 1, &status, nullptr), SC_OK);
    EXPECT(sc_center(nullptr, dtype, n, V, stride, ids.data(), q.data(), K, sampled.data(),
                     rlp.data(), resp.data(), adv.data(), n, T, &nv, stats.data(), idx.data(),
                     hl.data(), coef.data(), nullptr, out_dtype, stride, mode, SC_IS_NONE, 0.5f,
                     2.f, 1, &status, nullptr), SC_OK);
    printf("rows case %d: n=%d V=%d K=%d in=%d out=%d mode=%d pad=%d T=%g status %u\n", c, n, V,
           K, dtype, out_dtype, mode, pad, T, status);
  }
  if (rec) fclose(rec);
}

// ---------------------------------------------------------------------------
// Rollout-side record: seeded random shapes (ties, equal rows that take the
// exact fallback, masks, a NaN row, K past 256, strides), each case's inputs
// and outputs written to `out` for a comparison with the oracle.
// ---------------------------------------------------------------------------
static void record(int cases, uint64_t seed0, const char* out) {
  FILE* rec = fopen(out, "wb");
  if (!rec) { ++failures; return; }
  for (int c = 0; c < cases; ++c) {
    std::mt19937_64 g(seed0 * 7919 + c);
    auto U = [&](int lo, int hi) { return lo + (int)(g() % (uint64_t)(hi - lo + 1)); };
    const int n = U(1, 4);
    const int V = (g() % 5 == 0) ? U(1, 40) : (g() % 4 == 0 ? U(9000, 20000) : U(41, 9000));
    const int K = std::min(V, (g() % 4 == 0) ? U(257, 1024) : U(1, 200));
    const int dtype = g() % 2 ? SC_BF16 : SC_F32;
    const int pad = g() % 3 == 0 ? U(1, 9) : 0;
    const int64_t stride = V + pad;
    const float T = (g() % 3 == 0) ? 0.7f : ((g() % 2) ? 1.3f : 1.f);
    const int with_sampled = g() % 4 != 0;
    const float scales[5] = {0.1f, 1.f, 3.f, 8.f, 30.f};
    std::vector<float> zf((size_t)n * stride, 0.f);
    std::vector<int32_t> sampled(n);
    for (int r = 0; r < n; ++r) {
      float* z = zf.data() + (size_t)r * stride;
      std::normal_distribution<float> nd(U(0, 3) == 0 ? 2.f : 0.f, scales[U(0, 4)]);
      for (int v = 0; v < V; ++v) z[v] = nd(g);
      const int kind = U(0, 9);
      if (kind == 0) for (int v = 0; v < V; ++v) z[v] = 0.5f;                      // all equal
      if (kind == 1) for (int v = 0; v < V; ++v) z[v] = std::round(z[v] * 4.f) / 4.f;   // ties
      if (kind == 2) for (int v = 0; v < V; v += 3) z[v] = -INFINITY;              // masked
      if (kind == 3) z[U(0, V - 1)] = NAN;                                         // flagged
      if (kind == 4) for (int v = 0; v < V; ++v) z[v] = (v % 7 == 0) ? 1.f : -1.f;  // two levels
      sampled[r] = (int)(g() % V);
    }
    std::vector<uint16_t> zb(zf.size());
    for (size_t i = 0; i < zf.size(); ++i) zb[i] = to_bf16(zf[i]);
    const void* logits = dtype == SC_BF16 ? (const void*)zb.data() : (const void*)zf.data();
    std::vector<int32_t> ids((size_t)n * K, -7);
    std::vector<float> probs((size_t)n * K, -7.f), lp(n, -7.f);
    uint32_t status = 0;
    EXPECT(sc_record(logits, dtype, n, V, stride, T, K, with_sampled ? sampled.data() : nullptr,
                     ids.data(), probs.data(), with_sampled ? lp.data() : nullptr, &status,
                     nullptr), SC_OK);
    const int32_t hdr[6] = {n, V, K, (int32_t)stride, dtype, with_sampled};
    fwrite(hdr, 4, 6, rec);
    fwrite(&T, 4, 1, rec);
    fwrite(zf.data(), 4, zf.size(), rec);
    fwrite(sampled.data(), 4, n, rec);
    fwrite(ids.data(), 4, ids.size(), rec);
    fwrite(probs.data(), 4, probs.size(), rec);
    fwrite(lp.data(), 4, n, rec);
    printf("record case %d: n=%d V=%d K=%d in=%d pad=%d T=%g sampled=%d status %u\n", c, n, V,
           K, dtype, pad, T, with_sampled, status);
  }
  fclose(rec);
}

// ---------------------------------------------------------------------------
// LM-head entry points on one seeded problem.
// ---------------------------------------------------------------------------
struct LmProblem {
  int n, V, d, K;
  std::vector<uint16_t> x, w;
  std::vector<int32_t> ids, sampled, resp;
  std::vector<float> q, adv;
  int64_t n_valid;
};

static LmProblem lm_problem(int n, int V, int d, int K, uint64_t seed) {
  LmProblem P{n, V, d, K};
  std::mt19937_64 g(seed);
  std::normal_distribution<float> nd(0.f, 1.f);
  P.x.resize((size_t)n * d);
  P.w.resize((size_t)V * d);
  for (auto& e : P.x) e = to_bf16(nd(g));
  for (auto& e : P.w) e = to_bf16(0.1f * nd(g));
  P.ids.resize((size_t)n * K);
  P.q.resize((size_t)n * K);
  P.sampled.resize(n);
  P.resp.resize(n);
  const int n_resp = 4, per = (n + n_resp - 1) / n_resp;
  P.n_valid = 0;
  std::vector<int> perm(V);
  for (int r = 0; r < n; ++r) {
    std::iota(perm.begin(), perm.end(), 0);
    for (int k = 0; k < K; ++k) std::swap(perm[k], perm[k + g() % (V - k)]);
    for (int k = 0; k < K; ++k) {
      P.ids[(size_t)r * K + k] = perm[k];
      P.q[(size_t)r * K + k] = 0.8f / K;
    }
    P.sampled[r] = (g() % 2) ? perm[g() % K] : (int)(g() % V);
    P.resp[r] = (r % per >= per - 3) ? -1 : r / per;
    P.n_valid += P.resp[r] >= 0;
  }
  P.adv = {0.8f, -0.6f, 0.3f, -0.5f};
  return P;
}

template <class T> static void put(FILE* f, const std::vector<T>& v) {
  fwrite(v.data(), sizeof(T), v.size(), f);
}

static void lmhead(const char* out_path, int n, int V, int d, int K, int chunk) {
  LmProblem P = lm_problem(n, V, d, K, 77);
  const float T = 1.f;
  std::vector<float> z((size_t)n * V), stats((size_t)n * SC_NSTATS, -7.f),
      hl((size_t)n * K, -7.f), coef((size_t)n * K, -7.f);
  std::vector<int32_t> idx((size_t)n * 2, -9);
  EXPECT(sc_lmhead_logits(P.x.data(), n, d, d, P.w.data(), V, d, z.data(), V, nullptr), SC_OK);
  const int64_t ws = sc_lmhead_workspace_size(n, V, K);
  std::vector<unsigned char> wsp((size_t)ws + 256);
  void* wsa = reinterpret_cast<void*>(((uintptr_t)wsp.data() + 255) & ~(uintptr_t)255);
  uint32_t status = 0;
  EXPECT(sc_logprobs_lmhead(P.x.data(), n, d, d, P.w.data(), V, d, P.ids.data(), K,
                            P.sampled.data(), P.resp.data(), T, stats.data(), idx.data(),
                            hl.data(), wsa, ws, &status, nullptr), SC_OK);
  int64_t nv = P.n_valid;
  EXPECT(sc_center(nullptr, SC_BF16, n, V, V, P.ids.data(), P.q.data(), K, P.sampled.data(),
                   nullptr, P.resp.data(), P.adv.data(), 4, T, &nv, stats.data(), idx.data(),
                   hl.data(), coef.data(), nullptr, SC_BF16, V, SC_ROW_DLOGITS, SC_IS_NONE, 0.5f,
                   2.f, 1, &status, nullptr), SC_OK);
  const int64_t dzs = (V + 3) / 4 * 4;
  std::vector<uint16_t> dz((size_t)n * dzs, 0x7777);
  EXPECT(sc_lmhead_dlogits(P.x.data(), n, d, d, P.w.data(), V, d, P.ids.data(), P.q.data(), K,
                           P.sampled.data(), P.resp.data(), P.adv.data(), 4, T, &nv,
                           stats.data(), idx.data(), hl.data(), 1, dz.data(), dzs, nullptr),
         SC_OK);
  std::vector<float> dh((size_t)n * d, -7.f), dw((size_t)V * d, 7.f);
  const int64_t bws = sc_lmhead_backward_workspace_size(chunk, V, d);
  std::vector<unsigned char> bwsp((size_t)bws + 256);
  void* bwa = reinterpret_cast<void*>(((uintptr_t)bwsp.data() + 255) & ~(uintptr_t)255);
  EXPECT(sc_lmhead_backward(P.x.data(), n, d, d, P.w.data(), V, d, P.ids.data(), P.q.data(), K,
                            P.sampled.data(), P.resp.data(), P.adv.data(), 4, T, &nv,
                            stats.data(), idx.data(), hl.data(), 1, dh.data(), SC_F32, d,
                            dw.data(), d, 0, chunk, bwa, bws, nullptr), SC_OK);
  FILE* f = fopen(out_path, "wb");
  const int hdr[6] = {n, V, d, K, chunk, (int)dzs};
  fwrite(hdr, 4, 6, f);
  put(f, P.x); put(f, P.w); put(f, P.ids); put(f, P.q); put(f, P.sampled); put(f, P.resp);
  put(f, P.adv);
  fwrite(&P.n_valid, 8, 1, f);
  put(f, z); put(f, stats); put(f, idx); put(f, hl); put(f, dz); put(f, dh); put(f, dw);
  fwrite(&status, 4, 1, f);
  fclose(f);
  printf("lmhead n=%d V=%d d=%d K=%d chunk=%d: status %u\n", n, V, d, K, chunk, status);
}

static void replay(int n, int V, int d, int chunk) {
  const int K = 8;
  LmProblem P = lm_problem(n, V, d, K, 91);
  std::vector<float> stats((size_t)n * SC_NSTATS, 0.f), hl((size_t)n * K, -3.f);
  std::vector<int32_t> idx((size_t)n * 2, -1);
  for (int r = 0; r < n; ++r) {
    stats[(size_t)r * SC_NSTATS + SC_STAT_LSE] = 4.f;
    stats[(size_t)r * SC_NSTATS + SC_STAT_RHO] = 1.f;
    stats[(size_t)r * SC_NSTATS + SC_STAT_S] = 1.f;
    stats[(size_t)r * SC_NSTATS + SC_STAT_WEIGHT] = 1.f;
  }
  int64_t nv = P.n_valid;
  std::vector<float> dh((size_t)n * d), dw((size_t)V * d);
  const int64_t bws = sc_lmhead_backward_workspace_size(chunk, V, d);
  std::vector<unsigned char> bwsp((size_t)bws + 256);
  void* bwa = reinterpret_cast<void*>(((uintptr_t)bwsp.data() + 255) & ~(uintptr_t)255);
  EXPECT(sc_lmhead_backward(P.x.data(), n, d, d, P.w.data(), V, d, P.ids.data(), P.q.data(), K,
                            P.sampled.data(), P.resp.data(), P.adv.data(), 4, 1.f, &nv,
                            stats.data(), idx.data(), hl.data(), 1, dh.data(), SC_F32, d,
                            dw.data(), d, 0, chunk, bwa, bws, nullptr), SC_OK);
  printf("replay sc_lmhead_backward n=%d V=%d d=%d chunk_rows=%d workspace %lld bytes\n", n, V,
         d, chunk, (long long)bws);
}

int main(int argc, char** argv) {
  const std::string mode = argc > 1 ? argv[1] : "";
  if (mode == "abi") {
    abi_checks();
  } else if (mode == "rows" && argc > 3) {
    rows(atoi(argv[2]), (uint64_t)atoll(argv[3]), argc > 4 ? argv[4] : nullptr);
  } else if (mode == "lmhead" && argc > 7) {
    lmhead(argv[2], atoi(argv[3]), atoi(argv[4]), atoi(argv[5]), atoi(argv[6]), atoi(argv[7]));
  } else if (mode == "record" && argc > 4) {
    record(atoi(argv[3]), (uint64_t)atoll(argv[4]), argv[2]);
  } else if (mode == "replay" && argc > 5) {
    replay(atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5]));
  } else {
    fprintf(stderr, "usage: see the header of harness.cpp\n");
    return 2;
  }
  printf("buffer accesses out of range: %ld loads (prefetch past a row), %ld stores\n",
         emu::oob_loads, emu::oob_stores);
  if (failures || emu::oob_stores) {
    printf("HARNESS FAILED\n");
    return 1;
  }
  printf("HARNESS OK\n");
  return 0;
}
