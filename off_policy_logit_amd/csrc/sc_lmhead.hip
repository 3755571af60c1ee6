// Fused LM-head statistics of the SC correction for gfx950.
//
// In the trainer step of the Score Centering page (section "Score
// Centering") the policy is evaluated on every vocabulary id at the rollout's
// temperature, and log-probabilities are read at the recorded ids H and at
// the sampled id a.  Here the logits z = X W^T (X: final hidden states [n, d],
// W: vocabulary projection [V, d], both bf16) are produced tile by tile by
// bf16 MFMA with fp32 accumulation and consumed in the same kernel by the
// per-row online softmax statistics, so the [n, V] logits never reach HBM.
// (The page's SC worker has no fused LM-head path; this is an addition with
// the same outputs as the unfused statistics pass.)
//
// Three kernels:
//   k_lm_stage     per row: validate and sort the recorded ids (id, slot).
//   k_lm_main      per (256-row tile, vocabulary split): MFMA GEMM over d in
//                  64-wide k stages, double-buffered through LDS; after each
//                  256-id vocabulary chunk the epilogue folds the 256 x 256
//                  logit tile into per-row running (max, tail sum, entropy
//                  sum, argmax) and captures the logits at H and at a.
//   k_lm_finalize  per row: merge the split states in a fixed order, add the
//                  recorded ids, write the same statistics as sc_logprobs.
// k_lm_main<1> instead stores the logit tile (a check of the GEMM with the
// identical accumulation order; with other operands it is the plain GEMM
// C = A B^T of the backward, fp32 or bf16, optionally added to C);
// k_lm_main<2> recomputes the logits and
// writes the bf16 dLogits of the SC step loss, alpha p_v, for every id, and
// k_lm_dz_fix then writes the recorded and sampled ids (the backward pass:
// dLogits for a bounded chunk of rows, consumed by the dHidden and dW GEMMs).
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "sc.h"
#include "sc_device.h"
#include "sc_internal.h"

#include <mutex>

namespace sc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTV = kLmTileV;           // vocabulary ids per chunk (MFMA M)
constexpr int kTP = kLmTileP;           // rows per tile (MFMA N)
constexpr int kKB = kLmKStage;          // k per stage
#ifndef SC_LM_WAVE_ROWS
#define SC_LM_WAVE_ROWS 64
#endif
constexpr int kWR = SC_LM_WAVE_ROWS;    // rows per wave (kWR / 32 MFMA column blocks)
constexpr int kB = 2 * (kLmTileP / kWR) * 64;   // threads: 2 (vocab halves) x kTP / kWR waves
constexpr int kPitch = kKB * 2 + 16;    // LDS bytes per tile row (bank rotation)
constexpr int kBuf = kTV * kPitch;      // one operand buffer
// Hit words of the chunk, 8 per row at a row stride of 9 words: the 32 rows
// a wave's lanes read at once fall in 32 different banks.
constexpr int kBmS = 9;
constexpr int kOffBm = 4 * kBuf;        // [kTP][kBmS] hit words of the chunk
constexpr int kOffBeg = kOffBm + kTP * kBmS * 4;
constexpr int kLds = kOffBeg + kTP * 4;
static_assert(kTV == 256 && kTP == 256 && kKB == 64, "tile shape is fixed");
static_assert(kLds <= 160 * 1024, "LDS budget");

constexpr int kNoIdx = 0x7fffffff;
constexpr double kLn2d = 0.6931471805599453;

SC_DEV int lm_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

SC_DEV float scale2(float x, int k) { return ldexpf(x, k); }
SC_DEV double scale2(double x, int k) { return ldexp(x, k); }

// Merge running state (m, s, hy, am) with (m2, s2, h2, am2).  s is a sum of
// 2^(z c - E(m)) over ids whose logits are at most m, with the integer
// reference E(m) = ref_exp(m), and hy the sum of those terms times their
// exponents z c - E(m); moving a state to a larger reference multiplies s by
// a power of two (and subtracts the shift times s from hy first): exact.
template <typename F>
SC_DEV void lm_merge(float& m, F& s, F& hy, int& am, float m2, F s2, F h2, int am2,
                     float c_hi) {
  const float M = fmaxf(m, m2);
  const float EM = ref_exp(M, c_hi);
  const float D1 = EM - ref_exp(m, c_hi), D2 = EM - ref_exp(m2, c_hi);
  const int k1 = (int)fminf(D1, 2048.f), k2 = (int)fminf(D2, 2048.f);
  const F t1 = scale2(hy - (F)D1 * s, -k1), t2 = scale2(h2 - (F)D2 * s2, -k2);
  am = (m2 > m || (m2 == m && am2 < am)) ? am2 : am;
  s = scale2(s, -k1) + scale2(s2, -k2);
  hy = t1 + t2;
  m = M;
}

// ---------------------------------------------------------------------------
// Stage: one workgroup per row.  Sorted keys (id << 32 | slot) of the recorded
// ids, the sampled id and the data-error flags.  A padding row or a row with
// an error gets no keys and sampled id -1, so the main kernel captures nothing
// for it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lm_stage(LmParams P) {
  __shared__ long long key[1024];
  __shared__ uint32_t sh_fl;
  const int t = threadIdx.x;
  const int64_t p = blockIdx.x;
  const int K = P.k;
  const int resp = P.resp_idx ? P.resp_idx[p] : 0;
  if (resp < 0) {
    if (t == 0) { P.scount[p] = 0; P.sa[p] = -1; P.sflags[p] = 0u; }
    return;
  }
  int P2 = 2;
  while (P2 < K) P2 <<= 1;
  if (t == 0) sh_fl = 0u;
  __syncthreads();
  uint32_t fl = 0;
  for (int i = t; i < P2; i += 256) {
    long long kv = 0x7fffffffffffffffll;
    if (i < K) {
      const int32_t id = P.head_ids[p * K + i];
      if (id < 0 || id >= P.vocab) fl |= SC_DEV_BAD_ID;
      kv = (long long)(((unsigned long long)(uint32_t)id << 32) | (uint32_t)i);
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int k2 = 2; k2 <= P2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P2; i += 256) {
        const int ij = i ^ j;
        if (ij > i) {
          const long long x = key[i], y = key[ij];
          const bool up = (i & k2) == 0;
          if ((x > y) == up) { key[i] = y; key[ij] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i + 1 < K; i += 256)
    if ((key[i] >> 32) == (key[i + 1] >> 32)) fl |= SC_DEV_DUP_ID;
  const int32_t a = P.sampled[p];
  if (t == 0 && (a < 0 || a >= P.vocab)) fl |= SC_DEV_BAD_SAMPLED;
  if (fl) atomicOr(&sh_fl, fl);
  __syncthreads();
  const uint32_t f = sh_fl;
  for (int i = t; i < K; i += 256) P.skey[p * K + i] = key[i];
  if (t == 0) {
    P.scount[p] = f ? 0 : K;
    P.sa[p] = f ? -1 : a;
    P.sflags[p] = f;
  }
}

// ---------------------------------------------------------------------------
// Main: GEMM tile loop with the statistics (or store) epilogue.
// ---------------------------------------------------------------------------
// Per-row factors of the dLogits row (Score Centering loss, global token
// mean): scale = -A wt / (T N_valid) and the off-head factor alpha =
// -scale (rho + 1 - S) (centering) or -scale; zero for padding rows, NaN for
// rows whose statistics are NaN or whose response index is out of range.
SC_DEV void lm_row_factors(const LmParams& P, int64_t p, double& scale, double& alpha) {
  const int resp = P.resp_idx ? P.resp_idx[p] : 0;
  if (resp < 0) { scale = 0.0; alpha = 0.0; return; }
  if (resp >= P.n_responses) { scale = alpha = (double)__builtin_nanf(""); return; }
  const float* st = P.stats_in + p * SC_NSTATS;
  scale = -(double)P.advantages[resp] * (double)st[SC_STAT_WEIGHT] /
          ((double)P.temperature * (double)P.n_valid[0]);
  alpha = P.centering ? -scale * ((double)st[SC_STAT_RHO] + 1.0 - (double)st[SC_STAT_S])
                      : -scale;
}

template <int MODE>
__global__ __launch_bounds__(kB) void k_lm_main(LmParams P) {
  constexpr bool STORE = MODE != 0;
  extern __shared__ __align__(16) unsigned char lds[];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wv = w & 1, wp = w >> 1;   // wave's vocabulary half, row quarter
  const int h = l >> 5, lc = l & 31;

  // Work item.  Workgroups are dispatched in index order, round-robin over
  // the 8 XCDs (blockIdx mod 8), so the ~256 resident at a time take
  // consecutive indices.
  //  order 0 (W, the vocabulary-side operand, is the larger one): row tiles
  //    vary fastest, so the resident blocks cover a few consecutive splits
  //    (runs of 256-id chunks) for every row tile and each W chunk is read by
  //    all row tiles at about the same time (one XCD's row tiles through its
  //    L2, the XCDs through the memory-side cache); a block lives only a few
  //    chunks, so the blocks sharing a chunk stay in step.
  //  order 1 (the row-side operand is the larger one): each XCD's group of
  //    lm_pt x lm_sp concurrent workgroups covers lm_pt row tiles x lm_sp
  //    splits, so every chunk is read by lm_pt and every row tile by lm_sp
  //    workgroups sharing that XCD's L2.
  const int b = blockIdx.x;
  int split, ptile;
  if (P.order == 0) {
    split = b / P.n_ptiles;
    ptile = b - split * P.n_ptiles;
  } else {
    const int xcd = b & 7, idx = b >> 3;
    const int grp = idx / (P.lm_pt * P.lm_sp), loc = idx % (P.lm_pt * P.lm_sp);
    const int sg = P.splits / P.lm_sp;                 // split groups
    split = (grp % sg) * P.lm_sp + loc % P.lm_sp;
    ptile = ((grp / sg) * P.lm_pt + loc / P.lm_sp) * 8 + xcd;
  }
  if (split >= P.splits || ptile >= P.n_ptiles) return;
  const int64_t p0 = (int64_t)ptile * kTP;
  const int c_begin = (int)((int64_t)split * P.n_chunks / P.splits);
  const int c_end = (int)((int64_t)(split + 1) * P.n_chunks / P.splits);
  const int n_ck = c_end - c_begin;
  if (n_ck <= 0) return;  // the host keeps splits <= chunks
  const int ST = P.d / kKB;
  const int total = n_ck * ST;
  const float c_hi = P.c_hi, c_lo = P.c_lo;
  const int V = (int)P.vocab;

  // Loader: thread t moves 16 bytes of rows (t >> 3) + 64 j, j < 4, of each
  // operand per stage, through one buffer resource per operand tile, the
  // whole offset in the per-lane operand (the range check covers it; a
  // scalar offset would not be checked).  Rows past the end lie beyond the
  // resource and read zeros; their results are masked or never written.
  // (The host keeps 256 rows of either operand below 2^31 bytes.)
  constexpr int kLJ = kTV * kKB * 2 / 16 / kB;  // 16-byte loads per operand
  constexpr int kRS = kB / 8;                    // rows covered by one load round
  const int lrow = t >> 3, lcol = t & 7;
  const uint32_t xlane = (uint32_t)(lrow * P.xs * 2 + lcol * 16);
  const uint32_t wlane = (uint32_t)(lrow * P.ws * 2 + lcol * 16);
  const uint32_t xstep = (uint32_t)(kRS * P.xs * 2), wstep = (uint32_t)(kRS * P.ws * 2);
  const int64_t xrows = P.n_rows - p0 < kTP ? P.n_rows - p0 : kTP;
  const rsrc_t rx = make_rsrc(P.x + p0 * P.xs, (uint32_t)(xrows * P.xs * 2));
  rsrc_t rw = make_rsrc(P.w, 0u);
  auto set_chunk_rows = [&](int ck) {
    const int64_t v0 = (int64_t)ck * kTV;
    const int64_t rows = V - v0 < kTV ? V - v0 : kTV;
    rw = make_rsrc(P.w + v0 * P.ws, (uint32_t)(rows * P.ws * 2));
  };

  u32x4 ra[kLJ], rb[kLJ];
  auto load = [&](int g) {
    const int ks = g % ST;
    const int ck = c_begin + g / ST;
    if (ks == 0) set_chunk_rows(ck);
    const uint32_t kb = (uint32_t)(ks * kKB * 2);
#pragma unroll
    for (int j = 0; j < kLJ; ++j) {
      ra[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, wlane + j * wstep + kb, 0, 0);
      rb[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xlane + j * xstep + kb, 0, 0);
    }
  };
  auto store = [&](int buf) {
    unsigned char* A = lds + buf * 2 * kBuf;
    unsigned char* Bm = A + kBuf;
#pragma unroll
    for (int j = 0; j < kLJ; ++j) {
      const int o = (lrow + kRS * j) * kPitch + lcol * 16;
      *reinterpret_cast<u32x4*>(A + o) = ra[j];
      *reinterpret_cast<u32x4*>(Bm + o) = rb[j];
    }
  };

  constexpr int NJ = kWR / 32;  // column blocks (rows of the tile) per wave
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Issue priority: a wave raises its priority while it runs a stage's
  // fragment reads and MFMAs, so that when the SIMD's other wave is in its
  // loads, LDS stores or epilogue the MFMA stream is served first.  Per k
  // step, one of the compiler's strategies for interleaving LDS reads with
  // MFMAs replaces its default order (strategy 0 for the statistics kernel,
  // 1 for the store epilogues: the faster of the two for each).  Together
  // they made the 16,384-row slice 6-8% faster; the MFMA order, and so
  // every result, is unchanged.
  auto compute = [&](int buf) {
    __builtin_amdgcn_s_setprio(1);
    const unsigned char* A = lds + buf * 2 * kBuf + (wv * 128 + lc) * kPitch + h * 16;
    const unsigned char* Bm = lds + buf * 2 * kBuf + kBuf + (wp * kWR + lc) * kPitch + h * 16;
#pragma unroll
    for (int u = 0; u < kKB / 16; ++u) {
      bf16x8 fa[4], fb[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(A + i * 32 * kPitch + u * 32);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(Bm + j * 32 * kPitch + u * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      if constexpr (MODE == 0) __builtin_amdgcn_iglp_opt(0);
      else __builtin_amdgcn_iglp_opt(1);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ------------------------------------------------------------ row state
  // Thread t < 256 owns row t of the tile for the recorded-id cursor; each
  // lane owns NJ rows (j) of the tile for the running statistics.
  uint32_t* bm = reinterpret_cast<uint32_t*>(lds + kOffBm);
  int* beg = reinterpret_cast<int*>(lds + kOffBeg);
  const int64_t my_p = p0 + t;
  int cur = 0, cnt = 0, nid = kNoIdx;
  float sm[NJ], ss[NJ], sh[NJ];
  int sam[NJ], sa_l[NJ];
  // dLogits mode: value alpha p_v = sign(alpha) 2^((z - R) c - G) by the
  // exact exponent of the row kernels' pass 2 (p2_value), with the reference
  // R = lse T rounded to fp32 (R >= every logit of the row, so that the
  // exponent is small where the values are large), G = lse log2(e) - R c -
  // log2|alpha|, and lse = the fp32 statistic plus its remainder column.
  Pass2 dzq[NJ];
  if (MODE == 2) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t p = p0 + wp * kWR + j * 32 + lc;
      double sc = 0.0, al = 0.0, lse = 0.0;
      if (p < P.n_rows) {
        lm_row_factors(P, p, sc, al);
        const float* st = P.stats_in + p * SC_NSTATS;
        lse = (double)st[SC_STAT_LSE] + (double)st[SC_STAT_LSE_LO];
      }
      const float R = (float)(lse * (double)P.temperature);
      const double G = lse * 1.4426950408889634 - (double)R * P.c64 - log2(fabs(al));
      int g = 0;
      dzq[j] = pass2_setup(R, P.c_hi, P.c_lo, G, al < 0.0, g);
    }
  }
  if (!STORE) {
    cnt = (t < kTP && my_p < P.n_rows) ? P.scount[my_p] : 0;
    // first recorded id at or after this split's first vocabulary id
    const int sv0 = c_begin * kTV;
    int lo = 0, hi = cnt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)(P.skey[my_p * P.k + mid] >> 32) < sv0) lo = mid + 1; else hi = mid;
    }
    cur = lo;
    nid = cur < cnt ? (int)(P.skey[my_p * P.k + cur] >> 32) : kNoIdx;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t p = p0 + wp * kWR + j * 32 + lc;
      sm[j] = -FLT_MAX; ss[j] = 0.f; sh[j] = 0.f; sam[j] = kNoIdx;
      sa_l[j] = p < P.n_rows ? P.sa[p] : -1;
    }
  }
  // Hit words of chunk ck for row t: bit (v - v0) of word (v - v0) / 32.
  auto setup = [&](int ck) {
    if (t >= kTP) return;
    const int v0 = ck * kTV, v1 = v0 + kTV;
#pragma unroll
    for (int q = 0; q < 8; ++q) bm[t * kBmS + q] = 0u;
    beg[t] = cur;
    while (nid < v1) {
      const int o = nid - v0;
      bm[t * kBmS + (o >> 5)] |= 1u << (o & 31);
      ++cur;
      nid = cur < cnt ? (int)(P.skey[my_p * P.k + cur] >> 32) : kNoIdx;
    }
  };

  auto epilogue = [&](int ck) {
    const int v0 = ck * kTV;
    if (MODE == 2) {
      // each value is formed and rounded to bf16 once, then stored to the
      // row-major dLogits and, when asked, to the transposed copy dzt[v][p]
      // (lanes hold consecutive rows p, so each transposed store instruction
      // writes 64 contiguous bytes per id; rows past n_rows, up to dzt_cols,
      // are written there as 0)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t p = p0 + wp * kWR + j * 32 + lc;
        const bool live = p < P.n_rows;
        const bool tcol = P.dzt != nullptr && p < P.dzt_cols;
        if (!live && !tcol) continue;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            // rows 8 g4 + 4 h + (0..3) of the block: four consecutive ids
            const int v = v0 + wv * 128 + bi * 32 + 8 * g4 + 4 * h;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = p2_value<true>(acc[bi][j][4 * g4 + e], dzq[j]);
            u32x2 wv2;
            wv2[0] = live ? pack_bf16x2(x[0], x[1]) : 0u;
            wv2[1] = live ? pack_bf16x2(x[2], x[3]) : 0u;
            if (tcol) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (v + e < V)
                  P.dzt[(int64_t)(v + e) * P.dzts + p] = (uint16_t)(wv2[e >> 1] >> (16 * (e & 1)));
            }
            if (!live) continue;
            uint16_t* orow = P.dz + p * P.dzs;
            if (v + 3 < V) {
              *reinterpret_cast<u32x2*>(orow + v) = wv2;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (v + e < V) orow[v + e] = (uint16_t)(wv2[e >> 1] >> (16 * (e & 1)));
                else if (v + e < P.dz_cols) orow[v + e] = 0;
              }
            }
          }
      }
      return;
    }
    if (STORE) {
      // out[p][v]: four consecutive ids per (block, g4) group of this lane
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t p = p0 + wp * kWR + j * 32 + lc;
        if (p >= P.n_rows) continue;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int v = v0 + wv * 128 + bi * 32 + 8 * g4 + 4 * h;
            float a4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a4[e] = acc[bi][j][4 * g4 + e];
            if (P.out16) {
              uint16_t* orow = P.out16 + p * P.os;
              if (P.out_vec && v + 3 < V) {
                u32x2 wv2;
                wv2[0] = pack_bf16x2(a4[0], a4[1]);
                wv2[1] = pack_bf16x2(a4[2], a4[3]);
                *reinterpret_cast<u32x2*>(orow + v) = wv2;
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (v + e < V) orow[v + e] = (uint16_t)f32_to_bf16(a4[e]);
              }
            } else {
              float* orow = P.out + p * P.os;
              if (P.out_vec && v + 3 < V) {
                f32x4 x = {a4[0], a4[1], a4[2], a4[3]};
                if (P.out_accum) x += *reinterpret_cast<const f32x4*>(orow + v);
                *reinterpret_cast<f32x4*>(orow + v) = x;
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (v + e < V) orow[v + e] = P.out_accum ? orow[v + e] + a4[e] : a4[e];
              }
            }
          }
      }
      return;
    }
    const bool ragged = v0 + kTV > V;
    if (ragged) {
      // row offset bi * 32 + 8 (i / 4) + i % 4 (a constant) against this
      // lane's bound, so no per-element index is kept in registers
      const int lim = V - v0 - wv * 128 - 4 * h;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool out = bi * 32 + 8 * (i >> 2) + (i & 3) >= lim;
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[bi][j][i] = out ? -INFINITY : acc[bi][j][i];
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ploc = wp * kWR + j * 32 + lc;
      // chunk maximum of this lane's 64 logits of row ploc
      float bmx = -INFINITY;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int i = 0; i < 16; ++i) bmx = fmaxf(bmx, acc[bi][j][i]);
      if (bmx > sm[j]) {
        // first (lowest id) element equal to the new maximum
        int e = 0;
#pragma unroll
        for (int bi = 3; bi >= 0; --bi)
#pragma unroll
          for (int i = 15; i >= 0; --i) e = acc[bi][j][i] == bmx ? bi * 16 + i : e;
        sam[j] = v0 + wv * 128 + (e >> 4) * 32 + lm_row(e & 15, h);
      }
      // the row's integer reference E = ref_exp(max): rebase by 2^-(E' - E)
      const float mn = fmaxf(sm[j], bmx);
      const float E = ref_exp(mn, c_hi);
      const float D = E - ref_exp(sm[j], c_hi);
      const int kd = (int)fminf(D, 2048.f);
      sh[j] = ldexpf(fmaf(-D, ss[j], sh[j]), -kd);
      ss[j] = ldexpf(ss[j], -kd);
      sm[j] = mn;
      float sb[4], h_acc = 0.f;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int vb = v0 + wv * 128 + bi * 32;    // first id of the block
        const uint32_t hw = bm[ploc * kBmS + wv * 4 + bi];
        uint32_t word = hw;
        if (ragged) {
          const int nv = V - vb;                    // valid ids in the block
          word |= nv <= 0 ? 0xffffffffu : (nv >= 32 ? 0u : ~((1u << nv) - 1u));
        }
        const uint32_t wh = word >> (4 * h);
        // 2^(z c - E), z c = z c_hi + z c_lo; summed pairwise.  A recorded
        // id's exponent is replaced by -2^100 first, which makes its term and
        // its entropy product exactly 0 (one select instead of two).
        float e16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool ex = (wh >> (8 * (i >> 2) + (i & 3))) & 1u;
          const float y0 = fmaf(acc[bi][j][i], c_lo, fmaf(acc[bi][j][i], c_hi, -E));
          const float y = ex ? -0x1p100f : y0;
          const float e = exp2_fast(y);
          e16[i] = e;
          h_acc = fmaf(e, y, h_acc);
        }
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
          for (int i = 0; i + w < 16; i += 2 * w) e16[i] += e16[i + w];
        sb[bi] = e16[0];
        // Captures: logits at recorded ids (rare) and at the sampled id.
        uint32_t bits = hw & (0x0f0f0f0fu << (4 * h));   // this lane's rows
        while (bits) {
          const int o = __builtin_ctz(bits);
          bits &= bits - 1u;
          const int ih = (o >> 3) * 4 + (o & 3);
          float z = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) z = i == ih ? acc[bi][j][i] : z;
          const int64_t p = p0 + ploc;
          const int v = vb + o;
          for (int q = beg[ploc]; q < P.k; ++q) {
            const long long kv = P.skey[p * P.k + q];
            if ((int)(kv >> 32) == v) {
              P.head_raw[p * P.k + (int)(kv & 0xffffffff)] = z;
              break;
            }
          }
        }
        const unsigned ao = (unsigned)(sa_l[j] - vb);
        if (ao < 32u && ((ao >> 2) & 1u) == (unsigned)h) {
          const int ia = (int)((ao >> 3) * 4 + (ao & 3));
          float za = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) za = i == ia ? acc[bi][j][i] : za;
          P.za[p0 + ploc] = za;
        }
      }
      ss[j] += (sb[0] + sb[1]) + (sb[2] + sb[3]);
      sh[j] += h_acc;
    }
  };

  // ------------------------------------------------------------ main loop
  load(0);
  store(0);
  if (!STORE) setup(c_begin);
  __syncthreads();
  for (int g = 0; g < total; ++g) {
    const int ks = g % ST;
    if (!STORE && ks == 0 && g > 0) {
      setup(c_begin + g / ST);
      __syncthreads();
    }
    const bool more = g + 1 < total;
    if (more) load(g + 1);
    compute(g & 1);
    if (more) store((g + 1) & 1);
    if (ks == ST - 1) {
      // after the store: no prefetched operands are live in registers
      epilogue(c_begin + g / ST);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
    }
    __syncthreads();
  }
  if (STORE) return;

  // ------------------------------------------------------------ merge
  // lanes l and l ^ 32 hold the same rows; waves wv = 0, 1 hold the same rows
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float m2 = __shfl_xor(sm[j], 32), s2 = __shfl_xor(ss[j], 32);
    const float h2 = __shfl_xor(sh[j], 32);
    const int a2 = __shfl_xor(sam[j], 32);
    lm_merge(sm[j], ss[j], sh[j], sam[j], m2, s2, h2, a2, c_hi);
  }
  float4* xch = reinterpret_cast<float4*>(lds);  // operand buffers are free now
  if (wv == 1 && h == 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      xch[wp * kWR + j * 32 + lc] = make_float4(sm[j], ss[j], sh[j], __int_as_float(sam[j]));
  }
  __syncthreads();
  if (wv == 0 && h == 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ploc = wp * kWR + j * 32 + lc;
      const float4 o = xch[ploc];
      lm_merge(sm[j], ss[j], sh[j], sam[j], o.x, o.y, o.z, __float_as_int(o.w), c_hi);
      const int64_t p = p0 + ploc;
      if (p < P.n_rows)
        P.state[(int64_t)split * P.n_rows + p] =
            make_float4(sm[j], ss[j], sh[j], __int_as_float(sam[j]));
    }
  }
}

// ---------------------------------------------------------------------------
// Finalize: one wave per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lm_finalize(LmParams P) {
  __shared__ uint32_t sh_status;
  const int t = threadIdx.x, l = t & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (t >> 6);
  if (t == 0) sh_status = 0u;
  __syncthreads();
  const int K = P.k;
  const float c_hi = P.c_hi;
  const double c64 = P.c64;
  const float qnan = __builtin_nanf("");
  if (p < P.n_rows) {
    float* stats = P.row_stats + p * SC_NSTATS;
    int32_t* ridx = P.row_idx + p * 2;
    const int resp = P.resp_idx ? P.resp_idx[p] : 0;
    if (resp < 0) {
      if (l == 0) {
        stats[SC_STAT_LSE] = 0.f; stats[SC_STAT_LOGP_A] = 0.f; stats[SC_STAT_TAIL] = 0.f;
        stats[SC_STAT_P_H] = 0.f; stats[SC_STAT_ENTROPY] = 0.f; stats[SC_STAT_LSE_LO] = 0.f;
        ridx[0] = -1; ridx[1] = -1;
      }
      if (P.head_logp)
        for (int k = l; k < K; k += kWave) P.head_logp[p * K + k] = 0.f;
    } else {
      uint32_t fl = P.sflags[p];
      // merge the split states in a fixed butterfly order (lane l takes
      // splits l, l + 64, ... in order, then the butterfly), in float64
      float m = -FLT_MAX;
      double s = 0.0, hy = 0.0;
      int am = kNoIdx;
      for (int q = l; q < P.splits; q += kWave) {
        const float4 st = P.state[(int64_t)q * P.n_rows + p];
        lm_merge<double>(m, s, hy, am, st.x, (double)st.y, (double)st.z,
                         __float_as_int(st.w), c_hi);
      }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float m2 = __shfl_xor(m, o);
        const double s2 = __shfl_xor(s, o), h2 = __shfl_xor(hy, o);
        const int a2 = __shfl_xor(am, o);
        lm_merge<double>(m, s, hy, am, m2, s2, h2, a2, c_hi);
      }
      // s and hy are relative to the integer reference E; the recorded ids'
      // terms 2^(z c - E) (their logits were captured by the main kernel)
      // join them in float64
      const double E = (double)ref_exp(m, c_hi);
      double sH = 0.0, hH = 0.0;
      bool ninf = false;
      int aslot = kNoIdx;
      const int32_t a = P.sampled[p];
      for (int k = l; k < K; k += kWave) {
        const float z = fl ? 0.f : P.head_raw[p * K + k];
        const double y = (double)z * c64 - E;
        const double e = exp2(y);
        ninf |= !(z > -INFINITY);
        sH += e;
        hH += e > 0.0 ? e * y : 0.0;
        if (P.head_ids[p * K + k] == a) aslot = min(aslot, k);
      }
      sH = wave_sum(sH);
      hH = wave_sum(hH);
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) aslot = min(aslot, __shfl_xor(aslot, o));
      const double stot = s + sH;
      const double log2s = log2(stot);
      const float za = fl ? 0.f : P.za[p];
      if (!(stot < INFINITY) || !(m > -FLT_MAX) || !(m < INFINITY) || !(za > -INFINITY) ||
          !(hy + hH == hy + hH) || wave_or(ninf ? 1u : 0u))
        fl |= SC_DEV_NONFINITE;
      const bool bad = fl != 0;
      double ph = 0.0;
      for (int k = l; k < K; k += kWave) {
        const float z = bad ? 0.f : P.head_raw[p * K + k];
        const double l2 = (double)z * c64 - E - log2s;
        ph += exp2(l2);
        if (P.head_logp) P.head_logp[p * K + k] = bad ? qnan : (float)(l2 * kLn2d);
      }
      ph = wave_sum(ph);
      if (l == 0) {
        const double lse64 = (E + log2s) * kLn2d;
        stats[SC_STAT_LSE] = bad ? qnan : (float)lse64;
        stats[SC_STAT_LSE_LO] = bad ? qnan : (float)(lse64 - (double)(float)lse64);
        stats[SC_STAT_LOGP_A] = bad ? qnan : (float)(((double)za * c64 - E - log2s) * kLn2d);
        stats[SC_STAT_TAIL] = bad ? qnan : (float)(s / stot);
        stats[SC_STAT_P_H] = bad ? qnan : (float)ph;
        stats[SC_STAT_ENTROPY] = bad ? qnan : (float)((log2s - (hy + hH) / stot) * kLn2d);
        ridx[0] = bad ? -1 : am;
        ridx[1] = bad ? -1 : (aslot == kNoIdx ? -1 : aslot);
        if (fl) atomicOr(&sh_status, fl);
      }
    }
  }
  __syncthreads();
  if (t == 0 && sh_status && P.dev_status) atomicOr(P.dev_status, sh_status);
}

// ---------------------------------------------------------------------------
// dLogits at the recorded ids and at the sampled id (one wave per row), after
// k_lm_main<2> wrote alpha p_v everywhere: slot k gets
// scale ([k = a_slot] - q_k - (1 - S) p_k) (centering) or scale ([..] - p_k);
// a sampled id outside the recorded set gets alpha p_a + scale.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lm_dz_fix(LmParams P) {
  const int t = threadIdx.x, l = t & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (t >> 6);
  if (p >= P.n_rows) return;
  const int resp = P.resp_idx ? P.resp_idx[p] : 0;
  if (resp < 0) return;
  double scale = 0.0, alpha = 0.0;
  lm_row_factors(P, p, scale, alpha);
  const float* st = P.stats_in + p * SC_NSTATS;
  const double oms = 1.0 - (double)st[SC_STAT_S];
  const int K = P.k;
  const int a_slot = P.idx_in[p * 2 + 1];
  uint16_t* orow = P.dz + p * P.dzs;
  for (int k = l; k < K; k += kWave) {
    const int32_t id = P.head_ids[p * K + k];
    if (id < 0 || id >= P.vocab) continue;
    const double pk = exp((double)P.head_logp_in[p * K + k]);
    const double ind = k == a_slot ? 1.0 : 0.0;
    const double v = P.centering ? scale * (ind - (double)P.head_probs[p * K + k] - oms * pk)
                                 : scale * (ind - pk);
    orow[id] = (uint16_t)f32_to_bf16((float)v);
    if (P.dzt) P.dzt[(int64_t)id * P.dzts + p] = (uint16_t)f32_to_bf16((float)v);
  }
  if (l == 0 && a_slot < 0) {
    const int32_t a = P.sampled[p];
    if (a >= 0 && a < P.vocab) {
      const double pa = exp((double)st[SC_STAT_LOGP_A]);
      const uint16_t va = (uint16_t)f32_to_bf16((float)(alpha * pa + scale));
      orow[a] = va;
      if (P.dzt) P.dzt[(int64_t)a * P.dzts + p] = va;
    }
  }
}

// bf16 transpose through a 64 x 64 LDS tile.  With 16-byte aligned rows
// (vec) each thread moves 8 consecutive elements per access; otherwise one.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src,
                                                        int64_t rows, int64_t cols, int64_t ss,
                                                        uint16_t* __restrict__ dst, int64_t rpad,
                                                        int64_t ds, int vec) {
  __shared__ __align__(16) uint16_t tile[64][72];   // 144-byte rows: 16-byte aligned, banks rotate
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  if (vec) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = t + 256 * q, r = idx >> 3, c8 = (idx & 7) * 8;
      const int64_t gr = r0 + r, gc = c0 + c8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (gr < rows) {
        if (gc + 7 < cols) {
          x = *reinterpret_cast<const u32x4*>(src + gr * ss + gc);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) e[k] = gc + k < cols ? src[gr * ss + gc + k] : (uint16_t)0;
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = (uint32_t)e[2 * k] | ((uint32_t)e[2 * k + 1] << 16);
        }
      }
      *reinterpret_cast<u32x4*>(&tile[r][c8]) = x;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = t + 256 * q, cc = idx >> 3, r8 = (idx & 7) * 8;
      const int64_t gc = c0 + cc, gr = r0 + r8;
      if (gc >= cols || gr >= rpad) continue;
      u32x4 x;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[k] = (uint32_t)tile[r8 + 2 * k][cc] | ((uint32_t)tile[r8 + 2 * k + 1][cc] << 16);
      *reinterpret_cast<u32x4*>(dst + gc * ds + gr) = x;
    }
    return;
  }
  const int tx = t & 63, ty = t >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + ty + 4 * i, cc = c0 + tx;
    tile[ty + 4 * i][tx] = (r < rows && cc < cols) ? src[r * ss + cc] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t cc = c0 + ty + 4 * i, r = r0 + tx;
    if (cc < cols && r < rpad) dst[cc * ds + r] = tile[tx][ty + 4 * i];
  }
}

// Set on every launch: no cached flag, so concurrent callers share no state.
template <int MODE>
hipError_t set_lds_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lm_main<MODE>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t rows, int64_t cols, int64_t ss,
                                 uint16_t* dst, int64_t rpad, int64_t ds, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rpad + 63) / 64));
  // the vector path needs 16-byte aligned rows and whole 64-row output tiles
  const int vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0) &&
                  ss % 8 == 0 && ds % 8 == 0 && rpad % 64 == 0;
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, src, rows, cols, ss, dst, rpad, ds,
                     vec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Workspace of sc_logprobs_lmhead_static, the entry point for callers that
// cannot allocate: one static device array per GPU, shared by every call on
// that GPU (calls that overlap on one GPU race; nothing in it needs clearing,
// since each kernel writes every workspace entry it later reads).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; host code uses this address,
// never the array's name (which stands for the symbol, not device memory).
hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_lmhead(const LmParams& P, int mode, hipStream_t s) {
  int grid = P.splits * P.n_ptiles;
  if (P.order == 1) {
    const int per_round = 8 * P.lm_pt;                // row tiles per group round
    grid = ((P.n_ptiles + per_round - 1) / per_round) * 8 * P.lm_pt * P.splits;
  }
  hipError_t e = hipSuccess;
  if (mode == 1) {
    if ((e = set_lds_attr<1>()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_lm_main<1>, dim3(grid), dim3(kB), kLds, s, P);
    return hipGetLastError();
  }
  if (mode == 2) {
    if ((e = set_lds_attr<2>()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_lm_main<2>, dim3(grid), dim3(kB), kLds, s, P);
    hipLaunchKernelGGL(k_lm_dz_fix, dim3((unsigned)((P.n_rows + 3) / 4)), dim3(256), 0, s, P);
    return hipGetLastError();
  }
  if ((e = set_lds_attr<0>()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lm_stage, dim3((unsigned)P.n_rows), dim3(256), 0, s, P);
  hipLaunchKernelGGL(k_lm_main<0>, dim3(grid), dim3(kB), kLds, s, P);
  hipLaunchKernelGGL(k_lm_finalize, dim3((unsigned)((P.n_rows + 3) / 4)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace sc
