// HIP kernels of the score-centering (SC) correction for gfx950.
//
// Method: "Score Centering" example page of Agent Lightning, section
// "Score Centering" (token loss, P_H, Q_H, rho with 1e-6 clamps, tail
// proportional to the trainer policy), section "Training" (group standard
// deviation normalisation), and the rollout_corr/k3_kl diagnostic.
//
// One workgroup per logits row (the kernel also loops over rows when the grid
// is smaller than the row count).
// Per row:
//   stage     recorded ids -> LDS id set (id -> slot) and a bitmap over the
//             row's 16-byte vectors marking those that hold a recorded id or
//             the sampled id; range and duplicate checks.
//   pass 1    one coalesced stream of the row: per-thread running max of the
//             raw logits (with its lowest index), and the off-head tail sum
//             2^(z c - E_t) (c = log2(e) / T) over the unmarked vectors,
//             summed directly (never as 1 - P_H) in float64, relative to an
//             integer exponent E_t that follows the thread's largest unmarked
//             logit, so that the terms that dominate the tail are computed
//             from small exponents.
//             Marked vectors are copied, as the stream meets them, to an LDS
//             list whose entry order is fixed by a prefix sum over threads.
//   finalize  workgroup max / argmax; the listed vectors resolved element by
//             element over all threads (recorded logits, the sampled logit,
//             the tail members among them, in float64); the head terms in
//             float64; lse, log p at H and at a, P_H, tau, entropy; then Q_H,
//             rho, c, S, loss, TV, KL(mu_hat || p), K3 in float64.
//   pass 2    (optional) the row streamed again to write one output element
//             per vocabulary id: off-head ids get alpha * p_v from one exp2 of
//             an exactly formed exponent; the listed vectors are written from
//             the list, one 16-byte store each (in the fused kind before the
//             stream, their values formed element-parallel).
#include "sc_device.h"
#include "sc_internal.h"

#include <cfloat>
#include <type_traits>

namespace sc {

enum KernelKind { KIND_LOGPROBS = 0, KIND_CENTER = 1, KIND_CORRECT = 2 };

// Stats columns (mirror of sc.h; duplicated here so device code needs no C header)
enum {
  C_LSE = 0, C_LOGP_A = 1, C_TAIL = 2, C_P_H = 3, C_Q_H = 4, C_RHO = 5,
  C_S = 6, C_LOSS = 7, C_TV = 8, C_KL = 9, C_K3 = 10, C_ENT = 11, C_W = 12,
  C_WT = 13, C_RKL = 14, C_LSE_LO = 15, C_N = 16
};
enum { IS_NONE = 0, IS_TIS = 1, IS_MIS = 2 };
enum { F_BAD_ID = 1, F_DUP_ID = 2, F_BAD_SAMPLED = 4, F_NONFINITE = 8, F_BAD_RESP = 16 };
enum { M_DLOGITS = 0, M_SCORE = 1, M_CORRECTION = 2 };

constexpr double kLn2d = 0.6931471805599453;
constexpr double kLog2ed = 1.4426950408889634;

// Keep a when c, else b (whole raw vectors; selects, no branch).
SC_DEV u32x4 keep_if(bool c, const u32x4& a, const u32x4& b) {
  u32x4 o;
  o.x = c ? a.x : b.x; o.y = c ? a.y : b.y; o.z = c ? a.z : b.z; o.w = c ? a.w : b.w;
  return o;
}
SC_DEV f32x4 keep_if(bool c, const f32x4& a, const f32x4& b) {
  f32x4 o;
  o.x = c ? a.x : b.x; o.y = c ? a.y : b.y; o.z = c ? a.z : b.z; o.w = c ? a.w : b.w;
  return o;
}
SC_DEV uint32_t keep_if(bool c, uint32_t a, uint32_t b) { return c ? a : b; }
SC_DEV float keep_if(bool c, float a, float b) { return c ? a : b; }

template <typename TI, typename TO, bool VECTOR, int B, int KIND, int kU, int WAVES>
__global__ __launch_bounds__(B) __attribute__((amdgpu_waves_per_eu(WAVES)))
void k_row(RowParams P) {
  static_assert(32 % kU == 0, "tile must divide the 32-bit bitmap word");
  using IO = RowIO<TI, VECTOR>;
  using Raw = typename IO::raw;
  constexpr int N = IO::N;
  constexpr int NW = B / kWave;
  constexpr bool kBf16In = std::is_same<TI, uint16_t>::value;
  const bool has_out = (KIND != KIND_LOGPROBS) && P.row_out != nullptr;
  const int t = threadIdx.x;
  const int K = P.k;
  const int V = (int)P.vocab;
  const int n_full = V / N;                 // full vectors per row
  const int rem = V - n_full * N;        // elements of the partial vector
  const int J = n_full > t ? (n_full - 1 - t) / B + 1 : 0;  // my vectors
  const float c_hi = P.c_hi, c_lo = P.c_lo;
  const double c64 = P.c64;

  extern __shared__ __align__(16) unsigned char lds[];
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds + P.off_bitmap);
  int* hkey = reinterpret_cast<int*>(lds + P.off_hkey);
  int* hval = reinterpret_cast<int*>(lds + P.off_hval);
  float* headz = reinterpret_cast<float*>(lds + P.off_headz);     // logits at H
  double* headp = reinterpret_cast<double*>(lds + P.off_headp);   // p at H
  double* headlp = reinterpret_cast<double*>(lds + P.off_headlp); // log p at H
  float* hout = reinterpret_cast<float*>(lds + P.off_hout);       // output value at H
  float* lval = reinterpret_cast<float*>(lds + P.off_lval);       // listed vectors' values
  int* lvec = reinterpret_cast<int*>(lds + P.off_lvec);           // listed vectors' indices
  int16_t* lslot = reinterpret_cast<int16_t*>(lds + P.off_lslot); // listed elements' slots in H

  __shared__ float redf[NW];
  __shared__ int redi[NW];
  __shared__ double redd[4 * NW];
  __shared__ uint32_t sh_flags;
  __shared__ float sh_za;
  __shared__ uint32_t sh_status;
  __shared__ int sh_ninf;
  __shared__ int sh_am;
  __shared__ int lbase[B];   // each thread's first list entry

  const uint32_t hmask = (uint32_t)P.hs - 1;
  const int hshift = P.hshift;
  const float qnan = __builtin_nanf("");

  if (t == 0) sh_status = 0;

  for (int64_t row = blockIdx.x; row < P.n_rows; row += gridDim.x) {
    const int resp = P.resp_idx ? P.resp_idx[row] : 0;
    const int32_t a = P.sampled[row];
    const int my_id = t < K ? P.head_ids[row * K + t] : -1;   // slot t (K <= B)
    float* stats = P.row_stats + row * C_N;
    int32_t* ridx = P.row_idx + row * 2;

    __syncthreads();  // LDS of the previous row is no longer read

    // ------------------------------------------------------------ padding
    if (resp < 0) {
      if (t == 0) {
        if (KIND != KIND_CENTER) {
          stats[C_LSE] = 0.f; stats[C_LOGP_A] = 0.f; stats[C_TAIL] = 0.f;
          stats[C_LSE_LO] = 0.f;
          ridx[0] = -1; ridx[1] = -1;
        }
        if (KIND == KIND_LOGPROBS) { stats[C_P_H] = 0.f; stats[C_ENT] = 0.f; }
        if (KIND != KIND_LOGPROBS)
          for (int col = C_P_H; col <= C_RKL; ++col) stats[col] = 0.f;
      }
      for (int k = t; k < K; k += B) {
        if (KIND != KIND_CENTER && P.head_logp) P.head_logp[row * K + k] = 0.f;
        if (KIND != KIND_LOGPROBS && P.coef) P.coef[row * K + k] = 0.f;
      }
      if (has_out) {   // a zero row, in whole vectors where the row allows
        TO* orow = reinterpret_cast<TO*>(P.row_out) + row * P.out_stride;
        int i0 = 0;
        if (VECTOR) {
          float zero[N];
#pragma unroll
          for (int i = 0; i < N; ++i) zero[i] = 0.f;
          for (int j = t; j < n_full; j += B) RowOut<TO, N>::store(orow, j, zero);
          i0 = n_full * N;
        }
        for (int i = i0 + t; i < V; i += B) store_elem(orow, i, 0.f);
      }
      continue;
    }

    // (sc_center without an output row reads no logits: they may be absent)
    const TI* zrow = P.logits ? reinterpret_cast<const TI*>(P.logits) + row * P.row_stride
                              : nullptr;
    const bool a_ok = a >= 0 && a < V;
    const bool need_stage = (KIND != KIND_CENTER) || has_out;

    // Vector j of this thread is row vector j * B + t.  Every thread owns at
    // least Jmin vectors, so tiles of kU vectors below Jt are loaded with the
    // same unconditional code by the whole workgroup; the remaining J - Jt
    // vectors of a thread (fewer than kU + 1) are handled one at a time.  On
    // the vector path the row's full vectors are read through a buffer
    // resource over exactly those bytes.
    const int Jmin = n_full / B;
    const int Jt = (Jmin / kU) * kU;
    const rsrc_t zr = make_rsrc(zrow, VECTOR ? (uint32_t)n_full * 16u : 0u);
    auto ld = [&](int j, auto ntc) -> Raw {
      constexpr bool NT = decltype(ntc)::value;
      if constexpr (VECTOR)
        return IO::template bload<NT ? kNT : 0>(zr, (uint32_t)(j * B + t) * 16u);
      else
        return IO::template load<NT>(zrow, (int64_t)j * B + t);
    };
    // A tile's loads.  The stream below also fetches the tile after the
    // thread's last full one, never consumed: on the vector path its
    // vectors beyond the row read zeros without a memory access, on the
    // scalar path the index is held at the thread's last vector.
    auto load_tile = [&](Raw (&r)[kU], int j0, auto ntc) {
#pragma unroll
      for (int u = 0; u < kU; ++u) r[u] = ld(VECTOR ? j0 + u : min(j0 + u, J - 1), ntc);
    };
    // The thread's full tiles in order, software pipelined: the loads of the
    // next tile are issued before the current one is consumed, so that every
    // wave keeps a tile of loads in flight while it computes.  The loads
    // are unconditional: a load under a branch would leave the compiler's
    // wait counts at the join unable to tell the tiles apart, and it would
    // wait for the prefetch as well.
    auto stream_tiles = [&](auto ntc, auto&& consume) {
      if (Jt == 0) return;
      Raw cur[kU];
      load_tile(cur, 0, ntc);
      for (int j0 = 0; j0 < Jt; j0 += kU) {
        Raw nxt[kU];
        load_tile(nxt, j0 + kU, ntc);
        consume(cur, j0);
#pragma unroll
        for (int u = 0; u < kU; ++u) cur[u] = nxt[u];
      }
    };
    auto tile_bits = [&](int j0) -> uint32_t {
      return (bitmap[(j0 >> 5) * B + t] >> (j0 & 31)) & ((1u << kU) - 1u);
    };
    auto is_marked = [&](int j) -> bool {
      return (bitmap[(j >> 5) * B + t] >> (j & 31)) & 1u;
    };
    // Marked-vector list: each thread's marked vectors (and, for its owner,
    // the partial last vector, which the bitmap never holds) take
    // consecutive entries from lpos on; lpos comes from a prefix sum over
    // threads, so the list order, and every sum taken over it, is the same on
    // every run.  capture() appends one vector as the stream meets it.
    int lpos = 0, n_ent = 0;
    auto capture = [&](int n, const float (&v)[N]) {
      lvec[lpos] = n;
#pragma unroll
      for (int i = 0; i < N; ++i) lval[lpos * N + i] = v[i];
      ++lpos;
    };
    const bool rem_owner = rem > 0 && t == (int)(n_full % B);
    auto capture_partial = [&]() {
      float v[N];
#pragma unroll
      for (int i = 0; i < N; ++i)
        v[i] = i < rem ? load_elem(zrow, (int64_t)n_full * N + i) : -INFINITY;
      capture(n_full, v);
      return v[0];
    };

    // ------------------------------------------------------------ stage
    if (need_stage) {
      for (int w = 0; w < P.bm_wpt; ++w) bitmap[w * B + t] = 0u;
      for (int i = t; i < P.hs; i += B) hkey[i] = -1;
      for (int k = t; k < K; k += B) headz[k] = qnan;
      for (int i = t; i < P.ke * N; i += B) lslot[i] = -1;
    }
    if (t == 0) { sh_flags = 0; sh_za = qnan; sh_ninf = 0; }
    __syncthreads();
    if (need_stage) {
      uint32_t fl = 0;
      auto mark = [&](int v) {
        const int n = v / N;
        if (n < n_full) {
          const int j = n / B;
          const int tt = (int)(n - j * B);
          atomicOr(&bitmap[(j >> 5) * B + tt], 1u << (j & 31));
        }
      };
      for (int k = t; k < K; k += B) {
        const int32_t id = k == t ? my_id : P.head_ids[row * K + k];
        if (id < 0 || id >= V) {
          fl |= F_BAD_ID;
        } else {
          if (!idset_insert(hkey, hval, hmask, hshift, id, k)) fl |= F_DUP_ID;
          mark(id);
        }
      }
      if (t == 0) {
        if (!a_ok) fl |= F_BAD_SAMPLED; else mark(a);
      }
      if (fl) atomicOr(&sh_flags, fl);
      __syncthreads();
      int cnt = rem_owner ? 1 : 0;
      for (int w = 0; w < P.bm_wpt; ++w) cnt += __builtin_popcount(bitmap[w * B + t]);
      lpos = block_excl_scan<B>(cnt, redi, n_ent);
      // The list slot of every recorded id, without a lookup per listed
      // element later: thread tt lists its marked vectors in stream order
      // (j ascending) from lbase[tt] on, then the partial last vector if it
      // owns it, so the entry of vector n = j B + tt is lbase[tt] plus the
      // marked vectors of tt below j.  Other listed elements keep -1.
      {
        lbase[t] = lpos;
        __syncthreads();
        for (int k = t; k < K; k += B) {
          const int32_t id = k == t ? my_id : P.head_ids[row * K + k];
          if (id < 0 || id >= V) continue;
          const int n = id / N;
          const int tt = n % B;
          int entry = lbase[tt];
          if (n < n_full) {
            const int j = n / B;
            for (int w = 0; w < (j >> 5); ++w) entry += __builtin_popcount(bitmap[w * B + tt]);
            entry += __builtin_popcount(bitmap[(j >> 5) * B + tt] & ((1u << (j & 31)) - 1u));
          } else {
            for (int w = 0; w < P.bm_wpt; ++w) entry += __builtin_popcount(bitmap[w * B + tt]);
          }
          lslot[entry * N + (id - n * N)] = (int16_t)k;
        }
      }
    }

    float m = 0.f;          // row max of raw logits
    float E_row = 0.f;      // ceil(m c_hi): exponent reference of the row's sums
    double l2s = 0.0;       // log2 sum_v 2^(z_v c - E_row)
    double lse = 0.0, logp_a = 0.0, tau = 0.0, P_H = 0.0, entropy = 0.0;
    int argmax = -1, a_slot = -1;

    if (KIND != KIND_CENTER) {
      // ---------------------------------------------------------- pass 1
      // m_t: running max of the unmarked vectors (argmax; starts at -FLT_MAX
      // so that all -inf vectors never count; the marked vectors' elements
      // are compared in the finalize, from the list); am_vec: the thread's
      // vector that last raised it (strictly, so the first of equal maxima is
      // kept).  E_t = ref_exp(m_t): the exponent reference of
      // s_t = sum 2^(z c - E_t) (float64) and of h_t = sum 2^(z c - E_t)
      // (z c - E_t) over unmarked vectors.  When E_t rises by D, s_t scales by
      // 2^-D and h_t by 2^-D after subtracting D s_t, both exactly.
      float m_t = -FLT_MAX, E_t = ref_exp(-FLT_MAX, c_hi);
      double s_t = 0.0;
      float h_t = 0.f;
      int am_vec = -1;
      auto rebase = [&](float E_new) {
        const float D = E_new - E_t;                 // >= 0
        const int kd = (int)fminf(D, 2048.f);
        h_t = ldexpf(fmaf(-D, (float)s_t, h_t), -kd);
        s_t = ldexp(s_t, -kd);
        E_t = E_new;
      };
      // Exp sum (pairwise) and exponent-weighted sum of one vector relative to
      // E_t: y = z c_hi - E_t + z c_lo (two fma).  A -inf entry makes its
      // term 0 * -inf = NaN in acch; the stream leaves h_t NaN then and the
      // thread recomputes it after the stream (see below).
      auto vec_sums = [&](const float (&v)[N], float& acc, float& acch) {
        float e[N];
        acch = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float y = fmaf(v[i], c_lo, fmaf(v[i], c_hi, -E_t));
          e[i] = exp2_fast(y);
          acch = fmaf(e[i], y, acch);
        }
#pragma unroll
        for (int w = 1; w < N; w <<= 1)
#pragma unroll
          for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
        acc = e[0];
      };
      // An unmarked vector's maximum and its argmax bookkeeping; a marked
      // vector is captured to the list instead (its maximum is taken there).
      auto scan_vec = [&](const float (&v)[N], int j, bool marked, float& m_run) {
        float vm = v[0];
#pragma unroll
        for (int i = 1; i < N; ++i) vm = fmaxf(vm, v[i]);
        const float vu = marked ? -FLT_MAX : vm;
        am_vec = vu > m_run ? j : am_vec;          // strictly: first of equal maxima
        m_run = fmaxf(m_run, vu);
        if (marked) capture(j * B + t, v);
      };
      // Branch-free sums: marked vectors are summed too and the sum is
      // dropped (they are resolved element by element after the stream).
      // The maximum is raised once per group of kG vectors, so one rebase
      // serves kG vectors, and each group's sums are added in fp32 first.
      // The exponent reference follows the largest unmarked logit, not the
      // row maximum: where the maximum is a recorded id, the tail's largest
      // terms, which make up tau, then have exponents near 0, and rounding
      // each exponent to fp32 (relative 2^-24 of its size) costs them little.
      // A marked vector above the reference may overflow its dropped sum;
      // the selects keep that out.
      constexpr int kG = kU >= 4 ? 4 : kU;
      auto process = [&](const Raw (&r)[kU], int j0) {
        const uint32_t bits = tile_bits(j0);
#pragma unroll
        for (int u0 = 0; u0 < kU; u0 += kG) {
          float v[kG][N];
          float m_run = m_t;
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            IO::unpack(r[u0 + u], v[u]);
            scan_vec(v[u], j0 + u0 + u, (bits >> (u0 + u)) & 1u, m_run);
          }
          m_t = m_run;
          rebase(ref_exp(m_t, c_hi));
          float sg = 0.f, hg = 0.f;
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            float acc, acch;
            vec_sums(v[u], acc, acch);
            const bool marked = (bits >> (u0 + u)) & 1u;
            sg += marked ? 0.f : acc;
            hg += marked ? 0.f : acch;
          }
          s_t += (double)sg;
          h_t += hg;
        }
      };
      {
        std::integral_constant<bool, KIND == KIND_LOGPROBS> nt;
        stream_tiles(nt, process);
        for (int j = Jt; j < J; ++j) {
          float v[N];
          IO::unpack(ld(j, nt), v);
          const bool marked = is_marked(j);
          float m_run = m_t;
          scan_vec(v, j, marked, m_run);
          m_t = m_run;
          rebase(ref_exp(m_t, c_hi));
          float acc, acch;
          vec_sums(v, acc, acch);
          s_t += (double)(marked ? 0.f : acc);
          h_t += marked ? 0.f : acch;
        }
      }
      // A -inf logit among this thread's unmarked vectors left h_t NaN (its
      // term 0 * -inf): recompute the entropy sum against the final E_t with
      // the term clamped to 0, reading the thread's vectors again.  A NaN
      // logit leaves s_t NaN as well (the row is flagged) and is left alone.
      // Such a row takes the careful pass-2 value (sh_ninf).
      if (h_t != h_t && s_t == s_t) {
        sh_ninf = 1;
        float hh = 0.f;
        for (int j = 0; j < J; ++j) {
          if (is_marked(j)) continue;
          float v[N];
          IO::unpack(ld(j, std::false_type{}), v);
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const float y = fmaf(v[i], c_lo, fmaf(v[i], c_hi, -E_t));
            hh = fmaf(exp2_fast(y), fmaxf(y, -FLT_MAX), hh);
          }
        }
        h_t = hh;
      }
      // The partial last vector (vocab not a multiple of N) goes to the
      // list: its maximum and its sums are taken with the list.
      if (rem_owner) capture_partial();
      // Argmax candidates, keyed by element index.  The stream's: the first
      // element of the unmarked vector that holds the thread's maximum
      // (vectors do not overlap, so among the threads holding the row maximum
      // the lowest key is the vector of the row's first maximum; its owner
      // finds the element below).  The list's: each listed element by its own
      // index, the lower index first among equal values.
      const int am_key = am_vec >= 0 ? (am_vec * B + t) * N : 0x7fffffff;
      __syncthreads();   // every list entry is written
      float lm = -FLT_MAX;
      int lk = 0x7fffffff;
      for (int i = t; i < n_ent * N; i += B) {
        const int e = i / N;
        const int id = lvec[e] * N + (i - e * N);
        const float z = lval[i];
        if (id < V && (z > lm || (z == lm && id < lk))) { lm = z; lk = id; }
      }
      const bool from_list = lm > m_t || (lm == m_t && lk < am_key);

      // ---------------------------------------------------------- finalize
      float mv = from_list ? lm : m_t;
      const int my_key = from_list ? lk : am_key;
      int mi = my_key;
      block_argmax<B>(mv, mi, redf, redi);
      m = mv;
      argmax = mi;
      // Only the thread whose candidate won writes the row's argmax: a
      // listed element as it is, a streamed vector after reading it again to
      // find the element (one load per workgroup, awaited after the list
      // below).
      const bool am_owner = !from_list && mi < n_full * N && my_key == mi;
      const bool am_listed = from_list && my_key == mi;
      Raw am_raw = IO::ninf();
      if (am_owner) am_raw = ld(am_vec, std::false_type{});
      E_row = ref_exp(m, c_hi);
      // This thread's unmarked sums, moved to the row's reference (powers of
      // two: exact).  Then its marked vectors: recorded logits to headz, the
      // sampled logit to sh_za, every other element a tail term in float64.
      const double Dd = (double)(E_row - E_t);
      const int kd = (int)fmin(Dd, 2048.0);
      double s_tail = ldexp(s_t, -kd);
      double h_sum = ldexp((double)h_t - Dd * s_t, -kd);
      // Tail members of the list (the marked vectors' other elements):
      // 2^(z c - E_row) in float64.  They are few (at most (K + 2) N per row)
      // and can carry much of the tail mass where the recorded ids cluster,
      // so they are formed to float64 accuracy.
      for (int i = t; i < n_ent * N; i += B) {
        const int e = i / N;
        const int id = lvec[e] * N + (i - e * N);
        if (id >= V) continue;
        const float z = lval[i];
        const int slot = lslot[i];
        if (slot >= 0) {
          headz[slot] = z;
        } else {
          const double y = (double)z * c64 - (double)E_row;
          const double ez = exp2(y);
          s_tail += ez;
          h_sum += ez > 0.0 ? ez * y : 0.0;
        }
        if (id == a) sh_za = z;
      }
      if (am_listed) sh_am = mi;
      if (am_owner) {   // the first element equal to the row maximum
        int i0 = 0;
#pragma unroll
        for (int i = N - 1; i >= 0; --i)
          if (IO::elem(am_raw, i) == m) i0 = i;
        sh_am = mi + i0;
      }
      __syncthreads();
      if (mi < n_full * N) argmax = sh_am;
      // Recorded ids: 2^(z c - E_row) and its exponent-weighted term.
      double s_head = 0.0;
      uint32_t fl = 0;
      for (int k = t; k < K; k += B) {
        const float hz = headz[k];
        if (hz == -INFINITY) fl |= F_NONFINITE;
        const double y = (double)hz * c64 - (double)E_row;
        const double e = exp2(y);
        headp[k] = e;
        s_head += e;
        h_sum += e > 0.0 ? e * y : 0.0;
      }
      double sums[3] = {s_tail, s_head, h_sum};
      block_sum<B, 3>(sums, redd);
      const double s = sums[0] + sums[1];
      const double rs = 1.0 / s;
      l2s = log2(s);
      lse = ((double)E_row + l2s) * kLn2d;
      tau = sums[0] * rs;
      P_H = sums[1] * rs;
      entropy = kLn2d * (l2s - sums[2] * rs);
      const float za = sh_za;
      logp_a = ((double)za * c64 - (double)E_row - l2s) * kLn2d;
      for (int k = t; k < K; k += B) {
        const double y = (double)headz[k] * c64 - (double)E_row;
        headp[k] *= rs;
        headlp[k] = (y - l2s) * kLn2d;
      }
      if (!(s < INFINITY) || !(m > -FLT_MAX) || !(m < INFINITY) || za == -INFINITY)
        fl |= F_NONFINITE;
      if (fl) atomicOr(&sh_flags, fl);
      a_slot = a_ok ? idset_find(hkey, hval, hmask, hshift, a) : -1;
      __syncthreads();
    } else {
      // sc_center: pass-1 results come from memory (the log-sum-exp as its
      // fp32 value plus the fp32 remainder in column C_LSE_LO); the row max
      // is read back at the recorded argmax when the row is streamed again.
      // With the logits at hand, log p and p at H and log p(a) are formed in
      // float64 from the logits and that log-sum-exp, as in the fused
      // kernel: rho p_k reaches 1e5 and more where the tail mass is clamped,
      // and p_k from its stored fp32 log would carry |log p_k| 2^-24 of
      // relative error into c_k.  Without the logits the stored logs serve.
      lse = (double)stats[C_LSE] + (double)stats[C_LSE_LO];
      const double F = lse * kLog2ed;
      const bool zin = P.logits != nullptr;
      logp_a = (zin && a >= 0 && a < V) ? ((double)load_elem(zrow, a) * c64 - F) * kLn2d
                                        : (double)stats[C_LOGP_A];
      tau = stats[C_TAIL];
      a_slot = ridx[1];
      argmax = ridx[0];
      double ph = 0.0;
      for (int k = t; k < K; k += B) {
        const int32_t id = P.head_ids[row * K + k];
        if (zin && id >= 0 && id < V) {
          const double y = (double)load_elem(zrow, id) * c64 - F;
          headlp[k] = y * kLn2d;
          headp[k] = exp2(y);
        } else {
          const double lp = P.head_logp[row * K + k];
          headlp[k] = lp;
          headp[k] = exp(lp);    // p_k from its stored fp32 log, in float64
        }
        ph += headp[k];
      }
      double sums[1] = {ph};
      block_sum<B, 1>(sums, redd);
      P_H = sums[0];
      if (has_out) m = (argmax >= 0 && argmax < V) ? load_elem(zrow, argmax) : qnan;
      if (t == 0) sh_ninf = 1;   // the row's -inf entries are not known here
      __syncthreads();
    }

    const uint32_t flags = sh_flags;

    if (KIND == KIND_LOGPROBS) {
      if (t == 0) {
        const bool bad = flags != 0;
        const float lse32 = (float)lse;
        stats[C_LSE] = bad ? qnan : lse32;
        stats[C_LSE_LO] = bad ? qnan : (float)(lse - (double)lse32);
        stats[C_LOGP_A] = bad ? qnan : (float)logp_a;
        stats[C_TAIL] = bad ? qnan : (float)tau;
        stats[C_P_H] = bad ? qnan : (float)P_H;
        stats[C_ENT] = bad ? qnan : (float)entropy;
        ridx[0] = bad ? -1 : argmax;
        ridx[1] = bad ? -1 : a_slot;
        if (flags) sh_status |= flags;
      }
      if (P.head_logp)
        for (int k = t; k < K; k += B) P.head_logp[row * K + k] = flags ? qnan : (float)headlp[k];
      continue;
    }

    // -------------------------------------------------------------- center
    double d1[1] = {0.0};
    for (int k = t; k < K; k += B) d1[0] += (double)P.head_probs[row * K + k];
    block_sum<B, 1>(d1, redd);
    const double Q_H = d1[0];
    const double rho = fmax(1.0 - Q_H, kClamp) / fmax(tau, kClamp);
    const double S = Q_H + rho * tau;
    double d2[4] = {0.0, 0.0, 0.0, 0.0};
    for (int k = t; k < K; k += B) {
      const double q = (double)P.head_probs[row * K + k];
      const double p = headp[k];
      const double lp = headlp[k];
      const double ck = q - rho * p;
      if (P.coef) P.coef[row * K + k] = flags ? qnan : (float)ck;
      d2[0] += ck * lp;
      d2[1] += fabs(q - p);
      const double lq = logf((float)q);     // fp32 ln q: KL's bar is abs 1e-6
      if (q > 0.0) d2[2] += q * (lq - lp);
      if (p > 0.0) d2[3] += p * (lp - lq);   // reverse KL, head part
    }
    block_sum<B, 4>(d2, redd);

    uint32_t rflags = flags;
    if (resp >= P.n_responses) rflags |= F_BAD_RESP;
    if (KIND == KIND_CENTER && has_out && !(m > -FLT_MAX && m < INFINITY)) rflags |= F_NONFINITE;
    const double A = (resp < P.n_responses) ? (double)P.advantages[resp] : (double)qnan;
    // importance ratio of the sampled token and its stop-gradient weight
    double w = (double)qnan, wt = 1.0;
    double k3 = (double)qnan;
    if (P.rollout_logp) {
      // one float64 exponential: w = e^d and K3 = (w - 1) - d (for small |d|
      // the subtraction leaves an absolute error near 1e-16, far below K3's bar)
      const double d = logp_a - (double)P.rollout_logp[row];
      w = exp(d);
      k3 = (w - 1.0) - d;
      if (P.is_mode == IS_TIS) wt = fmin(w, (double)P.is_hi);
      else if (P.is_mode == IS_MIS) wt = (w >= (double)P.is_lo && w <= (double)P.is_hi) ? w : 0.0;
    }
    const double loss = -A * wt * (logp_a - (P.centering ? d2[0] : 0.0));
    const double tv = 0.5 * (d2[1] + fabs(rho - 1.0) * tau);
    const double lrho = (double)logf((float)rho);
    double kl = d2[2];
    if (rho * tau > 0.0) kl += rho * tau * lrho;
    const double rkl = d2[3] - (tau > 0.0 ? tau * lrho : 0.0);

    if (t == 0) {
      const bool bad = rflags != 0;
      if (KIND == KIND_CORRECT) {
        const float lse32 = (float)lse;
        stats[C_LSE] = bad ? qnan : lse32;
        stats[C_LSE_LO] = bad ? qnan : (float)(lse - (double)lse32);
        stats[C_LOGP_A] = bad ? qnan : (float)logp_a;
        stats[C_TAIL] = bad ? qnan : (float)tau;
        stats[C_ENT] = bad ? qnan : (float)entropy;
        ridx[0] = bad ? -1 : argmax;
        ridx[1] = bad ? -1 : a_slot;
      }
      stats[C_P_H] = bad ? qnan : (float)P_H;
      stats[C_Q_H] = bad ? qnan : (float)Q_H;
      stats[C_RHO] = bad ? qnan : (float)rho;
      stats[C_S] = bad ? qnan : (float)S;
      stats[C_LOSS] = bad ? qnan : (float)loss;
      stats[C_TV] = bad ? qnan : (float)tv;
      stats[C_KL] = bad ? qnan : (float)kl;
      stats[C_K3] = bad ? qnan : (float)k3;
      stats[C_W] = bad ? qnan : (float)w;
      stats[C_WT] = bad ? qnan : (float)wt;
      stats[C_RKL] = bad ? qnan : (float)rkl;
      if (rflags) sh_status |= rflags;
    }
    if (KIND == KIND_CORRECT && P.head_logp)
      for (int k = t; k < K; k += B) P.head_logp[row * K + k] = rflags ? qnan : (float)headlp[k];

    if (!has_out) continue;

    // -------------------------------------------------------------- pass 2
    // Off-head entries are alpha * p_v; recorded ids take hout[k]; the
    // sampled id, when outside H, adds `scale`.  The score rows carry the
    // weight wt; without centering mu_hat is replaced by p (score e_a - p).
    double scale = 1.0, alpha;
    if (P.row_mode == M_CORRECTION) {
      alpha = rho - 1.0;
      scale = 0.0;
    } else {
      if (P.row_mode == M_DLOGITS)
        scale = -A / ((double)P.temperature * (double)P.n_valid[0]);
      scale *= wt;
      alpha = P.centering ? -scale * (rho + 1.0 - S) : -scale;
    }
    if (rflags) { alpha = (double)qnan; scale = (double)qnan; }
    for (int k = t; k < K; k += B) {
      const double p = headp[k];
      double val;
      if (P.row_mode == M_CORRECTION) {
        val = (double)P.head_probs[row * K + k] - p;
      } else {
        const double ind = (k == a_slot) ? 1.0 : 0.0;
        val = P.centering ? scale * (ind - (double)P.head_probs[row * K + k] - (1.0 - S) * p)
                          : scale * (ind - p);
      }
      hout[k] = rflags ? qnan : (float)val;
    }
    __syncthreads();

    // log2 normaliser F of p_v = 2^(z c - F); value_v = sign(alpha) 2^((z - m) c - G)
    // with G = F - m c - log2 |alpha|.
    const double F = (KIND == KIND_CENTER) ? lse * kLog2ed : (double)E_row + l2s;
    const double G = rflags ? (double)qnan : F - (double)m * c64 - log2(fabs(alpha));
    int g = 0;
    const Pass2 Q = pass2_setup(m, c_hi, c_lo, G, alpha < 0.0, g);
    // Results below 2^-126 need the careful value: only when the row's scale
    // leaves room for them (with bf16 output, values below 2^-134 round to
    // zero anyway).
    const bool careful = !kBf16In || sh_ninf != 0 || g < (std::is_same<TO, uint16_t>::value ? 8 : 24);
    TO* orow = reinterpret_cast<TO*>(P.row_out) + row * P.out_stride;

    // Stream the row; marked vectors are not stored here but from the list
    // below (the sc_center kind lists them now, as the stream meets them; the
    // fused kind listed them in pass 1).  On the vector path a marked
    // vector's store is dropped by its offset, so the loop has no branch.
    using RO = RowOut<TO, N>;
    const rsrc_t orr = make_rsrc(orow, VECTOR ? (uint32_t)n_full * RO::BYTES : 0u);
    auto put = [&](int j, bool skip, const float (&o)[N]) {
      if constexpr (VECTOR)
        RO::bstore(orr, skip ? kSkip : (uint32_t)(j * B + t) * RO::BYTES, o);
      else if (!skip)
        RO::store(orow, (int64_t)j * B + t, o);
    };
    auto stream2 = [&](auto carefulc) {
      constexpr bool CF = decltype(carefulc)::value;
      std::integral_constant<bool, true> nt;
      auto emit = [&](const Raw (&r)[kU], int j0) {
        const uint32_t bits = tile_bits(j0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          float o[N];
#pragma unroll
          for (int i = 0; i < N; ++i) o[i] = p2_value<CF>(IO::elem(r[u], i), Q);
          const bool marked = (bits >> u) & 1u;
          put(j0 + u, marked, o);
          if (KIND == KIND_CENTER && marked) {
            float v[N];
            IO::unpack(r[u], v);
            capture((j0 + u) * B + t, v);
          }
        }
      };
      stream_tiles(nt, emit);
      for (int j = Jt; j < J; ++j) {
        const bool marked = is_marked(j);
        if (KIND != KIND_CENTER && marked) continue;
        const Raw r = ld(j, nt);
        if (marked) {
          float v[N];
          IO::unpack(r, v);
          capture(j * B + t, v);
          continue;
        }
        float o[N];
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = p2_value<CF>(IO::elem(r, i), Q);
        put(j, false, o);
      }
    };
    if (KIND == KIND_CORRECT) {
      // The listed vectors first, while the stream below keeps the memory
      // busy: each listed element's value (recorded ids take hout, the
      // sampled id outside H the float64 value alpha p_a + scale, every other
      // element the streamed value) computed element-parallel from the slot
      // the finalize found, in place of its logit; then one store per vector.
      const float va = (a_ok && a_slot < 0)
                           ? (float)(alpha * exp2((double)sh_za * c64 - F) + scale) : 0.f;
      for (int i = t; i < n_ent * N; i += B) {
        const int e = i / N;
        const int id = lvec[e] * N + (i - e * N);
        float val = 0.f;
        if (id < V) {
          const int slot = lslot[i];
          if (slot >= 0) val = hout[slot];
          else if (id == a) val = va;
          else val = p2_value<true>(lval[i], Q);
        }
        lval[i] = val;
      }
      __syncthreads();
      for (int e = t; e < n_ent; e += B) {
        const int n = lvec[e];
        float o[N];
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = lval[e * N + i];
        if (n < n_full) {
          RowOut<TO, N>::store(orow, n, o);
        } else {
          for (int i = 0; i < rem; ++i) store_elem(orow, (int64_t)n * N + i, o[i]);
        }
      }
    }
    if (careful) stream2(std::true_type{});
    else stream2(std::false_type{});
    if (KIND == KIND_CENTER) {
      if (rem_owner) capture_partial();
      __syncthreads();
    }
    // sc_center lists its vectors as its stream meets them: their values
    // and stores come after the stream, one thread per listed vector.
    if (KIND == KIND_CENTER)
    for (int e = t; e < n_ent; e += B) {
      const int n = lvec[e];
      float o[N];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int id = n * N + i;
        const float z = lval[e * N + i];
        float val = 0.f;
        if (id < V) {
          const int slot = lslot[e * N + i];
          if (slot >= 0) val = hout[slot];
          else if (id == a) val = (float)(alpha * exp2((double)z * c64 - F) + scale);
          else val = p2_value<true>(z, Q);
        }
        o[i] = val;
      }
      if (n < n_full) {
        RowOut<TO, N>::store(orow, n, o);
      } else {
        for (int i = 0; i < rem; ++i) store_elem(orow, (int64_t)n * N + i, o[i]);
      }
    }
  }

  __syncthreads();
  if (t == 0 && sh_status && P.dev_status) atomicOr(P.dev_status, sh_status);
}

// ---------------------------------------------------------------------------
// Group normalisation: one thread per group, float64 two-pass mean / std.
// ---------------------------------------------------------------------------
__global__ void k_group_norm(const float* __restrict__ rewards, int n_groups,
                             int G, int mode, float eps, float* __restrict__ adv) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const float* r = rewards + (int64_t)g * G;
  float* o = adv + (int64_t)g * G;
  double sum = 0.0;
  for (int i = 0; i < G; ++i) sum += (double)r[i];
  const double mean = sum / G;
  if (mode == 2) {
    for (int i = 0; i < G; ++i) o[i] = (float)((double)r[i] - mean);
    return;
  }
  if (G == 1) { o[0] = 0.f; return; }
  double ss = 0.0;
  for (int i = 0; i < G; ++i) { const double d = (double)r[i] - mean; ss += d * d; }
  const double sd = sqrt(ss / (mode == 0 ? (double)(G - 1) : (double)G));
  for (int i = 0; i < G; ++i) o[i] = (float)(((double)r[i] - mean) / (sd + (double)eps));
}

// ---------------------------------------------------------------------------
// Exact count of valid rows (single workgroup, int64).
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(B) void k_count_valid(const int32_t* __restrict__ resp,
                                                   int64_t n, int64_t* out, int acc) {
  __shared__ unsigned long long red[B / kWave];
  unsigned long long c = 0;
  for (int64_t i = threadIdx.x; i < n; i += B) c += resp[i] >= 0 ? 1ull : 0ull;
  c = wave_sum(c);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
    for (int w = 0; w < B / kWave; ++w) s += red[w];
    out[0] = (acc ? out[0] : 0) + (int64_t)s;
  }
}

// ---------------------------------------------------------------------------
// Step reductions: fixed-order float64 sums (single workgroup).
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(B) void k_batch_sums(const float* __restrict__ st,
                                                  const int32_t* __restrict__ resp,
                                                  int64_t n, const int64_t* n_valid,
                                                  double* batch, int acc) {
  constexpr int NS = 8;   // summed statistics
  constexpr int SUMS[NS] = {C_LOSS, C_K3, C_TV, C_KL, C_Q_H, C_P_H, C_ENT, C_RKL};
  __shared__ double red[(NS + 2) * (B / kWave)];
  __shared__ float redf[B / kWave];
  __shared__ int redi[B / kWave];
  double v[NS + 2];
#pragma unroll
  for (int j = 0; j < NS + 2; ++j) v[j] = 0.0;
  float wmax = -INFINITY;
  // Rows t, t + B, ... in order; R rows' loads are issued together (a padding
  // row's statistics are read too and then skipped), so the loop waits on
  // memory once per R rows instead of twice per row.
  constexpr int R = 4;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += (int64_t)R * B) {
    int rv[R];
    float x[R][NS + 1];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int64_t i = i0 + (int64_t)q * B;
      rv[q] = i < n ? resp[i] : -1;
      const float* s = st + (i < n ? i : 0) * C_N;
#pragma unroll
      for (int j = 0; j < NS; ++j) x[q][j] = s[SUMS[j]];
      x[q][NS] = s[C_W];
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (rv[q] < 0) continue;
#pragma unroll
      for (int j = 0; j < NS; ++j) v[j] += (double)x[q][j];
      v[NS] += 1.0;
      v[NS + 1] += (x[q][0] != x[q][0]) ? 1.0 : 0.0;   // x[q][0] is the loss
      wmax = fmaxf(wmax, x[q][NS]);
    }
  }
  block_sum<B, NS + 2>(v, red);
  int dummy = 0;
  block_argmax<B>(wmax, dummy, redf, redi);
  if (threadIdx.x == 0) {
    const double nv = (double)n_valid[0];
    for (int j = 0; j < NS + 2; ++j) batch[j] = (acc ? batch[j] : 0.0) + v[j];
    batch[NS + 2] = acc ? fmax(batch[NS + 2], (double)wmax) : (double)wmax;
    for (int j = 0; j < NS; ++j) batch[NS + 3 + j] = batch[j] / nv;
  }
}

// ---------------------------------------------------------------------------
// Reference copy: the memory system's rate for a read-once / write-once
// stream of the same bytes, with no arithmetic.  One workgroup of 512 threads
// per 512 KiB chunk; each thread keeps 8 16-byte loads in flight, loads and
// stores nontemporal, through buffer resources over the chunk (the last chunk
// may be shorter: its out-of-range vectors read zeros and drop their stores).
// ---------------------------------------------------------------------------
constexpr int kCopyB = 512;
constexpr int kCopyU = 8;
constexpr uint32_t kCopyChunk = 512u << 10;

__global__ __launch_bounds__(kCopyB) void k_copy(const unsigned char* __restrict__ src,
                                                 unsigned char* __restrict__ dst,
                                                 int64_t bytes) {
  const int64_t base = (int64_t)blockIdx.x * kCopyChunk;
  const int64_t left = bytes - base;
  const uint32_t n = left < (int64_t)kCopyChunk ? (uint32_t)left : kCopyChunk;
  const rsrc_t rs = make_rsrc(src + base, n);
  const rsrc_t rd = make_rsrc(dst + base, n);
  constexpr uint32_t step = kCopyB * 16u * kCopyU;
  for (uint32_t o = threadIdx.x * 16u; o < kCopyChunk; o += step) {
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + u * kCopyB * 16u, 0, kNT);
#pragma unroll
    for (int u = 0; u < kCopyU; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, o + u * kCopyB * 16u, 0, kNT);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename TI, typename TO, bool VECTOR, int B, int KIND>
static hipError_t launch_row_t(const RowParams& P, int grid, hipStream_t s) {
  constexpr int U = KIND == KIND_LOGPROBS ? SC_STATS_TILE
                  : KIND == KIND_CENTER ? SC_CENTER_TILE : SC_FUSED_TILE;
  constexpr int W = KIND == KIND_LOGPROBS ? SC_STATS_WAVES
                  : KIND == KIND_CENTER ? SC_CENTER_WAVES : SC_FUSED_WAVES;
  auto kern = k_row<TI, TO, VECTOR, B, KIND, U, W>;
  if (P.lds_bytes > 64 * 1024) {  // large K: opt in to more than 64 KiB of LDS
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)P.lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(B), P.lds_bytes, s, P);
  return hipGetLastError();
}

template <int B, int KIND>
static hipError_t launch_row_b(const RowParams& P, int grid, hipStream_t s) {
  const bool in_bf = P.in_dtype == 1, out_bf = P.out_dtype == 1;
  if (P.vector) {
    if (in_bf) return out_bf ? launch_row_t<uint16_t, uint16_t, true, B, KIND>(P, grid, s)
                             : launch_row_t<uint16_t, float, true, B, KIND>(P, grid, s);
    return out_bf ? launch_row_t<float, uint16_t, true, B, KIND>(P, grid, s)
                  : launch_row_t<float, float, true, B, KIND>(P, grid, s);
  }
  if (in_bf) return out_bf ? launch_row_t<uint16_t, uint16_t, false, B, KIND>(P, grid, s)
                           : launch_row_t<uint16_t, float, false, B, KIND>(P, grid, s);
  return out_bf ? launch_row_t<float, uint16_t, false, B, KIND>(P, grid, s)
                : launch_row_t<float, float, false, B, KIND>(P, grid, s);
}

hipError_t launch_row(const RowParams& P, int kind, int grid, hipStream_t s) {
  switch (kind) {
    case KIND_LOGPROBS: return launch_row_b<SC_STATS_BLOCK, KIND_LOGPROBS>(P, grid, s);
    case KIND_CENTER: return launch_row_b<SC_CENTER_BLOCK, KIND_CENTER>(P, grid, s);
    default: return launch_row_b<SC_FUSED_BLOCK, KIND_CORRECT>(P, grid, s);
  }
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t grid = (bytes + kCopyChunk - 1) / kCopyChunk;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)grid), dim3(kCopyB), 0, s,
                     static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst),
                     bytes);
  return hipGetLastError();
}

hipError_t launch_group_norm(const float* r, int n_groups, int G, int mode,
                             float eps, float* adv, hipStream_t s) {
  const int b = 64;
  hipLaunchKernelGGL(k_group_norm, dim3((n_groups + b - 1) / b), dim3(b), 0, s,
                     r, n_groups, G, mode, eps, adv);
  return hipGetLastError();
}

hipError_t launch_count_valid(const int32_t* resp, int64_t n, int64_t* out,
                              int acc, hipStream_t s) {
  hipLaunchKernelGGL((k_count_valid<1024>), dim3(1), dim3(1024), 0, s, resp, n,
                     out, acc);
  return hipGetLastError();
}

hipError_t launch_batch_sums(const float* st, const int32_t* resp, int64_t n,
                             const int64_t* n_valid, double* batch, int acc,
                             hipStream_t s) {
  hipLaunchKernelGGL((k_batch_sums<1024>), dim3(1), dim3(1024), 0, s, st, resp,
                     n, n_valid, batch, acc);
  return hipGetLastError();
}

}  // namespace sc
