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
//             raw logits (with its lowest index), and the sum of
//             2^((z - m) log2(e) / T) over unmarked vectors (the off-head tail,
//             summed directly, never as 1 - P_H).  Marked vectors are copied
//             to a short LDS list instead.
//   finalize  workgroup max / argmax / tail sum, the marked vectors resolved
//             element by element (recorded logits, the sampled logit, their
//             tail members), lse, log p at H and at a, P_H, tau; then Q_H,
//             rho, c, S, loss, TV, KL(mu_hat || p), K3 in float64.
//   pass 2    (optional) the row streamed again to write one output element
//             per vocabulary id: off-head ids get alpha * p_v (a single exp2 of
//             a fused multiply-add), marked vectors take the exact per-id value.
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
  C_WT = 13, C_RKL = 14, C_RES = 15, C_N = 16
};
enum { IS_NONE = 0, IS_TIS = 1, IS_MIS = 2 };
enum { F_BAD_ID = 1, F_DUP_ID = 2, F_BAD_SAMPLED = 4, F_NONFINITE = 8, F_BAD_RESP = 16 };
enum { M_DLOGITS = 0, M_SCORE = 1, M_CORRECTION = 2 };

// kU: 16-byte vectors per thread per pipelined tile (divides 32).
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
  const bool has_out = (KIND != KIND_LOGPROBS) && P.row_out != nullptr;
  const int t = threadIdx.x;
  const int K = P.k;
  const int V = (int)P.vocab;
  const int n_full = V / N;                 // full vectors per row
  const int rem = V - n_full * N;        // elements of the partial vector
  const int J = n_full > t ? (n_full - 1 - t) / B + 1 : 0;  // my vectors
  const float c = P.c;                          // log2(e) / T

  extern __shared__ __align__(16) unsigned char lds[];
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds + P.off_bitmap);
  int* hkey = reinterpret_cast<int*>(lds + P.off_hkey);
  int* hval = reinterpret_cast<int*>(lds + P.off_hval);
  float* headz = reinterpret_cast<float*>(lds + P.off_headz);  // logits at H
  float* headp = reinterpret_cast<float*>(lds + P.off_headp);  // p at H
  float* hout = reinterpret_cast<float*>(lds + P.off_hout);    // log p / output at H
  int* ent_vec = reinterpret_cast<int*>(lds + P.off_entvec);
  float* ent_val = reinterpret_cast<float*>(lds + P.off_entval);
  int* ent_slot = reinterpret_cast<int*>(lds + P.off_entslot);  // slot or -1 per listed element
  int* vkey = reinterpret_cast<int*>(lds + P.off_vkey);          // listed vector -> entry
  int* vval = reinterpret_cast<int*>(lds + P.off_vval);
  int* hid = reinterpret_cast<int*>(lds + P.off_hid);            // recorded id of each slot

  __shared__ float redf[4 * NW];
  __shared__ int redi[NW];
  __shared__ double redd[4 * NW];
  __shared__ unsigned long long redu[2 * NW];
  __shared__ int sh_ent;
  __shared__ uint32_t sh_flags;
  __shared__ float sh_za;
  __shared__ uint32_t sh_status;

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
          ridx[0] = -1; ridx[1] = -1;
        }
        if (KIND == KIND_LOGPROBS) { stats[C_P_H] = 0.f; stats[C_ENT] = 0.f; }
        if (KIND != KIND_LOGPROBS)
          for (int col = C_P_H; col <= C_RES; ++col) stats[col] = 0.f;
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

    const TI* zrow = reinterpret_cast<const TI*>(P.logits) + row * P.row_stride;
    const bool a_ok = a >= 0 && a < V;
    const bool need_stage = (KIND != KIND_CENTER) || has_out;

    // Vector j of this thread is row vector j * B + t.  Every thread owns at
    // least Jmin vectors, so tiles of kU vectors below Jt are loaded with the
    // same unconditional code by the whole workgroup; the remaining J - Jt
    // vectors of a thread (fewer than kU + 1) are handled one at a time.
    const int Jmin = n_full / B;
    const int Jt = (Jmin / kU) * kU;
    auto load_tile = [&](Raw (&r)[kU], int j0, auto nt) {
      const int64_t n0 = (int64_t)j0 * B + t;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        r[u] = IO::template load<decltype(nt)::value>(zrow, n0 + u * B);
    };
    auto load_one = [&](int j, auto nt) -> Raw {
      return IO::template load<decltype(nt)::value>(zrow, (int64_t)j * B + t);
    };
    auto tile_bits = [&](int j0) -> uint32_t {
      return (bitmap[(j0 >> 5) * B + t] >> (j0 & 31)) & ((1u << kU) - 1u);
    };
    auto append = [&](int n, const float (&v)[N]) {
      const int e = atomicAdd(&sh_ent, 1);
      if (e < P.ke) {
        idset_insert(vkey, vval, (uint32_t)P.vs - 1, P.vshift, (int32_t)n, e);
        ent_vec[e] = (int)n;
#pragma unroll
        for (int i = 0; i < N; ++i) ent_val[e * N + i] = v[i];
      }
    };

    // List this thread's marked vectors (read again: the stream skipped them).
    auto list_marked = [&]() {
      for (int w = 0; w < P.bm_wpt; ++w) {
        uint32_t word = bitmap[w * B + t];
        while (word) {
          const int j = w * 32 + __builtin_ctz(word);
          word &= word - 1u;
          float v[N];
          IO::unpack(IO::template load<false>(zrow, (int64_t)j * B + t), v);
          append(j * B + t, v);
        }
      }
    };

    // Map recorded ids and the sampled id onto the listed vectors: ent_slot
    // gets the slot of every recorded element (-1 elsewhere), headz the
    // recorded logits and sh_za the sampled logit.  Ends with a barrier.
    auto resolve_slots = [&](int n_ent) {
      for (int i = t; i < n_ent * N; i += B) ent_slot[i] = -1;
      __syncthreads();
      for (int k = t; k < K; k += B) {
        const int id = hid[k];
        if (id < 0 || id >= V) continue;
        const int e = idset_find(vkey, vval, (uint32_t)P.vs - 1, P.vshift, id / N);
        if (e < 0) continue;
        headz[k] = ent_val[e * N + id % N];
        ent_slot[e * N + id % N] = k;
      }
      if (t == 0 && a_ok) {
        const int e = idset_find(vkey, vval, (uint32_t)P.vs - 1, P.vshift, a / N);
        if (e >= 0) sh_za = ent_val[e * N + a % N];
      }
      __syncthreads();
    };

    // ------------------------------------------------------------ stage
    if (need_stage) {
      for (int w = 0; w < P.bm_wpt; ++w) bitmap[w * B + t] = 0u;
      for (int i = t; i < P.hs; i += B) hkey[i] = -1;
      for (int i = t; i < P.vs; i += B) vkey[i] = -1;
      for (int k = t; k < K; k += B) headz[k] = qnan;
    }
    if (t == 0) { sh_ent = 0; sh_flags = 0; sh_za = qnan; }
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
        hid[k] = id;
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
    }

    float m = 0.f;        // row max of raw logits (pass-1 kernels)
    float log2s = 0.f;    // log2 sum_v 2^((z_v - m) c)
    float lse = 0.f, logp_a = 0.f, tau = 0.f, entropy = 0.f;
    int argmax = -1, a_slot = -1;

    if (KIND != KIND_CENTER) {
      // ---------------------------------------------------------- pass 1
      // Online update per vector: running max m_t (starts at -FLT_MAX so
      // that all-(-inf) vectors rescale by 2^0 and add 2^-inf = 0), tail sum
      // s_t relative to m_t, h_t = sum 2^((z - m_t) c) (z - m_t) for the
      // entropy, and the index of the vector that raised m_t (strictly, so
      // the first of equal maxima is kept).
      float m_t = -FLT_MAX, s_t = 0.f, h_t = 0.f;
      int am_vec = -1;
      Raw am_raw = IO::ninf();  // the vector that raised m_t, kept in registers
      int am_direct = -1;
      auto vec_update = [&](const float (&v)[N], const Raw& rv, int j) {
        float vm = v[0];
#pragma unroll
        for (int i = 1; i < N; ++i) vm = fmaxf(vm, v[i]);
        const float m_new = fmaxf(m_t, vm);
        am_raw = keep_if(vm > m_t, rv, am_raw);
        am_vec = vm > m_t ? j : am_vec;
        const float r = exp2_fast((m_t - m_new) * c);
        h_t = r * (h_t - (m_new - m_t) * s_t);
        s_t *= r;
        m_t = m_new;
      };
      // exp sum and exp-weighted offset sum of one vector.  A -inf entry
      // makes its term 0 * -inf = NaN in acch; the stream leaves h_t NaN
      // then and the thread recomputes it after the stream (see below).
      auto vec_sums = [&](const float (&v)[N], float& acc, float& acch) {
        acc = 0.f;
        acch = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float d = v[i] - m_t;
          const float e = exp2_fast(d * c);
          acc += e;
          acch = fmaf(e, d, acch);
        }
      };
      // Branch-free: marked vectors are summed too and the sum is dropped
      // (they are resolved element by element after the stream).  The
      // running max is raised once per group of kG vectors, so one rescale
      // serves kG vectors.
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
            float vm = v[u][0];
#pragma unroll
            for (int i = 1; i < N; ++i) vm = fmaxf(vm, v[u][i]);
            am_raw = keep_if(vm > m_run, r[u0 + u], am_raw);
            am_vec = vm > m_run ? j0 + u0 + u : am_vec;   // strictly: first of equal maxima
            m_run = fmaxf(m_run, vm);
          }
          const float rs = exp2_fast((m_t - m_run) * c);
          h_t = rs * (h_t - (m_run - m_t) * s_t);
          s_t *= rs;
          m_t = m_run;
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            float acc, acch;
            vec_sums(v[u], acc, acch);
            const bool marked = (bits >> (u0 + u)) & 1u;
            s_t += marked ? 0.f : acc;
            h_t += marked ? 0.f : acch;
          }
        }
      };
      {
        std::integral_constant<bool, KIND == KIND_LOGPROBS> nt;
        for (int j0 = 0; j0 < Jt; j0 += kU) {
          Raw r[kU];
          load_tile(r, j0, nt);
          process(r, j0);
        }
        for (int j = Jt; j < J; ++j) {
          float v[N];
          const Raw rv = load_one(j, nt);
          IO::unpack(rv, v);
          vec_update(v, rv, j);
          float acc, acch;
          vec_sums(v, acc, acch);
          const bool marked = (bitmap[(j >> 5) * B + t] >> (j & 31)) & 1u;
          s_t += marked ? 0.f : acc;
          h_t += marked ? 0.f : acch;
        }
      }
      // A -inf logit among this thread's unmarked vectors left h_t NaN (its
      // term 0 * -inf): recompute the entropy sum against the final m_t with
      // the term clamped to 0, reading the thread's vectors again.  A NaN
      // logit leaves s_t NaN as well (the row is flagged) and is left alone.
      if (h_t != h_t && s_t == s_t) {
        float hh = 0.f;
        for (int j = 0; j < J; ++j) {
          if ((bitmap[(j >> 5) * B + t] >> (j & 31)) & 1u) continue;
          float v[N];
          IO::unpack(load_one(j, std::false_type{}), v);
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const float d = v[i] - m_t;
            hh = fmaf(exp2_fast(d * c), fmaxf(d, -FLT_MAX), hh);
          }
        }
        h_t = hh;
      }
      list_marked();
      // The partial last vector (vocab not a multiple of N) always goes to the
      // LDS list; its owner is the thread of vector index n_full.
      if (rem > 0 && t == (int)(n_full % B)) {
        float v[N];
        float tm = -INFINITY;
        int idx = -1;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          v[i] = i < rem ? load_elem(zrow, n_full * N + i) : -INFINITY;
          if (v[i] > tm) { tm = v[i]; idx = (int)(n_full * N + i); }
        }
        if (tm > m_t) {
          const float r = exp2_fast((m_t - tm) * c);
          h_t = r * (h_t - (tm - m_t) * s_t);
          s_t *= r;
          m_t = tm;
          am_direct = idx;
        }
        append(n_full, v);
      }
      // Element index of my maximum: the first element equal to m_t in the
      // vector that raised it (kept in registers during the stream).
      int am_t = 0x7fffffff;
      if (am_direct >= 0) {
        am_t = am_direct;
      } else if (am_vec >= 0) {
#pragma unroll
        for (int i = N - 1; i >= 0; --i)
          if (IO::elem(am_raw, i) == m_t) am_t = (int)((am_vec * B + t) * N + i);
      }

      // ---------------------------------------------------------- finalize
      float mv = m_t;
      int mi = am_t;
      block_argmax<B>(mv, mi, redf, redi);
      m = mv;
      argmax = mi;
      const float r_t = exp2_fast((m_t - m) * c);
      float tail_part = s_t * r_t;
      float h_part = r_t * (h_t - (m - m_t) * s_t);
      // Resolve the listed vectors: each recorded id (and the sampled id)
      // finds its vector's list entry through the vector map; every other
      // listed element is a tail term.  Tail terms are summed as 64-bit
      // fixed point (2^-52 units; each term is <= 1 since z <= m): integer
      // sums are exact, so the total does not depend on the listing order.
      const int n_ent = min(sh_ent, P.ke);
      resolve_slots(n_ent);
      // The entropy sum D = sum_v 2^((z - m) c) (z - m) takes every listed
      // element (recorded ids included) in signed 2^-32 fixed point, added
      // modulo 2^64 (terms are >= -0.37 T each).
      unsigned long long tail_fx = 0ull, h_fx = 0ull;
      for (int i = t; i < n_ent * N; i += B) {
        const int vid = ent_vec[i / N] * N + (i % N);
        if (vid >= V) continue;
        const float d = ent_val[i] - m;
        const float e = exp2_fast(d * c);
        if (ent_slot[i] < 0) tail_fx += (unsigned long long)(e * 0x1p52f);
        h_fx += (unsigned long long)(long long)(e * fmaxf(d, -FLT_MAX) * 0x1p32f);
      }
      unsigned long long fx[2] = {tail_fx, h_fx};
      block_sum<B, 2>(fx, redu);
      tail_part += t == 0 ? (float)((double)fx[0] * 0x1p-52) : 0.f;
      h_part += t == 0 ? (float)((double)(long long)fx[1] * 0x1p-32) : 0.f;
      float head_part = 0.f;
      for (int k = t; k < K; k += B) head_part += exp2_fast((headz[k] - m) * c);
      float sums[3] = {tail_part, head_part, h_part};
      block_sum<B, 3>(sums, redf);
      const float s = sums[0] + sums[1];
      log2s = log2f(s);
      // entropy = ln s - D / (T s), with 1 / T = c ln 2
      entropy = (log2s - sums[2] * c / s) * kLn2;
      lse = (m * c + log2s) * kLn2;
      tau = sums[0] / s;
      const float za = sh_za;
      logp_a = ((za - m) * c - log2s) * kLn2;
      uint32_t fl = 0;
      for (int k = t; k < K; k += B) {
        const float hz = headz[k];
        if (hz == -INFINITY) fl |= F_NONFINITE;
        const float l2 = (hz - m) * c - log2s;
        headp[k] = exp2_fast(l2 + 32.f) * 0x1p-32f;  // subnormal-exact
        hout[k] = l2 * kLn2;                          // log p at H
      }
      if (!(s < INFINITY) || !(m > -FLT_MAX) || !(m < INFINITY) || za == -INFINITY)
        fl |= F_NONFINITE;
      if (fl) atomicOr(&sh_flags, fl);
      a_slot = a_ok ? idset_find(hkey, hval, hmask, hshift, a) : -1;
      __syncthreads();
    } else {
      // sc_center: pass-1 results come from memory
      lse = stats[C_LSE];
      logp_a = stats[C_LOGP_A];
      tau = stats[C_TAIL];
      a_slot = ridx[1];
      argmax = ridx[0];
      for (int k = t; k < K; k += B) {
        const float lp = P.head_logp[row * K + k];
        hout[k] = lp;
        headp[k] = expf(lp);
      }
      __syncthreads();
    }

    const uint32_t flags = sh_flags;

    if (KIND == KIND_LOGPROBS) {
      float ph = 0.f;
      for (int k = t; k < K; k += B) ph += headp[k];
      float sums[1] = {ph};
      block_sum<B, 1>(sums, redf);
      if (t == 0) {
        const bool bad = flags != 0;
        stats[C_LSE] = bad ? qnan : lse;
        stats[C_LOGP_A] = bad ? qnan : logp_a;
        stats[C_TAIL] = bad ? qnan : tau;
        stats[C_P_H] = bad ? qnan : sums[0];
        stats[C_ENT] = bad ? qnan : entropy;
        ridx[0] = bad ? -1 : argmax;
        ridx[1] = bad ? -1 : a_slot;
        if (flags) sh_status |= flags;
      }
      if (P.head_logp)
        for (int k = t; k < K; k += B) P.head_logp[row * K + k] = flags ? qnan : hout[k];
      continue;
    }

    // -------------------------------------------------------------- center
    double d1[2] = {0.0, 0.0};
    for (int k = t; k < K; k += B) {
      d1[0] += (double)P.head_probs[row * K + k];
      d1[1] += (double)headp[k];
    }
    block_sum<B, 2>(d1, redd);
    const double Q_H = d1[0], P_H = d1[1];
    const double taud = (double)tau;
    const double rho = fmax(1.0 - Q_H, kClamp) / fmax(taud, kClamp);
    const double S = Q_H + rho * taud;
    double d2[4] = {0.0, 0.0, 0.0, 0.0};
    for (int k = t; k < K; k += B) {
      const double q = (double)P.head_probs[row * K + k];
      const double p = (double)headp[k];
      const double lp = (double)hout[k];
      const double ck = q - rho * p;
      if (P.coef) P.coef[row * K + k] = flags ? qnan : (float)ck;
      d2[0] += ck * lp;
      d2[1] += fabs(q - p);
      const double lq = (double)logf((float)q);
      if (q > 0.0) d2[2] += q * (lq - lp);
      if (p > 0.0) d2[3] += p * (lp - lq);   // reverse KL, head part
    }
    block_sum<B, 4>(d2, redd);

    uint32_t rflags = flags;
    if (resp >= P.n_responses) rflags |= F_BAD_RESP;
    const double A = (resp < P.n_responses) ? (double)P.advantages[resp] : (double)qnan;
    // importance ratio of the sampled token and its stop-gradient weight
    double w = (double)qnan, wt = 1.0;
    double k3 = (double)qnan;
    if (P.rollout_logp) {
      const double d = (double)logp_a - (double)P.rollout_logp[row];
      k3 = (double)expm1f((float)d) - d;
      w = (double)expf((float)d);
      if (P.is_mode == IS_TIS) wt = fmin(w, (double)P.is_hi);
      else if (P.is_mode == IS_MIS) wt = (w >= (double)P.is_lo && w <= (double)P.is_hi) ? w : 0.0;
    }
    const double loss = -A * wt * ((double)logp_a - (P.centering ? d2[0] : 0.0));
    const double tv = 0.5 * (d2[1] + fabs(rho - 1.0) * taud);
    const double lrho = (double)logf((float)rho);
    double kl = d2[2];
    if (rho * taud > 0.0) kl += rho * taud * lrho;
    const double rkl = d2[3] - (taud > 0.0 ? taud * lrho : 0.0);

    if (t == 0) {
      const bool bad = rflags != 0;
      if (KIND == KIND_CORRECT) {
        stats[C_LSE] = bad ? qnan : lse;
        stats[C_LOGP_A] = bad ? qnan : logp_a;
        stats[C_TAIL] = bad ? qnan : tau;
        stats[C_ENT] = bad ? qnan : entropy;
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
      stats[C_RES] = 0.f;
      if (rflags) sh_status |= rflags;
    }
    if (KIND == KIND_CORRECT && P.head_logp)
      for (int k = t; k < K; k += B) P.head_logp[row * K + k] = rflags ? qnan : hout[k];

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
    __syncthreads();  // all reads of hout as log p are done
    for (int k = t; k < K; k += B) {
      const double p = (double)headp[k];
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

    const bool neg = alpha < 0.0;
    // p_v = 2^((z_v - mref) c - lref); value = sign(alpha) 2^((z_v - mref) c + off)
    // computed as 2^(y + 32) 2^-32 so that results below 2^-126 stay exact
    // subnormals (the exp2 instruction flushes them).
    const float mref = (KIND == KIND_CORRECT) ? m : 0.f;
    const double lref = (KIND == KIND_CORRECT) ? (double)log2s
                                               : (double)lse * 1.4426950408889634;
    const float off = log2f(fabsf((float)alpha)) - (float)lref + 32.f;
    const float add_a = (float)scale;
    TO* orow = reinterpret_cast<TO*>(P.row_out) + row * P.out_stride;

    // Stream the row; marked vectors are not stored here (the sc_center kind
    // lists them now, the fused kind listed them in pass 1).
    // One output vector; the sign is a compile-time choice so that the
    // negation folds into the bf16 conversion.
    auto out_vec = [&](const Raw& r, float (&o)[N], auto negc) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float e = exp2_fast(fmaf(IO::elem(r, i) - mref, c, off)) * 0x1p-32f;
        o[i] = decltype(negc)::value ? -e : e;
      }
    };
    auto stream2 = [&](auto negc) {
      std::integral_constant<bool, true> nt;
      for (int j0 = 0; j0 < Jt; j0 += kU) {
        Raw r[kU];
        load_tile(r, j0, nt);
        const uint32_t bits = tile_bits(j0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          float o[N];
          out_vec(r[u], o, negc);
          if (!((bits >> u) & 1u)) RowOut<TO, N>::store(orow, (j0 + u) * B + t, o);
        }
      }
      for (int j = Jt; j < J; ++j) {
        if ((bitmap[(j >> 5) * B + t] >> (j & 31)) & 1u) continue;
        float o[N];
        out_vec(load_one(j, nt), o, negc);
        RowOut<TO, N>::store(orow, j * B + t, o);
      }
    };
    if (neg) stream2(std::true_type{});
    else stream2(std::false_type{});
    if (KIND == KIND_CENTER) list_marked();
    if (KIND == KIND_CENTER && rem > 0 && t == (int)(n_full % B)) {
      float v[N];
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = i < rem ? load_elem(zrow, n_full * N + i) : 0.f;
      append(n_full, v);
    }
    __syncthreads();
    // Marked vectors: exact values, one element per thread.
    const int n_ent = min(sh_ent, P.ke);
    if (KIND == KIND_CENTER) resolve_slots(n_ent);
    for (int i = t; i < n_ent * N; i += B) {
      const int e = i / N, l = i - e * N;
      const int vid = ent_vec[e] * N + l;
      if (vid >= V) continue;
      const int slot = ent_slot[i];
      float val;
      if (slot >= 0) {
        val = hout[slot];
      } else {
        val = exp2_fast(fmaf(ent_val[i] - mref, c, off)) * 0x1p-32f;
        val = neg ? -val : val;
        if (vid == a) val += add_a;
      }
      store_elem(orow, vid, val);
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
