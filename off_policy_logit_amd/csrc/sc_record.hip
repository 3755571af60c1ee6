// Rollout-side record of the SC correction for gfx950: per position, the
// top-k candidate ids of the rollout softmax with their probabilities and the
// log-probability of the sampled token (Score Centering page, section "Score
// Centering": the rollout records the top K behaviour probabilities of the
// sampling call, keeping their normalisation, and the sampled token's
// log-probability separately).
//
// One workgroup per row.  Candidates are ordered by the
// 64-bit key (order(z) << 32 | ~id): larger logit first, equal logits by
// lower id, every key distinct.  The row is streamed once:
//   * online max and sum of 2^((z - m) c) give the row's log-sum-exp;
//   * a 4096-bin histogram of the key's top 12 bits (sign, exponent, 3
//     mantissa bits) counts the elements at or above each wave's running
//     lower bound b_w on the bin of the k-th largest key, and each wave
//     appends those elements to its own LDS candidate buffer;
//   * b_w is raised from the histogram as the stream goes (any partial count
//     gives a valid lower bound), and the buffer is compacted to it.
// After the stream the exact bin b* of the k-th largest key is read off the
// histogram (exact above every b_w), the buffered keys at or above b* are
// ordered (by rank for at most 256 keys, else a bitonic sort in LDS) and the
// first k are the record.  A row whose
// candidates overflow a buffer or the sort array (heavy ties) takes the exact
// fallback: radix selection over the remaining key bits with further passes
// over the row, at most five, then one collection pass.  A wave whose buffer
// overflowed keeps counting (so the histogram stays exact above every bound)
// but stops buffering.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <algorithm>

#include "sc.h"
#include "sc_device.h"
#include "sc_internal.h"

namespace sc {
namespace {

#ifndef SC_RECORD_BLOCK
#define SC_RECORD_BLOCK 256
#endif
#ifndef SC_RECORD_TILE
#define SC_RECORD_TILE 4
#endif
#ifndef SC_RECORD_WAVES
#define SC_RECORD_WAVES 4
#endif
constexpr int kRB = SC_RECORD_BLOCK;     // threads per workgroup
constexpr int kRNW = kRB / kWave;        // waves
constexpr int kHBits = 12;               // histogram bits of the key
constexpr int kNBins = 1 << kHBits;
constexpr int kSortMax = 2048;           // sort array (overlays the histogram)
constexpr int kRU = SC_RECORD_TILE;      // vectors per thread per iteration
constexpr int kRankMax = kRB;            // candidate sets ordered by rank (O(n^2))
static_assert(kSortMax * 8 == kNBins * 4, "sort array overlays the histogram");

// Monotone unsigned key of a float (NaN excluded by the caller); -0 -> +0.
SC_DEV uint32_t okey(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
SC_DEV float okey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
SC_DEV unsigned long long key64(float x, uint32_t id) {
  return ((unsigned long long)okey(x) << 32) | (unsigned long long)(~id);
}
SC_DEV int bin_of(uint32_t k) { return (int)(k >> (32 - kHBits)); }
// Smallest float whose bin is >= b (so x >= bin_floor(b) <=> bin(x) >= b for
// every non-NaN x); -inf below the -inf bin.
SC_DEV float bin_floor(int b) {
  const uint32_t kk = (uint32_t)b << (32 - kHBits);
  if (kk <= 0x007fffffu) return -INFINITY;       // at or below the key of -inf
  if (kk > 0xff800000u) return INFINITY;         // above +inf (NaN keys)
  return okey_value(kk);
}
SC_DEV int lane_rank(unsigned long long bal) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// At four waves per SIMD (the default), at most 128 VGPRs: the row stream,
// the hot loop, stays free of spills; the rare paths (fallback passes, sort)
// may spill.
template <typename T, bool VECTOR>
__global__ __launch_bounds__(kRB) __attribute__((amdgpu_waves_per_eu(SC_RECORD_WAVES)))
void k_record(RecParams P) {
  using IO = RowIO<T, VECTOR>;
  using Raw = typename IO::raw;
  constexpr int N = IO::N;
  constexpr int B = kRB;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int V = (int)P.vocab;
  const int K = P.k;
  const int cap = P.cap;
  const float c = P.c;
  const int n_full = V / N, rem = V - n_full * N;

  extern __shared__ __align__(16) unsigned char lds[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds);                       // [kNBins]
  unsigned long long* sarr = reinterpret_cast<unsigned long long*>(lds);   // [kSortMax]
  unsigned long long* buf = reinterpret_cast<unsigned long long*>(lds + kNBins * 4) +
                            (size_t)w * cap;                               // [cap] per wave
  __shared__ float redf[4 * kRNW];
  __shared__ double redd[kRNW];
  __shared__ int redi[kRNW];
  // 0: flags, 1: overflow, 2: sort count, 3: status, 4: highest counted bin
  __shared__ unsigned int sh_u[5];
  __shared__ unsigned int wcnt[kRNW];   // keys appended to each wave's buffer
  __shared__ int sh_i[2];               // bin and count above it, from find_kth

  const float qnan = __builtin_nanf("");
  if (t == 0) sh_u[3] = 0u;

  for (int64_t row = blockIdx.x; row < P.n_rows; row += gridDim.x) {
    const T* zrow = reinterpret_cast<const T*>(P.logits) + row * P.row_stride;
    __syncthreads();                     // previous row's LDS reads are done
    for (int i = t; i < kNBins; i += B) hist[i] = 0u;
    if (t == 0) { sh_u[0] = 0u; sh_u[1] = 0u; sh_u[2] = 0u; sh_u[4] = 0u; }
    if (t < kRNW) wcnt[t] = 0u;
    __syncthreads();

    // ------------------------------------------------ exact bin of the k-th key
    // Thread t sums bins [lo, lo + PER), lo = kNBins - PER (t + 1); a block
    // scan in thread order (descending bins) finds the bin where the count
    // from the top reaches `need`; returns it and the count strictly above it.
    // (Bins are addressed as lo + q, one base register plus constant offsets.)
    constexpr int PER = kNBins / B;
    auto find_kth = [&](int need, int& bin_out, int& above_out) {
      const int lo = kNBins - PER * (t + 1);
      int sum = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) sum += (int)hist[lo + q];
      int x = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      __syncthreads();
      if (lane == kWave - 1) redi[w] = x;
      __syncthreads();
      int wave_off = 0;
      for (int q = 0; q < w; ++q) wave_off += redi[q];
      const int incl = wave_off + x, excl = incl - sum;
      if (excl < need && incl >= need) {
        int acc = excl;
#pragma unroll 1
        for (int q = PER - 1; q >= 0; --q) {   // one thread, once per call
          const int h = (int)hist[lo + q];
          if (acc + h >= need) { sh_i[0] = lo + q; sh_i[1] = acc; break; }
          acc += h;
        }
      }
      __syncthreads();
      bin_out = sh_i[0];
      above_out = sh_i[1];
    };
    // -------------------------------------------------------------- stream
    // The sum in two levels: each tile's kRU N terms in fp32 first, then the
    // tile sums into s_t.  A flat row gives a thread ~1,000 comparable
    // terms; added one by one to a running fp32 sum they would lose ~1e-5 of
    // it, ~30 tile sums lose a few 1e-7.  The workgroup adds the threads'
    // sums in float64.
    float m_t = -FLT_MAX, s_t = 0.f;
    int b_w = 0;            // wave-uniform lower bound on the k-th key's bin
    float thr = -INFINITY;  // bin_floor(b_w)

    // Raise b_w from the histogram and drop buffered keys below it.
    // Wave-local; counts that other waves are still adding only make the
    // bound lower (still valid: every count read is part of the final one).
    // Logits of both signs leave long runs of empty bins between them (the
    // small magnitudes), so the scan is two-level: each lane sums one group
    // of 32 bins (64 groups, 2,048 bins per step, from the highest bin any
    // wave has reported down to b_w's group); a wave scan finds the group
    // where the count from the top reaches k, then a scan of that group's
    // bins finds the bin.
    constexpr int kGB = 32;                      // bins per group
    auto refresh = [&]() {
      // The count once for the wave (the branches below are the wave's),
      // after every lane's pushes of the tiles before: the wave runs in
      // lockstep, and the barrier (no instruction) keeps the compiler from
      // moving the read above them.
      __builtin_amdgcn_wave_barrier();
      const int cnt = __builtin_amdgcn_readfirstlane((int)__atomic_load_n(&wcnt[w], __ATOMIC_RELAXED));
      if (cnt > cap) return;                     // overflowed: the row takes the fallback
      int total = 0, found = -1;
      // start at the highest bin any wave has reported (this wave's max
      // included); missing a higher count only lowers the bound
      const float wm = wave_max(m_t);
      if (lane == 0) atomicMax(&sh_u[4], (unsigned)bin_of(okey(wm)));
      const int top0 = __builtin_amdgcn_readfirstlane((int)__atomic_load_n(&sh_u[4], __ATOMIC_RELAXED));
      const int gw = b_w / kGB;
      for (int g0 = top0 / kGB; g0 >= gw && found < 0; g0 -= kWave) {
        const int g = g0 - lane;
        int gs = 0;
        if (g >= gw) {
          // 16-byte reads, the chunk order rotated by lane (fewer bank conflicts)
          const uint4* hp = reinterpret_cast<const uint4*>(hist + g * kGB);
#pragma unroll
          for (int q = 0; q < kGB / 4; ++q) {
            const uint4 v4 = hp[(q + lane) & (kGB / 4 - 1)];
            gs += (int)(v4.x + v4.y + v4.z + v4.w);
          }
        }
        int x = gs;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {   // inclusive scan, lane 0 = top group
          const int y = __shfl_up(x, o);
          if (lane >= o) x += y;
        }
        const unsigned long long hit = __ballot(total + x >= K);
        if (hit) {
          const int lg = __builtin_ctzll(hit);
          const int grp = g0 - lg;
          const int above = total + __shfl(x - gs, lg);   // counted above the group
          // lane i < 32 takes bin grp * 32 + 31 - i (descending)
          int y = lane < kGB ? (int)__atomic_load_n(&hist[grp * kGB + kGB - 1 - lane],
                                                    __ATOMIC_RELAXED) : 0;
#pragma unroll
          for (int o = 1; o < kGB; o <<= 1) {
            const int yy = __shfl_up(y, o);
            if (lane >= o) y += yy;
          }
          // counts only grow, so the group's bins reach k again
          const unsigned long long hit2 = __ballot(lane < kGB && above + y >= K);
          found = hit2 ? grp * kGB + kGB - 1 - __builtin_ctzll(hit2) : -1;
        }
        total += __shfl(x, kWave - 1);
      }
      if (found > b_w) {
        b_w = found;
        thr = bin_floor(b_w);
        int kept = 0;
        for (int base = 0; base < cnt; base += kWave) {
          const int i = base + lane;
          const unsigned long long kv = i < cnt ? buf[i] : 0ull;
          const bool keep = i < cnt && bin_of((uint32_t)(kv >> 32)) >= b_w;
          const unsigned long long bal = __ballot(keep);
          // every lane of the group has read before any lane writes
          if (keep) buf[kept + lane_rank(bal)] = kv;
          kept += __builtin_popcountll(bal);
        }
        if (lane == 0) wcnt[w] = (unsigned)kept;
      }
    };

    // A candidate (x >= thr, so its bin is >= b_w): counted in the histogram
    // and appended to the wave's buffer by its own lane, with LDS atomics; no
    // other lane takes part, so rare candidates cost little.  Past the
    // buffer's capacity the count still grows (the row then takes the exact
    // fallback) and the histogram stays exact.
    auto push = [&](float x, int id) {
      const uint32_t kx = okey(x);
      atomicAdd(&hist[bin_of(kx)], 1u);
      const unsigned pos = atomicAdd(&wcnt[w], 1u);
      if (pos < (unsigned)cap) buf[pos] = key64(x, (uint32_t)id);
    };

    // Element i (run time) of a packed vector: a select chain.
    auto elem_rt = [](const Raw& w, int i) -> float {
      float x = IO::elem(w, 0);
#pragma unroll
      for (int q = 1; q < N; ++q) x = (i == q) ? IO::elem(w, q) : x;
      return x;
    };
    // One tile of kRU vectors per lane: the maxima, one rescale of the running
    // sum, the exp sums.  Vectors whose maximum reaches the bound are only
    // flagged here; their elements are tested and pushed afterwards by the
    // lanes that hold them (few once the bound has risen).
    auto tile = [&](const Raw (&r)[kRU], int j0) {
      float v[kRU][N];
      float m_run = m_t;
      uint32_t cmask = 0u;
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        IO::unpack(r[u], v[u]);
        float vm = v[u][0];
#pragma unroll
        for (int i = 1; i < N; ++i) vm = fmaxf(vm, v[u][i]);
        m_run = fmaxf(m_run, vm);
        const bool act = j0 + u * B + t < n_full;
        cmask |= (act && vm >= thr) ? (1u << u) : 0u;
      }
      s_t *= exp2_fast((m_t - m_run) * c);   // exactly 1 unless the max rose
      m_t = m_run;
      float ts = 0.f;   // the tile's terms (kRU N of them) in fp32 first
#pragma unroll
      for (int u = 0; u < kRU; ++u)
#pragma unroll
        for (int i = 0; i < N; ++i) ts += exp2_fast((v[u][i] - m_t) * c);
      s_t += ts;
      if (cmask) {
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
          if (!((cmask >> u) & 1u)) continue;
          float x[N];
          IO::unpack(r[u], x);
          uint32_t em = 0u;
#pragma unroll
          for (int i = 0; i < N; ++i) em |= (x[i] >= thr) ? (1u << i) : 0u;
          const int jv = j0 + u * B + t;
          for (; em; em &= em - 1u) {
            const int i = __builtin_ctz(em);
            push(elem_rt(r[u], i), jv * N + i);
          }
        }
      }
    };

    // Uniform trip count for every thread: tiles of kRU vectors per thread.
    // The next tile is loaded before the current one is processed, so every
    // wave keeps a tile of loads in flight while it computes.
    int iter = 0;
    Raw nx[kRU];
    auto load_tile = [&](Raw (&r)[kRU], int j0) {
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        const int j = j0 + u * B + t;
        r[u] = j < n_full ? IO::template load<true>(zrow, j) : IO::ninf();   // streamed once
      }
    };
    if (n_full > 0) load_tile(nx, 0);
    for (int j0 = 0; j0 < n_full; j0 += B * kRU, ++iter) {
      Raw r[kRU];
#pragma unroll
      for (int u = 0; u < kRU; ++u) r[u] = nx[u];
      if (j0 + B * kRU < n_full) load_tile(nx, j0 + B * kRU);
      if (iter > 0 && ((iter & (iter + 1)) == 0 ||
                       __builtin_amdgcn_readfirstlane(
                           (int)__atomic_load_n(&wcnt[w], __ATOMIC_RELAXED)) > cap / 2))
        refresh();                             // tiles 1, 3, 7, 15, ... or a filling buffer
      if (iter == 0 && K <= B) {
        // Initial bound: the k-th largest of the B per-thread maxima of this
        // tile is at most the row's k-th largest logit (they are k distinct
        // elements), so its bin is a valid b_w.  The maxima are counted in
        // the histogram only to find that bin, then removed again.
        float tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
          float v[N];
          IO::unpack(r[u], v);
#pragma unroll
          for (int i = 0; i < N; ++i) tm = fmaxf(tm, v[i]);
        }
        const int tb = bin_of(okey(tm));       // NaN maxima only lower the bound
        atomicAdd(&hist[tb], 1u);
        __syncthreads();
        int b0 = 0, ab0 = 0;
        find_kth(K, b0, ab0);
        atomicSub(&hist[tb], 1u);
        if (t == 0) atomicMax(&sh_u[4], (unsigned)bin_of(okey(tm)));
        __syncthreads();
        b_w = b0;
        thr = bin_floor(b_w);
      }
      tile(r, j0);
    }
    // the partial last vector (vocab not a multiple of N): its owner lane
    if (rem > 0) {
      const bool mine = t == (n_full % B);
      float v[N];
#pragma unroll
      for (int i = 0; i < N; ++i)
        v[i] = (mine && i < rem) ? load_elem(zrow, n_full * N + i) : -INFINITY;
      float vm = -INFINITY;
#pragma unroll
      for (int i = 0; i < N; ++i) vm = fmaxf(vm, v[i]);
      if (mine) {
        const float mn = fmaxf(m_t, vm);
        s_t *= exp2_fast((m_t - mn) * c);
        m_t = mn;
#pragma unroll
        for (int i = 0; i < N; ++i) s_t += exp2_fast((v[i] - m_t) * c);
      }
      if (mine && vm >= thr) {
#pragma unroll
        for (int i = 0; i < N; ++i)
          if (i < rem && v[i] >= thr) push(v[i], n_full * N + i);
      }
    }
    __syncthreads();                           // every push is done
    if (lane == 0 && wcnt[w] > (unsigned)cap) atomicOr(&sh_u[1], 1u);

    // row max and sum
    float mv = m_t;
    int dummy = 0;
    block_argmax<B>(mv, dummy, redf, redi);
    const float m = mv;
    double part[1] = {(double)s_t * (double)exp2_fast((m_t - m) * c)};
    block_sum<B, 1>(part, redd);
    const float log2s = (float)log2(part[0]);
    // a NaN logit makes the sum NaN (exp2 propagates it), +inf makes the max
    // +inf, an all -inf row leaves the max at -FLT_MAX
    if (t == 0 && (!(m > -FLT_MAX) || !(m < INFINITY) || !(part[0] < INFINITY)))
      atomicOr(&sh_u[0], (unsigned)SC_DEV_NONFINITE);

    if (t == 0) { sh_i[0] = 0; sh_i[1] = 0; }
    int bstar = 0, above = 0;
    find_kth(K, bstar, above);
    int count_at = (int)hist[bstar];
    const uint32_t flags0 = sh_u[0];
    const bool fast = sh_u[1] == 0u && above + count_at <= kSortMax;
    __syncthreads();                     // histogram reads done before the overlay

    // --------------------------------------------------------- collect
    int n_cand = 0;
    if (flags0) {
      n_cand = 0;
    } else if (fast) {
      const int nb = min((int)wcnt[w], cap);
      for (int i = lane; i < nb; i += kWave) {
        const unsigned long long kv = buf[i];
        if (bin_of((uint32_t)(kv >> 32)) >= bstar) {
          const unsigned int pos = atomicAdd(&sh_u[2], 1u);
          if (pos < (unsigned)kSortMax) sarr[pos] = kv;
        }
      }
      __syncthreads();
      n_cand = (int)sh_u[2];
    } else {
      // Exact fallback: radix selection over the remaining key bits, one
      // more pass over the row per level, then a collection pass.
      unsigned long long prefix = (unsigned long long)bstar;
      int pbits = kHBits;
      int need = K - above;
      while (pbits < 64 && above + count_at > kSortMax) {
        const int nb = min(kHBits, 64 - pbits);
        const int shift = 64 - pbits - nb;
        for (int i = t; i < kNBins; i += B) hist[i] = 0u;
        __syncthreads();
        for (int id = t; id < V; id += B) {
          const unsigned long long kv = key64(load_elem(zrow, id), (uint32_t)id);
          if ((kv >> (64 - pbits)) == prefix)
            atomicAdd(&hist[(int)((kv >> shift) & ((1ull << nb) - 1ull))], 1u);
        }
        __syncthreads();
        int d = 0, ab = 0;
        find_kth(need, d, ab);
        count_at = (int)hist[d];
        above += ab;
        need -= ab;
        prefix = (prefix << nb) | (unsigned long long)d;
        pbits += nb;
        __syncthreads();
      }
      for (int id = t; id < V; id += B) {
        const unsigned long long kv = key64(load_elem(zrow, id), (uint32_t)id);
        if ((kv >> (64 - pbits)) >= prefix) {
          const unsigned int pos = atomicAdd(&sh_u[2], 1u);
          if (pos < (unsigned)kSortMax) sarr[pos] = kv;
        }
      }
      __syncthreads();
      n_cand = (int)sh_u[2];
    }
    n_cand = min(n_cand, kSortMax);

    // -------------------------------------------- order the candidates
    // Small sets: each key's rank is the number of larger keys (all keys are
    // distinct); the first k go to `ord` (the wave buffers, free now).
    // Larger sets: bitonic sort of sarr in place.
    unsigned long long* ord = reinterpret_cast<unsigned long long*>(lds + kNBins * 4);
    const bool by_rank = n_cand <= kRankMax;
    if (by_rank) {
      // zero keys pad the set to a multiple of 4 (a zero key is below every
      // real one), so every thread reads it 32 bytes at a time
      const int n4 = (n_cand + 3) & ~3;
      if (t < n4 - n_cand) sarr[n_cand + t] = 0ull;
      __syncthreads();
      for (int i = t; i < n_cand; i += B) {
        const unsigned long long ki = sarr[i];
        int rank = 0;
        for (int j2 = 0; j2 < n4; j2 += 4) {
          const ulonglong2 a0 = *reinterpret_cast<const ulonglong2*>(sarr + j2);
          const ulonglong2 a1 = *reinterpret_cast<const ulonglong2*>(sarr + j2 + 2);
          rank += (a0.x > ki ? 1 : 0) + (a0.y > ki ? 1 : 0) + (a1.x > ki ? 1 : 0) +
                  (a1.y > ki ? 1 : 0);
        }
        if (rank < K) ord[rank] = ki;
      }
      __syncthreads();
    }
    int P2 = 1;
    while (!by_rank && P2 < n_cand) P2 <<= 1;
    for (int i = n_cand + t; i < P2; i += B) sarr[i] = 0ull;
    __syncthreads();
    for (int k2 = 2; k2 <= P2; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        for (int i = t; i < P2; i += B) {
          const int ij = i ^ j;
          if (ij > i) {
            const unsigned long long x = sarr[i], y = sarr[ij];
            if ((x < y) == ((i & k2) == 0)) { sarr[i] = y; sarr[ij] = x; }
          }
        }
        __syncthreads();
      }
    }

    // ------------------------------------------------------------- outputs
    uint32_t flags = flags0;
    int32_t a = -1;
    if (P.sampled) {
      a = P.sampled[row];
      if (a < 0 || a >= V) flags |= SC_DEV_BAD_SAMPLED;
    }
    float za = 0.f;
    if (a >= 0 && a < V) {
      za = load_elem(zrow, a);
      if (za == -INFINITY) flags |= SC_DEV_NONFINITE;
    }
    for (int k = t; k < K; k += B) {
      int32_t id = -1;
      float q = qnan;
      if (!flags) {
        const unsigned long long kv = by_rank ? ord[k] : sarr[k];
        id = (int32_t)(~(uint32_t)(kv & 0xffffffffull));
        const float z = okey_value((uint32_t)(kv >> 32));
        q = exp2_fast((z - m) * c - log2s + 32.f) * 0x1p-32f;   // subnormal-exact
      }
      P.head_ids[row * K + k] = id;
      P.head_probs[row * K + k] = q;
    }
    if (t == 0) {
      // log p(a) in float64: the logit difference is exact there, and the
      // fp32 log-sum-exp of the row enters only through log2 of its sum
      const double lpa = (((double)za - (double)m) * P.c64 - log2(part[0])) *
                         0.6931471805599453;
      if (P.sampled_logp) P.sampled_logp[row] = (flags || a < 0) ? qnan : (float)lpa;
      if (flags) sh_u[3] |= flags;
    }
  }
  __syncthreads();
  if (t == 0 && sh_u[3] && P.dev_status) atomicOr(P.dev_status, sh_u[3]);
}

}  // namespace

// Per-wave buffer: room for the rank output (k keys over all waves) too.
int record_cap(int k) { return k <= 256 ? 512 : 1024; }

size_t record_lds_bytes(int k) {
  return (size_t)kNBins * 4 + (size_t)kRNW * record_cap(k) * 8;
}

// One workgroup per row: rows take different times (their candidate
// counts differ), and the hardware's dispatch of the next workgroup to
// whichever slot frees up balances them (a persistent grid of the resident
// count, rows assigned in turn, took 10% longer).
hipError_t launch_record(RecParams P, hipStream_t s) {
  P.cap = record_cap(P.k);
  const size_t lds = record_lds_bytes(P.k);
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)P.n_rows), dim3(kRB), lds, s, P);
    return hipGetLastError();
  };
  if (P.in_dtype == 1)
    return P.vector ? go(k_record<uint16_t, true>) : go(k_record<uint16_t, false>);
  return P.vector ? go(k_record<float, true>) : go(k_record<float, false>);
}

}  // namespace sc
