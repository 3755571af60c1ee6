// Device-side building blocks of the SC kernels for gfx950 (wave64).
//
// Wave and workgroup reductions, 16-byte vector access to bf16 / fp32 rows,
// the per-row set of recorded ids kept in LDS, and fp32 -> bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr double kClamp = 1e-6;  // clamp constant of rho (Score Centering)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define SC_DEV __device__ __forceinline__

SC_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes, butterfly over __shfl_xor)
// ---------------------------------------------------------------------------
SC_DEV float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <typename F>
SC_DEV F wave_sum(F v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
SC_DEV uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}
// (value, index) maximum; equal values keep the lower index.
SC_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// Workgroup reductions through a small LDS scratch.  Every thread of the
// block must call them (they contain barriers); the result is returned to all
// threads.  Each wave writes its partial, then every wave combines the B / 64
// partials with a fixed butterfly, so the order is the same for all threads
// and all runs.
template <int B>
SC_DEV void block_argmax(float& v, int& i, float* redf, int* redi) {
  constexpr int NW = B / kWave;
  wave_argmax(v, i);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) { redf[w] = v; redi[w] = i; }
  __syncthreads();
  float x = l < NW ? redf[l] : -INFINITY;
  int xi = l < NW ? redi[l] : 0x7fffffff;
#pragma unroll
  for (int o = NW / 2; o > 0; o >>= 1) {
    const float ox = __shfl_xor(x, o);
    const int oi = __shfl_xor(xi, o);
    if (ox > x || (ox == x && oi < xi)) { x = ox; xi = oi; }
  }
  v = __shfl(x, 0);
  i = __shfl(xi, 0);
}

template <int B, int N, typename F>
SC_DEV void block_sum(F (&v)[N], F* red) {
  constexpr int NW = B / kWave;
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = wave_sum(v[n]);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) red[n * NW + w] = v[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    F x = l < NW ? red[n * NW + l] : F(0);
#pragma unroll
    for (int o = NW / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    v[n] = __shfl(x, 0);
  }
}

// Exclusive prefix sum of one int per thread over the workgroup (thread
// order); `total` gets the sum of all.  Every thread must call it.
template <int B>
SC_DEV int block_excl_scan(int v, int* red, int& total) {
  constexpr int NW = B / kWave;
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += l >= o ? y : 0;
  }
  __syncthreads();
  if (l == kWave - 1) red[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int r = red[i];
    base += i < w ? r : 0;
    tot += r;
  }
  total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Row element access.  A row is read as "vectors" of N consecutive elements:
// 16 bytes (N = 8 bf16 or 4 fp32) on the vector path, N = 1 on the scalar
// path.  bf16 is carried as its raw 16 bits.
// ---------------------------------------------------------------------------
SC_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (gfx950 converts in
// hardware, two values per v_cvt_pk_bf16_f32).
SC_DEV uint32_t f32_to_bf16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
// Two values in one v_cvt_pk_bf16_f32 (the pair converted as a vector).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
SC_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Buffer resource over the `bytes` bytes at p (raw addressing, gfx9 format
// word).  A buffer access whose offset lies at or beyond `bytes` reads zeros
// and drops a store, so the row streams read 16-byte vectors through one
// resource per row, and a store is skipped on purpose by giving it an offset
// of kSkip or more (bytes stays below 2^31).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kSkip = 0x80000000u;
SC_DEV rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a buffer access: 0 default, 2 nontemporal (last use).
constexpr int kNT = 2;

// RowIO<T, VECTOR>: `raw` is one vector as loaded (16 bytes, or one element
// on the scalar path); load() fetches vector n of a row, unpack() widens it to
// fp32 and ninf() is a vector of -inf (padding of a partial tile).  On the
// vector path bload() fetches the vector at byte offset `off` of a row
// resource.
template <typename T, bool VECTOR> struct RowIO;

template <> struct RowIO<uint16_t, true> {   // bf16, 16-byte vectors
  static constexpr int N = 8;
  typedef u32x4 raw;
  template <bool NT>
  static SC_DEV raw load(const uint16_t* row, int64_t n) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + n;
    return NT ? __builtin_nontemporal_load(p) : *p;
  }
  template <int AUX>
  static SC_DEV raw bload(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  }
  static SC_DEV void unpack(const raw& w, float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static SC_DEV raw ninf() { u32x4 w = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u}; return w; }
  static SC_DEV float elem(const raw& w, int i) {  // i is a compile-time constant after unrolling
    return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
  }
};
template <> struct RowIO<float, true> {      // fp32, 16-byte vectors
  static constexpr int N = 4;
  typedef f32x4 raw;
  template <bool NT>
  static SC_DEV raw load(const float* row, int64_t n) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row) + n;
    return NT ? __builtin_nontemporal_load(p) : *p;
  }
  template <int AUX>
  static SC_DEV raw bload(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
  }
  static SC_DEV void unpack(const raw& w, float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = w[i];
  }
  static SC_DEV raw ninf() { f32x4 w = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}; return w; }
  static SC_DEV float elem(const raw& w, int i) { return w[i]; }
};
template <> struct RowIO<uint16_t, false> {  // bf16, one element at a time
  static constexpr int N = 1;
  typedef uint32_t raw;
  template <bool NT>
  static SC_DEV raw load(const uint16_t* row, int64_t n) { return row[n]; }
  static SC_DEV void unpack(const raw& w, float (&v)[N]) { v[0] = __uint_as_float(w << 16); }
  static SC_DEV raw ninf() { return 0xff80u; }
  static SC_DEV float elem(const raw& w, int) { return __uint_as_float(w << 16); }
};
template <> struct RowIO<float, false> {     // fp32, one element at a time
  static constexpr int N = 1;
  typedef float raw;
  template <bool NT>
  static SC_DEV raw load(const float* row, int64_t n) { return row[n]; }
  static SC_DEV void unpack(const raw& w, float (&v)[N]) { v[0] = w; }
  static SC_DEV raw ninf() { return -INFINITY; }
  static SC_DEV float elem(const raw& w, int) { return w; }
};

SC_DEV float load_elem(const uint16_t* row, int64_t i) { return bf16_to_f32(row[i]); }
SC_DEV float load_elem(const float* row, int64_t i) { return row[i]; }

// Store N output values of one vector (bf16 bits or fp32), nontemporal.
// bstore() writes them at byte offset `off` of an output-row resource
// (BYTES = N x the element size); off >= kSkip drops the store.
template <typename O, int N> struct RowOut;
template <> struct RowOut<uint16_t, 8> {
  static constexpr uint32_t BYTES = 16;
  static SC_DEV u32x4 pack(const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    return w;
  }
  static SC_DEV void store(uint16_t* row, int64_t n, const float (&v)[8]) {
    __builtin_nontemporal_store(pack(v), reinterpret_cast<u32x4*>(row) + n);
  }
  static SC_DEV void bstore(rsrc_t r, uint32_t off, const float (&v)[8]) {
    __builtin_amdgcn_raw_buffer_store_b128(pack(v), r, off, 0, kNT);
  }
};
template <> struct RowOut<uint16_t, 4> {
  static constexpr uint32_t BYTES = 8;
  static SC_DEV u32x2 pack(const float (&v)[4]) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    return w;
  }
  static SC_DEV void store(uint16_t* row, int64_t n, const float (&v)[4]) {
    __builtin_nontemporal_store(pack(v), reinterpret_cast<u32x2*>(row) + n);
  }
  static SC_DEV void bstore(rsrc_t r, uint32_t off, const float (&v)[4]) {
    __builtin_amdgcn_raw_buffer_store_b64(pack(v), r, off, 0, kNT);
  }
};
template <> struct RowOut<float, 8> {
  static constexpr uint32_t BYTES = 32;
  static SC_DEV void store(float* row, int64_t n, const float (&v)[8]) {
    f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    f32x4* p = reinterpret_cast<f32x4*>(row) + 2 * n;
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  }
  static SC_DEV void bstore(rsrc_t r, uint32_t off, const float (&v)[8]) {
    const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), r, off, 0, kNT);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), r, off + 16u, 0, kNT);
  }
};
template <> struct RowOut<float, 4> {
  static constexpr uint32_t BYTES = 16;
  static SC_DEV void store(float* row, int64_t n, const float (&v)[4]) {
    f32x4 a = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(row) + n);
  }
  static SC_DEV void bstore(rsrc_t r, uint32_t off, const float (&v)[4]) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), r, off, 0, kNT);
  }
};
template <> struct RowOut<uint16_t, 1> {
  static constexpr uint32_t BYTES = 2;
  static SC_DEV void store(uint16_t* row, int64_t n, const float (&v)[1]) {
    row[n] = (uint16_t)f32_to_bf16(v[0]);
  }
};
template <> struct RowOut<float, 1> {
  static constexpr uint32_t BYTES = 4;
  static SC_DEV void store(float* row, int64_t n, const float (&v)[1]) { row[n] = v[0]; }
};

SC_DEV void store_elem(uint16_t* row, int64_t i, float v) { row[i] = (uint16_t)f32_to_bf16(v); }
SC_DEV void store_elem(float* row, int64_t i, float v) { row[i] = v; }

// Reference exponent of a running maximum x: ceil(x c_hi), an integer held in
// a float, clamped to +-2^60 so that it stays finite while nothing finite has
// been seen (x = -FLT_MAX) or when x is +inf (such a row is flagged).
SC_DEV float ref_exp(float x, float c_hi) {
  return fminf(fmaxf(ceilf(x * c_hi), -0x1p60f), 0x1p60f);
}

// Per-row constants of the pass-2 value sign(alpha) 2^((z - m) c - G):
// G = Gint + gq + glo with Gint an integer, gq on the 2^-14 grid in (-1, 0]
// and |glo| < 2^-14.
struct Pass2 {
  float m, c_hi, c_lo;
  float gq;      // gq (as above)
  float nglo;    // -glo ln 2
  float scl;     // sign(alpha) 2^-Gint (NaN for a flagged row, +-0 when all values underflow)
  float scl_lo;  // scl 2^-64, for exponents moved up by 64 (subnormal results)
};

// Pass-2 value of one logit z.  d = z - m is exact for bf16 z and m (else its
// rounding error de comes from a two-sum).  P = RN(d c_hi) and its exact
// residual Pe = d c_hi - P (one fma); yh = P - gq is exact because gq lies on
// a grid no finer than P's (|P| < 2^10) and shrinks |P|.  The small remainder
// k = ln 2 (Pe + d c_lo - glo) (|k| < 2^-14) is applied as 2^yh (1 + k), and
// the power of two comes last, in one multiply (a single rounding when the
// result is subnormal).  CAREFUL adds what rare rows need: -inf logits give 0
// (not NaN), fp32 logits take the two-sum, and exponents below -96 are moved
// up by 64 (back in the final multiply) so that the exp2 instruction, which
// flushes results below 2^-126, keeps them.
template <bool CAREFUL>
SC_DEV float p2_value(float z, const Pass2& Q) {
#pragma clang fp contract(off)
  float d = z - Q.m;
  float de = 0.f;
  if (CAREFUL) {
    const float zz = d + Q.m;          // two-sum of z and -m
    const float mm = d - zz;
    de = (z - zz) - (Q.m + mm);
    de = d >= -0x1p20f ? de : 0.f;     // -inf (or a NaN row): no residual
    d = fmaxf(d, -0x1p20f);
  }
  const float P = d * Q.c_hi;
  const float Pe = fmaf(d, Q.c_hi, -P);
  float yh = P - Q.gq;
  float scl = Q.scl;
  if (CAREFUL) {
    const bool low = yh < -96.f;
    yh = low ? yh + 64.f : yh;         // exact: the magnitude shrinks
    scl = low ? Q.scl_lo : scl;
  }
  const float r = CAREFUL ? fmaf(de, Q.c_hi, Pe) : Pe;
  const float k = fmaf(fmaf(d, Q.c_lo, r), kLn2, Q.nglo);
  const float e = exp2_fast(yh);
  return fmaf(e, k, e) * scl;
}

// Per-row constants for the value sign 2^((z - m) c - G), c = c_hi + c_lo:
// G = Gint + gq + glo split as above (Gint clamped at -126 for a factor
// beyond 2^126; G above 10^4, alpha = 0 included, makes every value a signed
// zero; a NaN G makes every value NaN).  g returns Gint (2^20 for a row of
// zeros, 0 for a NaN row).
SC_DEV Pass2 pass2_setup(float m, float c_hi, float c_lo, double G, bool neg, int& g) {
  Pass2 Q;
  Q.m = m;
  Q.c_hi = c_hi;
  Q.c_lo = c_lo;
  Q.gq = 0.f;
  Q.nglo = 0.f;
  Q.scl = __builtin_nanf("");
  Q.scl_lo = Q.scl;
  g = 0;
  const float sgn = neg ? -1.f : 1.f;
  if (!(G == G)) return Q;
  G = fmax(G, -1.0e4);
  if (G > 1.0e4) {
    Q.scl = 0.f * sgn;
    Q.scl_lo = Q.scl;
    g = 1 << 20;
    return Q;
  }
  double gi = ceil(G);
  double gq = ceil((G - gi) * 16384.0) / 16384.0;   // (-1, 0]
  const double glo = (G - gi) - gq;                 // (-2^-14, 0]
  if (gi < -126.0) { gq += gi + 126.0; gi = -126.0; }
  g = (int)gi;
  Q.gq = (float)gq;
  Q.nglo = (float)(-glo * 0.6931471805599453);
  Q.scl = g > 160 ? 0.f * sgn : ldexpf(sgn, -g);
  Q.scl_lo = g + 64 > 160 ? 0.f * sgn : ldexpf(sgn, -g - 64);
  return Q;
}

// ---------------------------------------------------------------------------
// Recorded-id set in LDS: open addressing with linear probing, id -> slot.
// Capacity is a power of two >= 2K, so probes always reach an empty key.
// ---------------------------------------------------------------------------
SC_DEV uint32_t id_hash(int32_t id, int shift) {
  return ((uint32_t)id * 0x9E3779B1u) >> shift;
}
// Returns false when `id` is already present (a duplicate record).
SC_DEV bool idset_insert(int* keys, int* vals, uint32_t mask, int shift,
                         int32_t id, int slot) {
  uint32_t h = id_hash(id, shift);
  for (;;) {
    int prev = atomicCAS(&keys[h], -1, id);
    if (prev == -1) { vals[h] = slot; return true; }
    if (prev == id) return false;
    h = (h + 1) & mask;
  }
}
SC_DEV int idset_find(const int* keys, const int* vals, uint32_t mask,
                      int shift, int32_t id) {
  uint32_t h = id_hash(id, shift);
  for (;;) {
    int key = keys[h];
    if (key == id) return vals[h];
    if (key == -1) return -1;
    h = (h + 1) & mask;
  }
}

}  // namespace sc
