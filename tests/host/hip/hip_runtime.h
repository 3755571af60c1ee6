// Host emulation of the HIP device environment the library's kernels use,
// for running them on the CPU under AddressSanitizer and UndefinedBehavior-
// Sanitizer.  Test infrastructure only: it never runs on a GPU and the
// library never includes it (the harness build puts this directory first on
// the include path).
//
// One workgroup runs at a time.  Every GPU thread is a fiber;
// __syncthreads is a workgroup barrier and the wave operations (shuffles, the
// 32x32x16 bf16 MFMA) are wave barriers that switch fibers, so a missing or
// divergent barrier shows up as a deadlock report.  Buffer-resource accesses
// are bounds checked against the resource's size: a load past it returns
// zeros (as on the GPU) and is counted, a store past it is dropped and
// counted unless its offset is the deliberate skip offset (>= 2^31).
#pragma once
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cfloat>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(x)
#define __shared__ static
#define amdgpu_waves_per_eu(x)
#define __align__(x) __attribute__((aligned(x)))
#define HIP_SYMBOL(x) (x)

typedef int hipError_t;
typedef void* hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidDevice = 101 };
enum { hipFuncAttributeMaxDynamicSharedMemorySize = 8 };
inline hipError_t hipFuncSetAttribute(const void*, int, int) { return hipSuccess; }
inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  return hipSuccess;
}

namespace emu {
struct Dim { unsigned x = 1, y = 1, z = 1; };
struct Fiber {
  void* sp = nullptr;          // saved stack pointer while switched out
  int state = 0;               // 0 runnable, 1 at a block barrier, 2 at a wave barrier, 3 done
  unsigned long long gen = 0;
  std::vector<char> stack;
};
extern int cur;                  // running fiber (thread index in the workgroup)
extern int nthreads;
extern Fiber* fibers;
extern unsigned long long block_gen, wave_gen[64];
extern int block_arrived, wave_arrived[64];
extern unsigned char shfl_buf[2][64][64][8];
extern float mfma_a[2][64][64][8], mfma_b[2][64][64][8];
extern unsigned char exch_parity[64 * 64];   // per thread: which exchange buffer is next
extern Dim bid, gdim, bdim;
extern unsigned char* dyn_lds;
extern long oob_loads, oob_stores;
void yield_block();
void yield_wave();
void run_block(void (*body)(void*), void* arg, unsigned nthr);

// Separate heap allocation per named LDS array of the row kernels (the source
// transform routes them here), so that an index past one array is reported
// even where the real layout would place it inside a neighbour.
struct LdsArrays { std::vector<std::vector<unsigned char>> bufs; };
extern LdsArrays* lds_arrays;
template <class T> T* lds_arr(int idx, long count) {
  auto& v = lds_arrays->bufs[idx];
  if (v.empty()) v.resize((size_t)(count > 0 ? count : 1) * sizeof(T));
  return reinterpret_cast<T*>(v.data());
}
}  // namespace emu

#define threadIdx (::emu::Dim{(unsigned)::emu::cur, 0, 0})
#define blockIdx (::emu::bid)
#define gridDim (::emu::gdim)
#define blockDim (::emu::bdim)

inline void __syncthreads() { emu::yield_block(); }
inline void __threadfence() {}
inline void __threadfence_block() {}

// Wave exchanges (shuffles, MFMA operands) alternate between two buffers:
// a lane writes buffer b of exchange n + 2 only after the wave barrier of
// exchange n + 1, which every lane reaches after reading exchange n, so one
// barrier per exchange suffices.
inline int emu_next_buffer() {
  const int b = emu::exch_parity[emu::cur];
  emu::exch_parity[emu::cur] = (unsigned char)(b ^ 1);
  return b;
}

// Wave shuffles: every lane deposits its value, the wave meets, every lane
// reads its source lane's value.
template <class T> inline T emu_shfl(T v, int kind, int arg) {
  static_assert(sizeof(T) <= 8, "shuffle of at most 8 bytes");
  const int lane = emu::cur % 64, w = emu::cur / 64, b = emu_next_buffer();
  memcpy(emu::shfl_buf[b][w][lane], &v, sizeof(T));
  emu::yield_wave();
  int src;
  if (kind == 0) src = lane ^ arg;                       // xor
  else if (kind == 1) src = arg & 63;                    // broadcast
  else src = lane - arg < 0 ? lane : lane - arg;         // up
  T r;
  memcpy(&r, emu::shfl_buf[b][w][src], sizeof(T));
  return r;
}
// Ballot: every lane deposits its predicate, the wave meets, every lane
// reads all 64 (lanes past a partial last wave read as false).
inline unsigned long long __ballot(int pred) {
  const int lane = emu::cur % 64, w = emu::cur / 64, b = emu_next_buffer();
  emu::shfl_buf[b][w][lane][0] = pred ? 1 : 0;
  emu::yield_wave();
  const int wsize = emu::nthreads - w * 64 < 64 ? emu::nthreads - w * 64 : 64;
  unsigned long long m = 0;
  for (int l = 0; l < wsize; ++l) m |= (unsigned long long)(emu::shfl_buf[b][w][l][0] & 1) << l;
  return m;
}
// Lane counts: src1 plus the bits of src0 that belong to lower lanes (the low
// word covers lanes 0-31, the high word lanes 32-63).
inline uint32_t emu_mbcnt_lo(uint32_t m, uint32_t acc) {
  const int lane = emu::cur % 64;
  const uint32_t below = lane >= 32 ? 0xffffffffu : ((1u << lane) - 1u);
  return acc + (uint32_t)__builtin_popcount(m & below);
}
inline uint32_t emu_mbcnt_hi(uint32_t m, uint32_t acc) {
  const int lane = emu::cur % 64;
  const uint32_t below = lane < 32 ? 0u : ((1u << (lane - 32)) - 1u);
  return acc + (uint32_t)__builtin_popcount(m & below);
}
#define __builtin_amdgcn_mbcnt_lo emu_mbcnt_lo
#define __builtin_amdgcn_mbcnt_hi emu_mbcnt_hi
template <class T> inline T __shfl_xor(T v, int m, int = 64) { return emu_shfl(v, 0, m); }
template <class T> inline T __shfl(T v, int s, int = 64) { return emu_shfl(v, 1, s); }
template <class T> inline T __shfl_up(T v, unsigned d, int = 64) { return emu_shfl(v, 2, (int)d); }

// Fibers never run concurrently: plain read-modify-write is atomic here.
template <class T> inline T atomicCAS(T* p, T cmp, T val) { T o = *p; if (o == cmp) *p = val; return o; }
template <class T> inline T atomicOr(T* p, T v) { T o = *p; *p = o | v; return o; }
template <class T> inline T atomicMin(T* p, T v) { T o = *p; *p = o < v ? o : v; return o; }
template <class T> inline T atomicMax(T* p, T v) { T o = *p; *p = o > v ? o : v; return o; }
template <class T> inline T atomicAdd(T* p, T v) { T o = *p; *p = o + v; return o; }
template <class T> inline T atomicSub(T* p, T v) { T o = *p; *p = o - v; return o; }

#define __builtin_amdgcn_exp2f(x) exp2f(x)
// Lane 0's value for the whole wave (a wave collective: every lane of the
// wave must call it).
inline int emu_readfirstlane(int v) {
  const int lane = emu::cur % 64, w = emu::cur / 64, b = emu_next_buffer();
  memcpy(emu::shfl_buf[b][w][lane], &v, sizeof(int));
  emu::yield_wave();
  int r;
  memcpy(&r, emu::shfl_buf[b][w][0], sizeof(int));
  return r;
}
#define __builtin_amdgcn_readfirstlane(x) emu_readfirstlane(x)
// The fibers of a wave do not run in lockstep: a wave barrier stands in for
// it where the kernel relies on it.
#define __builtin_amdgcn_wave_barrier() ::emu::yield_wave()
#define __builtin_amdgcn_s_setprio(x) ((void)0)
#define __builtin_amdgcn_iglp_opt(x) ((void)0)
inline long long clock64() { return 0; }
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
inline float __int_as_float(int u) { float f; memcpy(&f, &u, 4); return f; }
inline int __float_as_int(float f) { int u; memcpy(&u, &f, 4); return u; }
struct float4 { float x, y, z, w; };
struct alignas(16) uint4 { unsigned int x, y, z, w; };
struct alignas(16) ulonglong2 { unsigned long long x, y; };
inline float4 make_float4(float a, float b, float c, float d) { return float4{a, b, c, d}; }

// v_mfma_f32_32x32x16_bf16: D = C + A B^T over one wave.  Lane l holds
// A[l % 32][8 (l / 32) + j] and B[l % 32][8 (l / 32) + j], j < 8, and
// returns D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32] in element i < 16.  The
// 16 products of an element are summed in float64 and added to C once.
typedef float emu_f32x16 __attribute__((ext_vector_type(16)));
template <class BF8>
inline emu_f32x16 emu_mfma_32x32x16_bf16(BF8 a, BF8 b, emu_f32x16 c, int, int, int) {
  const int lane = emu::cur % 64, w = emu::cur / 64, e = emu_next_buffer();
  for (int j = 0; j < 8; ++j) {
    emu::mfma_a[e][w][lane][j] = (float)a[j];
    emu::mfma_b[e][w][lane][j] = (float)b[j];
  }
  emu::yield_wave();
  emu_f32x16 d = c;
  const int col = lane % 32, h = lane / 32;
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i / 4) + 4 * h + (i % 4);
    double s = 0.0;
    for (int k = 0; k < 16; ++k)
      s += (double)emu::mfma_a[e][w][row + 32 * (k / 8)][k % 8] *
           (double)emu::mfma_b[e][w][col + 32 * (k / 8)][k % 8];
    d[i] = (float)((double)c[i] + s);
  }
  return d;
}
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16 emu_mfma_32x32x16_bf16

// Buffer resources: base and size in bytes (raw addressing).
struct emu_rsrc { unsigned char* base; uint32_t bytes; };
#define __amdgpu_buffer_rsrc_t emu_rsrc
inline emu_rsrc emu_make_rsrc(void* p, short, int n, int) {
  return emu_rsrc{static_cast<unsigned char*>(p), (uint32_t)n};
}
#define __builtin_amdgcn_make_buffer_rsrc emu_make_rsrc
typedef uint32_t emu_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t emu_u32x2 __attribute__((ext_vector_type(2)));
inline emu_u32x4 emu_bload128(emu_rsrc r, uint32_t off, int soff, int) {
  emu_u32x4 v = {0u, 0u, 0u, 0u};
  if (soff != 0 || (uint64_t)off + 16 > r.bytes) { ++emu::oob_loads; return v; }
  memcpy(&v, r.base + off, 16);
  return v;
}
#define __builtin_amdgcn_raw_buffer_load_b128 emu_bload128
template <class V>
inline void emu_bstore(const V& v, emu_rsrc r, uint32_t off, int soff) {
  if (off >= 0x80000000u) return;                       // deliberate skip
  if (soff != 0 || (uint64_t)off + sizeof(V) > r.bytes) {
    ++emu::oob_stores;
    fprintf(stderr, "EMU OUT-OF-RANGE STORE offset %u size %u\n", off, r.bytes);
    return;
  }
  memcpy(r.base + off, &v, sizeof(V));
}
inline void emu_bstore128(emu_u32x4 v, emu_rsrc r, uint32_t off, int soff, int) { emu_bstore(v, r, off, soff); }
inline void emu_bstore64(emu_u32x2 v, emu_rsrc r, uint32_t off, int soff, int) { emu_bstore(v, r, off, soff); }
#define __builtin_amdgcn_raw_buffer_store_b128 emu_bstore128
#define __builtin_amdgcn_raw_buffer_store_b64 emu_bstore64

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

namespace emu {
template <class F> struct Thunk {
  F f;
  static void call(void* p) { static_cast<Thunk*>(p)->f(); }
};
// Runs every workgroup of a launch in turn (x and y grid dimensions).
template <class... A, class... B>
void launch(void (*kern)(A...), dim3 grid, dim3 block, size_t lds, B... args) {
  gdim = Dim{grid.x, grid.y, 1};
  bdim = Dim{block.x, 1, 1};
  for (unsigned by = 0; by < grid.y; ++by)
    for (unsigned bx = 0; bx < grid.x; ++bx) {
      bid = Dim{bx, by, 0};
      std::vector<unsigned char> mem(lds ? lds : 1);
      dyn_lds = mem.data();
      LdsArrays arrays;
      arrays.bufs.resize(16);
      lds_arrays = &arrays;
      auto f = [&]() { kern(args...); };
      Thunk<decltype(f)> th{f};
      run_block(&Thunk<decltype(f)>::call, &th, block.x);
    }
}
}  // namespace emu
#define hipLaunchKernelGGL(kern, grid, block, lds, stream, ...) \
  ::emu::launch(kern, grid, block, lds, __VA_ARGS__)
