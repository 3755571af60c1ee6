// Fiber scheduler of the host emulation (see hip/hip_runtime.h): runs the
// threads of one workgroup as fibers, releasing a block barrier when every
// thread has reached it and a wave barrier when every thread of that wave
// has; a round in which no fiber can move is reported as a deadlock.
//
// Fibers switch through emu_switch (x86-64: the callee-saved registers, the
// SSE and x87 control words and the stack pointer), which, unlike glibc's
// swapcontext, makes no system call; every switch is announced to
// AddressSanitizer with its fiber interface so that it tracks the stacks.
#include <hip/hip_runtime.h>

#include <algorithm>

extern "C" {
void emu_switch(void** save_sp, void* load_sp);
void __sanitizer_start_switch_fiber(void** fake_stack_save, const void* bottom, size_t size);
void __sanitizer_finish_switch_fiber(void* fake_stack_save, const void** bottom_old,
                                     size_t* size_old);
void __asan_unpoison_memory_region(void const volatile* addr, size_t size);
}

asm(R"(
  .text
  .globl emu_switch
  .type emu_switch, @function
emu_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  subq $8, %rsp
  stmxcsr (%rsp)
  fnstcw 4(%rsp)
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  ldmxcsr (%rsp)
  fldcw 4(%rsp)
  addq $8, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size emu_switch, .-emu_switch
)");

namespace emu {
int cur;
int nthreads;
Fiber* fibers;
unsigned long long block_gen, wave_gen[64];
int block_arrived, wave_arrived[64];
unsigned char shfl_buf[2][64][64][8];
float mfma_a[2][64][64][8], mfma_b[2][64][64][8];
unsigned char exch_parity[64 * 64];
Dim bid, gdim, bdim;
unsigned char* dyn_lds;
LdsArrays* lds_arrays;
long oob_loads, oob_stores;

static void (*g_body)(void*);
static void* g_arg;
static void* sched_sp;                 // the scheduler's saved stack pointer
static const void* main_bottom;        // the scheduler's stack, for the sanitizer
static size_t main_size;

static void to_scheduler(bool dying) {
  void* fake = nullptr;
  __sanitizer_start_switch_fiber(dying ? nullptr : &fake, main_bottom, main_size);
  emu_switch(&fibers[cur].sp, sched_sp);
  __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
}

static void to_fiber(int i) {
  void* fake = nullptr;
  __sanitizer_start_switch_fiber(&fake, fibers[i].stack.data(), fibers[i].stack.size());
  emu_switch(&sched_sp, fibers[i].sp);
  __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
}

// First code of every fiber (entered by emu_switch's return).
static void fiber_entry() {
  __sanitizer_finish_switch_fiber(nullptr, &main_bottom, &main_size);
  g_body(g_arg);
  fibers[cur].state = 3;
  to_scheduler(true);
  abort();  // a finished fiber is never resumed
}

void yield_block() {
  Fiber& f = fibers[cur];
  f.state = 1;
  f.gen = block_gen;
  if (++block_arrived == nthreads) { block_arrived = 0; ++block_gen; }
  to_scheduler(false);
}

void yield_wave() {
  const int w = cur / 64;
  const int wsize = std::min(64, nthreads - w * 64);
  Fiber& f = fibers[cur];
  f.state = 2;
  f.gen = wave_gen[w];
  if (++wave_arrived[w] == wsize) { wave_arrived[w] = 0; ++wave_gen[w]; }
  to_scheduler(false);
}

// A new fiber's stack holds what emu_switch pops: the control words, six
// registers and the return address fiber_entry, placed so that the stack is
// 16-byte aligned minus 8 at fiber_entry's first instruction, as after a call.
static void init_stack(Fiber& f) {
  if (f.stack.empty()) f.stack.resize(1 << 18);
  // a reused stack still carries the redzones of the frames a finished
  // fiber left on it (fiber_entry never returns): clear them
  __asan_unpoison_memory_region(f.stack.data(), f.stack.size());
  uintptr_t top = ((uintptr_t)f.stack.data() + f.stack.size()) & ~(uintptr_t)15;
  uint64_t* sp = reinterpret_cast<uint64_t*>(top) - 2;   // [entry] [pad], 16-aligned
  sp[0] = (uint64_t)(uintptr_t)&fiber_entry;
  sp -= 6;                                               // rbp rbx r12 r13 r14 r15
  for (int i = 0; i < 6; ++i) sp[i] = 0;
  sp -= 1;                                               // mxcsr, x87 control word
  uint32_t mx;
  uint16_t cw;
  asm volatile("stmxcsr %0" : "=m"(mx));
  asm volatile("fnstcw %0" : "=m"(cw));
  uint32_t words[2] = {mx, cw};
  memcpy(sp, words, 8);
  f.sp = sp;
}

void run_block(void (*body)(void*), void* arg, unsigned nthr) {
  if (nthr > 64 * 64) { fprintf(stderr, "EMU: workgroup too large\n"); abort(); }
  g_body = body;
  g_arg = arg;
  nthreads = (int)nthr;
  // fibers and their stacks are kept from one workgroup to the next (a
  // fresh 256 KiB stack per thread and workgroup costs more than the work)
  static std::vector<Fiber> fs;
  if (fs.size() < nthr) fs.resize(nthr);
  for (unsigned i = 0; i < nthr; ++i) { fs[i].state = 0; fs[i].gen = 0; }
  fibers = fs.data();
  block_gen = 0;
  block_arrived = 0;
  for (int w = 0; w < 64; ++w) { wave_gen[w] = 0; wave_arrived[w] = 0; }
  memset(exch_parity, 0, sizeof(exch_parity));
  for (unsigned i = 0; i < nthr; ++i) init_stack(fs[i]);
  for (;;) {
    bool progress = false, all_done = true;
    for (unsigned i = 0; i < nthr; ++i) {
      Fiber& f = fs[i];
      if (f.state == 3) continue;
      all_done = false;
      const bool ready = f.state == 0 || (f.state == 1 && block_gen > f.gen) ||
                         (f.state == 2 && wave_gen[i / 64] > f.gen);
      if (!ready) continue;
      f.state = 0;
      cur = (int)i;
      to_fiber((int)i);
      progress = true;
    }
    if (all_done) break;
    if (!progress) {
      fprintf(stderr, "EMU DEADLOCK: workgroup (%u, %u), thread states:", bid.x, bid.y);
      for (unsigned i = 0; i < nthr; ++i) fprintf(stderr, " %d", fs[i].state);
      fprintf(stderr, "\n");
      abort();
    }
  }
}
}  // namespace emu
