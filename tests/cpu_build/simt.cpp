// Fiber scheduler and cross-lane operations of the host emulation (simt.h).
#include "simt.h"

#include <sys/mman.h>

#include <cstdarg>
#include <map>
#include <string>
#include <vector>

#if defined(__has_feature)
#if __has_feature(address_sanitizer)
#define SIMT_ASAN 1
#include <sanitizer/common_interface_defs.h>
#endif
#endif
// SIMT_TSAN: the kernels are built with ThreadSanitizer and this file, which
// is not instrumented, annotates the schedule: one TSan fiber per wave (its
// lanes are one program order, as in lockstep), switches without implied
// synchronisation, and a release/acquire pair per barrier generation of a
// workgroup.  Accesses of two waves of a workgroup that no barrier orders are
// then reported as data races.  Workgroups are ordered one after another: the
// __shared__ arrays here are one static object that every workgroup reuses,
// where the hardware gives each its own LDS.  With SIMT_TSAN_LANES=1 in the
// environment every lane is a fiber of its own, ordered with the other lanes
// of its wave only by the wave's cross-lane operations and wave barriers (a
// release/acquire pair per wave-operation generation) and by the workgroup's
// barriers: an exchange between lanes of one wave through memory with no such
// point between the write and the read is then reported too.  On the hardware
// such an exchange relies on the compiler keeping the accesses in program
// order, which nothing in the source asks of it.
#ifdef SIMT_TSAN
#include <sanitizer/tsan_interface.h>
#include <deque>
#endif

hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, int attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  const char* e = getenv("SIMT_COMPUTE_UNITS");
  *v = e ? atoi(e) : 256;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = nullptr;
  return hipSuccess;
}
hipError_t hipGetSymbolAddressImpl(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  return hipSuccess;
}

// Context switch between fiber stacks: saves the callee-saved registers on the
// current stack, stores the stack pointer in *from, and resumes the context
// whose stack pointer is `to` (no signal-mask system call, unlike swapcontext).
extern "C" void simt_switch(void** from, void* to);
asm(R"(
.text
.globl simt_switch
.type simt_switch,@function
simt_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
.size simt_switch, .-simt_switch
)");

#ifdef SIMT_LDS_POISON
// the linker's bounds of the section holding every __shared__ array
extern "C" char __start_simt_lds[] __attribute__((weak));
extern "C" char __stop_simt_lds[] __attribute__((weak));
#endif

namespace simt {

int errors = 0;
long workgroups_run = 0;
static int shard_index = 0, shard_count = 1;
void set_block_shard(int index, int count) {
  if (count < 1 || index < 0 || index >= count) {
    report("set_block_shard: index %d of %d", index, count);
    return;
  }
  shard_index = index;
  shard_count = count;
}
static int max_reports = 40;

void report(const char* fmt, ...) {
  ++errors;
  if (errors > max_reports) return;
  va_list ap;
  va_start(ap, fmt);
  fprintf(stderr, "[simt] ");
  vfprintf(stderr, fmt, ap);
  fprintf(stderr, "\n");
  va_end(ap);
}

enum State { RUNNABLE, WAVEOP, BARRIER, DONE };
struct Fiber {
  void* sp = nullptr;
  char* stack = nullptr;
  Ids ids;
  State st = DONE;
  const char* site = "";
  WaveFn fn = nullptr;
  const void* fctx = nullptr;
  long barriers = 0;
  long waveops = 0;  // cross-lane operations and wave barriers passed
  void* fake = nullptr;
};
struct Wave {
  unsigned char in[64][192];
  unsigned char out[64][192];
};

static const size_t STACK = 512 << 10;
static std::vector<Fiber> F;
static std::vector<Wave> W;
static void* sched_sp = nullptr;
static Fiber* cur = nullptr;
static std::function<void()> body_fn;
static int nthreads = 0;
#ifdef SIMT_ASAN
static void* sched_fake = nullptr;
static const void* sched_bottom = nullptr;
static size_t sched_size = 0;
#endif
#ifdef SIMT_TSAN
static void* tsan_host = nullptr;
static void* tsan_wave[16] = {};
static void* tsan_lane[1024] = {};
static bool tsan_lanes = false;                // a fiber per lane (SIMT_TSAN_LANES=1)
static std::deque<char>* tsan_bars = nullptr;  // one sync object per barrier generation
static std::deque<char>* tsan_wops[16];        // per wave: one per wave-operation generation
static char tsan_order;  // orders workgroups and launches one after another
#endif

const Ids& ids() { return cur->ids; }
int lane_id() { return (int)(cur->ids.tid.x & 63); }

static void to_scheduler() {
#ifdef SIMT_TSAN
  __tsan_switch_to_fiber(tsan_host, __tsan_switch_to_fiber_no_sync);
#endif
#ifdef SIMT_ASAN
  __sanitizer_start_switch_fiber(&cur->fake, sched_bottom, sched_size);
#endif
  simt_switch(&cur->sp, sched_sp);
#ifdef SIMT_ASAN
  __sanitizer_finish_switch_fiber(cur->fake, nullptr, nullptr);
#endif
}

static void trampoline() {
#ifdef SIMT_ASAN
  __sanitizer_finish_switch_fiber(nullptr, &sched_bottom, &sched_size);
#endif
#ifdef SIMT_TSAN
  __tsan_acquire(&tsan_order);
#endif
  body_fn();
#ifdef SIMT_TSAN
  __tsan_release(&tsan_order);
  __tsan_switch_to_fiber(tsan_host, __tsan_switch_to_fiber_no_sync);
#endif
  cur->st = DONE;
#ifdef SIMT_ASAN
  __sanitizer_start_switch_fiber(nullptr, sched_bottom, sched_size);
#endif
  void* dead;
  simt_switch(&dead, sched_sp);
  abort();  // a finished fiber is never resumed
}

static void resume(Fiber& f) {
  cur = &f;
#ifdef SIMT_TSAN
  __tsan_switch_to_fiber(tsan_lanes ? tsan_lane[f.ids.tid.x] : tsan_wave[f.ids.tid.x / 64],
                         __tsan_switch_to_fiber_no_sync);
#endif
#ifdef SIMT_ASAN
  __sanitizer_start_switch_fiber(&sched_fake, f.stack, STACK);
#endif
  simt_switch(&sched_sp, f.sp);
#ifdef SIMT_ASAN
  __sanitizer_finish_switch_fiber(sched_fake, nullptr, nullptr);
#endif
  cur = nullptr;
}

void wave_op(const char* site, WaveFn fn, const void* ctx, const void* in, size_t nin, void* out, size_t nout) {
  Fiber* f = cur;
  const int t = (int)f->ids.tid.x, w = t / 64, l = t % 64;
  memcpy(W[w].in[l], in, nin);
  f->st = WAVEOP;
  f->site = site;
  f->fn = fn;
  f->fctx = ctx;
#ifdef SIMT_TSAN
  char* sync = nullptr;
  if (tsan_lanes) {
    std::deque<char>& gens = *tsan_wops[w];
    while ((long)gens.size() <= f->waveops) gens.push_back(0);
    sync = &gens[f->waveops];
    __tsan_release(sync);
  }
#endif
  to_scheduler();
#ifdef SIMT_TSAN
  if (sync) __tsan_acquire(sync);
#endif
  ++f->waveops;
  memcpy(out, W[w].out[l], nout);
}

void barrier(const char* site) {
  Fiber* f = cur;
  f->st = BARRIER;
  f->site = site;
#ifdef SIMT_TSAN
  while ((long)tsan_bars->size() <= f->barriers) tsan_bars->push_back(0);
  char* sync = &(*tsan_bars)[f->barriers];
  __tsan_release(sync);
#endif
  to_scheduler();
#ifdef SIMT_TSAN
  __tsan_acquire(sync);
#endif
  ++f->barriers;
}

static void run_workgroup() {
  const int nwaves = (nthreads + 63) / 64;
  for (;;) {
    bool prog = false;
    for (int t = 0; t < nthreads; ++t)
      if (F[t].st == RUNNABLE) {
        resume(F[t]);
        prog = true;
      }
    // wave operations whose every live lane has arrived
    for (int w = 0; w < nwaves; ++w) {
      bool live[64] = {};
      int nlive = 0, nop = 0;
      const Fiber* first = nullptr;
      for (int l = 0; l < 64; ++l) {
        const int t = 64 * w + l;
        if (t >= nthreads || F[t].st == DONE) continue;
        live[l] = true;
        ++nlive;
        if (F[t].st == WAVEOP) {
          ++nop;
          if (!first) first = &F[t];
        }
      }
      if (nlive == 0 || nop != nlive) continue;
      for (int l = 0; l < 64; ++l)
        if (live[l] && (F[64 * w + l].fn != first->fn || strcmp(F[64 * w + l].site, first->site) != 0)) {
          report("wave %d: lanes wait at different cross-lane operations (%s vs %s)", w, first->site,
                 F[64 * w + l].site);
          break;
        }
      first->fn(W[w].in, W[w].out, live, first->fctx);
      for (int l = 0; l < 64; ++l)
        if (live[l]) F[64 * w + l].st = RUNNABLE;
      prog = true;
    }
    if (prog) continue;
    int nlive = 0, nbar = 0;
    for (int t = 0; t < nthreads; ++t) {
      if (F[t].st == DONE) continue;
      ++nlive;
      if (F[t].st == BARRIER) ++nbar;
    }
    if (nlive == 0) break;
    if (nbar == nlive) {
      for (int t = 0; t < nthreads; ++t)
        if (F[t].st == BARRIER) F[t].st = RUNNABLE;
      continue;
    }
    // nothing can move: some lanes at a barrier, others at a cross-lane
    // operation their wave does not complete
    std::map<std::string, int> where;
    for (int t = 0; t < nthreads; ++t)
      if (F[t].st != DONE)
        where[std::string(F[t].st == BARRIER ? "barrier " : "waveop ") + F[t].site + " wave " +
              std::to_string(t / 64)]++;
    report("deadlock in block %u: %d live lanes", F[0].ids.bid.x, nlive);
    for (auto& kv : where) fprintf(stderr, "    %4d lanes at %s\n", kv.second, kv.first.c_str());
    abort();
  }
  // every wave should pass the same number of barriers
  long b0 = -1;
  for (int t = 0; t < nthreads; ++t) {
    if (b0 < 0) b0 = F[t].barriers;
    if (F[t].barriers != b0) {
      report("block %u: lane %d passed %ld barriers, lane 0 %ld", F[0].ids.bid.x, t, F[t].barriers, b0);
      break;
    }
  }
}

void launch(dim3 grid, dim3 block, std::function<void()> body) {
  if (block.y != 1 || block.z != 1) {
    report("launch: block (%u, %u, %u) is not 1-D", block.x, block.y, block.z);
    return;
  }
  nthreads = (int)block.x;
  if (nthreads <= 0 || nthreads > 1024) {
    report("launch: %d threads per block", nthreads);
    return;
  }
  if ((int)F.size() < nthreads) {
    F.resize(1024);
    W.resize(16);
    for (auto& f : F) {
      f.stack = (char*)mmap(nullptr, STACK, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
      if (f.stack == MAP_FAILED) abort();
    }
  }
  body_fn = std::move(body);
  const long wg_first = workgroups_run + 1;  // index of this launch's first workgroup, as counted below
  (void)wg_first;
#ifdef SIMT_TSAN
  tsan_host = __tsan_get_current_fiber();
  {
    const char* e = getenv("SIMT_TSAN_LANES");
    tsan_lanes = e && e[0] == '1';
  }
  __tsan_release(&tsan_order);
#endif
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        if ((bx + (uint64_t)grid.x * (by + (uint64_t)grid.y * bz)) % shard_count != (uint64_t)shard_index) continue;
        ++workgroups_run;
#ifdef SIMT_LDS_POISON
        // before the first eight workgroups of a launch and every 32nd after
        // (the section holds every kernel's arrays, 4.5 MB: poisoning before
        // every workgroup nearly doubles the parity tests' time)
        {
          const long i = workgroups_run - wg_first;
          if (__start_simt_lds && (i < 8 || i % 32 == 0))
            memset(__start_simt_lds, 0xff, (size_t)(__stop_simt_lds - __start_simt_lds));
        }
#endif
#ifdef SIMT_TSAN
        // each workgroup: its own sync objects.  The wave (or lane) contexts
        // are created once and reused, like the fibers' stacks: workgroups are
        // ordered one after another, and creating and destroying thousands of
        // TSan fibers has crashed the runtime
        for (int w = 0; w < (nthreads + 63) / 64; ++w) {
          if (!tsan_wave[w]) tsan_wave[w] = __tsan_create_fiber(0);
          tsan_wops[w] = new std::deque<char>();
        }
        if (tsan_lanes)
          for (int t = 0; t < nthreads; ++t)
            if (!tsan_lane[t]) tsan_lane[t] = __tsan_create_fiber(0);
        tsan_bars = new std::deque<char>();
#endif
        for (int t = 0; t < nthreads; ++t) {
          Fiber& f = F[t];
          f.ids = Ids{Dim{(unsigned)t, 0, 0}, Dim{bx, by, bz}, Dim{grid.x, grid.y, grid.z}, Dim{block.x, 1, 1}};
          f.st = RUNNABLE;
          f.barriers = 0;
          f.waveops = 0;
          f.fake = nullptr;
          // initial frame: six zero registers, then the trampoline as the
          // return address (entered with rsp = 8 mod 16, as after a call)
          void** sp = (void**)(f.stack + STACK - 64);
          for (int i = 0; i < 6; ++i) sp[i] = nullptr;
          sp[6] = (void*)&trampoline;
          sp[7] = nullptr;
          f.sp = sp;
        }
        run_workgroup();
#ifdef SIMT_TSAN
        // every fiber released tsan_order as it finished: the scheduler frees
        // the workgroup's sync objects after all their uses
        __tsan_acquire(&tsan_order);
        for (int w = 0; w < (nthreads + 63) / 64; ++w) delete tsan_wops[w];
        delete tsan_bars;
#endif
      }
#ifdef SIMT_TSAN
  __tsan_acquire(&tsan_order);
#endif
}

// ---------------------------------------------------------------------------
// buffer accesses
// ---------------------------------------------------------------------------
void buf_access(const Rsrc& r, uint32_t voff, uint32_t soff, void* data, int n, bool store) {
  const uint64_t off = (uint64_t)voff + soff;
  if (off + (uint64_t)n > (1ull << 32)) {
    report("buffer offset wraps 2^32: voffset %u soffset %u size %d", voff, soff, n);
    if (!store) memset(data, 0, n);
    return;
  }
  const int step = n < 4 ? n : 4;
  for (int j = 0; j < n; j += step) {
    const uint64_t o = off + j;
    if (o + step <= r.nrec) {
      if (store)
        memcpy(r.base + o, (char*)data + j, step);
      else
        memcpy((char*)data + j, r.base + o, step);
    } else if (!store) {
      memset((char*)data + j, 0, step);
    }
  }
}

// ---------------------------------------------------------------------------
// cross-lane operations
// ---------------------------------------------------------------------------
typedef const unsigned char (*In)[192];
typedef unsigned char (*Out)[192];

void fn_nop(In, Out, const bool*, const void*) {}
void fn_readfirstlane(In in, Out out, const bool* live, const void*) {
  int f = 0;
  while (f < 64 && !live[f]) ++f;
  for (int l = 0; l < 64; ++l)
    if (live[l]) memcpy(out[l], in[f], 4);
}
void fn_readlane(In in, Out out, const bool* live, const void*) {
  int f = 0;
  while (f < 64 && !live[f]) ++f;
  int src;
  memcpy(&src, in[f] + 4, 4);
  for (int l = 0; l < 64; ++l) {
    if (!live[l]) continue;
    int s2;
    memcpy(&s2, in[l] + 4, 4);
    if (s2 != src) report("readlane: lane index not uniform (%d vs %d)", s2, src);
  }
  if (src < 0 || src > 63 || !live[src]) report("readlane: source lane %d is not live", src);
  for (int l = 0; l < 64; ++l)
    if (live[l]) memcpy(out[l], in[src & 63], 4);
}
void fn_bpermute(In in, Out out, const bool* live, const void*) {
  for (int l = 0; l < 64; ++l) {
    if (!live[l]) continue;
    int a;
    memcpy(&a, in[l], 4);
    const int s = (a >> 2) & 63;
    if (!live[s]) report("bpermute: lane %d reads lane %d, which is not live", l, s);
    memcpy(out[l], in[s] + 4, 4);
  }
}
void fn_shfl_xor(In in, Out out, const bool* live, const void*) {
  for (int l = 0; l < 64; ++l) {
    if (!live[l]) continue;
    int m;
    memcpy(&m, in[l] + 4, 4);
    const int s = (l ^ m) & 63;
    if (!live[s]) report("shfl_xor: lane %d reads lane %d, which is not live", l, s);
    memcpy(out[l], in[s], 4);
  }
}
void fn_dpp(In in, Out out, const bool* live, const void*) {
  for (int l = 0; l < 64; ++l) {
    if (!live[l]) continue;
    int p[6];
    memcpy(p, in[l], sizeof p);
    const int ctrl = p[2];
    int s;
    if (ctrl >= 0 && ctrl <= 0xff)
      s = (l & ~3) + ((ctrl >> (2 * (l & 3))) & 3);
    else if (ctrl == 0x140)
      s = (l & ~15) + (15 - (l & 15));
    else if (ctrl == 0x141)
      s = (l & ~7) + (7 - (l & 7));
    else {
      report("dpp control 0x%x not emulated", ctrl);
      s = l;
    }
    if (p[3] != 0xf || p[4] != 0xf) report("dpp masks %x %x not emulated", p[3], p[4]);
    int v;
    if (live[s])
      memcpy(&v, in[s] + 4, 4);
    else
      v = p[0];  // old
    memcpy(out[l], &v, 4);
  }
}

static float half_to_f(const unsigned char* p) {
  _Float16 h;
  memcpy(&h, p, 2);
  return (float)h;
}
static float bf16_to_f(const unsigned char* p) {
  uint16_t b;
  memcpy(&b, p, 2);
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void fn_mfma(In in, Out out, const bool* live, const void* ctx) {
  struct Ctx { int kind, asz, csz; };
  const Ctx& c = *static_cast<const Ctx*>(ctx);
  for (int l = 0; l < 64; ++l)
    if (!live[l]) report("mfma with lane %d not live", l);
  const int asz = c.asz;
  int M, N, K, per;  // per: operand elements per lane
  bool f32 = false, bf = false;
  switch (c.kind) {
    case K16x16x32_F16: M = N = 16; K = 32; per = 8; break;
    case K16x16x32_BF16: M = N = 16; K = 32; per = 8; bf = true; break;
    case K16x16x4_F32: M = N = 16; K = 4; per = 1; f32 = true; break;
    case K32x32x16_BF16: M = N = 32; K = 16; per = 8; bf = true; break;
    case K32x32x2_F32: M = N = 32; K = 2; per = 1; f32 = true; break;
    default: report("mfma kind %d", c.kind); return;
  }
  (void)K;
  static double A[32][32], B[32][32];
  // lane l supplies row (col) l % M of A (B), k = per * (l / M) + j
  for (int l = 0; l < 64; ++l) {
    const int i = l % M, kb = per * (l / M);
    for (int j = 0; j < per; ++j) {
      const unsigned char* pa = in[l] + (f32 ? 0 : 2 * j);
      const unsigned char* pb = in[l] + asz + (f32 ? 0 : 2 * j);
      double a, b;
      if (f32) {
        float fa, fb;
        memcpy(&fa, pa, 4);
        memcpy(&fb, pb, 4);
        a = fa;
        b = fb;
      } else if (bf) {
        a = bf16_to_f(pa);
        b = bf16_to_f(pb);
      } else {
        a = half_to_f(pa);
        b = half_to_f(pb);
      }
      A[i][kb + j] = a;
      B[kb + j][i] = b;
    }
  }
  const int Kt = per * (64 / M);
  for (int l = 0; l < 64; ++l) {
    const int col = l % N;
    const int nreg = c.csz / 4;
    for (int r = 0; r < nreg; ++r) {
      const int row = M == 16 ? 4 * (l / 16) + r : 8 * (r / 4) + 4 * (l / 32) + (r % 4);
      float acc;
      memcpy(&acc, in[l] + 2 * asz + 4 * r, 4);
      double s = 0;
      for (int k = 0; k < Kt; ++k) s += A[row][k] * B[k][col];
      const float d = (float)((double)acc + s);
      memcpy(out[l] + 4 * r, &d, 4);
    }
  }
}

}  // namespace simt
