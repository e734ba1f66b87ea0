// Host emulation of the HIP device environment the VDA kernels use, so that the
// library's own kernel sources compile and run on the CPU (a CPU build for
// checking, not a product path).
//
// Every lane of a workgroup is a fiber.  Cross-lane operations (readlane,
// readfirstlane, ds_bpermute, shfl_xor, DPP, the matrix-core MFMAs) are
// rendezvous points: once every live lane of the wave has arrived, the
// operation runs on all their operands at once.  s_barrier / __syncthreads is a
// rendezvous of every live lane of the workgroup.  __shared__ arrays are
// function-local statics (workgroups run one after another; with
// SIMT_LDS_POISON filled with all-ones bytes before most of a launch's first
// workgroups and a sample of the rest), buffer
// descriptors keep their range checks (per dword against num_records, zero on
// loads and dropped stores past it; an offset that wraps 2^32 is reported), and
// plain pointers are host memory, so AddressSanitizer sees every global and LDS
// access.  MFMA operand and accumulator layouts: lane l supplies row (A) or
// column (B) l % M with k = n (l / M) + j for its n elements j; accumulator
// register r of lane l is D[4 (l / 16) + r][l % 16] for M = 16 and
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] for M = 32.
//
// Limitation: lanes of one wave run in turn, not in lockstep, so between two
// rendezvous points a lane may run ahead of the others.  Code that passes data
// between lanes of one wave through LDS must separate the write and the read
// by a wave-level operation or __builtin_amdgcn_wave_barrier() (a rendezvous
// here), as the compiler also requires; without one the emulation reads stale
// values and the checks against the reference fail.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <type_traits>

// ---------------------------------------------------------------------------
// qualifiers and host API subset
// ---------------------------------------------------------------------------
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline __attribute__((always_inline))
#define __launch_bounds__(...)
#ifdef SIMT_LDS_POISON
// every __shared__ array in one section, which the launcher fills with
// all-ones bytes (NaN as float32 and bfloat16, -1 as an integer) before the
// first eight workgroups of each launch and every 32nd after: the hardware
// gives a workgroup LDS of undefined contents, so a kernel must write what it
// reads.  (AddressSanitizer leaves variables in a
// named section unguarded, so the sanitized builds keep plain statics.)
#define __shared__ static __attribute__((section("simt_lds")))
#else
#define __shared__ static
#endif
#define __align__(n) __attribute__((aligned(n)))

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorInvalidSymbol = 13,
  hipErrorInvalidDevice = 101,
  hipErrorLaunchFailure = 719
} hipError_t;
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
enum { hipDeviceAttributeMultiprocessorCount = 63 };

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

hipError_t hipGetLastError();
hipError_t hipGetDevice(int* d);
hipError_t hipDeviceGetAttribute(int* v, int attr, int dev);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipGetSymbolAddressImpl(void** p, const void* sym);
#define hipGetSymbolAddress(p, sym) hipGetSymbolAddressImpl((void**)(p), (const void*)(sym))
#define HIP_SYMBOL(x) (&(x))

// ---------------------------------------------------------------------------
// vector types
// ---------------------------------------------------------------------------
struct alignas(16) uint4 { unsigned x, y, z, w; };
struct alignas(8) uint2 { unsigned x, y; };
struct alignas(16) float4 { float x, y, z, w; };
struct alignas(8) float2 { float x, y; };
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return {a, b, c, d}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return {a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline float2 make_float2(float a, float b) { return {a, b}; }

inline float __int_as_float(int v) { float f; memcpy(&f, &v, 4); return f; }
inline float __uint_as_float(unsigned v) { float f; memcpy(&f, &v, 4); return f; }
inline int __float_as_int(float f) { int v; memcpy(&v, &f, 4); return v; }
inline unsigned __float_as_uint(float f) { unsigned v; memcpy(&v, &f, 4); return v; }
inline float __expf(float x) { return expf(x); }
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline unsigned min(unsigned a, unsigned b) { return a < b ? a : b; }
inline unsigned max(unsigned a, unsigned b) { return a > b ? a : b; }
inline long long min(long long a, long long b) { return a < b ? a : b; }
inline long long max(long long a, long long b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// the emulator
// ---------------------------------------------------------------------------
namespace simt {

struct Dim { unsigned x, y, z; };
struct Ids { Dim tid, bid, grid, block; };
const Ids& ids();
int lane_id();

// Report a problem found by the emulator (range, wrap, divergence, deadlock).
void report(const char* fmt, ...);
extern int errors;

// A wave operation: every live lane of the calling wave passes `in`; once all
// have, `fn(in, out, live)` runs once (in[l], out[l] for lane l; live[l] marks
// the lanes that took part) and each lane gets out[its lane].
typedef void (*WaveFn)(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void* ctx);
void wave_op(const char* site, WaveFn fn, const void* ctx, const void* in, size_t nin, void* out, size_t nout);
void barrier(const char* site);
void launch(dim3 grid, dim3 block, std::function<void()> body);
// Split launches over `count` processes: from this call on, a launch runs only
// the workgroups whose linear index (x fastest) is `index` modulo `count` (the
// others are skipped whole, so each process gives the results of its share).
void set_block_shard(int index, int count);
// Workgroups run by every launch since the process started.
extern long workgroups_run;

template <class T>
T wave_call(const char* site, WaveFn fn, const T& v, const void* ctx = nullptr) {
  T r;
  wave_op(site, fn, ctx, &v, sizeof(T), &r, sizeof(T));
  return r;
}

// buffer descriptors
struct Rsrc {
  char* base;
  uint32_t nrec;
};
inline Rsrc make_rsrc(void* p, short stride, int nrec, int flags) {
  (void)stride;
  (void)flags;
  return Rsrc{static_cast<char*>(p), (uint32_t)nrec};
}
// one access of `n` bytes at offset voff + soff: per dword (or the whole
// access if smaller) inside num_records, or zero / dropped
void buf_access(const Rsrc& r, uint32_t voff, uint32_t soff, void* data, int n, bool store);

}  // namespace simt

#define threadIdx (simt::ids().tid)
#define blockIdx (simt::ids().bid)
#define gridDim (simt::ids().grid)
#define blockDim (simt::ids().block)

#define __amdgpu_buffer_rsrc_t simt::Rsrc
#define __builtin_amdgcn_make_buffer_rsrc(p, s, n, f) simt::make_rsrc((void*)(p), (s), (n), (f))

typedef unsigned simt_v4u __attribute__((ext_vector_type(4)));
typedef unsigned simt_v2u __attribute__((ext_vector_type(2)));
inline simt_v4u simt_load_b128(simt::Rsrc r, uint32_t v, uint32_t s, int) {
  simt_v4u x;
  simt::buf_access(r, v, s, &x, 16, false);
  return x;
}
inline simt_v2u simt_load_b64(simt::Rsrc r, uint32_t v, uint32_t s, int) {
  simt_v2u x;
  simt::buf_access(r, v, s, &x, 8, false);
  return x;
}
inline uint32_t simt_load_b32(simt::Rsrc r, uint32_t v, uint32_t s, int) {
  uint32_t x;
  simt::buf_access(r, v, s, &x, 4, false);
  return x;
}
inline uint16_t simt_load_b16(simt::Rsrc r, uint32_t v, uint32_t s, int) {
  uint16_t x;
  simt::buf_access(r, v, s, &x, 2, false);
  return x;
}
template <class T>
inline void simt_store(T x, simt::Rsrc r, uint32_t v, uint32_t s, int n) {
  static_assert(sizeof(T) >= 2, "");
  simt::buf_access(r, v, s, &x, n, true);
}
#define __builtin_amdgcn_raw_buffer_load_b128(r, v, s, a) simt_load_b128((r), (v), (s), (a))
#define __builtin_amdgcn_raw_buffer_load_b64(r, v, s, a) simt_load_b64((r), (v), (s), (a))
#define __builtin_amdgcn_raw_buffer_load_b32(r, v, s, a) simt_load_b32((r), (v), (s), (a))
#define __builtin_amdgcn_raw_buffer_load_b16(r, v, s, a) simt_load_b16((r), (v), (s), (a))
#define __builtin_amdgcn_raw_buffer_store_b128(x, r, v, s, a) simt_store((x), (r), (v), (s), 16)
#define __builtin_amdgcn_raw_buffer_store_b64(x, r, v, s, a) simt_store((x), (r), (v), (s), 8)
#define __builtin_amdgcn_raw_buffer_store_b32(x, r, v, s, a) simt_store((x), (r), (v), (s), 4)
#define __builtin_amdgcn_raw_buffer_store_b16(x, r, v, s, a) simt_store((uint16_t)(x), (r), (v), (s), 2)

// scheduling hints and waits: nothing to emulate
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_s_setprio(x) ((void)0)
#define __builtin_amdgcn_s_waitcnt(x) ((void)0)
#define __builtin_amdgcn_s_barrier() simt::barrier(__FILE__ ":" SIMT_STR(__LINE__))
#define __syncthreads() simt::barrier(__FILE__ ":" SIMT_STR(__LINE__))
#define SIMT_STR2(x) #x
#define SIMT_STR(x) SIMT_STR2(x)

// math
#define __builtin_amdgcn_rcpf(x) (1.0f / (float)(x))
#define __builtin_amdgcn_rsqf(x) (1.0f / sqrtf((float)(x)))
#define __builtin_amdgcn_sqrtf(x) sqrtf((float)(x))

// ---------------------------------------------------------------------------
// cross-lane operations
// ---------------------------------------------------------------------------
namespace simt {
void fn_readfirstlane(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void*);
void fn_readlane(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void* ctx);
void fn_bpermute(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void*);
void fn_shfl_xor(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void* ctx);
void fn_dpp(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void* ctx);
void fn_mfma(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void* ctx);

template <class T>
T readfirstlane(T v, const char* site) {
  static_assert(sizeof(T) == 4, "");
  return wave_call(site, fn_readfirstlane, v);
}
// the source lane index must be wave-uniform; it travels with the payload
template <class T>
T readlane(T v, int l, const char* site) {
  static_assert(sizeof(T) == 4, "");
  struct P { T v; int l; } p{v, l};
  struct R { T v; int pad; } r;
  wave_op(site, fn_readlane, nullptr, &p, sizeof(P), &r, sizeof(R));
  return r.v;
}
inline int bpermute(int addr, int v, const char* site) {
  struct P { int a, v; } p{addr, v};
  int r;
  wave_op(site, fn_bpermute, nullptr, &p, sizeof(P), &r, 4);
  return r;
}
template <class T>
T shfl_xor(T v, int m, const char* site) {
  static_assert(sizeof(T) == 4, "");
  struct P { T v; int m; } p{v, m};
  T r;
  wave_op(site, fn_shfl_xor, nullptr, &p, sizeof(P), &r, sizeof(T));
  return r;
}
inline int update_dpp(int old, int src, int ctrl, int rm, int bm, bool bc, const char* site) {
  struct P { int old, src, ctrl, rm, bm, bc; } p{old, src, ctrl, rm, bm, bc};
  int r;
  wave_op(site, fn_dpp, nullptr, &p, sizeof(P), &r, 4);
  return r;
}

// MFMA shapes: M x N x K with the per-lane operand element count and type
enum MfmaKind { K16x16x32_F16, K16x16x32_BF16, K16x16x4_F32, K32x32x16_BF16, K32x32x2_F32 };
template <class A, class C>
C mfma(MfmaKind kind, const A& a, const A& b, const C& c, const char* site) {
  static_assert(2 * sizeof(A) + sizeof(C) <= 192, "");
  unsigned char p[192];
  memcpy(p, &a, sizeof(A));
  memcpy(p + sizeof(A), &b, sizeof(A));
  memcpy(p + 2 * sizeof(A), &c, sizeof(C));
  C r;
  struct Ctx { int kind, asz, csz; } ctx{kind, (int)sizeof(A), (int)sizeof(C)};
  wave_op(site, fn_mfma, &ctx, p, 2 * sizeof(A) + sizeof(C), &r, sizeof(C));
  return r;
}
}  // namespace simt

#define SIMT_SITE __FILE__ ":" SIMT_STR(__LINE__)
#define __builtin_amdgcn_readfirstlane(v) simt::readfirstlane((v), SIMT_SITE)
#define __builtin_amdgcn_readlane(v, l) simt::readlane((v), (l), SIMT_SITE)
#define __builtin_amdgcn_ds_bpermute(a, v) simt::bpermute((a), (v), SIMT_SITE)
#define __shfl_xor(v, m) simt::shfl_xor((v), (m), SIMT_SITE)
#define __builtin_amdgcn_update_dpp(o, s, c, rm, bm, bc) simt::update_dpp((o), (s), (c), (rm), (bm), (bc), SIMT_SITE)
#define __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, x, y, z) simt::mfma(simt::K16x16x32_F16, (a), (b), (c), SIMT_SITE)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) simt::mfma(simt::K16x16x32_BF16, (a), (b), (c), SIMT_SITE)
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) simt::mfma(simt::K32x32x16_BF16, (a), (b), (c), SIMT_SITE)
#define __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, x, y, z) \
  simt::mfma(simt::K16x16x4_F32, (float)(a), (float)(b), (c), SIMT_SITE)
#define __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, x, y, z) \
  simt::mfma(simt::K32x32x2_F32, (float)(a), (float)(b), (c), SIMT_SITE)

// lanes of a wave run in lockstep on the hardware; here they meet
namespace simt {
void fn_nop(const unsigned char (*in)[192], unsigned char (*out)[192], const bool* live, const void*);
inline void wave_sync(const char* site) {
  int x = 0;
  (void)wave_call(site, fn_nop, x);
}
}  // namespace simt
#define __builtin_amdgcn_wave_barrier() simt::wave_sync(SIMT_SITE)

// a launch runs every workgroup in turn, each as 1-D lanes of fibers
#define hipLaunchKernelGGL(K, G, B, S, ST, ...) simt::launch(dim3(G), dim3(B), [=]() { (K)(__VA_ARGS__); })
