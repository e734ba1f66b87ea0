// Checks of the emulator itself (simt.h), run on the host only:
//   selftest <case>
// "mfma":      every matrix-core shape against a plain float64 product of the
//              operands in the layout simt.h states (exit 0 when equal);
// "wrap":      a buffer load whose offset wraps 2^32 (must be reported);
// "range":     loads past num_records read zero and stores there are dropped;
// "barriers":  one wave passes one barrier fewer than the others (reported);
// "diverge":   half a wave reaches a cross-lane operation the other half
//              skips (reported as a deadlock: the process aborts);
// "race":      two waves write and read one __shared__ word with no barrier
//              between them, then with one (built with ThreadSanitizer: the
//              first must be reported, the second not);
// "lanerace" / "lanesync": lane 0 of a wave writes one __shared__ word and
//              lane 1 of the same wave reads it, with no wave barrier between
//              them, then with one (ThreadSanitizer with SIMT_TSAN_LANES=1:
//              the first must be reported, the second not);
// "poison":    (built with SIMT_LDS_POISON) a workgroup that reads LDS it did
//              not write sees all-ones bytes, not what the previous one left;
// "shard":     a launch split three ways runs workgroups 1, 4, 7 of nine in
//              the shard with index 1, and all nine after the split is undone.
// Each planted case is a kernel written for this check alone; none is built
// for a GPU.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "simt.h"

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

static int check_mfma() {
  // inputs: A[i][k] = a(i, k), B[k][j] = b(k, j), C = c(i, j), exact in half
  auto a = [](int i, int k) { return (float)((i * 7 + k * 3) % 11 - 5) / 4.f; };
  auto b = [](int k, int j) { return (float)((k * 5 + j * 2) % 13 - 6) / 8.f; };
  auto c = [](int i, int j) { return (float)(i - j) / 2.f; };
  int bad = 0;
  auto expect = [&](const char* name, int M, int K, int i, int j, float got) {
    double s = c(i, j);
    for (int k = 0; k < K; ++k) s += (double)a(i, k) * b(k, j);
    if (std::fabs(s - got) > 1e-4) {
      if (bad < 5) fprintf(stderr, "%s: D[%d][%d] = %g, want %g\n", name, i, j, got, s);
      ++bad;
    }
    (void)M;
  };
  std::vector<float> out16(64 * 4), out32(64 * 16);
  // 16 x 16 x 32, half and bfloat16 operands: lane l gives row/column l % 16,
  // k = 8 (l / 16) + j
  for (int kind = 0; kind < 2; ++kind) {
    simt::launch(dim3(1), dim3(64), [&]() {
      const int l = threadIdx.x, r = l % 16, kb = 8 * (l / 16);
      f4 acc;
      for (int q = 0; q < 4; ++q) acc[q] = c(4 * (l / 16) + q, r);
      f4 d;
      if (kind == 0) {
        h8 x, y;
        for (int j = 0; j < 8; ++j) x[j] = (_Float16)a(r, kb + j), y[j] = (_Float16)b(kb + j, r);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
      } else {
        b8 x, y;
        for (int j = 0; j < 8; ++j) x[j] = (__bf16)a(r, kb + j), y[j] = (__bf16)b(kb + j, r);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
      }
      for (int q = 0; q < 4; ++q) out16[l * 4 + q] = d[q];
    });
    for (int l = 0; l < 64; ++l)
      for (int q = 0; q < 4; ++q) expect(kind ? "16x16x32 bf16" : "16x16x32 f16", 16, 32, 4 * (l / 16) + q, l % 16, out16[l * 4 + q]);
  }
  // 16 x 16 x 4 float32: k = l / 16
  simt::launch(dim3(1), dim3(64), [&]() {
    const int l = threadIdx.x;
    f4 acc;
    for (int q = 0; q < 4; ++q) acc[q] = c(4 * (l / 16) + q, l % 16);
    const f4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(a(l % 16, l / 16), b(l / 16, l % 16), acc, 0, 0, 0);
    for (int q = 0; q < 4; ++q) out16[l * 4 + q] = d[q];
  });
  for (int l = 0; l < 64; ++l)
    for (int q = 0; q < 4; ++q) expect("16x16x4 f32", 16, 4, 4 * (l / 16) + q, l % 16, out16[l * 4 + q]);
  // 32 x 32: register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  for (int kind = 0; kind < 2; ++kind) {
    simt::launch(dim3(1), dim3(64), [&]() {
      const int l = threadIdx.x, r = l % 32;
      f16v acc;
      for (int q = 0; q < 16; ++q) acc[q] = c(8 * (q / 4) + 4 * (l / 32) + q % 4, r);
      f16v d;
      if (kind == 0) {
        b8 x, y;
        const int kb = 8 * (l / 32);
        for (int j = 0; j < 8; ++j) x[j] = (__bf16)a(r, kb + j), y[j] = (__bf16)b(kb + j, r);
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
      } else {
        d = __builtin_amdgcn_mfma_f32_32x32x2f32(a(r, l / 32), b(l / 32, r), acc, 0, 0, 0);
      }
      for (int q = 0; q < 16; ++q) out32[l * 16 + q] = d[q];
    });
    for (int l = 0; l < 64; ++l)
      for (int q = 0; q < 16; ++q)
        expect(kind ? "32x32x2 f32" : "32x32x16 bf16", 32, kind ? 2 : 16, 8 * (q / 4) + 4 * (l / 32) + q % 4, l % 32,
               out32[l * 16 + q]);
  }
  printf("mfma: %d mismatches\n", bad);
  return bad == 0 && simt::errors == 0 ? 0 : 1;
}

int main(int argc, char** argv) {
  const char* what = argc > 1 ? argv[1] : "";
  if (!strcmp(what, "mfma")) return check_mfma();
  if (!strcmp(what, "wrap")) {
    std::vector<uint32_t> buf(64, 7);
    simt::launch(dim3(1), dim3(64), [&]() {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(buf.data(), 0, 256, 0x00020000);
      (void)__builtin_amdgcn_raw_buffer_load_b128(r, 0xfffffff8u, 0, 0);
    });
    printf("wrap: %d reports\n", simt::errors);
    return simt::errors > 0 ? 0 : 1;
  }
  if (!strcmp(what, "range")) {
    std::vector<uint32_t> buf(8, 7);
    uint32_t got[2] = {1, 1};
    simt::launch(dim3(1), dim3(64), [&]() {
      const auto r = __builtin_amdgcn_make_buffer_rsrc(buf.data(), 0, 16, 0x00020000);  // 4 dwords
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, 4u * threadIdx.x, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(9u, r, 4u * threadIdx.x, 0, 0);
      if (threadIdx.x == 3) got[0] = v;
      if (threadIdx.x == 4) got[1] = v;
    });
    const bool ok = got[0] == 7 && got[1] == 0 && buf[3] == 9 && buf[4] == 7 && simt::errors == 0;
    printf("range: in-range %u, past the end %u, stores %u %u: %s\n", got[0], got[1], buf[3], buf[4],
           ok ? "ok" : "wrong");
    return ok ? 0 : 1;
  }
  if (!strcmp(what, "barriers")) {
    simt::launch(dim3(1), dim3(128), [&]() {
      __syncthreads();
      if (threadIdx.x < 64) __syncthreads();
    });
    printf("barriers: %d reports\n", simt::errors);
    return simt::errors > 0 ? 0 : 1;
  }
  if (!strcmp(what, "diverge")) {
    simt::launch(dim3(1), dim3(64), [&]() {
      int v = threadIdx.x;
      if (threadIdx.x < 32) v = __shfl_xor(v, 1);
      __syncthreads();
      (void)v;
    });
    return 0;  // not reached: the scheduler reports the deadlock and aborts
  }
  if (!strcmp(what, "race") || !strcmp(what, "norace")) {
    const bool fenced = !strcmp(what, "norace");
    simt::launch(dim3(2), dim3(128), [&]() {
      static int word;  // one word of LDS
      if (threadIdx.x == 0) word = 1;
      if (fenced) __syncthreads();
      if (threadIdx.x == 64) printf("%s: wave 1 reads %d\n", fenced ? "norace" : "race", word);
      if (!fenced) __syncthreads();
    });
    return 0;
  }
  if (!strcmp(what, "lanerace") || !strcmp(what, "lanesync")) {
    const bool synced = !strcmp(what, "lanesync");
    simt::launch(dim3(1), dim3(64), [&]() {
      static int word;  // one word of LDS
      if (threadIdx.x == 0) word = 7;
      if (synced) __builtin_amdgcn_wave_barrier();
      if (threadIdx.x == 1) printf("%s: lane 1 reads %d\n", synced ? "lanesync" : "lanerace", word);
      if (!synced) __builtin_amdgcn_wave_barrier();
    });
    return 0;
  }
  if (!strcmp(what, "poison")) {
    uint32_t got = 0;
    simt::launch(dim3(2), dim3(64), [&]() {
      __shared__ uint32_t w[64];
      if (blockIdx.x == 0) w[threadIdx.x] = 5;
      __syncthreads();
      if (blockIdx.x == 1 && threadIdx.x == 0) got = w[7];
    });
    printf("poison: workgroup 1 reads %08x\n", got);
    return got == 0xffffffffu ? 0 : 1;
  }
  if (!strcmp(what, "shard")) {
    std::vector<int> ran;
    simt::set_block_shard(1, 3);
    simt::launch(dim3(3, 3), dim3(64), [&]() {
      if (threadIdx.x == 0) ran.push_back((int)(blockIdx.x + 3 * blockIdx.y));
    });
    const bool split = ran == std::vector<int>{1, 4, 7} && simt::workgroups_run == 3;
    ran.clear();
    simt::set_block_shard(0, 1);
    simt::launch(dim3(9), dim3(64), [&]() {
      if (threadIdx.x == 0) ran.push_back((int)blockIdx.x);
    });
    const bool whole = ran.size() == 9 && simt::workgroups_run == 12;
    printf("shard: %s\n", split && whole && simt::errors == 0 ? "ok" : "wrong");
    return split && whole && simt::errors == 0 ? 0 : 1;
  }
  fprintf(stderr, "usage: selftest mfma|wrap|range|barriers|diverge|race|norace|lanerace|lanesync|poison|shard\n");
  return 2;
}
