// Host-side exercise of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (built by tests/test_host_sanitizers.py with the sanitizers on the
// host pass only).  Every call here fails its argument checks or only computes
// sizes, so nothing reaches a GPU; the sanitizers watch the descriptor
// validation, the workspace layouts and the argument checks of every entry
// point over a sweep of valid, extreme and invalid descriptors.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vdn_vda.h"

static int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static vdn_vda_desc desc(int B, int H, int T, int gh, int gw, int d, int L, int chunk, vdn_dtype dt, uint32_t flags) {
  vdn_vda_desc x;
  memset(&x, 0, sizeof x);
  x.B = B; x.H = H; x.T = T; x.grid_h = gh; x.grid_w = gw; x.d_k = d; x.d_v = d;
  x.n_text = L; x.chunk = chunk; x.dtype = dt; x.flags = flags; x.l2_eps = 1e-6f; x.rms_eps = 1e-6f;
  return x;
}

// fake device addresses, 8 GiB apart; never dereferenced (every call fails first)
static void* fake(int i) { return (void*)(uintptr_t)(0x7f0000000000ull + (uint64_t)i * (8ull << 30)); }

int main() {
  const int dims[][9] = {
      // B, H, T, gh, gw, d, L, chunk, dtype
      {1, 24, 60, 48, 84, 128, 256, 5, 1}, {1, 2, 20, 4, 4, 16, 8, 5, 0}, {1, 8, 40, 30, 52, 64, 64, 5, 1},
      {1, 4, 30, 32, 32, 128, 64, 5, 0},  {1, 24, 120, 48, 84, 128, 512, 5, 1}, {2, 3, 1, 1, 1, 32, 0, 1, 1},
      {1, 1, 32767, 1, 1, 128, 0, 1, 1},  {1, 16384, 2, 1, 1, 128, 380, 5, 1}, {3, 5, 7, 9, 11, 16, 13, 3, 0},
      // invalid or unsupported
      {0, 1, 1, 1, 1, 16, 0, 5, 1}, {1, 1, 1, 1, 1, 48, 0, 5, 1}, {1, 1, 1, 1, 1, 144, 0, 5, 1},
      {1, 1, 0, 1, 1, 16, 0, 5, 1}, {1, 1, 1, 1, 1, 16, -1, 5, 1}, {1, 1, 1, 1, 1, 16, 0, 0, 1},
      {1, 16, 2, 1000, 1000, 128, 0, 5, 1}, {2147483647, 2147483647, 2147483647, 2147483647, 2147483647, 128, 2147483647, 1, 1},
      {1, 1, 32768, 1, 1, 128, 0, 1, 1}, {1, 1, 3, 65535, 65535, 16, 0, 5, 1}, {-5, 3, 3, 3, 3, 16, 0, 5, 1},
  };
  const uint32_t flagsets[] = {0, VDN_VDA_EPILOGUE, VDN_VDA_EPILOGUE | VDN_VDA_DECAY_BRIDGE | VDN_VDA_QUERY_L2,
                               VDN_VDA_SCAN_CHUNKS, VDN_VDA_SCAN_FRAMES | VDN_VDA_SCAN_CHUNKS, 1u << 30};
  int valid = 0;
  for (const auto& r : dims) {
    for (uint32_t fl : flagsets) {
      vdn_vda_desc d = desc(r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7], (vdn_dtype)r[8], fl);
      const vdn_status st = vdn_vda_validate(&d);
      const size_t ws = vdn_vda_workspace_bytes(&d);
      EXPECT((st == VDN_OK) == (ws > 0));
      vdn_vda_layout l;
      EXPECT(vdn_vda_workspace_layout(&d, &l) == st);
      if (st == VDN_OK) {
        ++valid;
        EXPECT(l.total == ws && l.stats <= l.pinv && l.pinv <= l.total);
        vdn_vda_backward_layout bl;
        EXPECT(vdn_vda_backward_workspace_layout(&d, &bl) == VDN_OK);
        EXPECT(bl.total == vdn_vda_backward_workspace_bytes(&d));
        (void)vdn_vda_gates_workspace_bytes(&d, 3072);
        (void)vdn_vda_gates_workspace_bytes(&d, 12);
      }
      // every entry point with a NULL required pointer: an error, no launch
      EXPECT(vdn_vda_forward(&d, nullptr, fake(1), fake(2), (const float*)fake(3), fake(4), fake(5), fake(6),
                             fake(7), fake(8), nullptr, fake(9), fake(10), ws, nullptr) != VDN_OK);
      EXPECT(vdn_vda_forward_noalloc(&d, fake(0), fake(1), fake(2), (const float*)fake(3), fake(4), fake(5),
                                     fake(6), fake(7), fake(8), nullptr, nullptr, nullptr) != VDN_OK);
      EXPECT(vdn_vda_prepare(&d, fake(0), nullptr, fake(2), (const float*)fake(3), (const float*)fake(4),
                             (const float*)fake(5), (const float*)fake(6), fake(7), fake(8), fake(9), nullptr) != VDN_OK);
      EXPECT(vdn_vda_backward_readout(&d, nullptr, fake(1), nullptr, (const float*)fake(3), fake(4), fake(5), ws,
                                      fake(6), fake(7), nullptr, fake(8), 1u << 30, nullptr) != VDN_OK);
      EXPECT(vdn_vda_backward_scan(&d, nullptr, fake(1), ws, (float*)fake(2), fake(3), 1u << 30, nullptr) != VDN_OK);
      EXPECT(vdn_vda_backward_gram(&d, nullptr, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7),
                                   fake(8), fake(9), fake(10), fake(11), fake(12), 1u << 30, nullptr) != VDN_OK);
      EXPECT(vdn_vda_gates(&d, 3072, nullptr, fake(1), (const float*)fake(2), fake(3), fake(4), (float*)fake(5),
                           fake(6), 1u << 30, nullptr) != VDN_OK);
      EXPECT(vdn_vda_out_proj(&d, 3072, nullptr, fake(1), fake(2), fake(3), nullptr) != VDN_OK);
      hipEvent_t ev[VDN_VDA_STAGES + 1];
      memset(ev, 0, sizeof ev);
      EXPECT(vdn_vda_forward_timed(&d, fake(0), fake(1), fake(2), (const float*)fake(3), fake(4), fake(5), fake(6),
                                   fake(7), fake(8), nullptr, fake(9), fake(10), ws, nullptr, ev,
                                   VDN_VDA_STAGES + 1) == VDN_ERR_INVALID_ARG);
      // overlapping output: rejected before any launch
      if (st == VDN_OK) {
        EXPECT(vdn_vda_forward(&d, fake(0), fake(1), fake(2), (const float*)fake(3), fake(4), fake(5), fake(6),
                               fake(7), fake(8), nullptr, (char*)fake(0) + 16, fake(10), ws, nullptr) != VDN_OK);
      }
    }
  }
  EXPECT(vdn_vda_validate(nullptr) == VDN_ERR_INVALID_ARG);
  EXPECT(vdn_vda_workspace_bytes(nullptr) == 0);
  for (int s = -1; s < 8; ++s) EXPECT(vdn_vda_status_string((vdn_status)s) != nullptr);
  printf("host ABI check: %d valid descriptors, %d failures\n", valid, failures);
  return failures ? 1 : 0;
}
