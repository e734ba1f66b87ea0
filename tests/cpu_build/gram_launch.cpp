// The statistics launch of the forward pass alone, in the CPU build, at any
// shape (the full 768p clip included), meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer:
//   gram_launch B H T grid_h grid_w d L bits|data [shard count] [seed]
// It launches the library's statistics kernel exactly as vdn_vda_forward does
// (frames 1 .. T-2 of every head and the text frame, bfloat16 inputs, one
// launch), on exact-size 16-byte aligned host allocations of K, V, beta and of
// the text tensors, so that an access one byte past any of them is reported.
// "bits" fills every input with arbitrary bit patterns (NaN, infinite and
// negative beta included); "data" with unit keys, N(0, 1) values and sigmoid
// betas, and then compares sampled statistics with a float64 reference.
// "shard count" runs only every count-th workgroup from the shard-th, so that
// processes can share one launch; each reports the slots its workgroups
// wrote.  Exit status 0 when the emulator reported nothing (and, for "data",
// the sampled statistics agree).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "simt.h"
#include "vda_internal.h"
#include "vdn_vda.h"

namespace {

uint64_t splitmix(uint64_t& s) {
  uint64_t z = (s += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

double uniform(uint64_t& s) { return (splitmix(s) >> 11) * 0x1.0p-53; }

double normal(uint64_t& s) {
  const double u = uniform(s) + 0x1.0p-54, v = uniform(s);
  return sqrt(-2 * log(u)) * cos(6.283185307179586 * v);
}

uint16_t to_bf16(double x) {
  const float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fff + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

double from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// An exact-size allocation (every size here is a multiple of 16 bytes).
uint16_t* alloc16(size_t elems) {
  const size_t bytes = elems * 2;
  if (bytes % 16) {
    fprintf(stderr, "size %zu is not a multiple of 16 bytes\n", bytes);
    exit(2);
  }
  return (uint16_t*)aligned_alloc(16, bytes ? bytes : 16);
}

constexpr uint32_t kUnwritten = 0x7fbadbadu;  // a NaN payload no kernel produces

}  // namespace

int main(int argc, char** argv) {
  if (argc < 9) {
    fprintf(stderr, "usage: gram_launch B H T grid_h grid_w d L bits|data [shard count] [seed]\n");
    return 2;
  }
  const int B = atoi(argv[1]), H = atoi(argv[2]), T = atoi(argv[3]), gh = atoi(argv[4]), gw = atoi(argv[5]),
            d = atoi(argv[6]), L = atoi(argv[7]);
  const bool bits = strcmp(argv[8], "bits") == 0;
  const int shard = argc > 10 ? atoi(argv[9]) : 0, count = argc > 10 ? atoi(argv[10]) : 1;
  uint64_t seed = argc > 11 ? (uint64_t)atoll(argv[11]) : 1;
  const int U = gh * gw;

  vdn_vda_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.B = B; desc.H = H; desc.T = T; desc.grid_h = gh; desc.grid_w = gw; desc.d_k = d; desc.d_v = d;
  desc.n_text = L; desc.chunk = 5; desc.dtype = VDN_BF16; desc.flags = VDN_VDA_EPILOGUE;
  desc.l2_eps = 1e-6f; desc.rms_eps = 1e-6f;
  if (vdn_vda_validate(&desc) != VDN_OK || T < 3) {
    fprintf(stderr, "descriptor rejected (or T < 3: no frame to absorb)\n");
    return 2;
  }
  vda::Problem p{};
  p.B = B; p.H = H; p.T = T; p.U = U; p.D = d; p.L = L; p.C = 5; p.nc = (T + 4) / 5;
  p.bf16 = true; p.epilogue = true; p.l2_eps = 1e-6f; p.rms_eps = 1e-6f;

  const size_t ntok = (size_t)B * T * U * H, ttok = (size_t)B * L * H;
  uint16_t *k = alloc16(ntok * d), *v = alloc16(ntok * d), *beta = alloc16(ntok);
  uint16_t *kt = L ? alloc16(ttok * d) : nullptr, *vt = L ? alloc16(ttok * d) : nullptr,
           *bt = L ? alloc16(ttok) : nullptr;
  if (bits) {
    auto fill = [&](uint16_t* x, size_t n) {
      for (size_t i = 0; i < n; i += 4) {
        const uint64_t r = splitmix(seed);
        for (size_t j = 0; j < 4 && i + j < n; ++j) x[i + j] = (uint16_t)(r >> (16 * j));
      }
    };
    fill(k, ntok * d), fill(v, ntok * d), fill(beta, ntok);
    if (L) fill(kt, ttok * d), fill(vt, ttok * d), fill(bt, ttok);
  } else {
    auto unit_rows = [&](uint16_t* x, size_t rows) {
      std::vector<double> r(d);
      for (size_t i = 0; i < rows; ++i) {
        double s = 0;
        for (int j = 0; j < d; ++j) s += (r[j] = normal(seed)) * r[j];
        for (int j = 0; j < d; ++j) x[i * d + j] = to_bf16(r[j] / sqrt(s));
      }
    };
    unit_rows(k, ntok);
    for (size_t i = 0; i < ntok * d; ++i) v[i] = to_bf16(normal(seed));
    for (size_t i = 0; i < ntok; ++i) beta[i] = to_bf16(1 / (1 + exp(-normal(seed))));
    if (L) {
      unit_rows(kt, ttok);
      for (size_t i = 0; i < ttok * d; ++i) vt[i] = to_bf16(normal(seed));
      for (size_t i = 0; i < ttok; ++i) bt[i] = to_bf16(1 / (1 + exp(-normal(seed))));
    }
  }

  // the statistics region of the workspace: [B H][T + 1 slots][A, B][d][d]
  const size_t slot_floats = (size_t)2 * d * d, nslots = (size_t)B * H * (T + 1);
  float* stats = (float*)aligned_alloc(256, (nslots * slot_floats * 4 + 255) / 256 * 256);
  for (size_t i = 0; i < nslots * slot_floats; ++i) memcpy(&stats[i], &kUnwritten, 4);

  // the launch vdn_vda_forward makes
  const int n_video = T - 2;
  const bool text = L > 0;
  const vda::GramPart parts[2] = {{k, v, beta, T, U, 1, n_video, 0},
                                  {text ? kt : k, text ? vt : v, text ? bt : beta, 1, L, 0, 1, T}};
  simt::set_block_shard(shard, count);
  if (vda::launch_gram(p, parts, 2, stats, nullptr) != hipSuccess) {
    fprintf(stderr, "launch failed\n");
    return 1;
  }

  // which slots this process's workgroups wrote, and (for "data") a sample of
  // them against a float64 reference
  auto written = [&](size_t slot) {
    for (size_t i = 0; i < slot_floats; ++i) {
      uint32_t u;
      memcpy(&u, &stats[slot * slot_floats + i], 4);
      if (u != kUnwritten) return true;
    }
    return false;
  };
  auto wholly_written = [&](size_t slot) {
    for (size_t i = 0; i < slot_floats; ++i) {
      uint32_t u;
      memcpy(&u, &stats[slot * slot_floats + i], 4);
      if (u == kUnwritten) return false;
    }
    return true;
  };
  std::vector<size_t> mine;
  int partial = 0, stray = 0;
  for (int bh = 0; bh < B * H; ++bh)
    for (int t = 0; t <= T; ++t) {
      const size_t slot = (size_t)bh * (T + 1) + t;
      const bool formed = (t >= 1 && t <= T - 2) || t == T;
      if (!written(slot)) continue;
      if (!formed) ++stray;
      else if (!wholly_written(slot)) ++partial;
      else mine.push_back(slot);
    }
  double worst_a = 0, worst_b = 0;
  int sampled = 0;
  if (!bits && !mine.empty()) {
    const size_t picks[] = {0, mine.size() / 3, mine.size() / 2, 2 * mine.size() / 3, mine.size() - 1};
    for (size_t pi : picks) {
      const size_t slot = mine[pi];
      const int bh = (int)(slot / (T + 1)), t = (int)(slot % (T + 1)), b = bh / H, h = bh % H;
      const bool tx = t == T;
      const int n = tx ? L : U;
      std::vector<double> A((size_t)d * d, 0), Bm((size_t)d * d, 0);
      for (int u = 0; u < n; ++u) {
        const size_t row = tx ? ((size_t)b * L + u) * H + h : (((size_t)b * T + t) * U + u) * H + h;
        const double be = from_bf16(tx ? bt[row] : beta[row]);
        const uint16_t* kr = (tx ? kt : k) + row * d;
        const uint16_t* vr = (tx ? vt : v) + row * d;
        for (int i = 0; i < d; ++i) {
          const double ki = be * from_bf16(kr[i]), vi = be * from_bf16(vr[i]);
          for (int j = 0; j < d; ++j) {
            const double kj = from_bf16(kr[j]);
            A[(size_t)i * d + j] += ki * kj;
            Bm[(size_t)i * d + j] += vi * kj;
          }
        }
      }
      const float* S = stats + slot * slot_floats;
      double ma = 0, mb = 0, ea = 0, eb = 0;
      for (size_t i = 0; i < (size_t)d * d; ++i) {
        ma = fmax(ma, fabs(A[i]));
        mb = fmax(mb, fabs(Bm[i]));
        ea = fmax(ea, fabs(S[i] - A[i]));
        eb = fmax(eb, fabs(S[(size_t)d * d + i] - Bm[i]));
      }
      worst_a = fmax(worst_a, ea / fmax(ma, 1e-30));
      worst_b = fmax(worst_b, eb / fmax(mb, 1e-30));
      ++sampled;
    }
  }
  printf("gram_launch B=%d H=%d T=%d U=%d d=%d L=%d %s shard %d/%d: workgroups %ld, slots written %zu, "
         "partly written %d, outside the formed slots %d, sampled %d (A %.2e, B %.2e), emulator errors %d\n",
         B, H, T, U, d, L, bits ? "bits" : "data", shard, count, simt::workgroups_run, mine.size(), partial, stray,
         sampled, worst_a, worst_b, simt::errors);
  const bool ok = simt::errors == 0 && partial == 0 && stray == 0 && (bits || (worst_a < 5e-3 && worst_b < 5e-3));
  free(k); free(v); free(beta); free(kt); free(vt); free(bt); free(stats);
  return ok ? 0 : 1;
}
