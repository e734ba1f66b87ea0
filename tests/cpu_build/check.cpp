// Self-checking CPU-build run of vdn_vda_forward (the library compiled for the
// host against simt.h), meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer:
//   check H T grid_h grid_w d L dtype(bf16|f32) [seed]
// Inputs are exact-size host allocations, so an access one byte past any
// tensor is reported.  Compares the statistics (A_t, B_t) and (I + A_t)^{-1}
// the forward leaves in its workspace with a float64 reference computed here,
// checks that the output is finite and that the emulator reported nothing;
// exit status 0 when all hold.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "vdn_vda.h"
#include "simt.h"

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fff + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static std::vector<double> inverse(std::vector<double> a, int n) {
  std::vector<double> inv(n * n, 0.0);
  for (int i = 0; i < n; ++i) inv[i * n + i] = 1;
  for (int c = 0; c < n; ++c) {
    int p = c;
    for (int r = c + 1; r < n; ++r)
      if (fabs(a[r * n + c]) > fabs(a[p * n + c])) p = r;
    for (int k = 0; k < n; ++k) {
      std::swap(a[c * n + k], a[p * n + k]);
      std::swap(inv[c * n + k], inv[p * n + k]);
    }
    const double d = a[c * n + c];
    for (int k = 0; k < n; ++k) {
      a[c * n + k] /= d;
      inv[c * n + k] /= d;
    }
    for (int r = 0; r < n; ++r) {
      if (r == c) continue;
      const double f = a[r * n + c];
      if (f == 0) continue;
      for (int k = 0; k < n; ++k) {
        a[r * n + k] -= f * a[c * n + k];
        inv[r * n + k] -= f * inv[c * n + k];
      }
    }
  }
  return inv;
}

int main(int argc, char** argv) {
  if (argc < 8) {
    fprintf(stderr, "usage: check H T grid_h grid_w d L bf16|f32 [seed]\n");
    return 2;
  }
  const int H = atoi(argv[1]), T = atoi(argv[2]), gh = atoi(argv[3]), gw = atoi(argv[4]), d = atoi(argv[5]),
            L = atoi(argv[6]);
  const bool bf = strcmp(argv[7], "bf16") == 0;
  const unsigned seed = argc > 8 ? (unsigned)atoi(argv[8]) : 1;
  const int B = 1, U = gh * gw;
  vdn_vda_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.B = B; desc.H = H; desc.T = T; desc.grid_h = gh; desc.grid_w = gw; desc.d_k = d; desc.d_v = d;
  desc.n_text = L; desc.chunk = 5; desc.dtype = bf ? VDN_BF16 : VDN_F32; desc.flags = VDN_VDA_EPILOGUE;
  desc.l2_eps = 1e-6f; desc.rms_eps = 1e-6f;
  if (vdn_vda_validate(&desc) != VDN_OK) {
    fprintf(stderr, "descriptor rejected\n");
    return 2;
  }
  std::mt19937 g(seed);
  std::normal_distribution<double> N(0, 1);
  const size_t ntok = (size_t)B * T * U * H, esz = bf ? 2 : 4;
  auto tensor = [&](size_t n) { return std::vector<unsigned char>(n * esz); };
  auto put = [&](std::vector<unsigned char>& t, size_t i, double x) {
    if (bf) {
      const uint16_t b = to_bf16((float)x);
      memcpy(&t[2 * i], &b, 2);
    } else {
      const float f = (float)x;
      memcpy(&t[4 * i], &f, 4);
    }
  };
  auto get = [&](const std::vector<unsigned char>& t, size_t i) {
    if (bf) {
      uint16_t b;
      memcpy(&b, &t[2 * i], 2);
      return from_bf16(b);
    }
    float f;
    memcpy(&f, &t[4 * i], 4);
    return (double)f;
  };
  auto q = tensor(ntok * d), k = tensor(ntok * d), v = tensor(ntok * d), gate = tensor(ntok * d), out = tensor(ntok * d);
  auto beta = tensor(ntok), kt = tensor((size_t)B * L * H * d), vt = tensor((size_t)B * L * H * d),
       bt = tensor((size_t)B * L * H);
  std::vector<float> alpha((size_t)B * T * H * d);
  auto unit_rows = [&](std::vector<unsigned char>& t, size_t rows) {
    std::vector<double> x(d);
    for (size_t r = 0; r < rows; ++r) {
      double s = 0;
      for (int j = 0; j < d; ++j) s += (x[j] = N(g)) * x[j];
      for (int j = 0; j < d; ++j) put(t, r * d + j, x[j] / sqrt(s));
    }
  };
  unit_rows(q, ntok);
  unit_rows(k, ntok);
  unit_rows(kt, (size_t)B * L * H);
  for (size_t i = 0; i < ntok * d; ++i) put(v, i, N(g)), put(gate, i, N(g));
  for (size_t i = 0; i < (size_t)B * L * H * d; ++i) put(vt, i, N(g));
  for (size_t i = 0; i < ntok; ++i) put(beta, i, 1 / (1 + exp(-N(g))));
  for (size_t i = 0; i < (size_t)B * L * H; ++i) put(bt, i, 1 / (1 + exp(-N(g))));
  for (auto& a : alpha) a = (float)(1 / (1 + exp(-(3 + N(g)))));

  const size_t ws = vdn_vda_workspace_bytes(&desc);
  vdn_vda_layout lay;
  vdn_vda_workspace_layout(&desc, &lay);
  // 256-byte aligned workspace
  std::vector<unsigned char> wsbuf(ws + 256);
  void* wsp = (void*)(((uintptr_t)wsbuf.data() + 255) & ~(uintptr_t)255);
  // exact-size, 16-byte aligned copies of every input (so AddressSanitizer sees
  // an access one byte past any tensor)
  auto dev = [&](const void* src, size_t n) {
    void* p = aligned_alloc(16, (n + 15) / 16 * 16);
    memcpy(p, src, n);
    return p;
  };
  void *dq = dev(q.data(), q.size()), *dk = dev(k.data(), k.size()), *dv = dev(v.data(), v.size()),
       *dg = dev(gate.data(), gate.size()), *db = dev(beta.data(), beta.size()),
       *dkt = L ? dev(kt.data(), kt.size()) : nullptr, *dvt = L ? dev(vt.data(), vt.size()) : nullptr,
       *dbt = L ? dev(bt.data(), bt.size()) : nullptr, *da = dev(alpha.data(), alpha.size() * 4),
       *dout = dev(out.data(), out.size());
  const vdn_status st = vdn_vda_forward(&desc, dq, dk, dv, (const float*)da, db, dkt, dvt, dbt, dg, nullptr, dout, wsp,
                                        ws, nullptr);
  if (st != VDN_OK) {
    fprintf(stderr, "forward: %s\n", vdn_vda_status_string(st));
    return 1;
  }
  memcpy(out.data(), dout, out.size());

  // reference statistics and inverse of every formed slot
  const bool split = bf && d >= 32;
  double worst_a = 0, worst_b = 0, worst_p = 0;
  auto slot_ref = [&](int h, int t, std::vector<double>& A, std::vector<double>& Bm) {
    A.assign(d * d, 0);
    Bm.assign(d * d, 0);
    const bool text = t == T;
    const int n = text ? L : U;
    for (int u = 0; u < n; ++u) {
      const size_t row = text ? ((size_t)u * H + h) : (((size_t)t * U + u) * H + h);
      const double b = text ? get(bt, row) : get(beta, row);
      for (int i = 0; i < d; ++i) {
        const double ki = text ? get(kt, row * d + i) : get(k, row * d + i);
        const double vi = text ? get(vt, row * d + i) : get(v, row * d + i);
        for (int j = 0; j < d; ++j) {
          const double kj = text ? get(kt, row * d + j) : get(k, row * d + j);
          A[i * d + j] += b * ki * kj;
          Bm[i * d + j] += b * vi * kj;
        }
      }
    }
  };
  std::vector<int> slots;
  for (int t = 1; t <= T - 2; ++t) slots.push_back(t);
  slots.push_back(T);  // the text frame
  for (int h = 0; h < H; ++h) {
    for (int t : slots) {
      std::vector<double> A, Bm;
      slot_ref(h, t, A, Bm);
      const size_t slot = (size_t)h * (T + 1) + t;
      const float* S = (const float*)((char*)wsp + lay.stats) + slot * 2 * d * d;
      double ma = 0, mb = 0, ea = 0, eb = 0;
      for (int i = 0; i < d * d; ++i) {
        ma = fmax(ma, fabs(A[i]));
        mb = fmax(mb, fabs(Bm[i]));
        ea = fmax(ea, fabs(S[i] - A[i]));
        eb = fmax(eb, fabs(S[d * d + i] - Bm[i]));
      }
      worst_a = fmax(worst_a, ea / fmax(ma, 1e-30));
      worst_b = fmax(worst_b, eb / fmax(mb, 1e-30));
      std::vector<double> P(A);
      for (int i = 0; i < d; ++i) P[i * d + i] += 1;
      const std::vector<double> Pi = inverse(P, d);
      const char* base = (const char*)wsp + lay.pinv + slot * (size_t)d * d * 4;
      std::vector<double> got(d * d, NAN);
      if (split) {
        const int NFR = d * d / 8, KS2 = d / 32;
        const uint16_t* hi = (const uint16_t*)base;
        const uint16_t* lo = hi + (size_t)NFR * 8;
        for (int f = 0; f < NFR; ++f) {
          const int l = f & 63, s = (f >> 6) % KS2, we = (f >> 6) / KS2;
          const int c = 32 * (we >> 1) + 2 * (l & 15) + (we & 1);
          for (int j = 0; j < 8; ++j)
            got[(32 * s + 8 * (l >> 4) + j) * d + c] = from_bf16(hi[8 * f + j]) + from_bf16(lo[8 * f + j]);
        }
      } else {
        const float* pf = (const float*)base;
        for (int i = 0; i < d * d; ++i) got[i] = pf[i];
      }
      double mp = 0, ep = 0;
      for (int i = 0; i < d * d; ++i) {
        mp = fmax(mp, fabs(Pi[i]));
        ep = fmax(ep, std::isnan(got[i]) ? INFINITY : fabs(got[i] - Pi[i]));
      }
      worst_p = fmax(worst_p, ep / mp);
    }
  }
  bool finite = true;
  for (size_t i = 0; i < ntok * d; ++i) finite = finite && std::isfinite(get(out, i));
  printf("H=%d T=%d U=%d d=%d L=%d %s: A %.2e  B %.2e  P^-1 %.2e  output %s  emulator errors %d\n", H, T, U, d, L,
         bf ? "bf16" : "f32", worst_a, worst_b, worst_p, finite ? "finite" : "NOT FINITE", simt::errors);
  const bool ok = worst_a < 5e-3 && worst_b < 5e-3 && worst_p < 5e-3 && finite && simt::errors == 0;
  free(dq); free(dk); free(dv); free(dg); free(db); free(dkt); free(dvt); free(dbt); free(da); free(dout);
  return ok ? 0 : 1;
}
