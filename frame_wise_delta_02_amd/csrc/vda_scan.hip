// vda_scan: the bidirectional frame recurrence of Video Delta Attention, and the
// gather of the two directions' states for the readout.
//
// Text state: S_T = B_T (I + A_T)^{-1}, the frame update from a zero state over
// the text tokens; both directions start from S_T / 2 so that the two readouts
// together count the prompt once ("Video DeltaNet" summary, onedev.kr/papers/80,
// section "어떻게 동작하나").  Each absorbed frame s applies
//     S <- (S Diag(alpha_s) + B_s)(I + A_s)^{-1}
// (section "어떻게 쓰나"); the reverse direction applies the same update in
// reverse frame order.  Anchor frames (0, T-1) are never absorbed (section
// "전제와 한계").  The forward scan records F_j after the last frame of chunk
// j, the reverse scan R_j after the first frame of chunk j; a query in chunk c
// reads F_{c-2} + R_{c+2} (S_T / 2 where a range is empty), so only F_0..F_{n-3}
// and R_2..R_{n-1} are produced.
//
// Parallel form: S <- Y P^{-1} acts on the rows of S independently, so each
// (batch, head, direction) is split into 16-row blocks that scan with no
// communication at all.  A workgroup keeps its 16 x d block of Y in LDS; each
// lane owns two adjacent columns of the state (fp32, in registers).  The next
// frame's P^{-1}, B and alpha are prefetched into registers while the current
// frame's MFMAs run.  Row blocks of one head go to the same XCD (blockIdx % 8)
// so the P^{-1}_s they all read is shared in that XCD's L2.
//
// The product Y P^{-1} runs in one of two ways:
//  * float32 inputs, or d = 16: v_mfma_f32_16x16x4f32 on fp32 operands.
//  * bfloat16 inputs, d >= 32: both operands split into bfloat16 hi + lo
//    (Y when it is formed, P^{-1} by the solve), and Y P^{-1} ~ Yh Ph + Yh Pl +
//    Yl Ph on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Each term is
//    exact in fp32; the split keeps about 16 significant bits of each operand
//    and the dropped Yl Pl is below 2^-16 of |Y||P|, two orders below the
//    bfloat16 rounding of the output.  The state stays fp32.  This is three
//    matrix-core passes at 16x the fp32 rate: a frame step costs about 3/16 of
//    the fp32 matrix-core time.
#include <type_traits>

#include "vda_internal.h"

namespace vda {
namespace {

// 16-row m-tiles per workgroup: the split path takes 32 rows, so a workgroup
// loads each P^{-1}_s once for twice the rows (the per-CU load path, not the
// matrix cores, bounds a frame step there) and B*H*2*d/32 workgroups stay
// within one per CU at 768p.
template <bool SPLIT>
constexpr int scan_mtiles() { return SPLIT ? 2 : 1; }

// P^{-1} fragments of one frame for one lane
template <int D, bool SPLIT>
struct PFrag;
template <int D>
struct PFrag<D, false> {  // column pair c0, c0+1 (c0 = 16*NV*wave + NV*(lane%16)), k = (d/4)(lane/16) + ks
  typedef float vec_t __attribute__((ext_vector_type(D >= 32 ? 2 : 1)));
  vec_t v[D / 4];
};
template <int D>
struct PFrag<D, true> {   // [e][ks]: fragment (2*wave + e, ks) of the hi and lo planes
  uint4 hi[2][D / 32], lo[2][D / 32];
};

// Three uses of one frame-step machinery:
//   SCAN_FRAMES  the bidirectional scan frame by frame (S_T first, then every
//                absorbed frame, recording F_j / R_j at chunk boundaries);
//   SCAN_COMPOSE each chunk's transition as one pair (M_c, J_c) with
//                S_out = S_in M_c + J_c: the chunk's frames scanned from
//                S = I with no writes (rows of M_c) and from S = 0 with the
//                writes (rows of J_c), every chunk of every direction at once;
//   SCAN_CHUNKS  the scan over those pairs, S <- S M_c + J_c, one step per
//                chunk (n_c - 2 serial steps instead of one per frame).
// Composing the frame updates of a chunk is exact in exact arithmetic, so the
// two routes give the same F_j and R_j up to rounding.
// Two more serve the backward pass (the derivative of the scan):
//   SCAN_STATES  the frame scan recording the state after every frame s into
//                slot s of fwd / rev ([B, H, T+2, d, d] each), the start state
//                S_T / 2 in slot 0 (forward) and slot T-1 (reverse);
//   SCAN_ADJOINT the adjoint recurrence, each direction in the reverse of its
//                own order: lambda <- (lambda + dRec_j) P_s Diag(alpha_s), the
//                record adjoints dF_j, dR_j (read from fwd / rev, [B, H, n_c, d, d])
//                added at the frames whose state they record; the adjoint at
//                frame s (after that addition, before the product) recorded in
//                slot s of chunk_m (forward) / chunk_j (reverse) ([B, H, T+1, d, d]),
//                the final adjoint (that of the start state) into s_text
//                ([B, H, 2, d, d]).
enum { SCAN_FRAMES = 0, SCAN_COMPOSE = 1, SCAN_CHUNKS = 2, SCAN_STATES = 3, SCAN_ADJOINT = 4 };

template <int D, bool SPLIT, int MODE>
__global__ __launch_bounds__(64 * (D / (D >= 32 ? 32 : 16)))
void scan_rows(const float* __restrict__ stats, const float* __restrict__ pinv,
               const float* __restrict__ alpha, float* __restrict__ s_text, float* __restrict__ fwd,
               float* __restrict__ rev, float* __restrict__ chunk_m, float* __restrict__ chunk_j, int B, int H,
               int T, int C, int nc) {
  static_assert(!SPLIT || D >= 32, "the bfloat16 split needs k-steps of 32");
  constexpr bool COMPOSE = MODE == SCAN_COMPOSE, CHUNKS = MODE == SCAN_CHUNKS;
  constexpr bool STATES = MODE == SCAN_STATES, ADJ = MODE == SCAN_ADJOINT;
  constexpr int MT = scan_mtiles<SPLIT>();
  constexpr int RB = 16 * MT;            // state rows per workgroup
  constexpr int NV = D >= 32 ? 2 : 1;    // adjacent columns per lane
  constexpr int WCOLS = 16 * NV;
  constexpr int KS = D / 4;
  constexpr int KS2 = D / 32;            // k-steps of the split product
  constexpr int NRB = D / RB;
  constexpr int LDY = D + 4;             // fp32 Y row (floats)
  constexpr int LDYS = D + 8;            // bfloat16 Y row (elements; 16-B aligned rows)
  constexpr int NFR = D * D / 8;         // 16-B fragments per plane
  constexpr int RBPU = COMPOSE ? 2 * NRB : NRB;  // row blocks per unit (COMPOSE: M rows, then J rows)
  typedef float vec_t __attribute__((ext_vector_type(NV)));
  constexpr int YBYTES = SPLIT ? 2 * 2 * RB * LDYS * 2 : 2 * RB * LDY * 4;
  __shared__ __attribute__((aligned(16))) unsigned char ybytes[YBYTES];
  float* ylds = reinterpret_cast<float*>(ybytes);            // [2][RB * LDY]      (fp32 path)
  __bf16* ysp = reinterpret_cast<__bf16*>(ybytes);           // [2 buf][2 plane][RB * LDYS]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // blockIdx -> (unit, row block) with all row blocks of a unit on one XCD
  // (blocks are dealt to the 8 XCDs round-robin), so the operand they all read
  // is fetched once into that XCD's L2; a unit is a (batch, head, direction),
  // with COMPOSE also a chunk.  The grid rounds the units up to a multiple of
  // 8; the blocks past the last unit exit at once.
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int groups = B * H * 2;
  const int nch = nc > 2 ? nc - 2 : 0;   // chunks with a record, per direction
  const int units = COMPOSE ? groups * nch : groups;
  int u, rbi;
  if (nblk == (units + 7) / 8 * 8 * RBPU) {
    const int xcd = bid % 8, slot = bid / 8;
    rbi = slot % RBPU;
    u = (slot / RBPU) * 8 + xcd;
  } else {
    rbi = bid % RBPU;
    u = bid / RBPU;
  }
  if (u >= units) return;
  const int g = COMPOSE ? u / nch : u;
  const int dir = g % 2;
  const int h = (g / 2) % H;
  const int b = g / (2 * H);
  const bool mpart = COMPOSE && rbi < NRB;  // COMPOSE: this block forms rows of M_c
  const int row0 = (COMPOSE && !mpart ? rbi - NRB : rbi) * RB;

  const size_t head = (size_t)(b * H + h);
  const float* P0 = pinv + head * (T + 1) * (size_t)(D * D);
  const float* S0 = stats + head * (T + 1) * (size_t)(2 * D * D) + (size_t)D * D;  // B part
  const float* A0 = alpha + (size_t)b * T * H * D + (size_t)h * D;                 // + s*H*D
  // chunk pairs of this (batch, head, direction): slot j of [n_c][d][d] each
  const size_t cslot = (head * 2 + dir) * (size_t)nc * (D * D);
  const float* CM = CHUNKS ? chunk_m + cslot : P0;
  // the per-step "B rows": B_s, J_c (SCAN_CHUNKS) or the record adjoints (SCAN_ADJOINT)
  const float* CJ = CHUNKS ? chunk_j + cslot : ADJ ? (dir == 0 ? fwd : rev) + head * (size_t)nc * (D * D) : S0;
  constexpr size_t BSTRIDE = (CHUNKS || ADJ) ? (size_t)D * D : (size_t)2 * D * D;  // slot stride of CJ

  const int c0 = wave * WCOLS + NV * (lane & 15);
  const int rr = 4 * (lane >> 4);  // first of this lane's 4 rows in each m-tile

  vec_t st[MT][4];  // this lane's entries of S: rows 16 mt + rr + r, columns c0..c0+NV-1
  // two register sets, A and B, of a frame's P^{-1} fragments, B rows and
  // alpha: one is multiplied while the other is loading
  PFrag<D, SPLIT> pfA, pfB;
  vec_t bwA[MT][4], bwB[MT][4], alA, alB;

  // fp32 path: k-step ks of lane group g = lane / 16 covers channel (d/4) g + ks,
  // so each lane reads a contiguous run of Y (128-bit LDS loads) and of P^{-1} rows
  const int kg = (D / 4) * (lane >> 4);
  // split path: the fragments of k-step ks of slot s of `base` (both column tiles, hi and lo)
  auto ld_p_ks = [&](const float* base, int s, int ks, PFrag<D, SPLIT>& dst) {
    if constexpr (SPLIT) {
      const uint4* F = reinterpret_cast<const uint4*>(base + (size_t)s * D * D) + (size_t)(2 * wave * KS2) * 64 + lane;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dst.hi[e][ks] = F[(e * KS2 + ks) * 64];
        dst.lo[e][ks] = F[NFR + (e * KS2 + ks) * 64];
      }
    }
  };
  auto ld_p = [&](const float* base, int s, PFrag<D, SPLIT>& dst) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) ld_p_ks(base, s, ks, dst);
    } else {
      const float* P = base + (size_t)s * D * D + c0 + (size_t)kg * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst.v[ks] = *reinterpret_cast<const vec_t*>(P + ks * D);
    }
  };
  auto ld_bw = [&](const float* base, size_t stride, int s, vec_t (&dst)[MT][4]) {
    const float* Bs = base + (size_t)s * stride + (size_t)(row0 + rr) * D + c0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[mt][r] = *reinterpret_cast<const vec_t*>(Bs + (16 * mt + r) * D);
  };
  auto ld_al = [&](int s) -> vec_t {
    return *reinterpret_cast<const vec_t*>(A0 + (size_t)s * H * D + c0);
  };
  // Y = S Diag(alpha) + B into buffer buf (alpha = 0 for the text frame; the
  // rows of M_c take no writes)
  auto put_y = [&](int buf, const vec_t (&sv)[MT][4], vec_t a, const vec_t (&bv)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vec_t y;
        if constexpr (COMPOSE)
          y = mpart ? sv[mt][r] * a : sv[mt][r] * a + bv[mt][r];
        else
          y = sv[mt][r] * a + bv[mt][r];
        const int row = 16 * mt + rr + r;
        if constexpr (SPLIT) {
          __bf16* yh = ysp + (2 * buf) * (RB * LDYS);
          __bf16* yl = yh + RB * LDYS;
          __bf16 h0, l0, h1, l1;
          split_bf16(y[0], h0, l0);
          split_bf16(y[1], h1, l1);
          *reinterpret_cast<bf16x2*>(&yh[row * LDYS + c0]) = bf16x2{h0, h1};
          *reinterpret_cast<bf16x2*>(&yl[row * LDYS + c0]) = bf16x2{l0, l1};
        } else {
          *reinterpret_cast<vec_t*>(&ylds[buf * (RB * LDY) + row * LDY + c0]) = y;
        }
      }
  };
  // S = Y P from buffer buf (P^{-1} of a frame, or M_c).  Split path: with
  // sn >= 0, k-step ks also issues slot sn's fragments of k-step ks (from
  // pbase) into pn, so the per-CU load path streams the next step's operand
  // while the matrix cores work on this one.
  auto mul = [&](int buf, const PFrag<D, SPLIT>& p, const float* pbase, int sn, PFrag<D, SPLIT>& pn) {
    if constexpr (SPLIT) {
      // A operand of m-tile mt: row 16 mt + lane%16, k = 32 ks + 8 (lane/16) .. +7.
      // The three terms of a tile share one accumulator: four independent
      // matrix-core chains (m-tile x column tile), each at most 3*(d/32) long.
      const __bf16* yh = ysp + (2 * buf) * (RB * LDYS) + (lane & 15) * LDYS + 8 * (lane >> 4);
      const __bf16* yl = yh + RB * LDYS;
      f32x4 acc[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        if (sn >= 0) ld_p_ks(pbase, sn, ks, pn);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 ah = *reinterpret_cast<const bf16x8*>(yh + 16 * mt * LDYS + 32 * ks);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(yl + 16 * mt * LDYS + 32 * ks);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const bf16x8 ph = __builtin_bit_cast(bf16x8, p.hi[e][ks]);
            const bf16x8 pl = __builtin_bit_cast(bf16x8, p.lo[e][ks]);
            acc[mt][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, ph, acc[mt][e], 0, 0, 0);
            acc[mt][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, pl, acc[mt][e], 0, 0, 0);
            acc[mt][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ph, acc[mt][e], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep each k-step's loads beside its products
      }
      // m-tile mt, column tile e, lane l, reg r: S[16 mt + 4 (l/16) + r][32 wave + 2 (l%16) + e]
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 2; ++e) st[mt][r][e] = acc[mt][e][r];
    } else {
      // two accumulators per tile (even and odd k-step groups) keep four
      // independent matrix-core chains in flight
      static_assert(SPLIT || MT == 1, "the fp32 product takes one m-tile");
      f32x4 acc[NV][2];
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[e][0] = acc[e][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* yrow = &ylds[buf * (RB * LDY) + (lane & 15) * LDY + kg];
#pragma unroll
      for (int k4 = 0; k4 < KS / 4; ++k4) {
        const float4 a4 = *reinterpret_cast<const float4*>(yrow + 4 * k4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < NV; ++e)
            acc[e][q & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], p.v[4 * k4 + q][e], acc[e][q & 1], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < NV; ++e) st[0][r][e] = acc[e][0][r] + acc[e][1][r];
    }
  };
  auto put_state = [&](float* dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<vec_t*>(dst + (size_t)(row0 + 16 * mt + rr + r) * D + c0) = st[mt][r];
  };

  // ---- step list of this direction -------------------------------------------
  // SCAN_FRAMES forward: frames 1 .. min(C*(nc-2)-1, T-2); reverse: T-2 .. max(2C, 1).
  // SCAN_COMPOSE: the frames of one chunk j in this direction's order (forward
  // chunks 0 .. nc-3, reverse chunks nc-1 .. 2; anchors excluded).
  // SCAN_CHUNKS: the chunk indices themselves.
  int first, last, step, nsteps, cj = 0;
  if constexpr (COMPOSE) {
    const int ci = u % nch;
    cj = dir == 0 ? ci : nc - 1 - ci;
    const int lo = max(C * cj, 1), hi = min(C * (cj + 1) - 1, T - 2);
    first = dir == 0 ? lo : hi;
    last = dir == 0 ? hi : lo;
    step = dir == 0 ? 1 : -1;
    nsteps = max(0, hi - lo + 1);
  } else if constexpr (CHUNKS) {
    first = dir == 0 ? 0 : nc - 1;
    step = dir == 0 ? 1 : -1;
    last = first + step * (nch - 1);
    nsteps = nch;
  } else if constexpr (ADJ) {
    // the forward scan's frames 1 .. e backwards, the reverse scan's b .. T-2 forwards
    const int e = nc >= 3 ? min(C * (nc - 2) - 1, T - 2) : 0;
    const int bl = nc >= 3 ? max(2 * C, 1) : T - 1;
    first = dir == 0 ? e : bl;
    last = dir == 0 ? 1 : T - 2;
    step = dir == 0 ? -1 : 1;
    nsteps = dir == 0 ? max(0, e) : max(0, T - 2 - bl + 1);
  } else {
    if (dir == 0) {
      first = 1;
      last = nc >= 3 ? min(C * (nc - 2) - 1, T - 2) : 0;
      step = 1;
    } else {
      first = T - 2;
      last = nc >= 3 ? max(2 * C, 1) : T - 1;
      step = -1;
    }
    nsteps = (dir == 0) ? max(0, last - first + 1) : max(0, first - last + 1);
  }
  (void)last;
  // this head's records: n_c chunk states; SCAN_STATES T+2 frame states;
  // SCAN_ADJOINT T+1 frame adjoints
  constexpr int NREC_EXTRA = STATES ? 2 : 1;
  const int nrec = (STATES || ADJ) ? T + NREC_EXTRA : nc;
  // (the composition pass writes no records, and its launch passes no record
  // buffers: no address is formed for it)
  float* out0 = COMPOSE ? nullptr
                        : (ADJ ? (dir == 0 ? chunk_m : chunk_j) : (dir == 0 ? fwd : rev)) + head * (size_t)nrec * D * D;
  const auto rec = make_rsrc(out0, (uint32_t)nrec * D * D * 4);

  vec_t zero4[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) zero4[mt][r] = vec_t(0.f);

  if constexpr (ADJ) {
    // ---- start: lambda = 0; the first frame's loads (with no frame, the text
    // slot and frame 0's alpha: in bounds, never used) -------------------------
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[mt][r] = vec_t(0.f);
    ld_bw(CJ, BSTRIDE, nsteps > 0 ? min(first / C, nc - 1) : 0, bwA);
    alA = ld_al(nsteps > 0 ? first : 0);
    ld_p(P0, nsteps > 0 ? first : T, pfA);
  } else if constexpr (COMPOSE) {
    // ---- start: rows row0.. of I (M_c) or of 0 (J_c); first frame's loads --
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < NV; ++e) st[mt][r][e] = (mpart && row0 + 16 * mt + rr + r == c0 + e) ? 1.f : 0.f;
    // with no frame in the chunk these re-read the text slot and frame 0's
    // alpha (in bounds, never used)
    const int s1 = nsteps > 0 ? first : T;
    ld_bw(S0, BSTRIDE, s1, bwA);
    alA = ld_al(nsteps > 0 ? first : 0);
    ld_p(P0, s1, pfA);
  } else {
    // ---- text frame (slot T): S_T = B_T P_T^{-1} -----------------------------
    // Set B holds the text frame.  The first step's loads (set A) are in flight
    // during its product; with no step to take they re-read the text slot
    // (SCAN_CHUNKS: chunk slot 0) and frame 0's alpha (in bounds, never used).
    ld_bw(S0, (size_t)2 * D * D, T, bwB);
    ld_p(P0, T, pfB);
    put_y(0, zero4, vec_t(0.f), bwB);
    if constexpr (CHUNKS) {
      const int j1 = nsteps > 0 ? first : 0;
      ld_bw(CJ, BSTRIDE, j1, bwA);
      alA = vec_t(1.f);
      ld_p(CM, j1, pfA);
    } else {
      const int s1 = nsteps > 0 ? first : T;
      ld_bw(S0, BSTRIDE, s1, bwA);
      alA = ld_al(nsteps > 0 ? first : 0);
      ld_p(P0, s1, pfA);
    }
    lds_barrier();
    mul(0, pfB, P0, -1, pfA);
    if (dir == 0 && !STATES) put_state(s_text + head * (size_t)(D * D));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[mt][r] *= 0.5f;
    if constexpr (STATES) put_state(out0 + (size_t)(dir == 0 ? 0 : T - 1) * (D * D));
  }

  // the record index after absorbing frame s (or -1)
  auto rec_after = [&](int s) -> int {
    if (dir == 0) {
      const int j = s / C;  // F_j after the last absorbed frame of chunk j
      const bool end = (s == min(C * (j + 1) - 1, T - 2));
      return (end && j <= nc - 3) ? j : -1;
    }
    const int j = s / C;    // R_j after the first absorbed frame of chunk j
    const bool beg = (s == max(C * j, 1));
    return (beg && j >= 2) ? j : -1;
  };
  if constexpr (MODE == SCAN_FRAMES) {
    // chunks whose recorded state precedes every absorbed frame (empty coverage)
    if (dir == 0) {
      for (int j = 0; j <= nc - 3; ++j)
        if (min(C * (j + 1) - 1, T - 2) < 1) put_state(out0 + (size_t)j * D * D);
    } else {
      for (int j = nc - 1; j >= 2; --j)
        if (max(C * j, 1) > T - 2) put_state(out0 + (size_t)j * D * D);
    }
  }

  // One step: form Y from the current set, load the next step into the other
  // set (unconditionally: the last step re-reads its own slot), and multiply.
  // The loop body runs two steps with the sets swapped, so no register copy
  // waits for a load and the product only waits for the loads issued one step
  // earlier (the load counter is in order).  SCAN_CHUNKS: Y = S, and the set's
  // "B rows" are J_c, added after the product.
  auto frame = [&](int i, int s, int buf, const PFrag<D, SPLIT>& pc, const vec_t (&bc)[MT][4], vec_t ac,
                   PFrag<D, SPLIT>& pn, vec_t (&bn)[MT][4], vec_t& an) {
    const int sn = i + 1 < nsteps ? s + step : s;
    if constexpr (ADJ) {
      // lambda at frame s: the propagated adjoint plus the record adjoint of
      // the state frame s produces, if any; recorded, then Y = lambda
      const float inj = rec_after(s) >= 0 ? 1.f : 0.f;
      vec_t lam[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) lam[mt][r] = st[mt][r] + bc[mt][r] * inj;
      const uint32_t jo = (uint32_t)s * (uint32_t)(D * D * 4);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t o = jo + (uint32_t)(((row0 + 16 * mt + rr + r) * D + c0) * 4);
          if constexpr (NV == 2)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, lam[mt][r]),
                                                  rec, o, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, lam[mt][r][0]), rec, o, 0, 0);
        }
      put_y(buf, lam, vec_t(1.f), zero4);
    } else if constexpr (CHUNKS) {
      put_y(buf, st, vec_t(1.f), zero4);
    } else {
      put_y(buf, st, ac, bc);
    }
    ld_bw(CJ, BSTRIDE, ADJ ? min(sn / C, nc - 1) : sn, bn);  // needed first (next step's Y), so issued first
    if constexpr (CHUNKS)
      an = vec_t(1.f);
    else
      an = ld_al(sn);  // SCAN_ADJOINT: applied after the product
    if constexpr (!SPLIT) ld_p(CM, sn, pn);  // the split path loads P inside the product
    // keep the loads here, ahead of the product (the compiler would otherwise
    // sink them below it, next to their first use)
    asm volatile("" ::: "memory");
    lds_barrier();
    mul(buf, pc, CM, SPLIT ? sn : -1, pn);
    if constexpr (CHUNKS) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[mt][r] += bc[mt][r];
    }
    if constexpr (ADJ) {  // lambda <- (lambda P_s) Diag(alpha_s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[mt][r] *= ac;
    }
    if constexpr (!COMPOSE && !ADJ) {
      // record without a branch: the store is always issued and lands past the
      // buffer's end (dropped by the buffer unit) unless frame s ends a record,
      // so every step issues the same memory operations and the load waits need
      // not allow for a store that may or may not be in flight.  SCAN_CHUNKS
      // records after every step.
      const int j = (CHUNKS || STATES) ? s : rec_after(s);
      const uint32_t jo = j >= 0 ? (uint32_t)j * (uint32_t)(D * D * 4) : 0x80000000u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t o = jo + (uint32_t)(((row0 + 16 * mt + rr + r) * D + c0) * 4);
          if constexpr (NV == 2)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, st[mt][r]),
                                                  rec, o, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, st[mt][r][0]), rec, o, 0, 0);
        }
    }
  };
  // drain every load and store of the prologue once, so that the wait counts
  // inside the loop only have to account for the loop's own memory operations
  __builtin_amdgcn_s_waitcnt(0);
  for (int i = 0, s = first; i < nsteps; i += 2, s += 2 * step) {
    frame(i, s, 1, pfA, bwA, alA, pfB, bwB, alB);
    if (i + 1 >= nsteps) break;
    frame(i + 1, s + step, 0, pfB, bwB, alB, pfA, bwA, alA);
  }

  if constexpr (ADJ) put_state(s_text + (head * 2 + dir) * (size_t)(D * D));  // the start state's adjoint

  if constexpr (COMPOSE) {
    // ---- the chunk's pair: J_c rows as fp32 [d][d]; M_c rows in the layout
    // the product reads its right operand in (fp32 [d][d], or the two
    // bfloat16 fragment planes of the split path) ---------------------------
    const size_t off = cslot + (size_t)cj * (D * D);
    if (!mpart || !SPLIT) {
      put_state((mpart ? chunk_m : chunk_j) + off);
    } else if constexpr (SPLIT) {
      // This block's 32 rows are k-step rbi of M_c.  Each wave owns columns
      // 32 wave .. +31 of all 32 rows, so the relayout stays inside the wave:
      // rows go through the LDS buffer the last step did not use (every wave
      // has passed that step's barrier, so no wave still reads it), then each
      // lane gathers its fragments' 8 consecutive rows of one column.
      const int buf = nsteps > 0 && ((nsteps - 1) & 1) == 0 ? 0 : 1;
      put_y(buf, st, vec_t(1.f), zero4);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const __bf16* yh = ysp + (2 * buf) * (RB * LDYS);
      const __bf16* yl = yh + RB * LDYS;
      uint4* F = reinterpret_cast<uint4*>(chunk_m + off);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int col = 32 * wave + 2 * (lane & 15) + e;
        uint16_t hv[8], lv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = 8 * (lane >> 4) + j;
          hv[j] = __builtin_bit_cast(uint16_t, yh[row * LDYS + col]);
          lv[j] = __builtin_bit_cast(uint16_t, yl[row * LDYS + col]);
        }
        const size_t f = (size_t)((2 * wave + e) * KS2 + rbi) * 64 + lane;
        F[f] = make_uint4(hv[0] | (uint32_t)hv[1] << 16, hv[2] | (uint32_t)hv[3] << 16,
                          hv[4] | (uint32_t)hv[5] << 16, hv[6] | (uint32_t)hv[7] << 16);
        F[NFR + f] = make_uint4(lv[0] | (uint32_t)lv[1] << 16, lv[2] | (uint32_t)lv[3] << 16,
                                lv[4] | (uint32_t)lv[5] << 16, lv[6] | (uint32_t)lv[7] << 16);
      }
    }
  }
}

// Readout states: slot c < nc holds F_{c-2} + R_{c+2} (S_T/2 for a missing side),
// slot nc holds S_T (anchor frames).  With the decay bridge, slot c < nc holds
// F_{c-2} Diag(df) + R_{c+2} Diag(dr), df (dr) the per-key-channel product of
// alpha over chunk c-1 (c+1): those frames absorbed with zero writes, anchors
// included (ones where the chunk does not exist).  Written in the readout
// kernel's operand order (see vda_readout.hip): for every (m-tile, k-step,
// lane) the lane's matrix-core A-operand.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void gather_states(const float* __restrict__ s_text,
                                                     const float* __restrict__ fwd,
                                                     const float* __restrict__ rev,
                                                     const float* __restrict__ alpha,
                                                     void* __restrict__ rstates, int nc, int T, int H,
                                                     int C, int bridge) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int HALF = DP / 2;
  constexpr int MT = DP / 32;
  const int slot = blockIdx.x % (nc + 1);
  const size_t head = blockIdx.x / (nc + 1);
  // per-key-channel bridge factors of this slot (alpha [B, T, H, D])
  __shared__ float dfw[D], drv[D];
  if (threadIdx.x < D) {
    const int k = threadIdx.x, b = (int)(head / H), h = (int)(head % H);
    float df = 1.f, dr = 1.f;
    if (bridge && slot < nc) {
      if (slot >= 1)
        for (int s = C * (slot - 1); s < C * slot; ++s) df *= alpha[(((size_t)b * T + s) * H + h) * D + k];
      if (slot + 1 <= nc - 1)
        for (int s = C * (slot + 1); s < min(C * (slot + 2), T); ++s)
          dr *= alpha[(((size_t)b * T + s) * H + h) * D + k];
    }
    dfw[k] = df;
    drv[k] = dr;
  }
  __syncthreads();
  const float* ST = s_text + head * D * D;
  const float* Fp = nullptr;
  const float* Rp = nullptr;
  if (slot < nc) {
    if (slot >= 2) Fp = fwd + (head * nc + (slot - 2)) * D * D;
    if (slot + 2 <= nc - 1) Rp = rev + (head * nc + (slot + 2)) * D * D;
  }
  auto dv_of = [&](int mt, int m) { return HALF * ((m >> 2) & 1) + 16 * mt + 4 * (m >> 3) + (m & 3); };
  // The slot's state is wf F + wr R: a missing side reads S_T with weight 1/2,
  // and the anchor slot reads S_T twice with weight 1/2 (x/2 + x/2 = x exactly
  // for normal numbers),
  // so every fragment is four float4 loads with no branch.
  const float* Fs = Fp ? Fp : ST;
  const float* Rs = Rp ? Rp : ST;
  const float wf = Fp ? 1.f : 0.5f, wr = Rp ? 1.f : 0.5f;
  // row dv, channels ch .. ch + 4*NQ - 1 (zero past d); loads before arithmetic
  auto rowvals = [&](int dv, int ch, float4* o, auto nq) {
    constexpr int NQ = decltype(nq)::value;
    const size_t i = (size_t)(dv < D ? dv : 0) * D + ch;
    float4 f[NQ], r[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      f[j] = *reinterpret_cast<const float4*>(Fs + i + 4 * j);
      r[j] = *reinterpret_cast<const float4*>(Rs + i + 4 * j);
    }
    const float z = dv < D ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int c = ch + 4 * j;
      o[j] = make_float4(z * (wf * f[j].x * dfw[c] + wr * r[j].x * drv[c]),
                         z * (wf * f[j].y * dfw[c + 1] + wr * r[j].y * drv[c + 1]),
                         z * (wf * f[j].z * dfw[c + 2] + wr * r[j].z * drv[c + 2]),
                         z * (wf * f[j].w * dfw[c + 3] + wr * r[j].w * drv[c + 3]));
    }
  };

  if constexpr (BF16) {
    constexpr int KS = D / 16;
    constexpr int NF = MT * KS * 64;  // fragments per half (hi or lo)
    uint4* out = static_cast<uint4*>(rstates) + (size_t)blockIdx.x * 2 * NF;
#pragma unroll 2
    for (int f = threadIdx.x; f < NF; f += blockDim.x) {
      const int lane = f % 64, ks = (f / 64) % KS, mt = f / (64 * KS);
      float4 v[2];
      rowvals(dv_of(mt, lane & 31), (D / 2) * (lane >> 5) + 8 * ks, v, std::integral_constant<int, 2>());
      const float x[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 h0, l0, h1, l1;
        split_bf16(x[2 * e], h0, l0);
        split_bf16(x[2 * e + 1], h1, l1);
        hi[e] = __builtin_bit_cast(uint32_t, bf16x2{h0, h1});
        lo[e] = __builtin_bit_cast(uint32_t, bf16x2{l0, l1});
      }
      out[f] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      out[NF + f] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  } else {
    constexpr int KQ = D / 8;  // groups of 4 k-steps (32x32x2: one channel per half per step)
    constexpr int NF = MT * KQ * 64;
    float4* out = static_cast<float4*>(rstates) + (size_t)blockIdx.x * NF;
#pragma unroll 2
    for (int f = threadIdx.x; f < NF; f += blockDim.x) {
      const int lane = f % 64, kq = (f / 64) % KQ, mt = f / (64 * KQ);
      float4 v[1];
      rowvals(dv_of(mt, lane & 31), (D / 2) * (lane >> 5) + 4 * kq, v, std::integral_constant<int, 1>());
      out[f] = v[0];
    }
  }
}

template <int D, bool SPLIT>
hipError_t launch_scan_t(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                         float* s_text, float* fwd, float* rev, float* chunk_m, float* chunk_j, hipStream_t s) {
  constexpr int NV = D >= 32 ? 2 : 1;
  constexpr int threads = 64 * (D / (16 * NV));
  constexpr int NRB = D / (16 * scan_mtiles<SPLIT>());
  const auto xcd_grid = [](int units, int rows) { return (unsigned)((units + 7) / 8 * 8 * rows); };
  const unsigned grid = xcd_grid(p.B * p.H * 2, NRB);
  if (!p.chunked) {
    hipLaunchKernelGGL((scan_rows<D, SPLIT, SCAN_FRAMES>), dim3(grid), dim3(threads), 0, s, stats, pinv, alpha,
                       s_text, fwd, rev, nullptr, nullptr, p.B, p.H, p.T, p.C, p.nc);
    return hipGetLastError();
  }
  const int nch = p.nc > 2 ? p.nc - 2 : 0;
  if (nch > 0) {
    const unsigned cgrid = xcd_grid(p.B * p.H * 2 * nch, 2 * NRB);
    hipLaunchKernelGGL((scan_rows<D, SPLIT, SCAN_COMPOSE>), dim3(cgrid), dim3(threads), 0, s, stats, pinv, alpha,
                       nullptr, nullptr, nullptr, chunk_m, chunk_j, p.B, p.H, p.T, p.C, p.nc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_rows<D, SPLIT, SCAN_CHUNKS>), dim3(grid), dim3(threads), 0, s, stats, pinv, alpha,
                     s_text, fwd, rev, chunk_m, chunk_j, p.B, p.H, p.T, p.C, p.nc);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_scan_mode(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                            float* s_text, float* fwd, float* rev, float* chunk_m, float* chunk_j, hipStream_t s) {
  constexpr int NV = D >= 32 ? 2 : 1;
  constexpr int threads = 64 * (D / (16 * NV));
  const auto go = [&](auto split) {
    constexpr bool SPLIT = decltype(split)::value;
    constexpr int NRB = D / (16 * scan_mtiles<SPLIT>());
    const unsigned grid = (unsigned)((p.B * p.H * 2 + 7) / 8 * 8 * NRB);
    hipLaunchKernelGGL((scan_rows<D, SPLIT, MODE>), dim3(grid), dim3(threads), 0, s, stats, pinv, alpha, s_text,
                       fwd, rev, chunk_m, chunk_j, p.B, p.H, p.T, p.C, p.nc);
    return hipGetLastError();
  };
  if constexpr (D >= 32) {
    if (pinv_split(p)) return go(std::true_type());
  }
  return go(std::false_type());
}

template <int D>
hipError_t launch_scan_d(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                         float* s_text, float* fwd, float* rev, float* chunk_m, float* chunk_j, hipStream_t s) {
  if constexpr (D >= 32) {
    if (pinv_split(p)) return launch_scan_t<D, true>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
  }
  return launch_scan_t<D, false>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
}

template <int D>
hipError_t launch_gather_d(const Problem& p, const float* s_text, const float* fwd,
                           const float* rev, const float* alpha, void* rstates, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.H * (p.nc + 1));
  if (p.bf16)
    hipLaunchKernelGGL((gather_states<D, true>), dim3(grid), dim3(256), 0, s, s_text, fwd, rev, alpha, rstates,
                       p.nc, p.T, p.H, p.C, p.bridge ? 1 : 0);
  else
    hipLaunchKernelGGL((gather_states<D, false>), dim3(grid), dim3(256), 0, s, s_text, fwd, rev, alpha, rstates,
                       p.nc, p.T, p.H, p.C, p.bridge ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

size_t readout_slot_bytes(const Problem& p) {
  const int DP = p.D < 32 ? 32 : p.D;
  const int MT = DP / 32;
  if (p.bf16) return (size_t)2 * MT * (p.D / 16) * 64 * 16;
  return (size_t)MT * (p.D / 8) * 64 * 16;
}

hipError_t launch_scan_states(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                              float* states_f, float* states_r, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_scan_mode<16, SCAN_STATES>(p, stats, pinv, alpha, nullptr, states_f, states_r, nullptr, nullptr, s);
    case 32: return launch_scan_mode<32, SCAN_STATES>(p, stats, pinv, alpha, nullptr, states_f, states_r, nullptr, nullptr, s);
    case 64: return launch_scan_mode<64, SCAN_STATES>(p, stats, pinv, alpha, nullptr, states_f, states_r, nullptr, nullptr, s);
    case 128: return launch_scan_mode<128, SCAN_STATES>(p, stats, pinv, alpha, nullptr, states_f, states_r, nullptr, nullptr, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_adjoint(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                               const float* d_fwd, const float* d_rev, float* lam_f, float* lam_r,
                               float* lam_final, hipStream_t s) {
  float* df = const_cast<float*>(d_fwd);  // read only in this mode
  float* dr = const_cast<float*>(d_rev);
  switch (p.D) {
    case 16: return launch_scan_mode<16, SCAN_ADJOINT>(p, stats, pinv, alpha, lam_final, df, dr, lam_f, lam_r, s);
    case 32: return launch_scan_mode<32, SCAN_ADJOINT>(p, stats, pinv, alpha, lam_final, df, dr, lam_f, lam_r, s);
    case 64: return launch_scan_mode<64, SCAN_ADJOINT>(p, stats, pinv, alpha, lam_final, df, dr, lam_f, lam_r, s);
    case 128: return launch_scan_mode<128, SCAN_ADJOINT>(p, stats, pinv, alpha, lam_final, df, dr, lam_f, lam_r, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                       float* s_text, float* fwd, float* rev, float* chunk_m, float* chunk_j, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_scan_d<16>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
    case 32: return launch_scan_d<32>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
    case 64: return launch_scan_d<64>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
    case 128: return launch_scan_d<128>(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gather(const Problem& p, const float* s_text, const float* fwd, const float* rev,
                         const float* alpha, void* rstates, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_gather_d<16>(p, s_text, fwd, rev, alpha, rstates, s);
    case 32: return launch_gather_d<32>(p, s_text, fwd, rev, alpha, rstates, s);
    case 64: return launch_gather_d<64>(p, s_text, fwd, rev, alpha, rstates, s);
    case 128: return launch_gather_d<128>(p, s_text, fwd, rev, alpha, rstates, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vda
