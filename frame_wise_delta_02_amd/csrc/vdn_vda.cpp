// Host side of the C ABI: descriptor validation, workspace layout and the launch
// sequence of the VDA forward pass on the caller's stream.
#include <math.h>
#include <algorithm>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include <cmath>

#include "vda_internal.h"
#include "vdn_vda.h"

namespace vda {

// Workspace of vdn_vda_forward_noalloc, for callers that cannot allocate: one
// array per GPU, created when the library's code object is loaded on that GPU
// and held until the process ends.  Host code never passes `scratch` itself to
// a kernel (on the host the name is a stand-in, not the device address): the
// address each GPU gives for it is looked up once per device and kept.
__device__ __align__(256) uint8_t scratch[VDN_VDA_NOALLOC_MAX_WORKSPACE];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr size_t kAlign = 256;
// without a scan flag, (batch, head) pairs up to which the chunk-composed scan
// is chosen: at d = 128, 60 frames, chunks of 5 on MI355X the frame scan takes
// 74-82 us from 4 to 24 pairs and the chunk-composed one 47, 65, 81 and 97 us
// at 4, 8, 12 and 16 pairs, so the two cross near 11
constexpr size_t kChunkedScanMaxHeads = 10;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A byte range [p, p + n) of a caller's buffer; NULL or empty ranges overlap nothing.
struct Span {
  const void* p;
  size_t n;
};
bool overlaps(const Span& a, const Span& b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Per-call stage events (vdn_vda_forward_timed): events[i] is recorded after
// stage i, events[0] before the first kernel; NULL records nothing.
struct Marks {
  hipEvent_t* ev;
  hipError_t operator()(int i, hipStream_t s) const { return ev ? hipEventRecord(ev[i], s) : hipSuccess; }
};

// Bytes of the [B, T, U, H, d] and related tensors of a problem.
struct Sizes {
  size_t x, beta, alpha, text, beta_text, weight;
};
Sizes sizes_of(const vdn_vda_desc* d) {
  const size_t esz = d->dtype == VDN_BF16 ? 2 : 4;
  const size_t tok = (size_t)d->B * d->T * d->grid_h * d->grid_w * d->H;
  const size_t ttok = (size_t)d->B * d->n_text * d->H;
  return Sizes{tok * d->d_v * esz, tok * esz, (size_t)d->B * d->T * d->H * d->d_k * 4, ttok * d->d_v * esz,
               ttok * esz, (size_t)d->d_v * 4};
}

// True if any written range overlaps a read range or another written range.
bool any_overlap(const Span* outs, size_t n_out, const Span* ins, size_t n_in) {
  for (size_t a = 0; a < n_out; ++a) {
    for (size_t b = 0; b < n_in; ++b)
      if (overlaps(outs[a], ins[b])) return true;
    for (size_t b = a + 1; b < n_out; ++b)
      if (overlaps(outs[a], outs[b])) return true;
  }
  return false;
}

// The built head width a caller's width runs at: 16, 32, 64 or 128.
int padded_width(int d) { return d <= 16 ? 16 : d <= 32 ? 32 : d <= 64 ? 64 : 128; }

vdn_status check(const vdn_vda_desc* d) {
  if (!d) return VDN_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->grid_h < 1 || d->grid_w < 1) return VDN_ERR_INVALID_ARG;
  if (d->d_k < 1 || d->d_v < 1 || d->d_k > 128 || d->d_v > 128) return VDN_ERR_INVALID_ARG;
  if (d->d_k % 16 || d->d_v % 16) return VDN_ERR_INVALID_ARG;
  if (d->n_text < 0 || d->chunk < 1) return VDN_ERR_INVALID_ARG;
  if (d->dtype != VDN_F32 && d->dtype != VDN_BF16) return VDN_ERR_INVALID_ARG;
  if (d->flags & ~(uint32_t)(VDN_VDA_EPILOGUE | VDN_VDA_DEBUG_KEEP | VDN_VDA_DECAY_BRIDGE |
                             VDN_VDA_QUERY_L2 | VDN_VDA_SCAN_FRAMES | VDN_VDA_SCAN_CHUNKS))
    return VDN_ERR_INVALID_ARG;
  if ((d->flags & VDN_VDA_SCAN_FRAMES) && (d->flags & VDN_VDA_SCAN_CHUNKS)) return VDN_ERR_INVALID_ARG;
  if (!(d->l2_eps > 0.f) || !isfinite(d->l2_eps)) return VDN_ERR_INVALID_ARG;
  if (!(d->rms_eps > 0.f) || !isfinite(d->rms_eps)) return VDN_ERR_INVALID_ARG;
  // sizes must stay well inside 64-bit element counts and 32-bit grid dimensions
  const double U = (double)d->grid_h * d->grid_w;
  const double elems = (double)d->B * d->T * U * d->H * d->d_v;
  if (U > 2147483647.0 || elems > 9.0e15) return VDN_ERR_INVALID_ARG;
  // the kernels run at the built width D >= d (the offset limits below are theirs)
  const double D = padded_width(d->d_k);
  if ((double)d->B * d->T * d->H * d->grid_h > 4294967295.0) return VDN_ERR_INVALID_ARG;
  if ((double)d->B * d->n_text * d->H > 9.0e15) return VDN_ERR_INVALID_ARG;
  // the scan launches: up to 16 row blocks per (batch, head, direction, chunk),
  // the units rounded up to a multiple of 8
  if (((double)d->B * d->H * 2 * ((d->T + d->chunk - 1) / d->chunk) + 8) * 16 > 2147483647.0)
    return VDN_ERR_INVALID_ARG;
  // the scan's chunk records of one head must stay below 2^31 bytes: steps that
  // record nothing store at offset 2^31, past that buffer
  if ((double)((d->T + d->chunk - 1) / d->chunk) * D * D * 4.0 >= 2147483648.0)
    return VDN_ERR_INVALID_ARG;
  // a frame's (or the text's) token rows, plus a tile's overhang, are addressed
  // with 32-bit byte offsets
  if (((double)d->grid_h * d->grid_w + 64.0) * d->H * D * 4.0 > 4294967295.0) return VDN_ERR_INVALID_ARG;
  if (((double)d->n_text + 64.0) * d->H * D * 4.0 > 4294967295.0) return VDN_ERR_INVALID_ARG;
  // the statistics kernel's register prefetch reads a few tiles of 64 tokens
  // past a frame's last token (zero through the buffer range check); with 640
  // tokens of margin its 32-bit offsets cannot wrap back into the frame
  if (((double)d->grid_h * d->grid_w + 640.0) * d->H * D * 2.0 > 4294967295.0) return VDN_ERR_INVALID_ARG;
  if (((double)d->n_text + 640.0) * d->H * D * 2.0 > 4294967295.0) return VDN_ERR_INVALID_ARG;
  if (d->d_k != d->d_v) return VDN_ERR_UNSUPPORTED;
  return VDN_OK;
}

Problem problem(const vdn_vda_desc* d) {
  Problem p;
  p.B = d->B;
  p.H = d->H;
  p.T = d->T;
  p.U = d->grid_h * d->grid_w;
  p.D = padded_width(d->d_k);
  p.Du = d->d_k;
  p.L = d->n_text;
  p.C = d->chunk;
  p.nc = (d->T + d->chunk - 1) / d->chunk;
  p.bf16 = d->dtype == VDN_BF16;
  p.epilogue = (d->flags & VDN_VDA_EPILOGUE) != 0;
  p.bridge = (d->flags & VDN_VDA_DECAY_BRIDGE) != 0;
  p.qnorm = (d->flags & VDN_VDA_QUERY_L2) != 0;
  // The frame scan takes one workgroup per 32 (bfloat16) or 16 (float32) state
  // rows of each (batch, head, direction) and its critical path is one serial
  // step per frame; the chunk-composed scan adds a fully parallel composition
  // pass but takes one serial step per chunk.  It pays where the frame scan
  // leaves most compute units idle.
  if (d->flags & VDN_VDA_SCAN_CHUNKS)
    p.chunked = true;
  else if (d->flags & VDN_VDA_SCAN_FRAMES)
    p.chunked = false;
  else
    p.chunked = p.nc >= 3 && (size_t)p.B * p.H <= kChunkedScanMaxHeads;
  p.l2_eps = d->l2_eps;
  p.rms_eps = d->rms_eps;
  return p;
}

}  // namespace

Layout make_layout(const Problem& p) {
  const size_t heads = (size_t)p.B * p.H;
  const size_t dd = (size_t)p.D * p.D * sizeof(float);
  Layout l;
  size_t o = 0;
  l.stats = o;
  o = up(o + heads * (p.T + 1) * 2 * dd);
  l.pinv = o;
  o = up(o + heads * (p.T + 1) * dd);
  l.s_text = o;
  o = up(o + heads * dd);
  l.fwd = o;
  o = up(o + heads * p.nc * dd);
  l.rev = o;
  o = up(o + heads * p.nc * dd);
  l.rstates = o;
  o = up(o + heads * (p.nc + 1) * readout_slot_bytes(p));
  l.chunk_m = o;
  o = up(o + heads * 2 * p.nc * dd);
  l.chunk_j = o;
  o = up(o + heads * 2 * p.nc * dd);
  // the zero-padded copies, at widths between the built ones only
  const bool pad = p.Du != p.D;
  const size_t esz = p.bf16 ? 2 : 4;
  const size_t xb = pad ? (size_t)p.B * p.T * p.U * p.H * p.D * esz : 0;
  const size_t tb = pad ? (size_t)p.B * p.L * p.H * p.D * esz : 0;
  auto take = [&](size_t& field, size_t bytes) {
    field = o;
    o = up(o + bytes);
  };
  take(l.pad_q, xb);
  take(l.pad_k, xb);
  take(l.pad_v, xb);
  take(l.pad_gate, p.epilogue ? xb : 0);
  take(l.pad_out, xb);
  take(l.pad_alpha, pad ? (size_t)p.B * p.T * p.H * p.D * 4 : 0);
  take(l.pad_k_text, tb);
  take(l.pad_v_text, tb);
  take(l.pad_gain, pad && p.epilogue ? (size_t)p.D * 4 : 0);
  l.total = o;
  return l;
}

// Workspace of the backward pass's first stage.
struct BwdLayout {
  size_t rstates_t, dout, dsq;                                    // first stage
  size_t dF, dR, dST, lam_f, lam_r, dA, dB;                       // second stage (documented)
  size_t states_f, states_r, lam_final, p32, M, dPinv, tmp;       // second stage (internal)
  size_t gmats;                                                   // third stage (internal)
  size_t gain;                                                    // first stage (internal)
  // widths between the built ones: the zero-padded copies of the stages'
  // inputs and outputs (the forward's workspace holds q, gate, alpha, the gain)
  size_t pad_dy, pad_dq, pad_dgate, pad_dalpha, pad_k, pad_v, pad_dk, pad_dv, pad_k_text, pad_v_text,
      pad_dk_text, pad_dv_text;
  size_t total;
};
BwdLayout make_bwd_layout(const Problem& p) {
  const size_t heads = (size_t)p.B * p.H;
  const size_t dd = (size_t)p.D * p.D * 4;
  BwdLayout l;
  size_t o = 0;
  auto take = [&](size_t& field, size_t bytes) {
    field = o;
    o = up(o + bytes);
  };
  take(l.rstates_t, heads * (p.nc + 1) * readout_slot_bytes(p));
  const size_t esz = p.bf16 ? 2 : 4;
  take(l.dout, (size_t)p.B * p.T * p.U * p.H * p.D * esz);
  take(l.dsq, heads * p.T * dd);
  take(l.dF, heads * p.nc * dd);
  take(l.dR, heads * p.nc * dd);
  take(l.dST, heads * dd);
  take(l.lam_f, heads * (p.T + 1) * dd);
  take(l.lam_r, heads * (p.T + 1) * dd);
  take(l.dA, heads * (p.T + 1) * dd);
  take(l.dB, heads * (p.T + 1) * dd);
  take(l.states_f, heads * (p.T + 2) * dd);
  take(l.states_r, heads * (p.T + 2) * dd);
  take(l.lam_final, heads * 2 * dd);
  take(l.p32, heads * (p.T + 1) * dd);
  take(l.M, heads * (p.T + 1) * dd);
  take(l.dPinv, heads * (p.T + 1) * dd);
  take(l.tmp, heads * (p.T + 1) * dd);
  // five bfloat16 operand planes per slot (G hi, lo; dB hi, lo; dB^T hi), the
  // rows padded to 32 at d = 16
  take(l.gmats, heads * (p.T + 1) * 5 * (size_t)std::max(p.D, 32) * p.D * 2);
  // the gain gradient's sums per (batch, frame, head), float32 [B T H][d]
  take(l.gain, (size_t)p.B * p.T * p.H * p.D * 4);
  const bool pad = p.Du != p.D;
  const size_t xb = pad ? (size_t)p.B * p.T * p.U * p.H * p.D * esz : 0;
  const size_t tb = pad ? (size_t)p.B * p.L * p.H * p.D * esz : 0;
  for (size_t* f : {&l.pad_dy, &l.pad_dq, &l.pad_dgate}) take(*f, xb);
  take(l.pad_dalpha, pad ? (size_t)p.B * p.T * p.H * p.D * 4 : 0);
  for (size_t* f : {&l.pad_k, &l.pad_v, &l.pad_dk, &l.pad_dv}) take(*f, xb);
  for (size_t* f : {&l.pad_k_text, &l.pad_v_text, &l.pad_dk_text, &l.pad_dv_text}) take(*f, tb);
  l.total = o;
  return l;
}

// The adjacent maps are plain products over the H d channels of a token, with
// no tiling of the head width: they run at the caller's width, whatever it is.
Problem proj_problem(const vdn_vda_desc* d) {
  Problem p = problem(d);
  p.D = p.Du;
  return p;
}

// The adjacent maps' own checks: bfloat16, a model width that 16-byte rows and
// 32-bit panel offsets allow.
vdn_status check_proj(const vdn_vda_desc* d, int32_t d_model) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  if (d->dtype != VDN_BF16) return VDN_ERR_UNSUPPORTED;
  if (d_model < 8 || d_model % 8) return VDN_ERR_INVALID_ARG;
  const double rows = 256.0;  // one tile's rows of either operand
  if (rows * d_model * 2.0 >= 2147483648.0 || rows * d->H * d->d_v * 2.0 >= 2147483648.0) return VDN_ERR_INVALID_ARG;
  if ((double)d->B * d->T * d->grid_h * d->grid_w * std::max<double>(d_model, (double)d->H * d->d_v) > 9.0e15)
    return VDN_ERR_INVALID_ARG;
  // the GEMMs' row count B T U and their grids are 32-bit
  if ((double)d->B * d->T * d->grid_h * d->grid_w >= 2147483648.0) return VDN_ERR_INVALID_ARG;
  return VDN_OK;
}

}  // namespace vda

namespace vda {
namespace {

// Every check of the forward pass's arguments; with have_ws false the
// workspace is left out (the no-allocation entry point finds its own later).
vdn_status forward_args(const vdn_vda_desc* d, const void* q, const void* k, const void* v, const float* alpha,
                        const void* beta, const void* k_text, const void* v_text, const void* beta_text,
                        const void* gate, const float* rms_weight, const void* out, const void* workspace,
                        size_t workspace_bytes, bool have_ws) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  const bool epi = (d->flags & VDN_VDA_EPILOGUE) != 0;
  if (!q || !k || !v || !alpha || !beta || !out) return VDN_ERR_INVALID_ARG;
  if (d->n_text > 0 && (!k_text || !v_text || !beta_text)) return VDN_ERR_INVALID_ARG;
  if (epi && !gate) return VDN_ERR_INVALID_ARG;
  const Layout l = make_layout(problem(d));
  if (have_ws && (!workspace || workspace_bytes < l.total)) return VDN_ERR_WORKSPACE;
  const void* need16[] = {q, k, v, alpha, out, epi ? gate : nullptr,
                          d->n_text > 0 ? k_text : nullptr, d->n_text > 0 ? v_text : nullptr};
  for (const void* ptr : need16)
    if (ptr && !aligned(ptr, 16)) return VDN_ERR_ALIGNMENT;
  const size_t esz = d->dtype == VDN_BF16 ? 2 : 4;
  if (!aligned(beta, esz) || (d->n_text > 0 && !aligned(beta_text, esz)) ||
      (rms_weight && !aligned(rms_weight, 4)))
    return VDN_ERR_ALIGNMENT;
  if (have_ws && !aligned(workspace, kAlign)) return VDN_ERR_ALIGNMENT;
  // the output and the workspace are written while the inputs are read
  const Sizes z = sizes_of(d);
  const bool text = d->n_text > 0;
  const Span ins[] = {{q, z.x}, {k, z.x}, {v, z.x}, {alpha, z.alpha}, {beta, z.beta},
                      {text ? k_text : nullptr, z.text}, {text ? v_text : nullptr, z.text},
                      {text ? beta_text : nullptr, z.beta_text}, {epi ? gate : nullptr, z.x},
                      {rms_weight, z.weight}};
  const Span outs[] = {{out, z.x}, {have_ws ? workspace : nullptr, l.total}};
  if (any_overlap(outs, 2, ins, 10)) return VDN_ERR_INVALID_ARG;
  return VDN_OK;
}

// The forward pass behind vdn_vda_forward, vdn_vda_forward_timed and
// vdn_vda_forward_noalloc.
vdn_status forward_impl(const vdn_vda_desc* d, const void* q, const void* k, const void* v, const float* alpha,
                        const void* beta, const void* k_text, const void* v_text, const void* beta_text,
                        const void* gate, const float* rms_weight, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, const Marks& mark) {
  const vdn_status st = forward_args(d, q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out,
                                     workspace, workspace_bytes, true);
  if (st != VDN_OK) return st;
  const Problem p = problem(d);
  const Layout l = make_layout(p);

  char* ws = static_cast<char*>(workspace);
  hipError_t e = mark(0, stream);
  // a width between the built ones: the kernels run at p.D on zero-padded
  // copies (vda_pad.hip), the epilogue with eps d / D and the gain scaled by
  // sqrt(d / D), and the output's first d channels are copied back
  const bool pad = p.Du != p.D;
  Problem pr = p;  // the readout's problem
  void* out_k = out;
  if (pad) {
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t rows = (size_t)p.B * p.T * p.U * p.H, trows = (size_t)p.B * p.L * p.H;
    const size_t ub = (size_t)p.Du * esz, pb = (size_t)p.D * esz;
    auto copy = [&](const void*& src, size_t off, size_t n, size_t srow, size_t drow) {
      if (e == hipSuccess) e = launch_copy_rows(src, srow, ws + off, drow, srow, n, stream);
      src = ws + off;
    };
    copy(q, l.pad_q, rows, ub, pb);
    copy(k, l.pad_k, rows, ub, pb);
    copy(v, l.pad_v, rows, ub, pb);
    if (p.epilogue) copy(gate, l.pad_gate, rows, ub, pb);
    const void* a = alpha;
    copy(a, l.pad_alpha, (size_t)p.B * p.T * p.H, (size_t)p.Du * 4, (size_t)p.D * 4);
    alpha = static_cast<const float*>(a);
    if (p.L > 0) {
      copy(k_text, l.pad_k_text, trows, ub, pb);
      copy(v_text, l.pad_v_text, trows, ub, pb);
    }
    if (p.epilogue) {
      float* g = reinterpret_cast<float*>(ws + l.pad_gain);
      if (e == hipSuccess) e = launch_pad_gain(rms_weight, g, p.Du, p.D, stream);
      rms_weight = g;
      pr.rms_eps = p.rms_eps * (float)p.Du / (float)p.D;
    }
    out_k = ws + l.pad_out;
  }
  float* stats = reinterpret_cast<float*>(ws + l.stats);
  float* pinv = reinterpret_cast<float*>(ws + l.pinv);
  float* s_text = reinterpret_cast<float*>(ws + l.s_text);
  float* fwd = reinterpret_cast<float*>(ws + l.fwd);
  float* rev = reinterpret_cast<float*>(ws + l.rev);
  void* rstates = ws + l.rstates;
  float* chunk_m = reinterpret_cast<float*>(ws + l.chunk_m);
  float* chunk_j = reinterpret_cast<float*>(ws + l.chunk_j);

  const int n_video = p.T > 2 ? p.T - 2 : 0;
  // frame statistics of frames 1..T-2 (anchors are never absorbed) and of the
  // text frame (slot T) in one launch: the short text blocks run last, in the
  // final round of the video blocks
  // With no text tokens the text frame's units read nothing (their buffer
  // ranges are empty) and leave A = B = 0; the video tensors stand in for the
  // absent text pointers so that no address is formed from a null pointer.
  const bool text = p.L > 0;
  const GramPart parts[2] = {{k, v, beta, p.T, p.U, 1, n_video, 0},
                             {text ? k_text : k, text ? v_text : v, text ? beta_text : beta, 1, p.L, 0, 1, p.T}};
  if (e == hipSuccess) e = launch_gram(p, parts, 2, stats, stream);
  if (e == hipSuccess) e = mark(1, stream);
  if (e == hipSuccess) e = launch_solve(p, stats, pinv, stream);
  if (e == hipSuccess) e = mark(2, stream);
  if (e == hipSuccess) e = launch_scan(p, stats, pinv, alpha, s_text, fwd, rev, chunk_m, chunk_j, stream);
  if (e == hipSuccess) e = mark(3, stream);
  if (e == hipSuccess) e = launch_gather(p, s_text, fwd, rev, alpha, rstates, stream);
  if (e == hipSuccess) e = mark(4, stream);
  if (e == hipSuccess) e = launch_readout(pr, q, gate, rms_weight, rstates, out_k, stream);
  if (pad && e == hipSuccess) {
    const size_t esz = p.bf16 ? 2 : 4;
    e = launch_copy_rows(out_k, (size_t)p.D * esz, out, (size_t)p.Du * esz, (size_t)p.Du * esz,
                         (size_t)p.B * p.T * p.U * p.H, stream);
  }
  if (e == hipSuccess) e = mark(5, stream);
  return e == hipSuccess ? VDN_OK : VDN_ERR_HIP;
}

}  // namespace
}  // namespace vda

using namespace vda;

extern "C" {

vdn_status vdn_vda_validate(const vdn_vda_desc* d) { return check(d); }

size_t vdn_vda_workspace_bytes(const vdn_vda_desc* d) {
  if (check(d) != VDN_OK) return 0;
  return make_layout(problem(d)).total;
}

vdn_status vdn_vda_workspace_layout(const vdn_vda_desc* d, vdn_vda_layout* out) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  if (!out) return VDN_ERR_INVALID_ARG;
  const Layout l = make_layout(problem(d));
  out->stats = l.stats;
  out->pinv = l.pinv;
  out->s_text = l.s_text;
  out->fwd = l.fwd;
  out->rev = l.rev;
  out->readout_states = l.rstates;
  out->chunk_m = l.chunk_m;
  out->chunk_j = l.chunk_j;
  out->total = l.total;
  return VDN_OK;
}

vdn_status vdn_vda_prepare(const vdn_vda_desc* d, const void* q, const void* k, const void* v,
                           const float* wk_s, const float* wk_t, const float* wv_s,
                           const float* wv_t, void* q_hat, void* k_hat, void* v_hat,
                           hipStream_t stream) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  const Problem p = problem(d);
  // under VDN_VDA_QUERY_L2 the query is normalised by the forward pass instead
  if (p.qnorm) q = q_hat = nullptr;
  const void* ptrs[] = {k, v, wk_s, wk_t, wv_s, wv_t, k_hat, v_hat, q, q_hat};
  const int nreq = p.qnorm ? 8 : 10;
  for (int i = 0; i < nreq; ++i)
    if (!ptrs[i]) return VDN_ERR_INVALID_ARG;
  for (int i = 0; i < nreq; ++i)
    if (!aligned(ptrs[i], 16)) return VDN_ERR_ALIGNMENT;
  // outputs are written while inputs are still read: no byte may be shared
  const Sizes z = sizes_of(d);
  const size_t ws_ = (size_t)p.H * p.Du * 25 * 4, wt_ = (size_t)p.H * p.Du * 5 * 4;
  const Span ins[] = {{k, z.x}, {v, z.x}, {q, z.x}, {wk_s, ws_}, {wk_t, wt_}, {wv_s, ws_}, {wv_t, wt_}};
  const Span outs[] = {{k_hat, z.x}, {v_hat, z.x}, {q_hat, z.x}};
  if (any_overlap(outs, 3, ins, 7)) return VDN_ERR_INVALID_ARG;
  if (launch_prep(p, d->grid_h, d->grid_w, q, k, v, wk_s, wk_t, wv_s, wv_t, q_hat, k_hat, v_hat,
                  stream) != hipSuccess)
    return VDN_ERR_HIP;
  return VDN_OK;
}

vdn_status vdn_vda_forward(const vdn_vda_desc* d, const void* q, const void* k, const void* v,
                           const float* alpha, const void* beta, const void* k_text,
                           const void* v_text, const void* beta_text, const void* gate,
                           const float* rms_weight, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(d, q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, workspace,
                      workspace_bytes, stream, Marks{nullptr});
}

vdn_status vdn_vda_forward_timed(const vdn_vda_desc* d, const void* q, const void* k, const void* v,
                                 const float* alpha, const void* beta, const void* k_text,
                                 const void* v_text, const void* beta_text, const void* gate,
                                 const float* rms_weight, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                 int32_t n_events) {
  if (!events || n_events < VDN_VDA_STAGES + 1) return VDN_ERR_INVALID_ARG;
  for (int i = 0; i <= VDN_VDA_STAGES; ++i)
    if (!events[i]) return VDN_ERR_INVALID_ARG;
  return forward_impl(d, q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, workspace,
                      workspace_bytes, stream, Marks{events});
}

vdn_status vdn_vda_forward_noalloc(const vdn_vda_desc* d, const void* q, const void* k, const void* v,
                                   const float* alpha, const void* beta, const void* k_text,
                                   const void* v_text, const void* beta_text, const void* gate,
                                   const float* rms_weight, void* out, hipStream_t stream) {
  // every argument check first: nothing touches the GPU for a call that fails one
  const vdn_status st = forward_args(d, q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out,
                                     nullptr, 0, false);
  if (st != VDN_OK) return st;
  const size_t need = make_layout(problem(d)).total;
  if (need > (size_t)VDN_VDA_NOALLOC_MAX_WORKSPACE) return VDN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return VDN_ERR_HIP;
  return forward_impl(d, q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, ws,
                      (size_t)VDN_VDA_NOALLOC_MAX_WORKSPACE, stream, Marks{nullptr});
}

size_t vdn_vda_backward_workspace_bytes(const vdn_vda_desc* d) {
  if (check(d) != VDN_OK) return 0;
  return make_bwd_layout(problem(d)).total;
}

vdn_status vdn_vda_backward_workspace_layout(const vdn_vda_desc* d, vdn_vda_backward_layout* out) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  if (!out) return VDN_ERR_INVALID_ARG;
  const BwdLayout l = make_bwd_layout(problem(d));
  out->readout_states_t = l.rstates_t;
  out->d_out = l.dout;
  out->d_state_q = l.dsq;
  out->d_record_f = l.dF;
  out->d_record_r = l.dR;
  out->d_text_q = l.dST;
  out->lam_f = l.lam_f;
  out->lam_r = l.lam_r;
  out->d_a = l.dA;
  out->d_b = l.dB;
  out->total = l.total;
  return VDN_OK;
}

vdn_status vdn_vda_backward_readout(const vdn_vda_desc* d, const void* q, const void* gate,
                                    const float* rms_weight, const float* alpha, const void* dy,
                                    const void* fwd_workspace, size_t fwd_workspace_bytes, void* dq,
                                    void* dgate, float* d_rms_weight, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  const bool epi = (d->flags & VDN_VDA_EPILOGUE) != 0;
  // the raw query's gradient is formed with the epilogue's backward only
  if ((d->flags & VDN_VDA_QUERY_L2) && !epi) return VDN_ERR_UNSUPPORTED;
  if (!q || !alpha || !dy || !dq || !fwd_workspace) return VDN_ERR_INVALID_ARG;
  if (epi && (!gate || !dgate)) return VDN_ERR_INVALID_ARG;
  if (d_rms_weight && !epi) return VDN_ERR_INVALID_ARG;  // no gain without the epilogue
  const Problem p = problem(d);
  const Layout fl = make_layout(p);
  const BwdLayout bl = make_bwd_layout(p);
  if (fwd_workspace_bytes < fl.total) return VDN_ERR_WORKSPACE;
  if (!workspace || workspace_bytes < bl.total) return VDN_ERR_WORKSPACE;
  const void* need16[] = {q, dy, dq, alpha, epi ? gate : nullptr, epi ? dgate : nullptr};
  for (const void* ptr : need16)
    if (ptr && !aligned(ptr, 16)) return VDN_ERR_ALIGNMENT;
  if (rms_weight && !aligned(rms_weight, 4)) return VDN_ERR_ALIGNMENT;
  if (d_rms_weight && !aligned(d_rms_weight, 4)) return VDN_ERR_ALIGNMENT;
  if (!aligned(workspace, kAlign) || !aligned(fwd_workspace, kAlign)) return VDN_ERR_ALIGNMENT;
  {
    const Sizes z = sizes_of(d);
    const Span ins[] = {{q, z.x}, {epi ? gate : nullptr, z.x}, {rms_weight, z.weight}, {alpha, z.alpha},
                        {dy, z.x}, {fwd_workspace, fl.total}};
    const Span outs[] = {{dq, z.x}, {epi ? dgate : nullptr, z.x}, {workspace, bl.total}, {d_rms_weight, z.weight}};
    if (any_overlap(outs, 4, ins, 6)) return VDN_ERR_INVALID_ARG;
  }
  const char* fw = static_cast<const char*>(fwd_workspace);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = hipSuccess;
  // a width between the built ones: the forward's padded q, gate, alpha and
  // gain, dy padded here, dq and dgate padded then copied back; the gain's
  // gradient is sqrt(d / D) times the padded gain's (gamma' = gamma sqrt(d / D))
  Problem pr = p;
  void *dq_k = dq, *dgate_k = dgate;
  float gscale = 1.f;
  const size_t esz = p.bf16 ? 2 : 4;
  const size_t rows = (size_t)p.B * p.T * p.U * p.H, ub = (size_t)p.Du * esz, pb = (size_t)p.D * esz;
  if (p.Du != p.D) {
    q = fw + fl.pad_q;
    alpha = reinterpret_cast<const float*>(fw + fl.pad_alpha);
    if (epi) {
      gate = fw + fl.pad_gate;
      rms_weight = reinterpret_cast<const float*>(fw + fl.pad_gain);
      pr.rms_eps = p.rms_eps * (float)p.Du / (float)p.D;
      gscale = std::sqrt((float)p.Du / (float)p.D);
    }
    e = launch_copy_rows(dy, ub, ws + bl.pad_dy, pb, ub, rows, stream);
    dy = ws + bl.pad_dy;
    dq_k = ws + bl.pad_dq;
    dgate_k = epi ? ws + bl.pad_dgate : nullptr;
  }
  if (e == hipSuccess)
    e = launch_backward_readout(
        pr, q, gate, rms_weight, dy, fw + fl.rstates, reinterpret_cast<const float*>(fw + fl.s_text),
        reinterpret_cast<const float*>(fw + fl.fwd), reinterpret_cast<const float*>(fw + fl.rev), alpha,
        ws + bl.rstates_t, ws + bl.dout, dq_k, dgate_k, reinterpret_cast<float*>(ws + bl.dsq),
        reinterpret_cast<float*>(ws + bl.gain), d_rms_weight, p.Du, gscale, stream);
  if (p.Du != p.D && e == hipSuccess) {
    e = launch_copy_rows(dq_k, pb, dq, ub, ub, rows, stream);
    if (epi && e == hipSuccess) e = launch_copy_rows(dgate_k, pb, dgate, ub, ub, rows, stream);
  }
  return e == hipSuccess ? VDN_OK : VDN_ERR_HIP;
}

vdn_status vdn_vda_backward_scan(const vdn_vda_desc* d, const float* alpha, const void* fwd_workspace,
                                 size_t fwd_workspace_bytes, float* dalpha, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  if (!alpha || !fwd_workspace || !dalpha) return VDN_ERR_INVALID_ARG;
  const Problem p = problem(d);
  // every frame's state is recorded per head through one buffer descriptor
  if ((double)(d->T + 2) * p.D * p.D * 4.0 >= 2147483648.0) return VDN_ERR_INVALID_ARG;
  const Layout fl = make_layout(p);
  const BwdLayout bl = make_bwd_layout(p);
  if (fwd_workspace_bytes < fl.total) return VDN_ERR_WORKSPACE;
  if (!workspace || workspace_bytes < bl.total) return VDN_ERR_WORKSPACE;
  if (!aligned(alpha, 16) || !aligned(dalpha, 16)) return VDN_ERR_ALIGNMENT;
  if (!aligned(workspace, kAlign) || !aligned(fwd_workspace, kAlign)) return VDN_ERR_ALIGNMENT;
  {
    const Sizes z = sizes_of(d);
    const Span ins[] = {{alpha, z.alpha}, {fwd_workspace, fl.total}};
    const Span outs[] = {{dalpha, z.alpha}, {workspace, bl.total}};
    if (any_overlap(outs, 2, ins, 2)) return VDN_ERR_INVALID_ARG;
  }
  const char* fw = static_cast<const char*>(fwd_workspace);
  char* ws = static_cast<char*>(workspace);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  BwdScanBuffers w;
  w.stats = reinterpret_cast<const float*>(fw + fl.stats);
  w.pinv = reinterpret_cast<const float*>(fw + fl.pinv);
  w.alpha = alpha;
  w.dsq = f(bl.dsq);
  w.dF = f(bl.dF);
  w.dR = f(bl.dR);
  w.dST = f(bl.dST);
  w.states_f = f(bl.states_f);
  w.states_r = f(bl.states_r);
  w.lam_f = f(bl.lam_f);
  w.lam_r = f(bl.lam_r);
  w.lam_final = f(bl.lam_final);
  w.p32 = f(bl.p32);
  w.M = f(bl.M);
  w.dPinv = f(bl.dPinv);
  w.tmp = f(bl.tmp);
  w.dA = f(bl.dA);
  w.dB = f(bl.dB);
  w.dalpha = dalpha;
  w.s_text = reinterpret_cast<const float*>(fw + fl.s_text);
  w.fwd = reinterpret_cast<const float*>(fw + fl.fwd);
  w.rev = reinterpret_cast<const float*>(fw + fl.rev);
  const bool pad = p.Du != p.D;  // the forward's padded alpha, dalpha padded then copied back
  if (pad) {
    w.alpha = reinterpret_cast<const float*>(fw + fl.pad_alpha);
    w.dalpha = f(bl.pad_dalpha);
  }
  hipError_t e = launch_backward_scan(p, w, stream);
  if (pad && e == hipSuccess)
    e = launch_copy_rows(w.dalpha, (size_t)p.D * 4, dalpha, (size_t)p.Du * 4, (size_t)p.Du * 4,
                         (size_t)p.B * p.T * p.H, stream);
  return e == hipSuccess ? VDN_OK : VDN_ERR_HIP;
}

vdn_status vdn_vda_backward_gram(const vdn_vda_desc* d, const void* k, const void* v, const void* beta,
                                 const void* k_text, const void* v_text, const void* beta_text, void* dk,
                                 void* dv, void* dbeta, void* dk_text, void* dv_text, void* dbeta_text,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const vdn_status st = check(d);
  if (st != VDN_OK) return st;
  if (!k || !v || !beta || !dk || !dv || !dbeta) return VDN_ERR_INVALID_ARG;
  const bool text = d->n_text > 0;
  if (text && (!k_text || !v_text || !beta_text || !dk_text || !dv_text || !dbeta_text)) return VDN_ERR_INVALID_ARG;
  const Problem p = problem(d);
  const BwdLayout bl = make_bwd_layout(p);
  if (!workspace || workspace_bytes < bl.total) return VDN_ERR_WORKSPACE;
  const void* need16[] = {k, v, dk, dv, text ? k_text : nullptr, text ? v_text : nullptr,
                          text ? dk_text : nullptr, text ? dv_text : nullptr};
  for (const void* ptr : need16)
    if (ptr && !aligned(ptr, 16)) return VDN_ERR_ALIGNMENT;
  const size_t esz = d->dtype == VDN_BF16 ? 2 : 4;
  const void* need2[] = {beta, dbeta, text ? beta_text : nullptr, text ? dbeta_text : nullptr};
  for (const void* ptr : need2)
    if (ptr && !aligned(ptr, esz)) return VDN_ERR_ALIGNMENT;
  if (!aligned(workspace, kAlign)) return VDN_ERR_ALIGNMENT;
  // the outputs are written while the inputs are still read
  const size_t tok = (size_t)p.B * p.T * p.U * p.H, ttok = (size_t)p.B * p.L * p.H;
  const size_t xb = tok * p.Du * esz, tb = ttok * p.Du * esz;
  const Span ins[] = {{k, xb}, {v, xb}, {beta, tok * esz}, {text ? k_text : nullptr, tb},
                      {text ? v_text : nullptr, tb}, {text ? beta_text : nullptr, ttok * esz},
                      {workspace, workspace_bytes}};
  const Span outs[] = {{dk, xb}, {dv, xb}, {dbeta, tok * esz}, {text ? dk_text : nullptr, tb},
                       {text ? dv_text : nullptr, tb}, {text ? dbeta_text : nullptr, ttok * esz}};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlaps(o, i)) return VDN_ERR_INVALID_ARG;
  for (size_t a = 0; a < 6; ++a)
    for (size_t b = a + 1; b < 6; ++b)
      if (overlaps(outs[a], outs[b])) return VDN_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  BwdGramBuffers w;
  w.dA = reinterpret_cast<const float*>(ws + bl.dA);
  w.dB = reinterpret_cast<const float*>(ws + bl.dB);
  w.mats = ws + bl.gmats;
  w.k = k;
  w.v = v;
  w.beta = beta;
  w.k_text = k_text;
  w.v_text = v_text;
  w.beta_text = beta_text;
  w.dk = dk;
  w.dv = dv;
  w.dbeta = dbeta;
  w.dk_text = dk_text;
  w.dv_text = dv_text;
  w.dbeta_text = dbeta_text;
  // a width between the built ones: k, v (and the text's) padded here, dk, dv
  // padded then copied back (dbeta has no channel axis)
  hipError_t e = hipSuccess;
  const bool pad = p.Du != p.D;
  const size_t ub = (size_t)p.Du * esz, pb = (size_t)p.D * esz;
  if (pad) {
    auto in = [&](const void*& x, size_t off, size_t n) {
      if (e == hipSuccess) e = launch_copy_rows(x, ub, ws + off, pb, ub, n, stream);
      x = ws + off;
    };
    in(w.k, bl.pad_k, tok);
    in(w.v, bl.pad_v, tok);
    w.dk = ws + bl.pad_dk;
    w.dv = ws + bl.pad_dv;
    if (text) {
      in(w.k_text, bl.pad_k_text, ttok);
      in(w.v_text, bl.pad_v_text, ttok);
      w.dk_text = ws + bl.pad_dk_text;
      w.dv_text = ws + bl.pad_dv_text;
    }
  }
  if (e == hipSuccess) e = launch_backward_gram(p, w, stream);
  if (pad) {
    auto out = [&](const void* src, void* dst, size_t n) {
      if (e == hipSuccess) e = launch_copy_rows(src, pb, dst, ub, ub, n, stream);
    };
    out(w.dk, dk, tok);
    out(w.dv, dv, tok);
    if (text) {
      out(w.dk_text, dk_text, ttok);
      out(w.dv_text, dv_text, ttok);
    }
  }
  return e == hipSuccess ? VDN_OK : VDN_ERR_HIP;
}

size_t vdn_vda_gates_workspace_bytes(const vdn_vda_desc* d, int32_t d_model) {
  if (check_proj(d, d_model) != VDN_OK) return 0;
  const Problem p = proj_problem(d);
  const size_t F = (size_t)p.B * p.T;
  return up(F * proj_mean_splits(p) * d_model * 4) + up(F * d_model * 4);
}

vdn_status vdn_vda_gates(const vdn_vda_desc* d, int32_t d_model, const void* x, const void* w_gb,
                         const float* w_alpha, void* gate, void* beta, float* alpha, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  const vdn_status st = check_proj(d, d_model);
  if (st != VDN_OK) return st;
  if (!x || !w_gb || !w_alpha || !gate || !beta || !alpha) return VDN_ERR_INVALID_ARG;
  const Problem p = proj_problem(d);
  const size_t need = vdn_vda_gates_workspace_bytes(d, d_model);
  if (!workspace || workspace_bytes < need) return VDN_ERR_WORKSPACE;
  const void* need16[] = {x, w_gb, w_alpha, gate, alpha};
  for (const void* ptr : need16)
    if (!aligned(ptr, 16)) return VDN_ERR_ALIGNMENT;
  if (!aligned(beta, 2)) return VDN_ERR_ALIGNMENT;
  if (!aligned(workspace, kAlign)) return VDN_ERR_ALIGNMENT;
  const size_t M = (size_t)p.B * p.T * p.U, F = (size_t)p.B * p.T, HD = (size_t)p.H * p.D;
  const Span ins[] = {{x, M * d_model * 2}, {w_gb, (HD + p.H) * d_model * 2}, {w_alpha, HD * d_model * 4},
                      {workspace, workspace_bytes}};
  const Span outs[] = {{gate, M * HD * 2}, {beta, M * p.H * 2}, {alpha, F * HD * 4}};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlaps(o, i)) return VDN_ERR_INVALID_ARG;
  for (size_t a = 0; a < 3; ++a)
    for (size_t b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], outs[b])) return VDN_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  float* partial = reinterpret_cast<float*>(ws);
  float* xbar = reinterpret_cast<float*>(ws + up(F * proj_mean_splits(p) * d_model * 4));
  return launch_gates(p, d_model, x, w_gb, w_alpha, gate, beta, alpha, partial, xbar, stream) == hipSuccess
             ? VDN_OK
             : VDN_ERR_HIP;
}

vdn_status vdn_vda_out_proj(const vdn_vda_desc* d, int32_t d_model, const void* o, const void* w_o,
                            const void* y_in, void* y, hipStream_t stream) {
  const vdn_status st = check_proj(d, d_model);
  if (st != VDN_OK) return st;
  if (!o || !w_o || !y) return VDN_ERR_INVALID_ARG;
  const void* need16[] = {o, w_o, y_in, y};
  for (const void* ptr : need16)
    if (ptr && !aligned(ptr, 16)) return VDN_ERR_ALIGNMENT;
  const Problem p = proj_problem(d);
  const size_t M = (size_t)p.B * p.T * p.U, HD = (size_t)p.H * p.D;
  // y may be y_in itself (each element is read before it is written), nothing else
  const Span ys{y, M * d_model * 2};
  if (overlaps(ys, Span{o, M * HD * 2}) || overlaps(ys, Span{w_o, (size_t)d_model * HD * 2})) return VDN_ERR_INVALID_ARG;
  if (y_in && y_in != y && overlaps(ys, Span{y_in, M * d_model * 2})) return VDN_ERR_INVALID_ARG;
  return launch_out_proj(p, d_model, o, w_o, y_in, y, stream) == hipSuccess ? VDN_OK : VDN_ERR_HIP;
}

const char* vdn_vda_status_string(vdn_status s) {
  static_assert(sizeof(vdn_status) == sizeof(int), "vdn_status is an int-sized enum");
  // callers may pass any integer (C, ctypes); read its bits rather than load an
  // enum value outside the enumeration's range
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case VDN_OK: return "VDN_OK";
    case VDN_ERR_INVALID_ARG: return "VDN_ERR_INVALID_ARG: bad descriptor, size, NULL pointer or overlapping buffers";
    case VDN_ERR_UNSUPPORTED:
      return "VDN_ERR_UNSUPPORTED: valid request not implemented (d_k != d_v; float32 in the adjacent maps; "
             "the query norm's backward without the epilogue)";
    case VDN_ERR_WORKSPACE: return "VDN_ERR_WORKSPACE: workspace missing or too small";
    case VDN_ERR_ALIGNMENT: return "VDN_ERR_ALIGNMENT: pointer misaligned";
    case VDN_ERR_HIP: return "VDN_ERR_HIP: kernel launch failed";
  }
  return "unknown vdn_status";
}

}  // extern "C"
