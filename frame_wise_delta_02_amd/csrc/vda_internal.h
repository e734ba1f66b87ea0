// Internal declarations shared by the VDA HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdn_vda.h"

namespace vda {

// ---------------------------------------------------------------------------
// vector types for the gfx950 matrix-core builtins
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> two bfloat16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Two floats -> two IEEE halves (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 r = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Split x into hi + lo, both bfloat16: hi = bf16(x), lo = bf16(x - hi).
// hi + lo carries about 16 significant bits of x.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Raw buffer resource over [base, base + bytes): loads at or past `bytes`
// return zero and stores there are dropped (gfx9 descriptor, word 3 = 0x00020000).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}
// The same with the non-temporal cache policy (bit 1 of the cache-policy
// operand, NT on gfx950): for streams a kernel reads or writes exactly once,
// so they do not displace data that other workgroups or the next kernel
// re-read from L2 and the Infinity Cache.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ void buf_store16_nt(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 2);
}

// A wave-uniform value forced into a scalar register.  The optimiser drops
// __builtin_amdgcn_readfirstlane on values it already considers uniform, and
// may then compute them in vector registers anyway; a buffer descriptor built
// from such a value turns every load into a waterfall loop.  The asm is opaque.
// It is opaque to the hazard recognizer too: v_readfirstlane is a vector ALU
// instruction writing a scalar register, and on CDNA a vector memory
// instruction that reads a scalar register so written needs 5 wait states in
// between, which the hardware does not enforce.  The compiler inserts them for
// its own instructions but cannot see this one, so the s_nop 4 (5 wait
// states) comes with it, whatever the scheduler places after it.
__device__ __forceinline__ int sgpr(int v) {
  int r;
  asm volatile("v_readfirstlane_b32 %0, %1\n\ts_nop 4" : "=s"(r) : "v"(v));
  return r;
}

// Workgroup barrier for LDS exchange only.  __syncthreads() is a full
// workgroup fence, so it also waits for every global load in flight
// (s_waitcnt vmcnt(0)) and drains any software prefetch.  Here each wave only
// waits for its own LDS operations (lgkmcnt(0); gfx9 s_waitcnt encoding with
// vmcnt and expcnt left at their maxima) before s_barrier; the signal fences
// keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// launch plumbing
// ---------------------------------------------------------------------------
struct Problem {
  int B, H, T, U, D, L, C;  // D: the kernels' head width; C = frames per chunk
  int Du;                   // the caller's d_k = d_v (D rounded up to 16, 32, 64 or 128)
  int nc;                   // number of chunks
  bool bf16;
  bool epilogue;
  bool bridge;  // VDN_VDA_DECAY_BRIDGE
  bool qnorm;   // VDN_VDA_QUERY_L2: the readout normalises the raw query
  bool chunked; // scan over chunk-composed pairs (M_c, J_c) instead of frame by frame
  float l2_eps, rms_eps;
};

// Workspace offsets in bytes (see vdn_vda_layout).
struct Layout {
  size_t stats, pinv, s_text, fwd, rev, rstates, chunk_m, chunk_j;
  // widths between the built ones (Du < D): the inputs copied with their
  // channels zero-padded to D, the padded output, the padded gain
  size_t pad_q, pad_k, pad_v, pad_gate, pad_out, pad_alpha, pad_k_text, pad_v_text, pad_gain;
  size_t total;
};
Layout make_layout(const Problem& p);

// Format of the inverse (I + A_t)^{-1} in the workspace.  float32 [d][d] for
// float32 inputs and for d = 16.  For bfloat16 inputs with d >= 32 the same
// d*d*4 bytes hold it split into two bfloat16 planes, hi then lo
// (P^{-1} ~ hi + lo, about 16 significant bits), each in the scan's
// v_mfma_f32_16x16x32_bf16 B-operand order: 16-byte fragment
// f = ((2w + e) * (d/32) + ks) * 64 + l holds P^{-1}[32 ks + 8 (l/16) + j]
// [32 w + 2 (l%16) + e] for j = 0..7.
inline bool pinv_split(const Problem& p) { return p.bf16 && p.D >= 32; }

// Bytes of one readout state slot in the readout kernel's packed format.
size_t readout_slot_bytes(const Problem& p);

// Kernels are launched through these; each returns hipGetLastError().
// One part of a gram launch: frames t_first .. t_first + n_frames - 1 of K, V,
// beta laid out [B, T_in, U, H, d] (beta [B, T_in, U, H]), into stats slots
// t + slot_offset.  A launch takes one or two parts; the second part's blocks
// come after the first's.
struct GramPart {
  const void* k;
  const void* v;
  const void* beta;
  int T_in, U, t_first, n_frames, slot_offset;
};
hipError_t launch_gram(const Problem& p, const GramPart* parts, int nparts, float* stats, hipStream_t s);
// V^T K per frame with no beta, both [B, T, U, H, d] bfloat16, every frame t into
// out[B, H, T, d, d] (float32): the backward pass's dS_t = dO_t^T Q_t.
hipError_t launch_gram_plain(const Problem& p, const void* k, const void* v, float* out, hipStream_t s);
hipError_t launch_solve(const Problem& p, const float* stats, float* pinv, hipStream_t s);
// The bidirectional scan; with p.chunked, first every chunk's pair
// (M_c, J_c) into chunk_m / chunk_j ([B, H, 2, n_c, d, d] each), then the scan
// over chunks.
hipError_t launch_scan(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                       float* s_text, float* fwd, float* rev, float* chunk_m, float* chunk_j, hipStream_t s);
// Backward pass: the frame scan recording every frame's state (states_f,
// states_r: [B, H, T+2, d, d], start state S_T/2 in slot 0 / T-1), and the
// adjoint scan (d_fwd, d_rev: record adjoints [B, H, n_c, d, d]; lam_f, lam_r:
// adjoint at every frame [B, H, T+1, d, d]; lam_final [B, H, 2, d, d]).
hipError_t launch_scan_states(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                              float* states_f, float* states_r, hipStream_t s);
hipError_t launch_scan_adjoint(const Problem& p, const float* stats, const float* pinv, const float* alpha,
                               const float* d_fwd, const float* d_rev, float* lam_f, float* lam_r,
                               float* lam_final, hipStream_t s);
hipError_t launch_gather(const Problem& p, const float* s_text, const float* fwd, const float* rev,
                         const float* alpha, void* rstates, hipStream_t s);
hipError_t launch_readout(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                          const void* rstates, void* out, hipStream_t s);
// First stage of the backward pass (bfloat16 inputs): rstates_t <- the
// transposed query states; with p.epilogue dout <- do (bfloat16) and
// dgate <- the gate's adjoint, else do = dy; dq <- S_q^T do; dsq [B, H, T, d, d]
// <- do_t^T q_t.  rstates, s_text, fwd, rev: the forward's workspace sections.
// With dgamma (the epilogue only): gain_part [B T H, d] <- per-(frame, head)
// sums, then dgamma[j] <- gain_scale * their sum, for j < gain_n.
hipError_t launch_backward_readout(const Problem& p, const void* q, const void* gate, const float* rms_weight,
                                   const void* dy, const void* rstates, const float* s_text, const float* fwd,
                                   const float* rev, const float* alpha, void* rstates_t, void* dout, void* dq,
                                   void* dgate, float* dsq, float* gain_part, float* dgamma, int gain_n,
                                   float gain_scale, hipStream_t s);
// dgamma[j] = scale * sum over the B T H rows of gain_part [rows][D], j < n.
hipError_t launch_gain_grad_sum(const Problem& p, const float* gain_part, float* dgamma, int n, float scale,
                                hipStream_t s);
// The first stage for float32 inputs (vda_backward_f32.hip): slots <- S_q per
// chunk slot as plain float32 [d_v][d_k] (in the rstates_t section), the rest
// as launch_backward_readout.
hipError_t launch_backward_readout_f32(const Problem& p, const float* q, const float* gate, const float* rms_weight,
                                       const float* dy, const float* s_text, const float* fwd, const float* rev,
                                       const float* alpha, float* slots, float* dout, float* dq, float* dgate,
                                       float* dsq, float* gain_part, float* dgamma, int gain_n, float gain_scale,
                                       hipStream_t s);
// Second stage of the backward pass: buffers (float32 unless noted).
struct BwdScanBuffers {
  const float* stats;   // forward workspace: [B, H, T+1, 2d, d]
  const float* pinv;    // forward workspace (the two-plane format when split)
  const float* alpha;   // [B, T, H, d]
  const float* dsq;     // first stage: [B, H, T, d, d]
  float *dF, *dR;       // [B, H, n_c, d, d]
  float* dST;           // [B, H, d, d]
  float *states_f, *states_r;  // [B, H, T+2, d, d]
  float *lam_f, *lam_r;        // [B, H, T+1, d, d]
  float* lam_final;            // [B, H, 2, d, d]
  float* p32;                  // [B, H, T+1, d, d]
  float *M, *dPinv, *tmp;       // [B, H, T+1, d, d]
  float *dA, *dB;              // [B, H, T+1, d, d] (out)
  float* dalpha;               // [B, T, H, d] (out)
  const float *s_text, *fwd, *rev;  // forward workspace (the decay bridge's term)
};
hipError_t launch_backward_scan(const Problem& p, const BwdScanBuffers& w, hipStream_t s);
// Third stage: dk, dv, dbeta of every frame and of the text tokens from dA, dB.
struct BwdGramBuffers {
  const float *dA, *dB;                     // [B, H, T+1, d, d] (second stage)
  void* mats;                               // [B, H, T+1] x 5 d x d bfloat16 operand planes
  const void *k, *v, *beta;                 // [B, T, U, H, d], [B, T, U, H]
  const void *k_text, *v_text, *beta_text;  // [B, L, H, d], [B, L, H]
  void *dk, *dv, *dbeta;                    // as k, v, beta (out)
  void *dk_text, *dv_text, *dbeta_text;     // as the text inputs (out)
};
hipError_t launch_backward_gram(const Problem& p, const BwdGramBuffers& w, hipStream_t s);
hipError_t launch_backward_gram_f32(const Problem& p, const BwdGramBuffers& w, hipStream_t s);
// The linear maps either side of the path: gate logits and sigmoid(beta) from
// one bfloat16 product with the stacked weights, the frames' mean tokens, and
// sigmoid(W_alpha xbar) in float32; the output projection with Y_in added.
int proj_mean_splits(const Problem& p);
hipError_t launch_gates(const Problem& p, int d_model, const void* x, const void* w_gb, const float* w_alpha,
                        void* gate, void* beta, float* alpha, float* partial, float* xbar, hipStream_t s);
hipError_t launch_out_proj(const Problem& p, int d_model, const void* o, const void* w_o, const void* y_in, void* y,
                           hipStream_t s);
// Row copies for the widths between the built ones: dst row r = the first
// copy_bytes of src row r, zero-filled to dst_row_bytes (all multiples of 16);
// the padded gain (w or ones) * sqrt(d / D), zero beyond d.
hipError_t launch_copy_rows(const void* src, size_t src_row_bytes, void* dst, size_t dst_row_bytes,
                            size_t copy_bytes, size_t rows, hipStream_t s);
hipError_t launch_pad_gain(const float* w, float* dst, int d, int D, hipStream_t s);
hipError_t launch_prep(const Problem& p, int grid_h, int grid_w, const void* q, const void* k,
                       const void* v, const float* wk_s, const float* wk_t, const float* wv_s,
                       const float* wv_t, void* q_hat, void* k_hat, void* v_hat, hipStream_t s);

}  // namespace vda
