/*
 * vdn_vda.h -- C ABI of the MI355X (gfx950) Video Delta Attention forward pass.
 *
 * Video Delta Attention (VDA) is the frame-level delta-rule linear-attention
 * branch of Video DeltaNet.  Sources, cited by page title and section:
 *   [VDN-summary]   "프레임 단위 델타 규칙과 양방향 선형 메모리로 영상 확산 모델의
 *                   어텐션 병목을 걷어낸 Video DeltaNet" (onedev.kr/papers/80),
 *                   sections "어떻게 동작하나" (how it works), "무엇과 다른가"
 *                   (how it differs), "어떻게 쓰나" (how it is used),
 *                   "전제와 한계" (premises and limits).
 *   [VDN-H3-writeup] "VDN-H3: MiniMax H3 영상을 재생 시간보다 빠르게 생성하는
 *                   하이브리드 어텐션 모델" (discuss.pytorch.kr), section on the
 *                   hybrid attention structure.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  Every tensor is dense,
 *     row-major, contiguous, and 16-byte aligned (the workspace 256-byte).
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates or frees device memory and keeps no state between calls (the
 *     one exception: vdn_vda_forward_noalloc's own device array).
 *   - Work is enqueued on `stream` and the call returns without synchronising.
 *   - The return value is the only error channel.  Arguments are checked before
 *     anything is enqueued; on any error nothing is enqueued and outputs are
 *     untouched.  VDN_ERR_HIP reports a failed kernel launch (the stream may then
 *     hold part of the work).
 *   - Every buffer a call writes (outputs and workspace) must share no byte with
 *     any buffer it reads or with another buffer it writes; the byte ranges the
 *     shapes give are compared and an overlap is VDN_ERR_INVALID_ARG.  The one
 *     exception is stated with vdn_vda_out_proj.
 *   - Calls on distinct streams with distinct workspaces may run concurrently.
 *   - NaN/Inf inputs propagate; they are not detected.
 *
 * Shapes (B batch, T latent frames, U = grid_h * grid_w tokens per frame,
 * H heads, L text tokens, d_k = d_v = d):
 *   q, k, v, gate, out : [B, T, U, H, d]      in `dtype`
 *   beta               : [B, T, U, H]         in `dtype`, >= 0 (write strength per token)
 *   alpha              : [B, T, H, d_k]       float32, in [0, 1] (decay per key channel)
 *   k_text, v_text     : [B, L, H, d]         in `dtype`
 *   beta_text          : [B, L, H]            in `dtype`, >= 0
 *   rms_weight         : [d_v]                float32 (RMSNorm gain), NULL = all ones
 *   prep conv weights  : wk_s, wv_s [H*d, 5, 5], wk_t, wv_t [H*d, 5] float32;
 *                        channel index = h * d + j.
 */
#ifndef VDN_VDA_H
#define VDN_VDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VDN_OK = 0,
  VDN_ERR_INVALID_ARG = 1, /* bad shape/size, NULL required pointer, bad flag */
  VDN_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement */
  VDN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than vdn_vda_workspace_bytes() */
  VDN_ERR_ALIGNMENT = 4,   /* a pointer misses its alignment */
  VDN_ERR_HIP = 5          /* a kernel launch failed */
} vdn_status;

typedef enum {
  VDN_F32 = 0,  /* IEEE binary32 */
  VDN_BF16 = 1  /* bfloat16 */
} vdn_dtype;

enum {
  /* Apply RMSNorm over d_v and the sigmoid output gate to the readout
   * ([VDN-summary] "무엇과 다른가").  Requires `gate`.  Without this flag
   * `out` receives the raw readout o = (S_fwd + S_rev) q. */
  VDN_VDA_EPILOGUE = 1u << 0,
  /* Keep every intermediate in the workspace at the offsets that
   * vdn_vda_workspace_layout() reports.  The forward pass always leaves them
   * there, so the flag asks for nothing beyond the default; it is accepted for
   * callers that state the requirement. */
  VDN_VDA_DEBUG_KEEP = 1u << 1,
  /* VDA-Gather's decay bridge ([VDN-summary] "전제와 한계" names it without a
   * definition; reading used here): a non-anchor query in chunk c reads
   * F_{c-2} Diag(prod of alpha_s over chunk c-1) forward and
   * R_{c+2} Diag(prod of alpha_s over chunk c+1) in reverse -- the frames
   * between the summarised range and the query chunk, anchor frames included,
   * absorbed with zero writes (S <- S Diag(alpha_s)).  Chunk 0 has no forward
   * bridge, the last chunk no reverse bridge; anchor queries are unchanged.
   * Without the flag a query reads the boundary states as they are. */
  VDN_VDA_DECAY_BRIDGE = 1u << 2,
  /* Fuse the query's L2 normalisation ([VDN-summary] "무엇과 다른가") into the
   * readout.  vdn_vda_forward then takes the raw q and reads every
   * (token, head) row as q / sqrt(sum q^2 + l2_eps), the norm taken in float32
   * from the exact inputs, so q_hat is never materialised (nor rounded to
   * `dtype`).  vdn_vda_prepare leaves the query alone under this flag: its q
   * and q_hat are ignored and may be NULL. */
  VDN_VDA_QUERY_L2 = 1u << 3,
  /* How the bidirectional scan runs (at most one of the two; with neither the
   * library picks).  Frame by frame: one serial step per absorbed frame.
   * Chunk-composed ([VDN-summary] "전제와 한계": the chunk-parallel scan):
   * every chunk's frames are first folded, all chunks at once, into one pair
   * (M_c, J_c) with S_after = S_before M_c + J_c, then the scan takes one
   * serial step per chunk.  Both give the same states up to rounding; the
   * chunk-composed form shortens the serial path where few (batch, head)
   * pairs leave most of the GPU idle. */
  VDN_VDA_SCAN_FRAMES = 1u << 4,
  VDN_VDA_SCAN_CHUNKS = 1u << 5
};

/* Problem descriptor: a host struct owned by the caller, passed by pointer. */
typedef struct {
  int32_t B, H, T;         /* batch, heads, latent frames (T >= 1) */
  int32_t grid_h, grid_w;  /* token grid of a latent frame; U = grid_h * grid_w */
  int32_t d_k, d_v;        /* head widths: equal, a multiple of 16 up to 128 (see
                              vdn_vda_validate for which entry points take which) */
  int32_t n_text;          /* L text tokens per batch element (may be 0) */
  int32_t chunk;           /* latent frames per VAE chunk (the pages use 5); >= 1 */
  vdn_dtype dtype;         /* dtype of q, k, v, beta, text tensors, gate and out */
  uint32_t flags;          /* VDN_VDA_* bits */
  float l2_eps;            /* prep L2 normalisation: x / sqrt(sum x^2 + l2_eps); > 0 */
  float rms_eps;           /* RMSNorm: o / sqrt(mean o^2 + rms_eps); > 0 */
} vdn_vda_desc;

/* Byte offsets (from the workspace base) of the intermediates the forward pass
 * leaves in the workspace.  All are float32 except pinv with bfloat16 inputs.
 *   stats  [B, H, T+1, d_k + d_v, d_k]: rows 0..d_k-1 hold A_t = K_t^T Diag(beta_t) K_t,
 *          rows d_k.. hold B_t = V_t^T Diag(beta_t) K_t; slot T holds the text
 *          frame.  Anchor frames (0, T-1) are not formed.
 *   pinv   [B, H, T+1, d_k, d_k]: (I + A_t)^{-1}; slot T = text.  With
 *          VDN_BF16 and d_k >= 32 each slot's d_k*d_k*4 bytes instead hold
 *          P = (I + A_t)^{-1} as two bfloat16 planes, hi then lo (P ~ hi + lo),
 *          each as 16-byte fragments: fragment f = ((2w + e)(d_k/32) + s)*64 + l
 *          holds P[32s + 8(l/16) + j][32w + 2(l%16) + e] for j = 0..7
 *          (w < d_k/32, e < 2, s < d_k/32, l < 64).
 *   s_text [B, H, d_v, d_k]: the text state S_T.
 *   fwd    [B, H, n_c, d_v, d_k]: forward state after the last frame of chunk j.
 *   rev    [B, H, n_c, d_v, d_k]: reverse state after the first frame of chunk j.
 *   readout_states: the per-chunk states the readout reads, in the readout
 *          kernel's own packed operand order (not meant for callers).
 *   chunk_m, chunk_j [B, H, 2 (forward, reverse), n_c, d_v, d_k]: the chunk
 *          pairs (M_c, J_c) of the chunk-composed scan, written only when it
 *          runs, for the chunks that end in a record (forward 0..n_c-3,
 *          reverse 2..n_c-1).  J_c float32; M_c float32, or for VDN_BF16 with
 *          d_k >= 32 in the two-plane bfloat16 format of pinv.
 *   n_c = ceil(T / chunk).  Entries a query never reads are left unspecified.
 *   At a head width d between the built ones (48, 80, 96, 112) every section
 *   is laid out for the built width D the kernels run at (64 for 48, else 128)
 *   in place of d_k and d_v: the matrices are D x D with their leading d x d
 *   blocks those of the method and zeros elsewhere (the inverse's identity
 *   outside the block); the workspace also holds the zero-padded copies of the
 *   inputs and of the output (internal sections). */
typedef struct {
  size_t stats, pinv, s_text, fwd, rev, readout_states, chunk_m, chunk_j, total;
} vdn_vda_layout;

/* Check a descriptor without touching the GPU.  Host only.  Besides shapes,
 * widths and flags it enforces the kernels' 32-bit byte-offset limits, with
 * U = grid_h * grid_w and L = n_text: (U + 64) H d 4 and (L + 64) H d 4 bytes
 * (a frame's or the text's token rows plus a tile's overhang) and
 * (U + 640) H d 2 and (L + 640) H d 2 bytes (the statistics kernel's prefetch
 * past the last token) below 4 GiB, and one head's chunk records below 2^31
 * bytes, where d is the built width the kernels run at (the caller's width,
 * or the next of 16, 32, 64, 128).  VDN_ERR_INVALID_ARG when a limit fails or
 * a width is not a multiple of 16 in 16 .. 128, VDN_ERR_UNSUPPORTED for
 * d_k != d_v.  VDN_OK means the forward pass (vdn_vda_forward, _timed,
 * _noalloc) takes the descriptor.  Widths 48, 80, 96 and 112 run only there:
 * the kernels are built for 16, 32, 64 and 128 (matrix-core tiles of 16 and
 * 32), and the forward pass runs them at the next built width D on copies of
 * the inputs zero-padded to D channels, in its workspace, then copies the
 * output's d channels back (zero channels leave every result unchanged; the
 * epilogue takes rms_eps d / D and the gain scaled by sqrt(d / D), which
 * gives the same RMSNorm over the d true channels).  The backward pass takes
 * them the same way: it reads the forward's padded copies from the forward's
 * workspace, pads dy, k and v in its own, and copies every gradient's d
 * channels back (the gain's gradient scaled by sqrt(d / D)).  The prep (a
 * per-channel convolution and per-token norms) and the adjacent maps (plain
 * products over a token's H d channels) run at the width itself. */
vdn_status vdn_vda_validate(const vdn_vda_desc* d);

/* Workspace bytes vdn_vda_forward needs for `d`; 0 if `d` is invalid. */
size_t vdn_vda_workspace_bytes(const vdn_vda_desc* d);

/* Fill `out` (host) with the workspace offsets for `d`. */
vdn_status vdn_vda_workspace_layout(const vdn_vda_desc* d, vdn_vda_layout* out);

/*
 * vdn_vda_prepare -- the linear branch's feature preparation
 * ([VDN-summary] "무엇과 다른가": separable short convolution on K and V --
 * depthwise 5x5 spatial then 5-tap temporal -- then SiLU; L2 normalisation of
 * Q and K; no rotary embedding; "전제와 한계": the fused prep kernel).
 *   k_hat = L2(SiLU(conv_t(conv_s(k)))), v_hat = SiLU(conv_t(conv_s(v))), q_hat = L2(q).
 * The convolutions are cross-correlations per channel with zero padding 2 on
 * every side (rows, columns, frames); temporal taps are centred (t-2 .. t+2)
 * and cross chunk boundaries.  Text tokens are not convolved.
 * q, k, v: [B, T, U, H, d] raw features; q_hat, k_hat, v_hat: same shape,
 * out of place (must not alias the inputs).  Weights as in the header comment.
 * With VDN_VDA_QUERY_L2 in d->flags q and q_hat are ignored (may be NULL) and
 * the forward pass normalises the query instead.
 * Errors: VDN_ERR_INVALID_ARG (descriptor, NULL pointer), VDN_ERR_UNSUPPORTED
 * (d_k != d_v), VDN_ERR_ALIGNMENT,
 * VDN_ERR_HIP.
 */
vdn_status vdn_vda_prepare(const vdn_vda_desc* d,
                           const void* q, const void* k, const void* v,
                           const float* wk_s, const float* wk_t,
                           const float* wv_s, const float* wv_t,
                           void* q_hat, void* k_hat, void* v_hat,
                           hipStream_t stream);

/*
 * vdn_vda_forward -- the VDA forward pass on prepared features.
 * For each (batch, head):
 *   text state ([VDN-summary] "어떻게 동작하나"): S_T = B_T (I + A_T)^{-1} over the
 *     L text tokens (a leading virtual frame updated from a zero state);
 *   frame statistics and update ([VDN-summary] "어떻게 쓰나"):
 *     A_t = K_t^T Diag(beta_t) K_t,  B_t = V_t^T Diag(beta_t) K_t,
 *     S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1};
 *   bidirectional scan ([VDN-summary] "어떻게 동작하나"; anchors excluded,
 *     "전제와 한계"): both directions start from S_T / 2; the forward state
 *     of a query frame covers the non-anchor frames before its softmax window
 *     (its chunk and the neighbouring chunks), the reverse state those after it;
 *     anchor query frames (0, T-1) read S_T only;
 *     with VDN_VDA_DECAY_BRIDGE the two states are first decayed across the
 *     chunks next to the query's (see the flag);
 *   readout: o = (S_fwd + S_rev) q; with VDN_VDA_EPILOGUE,
 *     out = rms_weight * o / sqrt(mean(o^2) + rms_eps) * sigmoid(gate)
 *     ([VDN-summary] "무엇과 다른가"), else out = o.
 * q, k must be the prepared (unit-norm) features; with VDN_VDA_QUERY_L2, q is
 * the raw query and the readout normalises it (see the flag).  k_text, v_text, beta_text
 * may be NULL when n_text = 0 (then S_T = 0).  gate is required with
 * VDN_VDA_EPILOGUE and ignored without it.  out is written in `dtype` with
 * round-to-nearest-even.  With VDN_BF16 the frame statistics take
 * sqrt(beta) k and sqrt(beta) v as IEEE half operands (fp32 sums); a (frame,
 * head) whose |sqrt(beta) v| or |sqrt(beta) k| exceeds the half range (65504)
 * is recomputed on operands scaled by powers of two, so any finite bfloat16
 * value is handled (only that unit pays a second pass).  The state,
 * statistics, inverse and scan are float32;
 * with VDN_BF16 and d_k >= 32 the scan's product Y (I + A_t)^{-1} takes both
 * operands as bfloat16 hi + lo pairs (three bfloat16 matrix-core products,
 * fp32 accumulation, about 2^-16 relative per frame step).
 * Errors: VDN_ERR_INVALID_ARG, VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE,
 * VDN_ERR_ALIGNMENT, VDN_ERR_HIP.
 */
vdn_status vdn_vda_forward(const vdn_vda_desc* d,
                           const void* q, const void* k, const void* v,
                           const float* alpha, const void* beta,
                           const void* k_text, const void* v_text,
                           const void* beta_text,
                           const void* gate, const float* rms_weight,
                           void* out,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Backward pass, first stage: back through the epilogue and the readout.
 *
 * The forward pass is differentiated with respect to its inputs (the training
 * of the linear branch, [VDN-summary] "전제와 한계"); this stage covers the
 * readout o_t = S_q(t) q_t (S_q(t) = the forward plus the reverse state the
 * frame's queries read, [VDN-summary] "어떻게 동작하나") and, with
 * VDN_VDA_EPILOGUE, y = rms_weight * o / sqrt(mean o^2 + rms_eps) * sigmoid(gate)
 * ([VDN-summary] "무엇과 다른가").  Given the output's adjoint dy it writes
 *   dq    [B, T, U, H, d_k] = S_q(t)^T do per token                (dtype),
 *   dgate [B, T, U, H, d_v] = dy * rms_weight * n * s * (1 - s)     (dtype;
 *         n = o / sqrt(mean o^2 + rms_eps), s = sigmoid(gate); with VDN_VDA_EPILOGUE),
 *   d_rms_weight [d_v] = sum over every batch, frame, token and head of
 *         dy * s * n, the gradient of the RMSNorm gain (float32; with
 *         VDN_VDA_EPILOGUE, and only when d_rms_weight is not NULL; formed
 *         whether or not rms_weight is given, a NULL rms_weight being a gain
 *         of ones; overwritten, not accumulated),
 * and leaves in its workspace, at the offsets vdn_vda_backward_workspace_layout()
 * reports,
 *   d_out     [B, T, U, H, d_v] in dtype: do, the readout's adjoint
 *             (= rms_weight * s * dy * r - n * r * mean(rms_weight * s * dy * n),
 *             r = 1 / sqrt(mean o^2 + rms_eps)), divided by |q| per token with
 *             VDN_VDA_QUERY_L2; written with VDN_VDA_EPILOGUE only -- without it
 *             do is dy itself and dy is read in its place;
 *   d_state_q [B, H, T, d_v, d_k] float32: sum over the frame's tokens of
 *             do q^T, the adjoint of S_q(t), for every frame (the next stage
 *             turns these into the adjoints of the records and of S_T);
 *   readout_states_t: S_q^T per chunk slot in the readout kernel's operand
 *             order (not meant for callers).
 * d_rms_weight is summed in a fixed order (per (frame, head) in the readout
 * kernel, then over those sums), so it is the same from call to call.
 * fwd_workspace must hold what vdn_vda_forward left there for the same
 * descriptor and inputs (q, k, v, alpha, beta, text, gate, rms_weight); alpha
 * is read for the decay bridge.  dy, dq, dgate are device buffers owned by the
 * caller; dq and dgate must not alias any input.  With VDN_VDA_QUERY_L2 (the
 * forward normalised the raw query, q_n = q / sqrt(sum q^2 + l2_eps)) dq is the
 * gradient of the raw query, (dq_n - q_n (q_n . dq_n)) / |q| with dq_n = S_q^T do,
 * and d_out holds do / |q| per token (so that d_state_q = sum d_out q^T reads
 * the raw query).  Supported: VDN_BF16 and VDN_F32 (do, dq, dgate and d_out
 * then float32), and VDN_VDA_QUERY_L2 only with
 * VDN_VDA_EPILOGUE (else VDN_ERR_UNSUPPORTED).  Errors: VDN_ERR_INVALID_ARG
 * (NULL pointer, gate or dgate missing with the epilogue, d_rms_weight without
 * it, aliasing), VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE (either workspace too
 * small or NULL), VDN_ERR_ALIGNMENT (16 B for tensors, 4 B for d_rms_weight,
 * 256 B for workspaces), VDN_ERR_HIP.  Asynchronous on `stream`.
 */
/* Offsets (bytes from the base) of the backward workspace's documented
 * sections; the workspace also holds internal sections.  The second stage's
 * (float32):
 *   d_record_f, d_record_r [B, H, n_c, d_v, d_k]: adjoints of the records F_j, R_j
 *             (zero where no record is read);
 *   d_text_q  [B, H, d_v, d_k]: the part of S_T's adjoint that its direct
 *             readers give (anchor queries, sides reading S_T / 2, records the
 *             scan never reaches);
 *   lam_f, lam_r [B, H, T+1, d_v, d_k]: slot s holds the adjoint of the state
 *             each scan has after absorbing frame s, for the frames it absorbs,
 *             zero elsewhere; slot T of lam_f is the adjoint of S_T as a whole;
 *   d_a, d_b  [B, H, T+1, d_k, d_k] and [B, H, T+1, d_v, d_k]: dA_t, dB_t for the
 *             absorbed frames and the text frame (slot T), zero for the anchors.
 *             A_t is symmetric, so only dA_t + dA_t^T reaches an input; d_a
 *             holds -P_t d(P_t) P_t with d(P_t) = sum over the scans of Y^T lambda. */
typedef struct {
  size_t readout_states_t, d_out, d_state_q;
  size_t d_record_f, d_record_r, d_text_q, lam_f, lam_r, d_a, d_b;
  size_t total;
} vdn_vda_backward_layout;

/* Workspace bytes vdn_vda_backward_readout needs for `d`; 0 if `d` is invalid. */
size_t vdn_vda_backward_workspace_bytes(const vdn_vda_desc* d);

/* Fill `out` (host) with the backward workspace's offsets for `d`. */
vdn_status vdn_vda_backward_workspace_layout(const vdn_vda_desc* d, vdn_vda_backward_layout* out);

vdn_status vdn_vda_backward_readout(const vdn_vda_desc* d,
                                    const void* q, const void* gate,
                                    const float* rms_weight, const float* alpha,
                                    const void* dy,
                                    const void* fwd_workspace, size_t fwd_workspace_bytes,
                                    void* dq, void* dgate, float* d_rms_weight,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Backward pass, second stage: back through the coverage rules, the two scans
 * and (I + A_t)^{-1}.  Reads the first stage's d_state_q from `workspace` and
 * the forward's workspace; writes d_record_f / d_record_r / d_text_q, lam_f /
 * lam_r and d_a / d_b into `workspace` (see vdn_vda_backward_layout) and
 *   dalpha [B, T, H, d_k] float32: the gradient of alpha (zero for the anchors
 *          without the decay bridge).
 * Per absorbed frame s of a scan with adjoint lambda (the state's, after the
 * record adjoint of the state frame s produces is added): dY = lambda P_s,
 * dB_s += dY, dalpha_s += column sums of S_prev * dY, d(P_s) += Y_s^T lambda with
 * Y_s = S_prev Diag(alpha_s) + B_s, and lambda <- dY Diag(alpha_s) for the state
 * before; then dA_s = -P_s d(P_s) P_s (P_s = (I + A_s)^{-1}, [VDN-summary]
 * "어떻게 쓰나").  The text frame S_T = B_T P_T takes lambda = the adjoint of
 * S_T.  With VDN_VDA_DECAY_BRIDGE a query chunk's adjoint reaches the records
 * (and S_T / 2) column-scaled by its bridge's alpha products, and dalpha adds
 * the bridge's own term (frames of the bridged chunks, anchors included).
 * Supported: VDN_BF16 and VDN_F32; (T + 2) D D 4 < 2^31 (D the built width).  Errors as
 * vdn_vda_backward_readout.  Asynchronous on `stream`.
 */
vdn_status vdn_vda_backward_scan(const vdn_vda_desc* d, const float* alpha,
                                 const void* fwd_workspace, size_t fwd_workspace_bytes,
                                 float* dalpha,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Backward pass, third stage: back through the frame statistics
 * A_t = K_t^T Diag(beta_t) K_t and B_t = V_t^T Diag(beta_t) K_t ([VDN-summary]
 * "어떻게 쓰나") and the text frame's A_T, B_T.  Reads the second stage's d_a /
 * d_b from `workspace` and writes, per token (G = dA_t + dA_t^T of its frame),
 *   dk    = beta (G k + dB_t^T v),       dv = beta dB_t k,
 *   dbeta = k^T dA_t k + v^T dB_t k,
 * for every frame into dk, dv [B, T, U, H, d] and dbeta [B, T, U, H] (zero for
 * the anchor frames, which no scan absorbs) and for the text tokens into
 * dk_text, dv_text [B, L, H, d] and dbeta_text [B, L, H] (unused when
 * n_text = 0), all bfloat16.  G and dB_t enter the matrix cores as bfloat16
 * hi + lo pairs (dbeta sums d^2 products that largely cancel), dB_t^T (dk
 * only) rounded once to bfloat16.  k, v, beta and the text inputs are
 * those the forward pass read.  Outputs must overlap neither each other, the
 * inputs nor the workspace.  Supported: VDN_BF16 and VDN_F32 (beta and dbeta 4-byte aligned).  Errors: VDN_ERR_INVALID_ARG
 * (NULL pointer, overlap), VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE,
 * VDN_ERR_ALIGNMENT (16 B for k, v and the d-wide outputs, 2 B for beta and the
 * dbeta outputs, 256 B for the workspace), VDN_ERR_HIP.  Asynchronous on `stream`.
 */
vdn_status vdn_vda_backward_gram(const vdn_vda_desc* d, const void* k, const void* v, const void* beta,
                                 const void* k_text, const void* v_text, const void* beta_text,
                                 void* dk, void* dv, void* dbeta,
                                 void* dk_text, void* dv_text, void* dbeta_text,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The linear maps either side of the path ([VDN-summary] "무엇과 다른가": the
 * linear branch's sigmoid output gate, its separate decay and write gates, and
 * its own output projection summed with the softmax branch's into the residual
 * stream; "어떻게 쓰나": alpha per key channel per frame, beta per token;
 * "전제와 한계": the decay module in FP32).  The pages give no form for these
 * maps; the library takes linear maps of the attention block's input without
 * bias, weights stored [out, in]:
 *   gate  [B, T, U, H, d_v] bfloat16 = W_g x                (logits; the forward
 *                                       pass applies the sigmoid in its epilogue)
 *   beta  [B, T, U, H]      bfloat16 = sigmoid(w_beta x)
 *   alpha [B, T, H, d_k]    float32  = sigmoid(W_alpha xbar_t), xbar_t the mean
 *                                       of frame t's tokens, in float32
 * x [B, T, U, d_model] bfloat16; w_gb [H d_v + H, d_model] bfloat16 holds W_g's
 * rows then w_beta's; w_alpha [H d_k, d_model] float32.  Gate logits and beta
 * come from one bfloat16 matrix-core product (float32 accumulation, the
 * sigmoid applied before rounding).  The workspace (vdn_vda_gates_workspace_bytes)
 * holds the frames' token sums.  d_model a multiple of 8; the descriptor's
 * n_text, chunk and flags are ignored; any head width the descriptor allows;
 * VDN_BF16 only (else VDN_ERR_UNSUPPORTED).  Outputs must overlap neither each other, the inputs
 * nor the workspace.  Errors: VDN_ERR_INVALID_ARG (NULL pointer, d_model,
 * overlap), VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE, VDN_ERR_ALIGNMENT (16 B;
 * 2 B for beta; 256 B for the workspace), VDN_ERR_HIP.  Asynchronous on `stream`.
 */
size_t vdn_vda_gates_workspace_bytes(const vdn_vda_desc* d, int32_t d_model);
vdn_status vdn_vda_gates(const vdn_vda_desc* d, int32_t d_model, const void* x, const void* w_gb,
                         const float* w_alpha, void* gate, void* beta, float* alpha,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The linear branch's output projection merged into what the caller adds:
 *   y [B, T, U, d_model] = y_in + o W_O^T,
 * o [B, T, U, H, d_v] the forward pass's output, w_o [d_model, H d_v], y_in
 * [B, T, U, d_model] (NULL: zero; typically the softmax branch's projected
 * output plus the residual stream), all bfloat16; the sum is rounded once from
 * the bfloat16-rounded product.  y may be y_in itself and must overlap nothing
 * else.  d_model a multiple of 8; VDN_BF16 only.  Errors as vdn_vda_gates.
 * Asynchronous on `stream`.
 */
vdn_status vdn_vda_out_proj(const vdn_vda_desc* d, int32_t d_model, const void* o, const void* w_o,
                            const void* y_in, void* y, hipStream_t stream);

/*
 * vdn_vda_forward_timed -- vdn_vda_forward with per-stage timing events, for
 * benchmarks.  Same arguments, checks and results as vdn_vda_forward; in
 * addition it records events[0] on `stream` before its first kernel and
 * events[i] after stage i, i = 1..VDN_VDA_STAGES: frame statistics (the text
 * frame included), solve, scan, gather, readout (at a width between the
 * built ones the input copies fall in the first stage and the output's copy
 * back in the last).  The caller creates the
 * n_events >= VDN_VDA_STAGES + 1 events (hipEventCreate); nothing is kept
 * after the call returns.  Errors: those of vdn_vda_forward, and
 * VDN_ERR_INVALID_ARG for a NULL events array, too few events or a NULL event.
 */
enum { VDN_VDA_STAGES = 5 };
vdn_status vdn_vda_forward_timed(const vdn_vda_desc* d,
                                 const void* q, const void* k, const void* v,
                                 const float* alpha, const void* beta,
                                 const void* k_text, const void* v_text,
                                 const void* beta_text,
                                 const void* gate, const float* rms_weight,
                                 void* out,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, hipEvent_t* events, int32_t n_events);

/*
 * vdn_vda_forward_noalloc -- vdn_vda_forward without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments
 * (less the workspace), checks and results as vdn_vda_forward; the forward's
 * workspace is instead a device array inside the library, of
 * VDN_VDA_NOALLOC_MAX_WORKSPACE bytes, that every GPU the library runs on
 * holds from the library's load until the process ends.  The call allocates
 * and frees nothing.  Problems whose workspace (vdn_vda_workspace_bytes) is
 * larger return VDN_ERR_WORKSPACE before anything touches the GPU; 64 MiB
 * covers, e.g., 8 heads x 40 frames x 1560 tokens at d = 64, or one GPU's
 * 3-head share of the 768p clip.  The array's address on the current device is
 * looked up on the first call on that device (VDN_ERR_HIP if that fails) and
 * kept: this entry point, unlike the others, keeps that per-device address
 * between calls.  Every call on one GPU shares that GPU's array and leaves
 * its intermediates there (at vdn_vda_workspace_layout's offsets) until the
 * next call: calls that overlap in time on one GPU (two streams, two threads)
 * race on it and must be serialised by the caller.  The stream must belong to
 * the current device.
 */
#define VDN_VDA_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
vdn_status vdn_vda_forward_noalloc(const vdn_vda_desc* d,
                                   const void* q, const void* k, const void* v,
                                   const float* alpha, const void* beta,
                                   const void* k_text, const void* v_text,
                                   const void* beta_text,
                                   const void* gate, const float* rms_weight,
                                   void* out, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* vdn_vda_status_string(vdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* VDN_VDA_H */
