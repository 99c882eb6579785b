/*
 * ptdit.h -- C ABI of the PT-DiT attention core (GIIM + TCM) for AMD MI355X
 * (gfx950). Hand-written HIP kernels; no torch types cross this boundary.
 *
 * The operations are those of the Qihoo-T2X reading note (page "Qihoo-T2X --
 * Proxy-Tokenized DiT for Text-to-Any-Task"):
 *   - section 3 "Method", Eq. GIIM: z_s = CS(z_s, SA(Averaging(z_s))) with
 *     z_s in R^{N x D} reshaped to f x h x w and one proxy token per
 *     p_t x p_h x p_w window (window average);
 *   - section 3 "Method", Eq. TCM: z_hat = WSA(z_s) + z_s,
 *     z_w = SWSA(z_hat) + z_hat, the shifted windows being a 3D cyclic shift;
 *   - the code-correspondence section (module table and excerpt 2, PT-Block
 *     forward) for the call order and residual placement.
 *
 * Conventions shared by every call
 * --------------------------------
 *  Tokens.   x is [B][N][D], N = F*H*W, tokens row-major over (f, h, w);
 *            channels contiguous.
 *  Proxies.  [B][M][D], M = (F/p_t)*(H/p_h)*(W/p_w), row-major over the
 *            window grid (T, I, J).
 *  Heads.    head h owns channels [h*dh, (h+1)*dh), dh = D/heads; scores are
 *            scaled by 1/sqrt(dh); no positional term inside the core.
 *  Weights.  nn.Linear layout, y = x W^T + b. w_qkv is [3D][D]: rows 0..D-1
 *            are W_q, D..2D-1 W_k, 2D..3D-1 W_v; b_qkv is [3D] or NULL;
 *            w_o is [D][D]; b_o is [D] or NULL. The single output projection
 *            of an attention plays the role of to_out followed by
 *            linear_1_visual (two linear maps compose into one).
 *  Precision ("prec").
 *            PTDIT_BF16: weights and biases are bf16; projections and
 *            attention run on bf16 MFMA with fp32 accumulation; the library's
 *            intermediates (Q, K, V, attention output) are bf16; softmax
 *            statistics are fp32. Activation inputs may be bf16 or fp32
 *            (x_dt), outputs bf16 or fp32 (out_dt); the residual added is the
 *            input x itself, in its own dtype.
 *            PTDIT_F32: everything fp32 (fp32 MFMA); x_dt = out_dt = F32.
 *  Memory.   Every pointer except the stream is a DEVICE pointer, 16-byte
 *            aligned. The caller allocates and frees all memory, including
 *            the workspace (size from ptdit_workspace_bytes). The library
 *            never allocates device memory, never synchronises the stream
 *            and keeps no state between calls except the optional kernel
 *            trace (ptdit_trace_*). out must not alias x or the workspace.
 *  Low-precision copies (optional, PTDIT_BF16 precision only).
 *            out_lowp: a [B][N][D] bf16 buffer that receives bf16(out),
 *            rounded to nearest even, written by the same epilogue that
 *            writes an fp32 out. x_lowp: a [B][N][D] bf16 buffer that holds
 *            bf16(x) of an fp32 x (for example a previous call's out_lowp);
 *            the Q/K/V projection then reads it instead of rounding x
 *            itself, which gives bit-identical results, while the residual
 *            still adds the fp32 x. The library does not verify that x_lowp
 *            matches x. Either may be NULL. Given with bf16 precision
 *            beside a bf16 tensor, or with PTDIT_F32 precision, they are
 *            rejected with PTDIT_ERR_DTYPE; they must not overlap any other
 *            argument (PTDIT_ERR_ALIAS).
 *  Streams.  All work is enqueued asynchronously on `stream` (0 = default).
 *  Errors.   Every argument is checked on the host before any launch; on a
 *            failed check nothing is launched, outputs are untouched and a
 *            negative ptdit_status is returned. A failed launch returns
 *            PTDIT_ERR_HIP. ptdit_status_str names a status.
 */
#ifndef PTDIT_H
#define PTDIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PTDIT_BF16 = 0, PTDIT_F32 = 1 } ptdit_dtype;

typedef enum {
  PTDIT_OK = 0,
  PTDIT_ERR_NULL = -1,          /* a required pointer is NULL */
  PTDIT_ERR_SHAPE = -2,         /* a size is non-positive, D % heads != 0, dh unsupported ... */
  PTDIT_ERR_DIVISIBILITY = -3,  /* the proxy window does not divide the grid */
  PTDIT_ERR_DTYPE = -4,         /* unsupported dtype combination */
  PTDIT_ERR_ALIGN = -5,         /* a pointer is not 16-byte aligned */
  PTDIT_ERR_WORKSPACE = -6,     /* workspace missing or smaller than required */
  PTDIT_ERR_HIP = -7,           /* a kernel launch failed */
  PTDIT_ERR_ALIAS = -8,         /* output overlaps an input or the workspace */
  PTDIT_ERR_SCRATCH = -9        /* the no-allocation entry point's static scratch is too small */
} ptdit_status;

/* Token grid of one call: batch B, frames F, height H, width W (N = F*H*W),
 * model width D split into `heads` heads. */
typedef struct { int32_t B, F, H, W, D, heads; } ptdit_grid;

/* A 3D extent (proxy window, TCM window or shift) along (t, h, w). */
typedef struct { int32_t t, h, w; } ptdit_win3;

/* Weights of one attention module (layout in the header comment).
 * w_qkv_packed is optional (NULL: none): a copy of w_qkv that
 * ptdit_pack_window_weights wrote. The window calls (ptdit_window_sa,
 * ptdit_shift_window_sa, ptdit_window_sa_keep) then read it instead of
 * packing w_qkv into their workspace at every call; it must be the packing
 * of this very w_qkv (not checked: repack after changing the weights). The
 * other calls ignore it. */
typedef struct {
  const void* w_qkv;
  const void* b_qkv;
  const void* w_o;
  const void* b_o;
  const void* w_qkv_packed;
} ptdit_attn_w;

/* Operation codes for ptdit_workspace_bytes. */
typedef enum {
  PTDIT_OP_PROXY_SA = 0,
  PTDIT_OP_PROXY_XATTN = 1,
  PTDIT_OP_WINDOW_SA = 2,
  PTDIT_OP_SHIFT_WINDOW_SA = 3,
  PTDIT_OP_MLP = 4
} ptdit_op;

/*
 * ptdit_linear -- one projection, y = x W^T + b (+ residual).
 * Source: the Q/K/V/O linear maps inside every attention module of the code
 * correspondence table (proxy_attn1, pvisual_attn2, linear_1_visual, attn1).
 *   x        [rows][d_in], dtype x_dt
 *   w        [d_out][d_in], dtype = prec;  b: [d_out] (prec) or NULL
 *   residual [rows][d_out], dtype r_dt, or NULL (no residual)
 *   y        [rows][d_out], dtype y_dt
 * Requires rows >= 0, d_in and d_out positive multiples of 8.
 */
ptdit_status ptdit_linear(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in,
                          int32_t d_out, const void* w, const void* b,
                          const void* residual, ptdit_dtype r_dt,
                          void* y, ptdit_dtype y_dt, ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_proxy_pool -- Averaging(z_s) of Eq. GIIM (section 3, "Method"; the
 * get_proxy_token(..., mode="mean") row of the code-correspondence table).
 *   x        [B][N][D], dtype x_dt (BF16 or F32)
 *   proxies  [B][M][D], dtype out_dt (BF16 or F32)
 * Proxy (T, I, J) is the average of tokens (T*p_t+dt, I*p_h+di, J*p_w+dj).
 * Arithmetic (fixed, bit-reproducible): fp32 sums; for every (dt, di) the
 * row sum over dj is taken in index order; row sums are added over di in
 * index order; plane sums over dt in index order; then one IEEE fp32
 * division by p_t*p_h*p_w; a bf16 output is rounded to nearest, ties even.
 * Requires p to divide (F, H, W) (else PTDIT_ERR_DIVISIBILITY), D % 8 == 0.
 */
ptdit_status ptdit_proxy_pool(const void* x, ptdit_dtype x_dt, ptdit_grid g, ptdit_win3 p,
                              void* proxies, ptdit_dtype out_dt, hipStream_t stream);

/* MLP weights (nn.Linear layout): w1 [hidden][D], b1 [hidden], w2 [D][hidden],
 * b2 [D]; biases nullable; dtype as the projections' (bf16 unless prec F32). */
typedef struct {
  const void* w1;
  const void* b1;
  const void* w2;
  const void* b2;
} ptdit_mlp_w;

/*
 * ptdit_mlp -- the MLP of the PT-Block that follows the text cross-attention
 * (section 3: PT-Block = GIIM + TCM + text cross-attn + MLP; Figure 3):
 *   out = Lin(GELU(Lin(x; w1, b1)); w2, b2) (+ x when add_residual != 0),
 * GELU in its tanh form, 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))),
 * applied in fp32 to the first map's output before it is stored (bf16 with
 * PTDIT_BF16 precision, else fp32) in the workspace.
 *   x        [rows][D], dtype x_dt; x_lowp: optional bf16 copy of an fp32 x
 *            (read instead of x by the first map, bf16 precision only)
 *   out      [rows][D], dtype out_dt; out_lowp: optional bf16 copy of out
 *   ws       ptdit_workspace_bytes(PTDIT_OP_MLP, {rows,1,1,1,D,1}, hidden, ...)
 * Requires D % 8 == 0, hidden % 8 == 0. Errors as the attention calls.
 */
ptdit_status ptdit_mlp(const void* x, const void* x_lowp, ptdit_dtype x_dt, int64_t rows, int32_t D,
                       int32_t hidden, const ptdit_mlp_w* w, int32_t add_residual, void* out,
                       void* out_lowp, ptdit_dtype out_dt, void* ws, size_t ws_bytes, ptdit_dtype prec,
                       hipStream_t stream);

/*
 * ptdit_proxy_select -- proxy extraction by one token per window instead of
 * the average: the Top-Left and Random rows of the proxy-extraction ablation
 * (section 3, ablation notes) and get_proxy_token's mode "first"
 * (code-correspondence excerpt 1).
 *   x        [B][N][D], dtype x_dt (BF16 or F32)
 *   offsets  [B][M] int32 device array, or NULL for every window's top-left
 *            token. Proxy m = (T, I, J) of batch b is the token
 *            (T*p_t+dt, I*p_h+di, J*p_w+dj) with window-local offset
 *            o = (dt*p_h + di)*p_w + dj = offsets[b][m] mod P, P =
 *            p_t*p_h*p_w (any int32 is accepted; negative values wrap).
 *            Random proxies pass offsets the caller drew.
 *   proxies  [B][M][D], dtype out_dt: a copy of the selected tokens (bf16 to
 *            fp32 exact; fp32 to bf16 rounds to nearest, ties even).
 * Requires p to divide (F, H, W) (else PTDIT_ERR_DIVISIBILITY), D % 8 == 0.
 * Caller owns every buffer; proxies must not overlap x or offsets.
 */
ptdit_status ptdit_proxy_select(const void* x, ptdit_dtype x_dt, ptdit_grid g, ptdit_win3 p,
                                const int32_t* offsets, void* proxies, ptdit_dtype out_dt,
                                hipStream_t stream);

/*
 * ptdit_proxy_sa -- the proxy self-attention of GIIM (proxy_attn1 in the
 * code-correspondence table; excerpt 2 adds its input back):
 *   out = MHA(P, P) (+ P when add_residual != 0).
 *   proxies  [B][M][D], dtype p_dt;  out [B][M][D], dtype out_dt
 *   ws       workspace of ptdit_workspace_bytes(PTDIT_OP_PROXY_SA, ...) bytes
 */
ptdit_status ptdit_proxy_sa(const void* proxies, ptdit_dtype p_dt, int32_t B, int32_t M,
                            int32_t D, int32_t heads, const ptdit_attn_w* w,
                            int32_t add_residual, void* out, ptdit_dtype out_dt,
                            void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_proxy_sa_noalloc -- ptdit_proxy_sa without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as ptdit_proxy_sa; its
 * workspace is a static device array of PTDIT_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends (its device
 * address is looked up on the first call on a device). Requires
 * ptdit_workspace_bytes(PTDIT_OP_PROXY_SA, {B,1,1,M,D,heads}, M, ...) <=
 * PTDIT_NOALLOC_SCRATCH_BYTES, else PTDIT_ERR_SCRATCH (before any launch):
 * 32 MiB holds, e.g., B*M up to 3640 proxies of D = 1152 in bf16, 1820 in
 * fp32. Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must be ordered by
 * the caller. No scratch contents carry over between calls (every element
 * is written before it is read), so nothing is cleared.
 */
#define PTDIT_NOALLOC_SCRATCH_BYTES (32 << 20)
ptdit_status ptdit_proxy_sa_noalloc(const void* proxies, ptdit_dtype p_dt, int32_t B, int32_t M,
                                    int32_t D, int32_t heads, const ptdit_attn_w* w,
                                    int32_t add_residual, void* out, ptdit_dtype out_dt,
                                    ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_proxy_xattn -- CS(z_s, P') of Eq. GIIM (pvisual_attn2 followed by
 * linear_1_visual): every token is a query, the M attended proxies are keys
 * and values:  out = MHA(x, P') (+ x when add_residual != 0).
 *   x        [B][N][D], dtype x_dt;  proxies [B][M][D], dtype p_dt
 *   x_lowp   optional bf16 copy of an fp32 x, read by the query projection
 *   out      [B][N][D], dtype out_dt;  out_lowp: optional bf16 copy of out
 * The same call serves the PT-Block's text cross-attention, with the caption
 * embeddings [B][L][D] in place of the proxies (M = L).
 */
ptdit_status ptdit_proxy_xattn(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                               const void* proxies, ptdit_dtype p_dt, int32_t M,
                               const ptdit_attn_w* w, int32_t add_residual,
                               void* out, void* out_lowp, ptdit_dtype out_dt,
                               void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_window_sa -- WSA of Eq. TCM (attn1 on window-grouped tokens):
 * attention inside each win.t x win.h x win.w window of the grid, the grid
 * being zero-padded at the high end of every axis to a multiple of the window
 * (pad tokens are zero vectors, so their keys/values are the biases; their
 * outputs are dropped):  out = WSA(x) (+ x when add_residual != 0).
 *   x, out   [B][N][D];  x_lowp, out_lowp: optional bf16 copies (see above)
 * Requires a window of 1 to 128 tokens (win.t*win.h*win.w <= 128, else
 * PTDIT_ERR_SHAPE); any such window is accepted.
 *   ws       ptdit_workspace_bytes(PTDIT_OP_WINDOW_SA, g, 0, win, prec) bytes:
 *            Q/K/V [B][3][heads][N][dh] and the attention output [B][N][D]
 *            (prec, each at a 256-byte boundary), then, for bf16, 3 D^2 bf16
 *            of scratch where the fused path packs w_qkv in its kernel's
 *            load order when w->w_qkv_packed is NULL (nothing is cached
 *            between calls; see ptdit_pack_window_weights).
 */
ptdit_status ptdit_window_sa(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                             ptdit_win3 win, const ptdit_attn_w* w, int32_t add_residual,
                             void* out, void* out_lowp, ptdit_dtype out_dt,
                             void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_pack_window_weights -- w_qkv [3D][D] (bf16) rewritten in the load
 * order of the window calls' fused Q/K/V-projection + attention kernel (the
 * module table's attn1, Eq. TCM): for each pair of heads and each 32-wide
 * slice of the contraction, the pair's 432 Q/K/V weight rows as one
 * contiguous run, so the kernel reads whole cache lines. The packed copy
 * (ptdit_window_packed_bytes(D, heads) bytes, caller-owned, 16-byte
 * aligned) goes into ptdit_attn_w.w_qkv_packed. PTDIT_ERR_SHAPE where the
 * fused kernel does not apply (head width other than 72, an odd head count,
 * D % 128 != 0); ptdit_window_packed_bytes then returns 0. Same values as
 * the packing each window call does in its workspace when no copy is given.
 */
size_t ptdit_window_packed_bytes(int32_t D, int32_t heads);
ptdit_status ptdit_pack_window_weights(const void* w_qkv, int32_t D, int32_t heads, void* packed,
                                       hipStream_t stream);

/*
 * ptdit_shift_window_sa -- SWSA of Eq. TCM (window_shift, window attention,
 * window_Ishift): the zero-padded grid is rolled by -shift
 * (z[k] = y[(k + s) mod L] per axis), window attention runs under the
 * boundary mask, the result is rolled back by +shift and cropped. Mask: per
 * axis of padded length L, window w, shift s, rolled coordinate k is in
 * region 0 if k < L-w, 1 if L-w <= k < L-s, 2 otherwise; a query sees a key
 * only if their regions agree on every axis. No data is moved for the roll:
 * the kernels address tokens through it.
 *   out = SWSA(x) (+ x when add_residual != 0); 0 <= shift < win per axis.
 */
ptdit_status ptdit_shift_window_sa(const void* x, const void* x_lowp, ptdit_dtype x_dt,
                                   ptdit_grid g, ptdit_win3 win, ptdit_win3 shift,
                                   const ptdit_attn_w* w, int32_t add_residual,
                                   void* out, void* out_lowp, ptdit_dtype out_dt,
                                   void* ws, size_t ws_bytes, ptdit_dtype prec,
                                   hipStream_t stream);

/*
 * ptdit_window_sa_keep -- ptdit_window_sa (shift 0) or ptdit_shift_window_sa
 * that leaves in the workspace what the backward pass of Eq. TCM reads, so a
 * training step need not recompute it: on return ws holds the head-major
 * Q/K/V [B][3][heads][N][dh] (prec, biases added, the real tokens) at offset
 * 0 and the attention output [B][N][D] (prec) at the next 256-byte boundary
 * (each call needs its own workspace for them to survive), the layout
 * ptdit_window_attn_bwd and ptdit_linear_bwd take. The same workspace size
 * (ptdit_workspace_bytes) and errors as the plain calls; the fused path writes
 * Q/K/V in addition to its output, the unfused one writes them anyway.
 */
ptdit_status ptdit_window_sa_keep(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                                  ptdit_win3 win, ptdit_win3 shift, const ptdit_attn_w* w, int32_t add_residual,
                                  void* out, void* out_lowp, ptdit_dtype out_dt, void* ws, size_t ws_bytes,
                                  ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_roll3d -- the 3D cyclic shift of window_shift / window_Ishift as a
 * stand-alone copy (the attention calls never materialise it):
 * inverse == 0: y[t,i,j] = x[(t+s_t) mod F, (i+s_h) mod H, (j+s_w) mod W];
 * inverse != 0: y[t,i,j] = x[(t-s_t) mod F, ...]. x, y: [B][N][D], dtype dt;
 * bit-exact copy. Requires 0 <= shift, D % 8 == 0, F*H*W <= 2^30, B*F*H and
 * the 16-byte vectors of one grid row (W*D*size/16) below 2^31 - 1024
 * (PTDIT_ERR_SHAPE otherwise); y must not overlap x (PTDIT_ERR_ALIAS).
 */
ptdit_status ptdit_roll3d(const void* x, ptdit_grid g, ptdit_win3 shift, int32_t inverse,
                          void* y, ptdit_dtype dt, hipStream_t stream);

/*
 * Backward pass of the attention core (Qihoo-T2X reading note, section 3
 * "Method": the gradients of Eq. GIIM's and Eq. TCM's attentions; the pages
 * train at 2048^2, section 4). With S = Q K^T / sqrt(dh), A = softmax(S) over
 * the allowed keys, O = A V and dO = dL/dO: dV = A^T dO, dS = A * (dO V^T -
 * rowsum(A * dO V^T)), dQ = dS K / sqrt(dh), dK = dS^T Q / sqrt(dh). The
 * softmax is recomputed from Q and K; nothing of the forward call is needed
 * but its Q/K/V. Inputs are bf16 or fp32 (dt, all alike); gradients are fp32.
 * Every output is written (not accumulated) unless stated; errors are
 * returned before anything is launched.
 *
 * ptdit_window_attn_bwd -- the core of ptdit_window_sa (shift 0) or
 * ptdit_shift_window_sa: the same windows, padding, roll and boundary mask.
 *   qkv      [B][3][heads][N][dh] device, dt: the Q/K/V of the forward call
 *            (the projections of x, head-major)
 *   b_qkv    [3D] device, dt, or NULL: the forward's projection bias; pad
 *            tokens' keys/values are b_k/b_v (zero when NULL)
 *   d_o      [B][N][D] device, dt: gradient of the attention output (the
 *            input of the output projection)
 *   d_qkv    [B][3][heads][N][dh] device, fp32: dQ, dK, dV of the real tokens
 *   d_b_kv   [2][D] device, fp32, or NULL: the gradients that reach pad key /
 *            value slots are ADDED here (d b_k, d b_v); required (else
 *            PTDIT_ERR_NULL) when the window does not divide the grid. Each
 *            (window, head) sums its pad slots' gradients on chip and adds
 *            the sum with one device atomic per channel, so the order of the
 *            additions across windows (and with it the last bits of d_b_kv)
 *            can differ from run to run; d_qkv is written without atomics
 *            and is the same in every run
 *   win, shift as for the forward call (window <= 128 tokens, shift < window).
 */
ptdit_status ptdit_window_attn_bwd(const void* qkv, const void* b_qkv, const void* d_o, ptdit_dtype dt,
                                   ptdit_grid g, ptdit_win3 win, ptdit_win3 shift, float* d_qkv,
                                   float* d_b_kv, hipStream_t stream);

/*
 * ptdit_window_attn_bwd_tokens -- ptdit_window_attn_bwd with dQ, dK, dV
 * written token-major: d_qkv_t [B][N][3D], element [b][t][g*D + h*dh + d]
 * for g = Q, K, V, the output gradient of the Q/K/V projection as
 * ptdit_linear_bwd reads it (so no layout pass sits between the two), in
 * d_qkv_dt: PTDIT_F32, or PTDIT_BF16 (round to nearest even; only with
 * dt == PTDIT_BF16, else PTDIT_ERR_DTYPE), half the bytes to write and to
 * read back, and the precision the projection's gradient products take their
 * operands in anyway. Everything else, the padding / bias gradients (fp32)
 * and the errors as ptdit_window_attn_bwd.
 */
ptdit_status ptdit_window_attn_bwd_tokens(const void* qkv, const void* b_qkv, const void* d_o, ptdit_dtype dt,
                                          ptdit_grid g, ptdit_win3 win, ptdit_win3 shift, void* d_qkv_t,
                                          ptdit_dtype d_qkv_dt, float* d_b_kv, hipStream_t stream);

/*
 * ptdit_attn_bwd -- the core of ptdit_proxy_sa (queries = keys = proxies) or
 * ptdit_proxy_xattn (queries = tokens, keys = proxies), unmasked.
 *   q        batch b at q + b*q_bstride elements: [heads][Nq][dh], dt
 *   k, v     batch b at k / v + b*kv_bstride: [heads][Nk][dh], dt
 *            (so the fused [B][3][heads][M][dh] and [B][2][heads][M][dh]
 *            buffers of the forward calls are addressed in place)
 *   d_o      [B][Nq][heads*dh] device, dt
 *   d_q      batch b at d_q + b*dq_bstride: [heads][Nq][dh], fp32
 *   d_k, d_v batch b at + b*dkv_bstride: [heads][Nk][dh], fp32
 *   ws       ptdit_attn_bwd_workspace_bytes(...) bytes of device memory
 *   dh 64 or 72; B*heads <= 65535; every pointer 16-byte aligned; the
 *   outputs overlap neither the inputs nor each other nor ws (PTDIT_ERR_ALIAS;
 *   batch blocks with one stride are compared block by block, so d_q, d_k,
 *   d_v may be interleaved views of one [B][3][heads][L][dh] gradient buffer).
 */
ptdit_status ptdit_attn_bwd(const void* q, int64_t q_bstride, const void* k, const void* v,
                            int64_t kv_bstride, const void* d_o, ptdit_dtype dt, int32_t B, int32_t heads,
                            int32_t Nq, int32_t Nk, int32_t dh, float* d_q, int64_t dq_bstride, float* d_k,
                            float* d_v, int64_t dkv_bstride, void* ws, size_t ws_bytes, hipStream_t stream);
size_t ptdit_attn_bwd_workspace_bytes(int32_t B, int32_t heads, int32_t Nq, int32_t Nk, int32_t dh);

/*
 * ptdit_attn_bwd_tokens -- ptdit_attn_bwd with dQ written token-major:
 * d_q_t [B][Nq][heads*dh], element [b][q][h*dh + d], the output gradient of
 * the query projection as ptdit_linear_bwd reads it (so no layout pass sits
 * between the two), in d_q_dt: PTDIT_F32, or PTDIT_BF16 (round to nearest
 * even; only with dt == PTDIT_BF16, else PTDIT_ERR_DTYPE). d_k, d_v, the
 * workspace and the errors as ptdit_attn_bwd.
 */
ptdit_status ptdit_attn_bwd_tokens(const void* q, int64_t q_bstride, const void* k, const void* v,
                                   int64_t kv_bstride, const void* d_o, ptdit_dtype dt, int32_t B, int32_t heads,
                                   int32_t Nq, int32_t Nk, int32_t dh, void* d_q_t, ptdit_dtype d_q_dt, float* d_k,
                                   float* d_v, int64_t dkv_bstride, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ptdit_proxy_pool_bwd -- gradient of the window average (Eq. GIIM's
 * Averaging): every token of a proxy window receives d_proxies[proxy] / P,
 * P = p_t*p_h*p_w (IEEE fp32 division). d_proxies [B][M][D] fp32, d_x
 * [B][N][D] fp32 (written, or added to when accumulate != 0); D % 4 == 0,
 * N <= 2^30, B*N <= 2^31 - 1 (else PTDIT_ERR_SHAPE); both pointers 16-byte
 * aligned; d_x must not overlap d_proxies (PTDIT_ERR_ALIAS).
 * The gradient of the roll is the inverse roll: ptdit_roll3d(inverse = 1).
 */
ptdit_status ptdit_proxy_pool_bwd(const float* d_proxies, ptdit_grid g, ptdit_win3 p, float* d_x,
                                  int32_t accumulate, hipStream_t stream);

/*
 * ptdit_linear_bwd -- gradients of a projection Y = X W^T + b (the Q/K/V/O
 * maps of every attention module; note, code-correspondence module table):
 * d_x = dY W, d_w = dY^T X, d_b = sum over rows of dY (all fp32, written).
 *   x     [rows][d_in] device, x_dt (the forward's input of the map)
 *   w     [d_out][d_in] device, bf16 (the forward's weight)
 *   d_y   [rows][d_out] device, dy_dt (gradient of the map's output)
 *   d_x   [rows][d_in] fp32 or NULL (skipped); d_w [d_out][d_in] fp32 or NULL;
 *   d_b   [d_out] fp32 or NULL
 *   ws    ptdit_linear_bwd_workspace_bytes(rows, d_in, d_out) bytes
 * The products run on bf16 matrix cores with fp32 accumulation (fp32 x or
 * d_y are rounded to bf16 as operands; d_b sums d_y in fp32): d_x on the
 * projection kernels with a transposed copy of w, d_w on the same kernels
 * with token-contiguous (transposed) copies of d_y and x, the token axis
 * split over workgroups and the parts summed in a fixed order.
 * d_in, d_out multiples of 8, rows <= 65535*32; every pointer 16-byte aligned; outputs overlap
 * neither the inputs nor each other nor ws (PTDIT_ERR_ALIAS).
 */
ptdit_status ptdit_linear_bwd(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in, int32_t d_out,
                              const void* w, const void* d_y, ptdit_dtype dy_dt, float* d_x, float* d_w,
                              float* d_b, void* ws, size_t ws_bytes, hipStream_t stream);
size_t ptdit_linear_bwd_workspace_bytes(int64_t rows, int32_t d_in, int32_t d_out);

/*
 * ptdit_linear_bwd_dw_group -- the weight and bias gradients of n (1 to
 * PTDIT_MAX_DW_GROUP) projections of one shape (module table: the Q/K/V/O
 * maps; training at 2048^2, section 4), dW_i = dY_i^T X_i, db_i = sum of
 * the rows of dY_i, in one GEMM launch whose token splits cover all n
 * products, so each product needs fewer splits (and partial sums) than a
 * ptdit_linear_bwd call of its own; the splits of each product are summed in
 * split order (deterministic). For the gradients a backward pass can leave
 * to its end, as the block backward does with its four D x D maps.
 *   x, d_y  host arrays of n device pointers: X_i [rows][d_in], dY_i
 *           [rows][d_out], bf16, token-major (row r = token r)
 *   d_w     host array of n device pointers, fp32 [d_out][d_in] each
 *   d_b     NULL, or a host array of n device pointers (fp32 [d_out], an
 *           entry may be NULL: that db is not formed)
 *   ws      ptdit_linear_bwd_dw_group_workspace_bytes(n, rows, d_in, d_out)
 * Requires rows % 32 == 0, 256 <= rows <= 65535*32, 1024 <= d_out <= 4096,
 * d_in <= 4096, both multiples of 8 (else PTDIT_ERR_SHAPE; the workspace
 * size is then 0); outputs overlapping an input, the workspace or another
 * output: PTDIT_ERR_ALIAS.
 */
#define PTDIT_MAX_DW_GROUP 4
size_t ptdit_linear_bwd_dw_group_workspace_bytes(int32_t n, int64_t rows, int32_t d_in, int32_t d_out);
ptdit_status ptdit_linear_bwd_dw_group(int32_t n, const void* const* x, const void* const* d_y, int64_t rows,
                                       int32_t d_in, int32_t d_out, float* const* d_w, float* const* d_b, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/*
 * ptdit_linear_bwd_ex -- ptdit_linear_bwd with the two steps that join a
 * projection's input gradient into a block's backward folded into the d_x
 * product (the residual branches of Eq. GIIM / Eq. TCM: x_out = x_in +
 * branch(x_in), so d x_in = d x_out + d branch):
 *   d_x_add  [rows][d_in] fp32 or NULL: added to d_x (d_x = d_y W + d_x_add);
 *            may be d_x itself (in place), else disjoint from every output;
 *            requires d_x (PTDIT_ERR_NULL), and d_x_bf16 is then the rounding
 *            of the sum
 *   d_x_bf16 [rows][d_in] bf16 or NULL: d_x rounded to bf16 (nearest even),
 *            the operand precision of the matrix-core attention backward
 * d_x may be NULL when d_x_bf16 is given (only the bf16 gradient is written).
 * Everything else, the workspace and the errors as ptdit_linear_bwd.
 */
ptdit_status ptdit_linear_bwd_ex(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in, int32_t d_out,
                                 const void* w, const void* d_y, ptdit_dtype dy_dt, float* d_x,
                                 const float* d_x_add, uint16_t* d_x_bf16, float* d_w, float* d_b, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * Calls that recompute forward intermediates and chain the backward calls
 * into the gradient of a whole block (section 3, Eq. GIIM and Eq. TCM; the
 * pages train at 2048^2, section 4). Errors as everywhere: host checks
 * before any launch, outputs untouched on failure.
 *
 * ptdit_linear_heads -- y = x W^T + b with the output head-major: the Q, K
 * and V maps of an attention module (module table) as the attention cores
 * read them. x [B*Ntok][D] (x_dt); w [groups*D][D], b [groups*D] or NULL
 * (prec); y [B][groups][heads][Ntok][D/heads] (prec). groups 1..3 (Q; K,V;
 * Q,K,V); D/heads 64 or 72.
 */
ptdit_status ptdit_linear_heads(const void* x, ptdit_dtype x_dt, int32_t B, int32_t Ntok, int32_t D,
                                int32_t groups, int32_t heads, const void* w, const void* b, void* y,
                                ptdit_dtype prec, hipStream_t stream);

/*
 * ptdit_window_attn -- the attention core of ptdit_window_sa (shift 0) or
 * ptdit_shift_window_sa on given head-major Q/K/V (Eq. TCM): the same
 * padding (pad keys/values = b_k/b_v), roll and boundary mask.
 *   qkv   [B][3][heads][N][dh] (dt);  b_qkv [3D] (dt) or NULL
 *   o     [B][N][D] (dt): the attention output, the output projection's input
 * Window 1..128 tokens, 0 <= shift < window per axis.
 */
ptdit_status ptdit_window_attn(const void* qkv, const void* b_qkv, ptdit_dtype dt, ptdit_grid g, ptdit_win3 win,
                               ptdit_win3 shift, void* o, hipStream_t stream);

/*
 * ptdit_attn -- the unmasked attention core of ptdit_proxy_sa / ptdit_proxy_xattn
 * (Eq. GIIM's SA and CS) on given head-major Q/K/V, addressed as for
 * ptdit_attn_bwd (q + b*q_bstride: [heads][Nq][dh]; k, v + b*kv_bstride:
 * [heads][Nk][dh]); o [B][Nq][heads*dh] (dt). ws: ptdit_attn_workspace_bytes
 * bytes (bf16 with more than 512 keys; else 0 and ws may be NULL).
 */
ptdit_status ptdit_attn(const void* q, int64_t q_bstride, const void* k, const void* v, int64_t kv_bstride,
                        ptdit_dtype dt, int32_t B, int32_t heads, int32_t Nq, int32_t Nk, int32_t dh, void* o,
                        void* ws, size_t ws_bytes, hipStream_t stream);
size_t ptdit_attn_workspace_bytes(int32_t B, int32_t heads, int32_t Nk, ptdit_dtype dt);

/*
 * ptdit_heads_to_tokens -- fp32 layout change dst[b][t][(g*heads + h)*dh + d]
 * = src[b][g][h][t][d]: the attention backward's dQ/dK/dV as the
 * token-major output gradient of a Q/K/V projection (ptdit_linear_bwd's d_y).
 * dh % 4 == 0; src and dst 16-byte aligned and disjoint.
 */
ptdit_status ptdit_heads_to_tokens(const float* src, int32_t B, int32_t groups, int32_t heads, int32_t Ntok,
                                   int32_t dh, float* dst, hipStream_t stream);

/* ptdit_f32_to_bf16 -- dst[i] = bf16(src[i]), round to nearest even (the
 * operand precision of the bf16 backward kernels); n % 8 == 0, disjoint. */
ptdit_status ptdit_f32_to_bf16(const float* src, int64_t n, void* dst, hipStream_t stream);

/* ptdit_add_f32 -- out[i] = a[i] + b[i] (fp32): a residual's gradient
 * joining its branch's; n % 4 == 0; out may be a or b itself, not a shifted
 * view of either (PTDIT_ERR_ALIAS). */
ptdit_status ptdit_add_f32(const float* a, const float* b, int64_t n, float* out, hipStream_t stream);

/*
 * Calibration (benchmark aid, no part of the method): the ceilings this box
 * sustains, to price kernels beside the published peaks.
 * ptdit_calibrate_mfma -- `blocks` workgroups of 4 waves issue `iters` x 8
 * independent v_mfma_f32_16x16x32_bf16 on register operands; *flop receives
 * the bf16 FLOP launched; out: blocks*256 floats (written, meaningless).
 * ptdit_calibrate_read -- streams `bytes` (% 16 == 0) of buf with 16-byte
 * loads over `blocks` workgroups of 256 threads; out: blocks*256 floats.
 * ptdit_calibrate_copy -- dst[i] = src[i] over `bytes` (% 16 == 0), one
 * 16-byte load and store per lane and step, consecutive lanes on consecutive
 * 16 bytes: a copy of known size whose hardware counter readings (bytes
 * fetched and written at the last-level cache) scale other kernels'
 * readings; src and dst must not overlap (PTDIT_ERR_ALIAS).
 * Time any of them with events on `stream`.
 */
ptdit_status ptdit_calibrate_mfma(int32_t blocks, int32_t iters, float* out, int64_t* flop, hipStream_t stream);
ptdit_status ptdit_calibrate_read(const void* buf, int64_t bytes, int32_t blocks, float* out, hipStream_t stream);
ptdit_status ptdit_calibrate_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Workspace bytes needed by an attention call (M: proxies; win: the TCM window,
 * ignored for the GIIM ops) or by ptdit_mlp (op PTDIT_OP_MLP, rows = g.B*g.F*
 * g.H*g.W, M: the hidden width). Returns 0 for invalid arguments, including a
 * TCM window the window calls reject (a non-positive extent or more than 128
 * tokens). The window calls' workspace holds the head-major Q/K/V and the
 * attention output; when the fused kernel runs (bf16 precision, bf16 x or
 * x_lowp, head width 72, an even head count, windows of 32, 64 or 128
 * tokens) only the attention-output part is used. */
size_t ptdit_workspace_bytes(ptdit_op op, ptdit_grid g, int32_t M, ptdit_win3 win,
                             ptdit_dtype prec);

/* Human-readable name of a status. Never NULL. */
const char* ptdit_status_str(ptdit_status st);

/* Library version string. */
const char* ptdit_version(void);

/*
 * Kernel trace (profiling aid, not thread-safe): after ptdit_trace_enable(k),
 * every launch of kernel class k (see ptdit_kernel_class) is bracketed by a
 * pair of HIP events recorded on the launch stream, up to `capacity` launches.
 * ptdit_trace_read waits for the recorded events and writes up to `max`
 * durations in milliseconds; it returns the count. ptdit_trace_disable frees
 * the events. Events are host-side HIP objects; no device memory is used.
 */
typedef enum {
  PTDIT_K_POOL = 0,
  PTDIT_K_GEMM_QKV = 1,      /* Q/K/V projection of the token rows for window attention */
  PTDIT_K_GEMM_OUT = 2,      /* output projections of the token rows (+ residual), ptdit_linear */
  PTDIT_K_ATTN_FLASH = 3,    /* proxy self-attention and cross-attention cores */
  PTDIT_K_ATTN_WINDOW = 4,   /* window / shifted-window attention cores */
  PTDIT_K_ROLL = 5,
  PTDIT_K_GEMM_Q = 6,        /* query projection of the token rows for cross-attention */
  PTDIT_K_GEMM_PROXY = 7,    /* every projection of the proxy rows */
  PTDIT_K_GEMM_MLP = 8,      /* both linear maps of the MLP */
  PTDIT_K_BWD_WINDOW = 9,    /* window attention backward */
  PTDIT_K_BWD_DENSE = 10,    /* proxy / cross-attention backward (all three kernels) */
  PTDIT_K_BWD_POOL = 11,     /* window-average backward */
  PTDIT_K_BWD_LINEAR = 12,   /* projection gradients (all kernels of ptdit_linear_bwd) */
  PTDIT_K_WINDOW_FUSED = 13  /* Q/K/V projection fused with window / shifted-window attention */
} ptdit_kernel_class;

ptdit_status ptdit_trace_enable(int32_t kernel_class, int32_t capacity);
int32_t ptdit_trace_read(float* ms, int32_t max);
void ptdit_trace_disable(void);

#ifdef __cplusplus
}
#endif

#endif /* PTDIT_H */
