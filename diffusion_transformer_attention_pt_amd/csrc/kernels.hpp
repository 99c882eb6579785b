// Host-side launch interface of the PT-DiT attention-core kernels.
// Internal to the library: api.cpp validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptdit {

// Y = A W^T + bias (+ R). A: [M][K], W: [N][K], bias: [N], R/Y: [M][N].
// head_major: Y is instead written as [b][N/D groups][heads][Ntok][dh] with
// row m = b*Ntok + tok and column n = g*D + h*dh + d (no residual then).
constexpr int GEMM_MAX_GROUPS = 4;

struct GemmDesc {
  const void* A; int a_f32;
  const void* W; const void* bias;
  const void* R; int r_f32;
  void* Y; int y_f32;
  void* Y2;  // optional bf16 copy of Y (token-major fp32 Y only), else nullptr
  int64_t M; int N; int K;
  int head_major; int64_t Ntok; int heads; int dh; int D;
  int act = 0;  // 1: GELU (tanh form) after the bias; token-major output without residual only
  // strided / split contraction (bf16 DMA kernels only): row strides of A and
  // W (0: K), and splits over blockIdx.y with per-split element offsets of
  // A, W (along their rows) and Y
  int64_t lda = 0, ldw = 0, ks_a = 0, ks_w = 0, ks_y = 0;
  int splits = 1;
  // token-major operands: A [K][lda] and W [K][ldw] with the contraction
  // index as their row (ks_a, ks_w in rows), bf16, fp32 Y (the weight
  // gradient dY^T X); k_last: K of the last split when it differs (0: K);
  // k_valid: the tokens of the last split that exist (0: all of its K)
  int tn = 0, k_last = 0, k_valid = 0;
  // token-major only: groups > 1 products of this shape, operands and
  // outputs at gA[g], gW[g], gY[g] (A, W, Y are then not read)
  // w_kmajor: W is [K][ldw] with the contraction index as its row (a weight
  // [d_out][d_in] for dX = dY W), read without a transposed copy
  int w_kmajor = 0;
  int groups = 1;
  const void* gA[GEMM_MAX_GROUPS] = {};
  const void* gW[GEMM_MAX_GROUPS] = {};
  void* gY[GEMM_MAX_GROUPS] = {};
};
hipError_t launch_gemm_bf16(const GemmDesc& d, hipStream_t s);  // W, bias bf16
hipError_t launch_gemm_f32(const GemmDesc& d, hipStream_t s);   // everything fp32

struct PoolDesc {
  const void* x; int x_f32;
  void* out; int out_f32;
  int B, F, H, W, D;
  int pt, ph, pw;
};
hipError_t launch_pool(const PoolDesc& d, hipStream_t s);
// one token per window: offsets [B][M] (window-local, taken mod P) or null
hipError_t launch_select(const PoolDesc& d, const int32_t* offsets, hipStream_t s);

struct RollDesc {
  const void* x; void* y; int f32;
  int B, F, H, W, D;
  int st, sh, sw;  // already reduced mod the extents, sign applied
};
hipError_t launch_roll(const RollDesc& d, hipStream_t s);

// softmax(Q K^T * scale) V per (batch, head). Q/K/V head-major:
// row r of head h in batch b at base + b*bs + h*hs + r*dh. O: [B][Nq][D].
struct FlashDesc {
  const void* Q; int64_t q_bs, q_hs;
  const void* K; int64_t k_bs, k_hs;
  const void* V; int64_t v_bs, v_hs;
  void* O;
  int B, heads, Nq, Nk, dh, D;
  float scale;
  void* vt = nullptr;     // scratch for packed V^T blocks (bf16, more than 512 keys)
  size_t vt_bytes = 0;
};
hipError_t launch_flash(const FlashDesc& d, int f32, hipStream_t s);
// bytes of FlashDesc::vt that a bf16 launch with Nk keys needs (0: none)
size_t flash_vt_bytes(int B, int heads, int Nk);

// Window attention on head-major QKV [B][3][heads][Ntok][dh] with the grid
// zero-padded to (Fp, Hp, Wp), rolled by -shift, partitioned into windows
// (wt, wh, ww) and masked by region labels. Pad tokens use bias_qkv (or 0).
struct WindowDesc {
  const void* QKV; const void* bias_qkv;
  void* O;
  int B, F, H, W, D, heads, dh;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  float scale;
};
hipError_t launch_window(const WindowDesc& d, int f32, hipStream_t s);

// Window / shifted-window attention with the Q/K/V projection fused in
// (wfused.hip): X [B][N][D] bf16 -> attention output O [B][N][D] bf16, the
// same windows, roll, padding and mask as launch_window. bf16 only, dh = 72,
// an even head count, windows of 32, 64 or 128 tokens, D % 128 == 0.
struct WFusedDesc {
  const void* X; const void* w_qkv; const void* b_qkv;
  void* O;
  void* qkv_out = nullptr;  // optional head-major Q/K/V [B][3][heads][N][dh] (the backward's copy)
  void* w_packed = nullptr; // wfused_packed_bytes(D) bytes: w_qkv in the kernel's DMA order (launch_wfused_pack)
  int B, F, H, W, D, heads, dh;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  float scale;
};
bool wfused_supported(const WFusedDesc& d);
// packed weights: launch_wfused_pack writes them from w_qkv into w_packed,
// launch_wfused reads them from there (stream order joins the two)
size_t wfused_packed_bytes(int D);
hipError_t launch_wfused_pack(const WFusedDesc& d, hipStream_t s);
hipError_t launch_wfused(const WFusedDesc& d, hipStream_t s);

// util.hip: chaining the backward calls
hipError_t launch_heads_to_tokens(const float* src, float* dst, int B, int G, int heads, int Ntok, int dh,
                                  hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);  // n % 8 == 0
hipError_t launch_add_f32(const float* a, const float* b, float* out, int64_t n, hipStream_t s);  // n % 4 == 0

// calib.hip: on-box ceilings for the benchmark
int64_t calib_mfma_flop(int blocks, int iters);
hipError_t launch_calib_mfma(int blocks, int iters, float* out, hipStream_t s);
hipError_t launch_calib_read(const void* buf, int64_t bytes, int blocks, float* out, hipStream_t s);
hipError_t launch_calib_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

// Backward pass of the attention core (fp32 gradients).
struct WindowBwdDesc {
  const void* QKV; const void* bias_qkv; const void* dO;
  void* dQKV; float* dbias_kv;
  int tokens_out = 0;  // 0: dQKV head-major [B][3][heads][N][dh]; 1: token-major [B][N][3D]
  int out_bf16 = 0;    // dQKV in bf16 (bf16 inputs only), else fp32
  int B, F, H, W, D, heads, dh;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  float scale;
};
hipError_t launch_window_bwd(const WindowBwdDesc& d, int f32, hipStream_t s);

struct DenseBwdDesc {
  const void *q, *k, *v, *dO;
  int64_t q_bs, kv_bs;
  void* dq; float *dk, *dv;
  int64_t dq_bs, dkv_bs;
  int dq_tok = 0;   // dQ token-major [B][Nq][D] (else head-major [B][heads][Nq][dh])
  int dq_bf16 = 0;  // dQ in bf16 (bf16 inputs only), else fp32
  float* stats;  // [B][heads][Nq][3]
  float* part;   // [chunks][B][heads][Nk][2][dh] (chunks > 1)
  int B, heads, Nq, Nk, D, dh, qchunk, chunks;
  float scale;
};
hipError_t launch_dense_bwd(const DenseBwdDesc& d, int f32, hipStream_t s);

struct PoolBwdDesc {
  const float* dP; float* dx;
  int B, F, H, W, D;
  int pt, ph, pw;
  int accumulate;
};
hipError_t launch_pool_bwd(const PoolBwdDesc& d, hipStream_t s);

// Projection gradients (linear_bwd.hip).
struct WgradDesc {
  const void* dy; int dy_f32;
  const void* x; int x_f32;
  uint16_t* dyt;  // [d_out][ld] bf16 (ld = splits * tch of wgrad_plan; needed when dw is set)
  uint16_t* xt;   // [d_in][ld] bf16 (needed when dw is set)
  uint16_t* dyb;  // optional row-major bf16 copy of dY [rows][d_out], written with dyt
  float* part;  // [splits][d_out][d_in] (needed when dw is set)
  float* dbp;   // [colsum_splits(rows)][d_out] (needed when db is set)
  float* dw;    // [d_out][d_in] or null
  float* db;    // [d_out] or null
  int64_t rows;
  int d_in, d_out;
};
void wgrad_plan(int64_t rows, int d_in, int d_out, int& splits, int64_t& tch, int groups = 1);
// dW (and db) of n <= GEMM_MAX_GROUPS products of one shape, token-major bf16
// dY and X (wgrad_token_major), in one GEMM launch split over the tokens for
// all of them, then per product the column sums and the split-order reduction
struct WgradGroupDesc {
  int n;
  const void* dy[GEMM_MAX_GROUPS];  // bf16 [rows][d_out]
  const void* x[GEMM_MAX_GROUPS];   // bf16 [rows][d_in]
  float* dw[GEMM_MAX_GROUPS];       // [d_out][d_in]
  float* db[GEMM_MAX_GROUPS];       // [d_out] or null
  void* ws;                         // wgrad_group_ws_bytes
  int64_t rows;
  int d_in, d_out;
};
size_t wgrad_group_ws_bytes(int n, int64_t rows, int d_in, int d_out);
hipError_t launch_wgrad_group(const WgradGroupDesc& d, hipStream_t s);
int colsum_splits(int64_t rows);
// dW from token-major bf16 dY and X directly (no transposed copies)
bool wgrad_token_major(int64_t rows, int d_in, int d_out, int dy_f32, int x_f32);
hipError_t launch_transpose_bf16(const void* w, void* wt, int rows, int cols, hipStream_t s);
hipError_t launch_wgrad_operands(const WgradDesc& d, hipStream_t s);  // the transposed copies (and dyb)
hipError_t launch_wgrad(const WgradDesc& d, hipStream_t s);           // then dW from them, and db

}  // namespace ptdit
