// Projections of the PT-DiT attention core: Y = A W^T + b (+ residual).
//
// bf16 path: MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation. A workgroup
// computes a BM x BN tile with WM x WN waves; K advances in steps of 64 through
// a double-buffered LDS stage (one barrier per step, next step's global loads
// in flight during the MFMAs). LDS rows are 64 bf16 = 8 chunks of 16 bytes;
// chunk c of row r sits at slot c ^ (r & 7), so the 16 rows read by one MFMA
// operand fetch hit distinct banks.
//
// The MFMA is issued with the weight tile as its first operand and the
// activation tile as its second, so each lane's four accumulators are four
// consecutive OUTPUT COLUMNS of one row: the epilogue adds bias / residual and
// stores 4 contiguous values per lane, both for row-major outputs and for the
// head-major Q/K/V layout [b][group][head][token][dh] (dh % 4 == 0).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace ptdit {

struct GemmParams {
  const void* A;
  const uint16_t* W;
  const uint16_t* bias;
  const void* R;
  void* Y;
  uint16_t* Y2;  // optional bf16 copy of an fp32 token-major Y (same rounding as A operands)
  int64_t M;
  int N, K;
  int64_t Ntok;
  int heads, dh, D;
  int act;  // 1: GELU after the bias (token-major, no residual)
  // row strides of A and W (elements; K for dense operands) and, for a
  // contraction split over blockIdx.y, the per-split offsets of A, W (along
  // their rows) and Y (elements); splits = gridDim.y. The DMA kernels only.
  int64_t lda, ldw, ks_a, ks_w, ks_y;
  int splits;
  // token-major operands (gemm_pp_kernel TN instance): K of the last split
  // when it differs from K (0: the same; a multiple of 128), and the tokens of
  // that split that exist (0: all); the rows past them read as zero
  int k_last;
  int k_valid;
  // token-major instance only: `groups` products of one shape whose A, W
  // and Y bases are gA[g], gW[g], gY[g] (groups == 1: A, W, Y)
  int groups;
  const void* gA[GEMM_MAX_GROUPS];
  const void* gW[GEMM_MAX_GROUPS];
  void* gY[GEMM_MAX_GROUPS];
};

// XCD-aware tile order: hardware hands block i to XCD (i % 8); re-number so
// each XCD walks a contiguous range of logical tiles, then group GM row panels
// together so a panel of A and a band of W stay hot in that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int nb, int tiles_m, int tiles_n, int GM,
                                            int& tm, int& tn) {
  const int q = nb >> 3, rem = nb & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  const int logical = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
  const int group_size = GM * tiles_n;
  const int g = logical / group_size;
  const int first_m = g * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = logical - g * group_size;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Raw global->register staging of one 16-byte LDS chunk (8 elements of A).
// fp32 sources keep their 32 raw bytes until the LDS store, so the global
// loads stay in flight across the MFMAs instead of being waited on for the
// conversion.
template <typename TA> struct Stage;
template <> struct Stage<uint16_t> {
  uint4 v;
  __device__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ void zero() { v = uint4{0, 0, 0, 0}; }
  __device__ uint4 bf16() const { return v; }
};
template <> struct Stage<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ void zero() { a = b = float4{0.f, 0.f, 0.f, 0.f}; }
  __device__ uint4 bf16() const {
    return uint4{pack_bf2(a.x, a.y), pack_bf2(a.z, a.w), pack_bf2(b.x, b.y), pack_bf2(b.z, b.w)};
  }
};

// Pipeline (one barrier per 64-wide k step, LDS double buffer, register
// double buffer of MFMA fragments):
//   issue global loads of step kt+1 into staging registers
//   read fragments (kt, k 32..63)            | MFMAs on fragments (kt, k 0..31)
//   write staging registers to the other LDS buffer; barrier
//   read fragments (kt+1, k 0..31)           | MFMAs on fragments (kt, k 32..63)
// A buffer is rewritten one iteration after its last read, and every read of
// it completed before the barrier that separates the two.
template <typename TA, typename TR, typename TY, int BM, int BN, int WM, int WN, bool HEADMAJOR,
          bool KFULL>
__global__ void __launch_bounds__(WM* WN * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int ACH = BM * 8 / NT, WCH = BN * 8 / NT;
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile/thread mismatch");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");

  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (p.N + BN - 1) / BN;
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;  // grid larger than the tile count
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const TA* A = reinterpret_cast<const TA*>(p.A);
  const int K = p.K;
  const int KT = (K + 63) / 64;

  // Thread t stages chunk c = t % 8 of rows r0 + i * RS (i < ACH for A, i < WCH for W).
  // Rows past the edge are clamped: loaded but never stored.
  constexpr int RS = NT / 8;
  const int r0 = tid >> 3, c8 = (tid & 7) * 8;

  Stage<TA> ra[ACH];
  Stage<uint16_t> rw[WCH];
  auto gload = [&](int kt) {
    const int k = kt * 64 + c8;
    const bool ok = KFULL || k < K;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      int64_t gm = m0 + r0 + i * RS;
      gm = gm < p.M ? gm : p.M - 1;
      if (ok) ra[i].load(A + gm * K + k);
      else ra[i].zero();
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int gn = n0 + r0 + i * RS;
      gn = gn < p.N ? gn : p.N - 1;
      if (ok) rw[i].load(p.W + (int64_t)gn * K + k);
      else rw[i].zero();
    }
  };
  auto lstore = [&](int buf) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int row = r0 + i * RS;
      lds[buf][row * 8 + (c ^ (row & 7))] = ra[i].bf16();
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int row = r0 + i * RS;
      lds[buf][(BM + row) * 8 + (c ^ (row & 7))] = rw[i].bf16();
    }
  };
  // fragments of k sub-step kk (0: k 0..31, 1: k 32..63); (row & 7) == (lane & 7)
  auto lfrag = [&](int buf, int kk, uint4* wf, uint4* xf) {
    const int sw = (kk * 4 + (lane >> 4)) ^ (lane & 7);
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[i] = lds[buf][(BM + wn * TN + i * 16 + (lane & 15)) * 8 + sw];
#pragma unroll
    for (int j = 0; j < FM; ++j) xf[j] = lds[buf][(wm * TM + j * 16 + (lane & 15)) * 8 + sw];
  };

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = zero4();
  auto mma = [&](const uint4* wf, const uint4* xf) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_bf16(wf[i], xf[j], acc[i][j]);
  };

  uint4 w0[FN], x0[FM], w1[FN], x1[FM];
  gload(0);
  lstore(0);
  __syncthreads();
  lfrag(0, 0, w0, x0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) gload(kt + 1);
    lfrag(buf, 1, w1, x1);
    mma(w0, x0);
    if (more) lstore(buf ^ 1);
    __syncthreads();
    if (more) lfrag(buf ^ 1, 0, w0, x0);
    mma(w1, x1);
  }

  // Epilogue: lane holds C[m][n .. n+3].
  TY* Y = reinterpret_cast<TY*>(p.Y);
  const TR* R = reinterpret_cast<const TR*>(p.R);
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * TN + i * 16 + 4 * (lane >> 4);
    if (n >= p.N) continue;
    float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
    if (p.bias) {
      const float4 bv = load4f(p.bias + n);
      b0 = bv.x; b1 = bv.y; b2 = bv.z; b3 = bv.w;
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * TM + j * 16 + (lane & 15);
      if (m >= p.M) continue;
      float v0 = acc[i][j][0] + b0, v1 = acc[i][j][1] + b1;
      float v2 = acc[i][j][2] + b2, v3 = acc[i][j][3] + b3;
      if (p.act) {
        v0 = gelu_tanh(v0); v1 = gelu_tanh(v1); v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
      }
      if constexpr (HEADMAJOR) {
        const int g = n / p.D, hn = n - g * p.D;
        const int h = hn / p.dh, d = hn - h * p.dh;
        const int64_t b = m / p.Ntok, tok = m - b * p.Ntok;
        const int G = p.N / p.D;
        const int64_t off = (((b * G + g) * p.heads + h) * p.Ntok + tok) * p.dh + d;
        store4(Y + off, v0, v1, v2, v3);
      } else {
        const int64_t off = m * p.N + n;
        if (R) {
          const float4 r = load4f(R + off);
          v0 += r.x; v1 += r.y; v2 += r.z; v3 += r.w;
        }
        store4(Y + off, v0, v1, v2, v3);
        if constexpr (sizeof(TY) == 4)
          if (p.Y2) store4(p.Y2 + off, v0, v1, v2, v3);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Multi-stage variant: global -> LDS directly (global_load_lds_dwordx4), no
// staging registers, a ring of STAGES k-slices of 32 with STAGES-1 in flight.
//
// A DMA instruction moves 64 lanes x 16 bytes into 1 KB of LDS at a
// wave-uniform base, lane l landing at base + 16*l. The swizzle is therefore
// applied on the global side: LDS slot (row, p) receives global chunk
// c = p ^ swz(row), so fragment reads (16 rows, one chunk each) stay
// conflict-free:
//   bf16 rows (32 values = 4 chunks):  c = p ^ ((row >> 1) & 3)
//   fp32 rows (32 values = 8 chunks):  c = p ^ (row & 7); a fragment of 8
//   values is two chunks, converted to bf16 (v_cvt_pk_bf16_f32) after the read.
// Per k-slice each wave waits until its own loads for the slice have landed
// (s_waitcnt vmcnt), then one barrier publishes the slice to all waves and
// retires every read of the slot about to be refilled.
// ----------------------------------------------------------------------------

// Per-wave DMA plan of one k-slice of a BM x BN tile: instruction j moves 64
// 16-byte chunks (A rows for j < IA, W rows after); wave w owns j = w + i*NW.
// A wave with fewer than MAXI real instructions repeats its first one (same
// source, same LDS bytes), so every wave issues exactly MAXI per slice: the
// loops then have no wave-dependent branch and vmcnt targets are constants.
// Addresses are a wave-uniform base (the tile's first A or W row, in SGPRs)
// plus a 32-bit per-lane byte offset, so the DMA takes the saddr + voffset
// form and each instruction holds one VGPR.
template <typename TA, int BM, int BN, int NW>
struct DmaPlan {
  static constexpr int CA = DmaA<TA>::CPR;
  static constexpr int SA = BM * CA, SB = BN * 4;   // 16-byte slots per stage
  static constexpr int IA = SA / 64, IB = SB / 64, IT = IA + IB;
  static constexpr int MAXI = (IT + NW - 1) / NW;  // per wave, upper bound
  static_assert(SA % 64 == 0 && SB % 64 == 0, "stage must be whole DMA instructions");

  const char* a_base;
  const char* w_base;
  bool is_a[MAXI];
  uint32_t voff[MAXI];
  int dst[MAXI];

  __device__ __forceinline__ void init(const GemmParams& p, int64_t m0, int n0, int wave, int lane, int split_) {
    const int64_t lda = p.lda, ldw = p.ldw, split = split_;
    a_base = reinterpret_cast<const char*>(reinterpret_cast<const TA*>(p.A) + m0 * lda + split * p.ks_a);
    w_base = reinterpret_cast<const char*>(p.W + (int64_t)n0 * ldw + split * p.ks_w);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j0 = wave + i * NW;
      const int j = j0 < IT ? j0 : wave;
      is_a[i] = j < IA;
      if (j < IA) {
        const int sl = j * 64 + lane, row = sl / CA, pp = sl % CA;
        const int r = m0 + row < p.M ? row : (int)(p.M - 1 - m0);
        voff[i] = (uint32_t)(((int64_t)r * lda + DmaA<TA>::chunk(row, pp) * (16 / (int)sizeof(TA))) *
                             (int)sizeof(TA));
        dst[i] = j * 64;
      } else {
        const int sl = (j - IA) * 64 + lane, row = sl / 4, pp = sl % 4;
        const int r = n0 + row < p.N ? row : p.N - 1 - n0;
        voff[i] = (uint32_t)(((int64_t)r * ldw + (pp ^ ((row >> 1) & 3)) * 8) * 2);
        dst[i] = SA + (j - IA) * 64;
      }
    }
  }
  __device__ __forceinline__ void issue(int kt, uint4* st) const {
    const char* const ak = a_base + kt * (32 * (int)sizeof(TA));
    const char* const wk = w_base + kt * 64;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) PTDIT_GLDS16((is_a[i] ? ak : wk) + voff[i], st + dst[i]);
  }
  __device__ __forceinline__ void issue_head(int kt, uint4* st) const { issue(kt, st); }
};

// Token-major operands: the weight gradient dW = dY^T X contracts over the
// token index t, which is the row index of both dY [T][d_out] and X [T][d_in].
// A k-slice is 32 token rows x the tile's columns, staged as it lies in
// memory, in LDS rows of TN_CPR = 36 16-byte chunks (a 288-column W tile; a
// 256-column A tile leaves 4 chunks of a row unused, loaded with a copy of a
// real chunk). Token row r's chunk c sits at position c ^ (2 * ((r >> 3) & 1)):
// with the 576-byte pitch rows r .. r+3 start 64 bytes apart in the banks and
// the XOR moves rows 8 apart by 32 bytes, so the 8 rows x 32 bytes that a
// half-wave of one transposing read touches fall in distinct banks.
// Fragments are then read with ds_read_b64_tr_b16 (see tn_frag).
constexpr int TN_CPR = 36;
__device__ __forceinline__ int tn_pos(int row, int c) { return c ^ (2 * ((row >> 3) & 1)); }
// zeros in device memory (static storage, never written): 32 rows of up to
// TN_ZERO_LD elements (so a slice's per-lane offsets stay inside it). The
// final split, when its real tokens (k_valid) are fewer than its K (k_last,
// a multiple of 128), starts k_last - k_valid tokens early, so that it ends
// at the last token, and its first (k_last - k_valid) / 32 <= 3 k-slices
// (tokens of the split before it) read these zeros instead: they are issued
// in the prologue only, so the main loop carries no check.
constexpr int TN_ZERO_LD = 4096;
__device__ __attribute__((aligned(16))) uint16_t tn_zero_slice[32 * TN_ZERO_LD];

template <int BM, int BN, int NW>
struct DmaPlanTN {
  static_assert(BM <= 8 * TN_CPR && BN <= 8 * TN_CPR, "tile columns fit an LDS row");
  static constexpr int SA = 32 * TN_CPR, SB = 32 * TN_CPR;  // 16-byte slots per stage
  static constexpr int IA = SA / 64, IB = SB / 64, IT = IA + IB;
  static constexpr int MAXI = (IT + NW - 1) / NW;

  const char* a_base;
  const char* w_base;
  int64_t a_step, w_step;  // bytes per k-slice (32 token rows)
  int nz;                  // leading k-slices that read zeros (final split; <= 3)
  bool is_a[MAXI];
  uint32_t voff[MAXI];
  int dst[MAXI];

  __device__ __forceinline__ void init(const GemmParams& p, int64_t m0, int n0, int wave, int lane, int split_) {
    const int64_t lda = p.lda, ldw = p.ldw, split = split_;
    const bool last = split_ == p.splits - 1 && p.k_valid > 0;
    const int kl = p.k_last > 0 ? p.k_last : p.K;
    nz = last ? (kl - p.k_valid) / 32 : 0;
    const int64_t t0a = split * p.ks_a - 32 * nz, t0w = split * p.ks_w - 32 * nz;  // first token row
    a_base = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(p.A) + t0a * lda + m0);
    w_base = reinterpret_cast<const char*>(p.W + t0w * ldw + n0);
    a_step = 64 * lda;
    w_step = 64 * ldw;
    // real chunks of the tile's columns (M, N multiples of 8); positions past
    // them (row padding, a ragged last tile) load the last real chunk
    const int ca = (int)(p.M - m0 < BM ? (p.M - m0) / 8 : BM / 8);
    const int cw = p.N - n0 < BN ? (p.N - n0) / 8 : BN / 8;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j0 = wave + i * NW;
      const int j = j0 < IT ? j0 : wave;
      is_a[i] = j < IA;
      const int sl = (j < IA ? j : j - IA) * 64 + lane, row = sl / TN_CPR, pos = sl % TN_CPR;
      int c = tn_pos(row, pos);  // the chunk stored at pos (the map is its own inverse)
      const int cmax = j < IA ? ca : cw;
      if (c >= cmax) c = cmax - 1;
      voff[i] = (uint32_t)(((int64_t)row * (j < IA ? lda : ldw) + 8 * c) * 2);
      dst[i] = j < IA ? j * 64 : SA + (j - IA) * 64;
    }
  }
  __device__ __forceinline__ void issue(int kt, uint4* st) const {
    const char* const ak = a_base + kt * a_step;
    const char* const wk = w_base + kt * w_step;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) PTDIT_GLDS16((is_a[i] ? ak : wk) + voff[i], st + dst[i]);
  }
  // the prologue's slices 0..2: the final split's leading nz slices read the
  // zero region (offsets row * ld + column, ld <= TN_ZERO_LD, stay inside it)
  __device__ __forceinline__ void issue_head(int kt, uint4* st) const {
    const bool z = kt < nz;
    const char* const zero = reinterpret_cast<const char*>(tn_zero_slice);
    const char* const ak = z ? zero : a_base + kt * a_step;
    const char* const wk = z ? zero : w_base + kt * w_step;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) PTDIT_GLDS16((is_a[i] ? ak : wk) + voff[i], st + dst[i]);
  }
};

// Row-major bf16 A (as DmaPlan) with a k-major W: W [K][ldw] stored with the
// contraction index as its row, the way a weight [d_out][d_in] lies for
// dX = dY W (K = d_out). W's k-slice is 32 rows x the tile's columns, staged
// as it lies (the token-major layout of DmaPlanTN, read with tn_frag), so the
// product needs no transposed copy of the weight.
template <int BM, int BN, int NW>
struct DmaPlanMix {
  static_assert(BN <= 8 * TN_CPR, "tile columns fit an LDS row");
  static constexpr int SA = BM * 4, SB = 32 * TN_CPR;  // 16-byte slots per stage
  static constexpr int IA = SA / 64, IB = SB / 64, IT = IA + IB;
  static constexpr int MAXI = (IT + NW - 1) / NW;
  static_assert(SA % 64 == 0 && SB % 64 == 0, "stage must be whole DMA instructions");

  const char* a_base;
  const char* w_base;
  int w_step;  // bytes per 32 rows of W
  bool is_a[MAXI];
  uint32_t voff[MAXI];
  int dst[MAXI];

  __device__ __forceinline__ void init(const GemmParams& p, int64_t m0, int n0, int wave, int lane, int) {
    const int64_t lda = p.lda, ldw = p.ldw;
    a_base = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(p.A) + m0 * lda);
    w_base = reinterpret_cast<const char*>(p.W + n0);
    w_step = (int)(64 * ldw);
    const int cw = p.N - n0 < BN ? (p.N - n0) / 8 : BN / 8;  // real 8-column chunks of the tile
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j0 = wave + i * NW;
      const int j = j0 < IT ? j0 : wave;
      is_a[i] = j < IA;
      if (j < IA) {
        const int sl = j * 64 + lane, row = sl / 4, pp = sl % 4;
        const int r = m0 + row < p.M ? row : (int)(p.M - 1 - m0);
        voff[i] = (uint32_t)(((int64_t)r * lda + DmaA<uint16_t>::chunk(row, pp) * 8) * 2);
        dst[i] = j * 64;
      } else {
        const int sl = (j - IA) * 64 + lane, row = sl / TN_CPR, pos = sl % TN_CPR;
        int c = tn_pos(row, pos);  // the chunk stored at pos (the map is its own inverse)
        if (c >= cw) c = cw - 1;   // row padding / a ragged last tile: a real chunk, never stored
        voff[i] = (uint32_t)(((int64_t)row * ldw + 8 * c) * 2);
        dst[i] = SA + (j - IA) * 64;
      }
    }
  }
  __device__ __forceinline__ void issue(int kt, uint4* st) const {
    const char* const ak = a_base + kt * 64;
    const char* const wk = w_base + kt * w_step;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) PTDIT_GLDS16((is_a[i] ? ak : wk) + voff[i], st + dst[i]);
  }
  __device__ __forceinline__ void issue_head(int kt, uint4* st) const { issue(kt, st); }
};

// Fragment of a token-major operand: lane (i = lane % 16, g = lane / 16)
// needs fragment row col0 + 16 j + i at k = 8 g .. 8 g + 7, i.e. LDS token
// rows 8 g .. 8 g + 7 of one column. A transposing read (ds_read_b64_tr_b16)
// in which lane l of a 16-lane group points at token row R + (l >> 2),
// columns C + 4 (l & 3) .. +3 returns to lane i the column C + i at token
// rows R .. R + 3 (the lane layout measured on gfx950); two such reads
// (R = 8 g and 8 g + 4) make the fragment. Byte address of the first read of
// fragment j: base + 32 j, base = bE for even j, bO for odd j (the chunk XOR
// moves a lane by +-32 bytes depending on the parity of the 16-column block);
// the second read is 4 rows (2304 bytes) further.
struct TnFragBase {
  int bE, bO;
  __device__ __forceinline__ void init(int region_bytes, int col0w, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int krow = 8 * g + (i >> 2), b = g & 1;  // (krow >> 3) & 1 == g & 1
    const int byte = region_bytes + krow * TN_CPR * 16 + ((col0w >> 3) + ((i & 3) >> 1)) * 16 + 8 * (i & 1);
    const int bp = byte + 32 * b, bm = byte - 32 * b;
    // block j's chunk pair has bit 1 = ((col0w >> 4) + j) & 1; with it set the
    // XOR moves the lane down by 32 bytes
    const bool P = ((col0w >> 4) & 1) != 0;
    bE = P ? bm : bp;
    bO = P ? bp : bm;
  }
};
__device__ __forceinline__ uint2 tn_read(const uint4* st, int byte) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  typedef __attribute__((address_space(3))) char* lds_char;
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)((lds_char)(st) + byte));
  return __builtin_bit_cast(uint2, r);
}
template <int J>
__device__ __forceinline__ uint4 tn_frag(const uint4* st, const TnFragBase& fb) {
  const int base = (J & 1) ? fb.bO : fb.bE;
  const uint2 lo = tn_read(st, base + 32 * J);
  const uint2 hi = tn_read(st, base + 32 * J + 4 * TN_CPR * 16);
  return uint4{lo.x, lo.y, hi.x, hi.y};
}

// Epilogue staging through the ring: band j = tile rows {wm*TM + j*16 + r},
// i.e. WM*16 rows x BN columns, row pitch padded by 16 bytes. A bf16 band
// fills one ring slot, an fp32 band two, so BPP = STAGES (bf16) or STAGES/2
// (fp32) bands are staged per pass.

typedef unsigned int ntu4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  ntu4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<ntu4*>(p));
}
template <typename TY, int BN, int WM, int STAGES>
struct EpiShape {
  static constexpr int PITCH = BN + 16 / (int)sizeof(TY);  // elements
  static constexpr int ROWS = WM * 16;
  static constexpr int ROWS_PER_SLOT = sizeof(TY) == 2 ? ROWS : ROWS / 2;
  static constexpr int SLOT = (ROWS_PER_SLOT * PITCH * (int)sizeof(TY) + 15) / 16;  // uint4
  static constexpr int BPP = sizeof(TY) == 2 ? STAGES : STAGES / 2;
  static_assert(BPP >= 1, "fp32 staging spans two slots");
};

// Epilogue through LDS: lane holds C[m][n .. n+3]; stage 16-row bands (bias
// added, converted to TY), then write whole 16-byte chunks in row order so a
// wave's stores cover long contiguous runs (rows of the tile are consecutive
// tokens; head-major chunks never straddle a head, dh % 8 == 0). The ring
// must be drained (no DMA in flight, every fragment read retired) on entry.
template <typename TR, typename TY, int BM, int BN, int WM, int WN, int STAGES, bool HEADMAJOR, class SlotFn>
__device__ __forceinline__ void ring_epilogue(const GemmParams& p, const floatx4 (&acc)[BN / WN / 16][BM / WM / 16],
                                              const uint2 (&biasp)[BN / WN / 16], SlotFn&& slot, int tid,
                                              int lane, int wm, int wn, int64_t m0, int n0, int split) {
  constexpr int NW = WM * WN, TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  using ES = EpiShape<TY, BN, WM, STAGES>;
  constexpr int BPP = ES::BPP;
  TY* Y = reinterpret_cast<TY*>(p.Y) + (int64_t)split * p.ks_y;
  const TR* R = reinterpret_cast<const TR*>(p.R);
  constexpr int E = 16 / (int)sizeof(TY);          // elements per 16-byte chunk
  constexpr int CPRO = BN / E;                     // chunks per staged row
  const int lr = lane & 15;

  // Store-phase chunk assignment, fixed across bands: chunk q = tid + i*NT of
  // a band is staged row sr = q / CPRO, chunk cc = q % CPRO (compile-time
  // divisors). Head-major column parts (divisions by runtime sizes) are
  // computed once here; rows advance by 16 per band, tracked as (batch,
  // token) without division. Token-major addresses are recomputed per store,
  // which keeps the registers of the (still live) accumulators free.
  constexpr int NQ = (ES::ROWS * CPRO + NW * 64 - 1) / (NW * 64);
  constexpr int NQH = HEADMAJOR ? NQ : 1;
  int64_t colpart[NQH];
  const int64_t b0 = m0 / p.Ntok;            // one division per thread
  const int64_t t0 = m0 - b0 * p.Ntok;
  const int G = p.N / p.D;
  const int64_t bstride = (int64_t)G * p.heads * p.Ntok * p.dh;
  if constexpr (HEADMAJOR) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = tid + i * NW * 64;
      const int cc = q - (q / CPRO) * CPRO;
      const int n = n0 + cc * E;
      const int gg = n / p.D, hn = n - gg * p.D;
      const int h = hn / p.dh, d = hn - h * p.dh;
      colpart[i] = ((int64_t)(gg * p.heads + h) * p.Ntok) * p.dh + d;
    }
  }

  // band j lives in slot (j % BPP) [bf16] or slots 2*(j % BPP), 2*(j % BPP)+1 [fp32]
  auto band_base = [&](auto jI, int sr) -> TY* {
    constexpr int jj = decltype(jI)::value % BPP;
    if constexpr (sizeof(TY) == 2) {
      return reinterpret_cast<TY*>(slot(std::integral_constant<int, jj>{}));
    } else {
      return sr < ES::ROWS_PER_SLOT ? reinterpret_cast<TY*>(slot(std::integral_constant<int, 2 * jj>{}))
                                    : reinterpret_cast<TY*>(slot(std::integral_constant<int, 2 * jj + 1>{}));
    }
  };
  static_for<0, (FM + BPP - 1) / BPP>([&](auto passI) {
    constexpr int pass = decltype(passI)::value;
    // stage bands pass*BPP .. pass*BPP+BPP-1
    static_for<0, BPP>([&](auto kI) {
      constexpr int jb = pass * BPP + decltype(kI)::value;
      if constexpr (jb < FM) {
        const int sr = wm * 16 + lr;
        TY* base = band_base(std::integral_constant<int, jb>{}, sr);
        const int lrow = sr % ES::ROWS_PER_SLOT;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int c = wn * TN + i * 16 + 4 * (lane >> 4);
          float v0 = acc[i][jb][0] + __uint_as_float(biasp[i].x << 16);
          float v1 = acc[i][jb][1] + __uint_as_float(biasp[i].x & 0xffff0000u);
          float v2 = acc[i][jb][2] + __uint_as_float(biasp[i].y << 16);
          float v3 = acc[i][jb][3] + __uint_as_float(biasp[i].y & 0xffff0000u);
          if (p.act) {
            v0 = gelu_tanh(v0); v1 = gelu_tanh(v1); v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
          }
          store4(base + lrow * ES::PITCH + c, v0, v1, v2, v3);
        }
      }
    });
    ring_barrier();
    static_for<0, BPP>([&](auto kI) {
      constexpr int jb = pass * BPP + decltype(kI)::value;
      if constexpr (jb < FM) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int q = tid + i * NW * 64;
          const int sr = q / CPRO, cc = q - (q / CPRO) * CPRO;
          const int rr = (sr / 16) * TM + (sr % 16) + jb * 16;
          const int n = n0 + cc * E;
          if (q >= ES::ROWS * CPRO || n >= p.N || m0 + rr >= p.M) continue;
          const TY* sb = band_base(std::integral_constant<int, jb>{}, sr);
          const uint4 v = *reinterpret_cast<const uint4*>(sb + (sr % ES::ROWS_PER_SLOT) * ES::PITCH + cc * E);
          if constexpr (HEADMAJOR) {
            int64_t tok = t0 + rr, b = b0;
            while (tok >= p.Ntok) { tok -= p.Ntok; ++b; }
            *reinterpret_cast<uint4*>(Y + b * bstride + colpart[HEADMAJOR ? i : 0] + tok * p.dh) = v;
          } else {
            const int64_t off = (m0 + rr) * p.N + n;
            if constexpr (sizeof(TY) == 4) {
              float4 o = __builtin_bit_cast(float4, v);
              if (R) {
                const float4 r = load4f(R + off);
                o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
              }
              st_nt16(Y + off, __builtin_bit_cast(uint4, o));
              if (p.Y2) store4(p.Y2 + off, o.x, o.y, o.z, o.w);
            } else if (R) {
              float f[8], rv[8];
              unpack8(v, f);
              const float4 r0 = load4f(R + off), r1 = load4f(R + off + 4);
              rv[0] = r0.x; rv[1] = r0.y; rv[2] = r0.z; rv[3] = r0.w;
              rv[4] = r1.x; rv[5] = r1.y; rv[6] = r1.z; rv[7] = r1.w;
#pragma unroll
              for (int e = 0; e < 8; ++e) f[e] += rv[e];
              *reinterpret_cast<uint4*>(Y + off) = pack8(f);
            } else {
              *reinterpret_cast<uint4*>(Y + off) = v;
            }
          }
        }
      }
    });
    if constexpr (pass + 1 < (FM + BPP - 1) / BPP) ring_barrier();  // staging reused by the next pass
  });
}

// bias of this lane's output columns (4 bf16 per 16-column tile), kept packed
template <int FN>
__device__ __forceinline__ void load_bias(const GemmParams& p, int ncol0, int lane, uint2 (&biasp)[FN]) {
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = ncol0 + i * 16 + 4 * (lane >> 4);
    biasp[i] = (p.bias && n < p.N) ? *reinterpret_cast<const uint2*>(p.bias + n) : uint2{0u, 0u};
  }
}

// Each ring slot is its own __shared__ array and every slot index is a
// compile-time constant: the compiler's wait insertion then knows that
// fragment reads of slot s cannot alias the DMA in flight into other slots,
// and does not drain the ring before every read.
template <typename TA, typename TR, typename TY, int BM, int BN, int WM, int WN, int STAGES, bool HEADMAJOR>
__global__ void __launch_bounds__(WM* WN * 64, 1)
gemm_dma_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  using DP = DmaPlan<TA, BM, BN, NW>;
  using ES = EpiShape<TY, BN, WM, STAGES>;
  constexpr int SA = DP::SA, MAXI = DP::MAXI;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(STAGES >= 2 && STAGES <= 16, "ring depth");
  constexpr int SLOT = (DP::SA + DP::SB) > ES::SLOT ? (DP::SA + DP::SB) : ES::SLOT;

  __shared__ uint4 ring0[SLOT];
  __shared__ uint4 ring1[SLOT];
  __shared__ uint4 ring2[STAGES > 2 ? SLOT : 1];
  __shared__ uint4 ring3[STAGES > 3 ? SLOT : 1];
  __shared__ uint4 ring4[STAGES > 4 ? SLOT : 1];
  __shared__ uint4 ring5[STAGES > 5 ? SLOT : 1];
  __shared__ uint4 ring6[STAGES > 6 ? SLOT : 1];
  __shared__ uint4 ring7[STAGES > 7 ? SLOT : 1];
  __shared__ uint4 ring8[STAGES > 8 ? SLOT : 1];
  __shared__ uint4 ring9[STAGES > 9 ? SLOT : 1];
  __shared__ uint4 ring10[STAGES > 10 ? SLOT : 1];
  __shared__ uint4 ring11[STAGES > 11 ? SLOT : 1];
  __shared__ uint4 ring12[STAGES > 12 ? SLOT : 1];
  __shared__ uint4 ring13[STAGES > 13 ? SLOT : 1];
  __shared__ uint4 ring14[STAGES > 14 ? SLOT : 1];
  __shared__ uint4 ring15[STAGES > 15 ? SLOT : 1];
  auto slot = [&](auto sI) -> uint4* {
    constexpr int sl = decltype(sI)::value;
    if constexpr (sl == 0) return ring0;
    else if constexpr (sl == 1) return ring1;
    else if constexpr (sl == 2) return ring2;
    else if constexpr (sl == 3) return ring3;
    else if constexpr (sl == 4) return ring4;
    else if constexpr (sl == 5) return ring5;
    else if constexpr (sl == 6) return ring6;
    else if constexpr (sl == 7) return ring7;
    else if constexpr (sl == 8) return ring8;
    else if constexpr (sl == 9) return ring9;
    else if constexpr (sl == 10) return ring10;
    else if constexpr (sl == 11) return ring11;
    else if constexpr (sl == 12) return ring12;
    else if constexpr (sl == 13) return ring13;
    else if constexpr (sl == 14) return ring14;
    else return ring15;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave % WM, wn = wave / WM;
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (p.N + BN - 1) / BN;
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;  // grid larger than the tile count
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int KT = p.K / 32;

  DP dma;
  dma.init(p, m0, n0, wave, lane, blockIdx.y);

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = zero4();
  uint2 biasp[FN];  // fetched early, used in the epilogue
  load_bias<FN>(p, n0 + wn * TN, lane, biasp);

  const int g = lane >> 4, lr = lane & 15;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "fragment rows advance by 16");
  const int lofs_w = SA + DmaA<uint16_t>::lofs(wn * TN + lr, g);
  const int lofs_a = DmaA<TA>::lofs(wm * TM + lr, g);
  auto compute = [&](const uint4* st) {
    uint4 wf[FN], xf[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[i] = DmaA<uint16_t>::frag(st, lofs_w, i);
#pragma unroll
    for (int j = 0; j < FM; ++j) xf[j] = DmaA<TA>::frag(st, lofs_a, j);
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_bf16(wf[i], xf[j], acc[i][j]);
  };

  // Prologue: slices 0 .. STAGES-2 in flight (KT >= STAGES-1 is guaranteed by the host).
  static_for<0, STAGES - 1>([&](auto sI) { dma.issue(decltype(sI)::value, slot(sI)); });

  // Steady state: every slice kt < NMAIN refills the slot freed by slice
  // kt-1 with slice kt+STAGES-1 (< KT). Branch-free body.
  const int NMAIN = (KT - STAGES + 1) / STAGES * STAGES;
  for (int kt0 = 0; kt0 < NMAIN; kt0 += STAGES) {
    static_for<0, STAGES>([&](auto sI) {
      constexpr int s = decltype(sI)::value;
      wait_vm_lgkm0<(STAGES - 2) * MAXI>();
      ring_barrier();
      dma.issue(kt0 + s + STAGES - 1, slot(std::integral_constant<int, (s + STAGES - 1) % STAGES>{}));
      compute(slot(sI));
    });
  }
  // Tail: the last KT - NMAIN (< 2*STAGES-1) slices; slot of slice NMAIN + t is t % STAGES.
  static_for<0, 2 * STAGES - 2>([&](auto tI) {
    constexpr int t = decltype(tI)::value;
    const int kt = NMAIN + t;
    if (kt < KT) {
      const int ahead = min(STAGES - 2, KT - 1 - kt);
      wait_vm_dyn<(STAGES - 2) * MAXI>(ahead * MAXI);
      ring_barrier();
      if (kt + STAGES - 1 < KT)
        dma.issue(kt + STAGES - 1, slot(std::integral_constant<int, (t + STAGES - 1) % STAGES>{}));
      compute(slot(std::integral_constant<int, t % STAGES>{}));
    }
  });

  wait_vm_lgkm0<0>();
  ring_barrier();  // ring drained, every fragment read retired
  ring_epilogue<TR, TY, BM, BN, WM, WN, STAGES, HEADMAJOR>(p, acc, biasp, slot, tid, lane, wm, wn, m0, n0,
                                                          blockIdx.y);
}

// ----------------------------------------------------------------------------
// Ping-pong variant for the large token-row projections (bf16 A): the same
// 256 x 288 tile and 8 waves of 64 x 144 as gemm_dma_kernel, but the waves
// form two groups (W columns 0..143 and 144..287) that run one phase apart.
// Each SIMD holds one wave of each group, so while one group's waves run
// their MFMAs the other group's waves read their LDS fragments (and the LDS
// sees the reads of four waves at a time instead of eight).
//
// Every wave runs the same body for slice k:
//   refill slot (k-1) % 4 with slice k+3;  read slice k's fragments;
//   wait for slice k+1;  barrier;  MFMAs of slice k;  wait;  barrier
// (the refill is issued in the read phase, which waits at the barrier for
// the other group's MFMAs anyway, so the MFMA phase carries no DMA issue)
// Group 1 executes one extra barrier before its first body, group 0 one
// after its last, which offsets the groups by one phase. Counting barriers
// from the prologue's (#0): group 0 reads slice k between #2k and #2k+1,
// group 1 between #2k+1 and #2k+2. Hence slot k-1 is free for both groups
// from #2k on (group 0 refills after #2k, group 1 after #2k+1), and slice
// k+1, waited on by every wave before each barrier of its body k, is whole
// in LDS by #2k+2. Requires KT % 4 == 0 and KT >= 8.
//
// RKT > 0 (token-major output with a residual, KT == RKT == 36, one slice
// per accumulator block): the residual is folded into the accumulators
// during the main loop instead of being read in the epilogue. Each wave owns
// FN*FM = 36 accumulator blocks of 16x16; body k loads the residual of block
// k (one 4-value vector per lane, into buffer k % 2) just before its refill
// and adds it in body k+1's MFMA phase, after that body's first wait (two
// refills and one residual load may stay in flight) has retired it. The
// prologue loads block 35 between slices 1 and 2, in the same position
// relative to the refills, so the vmcnt targets stay constants. The loop is
// unrolled completely so that every block index is a constant. The epilogue
// then only writes.
// ----------------------------------------------------------------------------
// residual block loaded by steady body k of a wave with nb accumulator blocks
// (k = -1: the prologue's load); -1: none
constexpr int pp_rblock(int k, int nb) { return k < 0 ? nb + k : (k < nb - 1 ? k : -1); }

template <typename TR, typename TY, bool HEADMAJOR, int RKT, int BM = 256, bool TOKMAJ = false, bool WKM = false>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(GemmParams p_in) {
  GemmParams p = p_in;
  constexpr bool RIN = RKT > 0;
  static_assert(!TOKMAJ || (!RIN && !HEADMAJOR && BM == 256), "token-major operands: the weight gradient only");
  static_assert(!WKM || (!TOKMAJ && !HEADMAJOR), "k-major W: token-major output (dX = dY W)");
  static_assert(!RIN || (RKT == 36 && BM == 256), "one k-slice per accumulator block of a 64 x 144 wave tile");
  static_assert(BM == 256 || BM == 128, "wave tiles of 64 or 32 rows");
  using TA = uint16_t;
  constexpr int BN = 288, WM = 4, WN = 2, NW = 8, STAGES = 4;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int NB = FN * FM;  // accumulator blocks per wave
  constexpr int RL = RIN ? 1 : 0;
  static_assert(!RIN || !HEADMAJOR, "residual only for token-major output");
  using DP = typename std::conditional<
      TOKMAJ, DmaPlanTN<BM, BN, NW>,
      typename std::conditional<WKM, DmaPlanMix<BM, BN, NW>, DmaPlan<TA, BM, BN, NW>>::type>::type;
  using ES = EpiShape<TY, BN, WM, STAGES>;
  constexpr int SA = DP::SA, MAXI = DP::MAXI;
  constexpr int SLOT = (DP::SA + DP::SB) > ES::SLOT ? (DP::SA + DP::SB) : ES::SLOT;
  __shared__ uint4 ring0[SLOT];
  __shared__ uint4 ring1[SLOT];
  __shared__ uint4 ring2[SLOT];
  __shared__ uint4 ring3[SLOT];
  auto slot = [&](auto sI) -> uint4* {
    constexpr int sl = (decltype(sI)::value % STAGES + STAGES) % STAGES;
    if constexpr (sl == 0) return ring0;
    else if constexpr (sl == 1) return ring1;
    else if constexpr (sl == 2) return ring2;
    else return ring3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;  // wn is the group
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (p.N + BN - 1) / BN;
  int tm, tn, split;
  if constexpr (TOKMAJ) {
    // one-dimensional grid over (split, tm, tn): XCD k (the hardware hands
    // block i to XCD i % 8) walks a contiguous range of that order, tn
    // fastest, so the workgroups of an XCD share the dY slabs of their row
    // tiles and the X slabs of one split in its L2 (the row-major order of
    // the other kernels would spread a dY slab over four XCDs)
    // groups of one shape: the order is (group, split, tm, tn), tn fastest
    const int nt = tiles_m * tiles_n, per = nt * p.splits, total = per * p.groups;
    if ((int)blockIdx.x >= total) return;
    const int q = total >> 3, rem = total & 7, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    int logical = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
    if (p.groups > 1) {
      const int gi = logical / per;
      logical -= gi * per;
      // read from the kernel argument (a uniform scalar load), not the copy
      p.A = p_in.gA[gi];
      p.W = reinterpret_cast<const uint16_t*>(p_in.gW[gi]);
      p.Y = p_in.gY[gi];
    }
    split = logical / nt;
    const int in = logical - split * nt;
    tm = in / tiles_n;
    tn = in - tm * tiles_n;
  } else {
    if ((int)blockIdx.x >= tiles_m * tiles_n) return;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, 8, tm, tn);
    split = blockIdx.y;
  }
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int KT = RIN ? RKT : ((p.k_last > 0 && split == p.splits - 1) ? p.k_last : p.K) / 32;

  DP dma;
  dma.init(p, m0, n0, wave, lane, split);
  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = zero4();

  const int g = lane >> 4, lr = lane & 15;
  const int lofs_w = SA + DmaA<uint16_t>::lofs(wn * TN + lr, g);
  const int lofs_a = DmaA<TA>::lofs(wm * TM + lr, g);
  TnFragBase fbw, fba;
  if constexpr (TOKMAJ || WKM) fbw.init(SA * 16, wn * TN, lane);
  if constexpr (TOKMAJ) fba.init(0, wm * TM, lane);
  uint4 wf[FN], xf[FM];
  auto read_frags = [&](const uint4* st) {
    if constexpr (TOKMAJ) {
      static_for<0, FN>([&](auto iI) { wf[decltype(iI)::value] = tn_frag<decltype(iI)::value>(st, fbw); });
      static_for<0, FM>([&](auto jI) { xf[decltype(jI)::value] = tn_frag<decltype(jI)::value>(st, fba); });
    } else if constexpr (WKM) {
      static_for<0, FN>([&](auto iI) { wf[decltype(iI)::value] = tn_frag<decltype(iI)::value>(st, fbw); });
#pragma unroll
      for (int j = 0; j < FM; ++j) xf[j] = DmaA<TA>::frag(st, lofs_a, j);
    } else {
#pragma unroll
      for (int i = 0; i < FN; ++i) wf[i] = DmaA<uint16_t>::frag(st, lofs_w, i);
#pragma unroll
      for (int j = 0; j < FM; ++j) xf[j] = DmaA<TA>::frag(st, lofs_a, j);
    }
  };
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_bf16(wf[i], xf[j], acc[i][j]);
  };

  // residual of accumulator block b (i = b % FN, j = b / FN): the lane's row
  // and 4 columns, addressed as a wave-uniform base (the tile's first row) +
  // the block's uniform column offset + a 32-bit lane offset per row block.
  // Rows past M read row M - 1 (never stored: the epilogue drops them), so a
  // ragged last row tile needs no branch; columns need N % 288 == 0.
  using RV = typename std::conditional<sizeof(TR) == 4, float4, uint2>::type;
  const char* const rbase = reinterpret_cast<const char*>(reinterpret_cast<const TR*>(p.R) + m0 * p.N + n0 + wn * TN);
  uint32_t rlane[RIN ? FM : 1];
  if constexpr (RIN) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t row = min(m0 + wm * TM + j * 16 + lr, p.M - 1);
      rlane[j] = (uint32_t)(((int)(row - m0) * p.N + 4 * g) * (int)sizeof(TR));
    }
  }
  auto rload = [&](auto bI) -> RV {
    constexpr int b = decltype(bI)::value, i = b % FN, j = b / FN;
    const char* ra = rbase + i * 16 * (int)sizeof(TR) + rlane[j];
    if constexpr (sizeof(TR) == 4) {
      typedef float ntf4 __attribute__((ext_vector_type(4)));
      const ntf4 v = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(ra));
      return RV{v.x, v.y, v.z, v.w};
    } else {
      return *reinterpret_cast<const RV*>(ra);
    }
  };
  auto radd = [&](auto bI, const RV& v) {  // bI: compile-time block
    constexpr int bb = decltype(bI)::value;
    float f[4];
    if constexpr (sizeof(TR) == 4) {
      f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    } else {
      f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
      f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[bb % FN][bb / FN][r] += f[r];
  };
  RV rbuf[2];

  // body of slice k (slot t = k % 4). W: vm operations allowed in flight at
  // both waits (nothing is issued between them); RES: this body takes part in
  // the residual stream, with a compile-time slice index kI (block
  // pp_rblock(k) loaded, pp_rblock(k-1) added; -1: none).
  auto body = [&](auto tI, auto issueI, auto wI, auto resI, int k, auto kI) {
    constexpr int t = decltype(tI)::value;
    constexpr bool RES = RIN && decltype(resI)::value;
    constexpr int KC = decltype(kI)::value;
    if constexpr (RES) {
      constexpr int bn = pp_rblock(KC, NB);
      if constexpr (bn >= 0) rbuf[KC % 2] = rload(std::integral_constant<int, bn>{});
      // the residual load stays ahead of the refill
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (decltype(issueI)::value) dma.issue(k + 3, slot(std::integral_constant<int, t - 1>{}));
    read_frags(slot(std::integral_constant<int, t>{}));
    wait_vm_lgkm0<decltype(wI)::value>();
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RES) {
      constexpr int b = pp_rblock(KC - 1, NB);
      if constexpr (b >= 0) radd(std::integral_constant<int, b>{}, rbuf[(KC + 1) % 2]);
    }
    mfmas();
    wait_vm_lgkm0<decltype(wI)::value>();
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;

  // Prologue: slices 0..2 (and, with RIN, the residual of block NB-1 after
  // slice 1, into buffer 1), slice 0 landed (barrier #0); group 1 then takes
  // its extra barrier.
  dma.issue_head(0, slot(std::integral_constant<int, 0>{}));
  dma.issue_head(1, slot(std::integral_constant<int, 1>{}));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (RIN) rbuf[1] = rload(std::integral_constant<int, pp_rblock(-1, NB)>{});
  __builtin_amdgcn_sched_barrier(0);
  dma.issue_head(2, slot(std::integral_constant<int, 2>{}));
  wait_vm_lgkm0<2 * MAXI + RL>();
  ring_barrier();
  if (wn == 1) ring_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // Steady state: bodies k = 0 .. KT-5 (refill slice k+3 < KT - 1); at each
  // wait slices k+2, k+3 (and residual k) may stay in flight.
  const int NMAIN = KT - 4;
  using WS = std::integral_constant<int, 2 * MAXI + RL>;
  if constexpr (RIN) {
    static_for<0, RKT - 4>([&](auto kI) {
      constexpr int k = decltype(kI)::value;
      body(std::integral_constant<int, k % 4>{}, std::true_type{}, WS{}, std::true_type{}, k, kI);
    });
  } else {
    for (int k0 = 0; k0 < NMAIN; k0 += 4) {
      static_for<0, 4>([&](auto tI) {
        body(tI, std::true_type{}, WS{}, std::false_type{}, k0 + decltype(tI)::value, I0{});
      });
    }
  }
  // Tail: bodies KT-4 .. KT-1 (only the first refills, with slice KT-1).
  using RT = std::integral_constant<bool, RIN>;
  constexpr int NM = RIN ? RKT - 4 : 0;
  body(std::integral_constant<int, 0>{}, std::true_type{}, WS{}, RT{}, NMAIN, std::integral_constant<int, NM>{});
  body(std::integral_constant<int, 1>{}, std::false_type{}, std::integral_constant<int, MAXI + RL>{}, RT{},
       NMAIN + 1, std::integral_constant<int, NM + 1>{});
  body(std::integral_constant<int, 2>{}, std::false_type{}, std::integral_constant<int, RL>{}, RT{}, NMAIN + 2,
       std::integral_constant<int, NM + 2>{});
  body(std::integral_constant<int, 3>{}, std::false_type{}, I0{}, RT{}, NMAIN + 3, std::integral_constant<int, NM + 3>{});
  if (wn == 0) ring_barrier();

  wait_vm_lgkm0<0>();
  ring_barrier();
  GemmParams pe = p;
  if constexpr (RIN) pe.R = nullptr;  // every block's residual is in the accumulators
  uint2 biasp[FN];
  load_bias<FN>(p, n0 + wn * TN, lane, biasp);
  ring_epilogue<TR, TY, BM, BN, WM, WN, STAGES, HEADMAJOR>(pe, acc, biasp, slot, tid, lane, wm, wn, m0, n0, split);
}

// ----------------------------------------------------------------------------
// fp32 path: MFMA v_mfma_f32_16x16x4f32, 64x64 tiles, K steps of 16, one
// LDS stage. Used by the fp32 workload only.
// ----------------------------------------------------------------------------
struct GemmF32Params {
  const float* A;
  const float* W;
  const float* bias;
  const float* R;
  float* Y;
  int64_t M;
  int N, K;
  int64_t Ntok;
  int heads, dh, D;
  int act;
};

template <bool HEADMAJOR, int BM>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmF32Params p) {
  // BM x 64 tile (BM = 64: 4 waves of 32x32; BM = 32, for few rows: 4 waves
  // of 32x16), k-slices of 32 through a double-buffered LDS; the global
  // loads of slice k+2 are issued before slice k is computed (two register
  // sets), so each load has two slices of MFMA work to land.
  constexpr int BN = 64, BK = 32, LD = BK + 1;
  constexpr int WMN = BM / 32, WNN = 4 / WMN;     // waves along m and n
  constexpr int FN = BN / WNN / 16, FM = 2;       // 16x16 blocks per wave
  constexpr int RA = BM / 32;                     // A row groups of 32 per thread
  __shared__ float As[2][BM * LD];
  __shared__ float Ws[2][BN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WMN, wn = wave / WMN;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  floatx4 acc[FN][FM];
  for (int i = 0; i < FN; ++i)
    for (int j = 0; j < FM; ++j) acc[i][j] = zero4();

  // thread t moves rows (t >> 3) + 32 r, columns 4 * (t & 7) .. +3
  const int lrow = tid >> 3, lc = (tid & 7) * 4;
  int64_t ga[RA];
  int64_t gw[2];
#pragma unroll
  for (int r = 0; r < RA; ++r) {
    const int64_t gm = m0 + lrow + 32 * r;
    ga[r] = (gm < p.M ? gm : p.M - 1) * p.K;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int gn = n0 + lrow + 32 * r;
    gw[r] = (int64_t)(gn < p.N ? gn : p.N - 1) * p.K;
  }
  struct Slice { float4 a[RA], w[2]; };
  auto gload = [&](int k0, Slice& sl) {
    const int k = k0 + lc;
    const bool ok = k < p.K;  // K % 4 == 0: a chunk is in or out as a whole
#pragma unroll
    for (int r = 0; r < RA; ++r)
      sl.a[r] = ok ? *reinterpret_cast<const float4*>(p.A + ga[r] + k) : float4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 2; ++r)
      sl.w[r] = ok ? *reinterpret_cast<const float4*>(p.W + gw[r] + k) : float4{0, 0, 0, 0};
  };
  auto lstore = [&](int buf, const Slice& sl) {
#pragma unroll
    for (int r = 0; r < RA; ++r) {
      float* ad = &As[buf][(lrow + 32 * r) * LD + lc];
      ad[0] = sl.a[r].x; ad[1] = sl.a[r].y; ad[2] = sl.a[r].z; ad[3] = sl.a[r].w;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float* wd = &Ws[buf][(lrow + 32 * r) * LD + lc];
      wd[0] = sl.w[r].x; wd[1] = sl.w[r].y; wd[2] = sl.w[r].z; wd[3] = sl.w[r].w;
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kq = 0; kq < BK / 4; ++kq) {
      const int k = kq * 4 + (lane >> 4);
      float wf[FN], xf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) wf[i] = Ws[buf][(wn * FN * 16 + i * 16 + (lane & 15)) * LD + k];
#pragma unroll
      for (int j = 0; j < FM; ++j) xf[j] = As[buf][(wm * 32 + j * 16 + (lane & 15)) * LD + k];
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma_f32(wf[i], xf[j], acc[i][j]);
    }
  };

  const int KT = (p.K + BK - 1) / BK;
  Slice sl[2];
  gload(0, sl[0]);
  if (KT > 1) gload(BK, sl[1]);
  lstore(0, sl[0]);
  __syncthreads();
  // slice kt: computed from LDS buffer kt % 2; sl[(kt + 1) % 2] holds slice kt+1
  for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kt + u;
      if (k >= KT) break;
      if (k + 2 < KT) gload((k + 2) * BK, sl[u]);  // sl[u] (slice k) is already in LDS
      compute(u);
      if (k + 1 < KT) lstore(u ^ 1, sl[u ^ 1]);
      __syncthreads();
    }
  }
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * FN * 16 + i * 16 + 4 * (lane >> 4);
    if (n >= p.N) continue;
    float4 bv = p.bias ? *reinterpret_cast<const float4*>(p.bias + n) : float4{0, 0, 0, 0};
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * 32 + j * 16 + (lane & 15);
      if (m >= p.M) continue;
      float v0 = acc[i][j][0] + bv.x, v1 = acc[i][j][1] + bv.y;
      float v2 = acc[i][j][2] + bv.z, v3 = acc[i][j][3] + bv.w;
      if (p.act) {
        v0 = gelu_tanh(v0); v1 = gelu_tanh(v1); v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
      }
      if constexpr (HEADMAJOR) {
        const int g = n / p.D, hn = n - g * p.D;
        const int h = hn / p.dh, d = hn - h * p.dh;
        const int64_t b = m / p.Ntok, tok = m - b * p.Ntok;
        const int G = p.N / p.D;
        const int64_t off = (((b * G + g) * p.heads + h) * p.Ntok + tok) * p.dh + d;
        *reinterpret_cast<float4*>(p.Y + off) = float4{v0, v1, v2, v3};
      } else {
        const int64_t off = m * p.N + n;
        if (p.R) {
          const float4 r = *reinterpret_cast<const float4*>(p.R + off);
          v0 += r.x; v1 += r.y; v2 += r.z; v3 += r.w;
        }
        *reinterpret_cast<float4*>(p.Y + off) = float4{v0, v1, v2, v3};
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Dispatch
// ----------------------------------------------------------------------------
template <typename TA, typename TR, typename TY, int BM, int BN, int WM, int WN, bool HM>
static hipError_t run_bf16(const GemmParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * (int64_t)((p.N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  if (p.K % 64 == 0)
    hipLaunchKernelGGL((gemm_bf16_kernel<TA, TR, TY, BM, BN, WM, WN, HM, true>), dim3((unsigned)tiles),
                       dim3(WM * WN * 64), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<TA, TR, TY, BM, BN, WM, WN, HM, false>), dim3((unsigned)tiles),
                       dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <typename TA, typename TR, typename TY, int BM, int BN, int WM, int WN, int S, bool HM>
static hipError_t run_dma(const GemmParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * (int64_t)((p.N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dma_kernel<TA, TR, TY, BM, BN, WM, WN, S, HM>), dim3((unsigned)tiles, (unsigned)p.splits),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <typename TR, typename TY, bool HM, bool WKM = false>
static hipError_t run_pp(const GemmParams& p, hipStream_t s) {
  if (p.K % 128 != 0 || p.K < 256) return hipErrorInvalidValue;  // KT % 4 == 0, KT >= 8
  const int64_t tiles = ((p.M + 255) / 256) * (int64_t)((p.N + 287) / 288);
  if (tiles <= 0) return hipSuccess;
  const int64_t t128 = ((p.M + 127) / 128) * (int64_t)((p.N + 287) / 288);
  if (tiles * p.splits < 256 && t128 * p.splits <= 256) {
    // fewer 256-row tiles than CUs (the 1024^2 block's 8192-row projections
    // onto D): 128-row tiles (waves of 32 x 144) keep more CUs busy, in one
    // round still (a second, partial round would cost more than the idle
    // CUs: the 3456 x 1152 weight gradient split 4 ways over the tokens of a
    // 2048^2 block runs 142 us on 224 workgroups, 193 us on 432); the
    // residual is added in the epilogue
    hipLaunchKernelGGL((gemm_pp_kernel<TR, TY, HM, 0, 128, false, WKM>), dim3((unsigned)t128, (unsigned)p.splits),
                       dim3(512), 0, s, p);
    return hipGetLastError();
  }
  if constexpr (!HM) {
    // the model width D = 1152 with whole column tiles: residual folded into
    // the main loop (rows past M of a ragged last row tile are clamped)
    if (p.R && p.K == 36 * 32 && p.N % 288 == 0) {
      hipLaunchKernelGGL((gemm_pp_kernel<TR, TY, HM, 36, 256, false, WKM>), dim3((unsigned)tiles, (unsigned)p.splits),
                         dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_pp_kernel<TR, TY, HM, 0, 256, false, WKM>), dim3((unsigned)tiles, (unsigned)p.splits),
                     dim3(512), 0, s, p);
  return hipGetLastError();
}

// Tile choice. Token-row projections (M >= 2048 rows, K a multiple of 32) use
// 256x288 tiles: 288 = 4 heads of 72, and D = 1152 = 4 x 288, 3D = 12 x 288,
// so a 2048^2 image block yields exactly 256 (N = D) or 768 (N = 3D) tiles for
// 256 CUs. With bf16 A and K % 128 == 0 the ping-pong kernel takes them, else
// the multi-stage ring kernel. Proxy-row projections (few rows) take a small
// tile; odd shapes take the register-staged kernel.
template <typename TA, typename TR, typename TY, bool HM>
static hipError_t pick_tile(const GemmParams& p, hipStream_t s) {
  constexpr int STAGES = sizeof(TA) == 2 ? 4 : 3;
  // strided or split contractions (row strides other than K, splits over
  // blockIdx.y) go to the DMA kernels only
  if (p.lda != p.K || p.ldw != p.K || p.splits != 1) {
    const int64_t ld = p.lda > p.ldw ? p.lda : p.ldw;
    if (p.K % 32 != 0 || p.K / 32 < STAGES || (int64_t)288 * ld * (int64_t)sizeof(TA) >= (int64_t)1 << 31 ||
        p.splits < 1 || p.splits > 65535)
      return hipErrorInvalidValue;
    if constexpr (sizeof(TA) == 2) {
      // from 1024 rows: the weight gradients of the D x D output maps too
      // (1152 rows, ragged in 256-row tiles; the ping-pong kernel clamps the
      // rows past M on load and drops them on store)
      if (p.M >= 1024 && p.K % 128 == 0 && p.K >= 256 && !p.R) return run_pp<TR, TY, HM>(p, s);
    }
    if (p.M >= 1024) return run_dma<TA, TR, TY, 256, 288, 4, 2, STAGES, HM>(p, s);
    if (p.K / 32 < 4) return hipErrorInvalidValue;
    return run_dma<TA, TR, TY, 32, 64, 2, 2, 4, HM>(p, s);
  }
  // the DMA kernels address a tile's A / W rows with 32-bit byte offsets
  const bool off32 = (int64_t)288 * p.K * (int64_t)sizeof(TA) < (int64_t)1 << 31;
  if (!off32) return p.M >= 1024 ? run_bf16<TA, TR, TY, 128, 128, 2, 2, HM>(p, s)
                                 : run_bf16<TA, TR, TY, 64, 64, 2, 2, HM>(p, s);
  if constexpr (sizeof(TA) == 2) {
    if (p.M >= 2048 && p.K % 128 == 0 && p.K >= 256) return run_pp<TR, TY, HM>(p, s);
  }
  if (p.M >= 2048 && p.K % 32 == 0 && p.K / 32 >= STAGES)
    return run_dma<TA, TR, TY, 256, 288, 4, 2, STAGES, HM>(p, s);
  // few rows (proxies): a small tile for parallelism; a 4-slot ring measured
  // faster than 8 or 12 slots here (shorter prologue, same streaming rate)
  if (p.M < 1024 && p.K % 32 == 0 && p.K / 32 >= 4) {
    // From 512 rows (the video block's 864 proxies): 64-row tiles, 128
    // columns wide when that still gives about a workgroup a CU (fewer
    // re-reads of each A and W slab; measured at 864 x 3456, K = 1152:
    // 18.9 us against 22.3 on 64 x 64 tiles, 864 x 2304: 13.2 against
    // 16.0), else 64 wide (864 x 1152: 7.7 us against 9.1 on 32 x 64).
    if (p.M >= 512) {
      if (((p.M + 63) / 64) * (int64_t)((p.N + 127) / 128) >= 216)
        return run_dma<TA, TR, TY, 64, 128, 2, 2, 4, HM>(p, s);
      return run_dma<TA, TR, TY, 64, 64, 2, 2, 4, HM>(p, s);
    }
    // fewer rows (the 256 proxies of an image block): 32-row tiles when
    // 64-row tiles would leave CUs idle
    if (((p.M + 63) / 64) * (int64_t)((p.N + 63) / 64) < 256) return run_dma<TA, TR, TY, 32, 64, 2, 2, 4, HM>(p, s);
    return run_dma<TA, TR, TY, 64, 64, 2, 2, 4, HM>(p, s);
  }
  if (p.M >= 1024) return run_bf16<TA, TR, TY, 128, 128, 2, 2, HM>(p, s);
  return run_bf16<TA, TR, TY, 64, 64, 2, 2, HM>(p, s);
}

template <typename TA, typename TY>
static hipError_t pick_r(const GemmDesc& d, const GemmParams& p, hipStream_t s) {
  if (d.head_major) return pick_tile<TA, uint16_t, TY, true>(p, s);
  if (!d.R || d.r_f32) return pick_tile<TA, float, TY, false>(p, s);
  return pick_tile<TA, uint16_t, TY, false>(p, s);
}

hipError_t launch_gemm_bf16(const GemmDesc& d, hipStream_t s) {
  GemmParams p;
  p.A = d.A;
  p.W = reinterpret_cast<const uint16_t*>(d.W);
  p.bias = reinterpret_cast<const uint16_t*>(d.bias);
  p.R = d.R;
  p.Y = d.Y;
  p.Y2 = reinterpret_cast<uint16_t*>(d.Y2);
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.Ntok = d.Ntok > 0 ? d.Ntok : 1;
  p.heads = d.heads; p.dh = d.dh; p.D = d.D;
  p.act = d.act;
  p.lda = d.lda > 0 ? d.lda : d.K;
  p.ldw = d.ldw > 0 ? d.ldw : d.K;
  p.ks_a = d.ks_a; p.ks_w = d.ks_w; p.ks_y = d.ks_y;
  p.splits = d.splits > 0 ? d.splits : 1;
  p.k_last = d.k_last;
  p.k_valid = d.k_valid;
  p.groups = 1;
  for (int i = 0; i < GEMM_MAX_GROUPS; ++i) {
    p.gA[i] = i < d.groups ? d.gA[i] : nullptr;
    p.gW[i] = i < d.groups ? d.gW[i] : nullptr;
    p.gY[i] = i < d.groups ? d.gY[i] : nullptr;
  }
  if (d.w_kmajor) {
    // k-major W [K][ldw] (dX = dY W with the weight as it lies): the
    // ping-pong kernel's mixed instance; bf16 A, token-major output, an fp32
    // residual or none, no bias
    if (d.a_f32 || d.head_major || d.splits > 1 || d.act || d.bias || (d.R && !d.r_f32) || p.K % 128 || p.K < 256 ||
        p.N % 8 || p.N <= 0 || p.M <= 0 || p.lda != p.K || p.ldw < p.N || p.ldw % 8 ||
        (int64_t)2 * p.K * p.ldw >= ((int64_t)1 << 31) || (int64_t)512 * p.K >= ((int64_t)1 << 31))
      return hipErrorInvalidValue;
    return d.y_f32 ? run_pp<float, float, false, true>(p, s) : run_pp<float, uint16_t, false, true>(p, s);
  }
  if (d.tn) {
    // token-major bf16 operands (the weight gradient): the ping-pong kernel's
    // TN instance, 256 x 288 tiles, fp32 output, no bias / residual
    const int kl = d.k_last > 0 ? d.k_last : d.K;
    if (d.a_f32 || !d.y_f32 || d.R || d.bias || d.head_major || d.Y2 || p.K % 128 || p.K < 256 || kl % 128 ||
        kl < 256 || d.k_valid < 0 || d.k_valid > kl || d.k_valid % 32 ||
        (d.k_valid > 0 && d.k_valid < kl && (p.lda > TN_ZERO_LD || p.ldw > TN_ZERO_LD)) || p.M % 8 || p.N % 8 ||
        p.M <= 0 || p.N <= 0 || p.lda <= 0 || p.ldw <= 0 ||
        p.lda * 64 * 32 >= ((int64_t)1 << 31) || p.ldw * 64 * 32 >= ((int64_t)1 << 31))
      return hipErrorInvalidValue;
    const int64_t tiles = ((p.M + 255) / 256) * (int64_t)((p.N + 287) / 288);
    if (d.groups > 1) {  // products of this shape at gA/gW/gY (A, W, Y unused)
      if (d.groups > GEMM_MAX_GROUPS) return hipErrorInvalidValue;
      for (int i = 0; i < d.groups; ++i)
        if (!d.gA[i] || !d.gW[i] || !d.gY[i]) return hipErrorInvalidValue;
      p.groups = d.groups;
    }
    // one-dimensional grid: the kernel maps it onto (group, split, row tile, column tile)
    hipLaunchKernelGGL((gemm_pp_kernel<float, float, false, 0, 256, true>),
                       dim3((unsigned)(tiles * p.splits * p.groups)), dim3(512), 0, s, p);
    return hipGetLastError();
  }
  if (d.a_f32) {
    if (d.y_f32) return pick_r<float, float>(d, p, s);
    return pick_r<float, uint16_t>(d, p, s);
  }
  if (d.y_f32) return pick_r<uint16_t, float>(d, p, s);
  return pick_r<uint16_t, uint16_t>(d, p, s);
}

hipError_t launch_gemm_f32(const GemmDesc& d, hipStream_t s) {
  if (d.lda > 0 || d.ldw > 0 || d.splits > 1) return hipErrorInvalidValue;  // dense operands only
  GemmF32Params p;
  p.A = reinterpret_cast<const float*>(d.A);
  p.W = reinterpret_cast<const float*>(d.W);
  p.bias = reinterpret_cast<const float*>(d.bias);
  p.R = reinterpret_cast<const float*>(d.R);
  p.Y = reinterpret_cast<float*>(d.Y);
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.Ntok = d.Ntok > 0 ? d.Ntok : 1;
  p.heads = d.heads; p.dh = d.dh; p.D = d.D;
  p.act = d.act;
  // 32-row tiles (twice the workgroups) when 64-row tiles would leave fewer
  // than two workgroups per CU: proxy rows, and the output projections of
  // short token sequences
  const bool small = ((p.M + 63) / 64) * (int64_t)((p.N + 63) / 64) < 512;
  const int bm = small ? 32 : 64;
  const int64_t tiles = ((p.M + bm - 1) / bm) * (int64_t)((p.N + 63) / 64);
  if (tiles <= 0) return hipSuccess;
  if (d.head_major) {
    if (small) hipLaunchKernelGGL((gemm_f32_kernel<true, 32>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_f32_kernel<true, 64>), dim3((unsigned)tiles), dim3(256), 0, s, p);
  } else {
    if (small) hipLaunchKernelGGL((gemm_f32_kernel<false, 32>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_f32_kernel<false, 64>), dim3((unsigned)tiles), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ptdit
