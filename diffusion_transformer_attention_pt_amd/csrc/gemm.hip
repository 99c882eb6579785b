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
#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

struct GemmParams {
  const void* A;
  const uint16_t* W;
  const uint16_t* bias;
  const void* R;
  void* Y;
  int64_t M;
  int N, K;
  int64_t Ntok;
  int heads, dh, D;
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

template <typename TA, typename TR, typename TY, int BM, int BN, int WM, int WN, bool HEADMAJOR>
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
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const TA* A = reinterpret_cast<const TA*>(p.A);
  const int K = p.K;
  const int KT = (K + 63) / 64;

  uint4 ra[ACH], rw[WCH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + i * NT, row = q >> 3, c = q & 7;
      const int k = kt * 64 + c * 8;
      int64_t gm = m0 + row;
      gm = gm < p.M ? gm : p.M - 1;
      ra[i] = k < K ? load8_as_bf16(A + gm * K + k) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + i * NT, row = q >> 3, c = q & 7;
      const int k = kt * 64 + c * 8;
      int gn = n0 + row;
      gn = gn < p.N ? gn : p.N - 1;
      rw[i] = k < K ? *reinterpret_cast<const uint4*>(p.W + (int64_t)gn * K + k) : uint4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + i * NT, row = q >> 3, c = q & 7;
      lds[buf][row * 8 + (c ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + i * NT, row = q >> 3, c = q & 7;
      lds[buf][(BM + row) * 8 + (c ^ (row & 7))] = rw[i];
    }
  };

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = zero4();

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      const int sw = c ^ (lane & 7);  // (row & 7) == (lane & 7) for every fragment row
      uint4 wf[FN], xf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wn * TN + i * 16 + (lane & 15);
        wf[i] = lds[buf][(BM + row) * 8 + sw];
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wm * TM + j * 16 + (lane & 15);
        xf[j] = lds[buf][row * 8 + sw];
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = mfma_bf16(wf[i], xf[j], acc[i][j]);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
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
      }
    }
  }
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
};

template <bool HEADMAJOR>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmF32Params p) {
  constexpr int BM = 64, BN = 64, BK = 16, LD = BK + 1;
  __shared__ float As[BM * LD];
  __shared__ float Ws[BN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  floatx4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = zero4();

  const int lrow = tid >> 2, lc = (tid & 3) * 4;
  for (int k0 = 0; k0 < p.K; k0 += BK) {
    {
      int64_t gm = m0 + lrow;
      gm = gm < p.M ? gm : p.M - 1;
      int gn = n0 + lrow;
      gn = gn < p.N ? gn : p.N - 1;
      const int k = k0 + lc;
      float4 a = k < p.K ? *reinterpret_cast<const float4*>(p.A + gm * p.K + k) : float4{0, 0, 0, 0};
      float4 w = k < p.K ? *reinterpret_cast<const float4*>(p.W + (int64_t)gn * p.K + k) : float4{0, 0, 0, 0};
      As[lrow * LD + lc + 0] = a.x; As[lrow * LD + lc + 1] = a.y;
      As[lrow * LD + lc + 2] = a.z; As[lrow * LD + lc + 3] = a.w;
      Ws[lrow * LD + lc + 0] = w.x; Ws[lrow * LD + lc + 1] = w.y;
      Ws[lrow * LD + lc + 2] = w.z; Ws[lrow * LD + lc + 3] = w.w;
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < BK / 4; ++kq) {
      const int k = kq * 4 + (lane >> 4);
      float wf[2], xf[2];
      for (int i = 0; i < 2; ++i) wf[i] = Ws[(wn * 32 + i * 16 + (lane & 15)) * LD + k];
      for (int j = 0; j < 2; ++j) xf[j] = As[(wm * 32 + j * 16 + (lane & 15)) * LD + k];
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32(wf[i], xf[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 2; ++i) {
    const int n = n0 + wn * 32 + i * 16 + 4 * (lane >> 4);
    if (n >= p.N) continue;
    float4 bv = p.bias ? *reinterpret_cast<const float4*>(p.bias + n) : float4{0, 0, 0, 0};
    for (int j = 0; j < 2; ++j) {
      const int64_t m = m0 + wm * 32 + j * 16 + (lane & 15);
      if (m >= p.M) continue;
      float v0 = acc[i][j][0] + bv.x, v1 = acc[i][j][1] + bv.y;
      float v2 = acc[i][j][2] + bv.z, v3 = acc[i][j][3] + bv.w;
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
  hipLaunchKernelGGL((gemm_bf16_kernel<TA, TR, TY, BM, BN, WM, WN, HM>), dim3((unsigned)tiles),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <typename TA, typename TR, typename TY, bool HM>
static hipError_t pick_tile(const GemmParams& p, hipStream_t s) {
  if (p.M >= 2048) return run_bf16<TA, TR, TY, 256, 192, 2, 2, HM>(p, s);
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
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.Ntok = d.Ntok > 0 ? d.Ntok : 1;
  p.heads = d.heads; p.dh = d.dh; p.D = d.D;
  if (d.a_f32) {
    if (d.y_f32) return pick_r<float, float>(d, p, s);
    return pick_r<float, uint16_t>(d, p, s);
  }
  if (d.y_f32) return pick_r<uint16_t, float>(d, p, s);
  return pick_r<uint16_t, uint16_t>(d, p, s);
}

hipError_t launch_gemm_f32(const GemmDesc& d, hipStream_t s) {
  GemmF32Params p;
  p.A = reinterpret_cast<const float*>(d.A);
  p.W = reinterpret_cast<const float*>(d.W);
  p.bias = reinterpret_cast<const float*>(d.bias);
  p.R = reinterpret_cast<const float*>(d.R);
  p.Y = reinterpret_cast<float*>(d.Y);
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.Ntok = d.Ntok > 0 ? d.Ntok : 1;
  p.heads = d.heads; p.dh = d.dh; p.D = d.D;
  const int64_t tiles = ((p.M + 63) / 64) * (int64_t)((p.N + 63) / 64);
  if (tiles <= 0) return hipSuccess;
  if (d.head_major)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ptdit
