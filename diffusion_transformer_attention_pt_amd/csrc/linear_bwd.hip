// Gradients of the projections Y = X W^T + b (the Q/K/V/O maps of every
// attention module, Qihoo-T2X reading note, code-correspondence module table;
// trained at 2048^2, section 4): dX = dY W, dW = dY^T X, db = sum_t dY.
//
//   transpose_kernel  W [d_out][d_in] -> W^T [d_in][d_out] (bf16), so dX is
//                     an ordinary projection (the token-row GEMM kernels)
//   transpose_pad_kernel  dY and X to token-contiguous bf16 [column][token]
//                     (zero past the last token), so dW = dY^T X is an ordinary
//                     contraction over the token axis on the DMA GEMM kernels
//                     (those of the token-row projections), the token axis
//                     split over blockIdx.y into partials
//   colsum_kernel     partial column sums of dY over 128-row blocks
//   wgrad_reduce      fixed-order sum of the partials (deterministic)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

namespace {

constexpr int LB_NT = 256;

}  // namespace

// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(LB_NT) transpose_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                          int rows, int cols) {
  __shared__ uint16_t tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8)
    if (r0 + r < rows && c0 + tx < cols) tile[r][tx] = w[(int64_t)(r0 + r) * cols + c0 + tx];
  __syncthreads();
  for (int c = ty; c < 32; c += 8)
    if (c0 + c < cols && r0 + tx < rows) wt[(int64_t)(c0 + c) * rows + r0 + tx] = tile[tx][c];
}

// src [rows][cols] (bf16 or fp32) -> dst [cols][ld] bf16 (columns rows ..
// ld-1 zero; ld % 64 == 0), and optionally a row-major bf16 copy [rows][cols]:
// the token-contiguous operands of dW = dY^T X (and the bf16 A operand of
// dX = dY W). 64 x 64 tiles: 16 lanes read one row's 64 columns (4 each), the
// transposed writes are 8 consecutive tokens (16 bytes) of one column.
constexpr int TPD = 64, TPP = TPD + 2;  // tile, LDS pitch (elements)
__device__ __forceinline__ void ld4f(const float* p, float (&v)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ __forceinline__ void ld4f(const uint16_t* p, float (&v)[4]) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xffff0000u);
  v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xffff0000u);
}
template <typename T>
__global__ void __launch_bounds__(LB_NT) transpose_pad_kernel(const T* __restrict__ src, uint16_t* __restrict__ dst,
                                                              uint16_t* __restrict__ copy, int64_t rows, int cols,
                                                              int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TPD * TPP];
  const int64_t r0 = (int64_t)blockIdx.x * TPD;
  const int c0 = blockIdx.y * TPD;
  const int tid = threadIdx.x, lc = (tid & 15) * 4, lr = tid >> 4;  // 16 lanes a row
#pragma unroll
  for (int i = 0; i < TPD / 16; ++i) {
    const int r = lr + 16 * i;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    const bool ok = r0 + r < rows && c0 + lc < cols;  // cols % 4 == 0: a group is in or out
    if (ok) ld4f(src + (r0 + r) * cols + c0 + lc, v);
    const uint32_t p0 = pack_bf2(v[0], v[1]), p1 = pack_bf2(v[2], v[3]);
    *reinterpret_cast<uint32_t*>(&tile[r * TPP + lc]) = p0;
    *reinterpret_cast<uint32_t*>(&tile[r * TPP + lc + 2]) = p1;
    if (copy && ok) *reinterpret_cast<uint2*>(copy + (r0 + r) * cols + c0 + lc) = uint2{p0, p1};
  }
  __syncthreads();
  // 64 columns x 8 token groups = 512 writes of 16 bytes, two a thread
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = tid + i * LB_NT, c = item >> 3, tg = item & 7;
    if (c0 + c >= cols) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[(tg * 8 + 2 * j) * TPP + c] | ((uint32_t)tile[(tg * 8 + 2 * j + 1) * TPP + c] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + c) * ld + r0 + tg * 8) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// partial column sums of dY over token block blockIdx.y (CS_ROWS rows): four
// columns per lane (d_out % 8 == 0, 16-byte aligned rows), eight rows of
// loads in flight, four chains (row t % 4) combined in a fixed order
constexpr int CS_ROWS = 128;
template <typename TA> struct Col4;
template <> struct Col4<float> {
  __device__ static float4 ld(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct Col4<uint16_t> {
  __device__ static float4 ld(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return float4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                  __uint_as_float(v.y & 0xffff0000u)};
  }
};
template <typename TA>
__global__ void __launch_bounds__(LB_NT) colsum_kernel(const TA* __restrict__ dy, float* __restrict__ dbp,
                                                       int64_t rows, int d_out) {
  const int o = 4 * (blockIdx.x * LB_NT + threadIdx.x);
  if (o >= d_out) return;
  const int64_t t0 = (int64_t)blockIdx.y * CS_ROWS, t1 = min(rows, t0 + CS_ROWS);
  float4 s[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) s[c] = float4{0.f, 0.f, 0.f, 0.f};
  auto add = [](float4& a, const float4& b) { a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w; };
  int64_t t = t0;
  for (; t + 8 <= t1; t += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = Col4<TA>::ld(dy + (t + u) * d_out + o);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(s[u & 3], v[u]);
  }
  for (; t < t1; ++t) add(s[(t - t0) & 3], Col4<TA>::ld(dy + t * d_out + o));
  float4 r = s[0];
  add(r, s[1]);
  float4 r2 = s[2];
  add(r2, s[3]);
  add(r, r2);
  *reinterpret_cast<float4*>(dbp + (int64_t)blockIdx.y * d_out + o) = r;
}

__global__ void __launch_bounds__(LB_NT) wgrad_reduce_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ dbp, float* __restrict__ dw,
                                                             float* __restrict__ db, int splits, int csplits,
                                                             int64_t nw, int d_out) {
  const int64_t e = (int64_t)blockIdx.x * LB_NT + threadIdx.x;
  if (e < nw && dw) {
    // four loads in flight, added in split order
    float s = 0.f;
    int k = 0;
    for (; k + 4 <= splits; k += 4) {
      const float a0 = part[(int64_t)k * nw + e], a1 = part[(int64_t)(k + 1) * nw + e];
      const float a2 = part[(int64_t)(k + 2) * nw + e], a3 = part[(int64_t)(k + 3) * nw + e];
      s += a0; s += a1; s += a2; s += a3;
    }
    for (; k < splits; ++k) s += part[(int64_t)k * nw + e];
    dw[e] = s;
  }
  if (e < d_out && db) {
    float s = 0.f;
    int k = 0;
    for (; k + 4 <= csplits; k += 4) {
      const float a0 = dbp[(int64_t)k * d_out + e], a1 = dbp[(int64_t)(k + 1) * d_out + e];
      const float a2 = dbp[(int64_t)(k + 2) * d_out + e], a3 = dbp[(int64_t)(k + 3) * d_out + e];
      s += a0; s += a1; s += a2; s += a3;
    }
    for (; k < csplits; ++k) s += dbp[(int64_t)k * d_out + e];
    db[e] = s;
  }
}

// ----------------------------------------------------------------------------
int colsum_splits(int64_t rows) { return (int)((rows + CS_ROWS - 1) / CS_ROWS); }

void wgrad_plan(int64_t rows, int d_in, int d_out, int& splits, int64_t& tch) {
  // the DMA GEMM's tile for M = d_out rows of dW: 256 x 288 from 1024 rows,
  // 32 x 64 below; about one workgroup per CU in total
  const int64_t tiles = d_out >= 1024 ? (int64_t)((d_out + 255) / 256) * ((d_in + 287) / 288)
                                      : (int64_t)((d_out + 31) / 32) * ((d_in + 63) / 64);
  int64_t sp = 256 / tiles;
  if (sp < 1) sp = 1;
  tch = (rows + sp - 1) / sp;
  tch = (tch + 127) / 128 * 128;  // whole 128-token k-slices (the ping-pong kernel's unit)
  if (tch < 256) tch = 256;
  splits = (int)((rows + tch - 1) / tch);
}

hipError_t launch_transpose_bf16(const void* w, void* wt, int rows, int cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((cols + 31) / 32, (rows + 31) / 32), dim3(LB_NT), 0, s,
                     reinterpret_cast<const uint16_t*>(w), reinterpret_cast<uint16_t*>(wt), rows, cols);
  return hipGetLastError();
}

hipError_t launch_wgrad_operands(const WgradDesc& d, hipStream_t s) {
  if (d.rows == 0 || !d.dw) return hipSuccess;
  int splits;
  int64_t tch;
  wgrad_plan(d.rows, d.d_in, d.d_out, splits, tch);
  const int64_t ld = splits * tch;
  const dim3 gy((unsigned)(ld / TPD), (unsigned)((d.d_out + TPD - 1) / TPD)),
      gx((unsigned)(ld / TPD), (unsigned)((d.d_in + TPD - 1) / TPD));
  if (d.dy_f32)
    hipLaunchKernelGGL((transpose_pad_kernel<float>), gy, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.dy),
                       d.dyt, d.dyb, d.rows, d.d_out, ld);
  else
    hipLaunchKernelGGL((transpose_pad_kernel<uint16_t>), gy, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.dy),
                       d.dyt, d.dyb, d.rows, d.d_out, ld);
  if (d.x_f32)
    hipLaunchKernelGGL((transpose_pad_kernel<float>), gx, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.x),
                       d.xt, nullptr, d.rows, d.d_in, ld);
  else
    hipLaunchKernelGGL((transpose_pad_kernel<uint16_t>), gx, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.x),
                       d.xt, nullptr, d.rows, d.d_in, ld);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradDesc& d, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  int splits;
  int64_t tch;
  wgrad_plan(d.rows, d.d_in, d.d_out, splits, tch);
  const int64_t ld = splits * tch, nw = (int64_t)d.d_out * d.d_in;
  if (d.dw) {
    // dY^T [d_out][ld] and X^T [d_in][ld] (bf16, zero past rows), then
    // dW = dY^T (X^T)^T on the DMA GEMM kernels with the token axis as K,
    // split over blockIdx.y into partials [splits][d_out][d_in]
    // the transposed copies were written by launch_wgrad_operands
    GemmDesc g;
    g.A = d.dyt; g.a_f32 = 0;
    g.W = d.xt; g.bias = nullptr;
    g.R = nullptr; g.r_f32 = 1;
    g.Y = d.part; g.y_f32 = 1;
    g.Y2 = nullptr;
    g.M = d.d_out; g.N = d.d_in; g.K = (int)tch;
    g.head_major = 0; g.Ntok = d.d_out; g.heads = 0; g.dh = 0; g.D = d.d_in;
    g.lda = ld; g.ldw = ld; g.ks_a = tch; g.ks_w = tch; g.ks_y = nw; g.splits = splits;
    const hipError_t e = launch_gemm_bf16(g, s);
    if (e != hipSuccess) return e;
  }
  const int csplits = colsum_splits(d.rows);
  if (d.db) {
    const dim3 grid((d.d_out / 4 + LB_NT - 1) / LB_NT, csplits);
    if (d.dy_f32)
      hipLaunchKernelGGL((colsum_kernel<float>), grid, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.dy),
                         d.dbp, d.rows, d.d_out);
    else
      hipLaunchKernelGGL((colsum_kernel<uint16_t>), grid, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.dy),
                         d.dbp, d.rows, d.d_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = nw > d.d_out ? nw : d.d_out;
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n + LB_NT - 1) / LB_NT)), dim3(LB_NT), 0, s, d.part,
                     d.dbp, d.dw, d.db, splits, csplits, nw, d.d_out);
  return hipGetLastError();
}

}  // namespace ptdit
