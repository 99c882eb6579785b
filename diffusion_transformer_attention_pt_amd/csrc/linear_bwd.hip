// Gradients of the projections Y = X W^T + b (the Q/K/V/O maps of every
// attention module, Qihoo-T2X reading note, code-correspondence module table;
// trained at 2048^2, section 4): dX = dY W, dW = dY^T X, db = sum_t dY.
//
//   transpose_kernel  W [d_out][d_in] -> W^T [d_in][d_out] (bf16), so dX is
//                     an ordinary projection (the token-row GEMM kernels)
//   wgrad_kernel      dW = dY^T X on the matrix cores: 128 x 128 tiles of dW,
//                     the token axis split over workgroups; 64-token steps of
//                     dY and X are staged transposed ([column][token]) so both
//                     MFMA operands are contiguous 16-byte LDS reads
//   colsum_kernel     partial column sums of dY over 256-row blocks
//   wgrad_reduce      fixed-order sum of the partials (deterministic)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

namespace {

constexpr int LB_NT = 256;
constexpr int WG_BM = 128, WG_BN = 128, WG_KT = 32, WG_TP = WG_KT + 8;
constexpr int WG_QPT = WG_KT / 32;  // 4-token quads a staging thread takes per step

// 8 consecutive elements as bf16 (fp32 sources rounded to nearest even)
__device__ __forceinline__ uint4 ld8_bf16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ld8_bf16(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return uint4{pack_bf2(a.x, a.y), pack_bf2(a.z, a.w), pack_bf2(b.x, b.y), pack_bf2(b.z, b.w)};
}

// Column (token) index of element (row r, column k < WG_KT) in the transposed
// tiles: 16-byte groups of the row XOR-swizzled by the row's 8-row group
// (within the WG_KT columns), so that
// writes from 16 consecutive column chunks spread over the banks; reads of 8
// consecutive tokens stay one aligned 16-byte read.
__device__ __forceinline__ int swz(int r, int k) { return k ^ (((r >> 3) & (WG_KT / 8 - 1)) << 3); }

// t[(8 ch + e) * pitch + swz(8 ch + e, s0 + j)] = element e of v[j]: one
// 8-byte write per e (s0 % 4 == 0)
__device__ __forceinline__ void put_quad_cols(uint16_t* t, int pitch, int ch, int s0, const uint4 (&v)[4]) {
  const uint32_t a0[4] = {v[0].x, v[0].y, v[0].z, v[0].w}, a1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
  const uint32_t a2[4] = {v[2].x, v[2].y, v[2].z, v[2].w}, a3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = (e & 1) * 16;
    const uint32_t lo = ((a0[e >> 1] >> sh) & 0xffffu) | (((a1[e >> 1] >> sh) & 0xffffu) << 16);
    const uint32_t hi = ((a2[e >> 1] >> sh) & 0xffffu) | (((a3[e >> 1] >> sh) & 0xffffu) << 16);
    const int r = ch * 8 + e;
    *reinterpret_cast<uint2*>(&t[r * pitch + swz(r, s0)]) = uint2{lo, hi};
  }
}

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

// ----------------------------------------------------------------------------
struct WgradParams {
  const void* dy;
  const void* x;
  float* part;    // [splits][d_out][d_in]
  int64_t rows;
  int d_in, d_out;
  int64_t tch;    // tokens per split (a multiple of WG_KT)
};

// 4 waves in 2 x 2, each a 64 x 64 block of the 128 x 128 tile (4 x 4 MFMA
// tiles, two 32-token halves a step). Threads 0..127 stage dY, 128..255 stage
// X: two (8-column chunk, 4-token quad) items each, chunks fastest (16 lanes
// read one token row's 16 chunks: coalesced); the next step's loads are in
// flight during the current step's products (two LDS buffers, one barrier a
// step).
template <typename TA, typename TB>
__global__ void __launch_bounds__(LB_NT) wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t aT[2][WG_BM * WG_TP], bT[2][WG_BN * WG_TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int wm = w & 1, wn = w >> 1;
  const int tiles_n = (p.d_in + WG_BN - 1) / WG_BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n, split = blockIdx.y;
  const int o0 = tm * WG_BM, i0 = tn * WG_BN;
  const int64_t t_begin = (int64_t)split * p.tch, t_end = min(p.rows, t_begin + p.tch);
  const bool isA = tid < 128;
  const int it = tid & 127, ch = it & 15, kq0 = it >> 4;
  const int col = (isA ? o0 : i0) + ch * 8, ncols = isA ? p.d_out : p.d_in;
  uint4 v[WG_QPT][4];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int q = 0; q < WG_QPT; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + (kq0 + 8 * q) * 4 + j;
        const bool ok = t < t_end && col < ncols;
        if (isA)
          v[q][j] = ok ? ld8_bf16(reinterpret_cast<const TA*>(p.dy) + t * p.d_out + col) : uint4{0, 0, 0, 0};
        else
          v[q][j] = ok ? ld8_bf16(reinterpret_cast<const TB*>(p.x) + t * p.d_in + col) : uint4{0, 0, 0, 0};
      }
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();
  if (t_begin < t_end) load(t_begin);
  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += WG_KT, buf ^= 1) {
#pragma unroll
    for (int q = 0; q < WG_QPT; ++q) put_quad_cols(isA ? aT[buf] : bT[buf], WG_TP, ch, (kq0 + 8 * q) * 4, v[q]);
    __syncthreads();
    if (t0 + WG_KT < t_end) load(t0 + WG_KT);
#pragma unroll
    for (int kh = 0; kh < WG_KT / 32; ++kh) {
      uint4 af[4], bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ra = wm * 64 + j * 16 + c, rb = wn * 64 + j * 16 + c;
        af[j] = *reinterpret_cast<const uint4*>(&aT[buf][ra * WG_TP + swz(ra, kh * 32 + 8 * g)]);
        bf[j] = *reinterpret_cast<const uint4*>(&bT[buf][rb * WG_TP + swz(rb, kh * 32 + 8 * g)]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16(af[a], bf[b], acc[a][b]);
    }
  }
  // D[m = 4g + r][n = c] of block (a, b): dW[o][i]
  float* out = p.part + (int64_t)split * p.d_out * p.d_in;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + wn * 64 + b * 16 + c;
      if (i >= p.d_in) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = o0 + wm * 64 + a * 16 + 4 * g + r;
        if (o < p.d_out) out[(int64_t)o * p.d_in + i] = acc[a][b][r];
      }
    }
}

// partial column sums of dY over token block blockIdx.y (CS_ROWS rows)
constexpr int CS_ROWS = 256;
template <typename TA>
__global__ void __launch_bounds__(LB_NT) colsum_kernel(const TA* __restrict__ dy, float* __restrict__ dbp,
                                                       int64_t rows, int d_out) {
  const int o = blockIdx.x * LB_NT + threadIdx.x;
  if (o >= d_out) return;
  const int64_t t0 = (int64_t)blockIdx.y * CS_ROWS, t1 = min(rows, t0 + CS_ROWS);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;  // four chains, combined in a fixed order
  int64_t t = t0;
  for (; t + 4 <= t1; t += 4) {
    s0 += ld1(dy + t * d_out + o);
    s1 += ld1(dy + (t + 1) * d_out + o);
    s2 += ld1(dy + (t + 2) * d_out + o);
    s3 += ld1(dy + (t + 3) * d_out + o);
  }
  for (; t < t1; ++t) s0 += ld1(dy + t * d_out + o);
  dbp[(int64_t)blockIdx.y * d_out + o] = (s0 + s1) + (s2 + s3);
}

__global__ void __launch_bounds__(LB_NT) wgrad_reduce_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ dbp, float* __restrict__ dw,
                                                             float* __restrict__ db, int splits, int csplits,
                                                             int64_t nw, int d_out) {
  const int64_t e = (int64_t)blockIdx.x * LB_NT + threadIdx.x;
  if (e < nw && dw) {
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * nw + e];
    dw[e] = s;
  }
  if (e < d_out && db) {
    float s = 0.f;
    for (int k = 0; k < csplits; ++k) s += dbp[(int64_t)k * d_out + e];
    db[e] = s;
  }
}

// ----------------------------------------------------------------------------
int colsum_splits(int64_t rows) { return (int)((rows + CS_ROWS - 1) / CS_ROWS); }

int wgrad_splits(int64_t rows, int d_in, int d_out) {
  const int64_t tiles = (int64_t)((d_out + WG_BM - 1) / WG_BM) * ((d_in + WG_BN - 1) / WG_BN);
  int64_t s = (1024 + tiles - 1) / tiles;             // >= 1024 workgroups
  const int64_t most = (rows + 511) / 512;            // >= 512 tokens a split
  if (s > most) s = most;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

hipError_t launch_transpose_bf16(const void* w, void* wt, int rows, int cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((cols + 31) / 32, (rows + 31) / 32), dim3(LB_NT), 0, s,
                     reinterpret_cast<const uint16_t*>(w), reinterpret_cast<uint16_t*>(wt), rows, cols);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradDesc& d, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  const int splits = d.splits;
  int64_t tch = (d.rows + splits - 1) / splits;
  tch = (tch + WG_KT - 1) / WG_KT * WG_KT;
  const int64_t nw = (int64_t)d.d_out * d.d_in;
  if (d.dw) {
    WgradParams p;
    p.dy = d.dy; p.x = d.x; p.part = d.part; p.rows = d.rows; p.d_in = d.d_in; p.d_out = d.d_out; p.tch = tch;
    const int tiles = ((d.d_out + WG_BM - 1) / WG_BM) * ((d.d_in + WG_BN - 1) / WG_BN);
    const dim3 grid(tiles, splits);
    if (d.dy_f32 && d.x_f32) hipLaunchKernelGGL((wgrad_kernel<float, float>), grid, dim3(LB_NT), 0, s, p);
    else if (d.dy_f32) hipLaunchKernelGGL((wgrad_kernel<float, uint16_t>), grid, dim3(LB_NT), 0, s, p);
    else if (d.x_f32) hipLaunchKernelGGL((wgrad_kernel<uint16_t, float>), grid, dim3(LB_NT), 0, s, p);
    else hipLaunchKernelGGL((wgrad_kernel<uint16_t, uint16_t>), grid, dim3(LB_NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int csplits = colsum_splits(d.rows);
  if (d.db) {
    const dim3 grid((d.d_out + LB_NT - 1) / LB_NT, csplits);
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
