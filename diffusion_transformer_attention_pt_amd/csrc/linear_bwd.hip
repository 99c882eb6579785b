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
//   colsum_kernel     partial column sums of dY over 64-row blocks (when
//                     no transpose pass reads dY: otherwise that pass,
//                     which reads every element anyway, writes them)
//   wgrad_reduce      fixed-order sum of the partials (deterministic)
//
// With bf16 dY and X, 1024 <= d_out <= 4096, d_in <= 4096 and a token count
// that is a multiple of 32 (at least 256), dW = dY^T X runs on the ping-pong
// kernel's token-major instance straight from dY and X (both with the token
// index as their row): no transposed copies; the last split may be longer
// (k_last) and end in whole 32-token slices that read as zero (k_valid).
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

// The same for rows and cols that are multiples of 8 (every weight the
// projections take): 64 x 64 tiles moved in 16-byte pieces. Lane (t, q)
// reads 8 columns of W rows t and t + 32, and writes 8 consecutive entries
// (W rows 8q .. 8q + 7) of W^T rows t and t + 32; the LDS tile is 64 rows of
// 33 dwords (66 elements), so the 8 rows one transposed read walks are not
// all in one bank.
__global__ void __launch_bounds__(LB_NT) transpose16_kernel(const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ wt, int rows, int cols) {
  __shared__ uint32_t tile[64 * 33];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int q = threadIdx.x & 7, t = threadIdx.x >> 3;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = t + 32 * h;
    if (r0 + r < rows && c0 + 8 * q < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(w + (int64_t)(r0 + r) * cols + c0 + 8 * q);
      uint32_t* d = tile + r * 33 + 4 * q;
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
  }
  __syncthreads();
  const uint16_t* ts = reinterpret_cast<const uint16_t*>(tile);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = t + 32 * h;
    // rows and cols are multiples of 8: a chunk lies wholly inside or outside
    if (c0 + c < cols && r0 + 8 * q < rows) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)ts[(8 * q + 2 * e) * 66 + c] | ((uint32_t)ts[(8 * q + 2 * e + 1) * 66 + c] << 16);
      *reinterpret_cast<uint4*>(wt + (int64_t)(c0 + c) * rows + r0 + 8 * q) = uint4{o[0], o[1], o[2], o[3]};
    }
  }
}

// src [rows][cols] (bf16 or fp32) -> dst [cols][ld] bf16 (columns rows ..
// ld-1 zero; ld % 64 == 0), and optionally a row-major bf16 copy [rows][cols]:
// the token-contiguous operands of dW = dY^T X (and the bf16 A operand of
// dX = dY W). 64 x 64 tiles: 16 lanes read one row's 64 columns (4 each), the
// transposed writes are 8 consecutive tokens (16 bytes) of one column. With
// colp, the tile's column sums of src (fp32 values as read, the 16 row groups
// added in order) go to colp[tile row][column]: the partials of db = sum_t dY
// over 64-token blocks.
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
                                                              uint16_t* __restrict__ copy, float* __restrict__ colp,
                                                              int64_t rows, int cols, int64_t ld) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TPD * TPP];
  __shared__ __attribute__((aligned(16))) float csum[16][TPD];
  const int64_t r0 = (int64_t)blockIdx.x * TPD;
  const int c0 = blockIdx.y * TPD;
  const int tid = threadIdx.x, lc = (tid & 15) * 4, lr = tid >> 4;  // 16 lanes a row
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TPD / 16; ++i) {
    const int r = lr + 16 * i;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    const bool ok = r0 + r < rows && c0 + lc < cols;  // cols % 4 == 0: a group is in or out
    if (ok) ld4f(src + (r0 + r) * cols + c0 + lc, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] += v[j];
    const uint32_t p0 = pack_bf2(v[0], v[1]), p1 = pack_bf2(v[2], v[3]);
    *reinterpret_cast<uint32_t*>(&tile[r * TPP + lc]) = p0;
    *reinterpret_cast<uint32_t*>(&tile[r * TPP + lc + 2]) = p1;
    if (copy && ok) *reinterpret_cast<uint2*>(copy + (r0 + r) * cols + c0 + lc) = uint2{p0, p1};
  }
  if (colp) *reinterpret_cast<float4*>(&csum[lr][lc]) = float4{cs[0], cs[1], cs[2], cs[3]};
  __syncthreads();
  if (colp && tid < TPD && r0 < rows && c0 + tid < cols) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) t += csum[g][tid];
    colp[blockIdx.x * (int64_t)cols + c0 + tid] = t;
  }
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

// partial column sums of dY over token block blockIdx.y (CS_ROWS rows, the
// transpose tile's height, so both give the same partial layout): four
// columns per lane (d_out % 8 == 0, 16-byte aligned rows), eight rows of
// loads in flight, four chains (row t % 4) combined in a fixed order
constexpr int CS_ROWS = TPD;
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
// A workgroup: 64 four-column groups x 4 row chains; chain c (one wave)
// sums the rows t0 + c, t0 + c + 4, ... of its block in increasing order,
// eight loads in flight, and the chains are combined as (c0 + c1) + (c2 + c3)
template <typename TA>
__device__ __forceinline__ void colsum_body(const TA* __restrict__ dy, float* __restrict__ dbp, int64_t rows,
                                            int d_out) {
  __shared__ float4 chain[4][64];
  const int cq = threadIdx.x & 63, c = threadIdx.x >> 6;
  const int o = 4 * (blockIdx.x * 64 + cq);
  const int64_t t0 = (int64_t)blockIdx.y * CS_ROWS, t1 = min(rows, t0 + CS_ROWS);
  auto add = [](float4& a, const float4& b) { a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w; };
  float4 s = float4{0.f, 0.f, 0.f, 0.f};
  if (o < d_out) {
    int64_t t = t0 + c;
    for (; t + 28 < t1; t += 32) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = Col4<TA>::ld(dy + (t + 4 * u) * d_out + o);
#pragma unroll
      for (int u = 0; u < 8; ++u) add(s, v[u]);
    }
    for (; t < t1; t += 4) add(s, Col4<TA>::ld(dy + t * d_out + o));
  }
  chain[c][cq] = s;
  __syncthreads();
  if (c == 0 && o < d_out) {
    float4 r = chain[0][cq];
    add(r, chain[1][cq]);
    float4 r2 = chain[2][cq];
    add(r2, chain[3][cq]);
    add(r, r2);
    *reinterpret_cast<float4*>(dbp + (int64_t)blockIdx.y * d_out + o) = r;
  }
}
static int colsum_blocks(int d_out) { return (d_out / 4 + 63) / 64; }
template <typename TA>
__global__ void __launch_bounds__(LB_NT) colsum_kernel(const TA* __restrict__ dy, float* __restrict__ dbp,
                                                       int64_t rows, int d_out) {
  colsum_body<TA>(dy, dbp, rows, d_out);
}

// the products of one grouped weight-gradient launch, indexed by blockIdx.z
// (column sums) or blockIdx.y (reduction); a null dy / dw skips a product
struct WgradGroupPtrs {
  const uint16_t* dy[GEMM_MAX_GROUPS];
  float* dbp[GEMM_MAX_GROUPS];
  const float* part[GEMM_MAX_GROUPS];
  float* dw[GEMM_MAX_GROUPS];
  float* db[GEMM_MAX_GROUPS];
};
__global__ void __launch_bounds__(LB_NT) colsum_group_kernel(WgradGroupPtrs g, int64_t rows, int d_out) {
  const uint16_t* dy = g.dy[blockIdx.z];
  if (dy) colsum_body<uint16_t>(dy, g.dbp[blockIdx.z], rows, d_out);
}

// four consecutive elements a thread (nw and d_out multiples of 4, 16-byte
// aligned rows), eight partials in flight, each element summed in split
// order (deterministic)
__device__ __forceinline__ void add4(float4& s, const float4& v) {
  s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
}
__device__ __forceinline__ float4 sum_splits4(const float* __restrict__ part, int64_t stride, int n, int64_t e) {
  float4 s = float4{0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(part + (int64_t)(k + u) * stride + e);
#pragma unroll
    for (int u = 0; u < 8; ++u) add4(s, v[u]);
  }
  if (k < n) {  // the last (< 8) partials, loaded together, added in order
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = k + u < n ? *reinterpret_cast<const float4*>(part + (int64_t)(k + u) * stride + e)
                       : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k + u < n) add4(s, v[u]);
  }
  return s;
}

// db from the column-sum partials [csplits][d_out] (one per 64-row block,
// hundreds of them): a workgroup takes 64 columns; lane (c, r) sums the
// partials r, r + 16, r + 32, ... of columns 4c .. 4c + 3 in that order, and
// the 16 subtotals of a column are then added in the order r = 0 .. 15
// (fixed, so the result does not depend on scheduling)
constexpr int DB_COLS = 64;
__device__ __forceinline__ void db_reduce_block(const float* __restrict__ dbp, float* __restrict__ db, int csplits,
                                                int d_out, int blk) {
  __shared__ float4 sub[16][16];
  const int c = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int e = blk * DB_COLS + 4 * c;
  float4 s = float4{0.f, 0.f, 0.f, 0.f};
  if (e < d_out) {
    int k = r;
    for (; k + 48 < csplits; k += 64) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(dbp + (int64_t)(k + 16 * u) * d_out + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) add4(s, v[u]);
    }
    for (; k < csplits; k += 16) add4(s, *reinterpret_cast<const float4*>(dbp + (int64_t)k * d_out + e));
  }
  sub[r][c] = s;
  __syncthreads();
  if (r == 0 && e < d_out) {
    float4 t = sub[0][c];
#pragma unroll
    for (int i = 1; i < 16; ++i) add4(t, sub[i][c]);
    *reinterpret_cast<float4*>(db + e) = t;
  }
}
static int db_reduce_blocks(int d_out) { return (d_out + DB_COLS - 1) / DB_COLS; }

// blocks [0, nwb): dW, four elements a thread; blocks from nwb on: db
__global__ void __launch_bounds__(LB_NT) wgrad_reduce_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ dbp, float* __restrict__ dw,
                                                             float* __restrict__ db, int splits, int csplits,
                                                             int64_t nw, int d_out, int nwb) {
  if ((int)blockIdx.x >= nwb) {
    if (db) db_reduce_block(dbp, db, csplits, d_out, blockIdx.x - nwb);
    return;
  }
  const int64_t e = 4 * ((int64_t)blockIdx.x * LB_NT + threadIdx.x);
  if (e < nw && dw) *reinterpret_cast<float4*>(dw + e) = sum_splits4(part, nw, splits, e);
}
__global__ void __launch_bounds__(LB_NT) wgrad_reduce_group_kernel(WgradGroupPtrs g, int splits, int csplits,
                                                                   int64_t nw, int d_out, int nwb) {
  const int p = blockIdx.y;
  float* const dw = g.dw[p];
  float* const db = g.db[p];
  if ((int)blockIdx.x >= nwb) {
    if (db) db_reduce_block(g.dbp[p], db, csplits, d_out, blockIdx.x - nwb);
    return;
  }
  const int64_t e = 4 * ((int64_t)blockIdx.x * LB_NT + threadIdx.x);
  if (e < nw && dw) *reinterpret_cast<float4*>(dw + e) = sum_splits4(g.part[p], nw, splits, e);
}

// ----------------------------------------------------------------------------
int colsum_splits(int64_t rows) { return (int)((rows + CS_ROWS - 1) / CS_ROWS); }

void wgrad_plan(int64_t rows, int d_in, int d_out, int& splits, int64_t& tch, int groups) {
  // the DMA GEMM's tile for M = d_out rows of dW: 256 x 288 from 1024 rows,
  // 32 x 64 below; about one workgroup per CU in total, over all `groups`
  // products of this shape that one launch computes
  const int64_t tiles = (int64_t)groups * (d_out >= 1024 ? (int64_t)((d_out + 255) / 256) * ((d_in + 287) / 288)
                                                         : (int64_t)((d_out + 31) / 32) * ((d_in + 63) / 64));
  int64_t sp = 256 / tiles;
  if (sp < 1) sp = 1;
  tch = (rows + sp - 1) / sp;
  tch = (tch + 127) / 128 * 128;  // whole 128-token k-slices (the ping-pong kernel's unit)
  if (tch < 256) tch = 256;
  splits = (int)((rows + tch - 1) / tch);
}

hipError_t launch_transpose_bf16(const void* w, void* wt, int rows, int cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 8 == 0 && cols % 8 == 0) {
    hipLaunchKernelGGL(transpose16_kernel, dim3((cols + 63) / 64, (rows + 63) / 64), dim3(LB_NT), 0, s,
                       reinterpret_cast<const uint16_t*>(w), reinterpret_cast<uint16_t*>(wt), rows, cols);
    return hipGetLastError();
  }
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
  // the dY pass also writes db's partials (colsum_kernel then is not run)
  float* colp = d.db ? d.dbp : nullptr;
  if (d.dy_f32)
    hipLaunchKernelGGL((transpose_pad_kernel<float>), gy, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.dy),
                       d.dyt, d.dyb, colp, d.rows, d.d_out, ld);
  else
    hipLaunchKernelGGL((transpose_pad_kernel<uint16_t>), gy, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.dy),
                       d.dyt, d.dyb, colp, d.rows, d.d_out, ld);
  if (d.x_f32)
    hipLaunchKernelGGL((transpose_pad_kernel<float>), gx, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.x),
                       d.xt, nullptr, nullptr, d.rows, d.d_in, ld);
  else
    hipLaunchKernelGGL((transpose_pad_kernel<uint16_t>), gx, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.x),
                       d.xt, nullptr, nullptr, d.rows, d.d_in, ld);
  return hipGetLastError();
}

bool wgrad_token_major(int64_t rows, int d_in, int d_out, int dy_f32, int x_f32) {
  return !dy_f32 && !x_f32 && d_out >= 1024 && d_out <= 4096 && d_in <= 4096 && rows % 32 == 0 && rows >= 256;
}

// whole splits of tch tokens, the remainder joined to the last one when it is
// shorter than the kernel's 256-token minimum; the last split's K is rounded
// up to 128 tokens, the rows past its kv real ones read as zero
static void wgrad_tn_splits(int64_t rows, int64_t tch, int& sp, int64_t& kv, int64_t& kl) {
  sp = (int)((rows + tch - 1) / tch);
  kv = rows - (int64_t)(sp - 1) * tch;
  if (kv < 256 && sp > 1) {
    --sp;
    kv += tch;
  }
  kl = (kv + 127) / 128 * 128 < 256 ? 256 : (kv + 127) / 128 * 128;
}

size_t wgrad_group_ws_bytes(int n, int64_t rows, int d_in, int d_out) {
  int splits, sp;
  int64_t tch, kv, kl;
  wgrad_plan(rows, d_in, d_out, splits, tch, n);
  wgrad_tn_splits(rows, tch, sp, kv, kl);
  const size_t a = 255;
  const size_t pb = ((size_t)sp * d_out * d_in * 4 + a) & ~a, cb = ((size_t)colsum_splits(rows) * d_out * 4 + a) & ~a;
  return (size_t)n * (pb + cb);
}

hipError_t launch_wgrad_group(const WgradGroupDesc& d, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  if (d.n < 1 || d.n > GEMM_MAX_GROUPS || !wgrad_token_major(d.rows, d.d_in, d.d_out, 0, 0))
    return hipErrorInvalidValue;
  int splits, sp;
  int64_t tch, kv, kl;
  wgrad_plan(d.rows, d.d_in, d.d_out, splits, tch, d.n);
  wgrad_tn_splits(d.rows, tch, sp, kv, kl);
  const int64_t nw = (int64_t)d.d_out * d.d_in;
  const int csplits = colsum_splits(d.rows);
  const size_t a = 255;
  const size_t pb = ((size_t)sp * nw * 4 + a) & ~a, cb = ((size_t)csplits * d.d_out * 4 + a) & ~a;
  char* const ws = reinterpret_cast<char*>(d.ws);
  auto part = [&](int i) { return reinterpret_cast<float*>(ws + (size_t)i * pb); };
  auto dbp = [&](int i) { return reinterpret_cast<float*>(ws + (size_t)d.n * pb + (size_t)i * cb); };
  // one launch: the n products' splits, (group, split, row tile, column tile)
  GemmDesc g;
  g.A = d.dy[0]; g.a_f32 = 0;
  g.W = d.x[0]; g.bias = nullptr;
  g.R = nullptr; g.r_f32 = 1;
  g.Y = part(0); g.y_f32 = 1;
  g.Y2 = nullptr;
  g.M = d.d_out; g.N = d.d_in; g.K = sp == 1 ? (int)kl : (int)tch;
  g.head_major = 0; g.Ntok = d.d_out; g.heads = 0; g.dh = 0; g.D = d.d_in;
  g.lda = d.d_out; g.ldw = d.d_in; g.ks_a = tch; g.ks_w = tch; g.ks_y = nw; g.splits = sp;
  g.tn = 1; g.k_last = (int)kl; g.k_valid = (int)kv;
  g.groups = d.n;
  for (int i = 0; i < d.n; ++i) {
    g.gA[i] = d.dy[i];
    g.gW[i] = d.x[i];
    g.gY[i] = part(i);
  }
  hipError_t e = launch_gemm_bf16(g, s);
  if (e != hipSuccess) return e;
  // every product's column sums in one launch, then every product's
  // split-order reduction in one launch (the same sums as the per-call path)
  WgradGroupPtrs gp{};
  bool any_db = false;
  for (int i = 0; i < d.n; ++i) {
    gp.dy[i] = d.db[i] ? reinterpret_cast<const uint16_t*>(d.dy[i]) : nullptr;
    gp.dbp[i] = dbp(i);
    gp.part[i] = part(i);
    gp.dw[i] = d.dw[i];
    gp.db[i] = d.db[i];
    any_db = any_db || d.db[i];
  }
  if (any_db) {
    hipLaunchKernelGGL(colsum_group_kernel, dim3(colsum_blocks(d.d_out), csplits, d.n), dim3(LB_NT), 0, s,
                       gp, d.rows, d.d_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int nwb = (int)((nw / 4 + LB_NT - 1) / LB_NT);
  hipLaunchKernelGGL(wgrad_reduce_group_kernel, dim3((unsigned)(nwb + (any_db ? db_reduce_blocks(d.d_out) : 0)), d.n),
                     dim3(LB_NT), 0, s, gp, sp, csplits, nw, d.d_out, nwb);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradDesc& d, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  int splits;
  int64_t tch;
  wgrad_plan(d.rows, d.d_in, d.d_out, splits, tch);
  const int64_t ld = splits * tch, nw = (int64_t)d.d_out * d.d_in;
  const bool tn = wgrad_token_major(d.rows, d.d_in, d.d_out, d.dy_f32, d.x_f32);
  if (d.dw && tn) {
    int sp;
    int64_t kv, kl;
    wgrad_tn_splits(d.rows, tch, sp, kv, kl);
    GemmDesc g;
    g.A = d.dy; g.a_f32 = 0;
    g.W = d.x; g.bias = nullptr;
    g.R = nullptr; g.r_f32 = 1;
    g.Y = d.part; g.y_f32 = 1;
    g.Y2 = nullptr;
    g.M = d.d_out; g.N = d.d_in; g.K = (int)tch;
    g.head_major = 0; g.Ntok = d.d_out; g.heads = 0; g.dh = 0; g.D = d.d_in;
    g.lda = d.d_out; g.ldw = d.d_in; g.ks_a = tch; g.ks_w = tch; g.ks_y = nw; g.splits = sp;
    g.tn = 1; g.k_last = (int)kl; g.k_valid = (int)kv;
    if (sp == 1) g.K = (int)kl;
    const hipError_t e = launch_gemm_bf16(g, s);
    if (e != hipSuccess) return e;
    splits = sp;
  } else if (d.dw) {
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
  if (d.db && (!d.dw || tn)) {  // else the transpose pass wrote the partials
    const dim3 grid(colsum_blocks(d.d_out), csplits);
    if (d.dy_f32)
      hipLaunchKernelGGL((colsum_kernel<float>), grid, dim3(LB_NT), 0, s, reinterpret_cast<const float*>(d.dy),
                         d.dbp, d.rows, d.d_out);
    else
      hipLaunchKernelGGL((colsum_kernel<uint16_t>), grid, dim3(LB_NT), 0, s, reinterpret_cast<const uint16_t*>(d.dy),
                         d.dbp, d.rows, d.d_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nwb = d.dw ? (int)((nw / 4 + LB_NT - 1) / LB_NT) : 0;
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)(nwb + (d.db ? db_reduce_blocks(d.d_out) : 0))),
                     dim3(LB_NT), 0, s, d.part, d.dbp, d.dw, d.db, splits, csplits, nw, d.d_out, nwb);
  return hipGetLastError();
}

}  // namespace ptdit
