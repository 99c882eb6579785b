// Window-average proxy pooling (GIIM "Averaging") and the stand-alone 3D roll.
//
// Both are bandwidth-bound. Every thread owns 8 consecutive channels (one
// 16-byte bf16 vector) so a row of D channels is read by D/8 neighbouring
// threads in one coalesced sweep.
//
// Pool summation order (fixed, so the result is bit-reproducible): fp32;
// for each (dt, di) the row sum over dj runs in index order from 0; row sums
// are added over di in index order; plane sums over dt in index order; then
// one IEEE fp32 division by P = p_t*p_h*p_w (hipcc's default fp32 division
// is correctly rounded; this file is built without fast-math).
#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  __device__ static void load(const uint16_t* p, float* f) { unpack8(*reinterpret_cast<const uint4*>(p), f); }
  __device__ static void store(uint16_t* p, const float* f) { *reinterpret_cast<uint4*>(p) = pack8_sw(f); }
};
template <> struct Vec8<float> {
  __device__ static void load(const float* p, float* f) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ static void store(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = float4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<float4*>(p + 4) = float4{f[4], f[5], f[6], f[7]};
  }
};

struct PoolParams {
  const void* x;
  void* out;
  int B, F, H, W, D;
  int pt, ph, pw;
  int FT, HI, WJ;  // proxy grid
};

constexpr int POOL_CX = 16;   // channel chunks (of 8) per workgroup along x
constexpr int POOL_MAXR = 64; // max (dt, di) rows held in LDS

// Block (POOL_CX, ny): thread (tx, ty) sums rows r = ty, ty+ny, ... of the
// window for chunk tx into LDS; thread ty == 0 then adds them in order. The
// LDS holds the window's R = p_t * p_h row sums (dynamic size, R * 512 B).
template <typename TX, typename TO>
__global__ void __launch_bounds__(1024) pool_kernel(PoolParams p) {
  extern __shared__ float part[];
  const int C = p.D / 8;
  const int tx = threadIdx.x, ty = threadIdx.y, ny = blockDim.y;
  const int cx = blockIdx.y * POOL_CX + tx;
  const int M = p.FT * p.HI * p.WJ;
  const int bm = blockIdx.x;
  const int b = bm / M, m = bm - b * M;
  const int T = m / (p.HI * p.WJ), I = (m / p.WJ) % p.HI, J = m % p.WJ;
  const int R = p.pt * p.ph;
  const TX* x = reinterpret_cast<const TX*>(p.x);
  const int64_t N = (int64_t)p.F * p.H * p.W;

  if (cx < C) {
    for (int r = ty; r < R; r += ny) {
      const int dt = r / p.ph, di = r - dt * p.ph;
      const int t = T * p.pt + dt, i = I * p.ph + di;
      const TX* src = x + ((int64_t)b * N + ((int64_t)t * p.H + i) * p.W + (int64_t)J * p.pw) * p.D + cx * 8;
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int dj = 0;
      for (; dj + 8 <= p.pw; dj += 8) {  // eight independent loads in flight, adds in order
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) Vec8<TX>::load(src + (int64_t)(dj + u) * p.D, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = s[e] + v[u][e];
      }
      for (; dj + 4 <= p.pw; dj += 4) {  // four independent loads in flight, adds in order
        float v0[8], v1[8], v2[8], v3[8];
        Vec8<TX>::load(src + (int64_t)(dj + 0) * p.D, v0);
        Vec8<TX>::load(src + (int64_t)(dj + 1) * p.D, v1);
        Vec8<TX>::load(src + (int64_t)(dj + 2) * p.D, v2);
        Vec8<TX>::load(src + (int64_t)(dj + 3) * p.D, v3);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = (((s[e] + v0[e]) + v1[e]) + v2[e]) + v3[e];
      }
      for (; dj < p.pw; ++dj) {
        float v[8];
        Vec8<TX>::load(src + (int64_t)dj * p.D, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[(r * POOL_CX + tx) * 8 + e] = s[e];
    }
  }
  __syncthreads();
  if (ty == 0 && cx < C) {
    float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int dt = 0; dt < p.pt; ++dt) {
      float plane[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int di = 0; di < p.ph; ++di) {
        const int r = dt * p.ph + di;
#pragma unroll
        for (int e = 0; e < 8; ++e) plane[e] = plane[e] + part[(r * POOL_CX + tx) * 8 + e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tot[e] = tot[e] + plane[e];
    }
    const float P = (float)(p.pt * p.ph * p.pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) tot[e] = tot[e] / P;
    TO* out = reinterpret_cast<TO*>(p.out);
    Vec8<TO>::store(out + ((int64_t)b * M + m) * p.D + cx * 8, tot);
  }
}

// Fallback for windows with more than POOL_MAXR (dt, di) rows: one thread per
// chunk walks the whole window, same order.
template <typename TX, typename TO>
__global__ void __launch_bounds__(256) pool_serial_kernel(PoolParams p) {
  const int C = p.D / 8;
  const int M = p.FT * p.HI * p.WJ;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)p.B * M * C) return;
  const int cx = (int)(gid % C);
  const int64_t bm = gid / C;
  const int b = (int)(bm / M), m = (int)(bm % M);
  const int T = m / (p.HI * p.WJ), I = (m / p.WJ) % p.HI, J = m % p.WJ;
  const TX* x = reinterpret_cast<const TX*>(p.x);
  const int64_t N = (int64_t)p.F * p.H * p.W;
  float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int dt = 0; dt < p.pt; ++dt) {
    float plane[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int di = 0; di < p.ph; ++di) {
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const int t = T * p.pt + dt, i = I * p.ph + di;
      const TX* src = x + ((int64_t)b * N + ((int64_t)t * p.H + i) * p.W + (int64_t)J * p.pw) * p.D + cx * 8;
      for (int dj = 0; dj < p.pw; ++dj) {
        float v[8];
        Vec8<TX>::load(src + (int64_t)dj * p.D, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) plane[e] = plane[e] + s[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tot[e] = tot[e] + plane[e];
  }
  const float P = (float)(p.pt * p.ph * p.pw);
#pragma unroll
  for (int e = 0; e < 8; ++e) tot[e] = tot[e] / P;
  TO* out = reinterpret_cast<TO*>(p.out);
  Vec8<TO>::store(out + ((int64_t)b * M + m) * p.D + cx * 8, tot);
}

template <typename TX, typename TO>
static hipError_t run_pool(const PoolParams& p, hipStream_t s) {
  const int C = p.D / 8;
  const int M = p.FT * p.HI * p.WJ;
  const int R = p.pt * p.ph;
  if ((int64_t)p.B * M == 0) return hipSuccess;
  if (R <= POOL_MAXR) {
    int ny = R;
    while (ny * POOL_CX > 1024) ny = (ny + 1) / 2;
    dim3 grid(p.B * M, (C + POOL_CX - 1) / POOL_CX);
    hipLaunchKernelGGL((pool_kernel<TX, TO>), grid, dim3(POOL_CX, ny), (size_t)R * POOL_CX * 8 * sizeof(float), s,
                       p);
  } else {
    const int64_t total = (int64_t)p.B * M * C;
    hipLaunchKernelGGL((pool_serial_kernel<TX, TO>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const PoolDesc& d, hipStream_t s) {
  PoolParams p;
  p.x = d.x; p.out = d.out;
  p.B = d.B; p.F = d.F; p.H = d.H; p.W = d.W; p.D = d.D;
  p.pt = d.pt; p.ph = d.ph; p.pw = d.pw;
  p.FT = d.F / d.pt; p.HI = d.H / d.ph; p.WJ = d.W / d.pw;
  if (d.x_f32) return d.out_f32 ? run_pool<float, float>(p, s) : run_pool<float, uint16_t>(p, s);
  return d.out_f32 ? run_pool<uint16_t, float>(p, s) : run_pool<uint16_t, uint16_t>(p, s);
}

// ----------------------------------------------------------------------------
// Proxy selection: one thread per 8 channels of one proxy copies the chunk of
// the window token at the proxy's offset (bf16 -> fp32 exact, fp32 -> bf16
// rounded to nearest even, the same rounding as the pooled proxies).
// ----------------------------------------------------------------------------
template <typename TX, typename TO>
__global__ void __launch_bounds__(256) select_kernel(PoolParams p, const int32_t* offsets) {
  const int C = p.D / 8;
  const int M = p.FT * p.HI * p.WJ;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)p.B * M * C) return;
  const int cx = (int)(gid % C);
  const int64_t bm = gid / C;
  const int b = (int)(bm / M), m = (int)(bm % M);
  const int T = m / (p.HI * p.WJ), I = (m / p.WJ) % p.HI, J = m % p.WJ;
  const int P = p.pt * p.ph * p.pw;
  int o = 0;
  if (offsets) {
    o = offsets[bm] % P;
    o += o < 0 ? P : 0;
  }
  const int dt = o / (p.ph * p.pw), di = (o / p.pw) % p.ph, dj = o % p.pw;
  const int64_t N = (int64_t)p.F * p.H * p.W;
  const int64_t n = ((int64_t)(T * p.pt + dt) * p.H + (I * p.ph + di)) * p.W + (J * p.pw + dj);
  float v[8];
  Vec8<TX>::load(reinterpret_cast<const TX*>(p.x) + ((int64_t)b * N + n) * p.D + cx * 8, v);
  Vec8<TO>::store(reinterpret_cast<TO*>(p.out) + bm * p.D + cx * 8, v);
}

hipError_t launch_select(const PoolDesc& d, const int32_t* offsets, hipStream_t s) {
  PoolParams p;
  p.x = d.x; p.out = d.out;
  p.B = d.B; p.F = d.F; p.H = d.H; p.W = d.W; p.D = d.D;
  p.pt = d.pt; p.ph = d.ph; p.pw = d.pw;
  p.FT = d.F / d.pt; p.HI = d.H / d.ph; p.WJ = d.W / d.pw;
  const int64_t total = (int64_t)p.B * p.FT * p.HI * p.WJ * (p.D / 8);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (d.x_f32) {
    if (d.out_f32) hipLaunchKernelGGL((select_kernel<float, float>), grid, dim3(256), 0, s, p, offsets);
    else hipLaunchKernelGGL((select_kernel<float, uint16_t>), grid, dim3(256), 0, s, p, offsets);
  } else {
    if (d.out_f32) hipLaunchKernelGGL((select_kernel<uint16_t, float>), grid, dim3(256), 0, s, p, offsets);
    else hipLaunchKernelGGL((select_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, p, offsets);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// 3D cyclic roll: y[t,i,j] = x[(t+st) mod F, (i+sh) mod H, (j+sw) mod W].
// A roll moves whole grid rows (b, t, i) and rotates the tokens inside a row,
// so workgroups are laid out per destination row: the source row is one
// scalar computation per workgroup, and inside the row the source of vector
// e is e + sw * vec_per_tok, wrapped once by the row length (no division per
// vector). Each thread moves RU vectors (16 bytes each) with all its loads in
// flight before the stores.
// ----------------------------------------------------------------------------
struct RollParams {
  const uint4* x;
  uint4* y;
  int B, F, H, W;
  int vec_per_tok;
  int st, sh, sw;
};

constexpr int RU = 4;

__device__ __forceinline__ int roll_src(int e, int shift, int rowlen) {
  int se = e + shift;
  return se >= rowlen ? se - rowlen : se;
}

__global__ void __launch_bounds__(256) roll_kernel(RollParams p) {
  // destination row (b, t, i) = blockIdx.y + gridDim.y * blockIdx.z (the grid
  // splits rows over two dimensions so that any count fits)
  const int row = blockIdx.y + gridDim.y * blockIdx.z;
  if (row >= p.B * p.F * p.H) return;
  const int i = row % p.H, t = (row / p.H) % p.F, b = row / (p.H * p.F);
  int ts = t + p.st; ts -= ts >= p.F ? p.F : 0;
  int is = i + p.sh; is -= is >= p.H ? p.H : 0;
  const int rowlen = p.W * p.vec_per_tok, shift = p.sw * p.vec_per_tok;
  const uint4* src = p.x + (int64_t)((b * p.F + ts) * p.H + is) * rowlen;
  uint4* dst = p.y + (int64_t)row * rowlen;
  // four 16-byte vectors per lane, all loads issued before any store; the
  // indices of lanes past the row end are clamped to its last vector so the
  // loads need no branch, only the stores are predicated
  const int e = blockIdx.x * (256 * RU) + threadIdx.x, last = rowlen - 1;
  const uint4 v0 = src[roll_src(min(e, last), shift, rowlen)];
  const uint4 v1 = src[roll_src(min(e + 256, last), shift, rowlen)];
  const uint4 v2 = src[roll_src(min(e + 512, last), shift, rowlen)];
  const uint4 v3 = src[roll_src(min(e + 768, last), shift, rowlen)];
  if ((blockIdx.x + 1) * (256 * RU) <= rowlen) {
    // whole chunk inside the row (a workgroup-uniform test): plain stores
    dst[e] = v0; dst[e + 256] = v1; dst[e + 512] = v2; dst[e + 768] = v3;
  } else {
    if (e < rowlen) dst[e] = v0;
    if (e + 256 < rowlen) dst[e + 256] = v1;
    if (e + 512 < rowlen) dst[e + 512] = v2;
    if (e + 768 < rowlen) dst[e + 768] = v3;
  }
}

hipError_t launch_roll(const RollDesc& d, hipStream_t s) {
  RollParams p;
  p.x = reinterpret_cast<const uint4*>(d.x);
  p.y = reinterpret_cast<uint4*>(d.y);
  p.B = d.B; p.F = d.F; p.H = d.H; p.W = d.W;
  p.vec_per_tok = d.f32 ? d.D / 4 : d.D / 8;
  p.st = d.st; p.sh = d.sh; p.sw = d.sw;
  const int64_t rows = (int64_t)d.B * d.F * d.H;
  const int64_t rowlen = (int64_t)d.W * p.vec_per_tok;
  if (rows == 0 || rowlen == 0) return hipSuccess;
  // the kernel indexes rows and in-row vectors in 32 bits
  if (rows > INT32_MAX || rowlen > INT32_MAX - 1024) return hipErrorInvalidValue;
  const int64_t gy = rows < 65535 ? rows : 65535, gz = (rows + gy - 1) / gy;
  if (gz > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rowlen + 256 * RU - 1) / (256 * RU)), (unsigned)gy, (unsigned)gz);
  hipLaunchKernelGGL(roll_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ptdit
