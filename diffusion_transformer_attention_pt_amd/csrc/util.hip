// Element-wise and layout kernels that chain the backward calls of the
// PT-DiT attention core (the block's gradient through its residuals, Eq. GIIM
// and Eq. TCM of the Qihoo-T2X reading note, section 3; trained at 2048^2,
// section 4):
//   heads_to_tokens_kernel  fp32 [B][G][heads][Ntok][dh] -> [B][Ntok][G*heads*dh]
//                           (the attention backward's dQ/dK/dV to the token-major
//                           gradient of the Q/K/V projection's output)
//   f32_to_bf16_kernel      fp32 -> bf16, round to nearest even (the operand
//                           precision of the matrix-core backward kernels)
//   add_f32_kernel          out = a + b (a residual's gradient joining a branch's)
// All are HBM-bound streams of 16-byte vectors.
#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

namespace {
constexpr int UT_NT = 256;
}

// one thread per 4 consecutive floats of a destination row (dh % 4 == 0, so
// the 4 never straddle a head)
__global__ void __launch_bounds__(UT_NT) heads_to_tokens_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                                int64_t rows, int Ntok, int G, int heads, int dh) {
  const int D = heads * dh, q4 = G * D / 4;
  const int64_t i = (int64_t)blockIdx.x * UT_NT + threadIdx.x;
  if (i >= rows * q4) return;
  const int64_t row = i / q4;
  const int col = (int)(i - row * q4) * 4;
  const int64_t b = row / Ntok, t = row - b * Ntok;
  const int g = col / D, hd = col - g * D, h = hd / dh, d = hd - h * dh;
  const float4 v = *reinterpret_cast<const float4*>(src + (((b * G + g) * heads + h) * Ntok + t) * dh + d);
  *reinterpret_cast<float4*>(dst + row * (int64_t)G * D + col) = v;
}

// 8 values per thread (n % 8 == 0)
__global__ void __launch_bounds__(UT_NT) f32_to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                            int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * UT_NT + threadIdx.x;
  if (i >= n8) return;
  const float4 a = *reinterpret_cast<const float4*>(src + 8 * i);
  const float4 b = *reinterpret_cast<const float4*>(src + 8 * i + 4);
  *reinterpret_cast<uint4*>(dst + 8 * i) =
      uint4{pack_bf2(a.x, a.y), pack_bf2(a.z, a.w), pack_bf2(b.x, b.y), pack_bf2(b.z, b.w)};
}

// 4 values per thread (n % 4 == 0); out may be a or b (element-wise)
__global__ void __launch_bounds__(UT_NT) add_f32_kernel(const float* a, const float* b, float* out, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * UT_NT + threadIdx.x;
  if (i >= n4) return;
  const float4 x = *reinterpret_cast<const float4*>(a + 4 * i);
  const float4 y = *reinterpret_cast<const float4*>(b + 4 * i);
  *reinterpret_cast<float4*>(out + 4 * i) = float4{x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w};
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + UT_NT - 1) / UT_NT); }

hipError_t launch_heads_to_tokens(const float* src, float* dst, int B, int G, int heads, int Ntok, int dh,
                                  hipStream_t s) {
  const int64_t rows = (int64_t)B * Ntok, n = rows * G * heads * dh / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(heads_to_tokens_kernel, dim3(blocks_for(n)), dim3(UT_NT), 0, s, src, dst, rows, Ntok, G, heads,
                     dh);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks_for(n / 8)), dim3(UT_NT), 0, s, src, dst, n / 8);
  return hipGetLastError();
}

hipError_t launch_add_f32(const float* a, const float* b, float* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_f32_kernel, dim3(blocks_for(n / 4)), dim3(UT_NT), 0, s, a, b, out, n / 4);
  return hipGetLastError();
}

}  // namespace ptdit
