// Calibration kernels: the ceilings this box actually sustains, against
// which the benchmark prices its kernels beside the published peaks.
//   mfma_loop_kernel  back-to-back v_mfma_f32_16x16x32_bf16 on register
//                     operands (8 independent accumulator chains per wave,
//                     two waves per SIMD): the matrix rate at the clock the
//                     chip holds under a full matrix load
//   read_kernel       16-byte loads of a buffer, four in flight per lane,
//                     summed into one store per thread: the streaming HBM
//                     read rate (buffers larger than the 256 MB last-level
//                     cache read from HBM)
//   copy_kernel       a plain 16-byte-per-lane copy, the known-size reference
//                     for the hardware byte counters
#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

__global__ void __launch_bounds__(512) mfma_loop_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  // 8 accumulators in plain vector values and a 512-thread launch bound: the
  // loop is then the 8 MFMAs alone on VGPR accumulators (under a 256-thread
  // bound the compiler placed them in AGPRs and rotated them through moves
  // every iteration, which halved the measured rate)
  const uint4 ua = uint4{0x3f803f80u + (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const uint4 ub = uint4{0x3c003c00u, 0x3c003c00u + (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ua), b = __builtin_bit_cast(bf16x8_t, ub);
  floatx4 acc0 = zero4(), acc1 = zero4(), acc2 = zero4(), acc3 = zero4();
  floatx4 acc4 = zero4(), acc5 = zero4(), acc6 = zero4(), acc7 = zero4();
  for (int i = 0; i < iters; ++i) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc3, 0, 0, 0);
    acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc4, 0, 0, 0);
    acc5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc5, 0, 0, 0);
    acc6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc6, 0, 0, 0);
    acc7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc7, 0, 0, 0);
  }
  const floatx4 s4 = ((acc0 + acc1) + (acc2 + acc3)) + ((acc4 + acc5) + (acc6 + acc7));
  out[blockIdx.x * 256 + threadIdx.x] = s4[0] + s4[1] + s4[2] + s4[3];
}

__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ buf, int64_t n16, float* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
    acc ^= v0.x ^ v1.y ^ v2.z ^ v3.w ^ v0.w ^ v1.x ^ v2.y ^ v3.z;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = (float)(acc & 1u);
}

__global__ void __launch_bounds__(256) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int64_t calib_mfma_flop(int blocks, int iters) { return (int64_t)blocks * 4 * iters * 8 * 16 * 16 * 32 * 2; }

hipError_t launch_calib_mfma(int blocks, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* buf, int64_t bytes, int blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_calib_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace ptdit
