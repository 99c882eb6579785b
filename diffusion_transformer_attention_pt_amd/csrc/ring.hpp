// DMA-ring helpers shared by the projection GEMMs (gemm.hip) and the fused
// projection + window attention (wfused.hip), gfx950.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace ptdit {

template <int N>
__device__ __forceinline__ void wait_vm_dyn(int n) {
  if constexpr (N == 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (n >= N) wait_vm_lgkm0<N>();
    else wait_vm_dyn<N - 1>(n);
  }
}

// Barrier that orders LDS traffic without draining the in-flight DMA ring:
// the wave's own LDS operations complete first (s_waitcnt lgkmcnt(0); this
// target does not wait for them at s_barrier, and a ds_write of 64 lanes
// lands in passes of 16), the vector-memory counter is left alone. The
// compiler-level "memory" clobbers keep LDS accesses on their side.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Fragment addressing: a wave reads fragment j of 16 rows at row0 + 16*j,
// row0 = (wave's first row) + lane % 16, with the wave's first row a multiple
// of 8. The swizzles below depend on row bits 1..2 (bf16) or 0..2 (fp32),
// which 16*j never changes, so a lane computes its slot offset once (lofs)
// and fragment j sits at a constant distance from it: LDS reads then use
// immediate offsets from one base register per ring slot.
template <typename TA> struct DmaA;
template <> struct DmaA<uint16_t> {
  static constexpr int CPR = 4;  // 16-byte chunks per row per k-slice
  __device__ static int chunk(int row, int p) { return p ^ ((row >> 1) & 3); }
  __device__ static int lofs(int row0, int g) { return row0 * 4 + (g ^ ((row0 >> 1) & 3)); }
  // fragment j (rows row0 + 16 j, 8-value group g) -> 8 bf16
  __device__ static uint4 frag(const uint4* base, int lofs, int j) { return base[lofs + j * 64]; }
};
template <> struct DmaA<float> {
  static constexpr int CPR = 8;
  __device__ static int chunk(int row, int p) { return p ^ (row & 7); }
  __device__ static int lofs(int row0, int g) { return row0 * 8 + ((2 * g) ^ (row0 & 7)); }
  __device__ static uint4 frag(const uint4* base, int lofs, int j) {
    const uint4 lo = base[lofs + j * 128];
    const uint4 hi = base[(lofs ^ 1) + j * 128];  // chunk 2g+1 of the same row
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    auto cv = [](unsigned a, unsigned b) {
      return __builtin_bit_cast(unsigned, __builtin_convertvector(f2{__uint_as_float(a), __uint_as_float(b)}, bf2));
    };
    return uint4{cv(lo.x, lo.y), cv(lo.z, lo.w), cv(hi.x, hi.y), cv(hi.z, hi.w)};
  }
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace ptdit
