// Window and shifted-window self-attention with the Q/K/V projection fused
// in (bf16, head width 72): the TCM attentions of the Qihoo-T2X reading note,
// section 3 "Method", Eq. TCM, and the module table's attn1 on window-grouped
// tokens with window_shift / window_Ishift around it.
//
// One workgroup takes 128 window slots (128 / L whole windows of L tokens of
// the zero-padded, rolled grid) and one pair of heads.
//
// Phase 1 projects the slots' tokens onto the Q, K and V columns of both
// heads: 3 x 144 = 432 output columns, 27 column blocks of 16 (V's first,
// then Q's and K's). It is the ping-pong DMA-ring GEMM of gemm_pp_kernel (8
// waves in two groups one phase apart, a 4-slot ring of 32-wide k-slices fed
// by global_load_lds) on a 128 x 448 tile: waves of 64 rows x 7 blocks, the
// 28th block a copy of the first whose result is never used. V's blocks are
// computed transposed (tokens as the first MFMA operand), which leaves each
// lane 4 consecutive tokens of one channel, as the V^T staging wants them. The A rows are gathered through the
// window map (roll and zero padding applied per row), so nothing is
// materialised; rows of pad slots load any real row and are zeroed after the
// contraction, which leaves their K and V equal to the biases.
//
// Phase 2 writes Q and K row-major and V transposed (bf16) into the drained
// ring, then every wave computes 32 queries of one (window, head): S^T = K Q^T
// on the matrix cores, the boundary mask from per-slot region labels, an exact
// one-pass softmax over the window's L keys held in registers, O^T = V^T P^T.
// O goes back over the wave's own Q rows and leaves as whole 288-byte token
// rows (token-major bf16, the output projection's operand). Q, K and V never
// reach HBM, except in the KEEP instance (training forward), which also
// copies the staged Q/K/V of the real tokens out head-major for the backward.
// The arithmetic is that of the unfused path (same k order in the
// projection, same rounding to bf16, same attention steps), so both give the
// same attention output.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace ptdit {

namespace {

constexpr int WF_BM = 128;           // window slots per workgroup
constexpr int WF_DH = 72;            // head width
constexpr int WF_CPH = 2 * WF_DH;    // columns of one of Q/K/V for the head pair
constexpr int WF_NWR = 3 * WF_CPH;   // W rows per tile (432)
// LDS row pitch of staged Q / K / O (elements): 152 = 76 dwords, 12 mod 32
// banks, so the 16 rows of a 16-byte fragment read fall in distinct banks
// (a pitch of 144, 8 mod 32, repeats every 4 rows)
constexpr int WF_QP = WF_CPH + 8;
constexpr int WF_NBLK = WF_NWR / 16; // real column blocks (27)
constexpr int WF_WM = 2, WF_WN = 4, WF_NW = 8;
constexpr int WF_FM = WF_BM / WF_WM / 16;  // 4 row blocks per wave
constexpr int WF_FN = 7;                   // column blocks per wave (4 x 7 = 28)
constexpr int WF_SA = WF_BM * 4;           // 16-byte LDS slots of A per k-slice
constexpr int WF_SB = WF_NWR * 4;          // ... of W
constexpr int WF_IA = WF_SA / 64, WF_IT = WF_IA + WF_SB / 64;  // DMA instructions per slice
constexpr int WF_MAXI = (WF_IT + WF_NW - 1) / WF_NW;
constexpr int WF_PK_SLICE = WF_SB * 16;    // bytes of one packed weight k-slice (27 KB)
static_assert(WF_WN * WF_FN == WF_NBLK + 1, "one spare column block");

// staging of one window (both heads of the pair) in the drained ring (bytes)
template <int L>
struct WfStage {
  static constexpr int QB = L * WF_QP * 2;            // Q or K [L][144 + 8]
  static constexpr int VTP = L + 4;                   // V^T row pitch (elements)
  static constexpr int VB = WF_CPH * VTP * 2;         // V^T [144][L+4]
  // bytes per ring slot: Q and K of one window (L = 64) or two (L = 32), Q or
  // K alone (L = 128); V^T of one or two windows
  static constexpr int QK_SLOT = L == 128 ? QB : (L == 64 ? 2 * QB : 4 * QB);
  static constexpr int VT_SLOT = L == 32 ? 2 * VB : VB;
  static constexpr int SLOT_BYTES = QK_SLOT > VT_SLOT ? QK_SLOT : VT_SLOT;
  static_assert(L == 32 || L == 64 || L == 128, "window sizes with a fused kernel");
};

}  // namespace

struct WFusedParams {
  const uint16_t* X;     // [B][N][D] bf16
  const uint16_t* Wpk;   // w_qkv packed by wfused_pack_kernel: [head pair][k-slice][WF_SB 16-byte chunks]
  const uint16_t* bias;  // b_qkv [3D] bf16 or null
  uint16_t* O;           // [B][N][D] bf16
  uint16_t* QKV;         // KEEP: head-major Q/K/V [B][3][heads][N][72] bf16 of the real tokens
  int N, D;
  int F, H, Wd;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  int slots;       // B * Fp * Hp * Wp
  int row_tiles;   // ceil(slots / 128)
  int head_pairs;  // heads / 2
  float sl2;       // 1/sqrt(dh) * log2(e)
};

__device__ __forceinline__ int wf_region(int k, int L, int w, int s) {
  return k < L - w ? 0 : (k < L - s ? 1 : 2);
}

template <int L, bool MASKED, bool KEEP>
__global__ void __launch_bounds__(512, 1) wfused_kernel(WFusedParams p) {
  using SG = WfStage<L>;
  constexpr int SLOT = (WF_SA + WF_SB) * 16 > SG::SLOT_BYTES ? (WF_SA + WF_SB) : (SG::SLOT_BYTES + 15) / 16;
  __shared__ uint4 ring0[SLOT];
  __shared__ uint4 ring1[SLOT];
  __shared__ uint4 ring2[SLOT];
  __shared__ uint4 ring3[SLOT];
  __shared__ __attribute__((aligned(16))) int grow_s[WF_BM];  // global token row b*N + tok, or -1 (pad / past the grid)
  __shared__ __attribute__((aligned(16))) int lab_s[WF_BM];
  auto slot = [&](auto sI) -> uint4* {
    constexpr int sl = (decltype(sI)::value % 4 + 4) % 4;
    if constexpr (sl == 0) return ring0;
    else if constexpr (sl == 1) return ring1;
    else if constexpr (sl == 2) return ring2;
    else return ring3;
  };


  // XCD-aware tile order: block i runs on XCD i % 8; each XCD walks a
  // contiguous range of logical tiles. Logical tiles group GP head pairs
  // (2 when the pair count is even) with every row tile, the pair index
  // fastest: with 8 head pairs, two XCDs share a group, each takes half the
  // row tiles, keeps the group's 864 weight rows (2 MB) in its L2 and reads
  // each of its token rows once (the two pairs' workgroups of a row tile run
  // side by side).
  const int ntiles = p.row_tiles * p.head_pairs;
  // persistent: workgroup b takes tiles b, b + grid, ... (one workgroup per
  // CU, so a tile's output stores drain while the next tile's first slices
  // load); b + k*grid keeps b's XCD (grid % 8 == 0)
  for (int bid = blockIdx.x; bid < ntiles; bid += gridDim.x) {
  // thread indices re-derived per tile from an opaque copy of the thread id:
  // nothing tile-invariant is hoisted out of the loop and kept live across
  // the main loop (which would spill)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // wm is the ping-pong group; SIMD wave % 4 holds one of each
  const int g = lane >> 4, lr = lane & 15;
  int hp, rt;
  {
    const int q = ntiles >> 3, rem = ntiles & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    const int logical = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
    const int GP = (p.head_pairs & 1) ? 1 : 2;
    const int grp = logical / (p.row_tiles * GP), in = logical - grp * p.row_tiles * GP;
    rt = in / GP;
    hp = grp * GP + (in - rt * GP);
  }

  // the previous tile's last LDS reads (the output copy) are done before its
  // maps and ring are overwritten
  if (bid != (int)blockIdx.x) __syncthreads();
  // slot -> token map of the tile's rows (roll by -shift on the padded grid)
  if (tid < WF_BM) {
    const int s = rt * WF_BM + tid;
    int grow = -1, lab = -1;
    if (s < p.slots) {
      const int padN = p.Fp * p.Hp * p.Wp;
      const int b = s / padN, rem = s - b * padN;
      const int win = rem / L, e = rem - win * L;
      const int nWh = p.Hp / p.wh, nWw = p.Wp / p.ww;
      const int Tw = win / (nWh * nWw), Iw = (win / nWw) % nWh, Jw = win % nWw;
      const int a = e / (p.wh * p.ww), c = (e / p.ww) % p.wh, f = e % p.ww;
      const int rt_ = Tw * p.wt + a, ri = Iw * p.wh + c, rj = Jw * p.ww + f;
      int ot = rt_ + p.st; ot -= ot >= p.Fp ? p.Fp : 0;
      int oi = ri + p.sh; oi -= oi >= p.Hp ? p.Hp : 0;
      int oj = rj + p.sw; oj -= oj >= p.Wp ? p.Wp : 0;
      if (ot < p.F && oi < p.H && oj < p.Wd) grow = b * p.N + (ot * p.H + oi) * p.Wd + oj;
      lab = wf_region(rt_, p.Fp, p.wt, p.st) * 9 + wf_region(ri, p.Hp, p.wh, p.sh) * 3 +
            wf_region(rj, p.Wp, p.ww, p.sw);
    }
    grow_s[tid] = grow;
    lab_s[tid] = lab;
  }
  __syncthreads();

  // DMA plan: instruction j of a slice moves 64 16-byte chunks, A rows for
  // j < WF_IA (4 chunks a row, swizzled as DmaA<bf16>), W rows after; wave w
  // owns j = w + i*8 and repeats its first instruction to make WF_MAXI. The
  // weights come packed: the tile's k-slice of its 432 weight rows is one
  // contiguous 27 KB run already in LDS order, so each W instruction reads
  // 1 KB of whole cache lines (a row-major slice would fetch 64 bytes from
  // each of 16 rows, half lines, which the L2 serves at about two thirds of
  // the whole-line rate when every CU streams).
  const int KT = p.D / 32;  // multiple of 4, >= 8 (host check)
  const char* const a_base = reinterpret_cast<const char*>(p.X);
  const char* const w_base = reinterpret_cast<const char*>(p.Wpk) + (size_t)hp * KT * WF_PK_SLICE;
  bool is_a[WF_MAXI];
  uint32_t voff[WF_MAXI];
  int dst[WF_MAXI];
#pragma unroll
  for (int i = 0; i < WF_MAXI; ++i) {
    const int j0 = wave + i * WF_NW;
    const int j = j0 < WF_IT ? j0 : wave;
    is_a[i] = j < WF_IA;
    if (j < WF_IA) {
      const int sl = j * 64 + lane, row = sl >> 2, pp = sl & 3;
      const int gr = max(grow_s[row], 0);  // pad slots load row 0 (zeroed later)
      voff[i] = (uint32_t)gr * (uint32_t)(p.D * 2) + (uint32_t)((pp ^ ((row >> 1) & 3)) * 16);
      dst[i] = j * 64;
    } else {
      voff[i] = (uint32_t)((j - WF_IA) * 1024 + lane * 16);
      dst[i] = WF_SA + (j - WF_IA) * 64;
    }
  }
  auto issue = [&](int kt, uint4* st) {
    const char* const ak = a_base + kt * 64;
    const char* const wk = w_base + kt * WF_PK_SLICE;
#pragma unroll
    for (int i = 0; i < WF_MAXI; ++i) PTDIT_GLDS16((is_a[i] ? ak : wk) + voff[i], st + dst[i]);
  };

  floatx4 acc[WF_FN][WF_FM];
#pragma unroll
  for (int i = 0; i < WF_FN; ++i)
#pragma unroll
    for (int j = 0; j < WF_FM; ++j) acc[i][j] = zero4();
  // biases of this lane's columns, loaded before the main loop (the staging
  // would otherwise wait on one global round trip per column block): V blocks
  // hold one channel per lane (cb + lr), Q/K blocks four (cb + 4g .. +3)
  uint2 biasp[WF_FN];
#pragma unroll
  for (int i = 0; i < WF_FN; ++i) {
    const int b = wn * WF_FN + i, tg = b / 9, cb = (b - tg * 9) * 16;
    biasp[i] = uint2{0u, 0u};
    if (p.bias && b < WF_NBLK) {
      if (tg == 0) biasp[i].x = p.bias[2 * p.D + hp * WF_CPH + cb + lr];
      else biasp[i] = *reinterpret_cast<const uint2*>(p.bias + (tg - 1) * p.D + hp * WF_CPH + cb + 4 * g);
    }
  }

  const int lofs_a = DmaA<uint16_t>::lofs(wm * 64 + lr, g);
  const int lofs_w = WF_SA + DmaA<uint16_t>::lofs(wn * (WF_FN * 16) + lr, g);
  // the spare block (wave column 3, block 6) reads block 0's rows
  const int lofs_w6 = wn == 3 ? WF_SA + DmaA<uint16_t>::lofs(lr, g) : lofs_w + 6 * 64;
  uint4 wf[WF_FN], xf[WF_FM];
  auto read_frags = [&](const uint4* st) {
#pragma unroll
    for (int i = 0; i < WF_FN - 1; ++i) wf[i] = DmaA<uint16_t>::frag(st, lofs_w, i);
    wf[WF_FN - 1] = st[lofs_w6];
#pragma unroll
    for (int j = 0; j < WF_FM; ++j) xf[j] = DmaA<uint16_t>::frag(st, lofs_a, j);
  };
  // V's column blocks (the first 9 of the tile: all 7 of wave column 0, the
  // first 2 of wave column 1) are computed transposed, tokens as the first
  // operand, so a lane holds 4 consecutive tokens of one channel: the V^T
  // staging is then one 8-byte write per accumulator block
  const int nsw = wn == 0 ? WF_FN : (wn == 1 ? 2 : 0);
  auto mfmas = [&](auto nswI) {
    constexpr int NSW = decltype(nswI)::value;
#pragma unroll
    for (int i = 0; i < WF_FN; ++i)
#pragma unroll
      for (int j = 0; j < WF_FM; ++j)
        acc[i][j] = i < NSW ? mfma_bf16(xf[j], wf[i], acc[i][j]) : mfma_bf16(wf[i], xf[j], acc[i][j]);
  };
  // body of slice k (slot t = k % 4), as gemm_pp_kernel: refill slot t-1 with
  // slice k+3, read slice k's fragments, wait for slice k+1, barrier, MFMAs,
  // wait, barrier
  auto body = [&](auto tI, auto issueI, auto wI, int k, auto nswI) {
    constexpr int t = decltype(tI)::value;
    if constexpr (decltype(issueI)::value) issue(k + 3, slot(std::integral_constant<int, t - 1>{}));
    read_frags(slot(std::integral_constant<int, t>{}));
    wait_vm_lgkm0<decltype(wI)::value>();
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(nswI);
    wait_vm_lgkm0<decltype(wI)::value>();
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // the whole main loop is instantiated once per transposed-block count, so
  // the choice is one uniform branch outside it
  auto main_loop = [&](auto nswI) {
    issue(0, slot(std::integral_constant<int, 0>{}));
    issue(1, slot(std::integral_constant<int, 1>{}));
    issue(2, slot(std::integral_constant<int, 2>{}));
    wait_vm_lgkm0<2 * WF_MAXI>();
    ring_barrier();
    if (wm == 1) ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
    using WS = std::integral_constant<int, 2 * WF_MAXI>;
    for (int k0 = 0; k0 < KT - 4; k0 += 4) {
      static_for<0, 4>([&](auto tI) { body(tI, std::true_type{}, WS{}, k0 + decltype(tI)::value, nswI); });
    }
    body(std::integral_constant<int, 0>{}, std::true_type{}, WS{}, KT - 4, nswI);
    body(std::integral_constant<int, 1>{}, std::false_type{}, std::integral_constant<int, WF_MAXI>{}, KT - 3, nswI);
    body(std::integral_constant<int, 2>{}, std::false_type{}, std::integral_constant<int, 0>{}, KT - 2, nswI);
    body(std::integral_constant<int, 3>{}, std::false_type{}, std::integral_constant<int, 0>{}, KT - 1, nswI);
  };
  if (nsw == WF_FN) main_loop(std::integral_constant<int, WF_FN>{});
  else if (nsw == 2) main_loop(std::integral_constant<int, 2>{});
  else main_loop(std::integral_constant<int, 0>{});
  if (wm == 0) ring_barrier();
  wait_vm_lgkm0<0>();
  ring_barrier();  // ring drained: every DMA landed, every fragment read retired

  // ------------------------------------------------------------ phase 2
  // Staging in the drained ring (bf16), per window w of the tile with its two
  // heads side by side: Q_w, K_w [L][144] row-major and V^T_w [144][L+4]
  // (row = head * 72 + d). Every lane's window is wave-uniform, so slot
  // bases are scalar and only offsets vary per lane.
  const auto qk_base = [&](int w) -> char* {   // Q_w (K_w follows, except L = 128)
    if constexpr (L == 32) return reinterpret_cast<char*>(w >> 1 ? ring1 : ring0) + (w & 1) * 2 * SG::QB;
    else if constexpr (L == 64) return reinterpret_cast<char*>(w ? ring1 : ring0);
    else return reinterpret_cast<char*>(ring0);
  };
  const auto k_base = [&](int w) -> char* {
    if constexpr (L == 128) return reinterpret_cast<char*>(ring1);
    else return qk_base(w) + SG::QB;
  };
  const auto vt_base = [&](int w) -> uint16_t* {
    if constexpr (L == 32)
      return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(w >> 1 ? ring3 : ring2) + (w & 1) * SG::VB);
    else if constexpr (L == 64) return reinterpret_cast<uint16_t*>(w ? ring3 : ring2);
    else return reinterpret_cast<uint16_t*>(ring2);
  };

  // which of this lane's rows are real tokens (pad slots and rows past the
  // grid stage their bias only), read once: bit j for the Q/K layout (row
  // r0 + lr), bits 4j + e for the transposed V layout (rows r0 + 4g + e)
  uint32_t real_qk = 0, real_v = 0;
#pragma unroll
  for (int j = 0; j < WF_FM; ++j) {
    const int r0 = wm * 64 + j * 16;
    const int4 gr = *reinterpret_cast<const int4*>(&grow_s[r0 + 4 * g]);
    real_qk |= (grow_s[r0 + lr] >= 0 ? 1u : 0u) << j;
    real_v |= ((gr.x >= 0 ? 1u : 0u) | (gr.y >= 0 ? 2u : 0u) | (gr.z >= 0 ? 4u : 0u) | (gr.w >= 0 ? 8u : 0u))
              << (4 * j);
  }
  // accumulators (+ bias; pad rows zeroed first) -> bf16 staging
#pragma unroll
  for (int i = 0; i < WF_FN; ++i) {
    const int b = wn * WF_FN + i;  // wave-uniform
    if (b >= WF_NBLK) continue;
    const int tg = b / 9;          // tile column group: 0 V (transposed), 1 Q, 2 K
    const int cb = (b - tg * 9) * 16;
    if (tg == 0) {
      // lane: channel n of the pair's V, tokens r0 + 4g .. +3 of the block
      const int n = cb + lr;
      const float bvn = __uint_as_float((biasp[i].x & 0xffffu) << 16);
#pragma unroll
      for (int j = 0; j < WF_FM; ++j) {
        const int r0 = wm * 64 + j * 16;
        const int w = r0 / L;
        const uint32_t rv = real_v >> (4 * j);
        const float v0 = ((rv & 1u) ? acc[i][j][0] : 0.f) + bvn, v1 = ((rv & 2u) ? acc[i][j][1] : 0.f) + bvn;
        const float v2 = ((rv & 4u) ? acc[i][j][2] : 0.f) + bvn, v3 = ((rv & 8u) ? acc[i][j][3] : 0.f) + bvn;
        const uint2 pk = uint2{pack_bf2(v0, v1), pack_bf2(v2, v3)};
        *reinterpret_cast<uint2*>(vt_base(w) + n * SG::VTP + (r0 - w * L + 4 * g)) = pk;
      }
      continue;
    }
    const int gq = tg - 1;         // 0 Q, 1 K
    const int c = cb + 4 * g;      // column within the head pair (0..143)
    const uint2 bb = biasp[i];
    const float bv[4] = {__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u),
                         __uint_as_float(bb.y << 16), __uint_as_float(bb.y & 0xffff0000u)};
#pragma unroll
    for (int j = 0; j < WF_FM; ++j) {
      const int r0 = wm * 64 + j * 16;       // wave-uniform first row of the block
      const int w = r0 / L;                  // its window (uniform: 16 | L)
      const int e_ = r0 - w * L + lr;        // slot within the window
      const bool real = (real_qk >> j) & 1u;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (real ? acc[i][j][e] : 0.f) + bv[e];
      char* base = gq == 0 ? qk_base(w) : k_base(w);
      *reinterpret_cast<uint2*>(base + (e_ * WF_QP + c) * 2) = uint2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
    }
  }
  ring_barrier();
  if constexpr (KEEP) {
    // Q, K and V of the real tokens, head-major, from the staging: per
    // (slot, Q/K/V, head) 72 bf16 = 9 chunks of 16 bytes; a V chunk gathers 8
    // channel rows of the transposed V (adjacent lanes read adjacent slots)
    const int64_t heads = (int64_t)p.head_pairs * 2;
    for (int idx = tid; idx < WF_BM * 3 * 2 * 9; idx += 512) {
      const int sl = idx / 54, rem = idx - sl * 54;
      const int gq = rem / 18, hh = (rem / 9) & 1, ch = rem % 9;
      const int grow = grow_s[sl];
      if (grow < 0) continue;
      const int w = sl / L, e_ = sl - w * L;
      uint4 val;
      if (gq < 2) {
        val = *reinterpret_cast<const uint4*>((gq == 0 ? qk_base(w) : k_base(w)) +
                                              (e_ * WF_QP + hh * WF_DH + ch * 8) * 2);
      } else {
        const uint16_t* vs = vt_base(w) + (hh * WF_DH + ch * 8) * SG::VTP + e_;
        uint32_t u[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) u[k] = (uint32_t)vs[(2 * k) * SG::VTP] | ((uint32_t)vs[(2 * k + 1) * SG::VTP] << 16);
        val = uint4{u[0], u[1], u[2], u[3]};
      }
      const int64_t bb = grow / p.N, tok = grow - bb * p.N;
      *reinterpret_cast<uint4*>(p.QKV + (((bb * 3 + gq) * heads + hp * 2 + hh) * p.N + tok) * WF_DH + ch * 8) = val;
    }
    // every Q row read before a wave writes its O over its own Q rows
    ring_barrier();
  }

  // attention: wave -> 32 queries of one (window, head) pair
  constexpr int WPP = L / 32;  // waves per pair
  constexpr int NKT = L / 16;  // key tiles
  const int pr = wave / WPP, qb = (wave - pr * WPP) * 32;
  const int wi = pr >> 1, hh = pr & 1;
  char* const qs = qk_base(wi) + hh * WF_DH * 2;
  const char* const ks = k_base(wi) + hh * WF_DH * 2;
  const uint16_t* const vts = vt_base(wi);
  floatx4 sc[2][NKT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < NKT; ++t) sc[qt][t] = zero4();
  // S^T = K Q^T over the head's 72 dims in three 32-wide steps; dims past 72
  // (the other head's columns, or past the row) are masked to zero
#pragma unroll
  for (int kc = 0; kc < 3; ++kc) {
    const int dd = kc * 32 + 8 * g;
    const bool dok = dd < WF_DH;
    const int ddc = dok ? dd : 0;
    uint4 qf[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const uint4 v = *reinterpret_cast<const uint4*>(qs + ((qb + qt * 16 + lr) * WF_QP + ddc) * 2);
      qf[qt] = dok ? v : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const uint4 kv = *reinterpret_cast<const uint4*>(ks + ((t * 16 + lr) * WF_QP + ddc) * 2);
      const uint4 kf = dok ? kv : uint4{0, 0, 0, 0};
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) sc[qt][t] = mfma_bf16(kf, qf[qt], sc[qt][t]);
    }
  }
  float inv[2];
  floatx4 o[2][5];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = wi * L + qb + qt * 16 + lr;
    const int qlab = lab_s[qrow];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const int4 lab4 = *reinterpret_cast<const int4*>(&lab_s[wi * L + t * 16 + 4 * g]);
      const int labs[4] = {lab4.x, lab4.y, lab4.z, lab4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = !MASKED || labs[r] == qlab;
        const float v = ok ? sc[qt][t][r] * p.sl2 : -INFINITY;
        sc[qt][t][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));  // the four lane groups hold a query's keys
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (mx == -INFINITY) mx = 0.f;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(sc[qt][t][r] - mx);
        sc[qt][t][r] = e;
        rs += e;
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    inv[qt] = 1.f / rs;
#pragma unroll
    for (int dt = 0; dt < 5; ++dt) o[qt][dt] = zero4();
    // O^T = V^T P^T; rows past the head's 72 dims are computed on other data
    // (or clamped rows) and never stored
#pragma unroll
    for (int t0 = 0; t0 < NKT; t0 += 2) {
      const uint4 pf = uint4{pack_bf2(sc[qt][t0][0], sc[qt][t0][1]), pack_bf2(sc[qt][t0][2], sc[qt][t0][3]),
                             pack_bf2(sc[qt][t0 + 1][0], sc[qt][t0 + 1][1]),
                             pack_bf2(sc[qt][t0 + 1][2], sc[qt][t0 + 1][3])};
      const int kb = t0 * 16 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 5; ++dt) {
        const int vrow = min(hh * WF_DH + dt * 16 + lr, WF_CPH - 1);
        const uint16_t* row = vts + vrow * SG::VTP;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + kb);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + kb + 16);
        o[qt][dt] = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, pf, o[qt][dt]);
      }
    }
  }
  // O (bf16) over this wave's own Q rows: no other wave reads them (the other
  // head's waves read the other 72 columns)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    char* orow = qs + (qb + qt * 16 + lr) * WF_QP * 2;
#pragma unroll
    for (int dt = 0; dt < 5; ++dt) {
      const int dd = dt * 16 + 4 * g;
      if (dd < WF_DH)
        *reinterpret_cast<uint2*>(orow + dd * 2) =
            uint2{pack_bf2(o[qt][dt][0] * inv[qt], o[qt][dt][1] * inv[qt]),
                  pack_bf2(o[qt][dt][2] * inv[qt], o[qt][dt][3] * inv[qt])};
    }
  }
  ring_barrier();
  // O rows to HBM: wave v writes tile rows 16v .. 16v+15 (one window), each
  // row the pair's 144 channels = 18 chunks of 16 bytes
  {
    const int r0 = wave * 16, w = r0 / L;
    const char* ob = qk_base(w) + (r0 - w * L) * WF_QP * 2;
#pragma unroll
    for (int it = 0; it < (16 * 18 + 63) / 64; ++it) {
      const int idx = it * 64 + lane;
      if (idx < 16 * 18) {
        const int rr = idx / 18, ch = idx - rr * 18;
        const int grow = grow_s[r0 + rr];
        if (grow >= 0)
          *reinterpret_cast<uint4*>(p.O + (int64_t)grow * p.D + hp * WF_CPH + ch * 8) =
              *reinterpret_cast<const uint4*>(ob + (rr * WF_QP + ch * 8) * 2);
      }
    }
  }
  }  // tiles
}

// w_qkv -> the DMA order of the tiles' weight slices. Chunk s of the run of
// head pair hp and k-slice kt holds what the row-major plan would have placed
// at the tile's LDS position s: weight row wrow of tile row s >> 2 (tile rows:
// V's 144 columns of the pair, then Q's, then K's), 16-byte chunk
// (s & 3) ^ (((s >> 2) >> 1) & 3) of the k-slice (the DmaA<bf16> swizzle).
// One workgroup per (k-slice, head pair), k-slice fastest, so the two halves
// of each 128-byte weight line are read by neighbouring workgroups.
__global__ void __launch_bounds__(256) wfused_pack_kernel(const uint16_t* __restrict__ W, uint4* __restrict__ Wpk,
                                                          int D) {
  const int kt = blockIdx.x, hp = blockIdx.y, KT = gridDim.x;
  uint4* dst = Wpk + ((size_t)hp * KT + kt) * WF_SB;
  for (int s = threadIdx.x; s < WF_SB; s += 256) {
    const int row = s >> 2, pp = s & 3;
    const int tg = row / WF_CPH, cc = row - tg * WF_CPH;  // tile column groups: V, Q, K
    const int gq = tg == 0 ? 2 : tg - 1;                    // row group of w_qkv
    const int wrow = gq * D + hp * WF_CPH + cc;
    dst[s] = *reinterpret_cast<const uint4*>(W + (size_t)wrow * D + kt * 32 + (pp ^ ((row >> 1) & 3)) * 8);
  }
}

size_t wfused_packed_bytes(int D) { return (size_t)(D / WF_CPH) * (size_t)(D / 32) * WF_PK_SLICE; }

hipError_t launch_wfused_pack(const WFusedDesc& d, hipStream_t s) {
  if (!wfused_supported(d) || !d.w_packed) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wfused_pack_kernel, dim3((unsigned)(d.D / 32), (unsigned)(d.heads / 2)), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(d.w_qkv), reinterpret_cast<uint4*>(d.w_packed), d.D);
  return hipGetLastError();
}

bool wfused_supported(const WFusedDesc& d) {
  const int L = d.wt * d.wh * d.ww;
  if (L != 32 && L != 64 && L != 128) return false;
  if (d.dh != WF_DH || d.heads % 2 != 0 || d.D != d.heads * WF_DH) return false;
  if (d.D % 128 != 0 || d.D < 256) return false;                  // 4 | D/32 >= 8 slices
  const int64_t padN = (int64_t)d.Fp * d.Hp * d.Wp;
  const int64_t N = (int64_t)d.F * d.H * d.W;
  if ((int64_t)d.B * padN > INT32_MAX - WF_BM) return false;      // slot indices in 32 bits
  // 32-bit byte offsets of X rows and of W rows from their bases
  if ((int64_t)d.B * N * d.D * 2 >= ((int64_t)1 << 31)) return false;
  if ((int64_t)3 * d.D * d.D * 2 >= ((int64_t)1 << 31)) return false;
  return true;
}

// compute units of the current device (one persistent workgroup each)
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int L, bool M, bool K>
static hipError_t run_wfused(const WFusedParams& p, hipStream_t s) {
  const int ntiles = p.row_tiles * p.head_pairs;
  // a multiple of 8 workgroups (the XCD count), at most one per CU
  int grid = device_cus() / 8 * 8;
  if (grid < 8) grid = 8;
  if (grid > ntiles) grid = ntiles;
  hipLaunchKernelGGL((wfused_kernel<L, M, K>), dim3((unsigned)grid), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wfused(const WFusedDesc& d, hipStream_t s) {
  if (!wfused_supported(d) || !d.w_packed) return hipErrorInvalidValue;
  if (d.B == 0) return hipSuccess;
  WFusedParams p;
  p.X = reinterpret_cast<const uint16_t*>(d.X);
  p.Wpk = reinterpret_cast<const uint16_t*>(d.w_packed);
  p.bias = reinterpret_cast<const uint16_t*>(d.b_qkv);
  p.O = reinterpret_cast<uint16_t*>(d.O);
  p.QKV = reinterpret_cast<uint16_t*>(d.qkv_out);
  p.N = d.F * d.H * d.W;
  p.D = d.D;
  p.F = d.F; p.H = d.H; p.Wd = d.W;
  p.wt = d.wt; p.wh = d.wh; p.ww = d.ww;
  p.st = d.st; p.sh = d.sh; p.sw = d.sw;
  p.Fp = d.Fp; p.Hp = d.Hp; p.Wp = d.Wp;
  p.slots = d.B * d.Fp * d.Hp * d.Wp;
  p.row_tiles = (p.slots + WF_BM - 1) / WF_BM;
  p.head_pairs = d.heads / 2;
  p.sl2 = d.scale * 1.4426950408889634f;
  const bool masked = (d.st | d.sh | d.sw) != 0;
  const int L = d.wt * d.wh * d.ww;
  if (p.QKV) {  // the backward's copy of Q/K/V as well
    if (L == 32) return masked ? run_wfused<32, true, true>(p, s) : run_wfused<32, false, true>(p, s);
    if (L == 64) return masked ? run_wfused<64, true, true>(p, s) : run_wfused<64, false, true>(p, s);
    return masked ? run_wfused<128, true, true>(p, s) : run_wfused<128, false, true>(p, s);
  }
  if (L == 32) return masked ? run_wfused<32, true, false>(p, s) : run_wfused<32, false, false>(p, s);
  if (L == 64) return masked ? run_wfused<64, true, false>(p, s) : run_wfused<64, false, false>(p, s);
  return masked ? run_wfused<128, true, false>(p, s) : run_wfused<128, false, false>(p, s);
}

}  // namespace ptdit
