// Backward pass of the PT-DiT attention core (Qihoo-T2X reading note,
// section 3 "Method": Eq. GIIM and Eq. TCM; the pages train the model at
// 2048^2, section 4). The gradients are those of the forward maps: with
// S = Q K^T * scale, A = softmax(S) over the allowed keys and O = A V,
//   dV = A^T dO,  dA = dO V^T,  dS = A * (dA - rowsum(A * dA)),
//   dQ = dS K * scale,  dK = dS^T Q * scale   (per head).
// The softmax is recomputed from Q and K (nothing of the forward is kept but
// its inputs), exactly: every kernel takes the row maximum and sum over all
// keys before it forms a weight. Arithmetic is fp32; the gradients are fp32.
//
//   window_bwd_kernel  WSA / SWSA core: one workgroup per (window, head,
//                      batch) with the window's Q, K, V, dO in LDS; a
//                      query-major phase (softmax statistics, dQ) and a
//                      key-major phase (dK, dV). The roll, padding and
//                      boundary mask are the forward's addressing; the
//                      gradient of a pad key/value slot (the bias b_k/b_v)
//                      is added into d_bias_kv.
//   dense_bwd_q_kernel proxy SA / cross-attention, query-major: statistics
//                      and dQ, keys streamed through LDS in 64-key chunks.
//   dense_bwd_kv_kernel key-major: dK, dV of 64 keys over one chunk of the
//                      queries (partial sums when the queries are split).
//   dense_bwd_reduce   fixed-order sum of the partials (deterministic).
//   pool_bwd_kernel    window average: dx[token] (+)= dP[its proxy] / P.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

namespace {

constexpr int BW_NT = 256;  // threads per workgroup of every kernel here

// sum / max over the G consecutive lanes of a group (G = 1, 2, 4, 8)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int region_of(int k, int L, int w, int s) {
  return k < L - w ? 0 : (k < L - s ? 1 : 2);
}

// Transposed write of chunk ch (8 elements) of the four rows s0 .. s0+3:
// t[(8 ch + e) * pitch + s0 + j] = element e of v[j], one 8-byte write per e.
__device__ __forceinline__ void put_quad_t(uint16_t* t, int pitch, int ch, int s0, const uint4 (&v)[4]) {
  const uint32_t a0[4] = {v[0].x, v[0].y, v[0].z, v[0].w}, a1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
  const uint32_t a2[4] = {v[2].x, v[2].y, v[2].z, v[2].w}, a3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = (e & 1) * 16;
    const uint32_t lo = ((a0[e >> 1] >> sh) & 0xffffu) | (((a1[e >> 1] >> sh) & 0xffffu) << 16);
    const uint32_t hi = ((a2[e >> 1] >> sh) & 0xffffu) | (((a3[e >> 1] >> sh) & 0xffffu) << 16);
    *reinterpret_cast<uint2*>(&t[(ch * 8 + e) * pitch + s0]) = uint2{lo, hi};
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// Window attention backward
// ----------------------------------------------------------------------------
struct WindowBwdParams {
  const void* QKV;       // [B][3][heads][N][dh]
  const void* bias_qkv;  // [3D] or null (pad keys/values are b_k/b_v, else 0)
  const void* dO;        // [B][N][D]
  void* dQKV;            // dQ, dK, dV: element (b, g, h, token, d) at
                         // b*o_bs + g*o_gs + h*o_hs + token*o_ts + d
  int64_t o_bs, o_gs, o_hs, o_ts;  // head-major [B][3][heads][N][dh] or token-major [B][N][3D]
  int out_bf16;          // dQKV elements bf16 (matrix-core kernels only), else fp32
  float* dbias_kv;       // [2][D], accumulated into; null when nothing pads
  int F, H, W, D, heads;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  float scale;
};

// four consecutive gradient elements (e % 4 == 0) as fp32, or rounded to bf16
// (round to nearest even) when the caller asked for bf16
__device__ __forceinline__ void bwd_store4(const WindowBwdParams& p, int64_t e, float4 v) {
  if (p.out_bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.dQKV) + e) = uint2{pack_bf2(v.x, v.y), pack_bf2(v.z, v.w)};
  else
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.dQKV) + e) = v;
}

template <typename T, int DH, int KEYS>
__global__ void __launch_bounds__(BW_NT) window_bwd_kernel(WindowBwdParams p) {
  constexpr int PI = DH + 1;           // LDS row pitch in floats (odd: rows spread over the banks)
  constexpr int G = BW_NT / KEYS;      // threads per query (phase 1) and per key (phase 2)
  constexpr int PER = KEYS / G;        // keys per thread in phase 1
  __shared__ float qs[KEYS * PI], ks[KEYS * PI], vs[KEYS * PI], gs[KEYS * PI];
  __shared__ int tok_s[KEYS], lab_s[KEYS];
  __shared__ float m_s[KEYS], l_s[KEYS], d_s[KEYS];

  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int nWh = p.Hp / p.wh, nWw = p.Wp / p.ww;
  const int Tw = blockIdx.x / (nWh * nWw), Iw = (blockIdx.x / nWw) % nWh, Jw = blockIdx.x % nWw;
  const int wsz = p.wt * p.wh * p.ww;
  const int64_t N = (int64_t)p.F * p.H * p.W;
  const bool masked = (p.st | p.sh | p.sw) != 0;

  // slot s of the window -> token (-1: pad, -2: past the window), region label
  __shared__ float padg[2 * DH];  // pad keys' gradients: d b_k (0 .. DH-1), d b_v
  for (int i = threadIdx.x; i < 2 * DH; i += blockDim.x) padg[i] = 0.f;
  bool my_pad = false;
  for (int s = tid; s < KEYS; s += BW_NT) {
    int tok = -2, lab = 0;
    if (s < wsz) {
      const int a = s / (p.wh * p.ww), c = (s / p.ww) % p.wh, e = s % p.ww;
      const int rt = Tw * p.wt + a, ri = Iw * p.wh + c, rj = Jw * p.ww + e;
      int ot = rt + p.st; ot -= ot >= p.Fp ? p.Fp : 0;
      int oi = ri + p.sh; oi -= oi >= p.Hp ? p.Hp : 0;
      int oj = rj + p.sw; oj -= oj >= p.Wp ? p.Wp : 0;
      tok = (ot < p.F && oi < p.H && oj < p.W) ? (ot * p.H + oi) * p.W + oj : -1;
      lab = region_of(rt, p.Fp, p.wt, p.st) * 9 + region_of(ri, p.Hp, p.wh, p.sh) * 3 +
            region_of(rj, p.Wp, p.ww, p.sw);
    }
    tok_s[s] = tok;
    lab_s[s] = lab;
    my_pad |= tok == -1;
  }
  // pad slots' key / value gradients are summed per channel in LDS, then
  // added to d_bias_kv once per workgroup (not once per pad key)
  const bool any_pad = __syncthreads_or(my_pad) != 0;

  const T* base = reinterpret_cast<const T*>(p.QKV);
  const int64_t hs = N * DH, gsz = (int64_t)p.heads * hs;
  const T* Qb = base + (int64_t)b * 3 * gsz + h * hs;
  const T* Kb = Qb + gsz;
  const T* Vb = Qb + 2 * gsz;
  const T* bias = reinterpret_cast<const T*>(p.bias_qkv);
  const T* dOb = reinterpret_cast<const T*>(p.dO) + (int64_t)b * N * p.D + h * DH;
  for (int idx = tid; idx < KEYS * DH; idx += BW_NT) {
    const int s = idx / DH, d = idx - s * DH;
    const int tok = tok_s[s];
    float q = 0.f, k = 0.f, v = 0.f, g = 0.f;
    if (tok >= 0) {
      q = ld1(Qb + (int64_t)tok * DH + d);
      k = ld1(Kb + (int64_t)tok * DH + d);
      v = ld1(Vb + (int64_t)tok * DH + d);
      g = ld1(dOb + (int64_t)tok * p.D + d);
    } else if (tok == -1 && bias) {
      k = ld1(bias + p.D + h * DH + d);
      v = ld1(bias + 2 * p.D + h * DH + d);
    }
    qs[s * PI + d] = q; ks[s * PI + d] = k; vs[s * PI + d] = v; gs[s * PI + d] = g;
  }
  __syncthreads();

  float* dQb = reinterpret_cast<float*>(p.dQKV) + (int64_t)b * p.o_bs + h * p.o_hs;
  float* dKb = dQb + p.o_gs;
  float* dVb = dQb + 2 * p.o_gs;

  // Phase 1 (query slot i, keys sub, sub+G, ...): statistics and dQ.
  {
    const int i = tid / G, sub = tid % G;
    const int tq = tok_s[i], lq = lab_s[i];
    float s[PER], dp[PER];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = sub + u * G;
      const bool ok = tok_s[j] != -2 && (!masked || lab_s[j] == lq);
      float a = 0.f, c = 0.f;
#pragma unroll 8
      for (int d = 0; d < DH; ++d) {
        a += qs[i * PI + d] * ks[j * PI + d];
        c += gs[i * PI + d] * vs[j * PI + d];
      }
      s[u] = ok ? a * p.scale : -INFINITY;
      dp[u] = c;
      mx = fmaxf(mx, s[u]);
    }
    mx = group_max<G>(mx);
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      s[u] = s[u] == -INFINITY ? 0.f : expf(s[u] - mx);
      l += s[u];
    }
    l = group_sum<G>(l);
    const float rl = 1.f / l;
    float dsum = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      s[u] *= rl;  // softmax weight
      dsum += s[u] * dp[u];
    }
    dsum = group_sum<G>(dsum);
    if (sub == 0) { m_s[i] = mx; l_s[i] = l; d_s[i] = dsum; }
    // dQ_i = scale * sum_j A_ij (dA_ij - D_i) k_j; each lane sums its keys,
    // the group adds the parts, lane sub writes dims sub, sub+G, ...
    for (int d0 = 0; d0 < DH; d0 += G) {
      float part[G];
#pragma unroll
      for (int e = 0; e < G; ++e) part[e] = 0.f;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int j = sub + u * G;
        const float w = s[u] * (dp[u] - dsum);
#pragma unroll
        for (int e = 0; e < G; ++e)
          if (d0 + e < DH) part[e] += w * ks[j * PI + d0 + e];
      }
#pragma unroll
      for (int e = 0; e < G; ++e) part[e] = group_sum<G>(part[e]);
      float mine = 0.f;
#pragma unroll
      for (int e = 0; e < G; ++e) mine = e == sub ? part[e] : mine;
      if (tq >= 0 && d0 + sub < DH) dQb[(int64_t)tq * p.o_ts + d0 + sub] = mine * p.scale;
    }
  }
  __syncthreads();

  // Phase 2 (key slot j, queries sub, sub+G, ...): dK, dV.
  {
    const int j = tid / G, sub = tid % G;
    const int tk = tok_s[j], lk = lab_s[j];
    float dk[DH], dv[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) { dk[d] = 0.f; dv[d] = 0.f; }
    if (tk != -2) {
      for (int i = sub; i < KEYS; i += G) {
        // only real queries carry a gradient (pad outputs are cropped)
        if (tok_s[i] < 0 || (masked && lab_s[i] != lk)) continue;
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) {
          a += qs[i * PI + d] * ks[j * PI + d];
          c += gs[i * PI + d] * vs[j * PI + d];
        }
        const float w = expf(a * p.scale - m_s[i]) / l_s[i];
        const float ds = w * (c - d_s[i]);
#pragma unroll
        for (int d = 0; d < DH; ++d) {
          dv[d] += w * gs[i * PI + d];
          dk[d] += ds * qs[i * PI + d];
        }
      }
    }
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      dk[d] = group_sum<G>(dk[d]) * p.scale;
      dv[d] = group_sum<G>(dv[d]);
    }
    if (tk >= 0) {
      for (int d = sub; d < DH; d += G) {
        float k = 0.f, v = 0.f;
#pragma unroll
        for (int e = 0; e < DH; ++e) { k = e == d ? dk[e] : k; v = e == d ? dv[e] : v; }
        dKb[(int64_t)tk * p.o_ts + d] = k;
        dVb[(int64_t)tk * p.o_ts + d] = v;
      }
    } else if (tk == -1 && p.dbias_kv) {
      for (int d = sub; d < DH; d += G) {
        float k = 0.f, v = 0.f;
#pragma unroll
        for (int e = 0; e < DH; ++e) { k = e == d ? dk[e] : k; v = e == d ? dv[e] : v; }
        atomicAdd(&padg[d], k);
        atomicAdd(&padg[DH + d], v);
      }
    }
  }
  if (any_pad && p.dbias_kv) {  // uniform
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * DH; i += blockDim.x)
      atomicAdd(p.dbias_kv + (i < DH ? h * DH + i : p.D + h * DH + i - DH), padg[i]);
  }
}

// bf16 windows of at most 64 tokens on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation; A = softmax weights and dS rounded to bf16 as operands).
// Four waves; lane l: c = l % 16, g = l / 16.
//  phase 1, wave w owns queries 16w..16w+15 (query 16w + c per lane):
//    S^T = K Q^T and dP^T = V dO^T (key tile t: keys 16t + 4g + r, r < 4),
//    softmax over the 64 keys (the 4 lane groups of a column share a query),
//    D = sum A dP, dS = A (dP - D); dQ^T = K^T dS^T with dS^T packed from the
//    registers (contraction order: keys 16t0 + 4g + e, then 16(t0+1) + 4g + e);
//    A^T and dS^T go to LDS as [key][query].
//  phase 2, wave w owns keys 16w..16w+15: dV^T = dO^T A and dK^T = Q^T dS, the
//    contraction over the 64 queries read from the transposed LDS copies.
// LDS (54 KB at d_h = 72, so three workgroups share a CU): the transposed
// copies hold the DH real rows only, back to back; a 16-row dim tile that
// runs past DH reads the next copy's (or the K/V region's) first rows, whose
// products land in output rows >= DH, which are never stored. A^T and dS^T
// reuse the row-major K, V region once every wave's S^T, dP^T products have
// read it.
template <int DH>
__global__ void __launch_bounds__(BW_NT) window_bwd_mfma_kernel(WindowBwdParams p) {
  static_assert(DH % 8 == 0, "head width a multiple of 8");
  constexpr int KEYS = 64;
  constexpr int NKC = (DH + 31) / 32;  // 32-wide chunks of the head dim (dims past DH read as zero)
  // row pitch (elements) of the row-major K, V copies: an odd number of
  // 16-byte chunks, so the 16 rows of a fragment read start in distinct banks
  constexpr int RP = 8 * (DH / 8 + ((DH / 8) % 2 == 0 ? 1 : 2));
  constexpr int NDT = (DH + 15) / 16;  // 16-row tiles of the transposed copies / outputs
  constexpr int TP = KEYS + 8;         // row pitch of the transposed copies
  constexpr int T_SZ = DH * TP;        // one transposed copy (elements)
  constexpr int KV_SZ = KEYS * RP;     // one row-major copy
  static_assert(KEYS * TP <= KV_SZ, "A^T / dS^T fit in the K / V copies they replace");
  static_assert((NDT * 16 - DH) * TP <= 2 * KV_SZ, "overrun rows of the last transposed copy stay in LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * T_SZ + 2 * KV_SZ];
  __shared__ int tok_s[KEYS], lab_s[KEYS];
  uint16_t* const kT = lds;
  uint16_t* const qT = lds + T_SZ;
  uint16_t* const gT = lds + 2 * T_SZ;
  uint16_t* const kr = lds + 3 * T_SZ;
  uint16_t* const vr = kr + KV_SZ;
  uint16_t* const pT = kr;  // written after every wave's S^T, dP^T products
  uint16_t* const dsT = vr;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int nWh = p.Hp / p.wh, nWw = p.Wp / p.ww;
  const int Tw = blockIdx.x / (nWh * nWw), Iw = (blockIdx.x / nWw) % nWh, Jw = blockIdx.x % nWw;
  const int wsz = p.wt * p.wh * p.ww;
  const int64_t N = (int64_t)p.F * p.H * p.W;
  const bool masked = (p.st | p.sh | p.sw) != 0;

  bool my_pad = false;
  for (int s = tid; s < KEYS; s += BW_NT) {
    int tok = -2, lab = 0;
    if (s < wsz) {
      const int a = s / (p.wh * p.ww), cc = (s / p.ww) % p.wh, e = s % p.ww;
      const int rt = Tw * p.wt + a, ri = Iw * p.wh + cc, rj = Jw * p.ww + e;
      int ot = rt + p.st; ot -= ot >= p.Fp ? p.Fp : 0;
      int oi = ri + p.sh; oi -= oi >= p.Hp ? p.Hp : 0;
      int oj = rj + p.sw; oj -= oj >= p.Wp ? p.Wp : 0;
      tok = (ot < p.F && oi < p.H && oj < p.W) ? (ot * p.H + oi) * p.W + oj : -1;
      lab = region_of(rt, p.Fp, p.wt, p.st) * 9 + region_of(ri, p.Hp, p.wh, p.sh) * 3 +
            region_of(rj, p.Wp, p.ww, p.sw);
    }
    tok_s[s] = tok;
    lab_s[s] = lab;
    my_pad |= tok == -1;
  }
  // pad slots' key / value gradients are summed per channel in LDS, then
  // added to d_bias_kv once per workgroup (not once per pad key)
  const bool any_pad = __syncthreads_or(my_pad) != 0;

  const uint16_t* base = reinterpret_cast<const uint16_t*>(p.QKV);
  const int64_t hs = N * DH, gsz = (int64_t)p.heads * hs;
  const uint16_t* Qb = base + (int64_t)b * 3 * gsz + h * hs;
  const uint16_t* Kb = Qb + gsz;
  const uint16_t* Vb = Qb + 2 * gsz;
  const uint16_t* bias = reinterpret_cast<const uint16_t*>(p.bias_qkv);
  const uint16_t* dOb = reinterpret_cast<const uint16_t*>(p.dO) + (int64_t)b * N * p.D + h * DH;

  // staging: 16-byte chunks (8 dims) of every slot; row-major K, V and
  // transposed K, Q, dO (DH rows each).
  // One thread per (8-dim chunk, quad of slots), quads fastest: the four
  // slots' chunks are transposed in registers, so each transposed row gets
  // one 8-byte write (and a wave's writes fall in distinct banks)
  constexpr int CH = DH / 8, QUADS = KEYS / 4;  // chunks per row, slot quads
  for (int idx = tid; idx < CH * QUADS; idx += BW_NT) {
    const int ch = idx / QUADS, kq = idx - ch * QUADS;
    uint4 k4[4], v4[4], q4[4], g4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = tok_s[kq * 4 + j];
      k4[j] = v4[j] = q4[j] = g4[j] = uint4{0, 0, 0, 0};
      if (tok >= 0) {
        k4[j] = *reinterpret_cast<const uint4*>(Kb + (int64_t)tok * DH + ch * 8);
        v4[j] = *reinterpret_cast<const uint4*>(Vb + (int64_t)tok * DH + ch * 8);
        q4[j] = *reinterpret_cast<const uint4*>(Qb + (int64_t)tok * DH + ch * 8);
        g4[j] = *reinterpret_cast<const uint4*>(dOb + (int64_t)tok * p.D + ch * 8);
      } else if (tok == -1 && bias) {
        k4[j] = *reinterpret_cast<const uint4*>(bias + p.D + h * DH + ch * 8);
        v4[j] = *reinterpret_cast<const uint4*>(bias + 2 * p.D + h * DH + ch * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4*>(&kr[(kq * 4 + j) * RP + ch * 8]) = k4[j];
      *reinterpret_cast<uint4*>(&vr[(kq * 4 + j) * RP + ch * 8]) = v4[j];
    }
    put_quad_t(kT, TP, ch, kq * 4, k4);
    put_quad_t(qT, TP, ch, kq * 4, q4);
    put_quad_t(gT, TP, ch, kq * 4, g4);
  }
  __syncthreads();

  const int64_t dQb = (int64_t)b * p.o_bs + h * p.o_hs;  // element offsets in dQKV
  const int64_t dKb = dQb + p.o_gs;
  const int64_t dVb = dQb + 2 * p.o_gs;

  // ---- phase 1: queries of wave w
  {
    const int qs = w * 16 + c;
    const int qtok = tok_s[qs], qlab = lab_s[qs];
    uint4 qf[NKC], gf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      // B operands: column = this lane's query, k = dims kc*32 + 8g .. +8
      // (read back from the transposed copies would cost 8 LDS reads; the
      // row-major source is the global row, zero past DH)
      const int d = kc * 32 + 8 * g;
      qf[kc] = (qtok >= 0 && d < DH) ? *reinterpret_cast<const uint4*>(Qb + (int64_t)qtok * DH + d) : uint4{0, 0, 0, 0};
      gf[kc] = (qtok >= 0 && d < DH) ? *reinterpret_cast<const uint4*>(dOb + (int64_t)qtok * p.D + d)
                                     : uint4{0, 0, 0, 0};
    }
    floatx4 sc[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = zero4();
      dp[t] = zero4();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bool in = kc * 32 + 8 * g < DH;
        const uint4 ka = in ? *reinterpret_cast<const uint4*>(&kr[(t * 16 + c) * RP + kc * 32 + 8 * g])
                            : uint4{0, 0, 0, 0};
        const uint4 va = in ? *reinterpret_cast<const uint4*>(&vr[(t * 16 + c) * RP + kc * 32 + 8 * g])
                            : uint4{0, 0, 0, 0};
        sc[t] = mfma_bf16(ka, qf[kc], sc[t]);
        dp[t] = mfma_bf16(va, gf[kc], dp[t]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ks = t * 16 + 4 * g + r;
        const bool ok = tok_s[ks] != -2 && (!masked || lab_s[ks] == qlab);
        sc[t][r] = ok ? sc[t][r] * p.scale : -INFINITY;
        mx = fmaxf(mx, sc[t][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx == -INFINITY) mx = 0.f;  // slot past the window: no allowed key
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] = expf(sc[t][r] - mx);
        l += sc[t][r];
      }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float rl = l > 0.f ? 1.f / l : 0.f;
    float dd = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] *= rl;  // softmax weight A
        dd += sc[t][r] * dp[t][r];
      }
    dd += __shfl_xor(dd, 16, 64);
    dd += __shfl_xor(dd, 32, 64);
    __syncthreads();  // every wave is done with kr / vr, which pT / dsT overwrite
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ks = t * 16 + 4 * g + r;
        dp[t][r] = sc[t][r] * (dp[t][r] - dd);  // dS
        pT[ks * TP + qs] = (uint16_t)(pack_bf2(sc[t][r], 0.f) & 0xffffu);
        dsT[ks * TP + qs] = (uint16_t)(pack_bf2(dp[t][r], 0.f) & 0xffffu);
      }
    // dQ^T = K^T dS^T over the 64 keys (two MFMAs of 32 per dim tile)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      floatx4 acc = zero4();
#pragma unroll
      for (int t0 = 0; t0 < 4; t0 += 2) {
        const uint4 bf = uint4{pack_bf2(dp[t0][0], dp[t0][1]), pack_bf2(dp[t0][2], dp[t0][3]),
                               pack_bf2(dp[t0 + 1][0], dp[t0 + 1][1]), pack_bf2(dp[t0 + 1][2], dp[t0 + 1][3])};
        const int row = (dt * 16 + c) * TP, kb = t0 * 16 + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(&kT[row + kb]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&kT[row + kb + 16]);
        acc = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, bf, acc);
      }
      const int d = dt * 16 + 4 * g;
      if (qtok >= 0 && d < DH)
        bwd_store4(p, dQb + (int64_t)qtok * p.o_ts + d,
                   float4{acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale});
    }
  }
  __syncthreads();
  // pad keys' gradients (d b_k at 0 .. DH-1, d b_v after) are summed in the
  // transposed-K copy, which phase 2 no longer reads
  float* const padg = reinterpret_cast<float*>(kT);
  if (any_pad) {  // uniform
    for (int i = tid; i < 2 * DH; i += BW_NT) padg[i] = 0.f;
    __syncthreads();
  }

  // ---- phase 2: keys of wave w
  {
    const int ks = w * 16 + c;
    const int ktok = tok_s[ks];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      floatx4 av = zero4(), ak = zero4();
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int qo = kq * 32 + 8 * g;
        const uint4 pa = *reinterpret_cast<const uint4*>(&pT[ks * TP + qo]);
        const uint4 da = *reinterpret_cast<const uint4*>(&dsT[ks * TP + qo]);
        const uint4 ga = *reinterpret_cast<const uint4*>(&gT[(dt * 16 + c) * TP + qo]);
        const uint4 qa = *reinterpret_cast<const uint4*>(&qT[(dt * 16 + c) * TP + qo]);
        av = mfma_bf16(ga, pa, av);
        ak = mfma_bf16(qa, da, ak);
      }
      const int d = dt * 16 + 4 * g;
      if (d >= DH) continue;
      const float4 kv = float4{ak[0] * p.scale, ak[1] * p.scale, ak[2] * p.scale, ak[3] * p.scale};
      const float4 vv = float4{av[0], av[1], av[2], av[3]};
      if (ktok >= 0) {
        bwd_store4(p, dKb + (int64_t)ktok * p.o_ts + d, kv);
        bwd_store4(p, dVb + (int64_t)ktok * p.o_ts + d, vv);
      } else if (ktok == -1 && p.dbias_kv) {
        float* bk = &padg[d];
        float* bv = &padg[DH + d];
        atomicAdd(bk + 0, kv.x); atomicAdd(bk + 1, kv.y); atomicAdd(bk + 2, kv.z); atomicAdd(bk + 3, kv.w);
        atomicAdd(bv + 0, vv.x); atomicAdd(bv + 1, vv.y); atomicAdd(bv + 2, vv.z); atomicAdd(bv + 3, vv.w);
      }
    }
  }
  if (any_pad && p.dbias_kv) {  // uniform
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * DH; i += blockDim.x)
      atomicAdd(p.dbias_kv + (i < DH ? h * DH + i : p.D + h * DH + i - DH), padg[i]);
  }
}

// bf16 windows of 65..128 tokens (the 2 x 8 x 8 video windows) on the matrix
// cores. Eight waves, 16 queries (phase 1) and 16 keys (phase 2) a wave; Q,
// K, V, dO staged row-major (A / B operands of S and dP) and K, Q, dO
// transposed (A operands of dQ^T, dK^T, dV^T).
//  phase 1 (query-major), as the 64-token kernel over 8 key tiles: S^T, dP^T,
//    the exact softmax over the window's keys, D = sum A dP, dS = A (dP - D),
//    dQ^T = K^T dS^T; the query's max, 1/rowsum and D go to LDS.
//  phase 2 (key-major): S = Q K^T and dP = dO V^T recomputed for the wave's 16
//    keys (lane: key 16w + c, queries 16qt + 4g + r), A = exp(S - max) / sum
//    and dS = A (dP - D) from the stored statistics; dV^T = dO^T A and
//    dK^T = Q^T dS with A, dS packed from the registers (contraction order:
//    queries 16qt0 + 4g + e, then 16(qt0+1) + 4g + e). Nothing of size
//    keys x queries is written to LDS.
// LDS 148 KB at d_h = 72 (one workgroup per CU). A 16-row dim tile of a
// transposed copy that runs past DH reads the next region's first rows, whose
// products land in output rows >= DH, never stored.
template <int DH>
__global__ void __launch_bounds__(512) window_bwd_mfma128_kernel(WindowBwdParams p) {
  static_assert(DH % 8 == 0, "head width a multiple of 8");
  constexpr int KEYS = 128, NW = 8, NT = KEYS / 16;
  constexpr int NKC = (DH + 31) / 32;
  constexpr int RP = 8 * (DH / 8 + ((DH / 8) % 2 == 0 ? 1 : 2));  // odd count of 16-byte chunks
  constexpr int NDT = (DH + 15) / 16;
  constexpr int TP = KEYS + 8;
  constexpr int T_SZ = DH * TP, R_SZ = KEYS * RP;
  static_assert((NDT * 16 - DH) * TP <= R_SZ, "overrun rows of the last transposed copy stay in LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * T_SZ + 4 * R_SZ];
  __shared__ int tok_s[KEYS], lab_s[KEYS];
  __shared__ float st_s[KEYS * 3];  // per query: max, 1 / rowsum, D
  uint16_t* const kT = lds;
  uint16_t* const qT = lds + T_SZ;
  uint16_t* const gT = lds + 2 * T_SZ;
  uint16_t* const kr = lds + 3 * T_SZ;
  uint16_t* const vr = kr + R_SZ;
  uint16_t* const qr = vr + R_SZ;
  uint16_t* const gr = qr + R_SZ;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int nWh = p.Hp / p.wh, nWw = p.Wp / p.ww;
  const int Tw = blockIdx.x / (nWh * nWw), Iw = (blockIdx.x / nWw) % nWh, Jw = blockIdx.x % nWw;
  const int wsz = p.wt * p.wh * p.ww;
  const int64_t N = (int64_t)p.F * p.H * p.W;
  const bool masked = (p.st | p.sh | p.sw) != 0;

  __shared__ float padg[2 * DH];  // pad keys' gradients: d b_k (0 .. DH-1), d b_v
  for (int i = threadIdx.x; i < 2 * DH; i += blockDim.x) padg[i] = 0.f;
  bool my_pad = false;
  if (tid < KEYS) {
    const int s = tid;
    int tok = -2, lab = 0;
    if (s < wsz) {
      const int a = s / (p.wh * p.ww), cc = (s / p.ww) % p.wh, e = s % p.ww;
      const int rt = Tw * p.wt + a, ri = Iw * p.wh + cc, rj = Jw * p.ww + e;
      int ot = rt + p.st; ot -= ot >= p.Fp ? p.Fp : 0;
      int oi = ri + p.sh; oi -= oi >= p.Hp ? p.Hp : 0;
      int oj = rj + p.sw; oj -= oj >= p.Wp ? p.Wp : 0;
      tok = (ot < p.F && oi < p.H && oj < p.W) ? (ot * p.H + oi) * p.W + oj : -1;
      lab = region_of(rt, p.Fp, p.wt, p.st) * 9 + region_of(ri, p.Hp, p.wh, p.sh) * 3 +
            region_of(rj, p.Wp, p.ww, p.sw);
    }
    tok_s[s] = tok;
    lab_s[s] = lab;
    my_pad |= tok == -1;
  }
  // pad slots' key / value gradients are summed per channel in LDS, then
  // added to d_bias_kv once per workgroup (not once per pad key)
  const bool any_pad = __syncthreads_or(my_pad) != 0;

  const uint16_t* base = reinterpret_cast<const uint16_t*>(p.QKV);
  const int64_t hs = N * DH, gsz = (int64_t)p.heads * hs;
  const uint16_t* Qb = base + (int64_t)b * 3 * gsz + h * hs;
  const uint16_t* Kb = Qb + gsz;
  const uint16_t* Vb = Qb + 2 * gsz;
  const uint16_t* bias = reinterpret_cast<const uint16_t*>(p.bias_qkv);
  const uint16_t* dOb = reinterpret_cast<const uint16_t*>(p.dO) + (int64_t)b * N * p.D + h * DH;

  // staging: one thread per (8-dim chunk, quad of slots), quads fastest
  constexpr int CH = DH / 8, QUADS = KEYS / 4;
  static_assert(CH * QUADS <= NW * 64, "one staging item a thread");
  if (tid < CH * QUADS) {
    const int ch = tid / QUADS, kq = tid - ch * QUADS;
    uint4 k4[4], v4[4], q4[4], g4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = tok_s[kq * 4 + j];
      k4[j] = v4[j] = q4[j] = g4[j] = uint4{0, 0, 0, 0};
      if (tok >= 0) {
        k4[j] = *reinterpret_cast<const uint4*>(Kb + (int64_t)tok * DH + ch * 8);
        v4[j] = *reinterpret_cast<const uint4*>(Vb + (int64_t)tok * DH + ch * 8);
        q4[j] = *reinterpret_cast<const uint4*>(Qb + (int64_t)tok * DH + ch * 8);
        g4[j] = *reinterpret_cast<const uint4*>(dOb + (int64_t)tok * p.D + ch * 8);
      } else if (tok == -1 && bias) {
        k4[j] = *reinterpret_cast<const uint4*>(bias + p.D + h * DH + ch * 8);
        v4[j] = *reinterpret_cast<const uint4*>(bias + 2 * p.D + h * DH + ch * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (kq * 4 + j) * RP + ch * 8;
      *reinterpret_cast<uint4*>(&kr[r]) = k4[j];
      *reinterpret_cast<uint4*>(&vr[r]) = v4[j];
      *reinterpret_cast<uint4*>(&qr[r]) = q4[j];
      *reinterpret_cast<uint4*>(&gr[r]) = g4[j];
    }
    put_quad_t(kT, TP, ch, kq * 4, k4);
    put_quad_t(qT, TP, ch, kq * 4, q4);
    put_quad_t(gT, TP, ch, kq * 4, g4);
  }
  __syncthreads();

  const int64_t dQb = (int64_t)b * p.o_bs + h * p.o_hs;  // element offsets in dQKV
  const int64_t dKb = dQb + p.o_gs;
  const int64_t dVb = dQb + 2 * p.o_gs;

  // ---- phase 1: queries of wave w
  {
    const int qs = w * 16 + c;
    const int qtok = tok_s[qs], qlab = lab_s[qs];
    uint4 qf[NKC], gf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * g;
      qf[kc] = d < DH ? *reinterpret_cast<const uint4*>(&qr[qs * RP + d]) : uint4{0, 0, 0, 0};
      gf[kc] = d < DH ? *reinterpret_cast<const uint4*>(&gr[qs * RP + d]) : uint4{0, 0, 0, 0};
    }
    floatx4 sc[NT], dp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sc[t] = zero4();
      dp[t] = zero4();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bool in = kc * 32 + 8 * g < DH;
        const int r = (t * 16 + c) * RP + kc * 32 + 8 * g;
        const uint4 ka = in ? *reinterpret_cast<const uint4*>(&kr[r]) : uint4{0, 0, 0, 0};
        const uint4 va = in ? *reinterpret_cast<const uint4*>(&vr[r]) : uint4{0, 0, 0, 0};
        sc[t] = mfma_bf16(ka, qf[kc], sc[t]);
        dp[t] = mfma_bf16(va, gf[kc], dp[t]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ks = t * 16 + 4 * g + r;
        const bool ok = tok_s[ks] != -2 && (!masked || lab_s[ks] == qlab);
        sc[t][r] = ok ? sc[t][r] * p.scale : -INFINITY;
        mx = fmaxf(mx, sc[t][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx == -INFINITY) mx = 0.f;  // slot past the window: no allowed key
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] = expf(sc[t][r] - mx);
        l += sc[t][r];
      }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float rl = l > 0.f ? 1.f / l : 0.f;
    float dd = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] *= rl;
        dd += sc[t][r] * dp[t][r];
      }
    dd += __shfl_xor(dd, 16, 64);
    dd += __shfl_xor(dd, 32, 64);
    if (g == 0) {
      st_s[qs * 3] = mx;
      st_s[qs * 3 + 1] = rl;
      st_s[qs * 3 + 2] = dd;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) dp[t][r] = sc[t][r] * (dp[t][r] - dd);  // dS
    // dQ^T = K^T dS^T over the keys (two key tiles per MFMA)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      floatx4 acc = zero4();
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += 2) {
        const uint4 bf = uint4{pack_bf2(dp[t0][0], dp[t0][1]), pack_bf2(dp[t0][2], dp[t0][3]),
                               pack_bf2(dp[t0 + 1][0], dp[t0 + 1][1]), pack_bf2(dp[t0 + 1][2], dp[t0 + 1][3])};
        const int row = (dt * 16 + c) * TP, kb = t0 * 16 + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(&kT[row + kb]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&kT[row + kb + 16]);
        acc = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, bf, acc);
      }
      const int d = dt * 16 + 4 * g;
      if (qtok >= 0 && d < DH)
        bwd_store4(p, dQb + (int64_t)qtok * p.o_ts + d,
                   float4{acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale});
    }
  }
  __syncthreads();  // statistics of every query in LDS

  // ---- phase 2: keys of wave w
  {
    const int ks = w * 16 + c;
    const int ktok = tok_s[ks], klab = lab_s[ks];
    const bool kvalid = ktok != -2;
    uint4 kf[NKC], vf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * g;
      kf[kc] = d < DH ? *reinterpret_cast<const uint4*>(&kr[ks * RP + d]) : uint4{0, 0, 0, 0};
      vf[kc] = d < DH ? *reinterpret_cast<const uint4*>(&vr[ks * RP + d]) : uint4{0, 0, 0, 0};
    }
    floatx4 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) { dk[dt] = zero4(); dv[dt] = zero4(); }
#pragma unroll
    for (int qt0 = 0; qt0 < NT; qt0 += 2) {
      floatx4 pa[2], da[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int qt = qt0 + v;
        floatx4 sc = zero4(), dp = zero4();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const bool in = kc * 32 + 8 * g < DH;
          const int r = (qt * 16 + c) * RP + kc * 32 + 8 * g;
          const uint4 qa = in ? *reinterpret_cast<const uint4*>(&qr[r]) : uint4{0, 0, 0, 0};
          const uint4 ga = in ? *reinterpret_cast<const uint4*>(&gr[r]) : uint4{0, 0, 0, 0};
          sc = mfma_bf16(qa, kf[kc], sc);
          dp = mfma_bf16(ga, vf[kc], dp);
        }
        // S[query 16qt + 4g + r][key ks]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qrow = qt * 16 + 4 * g + r;
          const bool ok = kvalid && tok_s[qrow] != -2 && (!masked || lab_s[qrow] == klab);
          const float m = st_s[qrow * 3], rl = st_s[qrow * 3 + 1], dd = st_s[qrow * 3 + 2];
          const float a = ok ? expf(sc[r] * p.scale - m) * rl : 0.f;
          pa[v][r] = a;
          da[v][r] = a * (dp[r] - dd);
        }
      }
      const uint4 pf = uint4{pack_bf2(pa[0][0], pa[0][1]), pack_bf2(pa[0][2], pa[0][3]),
                             pack_bf2(pa[1][0], pa[1][1]), pack_bf2(pa[1][2], pa[1][3])};
      const uint4 df = uint4{pack_bf2(da[0][0], da[0][1]), pack_bf2(da[0][2], da[0][3]),
                             pack_bf2(da[1][0], da[1][1]), pack_bf2(da[1][2], da[1][3])};
      const int kb = qt0 * 16 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int row = (dt * 16 + c) * TP;
        const uint2 glo = *reinterpret_cast<const uint2*>(&gT[row + kb]);
        const uint2 ghi = *reinterpret_cast<const uint2*>(&gT[row + kb + 16]);
        const uint2 qlo = *reinterpret_cast<const uint2*>(&qT[row + kb]);
        const uint2 qhi = *reinterpret_cast<const uint2*>(&qT[row + kb + 16]);
        dv[dt] = mfma_bf16(uint4{glo.x, glo.y, ghi.x, ghi.y}, pf, dv[dt]);
        dk[dt] = mfma_bf16(uint4{qlo.x, qlo.y, qhi.x, qhi.y}, df, dk[dt]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = dt * 16 + 4 * g;
      if (d >= DH) continue;
      const float4 kv = float4{dk[dt][0] * p.scale, dk[dt][1] * p.scale, dk[dt][2] * p.scale, dk[dt][3] * p.scale};
      const float4 vv = float4{dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]};
      if (ktok >= 0) {
        bwd_store4(p, dKb + (int64_t)ktok * p.o_ts + d, kv);
        bwd_store4(p, dVb + (int64_t)ktok * p.o_ts + d, vv);
      } else if (ktok == -1 && p.dbias_kv) {
        float* bk = &padg[d];
        float* bv = &padg[DH + d];
        atomicAdd(bk + 0, kv.x); atomicAdd(bk + 1, kv.y); atomicAdd(bk + 2, kv.z); atomicAdd(bk + 3, kv.w);
        atomicAdd(bv + 0, vv.x); atomicAdd(bv + 1, vv.y); atomicAdd(bv + 2, vv.z); atomicAdd(bv + 3, vv.w);
      }
    }
  }
  if (any_pad && p.dbias_kv) {  // uniform
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * DH; i += blockDim.x)
      atomicAdd(p.dbias_kv + (i < DH ? h * DH + i : p.D + h * DH + i - DH), padg[i]);
  }
}

template <typename T, int DH>
static hipError_t pick_window_bwd(const WindowBwdDesc& d, hipStream_t s) {
  WindowBwdParams p;
  p.QKV = d.QKV; p.bias_qkv = d.bias_qkv; p.dO = d.dO; p.dQKV = d.dQKV; p.dbias_kv = d.dbias_kv;
  p.out_bf16 = d.out_bf16;
  p.F = d.F; p.H = d.H; p.W = d.W; p.D = d.D; p.heads = d.heads;
  const int64_t N = (int64_t)d.F * d.H * d.W;
  if (d.tokens_out) {  // [B][N][3D]: the Q/K/V projection's output gradient
    p.o_bs = N * 3 * d.D; p.o_gs = d.D; p.o_hs = DH; p.o_ts = 3 * (int64_t)d.D;
  } else {             // [B][3][heads][N][dh]
    p.o_hs = N * DH; p.o_gs = d.heads * p.o_hs; p.o_bs = 3 * p.o_gs; p.o_ts = DH;
  }
  p.wt = d.wt; p.wh = d.wh; p.ww = d.ww;
  p.st = d.st; p.sh = d.sh; p.sw = d.sw;
  p.Fp = d.Fp; p.Hp = d.Hp; p.Wp = d.Wp;
  p.scale = d.scale;
  const int nwin = (d.Fp / d.wt) * (d.Hp / d.wh) * (d.Wp / d.ww);
  const dim3 grid(nwin, d.heads, d.B);
  const int wsz = d.wt * d.wh * d.ww;
  if (d.out_bf16 && (sizeof(T) != 2 || wsz > 128)) return hipErrorInvalidValue;  // fp32 out only there
  if (sizeof(T) == 2 && wsz <= 64) hipLaunchKernelGGL((window_bwd_mfma_kernel<DH>), grid, dim3(BW_NT), 0, s, p);
  else if (sizeof(T) == 2 && wsz <= 128)
    hipLaunchKernelGGL((window_bwd_mfma128_kernel<DH>), grid, dim3(512), 0, s, p);
  else if (wsz <= 64) hipLaunchKernelGGL((window_bwd_kernel<T, DH, 64>), grid, dim3(BW_NT), 0, s, p);
  else if (wsz <= 128) hipLaunchKernelGGL((window_bwd_kernel<T, DH, 128>), grid, dim3(BW_NT), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_window_bwd(const WindowBwdDesc& d, int f32, hipStream_t s) {
  if (d.B == 0) return hipSuccess;
  if (d.dh == 72) return f32 ? pick_window_bwd<float, 72>(d, s) : pick_window_bwd<uint16_t, 72>(d, s);
  if (d.dh == 64) return f32 ? pick_window_bwd<float, 64>(d, s) : pick_window_bwd<uint16_t, 64>(d, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Dense attention backward (proxy self-attention, cross-attention)
// ----------------------------------------------------------------------------
struct DenseBwdParams {
  const void *q, *k, *v, *dO;
  int64_t q_bs, kv_bs;   // batch strides (elements) of q and of k / v
  void* dq;              // head-major [heads][Nq][dh] or token-major [Nq][D] a batch item
  float *dk, *dv;
  int64_t dq_bs, dkv_bs;
  int dq_tok, dq_bf16;   // dQ token-major; dQ in bf16 (matrix-core kernels only), else fp32
  float* stats;          // [B][heads][Nq][3]: row max, row sum, D = rowsum(A * dA)
  float* part;           // [chunks][B][heads][Nk][2][dh] when the queries are split
  int B, heads, Nq, Nk, D, qchunk, chunks;
  int qtiles;            // 64-query tiles per workgroup of the matrix-core query-major kernel
  float scale;
};

// element offset of dQ[b][h][query qi][0]
__device__ __forceinline__ int64_t dq_offset(const DenseBwdParams& p, int b, int h, int64_t qi, int dh) {
  return b * p.dq_bs + (p.dq_tok ? qi * p.D + (int64_t)h * dh : ((int64_t)h * p.Nq + qi) * dh);
}
// four consecutive dQ elements (e % 4 == 0), fp32 or rounded to bf16
__device__ __forceinline__ void dq_store4(const DenseBwdParams& p, int64_t e, float4 v) {
  if (p.dq_bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.dq) + e) = uint2{pack_bf2(v.x, v.y), pack_bf2(v.z, v.w)};
  else
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.dq) + e) = v;
}

constexpr int DB_Q = 64;   // queries per workgroup (query-major kernel)
constexpr int DB_K = 64;   // keys per LDS chunk / per workgroup (key-major kernel)

// 4 lanes per query; lane sub takes keys sub, sub+4, ... of each 64-key chunk.
template <typename T, int DH>
__global__ void __launch_bounds__(BW_NT) dense_bwd_q_kernel(DenseBwdParams p) {
  constexpr int PI = DH + 1, G = 4, PER = DB_K / G;
  __shared__ float ks[DB_K * PI], vs[DB_K * PI];
  const int tid = threadIdx.x, i = blockIdx.x * DB_Q + tid / G, sub = tid % G;
  const int h = blockIdx.y, b = blockIdx.z;
  const bool live = i < p.Nq;
  const T* Q = reinterpret_cast<const T*>(p.q) + b * p.q_bs + ((int64_t)h * p.Nq + (live ? i : 0)) * DH;
  const T* K = reinterpret_cast<const T*>(p.k) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const T* V = reinterpret_cast<const T*>(p.v) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const T* G0 = reinterpret_cast<const T*>(p.dO) + ((int64_t)b * p.Nq + (live ? i : 0)) * p.D + h * DH;
  float q[DH], g[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) { q[d] = live ? ld1(Q + d) : 0.f; g[d] = live ? ld1(G0 + d) : 0.f; }

  auto stage = [&](int c0, bool with_v) {
    __syncthreads();
    for (int idx = tid; idx < DB_K * DH; idx += BW_NT) {
      const int j = idx / DH, d = idx - j * DH, key = c0 + j;
      ks[j * PI + d] = key < p.Nk ? ld1(K + (int64_t)key * DH + d) : 0.f;
      if (with_v) vs[j * PI + d] = key < p.Nk ? ld1(V + (int64_t)key * DH + d) : 0.f;
    }
    __syncthreads();
  };

  // pass 1: row maximum and sum (online over the chunks)
  float mx = -INFINITY, l = 0.f;
  for (int c0 = 0; c0 < p.Nk; c0 += DB_K) {
    stage(c0, false);
#pragma unroll 4
    for (int u = 0; u < PER; ++u) {
      const int j = sub + u * G;
      if (c0 + j >= p.Nk) continue;
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) a += q[d] * ks[j * PI + d];
      const float sc = a * p.scale;
      if (sc > mx) { l = l * expf(mx - sc) + 1.f; mx = sc; }
      else l += expf(sc - mx);
    }
  }
  {
    const float m2 = group_max<G>(mx);
    l = group_sum<G>(mx == -INFINITY ? 0.f : l * expf(mx - m2));
    mx = m2;
  }
  const float rl = 1.f / l;
  // pass 2: D = sum_j A_ij dA_ij, X = sum_j A_ij dA_ij k_j, Y = sum_j A_ij k_j;
  // dQ = scale * (X - D * Y)
  float X[DH], Y[DH], Dl = 0.f;
#pragma unroll
  for (int d = 0; d < DH; ++d) { X[d] = 0.f; Y[d] = 0.f; }
  for (int c0 = 0; c0 < p.Nk; c0 += DB_K) {
    stage(c0, true);
    for (int u = 0; u < PER; ++u) {
      const int j = sub + u * G;
      if (c0 + j >= p.Nk) continue;
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        a += q[d] * ks[j * PI + d];
        c += g[d] * vs[j * PI + d];
      }
      const float w = expf(a * p.scale - mx) * rl;
      Dl += w * c;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        X[d] += w * c * ks[j * PI + d];
        Y[d] += w * ks[j * PI + d];
      }
    }
  }
  Dl = group_sum<G>(Dl);
#pragma unroll
  for (int d = 0; d < DH; ++d) { X[d] = group_sum<G>(X[d]); Y[d] = group_sum<G>(Y[d]); }
  if (!live) return;
  float* dq = reinterpret_cast<float*>(p.dq) + dq_offset(p, b, h, i, DH);  // fp32 inputs: fp32 dQ
  for (int d = sub; d < DH; d += G) {
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int e = 0; e < DH; ++e) { x = e == d ? X[e] : x; y = e == d ? Y[e] : y; }
    dq[d] = (x - Dl * y) * p.scale;
  }
  if (sub == 0) {
    float* st = p.stats + (((int64_t)b * p.heads + h) * p.Nq + i) * 3;
    st[0] = mx; st[1] = l; st[2] = Dl;
  }
}

// 4 lanes per key; lane sub takes queries sub, sub+4, ... of each 64-query tile.
template <typename T, int DH>
__global__ void __launch_bounds__(BW_NT) dense_bwd_kv_kernel(DenseBwdParams p) {
  constexpr int PI = DH + 1, G = 4;
  __shared__ float qs[DB_Q * PI], gs[DB_Q * PI], st[DB_Q * 3];
  const int tid = threadIdx.x, j = blockIdx.x * DB_K + tid / G, sub = tid % G;
  const int chunk = blockIdx.y, bh = blockIdx.z, b = bh / p.heads, h = bh - b * p.heads;
  const bool live = j < p.Nk;
  const T* K = reinterpret_cast<const T*>(p.k) + b * p.kv_bs + ((int64_t)h * p.Nk + (live ? j : 0)) * DH;
  const T* V = reinterpret_cast<const T*>(p.v) + b * p.kv_bs + ((int64_t)h * p.Nk + (live ? j : 0)) * DH;
  const T* Q = reinterpret_cast<const T*>(p.q) + b * p.q_bs + (int64_t)h * p.Nq * DH;
  const T* G0 = reinterpret_cast<const T*>(p.dO) + (int64_t)b * p.Nq * p.D + h * DH;
  const float* S = p.stats + ((int64_t)b * p.heads + h) * p.Nq * 3;
  float k[DH], v[DH], dk[DH], dv[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    k[d] = live ? ld1(K + d) : 0.f; v[d] = live ? ld1(V + d) : 0.f;
    dk[d] = 0.f; dv[d] = 0.f;
  }
  const int q0 = chunk * p.qchunk, q1 = min(p.Nq, q0 + p.qchunk);
  for (int t0 = q0; t0 < q1; t0 += DB_Q) {
    __syncthreads();
    for (int idx = tid; idx < DB_Q * DH; idx += BW_NT) {
      const int r = idx / DH, d = idx - r * DH, qi = t0 + r;
      qs[r * PI + d] = qi < q1 ? ld1(Q + (int64_t)qi * DH + d) : 0.f;
      gs[r * PI + d] = qi < q1 ? ld1(G0 + (int64_t)qi * p.D + d) : 0.f;
    }
    for (int idx = tid; idx < DB_Q * 3; idx += BW_NT) st[idx] = t0 + idx / 3 < q1 ? S[(int64_t)t0 * 3 + idx] : 0.f;
    __syncthreads();
    for (int r = sub; r < DB_Q; r += G) {
      if (t0 + r >= q1) break;
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        a += qs[r * PI + d] * k[d];
        c += gs[r * PI + d] * v[d];
      }
      const float w = expf(a * p.scale - st[r * 3]) / st[r * 3 + 1];
      const float ds = w * (c - st[r * 3 + 2]);
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        dv[d] += w * gs[r * PI + d];
        dk[d] += ds * qs[r * PI + d];
      }
    }
  }
#pragma unroll
  for (int d = 0; d < DH; ++d) { dk[d] = group_sum<G>(dk[d]); dv[d] = group_sum<G>(dv[d]); }
  if (!live) return;
  for (int d = sub; d < DH; d += G) {
    float kk = 0.f, vv = 0.f;
#pragma unroll
    for (int e = 0; e < DH; ++e) { kk = e == d ? dk[e] : kk; vv = e == d ? dv[e] : vv; }
    if (p.chunks == 1) {
      p.dk[b * p.dkv_bs + ((int64_t)h * p.Nk + j) * DH + d] = kk * p.scale;
      p.dv[b * p.dkv_bs + ((int64_t)h * p.Nk + j) * DH + d] = vv;
    } else {
      float* pt = p.part + ((((int64_t)chunk * p.B + b) * p.heads + h) * p.Nk + j) * 2 * DH;
      pt[d] = kk;
      pt[DH + d] = vv;
    }
  }
}

template <int DH>
__global__ void __launch_bounds__(BW_NT) dense_bwd_reduce_kernel(DenseBwdParams p) {
  const int64_t per = (int64_t)p.B * p.heads * p.Nk * DH;
  const int64_t e = (int64_t)blockIdx.x * BW_NT + threadIdx.x;
  if (e >= per) return;
  const int d = (int)(e % DH);
  const int64_t row = e / DH;  // (b * heads + h) * Nk + j
  const int64_t b = row / ((int64_t)p.heads * p.Nk), rest = row - b * p.heads * p.Nk;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < p.chunks; ++c) {  // fixed order
    const float* pt = p.part + ((int64_t)c * p.B * p.heads * p.Nk + row) * 2 * DH;
    sk += pt[d];
    sv += pt[DH + d];
  }
  p.dk[b * p.dkv_bs + rest * DH + d] = sk * p.scale;
  p.dv[b * p.dkv_bs + rest * DH + d] = sv;
}

// ---- matrix-core forms (bf16): lane l of a wave: c = l % 16, g = l / 16.
constexpr int DM_MAXK = 256;  // keys resident in LDS in the query-major kernel
constexpr int DM_QT = 4;      // most 64-query tiles per workgroup of the query-major kernel

// Staging in two steps (loads into registers, then LDS writes), so a tile's
// loads can be in flight while the previous tile is computed: one thread per
// (8-dim chunk, quad of rows), quads fastest; the row-major copy gets four
// 16-byte writes and the transposed copy one 8-byte write per transposed row
// (put_quad_t).
template <int DH, int ROWS>
struct QuadChunks {
  static constexpr int CH = ((DH + 31) / 32) * 4, QUADS = ROWS / 4, ITEMS = CH * QUADS;
  static_assert(ITEMS <= BW_NT, "one item a thread");
  uint4 v[4];
};
template <int DH, int ROWS>
__device__ __forceinline__ void load_quads(const uint16_t* src, int64_t rs, int r0, int nrows, int tid,
                                           QuadChunks<DH, ROWS>& qc) {
  constexpr int QUADS = QuadChunks<DH, ROWS>::QUADS;
  const int ch = tid / QUADS, kq = tid - ch * QUADS;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = kq * 4 + j;
    qc.v[j] = (tid < QuadChunks<DH, ROWS>::ITEMS && ch * 8 < DH && r0 + r < nrows)
                  ? *reinterpret_cast<const uint4*>(src + (int64_t)(r0 + r) * rs + ch * 8)
                  : uint4{0, 0, 0, 0};
  }
}
template <int DH, int ROWS, int RP, int TP>
__device__ __forceinline__ void put_quads(const QuadChunks<DH, ROWS>& qc, uint16_t* rowm, uint16_t* tr, int tid) {
  constexpr int QUADS = QuadChunks<DH, ROWS>::QUADS, NDT = (DH + 15) / 16;
  if (tid >= QuadChunks<DH, ROWS>::ITEMS) return;
  const int ch = tid / QUADS, kq = tid - ch * QUADS;
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&rowm[(kq * 4 + j) * RP + ch * 8]) = qc.v[j];
  if (ch * 8 < NDT * 16) put_quad_t(tr, TP, ch, kq * 4, qc.v);
}

// Query-major: every key of the head (Nk <= 256) resident in LDS, 16 queries
// a wave. One pass: all Nk scores and dP values of the lane's query column
// stay in registers (16 tiles of 4), so the softmax is exact without a
// second look at the keys; then D = sum A dP, dS = A (dP - D) and
// dQ^T = K^T dS^T with dS^T packed from the registers. Statistics to the
// workspace.
constexpr int DQ_NT = 512;  // 8 waves: two waves a SIMD share the staged keys
template <int DH>
__global__ void __launch_bounds__(DQ_NT) dense_bwd_q_mfma_kernel(DenseBwdParams p) {
  constexpr int NKC = (DH + 31) / 32, RP = NKC * 32 + 8, NDT = (DH + 15) / 16;
  constexpr int TP = DM_MAXK + 8, MT = DM_MAXK / 16;
  __shared__ __attribute__((aligned(16))) uint16_t kr[DM_MAXK * RP], vr[DM_MAXK * RP], kT[NDT * 16 * TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(p.v) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_bs + (int64_t)h * p.Nq * DH;
  const uint16_t* G0 = reinterpret_cast<const uint16_t*>(p.dO) + (int64_t)b * p.Nq * p.D + h * DH;
  {
    // all keys: K row-major and transposed, V row-major; one item per
    // (8-dim chunk, quad of keys), quads fastest, all loads of an item
    // before its writes
    constexpr int CH = NKC * 4, QUADS = DM_MAXK / 4;
    for (int idx = tid; idx < CH * QUADS; idx += DQ_NT) {
      const int ch = idx / QUADS, kq = idx - ch * QUADS;
      uint4 k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = kq * 4 + j;
        const bool ok = ch * 8 < DH && r < p.Nk;
        k4[j] = ok ? *reinterpret_cast<const uint4*>(K + (int64_t)r * DH + ch * 8) : uint4{0, 0, 0, 0};
        v4[j] = ok ? *reinterpret_cast<const uint4*>(V + (int64_t)r * DH + ch * 8) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<uint4*>(&kr[(kq * 4 + j) * RP + ch * 8]) = k4[j];
        *reinterpret_cast<uint4*>(&vr[(kq * 4 + j) * RP + ch * 8]) = v4[j];
      }
      if (ch * 8 < NDT * 16) put_quad_t(kT, TP, ch, kq * 4, k4);
    }
  }
  __syncthreads();
  const int ntiles = (p.Nk + 15) / 16;
  // the staged keys serve p.qtiles tiles of 128 queries (16 a wave)
  for (int qt = 0; qt < p.qtiles; ++qt) {
    const int qi = (blockIdx.x * p.qtiles + qt) * (DQ_NT / 4) + w * 16 + c;
    const bool live = qi < p.Nq;
    uint4 qf[NKC], gf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * g;
      qf[kc] = (live && d < DH) ? *reinterpret_cast<const uint4*>(Q + (int64_t)qi * DH + d) : uint4{0, 0, 0, 0};
      gf[kc] = (live && d < DH) ? *reinterpret_cast<const uint4*>(G0 + (int64_t)qi * p.D + d) : uint4{0, 0, 0, 0};
    }
    floatx4 sc[MT], dp[MT];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      sc[t] = zero4();
      dp[t] = zero4();
      if (t < ntiles) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const uint4 ka = *reinterpret_cast<const uint4*>(&kr[(t * 16 + c) * RP + kc * 32 + 8 * g]);
          const uint4 va = *reinterpret_cast<const uint4*>(&vr[(t * 16 + c) * RP + kc * 32 + 8 * g]);
          sc[t] = mfma_bf16(ka, qf[kc], sc[t]);
          dp[t] = mfma_bf16(va, gf[kc], dp[t]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] = t * 16 + 4 * g + r < p.Nk ? sc[t][r] * p.scale : -INFINITY;
        mx = fmaxf(mx, sc[t][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] = __expf(sc[t][r] - mx);  // keys past Nk: exp(-inf) = 0
        l += sc[t][r];
      }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float rl = 1.f / l;
    float dd = 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[t][r] *= rl;
        dd += sc[t][r] * dp[t][r];
      }
    dd += __shfl_xor(dd, 16, 64);
    dd += __shfl_xor(dd, 32, 64);
    floatx4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero4();
#pragma unroll
    for (int t0 = 0; t0 < MT; t0 += 2) {
      if (t0 < ntiles) {
        floatx4 ds[2];
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) ds[v][r] = sc[t0 + v][r] * (dp[t0 + v][r] - dd);
        const uint4 bf = uint4{pack_bf2(ds[0][0], ds[0][1]), pack_bf2(ds[0][2], ds[0][3]),
                               pack_bf2(ds[1][0], ds[1][1]), pack_bf2(ds[1][2], ds[1][3])};
        const int kb = t0 * 16 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int row = (dt * 16 + c) * TP;
          const uint2 lo = *reinterpret_cast<const uint2*>(&kT[row + kb]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&kT[row + kb + 16]);
          acc[dt] = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, bf, acc[dt]);
        }
      }
    }
    if (live) {
      const int64_t dq = dq_offset(p, b, h, qi, DH);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = dt * 16 + 4 * g;
        if (d < DH)
          dq_store4(p, dq + d,
                    float4{acc[dt][0] * p.scale, acc[dt][1] * p.scale, acc[dt][2] * p.scale, acc[dt][3] * p.scale});
      }
      if (g == 0) {
        float* st = p.stats + (((int64_t)b * p.heads + h) * p.Nq + qi) * 3;
        st[0] = mx; st[1] = l; st[2] = dd;
      }
    }
  }
}

// Query-major for more than 256 keys: the keys stream through the same LDS
// layout in chunks of 256, twice. Pass 1 keeps, per query, the running
// maximum m, sum l = sum exp(s - m) and U = sum exp(s - m) dP over the chunks
// seen so far (both sums rescaled by exp(m_old - m_new) when the maximum
// grows), so that after the last chunk D = sum A dP = U / l. Pass 2 restages
// every chunk and forms the exact A = exp(s - m) / l and dS = A (dP - D),
// accumulating dQ^T = K^T dS^T across the chunks. A chunk is contracted in
// two halves of 128 keys (8 tiles of 16 scores and dP values a lane).
// Statistics to the workspace as in the resident kernel.
template <int DH>
__global__ void __launch_bounds__(DQ_NT) dense_bwd_q_mfma_stream_kernel(DenseBwdParams p) {
  constexpr int NKC = (DH + 31) / 32, RP = NKC * 32 + 8, NDT = (DH + 15) / 16;
  constexpr int TP = DM_MAXK + 8, HT = DM_MAXK / 32;  // 16-key tiles in half a chunk
  __shared__ __attribute__((aligned(16))) uint16_t kr[DM_MAXK * RP], vr[DM_MAXK * RP], kT[NDT * 16 * TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(p.v) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_bs + (int64_t)h * p.Nq * DH;
  const uint16_t* G0 = reinterpret_cast<const uint16_t*>(p.dO) + (int64_t)b * p.Nq * p.D + h * DH;
  const int qi = blockIdx.x * (DQ_NT / 4) + w * 16 + c;
  const bool live = qi < p.Nq;
  uint4 qf[NKC], gf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int d = kc * 32 + 8 * g;
    qf[kc] = (live && d < DH) ? *reinterpret_cast<const uint4*>(Q + (int64_t)qi * DH + d) : uint4{0, 0, 0, 0};
    gf[kc] = (live && d < DH) ? *reinterpret_cast<const uint4*>(G0 + (int64_t)qi * p.D + d) : uint4{0, 0, 0, 0};
  }
  // chunk k0..k0+255: K, V row-major and K transposed (keys past Nk zero)
  auto stage = [&](int k0) {
    constexpr int CH = NKC * 4, QUADS = DM_MAXK / 4;
    __syncthreads();  // the previous chunk's reads are done
    for (int idx = tid; idx < CH * QUADS; idx += DQ_NT) {
      const int ch = idx / QUADS, kq = idx - ch * QUADS;
      uint4 k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = k0 + kq * 4 + j;
        const bool ok = ch * 8 < DH && r < p.Nk;
        k4[j] = ok ? *reinterpret_cast<const uint4*>(K + (int64_t)r * DH + ch * 8) : uint4{0, 0, 0, 0};
        v4[j] = ok ? *reinterpret_cast<const uint4*>(V + (int64_t)r * DH + ch * 8) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<uint4*>(&kr[(kq * 4 + j) * RP + ch * 8]) = k4[j];
        *reinterpret_cast<uint4*>(&vr[(kq * 4 + j) * RP + ch * 8]) = v4[j];
      }
      if (ch * 8 < NDT * 16) put_quad_t(kT, TP, ch, kq * 4, k4);
    }
    __syncthreads();
  };
  // scores (scaled; -inf past Nk) and dP of half hf of the staged chunk
  auto half = [&](int k0, int hf, floatx4 (&sc)[HT], floatx4 (&dp)[HT]) {
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      const int tt = hf * HT + t;
      sc[t] = zero4();
      dp[t] = zero4();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&kr[(tt * 16 + c) * RP + kc * 32 + 8 * g]);
        const uint4 va = *reinterpret_cast<const uint4*>(&vr[(tt * 16 + c) * RP + kc * 32 + 8 * g]);
        sc[t] = mfma_bf16(ka, qf[kc], sc[t]);
        dp[t] = mfma_bf16(va, gf[kc], dp[t]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[t][r] = k0 + tt * 16 + 4 * g + r < p.Nk ? sc[t][r] * p.scale : -INFINITY;
    }
  };

  // ---- pass 1: running statistics (the lane's partial sums over its keys;
  // the maximum is shared by the four lane groups of the query)
  float m = -INFINITY, l = 0.f, u = 0.f;
  for (int k0 = 0; k0 < p.Nk; k0 += DM_MAXK) {
    stage(k0);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (k0 + hf * HT * 16 >= p.Nk) break;  // uniform
      floatx4 sc[HT], dp[HT];
      half(k0, hf, sc, dp);
      float cm = -INFINITY;
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) cm = fmaxf(cm, sc[t][r]);
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float mn = fmaxf(m, cm);           // finite: every half holds a key
      const float al = __expf(m - mn);         // 0 on the first half (m = -inf)
      l *= al;
      u *= al;
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __expf(sc[t][r] - mn);
          l += e;
          u += e * dp[t][r];
        }
      m = mn;
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  u += __shfl_xor(u, 16, 64);
  u += __shfl_xor(u, 32, 64);
  const float rl = 1.f / l, dd = u * rl;

  // ---- pass 2: dS and dQ
  floatx4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero4();
  for (int k0 = 0; k0 < p.Nk; k0 += DM_MAXK) {
    stage(k0);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (k0 + hf * HT * 16 >= p.Nk) break;
      floatx4 sc[HT], dp[HT];
      half(k0, hf, sc, dp);
#pragma unroll
      for (int t0 = 0; t0 < HT; t0 += 2) {
        floatx4 ds[2];
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) ds[v][r] = __expf(sc[t0 + v][r] - m) * rl * (dp[t0 + v][r] - dd);
        const uint4 bf = uint4{pack_bf2(ds[0][0], ds[0][1]), pack_bf2(ds[0][2], ds[0][3]),
                               pack_bf2(ds[1][0], ds[1][1]), pack_bf2(ds[1][2], ds[1][3])};
        const int kb = (hf * HT + t0) * 16 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int row = (dt * 16 + c) * TP;
          const uint2 lo = *reinterpret_cast<const uint2*>(&kT[row + kb]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&kT[row + kb + 16]);
          acc[dt] = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, bf, acc[dt]);
        }
      }
    }
  }
  if (live) {
    const int64_t dq = dq_offset(p, b, h, qi, DH);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = dt * 16 + 4 * g;
      if (d < DH)
        dq_store4(p, dq + d,
                  float4{acc[dt][0] * p.scale, acc[dt][1] * p.scale, acc[dt][2] * p.scale, acc[dt][3] * p.scale});
    }
    if (g == 0) {
      float* st = p.stats + (((int64_t)b * p.heads + h) * p.Nq + qi) * 3;
      st[0] = m; st[1] = l; st[2] = dd;
    }
  }
}

// Key-major: KS * 64 keys per workgroup (KS sub-tiles of 16 a wave) over one
// chunk of the queries, 64-query tiles staged row-major (Q, dO: A operands of
// S = Q K^T, dP = dO V^T) and transposed (Q^T, dO^T: A operands of
// dK^T = Q^T dS, dV^T = dO^T A, contraction in the permuted query order of
// the registers). Every fragment read from LDS feeds KS products.
template <int DH, int KS>
__global__ void __launch_bounds__(BW_NT, 2) dense_bwd_kv_mfma_kernel(DenseBwdParams p) {
  constexpr int NKC = (DH + 31) / 32, RP = NKC * 32 + 8, NDT = (DH + 15) / 16, TP = DB_Q + 8;
  __shared__ __attribute__((aligned(16))) uint16_t qr[DB_Q * RP], gr[DB_Q * RP], qT[NDT * 16 * TP],
      gT[NDT * 16 * TP];
  __shared__ float st[DB_Q * 3];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.y, bh = blockIdx.z, b = bh / p.heads, h = bh - b * p.heads;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(p.k) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(p.v) + b * p.kv_bs + (int64_t)h * p.Nk * DH;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_bs + (int64_t)h * p.Nq * DH;
  const uint16_t* G0 = reinterpret_cast<const uint16_t*>(p.dO) + (int64_t)b * p.Nq * p.D + h * DH;
  const float* S = p.stats + ((int64_t)b * p.heads + h) * p.Nq * 3;
  int kj[KS];
  bool live[KS];
  uint4 kf[KS][NKC], vf[KS][NKC];
  floatx4 dk[KS][NDT], dv[KS][NDT];
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    kj[u] = blockIdx.x * (DB_K * KS) + u * DB_K + w * 16 + c;
    live[u] = kj[u] < p.Nk;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * g;
      kf[u][kc] = (live[u] && d < DH) ? *reinterpret_cast<const uint4*>(K + (int64_t)kj[u] * DH + d)
                                      : uint4{0, 0, 0, 0};
      vf[u][kc] = (live[u] && d < DH) ? *reinterpret_cast<const uint4*>(V + (int64_t)kj[u] * DH + d)
                                      : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) { dk[u][dt] = zero4(); dv[u][dt] = zero4(); }
  }
  const int q0 = chunk * p.qchunk, q1 = min(p.Nq, q0 + p.qchunk);
  // the next tile's global loads are issued before the current tile's
  // products and written to LDS after them
  QuadChunks<DH, DB_Q> qa, ga;
  float sv = 0.f;
  auto fetch = [&](int t0) {
    load_quads<DH, DB_Q>(Q, DH, t0, q1, tid, qa);
    load_quads<DH, DB_Q>(G0, p.D, t0, q1, tid, ga);
    if (tid < DB_Q * 3) sv = t0 + tid / 3 < q1 ? S[(int64_t)t0 * 3 + tid] : 0.f;
  };
  if (q0 < q1) fetch(q0);
  for (int t0 = q0; t0 < q1; t0 += DB_Q) {
    __syncthreads();
    put_quads<DH, DB_Q, RP, TP>(qa, qr, qT, tid);
    put_quads<DH, DB_Q, RP, TP>(ga, gr, gT, tid);
    if (tid < DB_Q * 3) st[tid] = tid % 3 == 1 ? (sv > 0.f ? 1.f / sv : 0.f) : sv;  // row sum -> its reciprocal
    __syncthreads();
    if (t0 + DB_Q < q1) fetch(t0 + DB_Q);
#pragma unroll
    for (int qt0 = 0; qt0 < 4; qt0 += 2) {
      floatx4 pa[KS][2], da[KS][2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int qt = qt0 + v;
        floatx4 sc[KS], dp[KS];
#pragma unroll
        for (int u = 0; u < KS; ++u) { sc[u] = zero4(); dp[u] = zero4(); }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const uint4 qa4 = *reinterpret_cast<const uint4*>(&qr[(qt * 16 + c) * RP + kc * 32 + 8 * g]);
          const uint4 ga4 = *reinterpret_cast<const uint4*>(&gr[(qt * 16 + c) * RP + kc * 32 + 8 * g]);
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            sc[u] = mfma_bf16(qa4, kf[u][kc], sc[u]);
            dp[u] = mfma_bf16(ga4, vf[u][kc], dp[u]);
          }
        }
        // S[query qt*16 + 4g + r][key of sub-tile u, column c]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qrow = qt * 16 + 4 * g + r;
          const bool qok = t0 + qrow < q1;
          const float m = st[qrow * 3], rl = st[qrow * 3 + 1], dd = st[qrow * 3 + 2];
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const float a = qok ? __expf(sc[u][r] * p.scale - m) * rl : 0.f;
            pa[u][v][r] = a;
            da[u][v][r] = a * (dp[u][r] - dd);
          }
        }
      }
      uint4 pf[KS], df[KS];
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        pf[u] = uint4{pack_bf2(pa[u][0][0], pa[u][0][1]), pack_bf2(pa[u][0][2], pa[u][0][3]),
                      pack_bf2(pa[u][1][0], pa[u][1][1]), pack_bf2(pa[u][1][2], pa[u][1][3])};
        df[u] = uint4{pack_bf2(da[u][0][0], da[u][0][1]), pack_bf2(da[u][0][2], da[u][0][3]),
                      pack_bf2(da[u][1][0], da[u][1][1]), pack_bf2(da[u][1][2], da[u][1][3])};
      }
      const int kb = qt0 * 16 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int row = (dt * 16 + c) * TP;
        const uint2 glo = *reinterpret_cast<const uint2*>(&gT[row + kb]);
        const uint2 ghi = *reinterpret_cast<const uint2*>(&gT[row + kb + 16]);
        const uint2 qlo = *reinterpret_cast<const uint2*>(&qT[row + kb]);
        const uint2 qhi = *reinterpret_cast<const uint2*>(&qT[row + kb + 16]);
        const uint4 gA = uint4{glo.x, glo.y, ghi.x, ghi.y}, qA = uint4{qlo.x, qlo.y, qhi.x, qhi.y};
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          dv[u][dt] = mfma_bf16(gA, pf[u], dv[u][dt]);
          dk[u][dt] = mfma_bf16(qA, df[u], dk[u][dt]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    if (!live[u]) continue;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = dt * 16 + 4 * g;
      if (d >= DH) continue;
      const float4 kk = float4{dk[u][dt][0], dk[u][dt][1], dk[u][dt][2], dk[u][dt][3]};
      const float4 vv = float4{dv[u][dt][0], dv[u][dt][1], dv[u][dt][2], dv[u][dt][3]};
      if (p.chunks == 1) {
        *reinterpret_cast<float4*>(p.dk + b * p.dkv_bs + ((int64_t)h * p.Nk + kj[u]) * DH + d) =
            float4{kk.x * p.scale, kk.y * p.scale, kk.z * p.scale, kk.w * p.scale};
        *reinterpret_cast<float4*>(p.dv + b * p.dkv_bs + ((int64_t)h * p.Nk + kj[u]) * DH + d) = vv;
      } else {
        float* pt = p.part + ((((int64_t)chunk * p.B + b) * p.heads + h) * p.Nk + kj[u]) * 2 * DH;
        *reinterpret_cast<float4*>(pt + d) = kk;
        *reinterpret_cast<float4*>(pt + DH + d) = vv;
      }
    }
  }
}

template <typename T, int DH>
static hipError_t run_dense_bwd(const DenseBwdDesc& d, hipStream_t s) {
  DenseBwdParams p;
  p.q = d.q; p.k = d.k; p.v = d.v; p.dO = d.dO;
  p.q_bs = d.q_bs; p.kv_bs = d.kv_bs;
  p.dq = d.dq; p.dk = d.dk; p.dv = d.dv; p.dq_bs = d.dq_bs; p.dkv_bs = d.dkv_bs;
  p.dq_tok = d.dq_tok; p.dq_bf16 = d.dq_bf16;
  if (d.dq_bf16 && sizeof(T) != 2) return hipErrorInvalidValue;  // the fp32 kernels write fp32
  p.stats = d.stats; p.part = d.part;
  p.B = d.B; p.heads = d.heads; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.qchunk = d.qchunk; p.chunks = d.chunks;
  p.scale = d.scale;
  constexpr bool BF = sizeof(T) == 2;
  const dim3 gq((d.Nq + DB_Q - 1) / DB_Q, d.heads, d.B), gk((d.Nk + DB_K - 1) / DB_K, d.chunks, d.B * d.heads);
  // matrix-core query-major kernel: several 128-query tiles a workgroup (the
  // staged keys serve them all) while that still leaves >= 512 workgroups
  const int64_t bh = (int64_t)d.heads * d.B;
  constexpr int QT = DQ_NT / 4;  // queries a tile (16 a wave)
  p.qtiles = 1;
  while (p.qtiles < DM_QT && (int64_t)((d.Nq + 2 * QT * p.qtiles - 1) / (2 * QT * p.qtiles)) * bh >= 512)
    p.qtiles *= 2;
  const int qpw = QT * p.qtiles;  // queries a workgroup
  const dim3 gqm((d.Nq + qpw - 1) / qpw, d.heads, d.B);
  if (BF && d.Nk <= DM_MAXK) {
    hipLaunchKernelGGL((dense_bwd_q_mfma_kernel<DH>), gqm, dim3(DQ_NT), 0, s, p);
  } else if (BF) {
    const dim3 gqs((d.Nq + QT - 1) / QT, d.heads, d.B);
    hipLaunchKernelGGL((dense_bwd_q_mfma_stream_kernel<DH>), gqs, dim3(DQ_NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((dense_bwd_q_kernel<T, DH>), gq, dim3(BW_NT), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // two 16-key sub-tiles a wave when there are at least 128 keys and the grid
  // keeps at least one workgroup per CU
  const dim3 gk2((d.Nk + 2 * DB_K - 1) / (2 * DB_K), d.chunks, d.B * d.heads);
  const bool ks2 = d.Nk >= 2 * DB_K && (int64_t)gk2.x * gk2.y * gk2.z >= 256;
  if (BF && ks2) hipLaunchKernelGGL((dense_bwd_kv_mfma_kernel<DH, 2>), gk2, dim3(BW_NT), 0, s, p);
  else if (BF) hipLaunchKernelGGL((dense_bwd_kv_mfma_kernel<DH, 1>), gk, dim3(BW_NT), 0, s, p);
  else hipLaunchKernelGGL((dense_bwd_kv_kernel<T, DH>), gk, dim3(BW_NT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || d.chunks == 1) return e;
  const int64_t n = (int64_t)d.B * d.heads * d.Nk * DH;
  hipLaunchKernelGGL((dense_bwd_reduce_kernel<DH>), dim3((unsigned)((n + BW_NT - 1) / BW_NT)), dim3(BW_NT), 0, s,
                     p);
  return hipGetLastError();
}

hipError_t launch_dense_bwd(const DenseBwdDesc& d, int f32, hipStream_t s) {
  if (d.B == 0 || d.Nq == 0) return hipSuccess;
  if (d.dh == 72) return f32 ? run_dense_bwd<float, 72>(d, s) : run_dense_bwd<uint16_t, 72>(d, s);
  if (d.dh == 64) return f32 ? run_dense_bwd<float, 64>(d, s) : run_dense_bwd<uint16_t, 64>(d, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Window-average backward: dx[b, t] (+)= dP[b, proxy(t)] / P, 4 floats a thread
// ----------------------------------------------------------------------------
struct PoolBwdParams {
  const float* dP;
  float* dx;
  int F, H, W, D;
  int pt, ph, pw;
  int64_t rows;  // B * N
  int accumulate;
  float P;
};

// PB_ROWS consecutive token rows per workgroup. A row's proxy depends on
// wave-uniform values only, so its index math runs once per row on the
// scalar unit, and consecutive rows of one proxy (the tokens of a window row)
// share its quotients. Lanes cover 2 * BW_NT float4 columns per
// pass; every load of a pass (d_x too, when accumulating) is issued before its
// first store, so no store waits for a load.
constexpr int PB_ROWS = 8;
template <bool ACC>
__global__ void __launch_bounds__(BW_NT) pool_bwd_kernel(PoolBwdParams p) {
  const float* __restrict__ dP = p.dP;
  float* __restrict__ dx = p.dx;
  const int q4 = p.D / 4;
  const int N = p.F * p.H * p.W;
  const int nh = p.H / p.ph, nw = p.W / p.pw, M = (p.F / p.pt) * nh * nw;
  const int64_t r0 = (int64_t)blockIdx.x * PB_ROWS;
  const int nr = (int)min((int64_t)PB_ROWS, p.rows - r0);
  typedef float f4 __attribute__((ext_vector_type(4)));
  for (int cb = 0; cb < q4; cb += 2 * BW_NT) {
    const int c0 = cb + threadIdx.x, c1 = c0 + BW_NT;
    // columns past the row load its last vector (in bounds, never stored)
    const int l0 = min(c0, q4 - 1), l1 = min(c1, q4 - 1);
    f4 v[PB_ROWS][2], a[ACC ? PB_ROWS : 1][2];
    // every row's proxy (batch-major index) before the first load: B*N and
    // N fit in 32 bits
    int64_t bm[PB_ROWS];
#pragma unroll
    for (int r = 0; r < PB_ROWS; ++r) {
      if (r >= nr) break;
      const int row = (int)(r0 + r), b = row / N, tok = row - b * N;
      const int t = tok / (p.H * p.W), i = (tok / p.W) % p.H, j = tok % p.W;
      bm[r] = (int64_t)b * M + ((t / p.pt) * nh + i / p.ph) * nw + j / p.pw;
    }
#pragma unroll
    for (int r = 0; r < PB_ROWS; ++r) {
      if (r >= nr) break;
      const int64_t row = r0 + r;
      const f4* src = reinterpret_cast<const f4*>(dP + bm[r] * p.D);
      v[r][0] = src[l0];
      v[r][1] = src[l1];
      if constexpr (ACC) {
        const f4* d4 = reinterpret_cast<const f4*>(dx + row * p.D);
        a[r][0] = d4[l0];
        a[r][1] = d4[l1];
      }
    }
    f4 q[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int r = 0; r < PB_ROWS; ++r) {
      if (r >= nr) break;
      f4* dst = reinterpret_cast<f4*>(dx + (r0 + r) * p.D);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (r == 0 || bm[r] != bm[r - 1]) {  // the first row of a run of one proxy
          const f4 g = v[r][h];
          q[h] = f4{g.x / p.P, g.y / p.P, g.z / p.P, g.w / p.P};
        }
        const int c = h ? c1 : c0;
        if (c >= q4) continue;
        f4 o = q[h];
        if constexpr (ACC) o = f4{o.x + a[r][h].x, o.y + a[r][h].y, o.z + a[r][h].z, o.w + a[r][h].w};
        dst[c] = o;
      }
    }
  }
}

hipError_t launch_pool_bwd(const PoolBwdDesc& d, hipStream_t s) {
  PoolBwdParams p;
  p.dP = d.dP; p.dx = d.dx;
  p.F = d.F; p.H = d.H; p.W = d.W; p.D = d.D;
  p.pt = d.pt; p.ph = d.ph; p.pw = d.pw;
  p.rows = (int64_t)d.B * d.F * d.H * d.W;
  p.accumulate = d.accumulate;
  p.P = (float)(d.pt * d.ph * d.pw);
  if (p.rows == 0 || d.D == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.rows + PB_ROWS - 1) / PB_ROWS));
  if (p.accumulate) hipLaunchKernelGGL((pool_bwd_kernel<true>), grid, dim3(BW_NT), 0, s, p);
  else hipLaunchKernelGGL((pool_bwd_kernel<false>), grid, dim3(BW_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ptdit
