// Attention cores of the PT-DiT block: proxy self-attention and the
// token->proxy cross-attention (GIIM), window and shifted-window attention
// (TCM).
//
// Layout trick shared by every core: scores are computed transposed,
// S^T = K Q^T, with the keys as the MFMA's first operand. A lane then holds
// four keys of ONE query (query = lane % 16), which is exactly the operand
// layout the next MFMA, O^T = V^T P^T, wants for P^T, and the O^T accumulator
// again keeps one query per lane % 16. Softmax statistics (row max, row sum)
// therefore live in registers of the lanes that own the query and are
// reduced across the four lanes l, l^16, l^32, l^48 only. No LDS round trip
// between the two products.
//
// Keys/values of the current block sit in LDS: K row-major (16-byte chunks),
// V transposed (bf16) so an O^T operand fetch is two 8-byte reads. The head
// dimension (72 = 2*32 + 8) is zero-padded to the MFMA contraction width;
// rows of O^T past dh are computed on zeros and never stored.
//
// Window attention never materialises padding or the cyclic roll: each
// window slot maps (rolled, padded) -> original coordinates; slots outside
// the real grid are pad tokens whose key/value are the projection biases.
#include "common.hpp"
#include "kernels.hpp"

namespace ptdit {

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 policy
template <int DH>
struct BF16P {
  using T = uint16_t;
  static constexpr int NKC = (DH + 31) / 32;  // contraction chunks (32) of the head dim
  static constexpr int NDT = (DH + 15) / 16;  // 16-row tiles of O^T
  static constexpr int DCH = DH / 8;          // 8-element chunks per head row
  static constexpr int TPV = 2;               // key tiles (16) per O^T MFMA
  struct QF { uint4 v[NKC]; };

  template <int KEYS>
  struct Smem {
    uint4 k[KEYS * DCH];
    uint16_t vt[NDT * 16][KEYS + 4];
  };

  __device__ static QF load_q(const T* row, int lane) {
    QF f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * (lane >> 4);
      f.v[kc] = (row && d < DH) ? *reinterpret_cast<const uint4*>(row + d) : uint4{0, 0, 0, 0};
    }
    return f;
  }

  template <int KEYS>
  __device__ static void zero_pad(Smem<KEYS>& sm, int tid, int nt) {
    for (int i = tid; i < (NDT * 16 - DH) * (KEYS + 4); i += nt)
      sm.vt[DH + i / (KEYS + 4)][i % (KEYS + 4)] = 0;
  }

  // Staging of chunk c (8 channels) of key slot s in two steps, so that a
  // thread's loads for all its chunks are in flight together: load() reads
  // the K and V chunk (NULL rows give zeros), put() writes them to LDS.
  struct Raw { uint4 k, v; };
  __device__ static Raw load(int c, const T* krow, const T* vrow) {
    return Raw{krow ? *reinterpret_cast<const uint4*>(krow + c * 8) : uint4{0, 0, 0, 0},
               vrow ? *reinterpret_cast<const uint4*>(vrow + c * 8) : uint4{0, 0, 0, 0}};
  }
  template <int KEYS>
  __device__ static void put(Smem<KEYS>& sm, int s, int c, const Raw& r) {
    const uint4 kv = r.k, vv = r.v;
    sm.k[s * DCH + c] = kv;
    sm.vt[c * 8 + 0][s] = (uint16_t)(vv.x & 0xffff); sm.vt[c * 8 + 1][s] = (uint16_t)(vv.x >> 16);
    sm.vt[c * 8 + 2][s] = (uint16_t)(vv.y & 0xffff); sm.vt[c * 8 + 3][s] = (uint16_t)(vv.y >> 16);
    sm.vt[c * 8 + 4][s] = (uint16_t)(vv.z & 0xffff); sm.vt[c * 8 + 5][s] = (uint16_t)(vv.z >> 16);
    sm.vt[c * 8 + 6][s] = (uint16_t)(vv.w & 0xffff); sm.vt[c * 8 + 7][s] = (uint16_t)(vv.w >> 16);
  }

  // Write chunk c of V for key slots 4*kq .. 4*kq+3 (already loaded),
  // transposed in registers: each V^T row gets one 8-byte write.
  template <int KEYS>
  __device__ static void put_vquad(Smem<KEYS>& sm, int kq, int c, const uint4* v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = (j & 1) * 16;
      const uint32_t a0 = (reinterpret_cast<const uint32_t*>(&v[0])[j >> 1] >> sh) & 0xffffu;
      const uint32_t a1 = (reinterpret_cast<const uint32_t*>(&v[1])[j >> 1] >> sh) & 0xffffu;
      const uint32_t a2 = (reinterpret_cast<const uint32_t*>(&v[2])[j >> 1] >> sh) & 0xffffu;
      const uint32_t a3 = (reinterpret_cast<const uint32_t*>(&v[3])[j >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<uint2*>(&sm.vt[c * 8 + j][kq * 4]) = uint2{a0 | (a1 << 16), a2 | (a3 << 16)};
    }
  }

  // S^T tile t: rows = keys t*16 .. +16, columns = the wave's 16 queries.
  template <int KEYS>
  __device__ static floatx4 score(const Smem<KEYS>& sm, const QF& q, int t, int lane) {
    floatx4 acc = zero4();
    const int key = t * 16 + (lane & 15);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = kc * 32 + 8 * (lane >> 4);
      const uint4 kf = d < DH ? sm.k[key * DCH + d / 8] : uint4{0, 0, 0, 0};
      acc = mfma_bf16(kf, q.v[kc], acc);
    }
    return acc;
  }

  // O^T += V^T P^T over key tiles t0, t0+1. Contraction index (lane group g,
  // element e) <-> key t0*16 + 4g + e for e < 4, (t0+1)*16 + 4g + e-4 else:
  // the keys whose probabilities the lane holds in p[0] and p[1].
  template <int KEYS>
  __device__ static void pv(const Smem<KEYS>& sm, floatx4* o, const floatx4* p, int t0, int lane) {
    const uint4 pf = uint4{pack_bf2(p[0][0], p[0][1]), pack_bf2(p[0][2], p[0][3]),
                           pack_bf2(p[1][0], p[1][1]), pack_bf2(p[1][2], p[1][3])};
    const int kb = t0 * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int drow = dt * 16 + (lane & 15);
      const uint2 lo = *reinterpret_cast<const uint2*>(&sm.vt[drow][kb]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&sm.vt[drow][kb + 16]);
      o[dt] = mfma_bf16(uint4{lo.x, lo.y, hi.x, hi.y}, pf, o[dt]);
    }
  }

  __device__ static void store_o(T* dst, float a, float b, float c, float d) { store4(dst, a, b, c, d); }
};

// ---------------------------------------------------------------- fp32 policy
template <int DH>
struct F32P {
  using T = float;
  static constexpr int NQ = DH / 4;          // contraction steps (4) of the head dim
  static constexpr int NDT = (DH + 15) / 16;
  static constexpr int DCH = DH / 8;
  static constexpr int TPV = 1;
  struct QF { float v[NQ]; };

  template <int KEYS>
  struct Smem {
    float k[KEYS][DH + 1];
    float v[KEYS][NDT * 16 + 1];
  };

  __device__ static QF load_q(const T* row, int lane) {
    QF f;
#pragma unroll
    for (int c = 0; c < NQ; ++c) f.v[c] = row ? row[4 * c + (lane >> 4)] : 0.f;
    return f;
  }

  template <int KEYS>
  __device__ static void zero_pad(Smem<KEYS>& sm, int tid, int nt) {
    constexpr int PADC = NDT * 16 - DH;
    for (int i = tid; i < PADC * KEYS; i += nt) sm.v[i / PADC][DH + i % PADC] = 0.f;
  }

  struct Raw { float4 k0, k1, v0, v1; };
  __device__ static Raw load(int c, const T* krow, const T* vrow) {
    const float4 z = float4{0.f, 0.f, 0.f, 0.f};
    return Raw{krow ? *reinterpret_cast<const float4*>(krow + c * 8) : z,
               krow ? *reinterpret_cast<const float4*>(krow + c * 8 + 4) : z,
               vrow ? *reinterpret_cast<const float4*>(vrow + c * 8) : z,
               vrow ? *reinterpret_cast<const float4*>(vrow + c * 8 + 4) : z};
  }
  template <int KEYS>
  __device__ static void put(Smem<KEYS>& sm, int s, int c, const Raw& r) {
    const float kk[8] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w, r.k1.x, r.k1.y, r.k1.z, r.k1.w};
    const float vv[8] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.k[s][c * 8 + e] = kk[e];
      sm.v[s][c * 8 + e] = vv[e];
    }
  }

  template <int KEYS>
  __device__ static floatx4 score(const Smem<KEYS>& sm, const QF& q, int t, int lane) {
    floatx4 acc = zero4();
    const int key = t * 16 + (lane & 15);
#pragma unroll
    for (int c = 0; c < NQ; ++c) acc = mfma_f32(sm.k[key][4 * c + (lane >> 4)], q.v[c], acc);
    return acc;
  }

  // Contraction index g = lane / 16 of MFMA r <-> key t0*16 + 4g + r.
  template <int KEYS>
  __device__ static void pv(const Smem<KEYS>& sm, floatx4* o, const floatx4* p, int t0, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = t0 * 16 + 4 * (lane >> 4) + r;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma_f32(sm.v[key][dt * 16 + (lane & 15)], p[0][r], o[dt]);
    }
  }

  __device__ static void store_o(T* dst, float a, float b, float c, float d) { store4(dst, a, b, c, d); }
};

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// ---------------------------------------------------------------- flash core
struct FlashParams {
  const void* Q; int64_t q_bs, q_hs;
  const void* K; int64_t k_bs, k_hs;
  const void* V; int64_t v_bs, v_hs;
  void* O;
  int Nq, Nk, D;
  float sl2;  // scale * log2(e)
};

// Workgroup = 4 waves x 16 queries of one (batch, head); keys stream through
// LDS in blocks of KB with an online softmax.
template <class P, int DH, int KB>
__global__ void __launch_bounds__(256) flash_kernel(FlashParams prm) {
  using T = typename P::T;
  constexpr int NT = 256, NTILE = KB / 16;
  __shared__ typename P::template Smem<KB> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int q = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const T* Qb = reinterpret_cast<const T*>(prm.Q) + b * prm.q_bs + h * prm.q_hs;
  const T* Kb = reinterpret_cast<const T*>(prm.K) + b * prm.k_bs + h * prm.k_hs;
  const T* Vb = reinterpret_cast<const T*>(prm.V) + b * prm.v_bs + h * prm.v_hs;
  const auto qf = P::load_q(q < prm.Nq ? Qb + (int64_t)q * DH : nullptr, lane);
  P::zero_pad(sm, tid, NT);

  float m_run = -INFINITY, l_run = 0.f;
  floatx4 o[P::NDT];
#pragma unroll
  for (int i = 0; i < P::NDT; ++i) o[i] = zero4();

  for (int k0 = 0; k0 < prm.Nk; k0 += KB) {
    // every load of the block first, then the LDS writes (after the barrier
    // that retires the previous block's reads)
    constexpr int ITEMS = KB * P::DCH, PER = (ITEMS + NT - 1) / NT;
    typename P::Raw raw[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      const int gk = k0 + s;
      const bool ok = idx < ITEMS && gk < prm.Nk;
      raw[i] = P::load(c, ok ? Kb + (int64_t)gk * DH : nullptr, ok ? Vb + (int64_t)gk * DH : nullptr);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      if (idx < ITEMS) P::put(sm, s, c, raw[i]);
    }
    __syncthreads();
    floatx4 sc[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) sc[t] = P::score(sm, qf, t, lane);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + t * 16 + 4 * (lane >> 4) + r;
        const float v = key < prm.Nk ? sc[t][r] * prm.sl2 : -INFINITY;
        sc[t][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = quad_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(sc[t][r] - m_new);
        sc[t][r] = e;
        rs += e;
      }
    rs = quad_sum(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < P::NDT; ++i) o[i] *= alpha;
#pragma unroll
    for (int t0 = 0; t0 < NTILE; t0 += P::TPV) P::pv(sm, o, &sc[t0], t0, lane);
  }

  if (q < prm.Nq) {
    const float inv = 1.f / l_run;
    T* Ob = reinterpret_cast<T*>(prm.O) + ((int64_t)b * prm.Nq + q) * prm.D + h * DH;
#pragma unroll
    for (int i = 0; i < P::NDT; ++i) {
      const int d = i * 16 + 4 * (lane >> 4);
      if (d < DH) P::store_o(Ob + d, o[i][0] * inv, o[i][1] * inv, o[i][2] * inv, o[i][3] * inv);
    }
  }
}

// ---------------------------------------------------------------- flash core, bf16, wide
// Workgroup = 8 waves x 32 queries (two 16-query tiles per wave) of one
// (batch, head). Keys stream in blocks of 64 through a double-buffered LDS
// stage: block b+1 is loaded into registers while block b is computed, then
// written to the other buffer (one barrier per block). V is transposed in
// registers four keys at a time, so its LDS writes are 8-byte and
// conflict-free. Both query tiles of a wave share every K / V^T fragment read.
constexpr int FW_WAVES = 8, FW_QPW = 32, FW_KB = 64;
constexpr int FW_Q = FW_WAVES * FW_QPW;

template <int DH>
__global__ void __launch_bounds__(FW_WAVES * 64) flash_bf16_wide(FlashParams prm) {
  using P = BF16P<DH>;
  constexpr int NT = FW_WAVES * 64, NKC = P::NKC, NDT = P::NDT, DCH = P::DCH;
  constexpr int VTP = FW_KB + 4;  // V^T row pitch (elements)
  __shared__ uint4 ks[2][FW_KB * DCH];
  __shared__ uint16_t vt[2][NDT * 16][VTP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = lane >> 4, lr = lane & 15;
  const uint16_t* Qb = reinterpret_cast<const uint16_t*>(prm.Q) + b * prm.q_bs + h * prm.q_hs;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(prm.K) + b * prm.k_bs + h * prm.k_hs;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(prm.V) + b * prm.v_bs + h * prm.v_hs;
  const int q0 = blockIdx.x * FW_Q + wave * FW_QPW;

  typename P::QF qf[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = q0 + t * 16 + lr;
    qf[t] = P::load_q(q < prm.Nq ? Qb + (int64_t)q * DH : nullptr, lane);
  }
  // zero the padded V^T rows (d >= DH) of both buffers once
  for (int i = tid; i < 2 * (NDT * 16 - DH) * VTP; i += NT) {
    const int bb = i / ((NDT * 16 - DH) * VTP), r = i % ((NDT * 16 - DH) * VTP);
    vt[bb][DH + r / VTP][r % VTP] = 0;
  }

  // staging work items per block: K chunks (key, c) and V quads (c, key quad)
  constexpr int KITEMS = FW_KB * DCH, VITEMS = DCH * (FW_KB / 4);
  constexpr int KPT = (KITEMS + NT - 1) / NT, VPT = (VITEMS + NT - 1) / NT;
  uint4 kreg[KPT], vreg[VPT][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int it = tid + i * NT;
      kreg[i] = uint4{0, 0, 0, 0};
      if (it < KITEMS) {
        const int key = it / DCH, c = it % DCH, gk = k0 + key;
        if (gk < prm.Nk) kreg[i] = *reinterpret_cast<const uint4*>(Kb + (int64_t)gk * DH + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int it = tid + i * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) vreg[i][e] = uint4{0, 0, 0, 0};
      if (it < VITEMS) {
        const int c = it / (FW_KB / 4), kq = it % (FW_KB / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gk = k0 + kq * 4 + e;
          if (gk < prm.Nk) vreg[i][e] = *reinterpret_cast<const uint4*>(Vb + (int64_t)gk * DH + c * 8);
        }
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int it = tid + i * NT;
      if (it < KITEMS) ks[buf][it] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int it = tid + i * NT;
      if (it < VITEMS) {
        const int c = it / (FW_KB / 4), kq = it % (FW_KB / 4);
        // row d = 8c + j holds keys kq*4 .. kq*4+3: gather element j of the 4 key vectors
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sh = (j & 1) * 16;
          const uint32_t a0 = (w0[j >> 1] >> sh) & 0xffffu, a1 = (w1[j >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (w2[j >> 1] >> sh) & 0xffffu, a3 = (w3[j >> 1] >> sh) & 0xffffu;
          *reinterpret_cast<uint2*>(&vt[buf][c * 8 + j][kq * 4]) = uint2{a0 | (a1 << 16), a2 | (a3 << 16)};
        }
      }
    }
  };

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  floatx4 o[2][NDT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[t][i] = zero4();

  const int nblk = (prm.Nk + FW_KB - 1) / FW_KB;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    const int k0 = blk * FW_KB;
    if (blk + 1 < nblk) gload(k0 + FW_KB);
    // S^T tiles: 4 key tiles x 2 query tiles, K fragments shared
    floatx4 sc[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sc[0][kt] = zero4();
      sc[1][kt] = zero4();
      const int key = kt * 16 + lr;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int d = kc * 32 + 8 * g;
        const uint4 kf = d < DH ? ks[buf][key * DCH + d / 8] : uint4{0, 0, 0, 0};
        sc[0][kt] = mfma_bf16(kf, qf[0].v[kc], sc[0][kt]);
        sc[1][kt] = mfma_bf16(kf, qf[1].v[kc], sc[1][kt]);
      }
    }
    const bool full = k0 + FW_KB <= prm.Nk;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kt * 16 + 4 * g + r;
          const float v = (full || key < prm.Nk) ? sc[t][kt][r] * prm.sl2 : -INFINITY;
          sc[t][kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = quad_max(mx);
      const float m_new = fmaxf(m_run[t], mx);
      const float alpha = fast_exp2(m_run[t] - m_new);
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(sc[t][kt][r] - m_new);
          sc[t][kt][r] = e;
          rs += e;
        }
      rs = quad_sum(rs);
      l_run[t] = l_run[t] * alpha + rs;
      m_run[t] = m_new;
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[t][i] *= alpha;
    }
    // O^T += V^T P^T, V^T fragments shared by both query tiles
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 pf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        pf[t] = uint4{pack_bf2(sc[t][2 * u][0], sc[t][2 * u][1]), pack_bf2(sc[t][2 * u][2], sc[t][2 * u][3]),
                      pack_bf2(sc[t][2 * u + 1][0], sc[t][2 * u + 1][1]),
                      pack_bf2(sc[t][2 * u + 1][2], sc[t][2 * u + 1][3])};
      const int kb = u * 32 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int drow = dt * 16 + lr;
        const uint2 lo = *reinterpret_cast<const uint2*>(&vt[buf][drow][kb]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&vt[buf][drow][kb + 16]);
        const uint4 vf = uint4{lo.x, lo.y, hi.x, hi.y};
        o[0][dt] = mfma_bf16(vf, pf[0], o[0][dt]);
        o[1][dt] = mfma_bf16(vf, pf[1], o[1][dt]);
      }
    }
    if (blk + 1 < nblk) {
      lstore(buf ^ 1);
    }
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = q0 + t * 16 + lr;
    if (q < prm.Nq) {
      const float inv = 1.f / l_run[t];
      uint16_t* Ob = reinterpret_cast<uint16_t*>(prm.O) + ((int64_t)b * prm.Nq + q) * prm.D + h * DH;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int d = i * 16 + 4 * g;
        if (d < DH) store4(Ob + d, o[t][i][0] * inv, o[t][i][1] * inv, o[t][i][2] * inv, o[t][i][3] * inv);
      }
    }
  }
}

// ---------------------------------------------------------------- flash core, bf16, single pass
// For up to 256 keys (every image workload: 256 proxies). Workgroup = 8 waves
// bound to one (batch, head) and a contiguous range of queries: K and V^T of
// that head are staged in LDS once, then each wave walks 32 queries (two
// 16-query tiles) at a time. All 256 scores of a query fit in the lane
// registers (16 key tiles x 4), so the softmax is exact in one pass: one
// max, then exp2(s * c - m * c) with c = scale * log2(e) folded into an FMA,
// no running rescale. Keys past Nk are staged as zeros and masked to -inf.
// Fragment loads run one step ahead of their MFMAs (sched_barrier fences
// keep the scheduler from hoisting all of them, which would not fit in
// registers); the next query block's Q fragments load into the current
// block's Q registers once the scores are done. No barrier inside the loop.
constexpr int FS_MAXK = 256, FS_KT = FS_MAXK / 16;

template <int DH>
__global__ void __launch_bounds__(FW_WAVES * 64) flash_bf16_single(FlashParams prm, int q_per_wg) {
  using P = BF16P<DH>;
  constexpr int NT = FW_WAVES * 64, NDT = P::NDT, DCH = P::DCH;
  constexpr int VTP = FS_MAXK + 4;
  // With a padded head (72 -> 80 rows of V^T), row DH of V^T is all ones, so
  // row DH of O^T = V^T P^T is the softmax denominator: the sum of the very
  // bf16 probabilities the numerator used, accumulated by the MFMA.
  constexpr bool ONES_ROW = NDT * 16 > DH;
  __shared__ uint4 ks[FS_MAXK * DCH];
  __shared__ uint16_t vt[NDT * 16][VTP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = lane >> 4, lr = lane & 15;
  const uint16_t* Qb = reinterpret_cast<const uint16_t*>(prm.Q) + b * prm.q_bs + h * prm.q_hs;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(prm.K) + b * prm.k_bs + h * prm.k_hs;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(prm.V) + b * prm.v_bs + h * prm.v_hs;
  const int qbeg = blockIdx.x * q_per_wg;
  const int qend = min(prm.Nq, qbeg + q_per_wg);

  // Q fragments: NKF chunks of 32 head dims for the 16x16x32 MFMA and, for
  // DH = 32 NKF + 8, the last 8 dims for one 16x16x16 MFMA (lane group g
  // holds dims 32 NKF + 4g .. +3; groups 2, 3 zero)
  constexpr bool TAIL = DH % 32 == 8;
  constexpr int NKF = DH / 32;
  static_assert(TAIL || DH % 32 == 0, "head dim 32k or 32k + 8");
  uint4 qv[2][NKF];
  uint2 qtl[2];
  auto load_qf = [&](int qblk) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = qblk + wave * FW_QPW + t * 16 + lr;
      const bool ok = q < qend;
      const uint16_t* row = Qb + (int64_t)q * DH;
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc)
        qv[t][kc] = ok ? *reinterpret_cast<const uint4*>(row + kc * 32 + 8 * g) : uint4{0, 0, 0, 0};
      qtl[t] = TAIL && ok && g < 2 ? *reinterpret_cast<const uint2*>(row + NKF * 32 + 4 * g) : uint2{0, 0};
    }
  };
  load_qf(qbeg);

  // stage K (chunks) and V^T (four keys per item) of all key slots, zero past
  // Nk: every load first, then the LDS writes (one load latency)
  {
    constexpr int KI = (FS_MAXK * DCH + NT - 1) / NT, VI = (DCH * (FS_MAXK / 4) + NT - 1) / NT;
    uint4 kr[KI], vr[VI][4];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = tid + i * NT;
      const int key = it / DCH, c = it % DCH;
      kr[i] = it < FS_MAXK * DCH && key < prm.Nk ? *reinterpret_cast<const uint4*>(Kb + (int64_t)key * DH + c * 8)
                                                 : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = tid + i * NT;
      const int c = it / (FS_MAXK / 4), kq = it % (FS_MAXK / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kq * 4 + e;
        vr[i][e] = it < DCH * (FS_MAXK / 4) && key < prm.Nk
                       ? *reinterpret_cast<const uint4*>(Vb + (int64_t)key * DH + c * 8)
                       : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = tid + i * NT;
      if (it < FS_MAXK * DCH) ks[it] = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = tid + i * NT;
      if (it >= DCH * (FS_MAXK / 4)) continue;
      const int c = it / (FS_MAXK / 4), kq = it % (FS_MAXK / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = (j & 1) * 16;
        const uint32_t a0 = (reinterpret_cast<const uint32_t*>(&vr[i][0])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a1 = (reinterpret_cast<const uint32_t*>(&vr[i][1])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a2 = (reinterpret_cast<const uint32_t*>(&vr[i][2])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a3 = (reinterpret_cast<const uint32_t*>(&vr[i][3])[j >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(&vt[c * 8 + j][kq * 4]) = uint2{a0 | (a1 << 16), a2 | (a3 << 16)};
      }
    }
  }
  for (int i = tid; i < (NDT * 16 - DH) * VTP; i += NT)
    vt[DH + i / VTP][i % VTP] = (ONES_ROW && i < VTP) ? (uint16_t)0x3f80u : (uint16_t)0;  // bf16 1.0
  __syncthreads();

  const float c2 = prm.sl2;
  const bool masked = prm.Nk < FS_MAXK;  // uniform
  struct KFr { uint4 v[NKF]; uint2 tail; };
  auto load_kf = [&](int kt, KFr& kf) {
    const int key = kt * 16 + lr;
#pragma unroll
    for (int kc = 0; kc < NKF; ++kc) kf.v[kc] = ks[key * DCH + kc * 4 + g];
    kf.tail = TAIL && g < 2 ? reinterpret_cast<const uint2*>(&ks[key * DCH + NKF * 4])[g] : uint2{0, 0};
  };
  auto load_vf = [&](int u, uint4* vf) {
    const int kbase = u * 32 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int drow = dt * 16 + lr;
      const uint2 lo = *reinterpret_cast<const uint2*>(&vt[drow][kbase]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&vt[drow][kbase + 16]);
      vf[dt] = uint4{lo.x, lo.y, hi.x, hi.y};
    }
  };

  for (int qblk = qbeg; qblk < qend; qblk += FW_Q) {
    // S^T for all 256 key slots of both query tiles
    floatx4 sc[2][FS_KT];
    KFr kf[2];
    load_kf(0, kf[0]);
#pragma unroll
    for (int kt = 0; kt < FS_KT; ++kt) {
      if (kt + 1 < FS_KT) load_kf(kt + 1, kf[(kt + 1) & 1]);
      const KFr& f = kf[kt & 1];
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t][kt] = TAIL ? mfma_bf16_k16(f.tail, qtl[t], zero4()) : zero4();
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc) {
        sc[0][kt] = mfma_bf16(f.v[kc], qv[0][kc], sc[0][kt]);
        sc[1][kt] = mfma_bf16(f.v[kc], qv[1][kc], sc[1][kt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (qblk + FW_Q < qend) load_qf(qblk + FW_Q);  // next block; scores no longer need the Q fragments
    if (masked) {
#pragma unroll
      for (int kt = 0; kt < FS_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt * 16 + 4 * g + r >= prm.Nk) sc[0][kt][r] = sc[1][kt][r] = -INFINITY;
    }

    // exact softmax numerators and sums; P^T packed to bf16 right away
    uint32_t pk[2][FS_KT][2];
    float lsum[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float mx = sc[t][0][0];
#pragma unroll
      for (int kt = 0; kt < FS_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[t][kt][r]);
      const float nmc = -quad_max(mx) * c2;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < FS_KT; ++kt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(fmaf(sc[t][kt][r], c2, nmc));
          if constexpr (!ONES_ROW) rs += e[r];
        }
        pk[t][kt][0] = pack_bf2(e[0], e[1]);
        pk[t][kt][1] = pack_bf2(e[2], e[3]);
      }
      if constexpr (!ONES_ROW) lsum[t] = quad_sum(rs);
    }

    // O^T = V^T P^T over key-tile pairs
    floatx4 o[2][NDT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[t][i] = zero4();
    uint4 vf[2][NDT];
    load_vf(0, vf[0]);
#pragma unroll
    for (int u = 0; u < FS_KT / 2; ++u) {
      if (u + 1 < FS_KT / 2) load_vf(u + 1, vf[(u + 1) & 1]);
      const uint4 pf0 = uint4{pk[0][2 * u][0], pk[0][2 * u][1], pk[0][2 * u + 1][0], pk[0][2 * u + 1][1]};
      const uint4 pf1 = uint4{pk[1][2 * u][0], pk[1][2 * u][1], pk[1][2 * u + 1][0], pk[1][2 * u + 1][1]};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[0][dt] = mfma_bf16(vf[u & 1][dt], pf0, o[0][dt]);
        o[1][dt] = mfma_bf16(vf[u & 1][dt], pf1, o[1][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (ONES_ROW) {
      // O^T row DH sits in tile DH / 16, element DH % 4 of lane group (DH % 16) / 4
      constexpr int DT = DH / 16, GR = (DH % 16) / 4, EL = DH % 4;
#pragma unroll
      for (int t = 0; t < 2; ++t) lsum[t] = __shfl(o[t][DT][EL], GR * 16 + lr);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = qblk + wave * FW_QPW + t * 16 + lr;
      if (q < qend) {
        const float inv = 1.f / lsum[t];
        uint16_t* Ob = reinterpret_cast<uint16_t*>(prm.O) + ((int64_t)b * prm.Nq + q) * prm.D + h * DH;
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          const int d = i * 16 + 4 * g;
          if (d < DH) store4(Ob + d, o[t][i][0] * inv, o[t][i][1] * inv, o[t][i][2] * inv, o[t][i][3] * inv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- flash core, bf16, ping-pong
// Up to FP_MAXK keys, all resident in LDS (K row-major chunks; V^T with a
// row of ones at DH, so the softmax denominator is accumulated by the MFMA
// as row DH of O^T). Keys are taken in blocks of 64 with an online softmax.
// Each wave owns 64 queries (four 16-query tiles), so every K or V^T
// fragment read from LDS feeds four MFMAs: with two tiles per wave the
// fragment reads, not the matrix core, set the pace.
// The 8 waves form two groups of four, one wave of each per SIMD, that run
// one phase apart: a wave alternates a VALU phase (softmax of one key block:
// max, exp2, bf16 pack; O rescaled when some running max grew) and an MFMA
// phase (P V of that block, then the scores of the next block, possibly of
// the next query block). Every phase ends at a workgroup barrier, so while
// one group's softmax occupies a SIMD's VALU the other group's products
// occupy its matrix core. K/V are read-only after staging: the barriers only
// keep the two groups in step.
constexpr int FP_MAXK = 512;

template <int DH>
constexpr int flash_pp_lds_bytes(int keys) {
  return keys * (DH / 8) * 16 + ((DH + 15) / 16) * 16 * (keys + 4) * 2;
}

// FP_QT 16-query tiles per wave, key blocks of FP_KB
constexpr int PP_QT = 2, PP_KB = 128;
template <int DH, int FP_QT, int FP_KB>
__global__ void __launch_bounds__(FW_WAVES * 64, 1) flash_bf16_pp(FlashParams prm, int q_per_wg, int nkb) {
  constexpr int FP_KT = FP_KB / 16, FP_QPW = 16 * FP_QT, FP_Q = FW_WAVES * FP_QPW;
  using P = BF16P<DH>;
  constexpr int NT = FW_WAVES * 64, NDT = P::NDT, DCH = P::DCH;
  static_assert(NDT * 16 > DH, "the denominator uses the ones row of V^T");
  extern __shared__ uint4 fp_smem[];
  const int keys = nkb * FP_KB, vtp = keys + 4;
  uint4* const ks = fp_smem;                                               // [keys][DCH]
  uint16_t* const vt = reinterpret_cast<uint16_t*>(fp_smem + keys * DCH);  // [NDT*16][vtp]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = lane >> 4, lr = lane & 15;
  const uint16_t* Qb = reinterpret_cast<const uint16_t*>(prm.Q) + b * prm.q_bs + h * prm.q_hs;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(prm.K) + b * prm.k_bs + h * prm.k_hs;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(prm.V) + b * prm.v_bs + h * prm.v_hs;
  const int qbeg = blockIdx.x * q_per_wg;
  const int qend = min(prm.Nq, qbeg + q_per_wg);
  const int Nk = prm.Nk;

  // Q fragments: NKF chunks of 32 head dims for the 16x16x32 MFMA, then the
  // last 8 dims (DH = 32 NKF + 8) for one 16x16x16 MFMA (lane group g holds
  // dims 32 NKF + 4g .. +3; groups 2, 3 zero)
  constexpr int NKF = DH / 32;
  static_assert(DH % 32 == 8, "head dim 32k + 8");
  struct QFr { uint4 v[NKF]; uint2 tail; };
  QFr qf[FP_QT];
  // addresses: a wave-uniform base (the wave's first query row) + a 32-bit
  // lane offset + a per-tile constant
  const uint32_t q_lane = (uint32_t)((lr * DH + 8 * g) * 2), q_tail = (uint32_t)((lr * DH + NKF * 32 + 4 * g) * 2);
  auto load_qf = [&](int qblk) {
    const int q0 = qblk + wave * FP_QPW;
    const char* base = reinterpret_cast<const char*>(Qb + (int64_t)q0 * DH);
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      const bool ok = q0 + t * 16 + lr < qend;
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc)
        qf[t].v[kc] = ok ? *reinterpret_cast<const uint4*>(base + q_lane + (t * 16 * DH + kc * 32) * 2)
                         : uint4{0, 0, 0, 0};
      qf[t].tail = ok && g < 2 ? *reinterpret_cast<const uint2*>(base + q_tail + t * 16 * DH * 2) : uint2{0, 0};
    }
  };
  load_qf(qbeg);

  // stage K (chunks) and V^T (four keys per item) of every key slot, zeros
  // past Nk; row DH of V^T is all ones, rows past it zero. Every load first,
  // then the LDS writes (one load latency).
  {
    constexpr int KI = (FP_MAXK * DCH + NT - 1) / NT, VI = (DCH * (FP_MAXK / 4) + NT - 1) / NT;
    uint4 kr[KI], vr[VI][4];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = tid + i * NT;
      const int key = it / DCH, c = it % DCH;
      kr[i] = it < keys * DCH && key < Nk ? *reinterpret_cast<const uint4*>(Kb + (int64_t)key * DH + c * 8)
                                          : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = tid + i * NT;
      const int c = it / (keys / 4), kq = it % (keys / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kq * 4 + e;
        vr[i][e] = it < DCH * (keys / 4) && key < Nk ? *reinterpret_cast<const uint4*>(Vb + (int64_t)key * DH + c * 8)
                                                     : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = tid + i * NT;
      if (it < keys * DCH) ks[it] = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = tid + i * NT;
      if (it >= DCH * (keys / 4)) continue;
      const int c = it / (keys / 4), kq = it % (keys / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = (j & 1) * 16;
        const uint32_t a0 = (reinterpret_cast<const uint32_t*>(&vr[i][0])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a1 = (reinterpret_cast<const uint32_t*>(&vr[i][1])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a2 = (reinterpret_cast<const uint32_t*>(&vr[i][2])[j >> 1] >> sh) & 0xffffu;
        const uint32_t a3 = (reinterpret_cast<const uint32_t*>(&vr[i][3])[j >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(&vt[(c * 8 + j) * vtp + kq * 4]) = uint2{a0 | (a1 << 16), a2 | (a3 << 16)};
      }
    }
  }
  for (int i = tid; i < (NDT * 16 - DH) * vtp; i += NT) vt[DH * vtp + i] = i < vtp ? (uint16_t)0x3f80u : (uint16_t)0;
  __syncthreads();

  const float c2 = prm.sl2;
  const bool tail_masked = Nk < keys;  // uniform: only the last key block holds slots past Nk

  floatx4 sc[FP_QT][FP_KT];
  uint32_t pk[FP_QT][FP_KT][2];
  floatx4 o[FP_QT][NDT];
  float m_run[FP_QT];

  auto scores = [&](int kb) {
    struct KFr { uint4 v[NKF]; uint2 tail; };
    KFr kf[2];
    auto load_kf = [&](int kt, KFr& f) {
      const int key = kb * FP_KB + kt * 16 + lr;
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc) f.v[kc] = ks[key * DCH + kc * 4 + g];
      f.tail = g < 2 ? reinterpret_cast<const uint2*>(&ks[key * DCH + NKF * 4])[g] : uint2{0, 0};
    };
    load_kf(0, kf[0]);
#pragma unroll
    for (int kt = 0; kt < FP_KT; ++kt) {
      if (kt + 1 < FP_KT) load_kf(kt + 1, kf[(kt + 1) & 1]);
      const KFr& f = kf[kt & 1];
#pragma unroll
      for (int t = 0; t < FP_QT; ++t) sc[t][kt] = mfma_bf16_k16(f.tail, qf[t].tail, zero4());
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc)
#pragma unroll
        for (int t = 0; t < FP_QT; ++t) sc[t][kt] = mfma_bf16(f.v[kc], qf[t].v[kc], sc[t][kt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv = [&](int kb) {
    uint4 vf[2][NDT];
    auto load_vf = [&](int u, uint4* f) {
      const uint16_t* base = vt + lr * vtp + kb * FP_KB + u * 32 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t* row = base + dt * 16 * vtp;
        const uint2 lo = *reinterpret_cast<const uint2*>(row);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
        f[dt] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    };
    load_vf(0, vf[0]);
#pragma unroll
    for (int u = 0; u < FP_KT / 2; ++u) {
      if (u + 1 < FP_KT / 2) load_vf(u + 1, vf[(u + 1) & 1]);
#pragma unroll
      for (int t = 0; t < FP_QT; ++t) {
        const uint4 pf = uint4{pk[t][2 * u][0], pk[t][2 * u][1], pk[t][2 * u + 1][0], pk[t][2 * u + 1][1]};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[t][dt] = mfma_bf16(vf[u & 1][dt], pf, o[t][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // softmax of key block kb; kb == 0 starts a query block (O is zero)
  auto softmax = [&](int kb) {
    if (kb == nkb - 1 && tail_masked) {
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool out = kb * FP_KB + kt * 16 + 4 * g + r >= Nk;
#pragma unroll
          for (int t = 0; t < FP_QT; ++t) sc[t][kt][r] = out ? -INFINITY : sc[t][kt][r];
        }
    }
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      float mx = sc[t][0][0];
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[t][kt][r]);
      mx = quad_max(mx);
      float m_new = mx;
      if (kb > 0) {
        m_new = fmaxf(m_run[t], mx);
        // rescale O only when some query's running max grew
        if (__builtin_amdgcn_ballot_w64(m_new > m_run[t]) != 0) {
          const float alpha = fast_exp2((m_run[t] - m_new) * c2);
#pragma unroll
          for (int i = 0; i < NDT; ++i) o[t][i] *= alpha;
        }
      }
      m_run[t] = m_new;
      const float nmc = -m_new * c2;
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = fast_exp2(fmaf(sc[t][kt][r], c2, nmc));
        pk[t][kt][0] = pack_bf2(e[0], e[1]);
        pk[t][kt][1] = pack_bf2(e[2], e[3]);
      }
    }
  };
  auto zero_o = [&]() {
#pragma unroll
    for (int t = 0; t < FP_QT; ++t)
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[t][i] = zero4();
  };
  // O^T row DH (the denominator) sits in tile DH / 16, element DH % 4 of lane group (DH % 16) / 4
  auto store_o = [&](int qblk) {
    constexpr int DT = DH / 16, GR = (DH % 16) / 4, EL = DH % 4;
    const int q0 = qblk + wave * FP_QPW;
    char* base = reinterpret_cast<char*>(reinterpret_cast<uint16_t*>(prm.O) + ((int64_t)b * prm.Nq + q0) * prm.D + h * DH);
    const uint32_t o_lane = (uint32_t)((lr * prm.D + 4 * g) * 2);
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      const float lsum = __shfl(o[t][DT][EL], GR * 16 + lr);
      if (q0 + t * 16 + lr < qend) {
        const float inv = 1.f / lsum;
        char* row = base + o_lane + (uint32_t)(t * 16 * prm.D * 2);
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          if (i * 16 + 4 * g < DH)
            store4(reinterpret_cast<uint16_t*>(row + i * 32), o[t][i][0] * inv, o[t][i][1] * inv, o[t][i][2] * inv,
                   o[t][i][3] * inv);
        }
      }
    }
  };
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // group 1 runs one phase behind group 0
  if (grp == 1) phase_end();
  scores(0);
  phase_end();
  for (int qblk = qbeg; qblk < qend; qblk += FP_Q) {
    const bool more = qblk + FP_Q < qend;
    for (int kb = 0; kb < nkb; ++kb) {
      // VALU phase: (next query block's Q, whose last scores are done,)
      // softmax of block kb (O starts at zero with block 0)
      if (kb == nkb - 1 && more) load_qf(qblk + FP_Q);
      softmax(kb);
      if (kb == 0) zero_o();
      phase_end();
      // MFMA phase: P V of block kb (then the finished block's output), then
      // the next scores
      pv(kb);
      if (kb + 1 < nkb) {
        scores(kb + 1);
      } else {
        store_o(qblk);
        if (more) scores(0);
      }
      phase_end();
    }
  }
  if (grp == 0) phase_end();
}

// ---------------------------------------------------------------- flash core, bf16, ping-pong, streamed keys
// More than FP_MAXK keys: the same two-group schedule (PP_QT tiles per wave,
// key blocks of 128), with K/V streamed through a ring of three LDS buffers.
// V^T is first packed per (batch, head, key block) into the exact LDS image
// of one block (80 rows of FPS_VTP elements: DH rows of V^T, the ones row,
// zero rows; keys past Nk zero), so both K and V^T move with direct
// global -> LDS DMA and no staging registers. Group 0 issues the DMA of step
// s + 2 at the end of its MFMA phase s (after that phase's last LDS read);
// every wave waits for its memory operations at the end of the next VALU
// phase, which reads no LDS, and the barrier closing that phase publishes the
// block. Step s's buffer (s mod 3) is read in the four phases starting at
// phase 2s, so the buffer refilled for step s + 2 (that of step s - 1) is
// free by then.
constexpr int FPS_KB = 128, FPS_VTP = FPS_KB + 4;
constexpr int FPS_VT_CHUNKS = (80 * FPS_VTP * 2 / 16 + 63) / 64 * 64;  // 16-byte chunks per packed block

// vt[b][h][kb] (FPS_VT_CHUNKS chunks): row r, key j at element r * FPS_VTP + j
template <int DH>
__global__ void __launch_bounds__(256) vt_pack_kernel(FlashParams prm, uint4* vt, int nkb) {
  const int h = blockIdx.y, b = blockIdx.z, heads = gridDim.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nkb * FPS_VT_CHUNKS) return;
  const int kb = idx / FPS_VT_CHUNKS, c = idx % FPS_VT_CHUNKS;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(prm.V) + b * prm.v_bs + h * prm.v_hs;
  uint16_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int el = c * 8 + j, r = el / FPS_VTP, key = el % FPS_VTP;
    const int gk = kb * FPS_KB + key;
    uint16_t v = 0;
    if (r < DH && key < FPS_KB && gk < prm.Nk) v = Vb[(int64_t)gk * DH + r];
    else if (r == DH && key < FPS_KB) v = 0x3f80u;  // bf16 1.0
    e[j] = v;
  }
  vt[((int64_t)(b * heads + h) * nkb + kb) * FPS_VT_CHUNKS + c] =
      uint4{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
            e[6] | ((uint32_t)e[7] << 16)};
}

template <int DH>
__global__ void __launch_bounds__(FW_WAVES * 64, 1)
    flash_bf16_pps(FlashParams prm, const uint4* __restrict__ vtp_all, int q_per_wg, int nkb) {
  constexpr int FP_QT = PP_QT, FP_KB = FPS_KB;
  constexpr int FP_KT = FP_KB / 16, FP_QPW = 16 * FP_QT, FP_Q = FW_WAVES * FP_QPW;
  using P = BF16P<DH>;
  constexpr int NDT = P::NDT, DCH = P::DCH;
  static_assert(NDT * 16 == 80 && DH < 80, "packed V^T holds 80 rows with the ones row at DH");
  constexpr int KCH = FP_KB * DCH;             // K chunks per block (rows are contiguous: a linear copy)
  constexpr int BUFC = KCH + FPS_VT_CHUNKS;    // chunks per ring buffer
  constexpr int NDMA = BUFC / 64;              // DMA instructions per block
  static_assert(KCH % 64 == 0 && FPS_VT_CHUNKS % 64 == 0, "whole DMA instructions");
  constexpr int DMA_PER_WAVE = (NDMA + 3) / 4;  // issued by the four waves of group 0
  extern __shared__ uint4 fp_smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int h = blockIdx.y, b = blockIdx.z, heads = gridDim.y;
  const int g = lane >> 4, lr = lane & 15;
  const uint16_t* Qb = reinterpret_cast<const uint16_t*>(prm.Q) + b * prm.q_bs + h * prm.q_hs;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(prm.K) + b * prm.k_bs + h * prm.k_hs;
  const uint4* VTb = vtp_all + (int64_t)(b * heads + h) * nkb * FPS_VT_CHUNKS;
  const int qbeg = blockIdx.x * q_per_wg;
  const int qend = min(prm.Nq, qbeg + q_per_wg);
  const int Nk = prm.Nk;
  const int last_kchunk = Nk * DCH - 1;
  const int nq = (qend - qbeg + FP_Q - 1) / FP_Q;
  const int S = nq * nkb;  // steps: (query block, key block)

  // DMA of key block kb into ring buffer buf: instruction j < KCH/64 copies K
  // chunks (clamped to the last real key), the rest the packed V^T block
  auto dma = [&](int kb, int buf, int j) {
    uint4* dst = fp_smem + buf * BUFC + j * 64;
    if (j < KCH / 64) {
      const int ch = min(kb * KCH + j * 64 + lane, last_kchunk);
      PTDIT_GLDS16(reinterpret_cast<const char*>(Kb) + (size_t)ch * 16, dst);
    } else {
      PTDIT_GLDS16(VTb + (size_t)kb * FPS_VT_CHUNKS + (j - KCH / 64) * 64 + lane, dst);
    }
  };
  auto dma_block_all = [&](int kb, int buf) {  // all eight waves (prologue)
    for (int j = wave; j < NDMA; j += FW_WAVES) dma(kb, buf, j);
  };
  auto dma_block_g0 = [&](int kb, int buf) {  // group 0 only
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int j = wave + 4 * i;
      if (j < NDMA) dma(kb, buf, j);
    }
  };

  constexpr int NKF = DH / 32;
  static_assert(DH % 32 == 8, "head dim 32k + 8");
  struct QFr { uint4 v[NKF]; uint2 tail; };
  QFr qf[FP_QT];
  const uint32_t q_lane = (uint32_t)((lr * DH + 8 * g) * 2), q_tail = (uint32_t)((lr * DH + NKF * 32 + 4 * g) * 2);
  auto load_qf = [&](int qblk) {
    const int q0 = qblk + wave * FP_QPW;
    const char* base = reinterpret_cast<const char*>(Qb + (int64_t)q0 * DH);
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      const bool ok = q0 + t * 16 + lr < qend;
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc)
        qf[t].v[kc] = ok ? *reinterpret_cast<const uint4*>(base + q_lane + (t * 16 * DH + kc * 32) * 2)
                         : uint4{0, 0, 0, 0};
      qf[t].tail = ok && g < 2 ? *reinterpret_cast<const uint2*>(base + q_tail + t * 16 * DH * 2) : uint2{0, 0};
    }
  };

  // prologue: Q of the first query block, key blocks of steps 0 and 1
  load_qf(qbeg);
  dma_block_all(0, 0);
  if (S > 1) dma_block_all(1 % nkb, 1);
  wait_vm_lgkm0<0>();
  __syncthreads();

  const float c2 = prm.sl2;
  const bool tail_masked = Nk < nkb * FP_KB;

  floatx4 sc[FP_QT][FP_KT];
  uint32_t pk[FP_QT][FP_KT][2];
  floatx4 o[FP_QT][NDT];
  float m_run[FP_QT];

  auto scores = [&](int buf) {
    const uint4* ks = fp_smem + buf * BUFC;
    struct KFr { uint4 v[NKF]; uint2 tail; };
    KFr kf[2];
    auto load_kf = [&](int kt, KFr& f) {
      const int key = kt * 16 + lr;
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc) f.v[kc] = ks[key * DCH + kc * 4 + g];
      f.tail = g < 2 ? reinterpret_cast<const uint2*>(&ks[key * DCH + NKF * 4])[g] : uint2{0, 0};
    };
    load_kf(0, kf[0]);
#pragma unroll
    for (int kt = 0; kt < FP_KT; ++kt) {
      if (kt + 1 < FP_KT) load_kf(kt + 1, kf[(kt + 1) & 1]);
      const KFr& f = kf[kt & 1];
#pragma unroll
      for (int t = 0; t < FP_QT; ++t) sc[t][kt] = mfma_bf16_k16(f.tail, qf[t].tail, zero4());
#pragma unroll
      for (int kc = 0; kc < NKF; ++kc)
#pragma unroll
        for (int t = 0; t < FP_QT; ++t) sc[t][kt] = mfma_bf16(f.v[kc], qf[t].v[kc], sc[t][kt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv = [&](int buf) {
    const uint16_t* vt = reinterpret_cast<const uint16_t*>(fp_smem + buf * BUFC + KCH);
    uint4 vf[2][NDT];
    auto load_vf = [&](int u, uint4* f) {
      const uint16_t* base = vt + lr * FPS_VTP + u * 32 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t* row = base + dt * 16 * FPS_VTP;
        const uint2 lo = *reinterpret_cast<const uint2*>(row);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
        f[dt] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    };
    load_vf(0, vf[0]);
#pragma unroll
    for (int u = 0; u < FP_KT / 2; ++u) {
      if (u + 1 < FP_KT / 2) load_vf(u + 1, vf[(u + 1) & 1]);
#pragma unroll
      for (int t = 0; t < FP_QT; ++t) {
        const uint4 pf = uint4{pk[t][2 * u][0], pk[t][2 * u][1], pk[t][2 * u + 1][0], pk[t][2 * u + 1][1]};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[t][dt] = mfma_bf16(vf[u & 1][dt], pf, o[t][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax = [&](int kb) {
    if (kb == nkb - 1 && tail_masked) {
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool out = kb * FP_KB + kt * 16 + 4 * g + r >= Nk;
#pragma unroll
          for (int t = 0; t < FP_QT; ++t) sc[t][kt][r] = out ? -INFINITY : sc[t][kt][r];
        }
    }
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      float mx = sc[t][0][0];
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[t][kt][r]);
      mx = quad_max(mx);
      float m_new = mx;
      if (kb > 0) {
        m_new = fmaxf(m_run[t], mx);
        if (__builtin_amdgcn_ballot_w64(m_new > m_run[t]) != 0) {
          const float alpha = fast_exp2((m_run[t] - m_new) * c2);
#pragma unroll
          for (int i = 0; i < NDT; ++i) o[t][i] *= alpha;
        }
      }
      m_run[t] = m_new;
      const float nmc = -m_new * c2;
#pragma unroll
      for (int kt = 0; kt < FP_KT; ++kt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = fast_exp2(fmaf(sc[t][kt][r], c2, nmc));
        pk[t][kt][0] = pack_bf2(e[0], e[1]);
        pk[t][kt][1] = pack_bf2(e[2], e[3]);
      }
    }
  };
  auto zero_o = [&]() {
#pragma unroll
    for (int t = 0; t < FP_QT; ++t)
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[t][i] = zero4();
  };
  auto store_o = [&](int qblk) {
    constexpr int DT = DH / 16, GR = (DH % 16) / 4, EL = DH % 4;
    const int q0 = qblk + wave * FP_QPW;
    char* base = reinterpret_cast<char*>(reinterpret_cast<uint16_t*>(prm.O) + ((int64_t)b * prm.Nq + q0) * prm.D + h * DH);
    const uint32_t o_lane = (uint32_t)((lr * prm.D + 4 * g) * 2);
#pragma unroll
    for (int t = 0; t < FP_QT; ++t) {
      const float lsum = __shfl(o[t][DT][EL], GR * 16 + lr);
      if (q0 + t * 16 + lr < qend) {
        const float inv = 1.f / lsum;
        char* row = base + o_lane + (uint32_t)(t * 16 * prm.D * 2);
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          if (i * 16 + 4 * g < DH)
            store4(reinterpret_cast<uint16_t*>(row + i * 32), o[t][i][0] * inv, o[t][i][1] * inv, o[t][i][2] * inv,
                   o[t][i][3] * inv);
        }
      }
    }
  };
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // group 1 runs one phase behind group 0
  if (grp == 1) phase_end();
  scores(0);
  phase_end();
  for (int s = 0; s < S; ++s) {
    const int qi = s / nkb, kb = s - qi * nkb;
    const int qblk = qbeg + qi * FP_Q;
    const bool more = qi + 1 < nq;
    // VALU phase: (next query block's Q, whose last scores are done,) softmax
    // of step s; the DMA issued in the last MFMA phase (step s + 1's block)
    // and the Q loads land before the barrier
    if (kb == nkb - 1 && more) load_qf(qblk + FP_Q);
    softmax(kb);
    if (kb == 0) zero_o();
    wait_vm_lgkm0<0>();
    phase_end();
    // MFMA phase: P V of step s (then the finished block's output), the
    // scores of step s + 1, then (group 0) the DMA of step s + 2
    pv(s % 3);
    if (kb == nkb - 1) store_o(qblk);
    if (s + 1 < S) scores((s + 1) % 3);
    if (grp == 0 && s + 2 < S) {
      __builtin_amdgcn_sched_barrier(0);
      dma_block_g0((s + 2) % nkb, (s + 2) % 3);
    }
    phase_end();
  }
  if (grp == 0) phase_end();
}

// ---------------------------------------------------------------- window core
struct WindowParams {
  const void* QKV;       // [B][3][heads][N][dh]
  const void* bias_qkv;  // [3D] or null
  void* O;               // [B][N][D]
  int F, H, W, D, heads;
  int wt, wh, ww;
  int st, sh, sw;
  int Fp, Hp, Wp;
  float sl2;
};

__device__ __forceinline__ int region(int k, int L, int w, int s) {
  return k < L - w ? 0 : (k < L - s ? 1 : 2);
}

// Workgroup = one (window, head, batch); NTILE waves of 16 query slots each;
// every key of the window is resident in LDS, so the softmax is one pass.
template <class P, int DH, int NTILE>
__global__ void __launch_bounds__(NTILE * 64) window_kernel(WindowParams prm) {
  using T = typename P::T;
  constexpr int NT = NTILE * 64;
  constexpr int NTILE2 = (NTILE + P::TPV - 1) / P::TPV * P::TPV;
  constexpr int KEYS = NTILE2 * 16;
  __shared__ typename P::template Smem<KEYS> sm;
  __shared__ int tok_s[KEYS];
  __shared__ __attribute__((aligned(16))) int lab_s[KEYS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int nWh = prm.Hp / prm.wh, nWw = prm.Wp / prm.ww;
  const int Tw = blockIdx.x / (nWh * nWw), Iw = (blockIdx.x / nWw) % nWh, Jw = blockIdx.x % nWw;
  const int wsz = prm.wt * prm.wh * prm.ww;
  const int64_t N = (int64_t)prm.F * prm.H * prm.W;

  for (int s = tid; s < KEYS; s += NT) {
    int tok = -2, lab = -1;
    if (s < wsz) {
      const int a = s / (prm.wh * prm.ww), c = (s / prm.ww) % prm.wh, e = s % prm.ww;
      const int rt = Tw * prm.wt + a, ri = Iw * prm.wh + c, rj = Jw * prm.ww + e;
      int ot = rt + prm.st; ot -= ot >= prm.Fp ? prm.Fp : 0;
      int oi = ri + prm.sh; oi -= oi >= prm.Hp ? prm.Hp : 0;
      int oj = rj + prm.sw; oj -= oj >= prm.Wp ? prm.Wp : 0;
      tok = (ot < prm.F && oi < prm.H && oj < prm.W) ? (ot * prm.H + oi) * prm.W + oj : -1;
      lab = region(rt, prm.Fp, prm.wt, prm.st) * 9 + region(ri, prm.Hp, prm.wh, prm.sh) * 3 +
            region(rj, prm.Wp, prm.ww, prm.sw);
    }
    tok_s[s] = tok;
    lab_s[s] = lab;
  }
  P::zero_pad(sm, tid, NT);
  __syncthreads();

  const T* base = reinterpret_cast<const T*>(prm.QKV);
  const int64_t hs = N * DH, gs = (int64_t)prm.heads * hs;
  const T* Qb = base + (int64_t)b * 3 * gs + h * hs;
  const T* Kb = Qb + gs;
  const T* Vb = Qb + 2 * gs;
  const T* bias = reinterpret_cast<const T*>(prm.bias_qkv);
  const T* bk = bias ? bias + prm.D + h * DH : nullptr;
  const T* bv = bias ? bias + 2 * prm.D + h * DH : nullptr;

  // Every global load of the window (K, V, this lane's query) is issued
  // before the first LDS write, so the thread waits for one latency.
  const int qs = wave * 16 + (lane & 15);
  const int qtok = tok_s[qs], qlab = lab_s[qs];
  if constexpr (P::TPV == 2) {
    // bf16: K chunk by chunk, V four slots at a time (transposed in registers)
    constexpr int KI = (KEYS * P::DCH + NT - 1) / NT, VI = (P::DCH * (KEYS / 4) + NT - 1) / NT;
    uint4 kreg[KI], vreg[VI][4];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = tid + i * NT;
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      const int tok = idx < KEYS * P::DCH ? tok_s[s] : -2;
      const T* kr = tok >= 0 ? Kb + (int64_t)tok * DH : (tok == -1 ? bk : nullptr);
      kreg[i] = kr ? *reinterpret_cast<const uint4*>(kr + c * 8) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int idx = tid + i * NT;
      const int c = idx / (KEYS / 4), kq = idx - c * (KEYS / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = idx < P::DCH * (KEYS / 4) ? tok_s[kq * 4 + e] : -2;
        const T* vr = tok >= 0 ? Vb + (int64_t)tok * DH : (tok == -1 ? bv : nullptr);
        vreg[i][e] = vr ? *reinterpret_cast<const uint4*>(vr + c * 8) : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = tid + i * NT;
      if (idx < KEYS * P::DCH) sm.k[idx] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int idx = tid + i * NT;
      const int c = idx / (KEYS / 4), kq = idx - c * (KEYS / 4);
      if (idx < P::DCH * (KEYS / 4)) P::put_vquad(sm, kq, c, vreg[i]);
    }
  } else {
    constexpr int ITEMS = KEYS * P::DCH, PER = (ITEMS + NT - 1) / NT;
    typename P::Raw raw[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      const int tok = idx < ITEMS ? tok_s[s] : -2;
      const T* kr = tok >= 0 ? Kb + (int64_t)tok * DH : (tok == -1 ? bk : nullptr);
      const T* vr = tok >= 0 ? Vb + (int64_t)tok * DH : (tok == -1 ? bv : nullptr);
      raw[i] = P::load(c, kr, vr);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      if (idx < ITEMS) P::put(sm, s, c, raw[i]);
    }
  }
  const auto qf = P::load_q(qtok >= 0 ? Qb + (int64_t)qtok * DH : nullptr, lane);
  __syncthreads();
  floatx4 sc[NTILE2];
#pragma unroll
  for (int t = 0; t < NTILE2; ++t) sc[t] = P::score(sm, qf, t, lane);
  // key slots of this lane: t*16 + 4*(lane/16) + r. Labels are read four at a
  // time; without a shift every real slot of a window shares one label, so
  // only the slots past the window need masking.
  const bool masked = (prm.st | prm.sh | prm.sw) != 0;
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NTILE2; ++t) {
    const int ks0 = t * 16 + 4 * (lane >> 4);
    const int4 lab4 = *reinterpret_cast<const int4*>(&lab_s[ks0]);
    const int labs[4] = {lab4.x, lab4.y, lab4.z, lab4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = ks0 + r < wsz && (!masked || labs[r] == qlab);
      const float v = ok ? sc[t][r] * prm.sl2 : -INFINITY;
      sc[t][r] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = quad_max(mx);
  if (mx == -INFINITY) mx = 0.f;  // slot past the window: keeps the idle column finite
  float rs = 0.f;
#pragma unroll
  for (int t = 0; t < NTILE2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(sc[t][r] - mx);
      sc[t][r] = e;
      rs += e;
    }
  rs = quad_sum(rs);
  floatx4 o[P::NDT];
#pragma unroll
  for (int i = 0; i < P::NDT; ++i) o[i] = zero4();
#pragma unroll
  for (int t0 = 0; t0 < NTILE2; t0 += P::TPV) P::pv(sm, o, &sc[t0], t0, lane);

  if (qtok >= 0) {
    const float inv = 1.f / rs;
    T* Ob = reinterpret_cast<T*>(prm.O) + ((int64_t)b * N + qtok) * prm.D + h * DH;
#pragma unroll
    for (int i = 0; i < P::NDT; ++i) {
      const int d = i * 16 + 4 * (lane >> 4);
      if (d < DH) P::store_o(Ob + d, o[i][0] * inv, o[i][1] * inv, o[i][2] * inv, o[i][3] * inv);
    }
  }
}

// ---------------------------------------------------------------- dispatch
template <class P, int DH>
static hipError_t run_flash(const FlashDesc& d, hipStream_t s) {
  FlashParams p;
  p.Q = d.Q; p.q_bs = d.q_bs; p.q_hs = d.q_hs;
  p.K = d.K; p.k_bs = d.k_bs; p.k_hs = d.k_hs;
  p.V = d.V; p.v_bs = d.v_bs; p.v_hs = d.v_hs;
  p.O = d.O; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.sl2 = d.scale * LOG2E;
  dim3 grid((d.Nq + 63) / 64, d.heads, d.B);
  // bf16 with at most 256 keys: one key block, staged once (one load latency
  // instead of one per 64 keys); fp32 blocks would not fit in LDS
  if constexpr (sizeof(typename P::T) == 2) {
    if (d.Nk > 128 && d.Nk <= 256) {
      hipLaunchKernelGGL((flash_kernel<P, DH, 256>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
    if (d.Nk > 64 && d.Nk <= 128) {
      hipLaunchKernelGGL((flash_kernel<P, DH, 128>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((flash_kernel<P, DH, 64>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DH>
static hipError_t run_flash_wide(const FlashDesc& d, hipStream_t s) {
  FlashParams p;
  p.Q = d.Q; p.q_bs = d.q_bs; p.q_hs = d.q_hs;
  p.K = d.K; p.k_bs = d.k_bs; p.k_hs = d.k_hs;
  p.V = d.V; p.v_bs = d.v_bs; p.v_hs = d.v_hs;
  p.O = d.O; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.sl2 = d.scale * LOG2E;
  dim3 grid((d.Nq + FW_Q - 1) / FW_Q, d.heads, d.B);
  hipLaunchKernelGGL((flash_bf16_wide<DH>), grid, dim3(FW_WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <int DH>
static hipError_t run_flash_single(const FlashDesc& d, hipStream_t s) {
  FlashParams p;
  p.Q = d.Q; p.q_bs = d.q_bs; p.q_hs = d.q_hs;
  p.K = d.K; p.k_bs = d.k_bs; p.k_hs = d.k_hs;
  p.V = d.V; p.v_bs = d.v_bs; p.v_hs = d.v_hs;
  p.O = d.O; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.sl2 = d.scale * LOG2E;
  // about one workgroup per CU: split each (batch, head) query range so that
  // B * heads * ranges ~ 256, ranges in whole 256-query blocks
  const int pairs = d.B * d.heads;
  int ranges = (256 + pairs - 1) / pairs;
  const int qblocks = (d.Nq + FW_Q - 1) / FW_Q;
  if (ranges > qblocks) ranges = qblocks;
  if (ranges < 1) ranges = 1;
  const int q_per_wg = (qblocks + ranges - 1) / ranges * FW_Q;
  dim3 grid((d.Nq + q_per_wg - 1) / q_per_wg, d.heads, d.B);
  hipLaunchKernelGGL((flash_bf16_single<DH>), grid, dim3(FW_WAVES * 64), 0, s, p, q_per_wg);
  return hipGetLastError();
}

template <int DH, int QT, int KB>
static hipError_t run_flash_pp(const FlashDesc& d, hipStream_t s) {
  constexpr int FP_Q = FW_WAVES * 16 * QT;
  FlashParams p;
  p.Q = d.Q; p.q_bs = d.q_bs; p.q_hs = d.q_hs;
  p.K = d.K; p.k_bs = d.k_bs; p.k_hs = d.k_hs;
  p.V = d.V; p.v_bs = d.v_bs; p.v_hs = d.v_hs;
  p.O = d.O; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.sl2 = d.scale * LOG2E;
  // about one workgroup per CU (the LDS holds every key of one head)
  const int pairs = d.B * d.heads;
  int ranges = (256 + pairs - 1) / pairs;
  const int qblocks = (d.Nq + FP_Q - 1) / FP_Q;
  if (ranges > qblocks) ranges = qblocks;
  if (ranges < 1) ranges = 1;
  const int q_per_wg = (qblocks + ranges - 1) / ranges * FP_Q;
  dim3 grid((d.Nq + q_per_wg - 1) / q_per_wg, d.heads, d.B);
  const int nkb = (d.Nk + KB - 1) / KB;
  const int lds = flash_pp_lds_bytes<DH>(nkb * KB);
  constexpr int max_lds = flash_pp_lds_bytes<DH>((FP_MAXK + KB - 1) / KB * KB);
  static_assert(max_lds <= 160 * 1024, "LDS");
  static bool attr_set = false;  // same value from every thread: a benign race
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_bf16_pp<DH, QT, KB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((flash_bf16_pp<DH, QT, KB>), grid, dim3(FW_WAVES * 64), lds, s, p, q_per_wg, nkb);
  return hipGetLastError();
}

template <int DH>
static hipError_t run_flash_pps(const FlashDesc& d, hipStream_t s) {
  constexpr int FP_Q = FW_WAVES * 16 * PP_QT;
  FlashParams p;
  p.Q = d.Q; p.q_bs = d.q_bs; p.q_hs = d.q_hs;
  p.K = d.K; p.k_bs = d.k_bs; p.k_hs = d.k_hs;
  p.V = d.V; p.v_bs = d.v_bs; p.v_hs = d.v_hs;
  p.O = d.O; p.Nq = d.Nq; p.Nk = d.Nk; p.D = d.D;
  p.sl2 = d.scale * LOG2E;
  const int nkb = (d.Nk + FPS_KB - 1) / FPS_KB;
  if (!d.vt || d.vt_bytes < flash_vt_bytes(d.B, d.heads, d.Nk)) return hipErrorInvalidValue;
  uint4* vt = reinterpret_cast<uint4*>(d.vt);
  hipLaunchKernelGGL((vt_pack_kernel<DH>), dim3((nkb * FPS_VT_CHUNKS + 255) / 256, d.heads, d.B), dim3(256), 0, s, p,
                     vt, nkb);
  const int pairs = d.B * d.heads;
  int ranges = (256 + pairs - 1) / pairs;
  const int qblocks = (d.Nq + FP_Q - 1) / FP_Q;
  if (ranges > qblocks) ranges = qblocks;
  if (ranges < 1) ranges = 1;
  const int q_per_wg = (qblocks + ranges - 1) / ranges * FP_Q;
  dim3 grid((d.Nq + q_per_wg - 1) / q_per_wg, d.heads, d.B);
  constexpr int lds = 3 * (FPS_KB * DH / 8 + FPS_VT_CHUNKS) * 16;
  static_assert(lds <= 160 * 1024, "LDS");
  static bool attr_set = false;  // same value from every thread: a benign race
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_bf16_pps<DH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((flash_bf16_pps<DH>), grid, dim3(FW_WAVES * 64), lds, s, p, vt, q_per_wg, nkb);
  return hipGetLastError();
}

size_t flash_vt_bytes(int B, int heads, int Nk) {
  if (Nk <= FP_MAXK) return 0;
  return (size_t)B * heads * ((Nk + FPS_KB - 1) / FPS_KB) * FPS_VT_CHUNKS * 16;
}

hipError_t launch_flash(const FlashDesc& d, int f32, hipStream_t s) {
  if (d.Nq == 0 || d.B == 0) return hipSuccess;
  if (!f32 && d.Nq >= 2048 && d.Nk > FS_MAXK && d.Nk <= FP_MAXK) {
    if (d.dh == 72) return run_flash_pp<72, PP_QT, PP_KB>(d, s);
  }
  if (!f32 && d.Nq >= 2048 && d.Nk <= FS_MAXK) {
    if (d.dh == 72) return run_flash_single<72>(d, s);
    if (d.dh == 64) return run_flash_single<64>(d, s);
  }
  // more keys: streamed through LDS (needs the packed V^T scratch)
  if (!f32 && d.Nq >= 2048 && d.dh == 72 && d.vt) return run_flash_pps<72>(d, s);
  if (!f32 && d.Nq >= 2048) {
    if (d.dh == 72) return run_flash_wide<72>(d, s);
    if (d.dh == 64) return run_flash_wide<64>(d, s);
  }
  if (d.dh == 72) return f32 ? run_flash<F32P<72>, 72>(d, s) : run_flash<BF16P<72>, 72>(d, s);
  if (d.dh == 64) return f32 ? run_flash<F32P<64>, 64>(d, s) : run_flash<BF16P<64>, 64>(d, s);
  return hipErrorInvalidValue;
}

template <class P, int DH, int NTILE>
static hipError_t run_window(const WindowDesc& d, hipStream_t s) {
  WindowParams p;
  p.QKV = d.QKV; p.bias_qkv = d.bias_qkv; p.O = d.O;
  p.F = d.F; p.H = d.H; p.W = d.W; p.D = d.D; p.heads = d.heads;
  p.wt = d.wt; p.wh = d.wh; p.ww = d.ww;
  p.st = d.st; p.sh = d.sh; p.sw = d.sw;
  p.Fp = d.Fp; p.Hp = d.Hp; p.Wp = d.Wp;
  p.sl2 = d.scale * LOG2E;
  const int nwin = (d.Fp / d.wt) * (d.Hp / d.wh) * (d.Wp / d.ww);
  dim3 grid(nwin, d.heads, d.B);
  hipLaunchKernelGGL((window_kernel<P, DH, NTILE>), grid, dim3(NTILE * 64), 0, s, p);
  return hipGetLastError();
}

template <class P, int DH>
static hipError_t pick_window(const WindowDesc& d, hipStream_t s) {
  const int wsz = d.wt * d.wh * d.ww;
  if (wsz <= 64) return run_window<P, DH, 4>(d, s);
  if (wsz <= 128) return run_window<P, DH, 8>(d, s);
  return hipErrorInvalidValue;
}

hipError_t launch_window(const WindowDesc& d, int f32, hipStream_t s) {
  if (d.B == 0) return hipSuccess;
  if (d.dh == 72) return f32 ? pick_window<F32P<72>, 72>(d, s) : pick_window<BF16P<72>, 72>(d, s);
  if (d.dh == 64) return f32 ? pick_window<F32P<64>, 64>(d, s) : pick_window<BF16P<64>, 64>(d, s);
  return hipErrorInvalidValue;
}

}  // namespace ptdit
