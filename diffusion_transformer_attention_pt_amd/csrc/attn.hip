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

  // Stage chunk c (8 channels) of key slot s; NULL rows stage zeros.
  template <int KEYS>
  __device__ static void stage(Smem<KEYS>& sm, int s, int c, const T* krow, const T* vrow) {
    const uint4 kv = krow ? *reinterpret_cast<const uint4*>(krow + c * 8) : uint4{0, 0, 0, 0};
    const uint4 vv = vrow ? *reinterpret_cast<const uint4*>(vrow + c * 8) : uint4{0, 0, 0, 0};
    sm.k[s * DCH + c] = kv;
    sm.vt[c * 8 + 0][s] = (uint16_t)(vv.x & 0xffff); sm.vt[c * 8 + 1][s] = (uint16_t)(vv.x >> 16);
    sm.vt[c * 8 + 2][s] = (uint16_t)(vv.y & 0xffff); sm.vt[c * 8 + 3][s] = (uint16_t)(vv.y >> 16);
    sm.vt[c * 8 + 4][s] = (uint16_t)(vv.z & 0xffff); sm.vt[c * 8 + 5][s] = (uint16_t)(vv.z >> 16);
    sm.vt[c * 8 + 6][s] = (uint16_t)(vv.w & 0xffff); sm.vt[c * 8 + 7][s] = (uint16_t)(vv.w >> 16);
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

  template <int KEYS>
  __device__ static void stage(Smem<KEYS>& sm, int s, int c, const T* krow, const T* vrow) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.k[s][c * 8 + e] = krow ? krow[c * 8 + e] : 0.f;
      sm.v[s][c * 8 + e] = vrow ? vrow[c * 8 + e] : 0.f;
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
    __syncthreads();
    for (int idx = tid; idx < KB * P::DCH; idx += NT) {
      const int s = idx / P::DCH, c = idx - s * P::DCH;
      const int gk = k0 + s;
      const bool ok = gk < prm.Nk;
      P::stage(sm, s, c, ok ? Kb + (int64_t)gk * DH : nullptr, ok ? Vb + (int64_t)gk * DH : nullptr);
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
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = exp2f(sc[t][r] - m_new);
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
  __shared__ int lab_s[KEYS];

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

  for (int idx = tid; idx < KEYS * P::DCH; idx += NT) {
    const int s = idx / P::DCH, c = idx - s * P::DCH;
    const int tok = tok_s[s];
    const T* kr = tok >= 0 ? Kb + (int64_t)tok * DH : (tok == -1 ? bk : nullptr);
    const T* vr = tok >= 0 ? Vb + (int64_t)tok * DH : (tok == -1 ? bv : nullptr);
    P::stage(sm, s, c, kr, vr);
  }
  __syncthreads();

  const int qs = wave * 16 + (lane & 15);
  const int qtok = tok_s[qs], qlab = lab_s[qs];
  const auto qf = P::load_q(qtok >= 0 ? Qb + (int64_t)qtok * DH : nullptr, lane);
  floatx4 sc[NTILE2];
#pragma unroll
  for (int t = 0; t < NTILE2; ++t) sc[t] = P::score(sm, qf, t, lane);
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NTILE2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ks = t * 16 + 4 * (lane >> 4) + r;
      const float v = lab_s[ks] == qlab && ks < wsz ? sc[t][r] * prm.sl2 : -INFINITY;
      sc[t][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = quad_max(mx);
  if (mx == -INFINITY) mx = 0.f;  // slot past the window: keeps the idle column finite
  float rs = 0.f;
#pragma unroll
  for (int t = 0; t < NTILE2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = exp2f(sc[t][r] - mx);
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
  hipLaunchKernelGGL((flash_kernel<P, DH, 64>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_flash(const FlashDesc& d, int f32, hipStream_t s) {
  if (d.Nq == 0 || d.B == 0) return hipSuccess;
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
