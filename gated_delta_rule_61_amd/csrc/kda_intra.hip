// KDA (per-channel gate) intra-chunk kernel, gfx950.  Per (chunk, v-head),
// with G[t][c] the chunk-local cumulative log-gate of key channel c:
//
//   Aqk[t][s] = scale * sum_c q[t][c] k[s][c] exp(G[t][c] - G[s][c])   s <= t
//   A  [t][s] = beta_t * sum_c k[t][c] k[s][c] exp(G[t][c] - G[s][c])  s <  t
//   Akk_inv   = (I + A)^-1
//
// and the gated operands of the chunk scan:
//   QG = Q o e^G,  KG = K o e^G,  KT = K o e^{G_last - G},  DG = e^{G_last}.
//
// What is computed follows "vLLM kimi_k3 amd ops kda/chunk_intra"
// (chunk_kda_fwd_kernel_inter_solve_fused: off-diagonal Aqk / Akk blocks of
// the four 16-token sub-chunks with a reference row per block, Aqk scaled by
// `scale`, Akk rows scaled by beta, forward substitution on the diagonal
// blocks and the block merge giving Akk_inv, stored row per token as
// [B, T, HV, 64]) and "fla ops/common/chunk_h.py" (USE_GK: per-channel decay
// of the state and k scaled by exp(gk_last - gk)).
//
// gfx950 design: 4 waves per work-group, wave w owns 16-token block w.
//   * the per-channel cumsum runs over LDS (each wave scans 16 tokens, then
//     adds the totals of the blocks before it);
//   * block pair (i, j), j <= i, is one fp16 MFMA product over the key
//     channels with every factor bounded:
//       row operand  x[t] o exp(G[t] - G[n_i]) o exp(G[n_i] - G[m_j])
//       col operand  k[s] o exp(G[m_j] - G[s])
//     (n_i first row of block i, m_j last row of block j).  For j < i every
//     exponent is <= 0.  The diagonal pair (j = i) carries exp(G[n_i] -
//     G[m_i]) >= 1, the decay inside one 16-token block; when that exceeds
//     10 nats (or an operand leaves the fp16 range) the wave recomputes its
//     diagonal block exactly, pair by pair, in fp32;
//   * beta / scale / causal masks on the fp32 accumulators; the 64 x 64
//     solve is the same forward substitution + block merge as the GDN
//     kernel;
//   * every global load a wave needs (its 16 gate rows, its q / k row, beta)
//     is issued at entry, so the memory latency is paid once;
//   * Aqk is staged in LDS (in the cumsum tile, free by then) and, like
//     Akk_inv, leaves in 16-byte row pieces, one tile per wave;
//   * the pairs' decay factors exp(G[n_i] - G[m_j]) are one LDS table built
//     by all threads (they do not depend on the row), and the bounded
//     operands convert to fp16 without clamping.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

using namespace intra;

constexpr float DIAG_MAX_DECAY = 10.0f;      // nats of decay inside a 16-token block
constexpr float DIAG_MAX_OPERAND = 30000.0f;  // largest fp16 operand the fast path accepts

// 16-bit (or fp32) conversions without clamping, for operands bounded by
// |q|, |k| (every exponent here is <= 0, except the diagonal pair's, whose
// operands the exact path takes over beyond DIAG_MAX_OPERAND)
template <typename P> __device__ __forceinline__ P to_bounded(float x) { return from_f<P>(x); }
template <> __device__ __forceinline__ f16_t to_bounded<f16_t>(float x) { return (_Float16)x; }
template <typename P> __device__ __forceinline__ uint32_t pack2_bounded(float lo, float hi) {
  return pack2<P>(lo, hi);
}
template <> __device__ __forceinline__ uint32_t pack2_bounded<f16_t>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
template <typename P> __device__ __forceinline__ void set_bounded(Frag<P>& f, int e, float x) { f.set(e, x); }
template <> __device__ __forceinline__ void set_bounded<f16_t>(Frag<f16_t>& f, int e, float x) {
  f.v[e] = (_Float16)x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

template <typename T, int DK, typename P = typename ComputeOf<T>::type>
__global__ __launch_bounds__(256) void kda_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ gk,
    const float* __restrict__ beta, float scale, T* __restrict__ Aqk_out,
    T* __restrict__ Akk_out, P* __restrict__ Ainv_ws, P* __restrict__ Aqk_ws,
    P* __restrict__ qg, P* __restrict__ kg, P* __restrict__ kt, float* __restrict__ GF,
    float* __restrict__ DG, const int64_t* __restrict__ cu, const int32_t* __restrict__ coff,
    int Tlen, int ttot, int N, int NT, int nslots, int Hk, int HV) {
  constexpr int KS = DK / 32;   // 32-channel slabs
  constexpr int CPL = DK / 64;  // channels per lane in the cumsum
  constexpr int GP = DK + 4;    // padded fp32 row of the cumsum tile
  constexpr int CP = DK + 8;    // padded row of the column-operand tile
  __shared__ __attribute__((aligned(16))) float sG[BT][GP];
  __shared__ __attribute__((aligned(16))) P sC[BT][CP];
  __shared__ __attribute__((aligned(16))) float sA[BT][AP];
  // exp(G[n_i] - G[m_j]) of block pair (i, j), j <= i, per channel
  __shared__ __attribute__((aligned(16))) float sE[10][DK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, grp = lane >> 4;
  int slot, hv, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, hv)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int hk = hv / (HV / Hk);

  // ---- every global load the wave needs before its math, issued up front
  // (addresses of rows past nrow are clamped to the last row, the values
  // masked where used): the wave's 16 gate rows, its operand row of q and
  // k, and beta of its rows
  const int cl = lane * CPL;
  float gx[16][CPL];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int tok = 16 * w + u < nrow ? 16 * w + u : nrow - 1;
    const float* gp = gk + ((size_t)(c0 + tok) * HV + hv) * DK + cl;
    if constexpr (CPL == 2) {
      const float2 v2 = *reinterpret_cast<const float2*>(gp);
      gx[u][0] = v2.x;
      gx[u][1] = v2.y;
    } else {
      gx[u][0] = gp[0];
    }
  }
  const int t = 16 * w + row;  // token (within the chunk) of this lane's operand row
  const bool tv = t < nrow;
  const int tc = tv ? t : nrow - 1;
  Frag<T> fq[KS], fk[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    load8(fq[s], q + ((size_t)(c0 + tc) * Hk + hk) * DK + 32 * s + 8 * grp);
    load8(fk[s], k + ((size_t)(c0 + tc) * Hk + hk) * DK + 32 * s + 8 * grp);
  }
  float braw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * grp + i < nrow ? 16 * w + 4 * grp + i : nrow - 1;
    braw[i] = beta[(size_t)(c0 + r) * HV + hv];
  }
  const float bt = beta[(size_t)(c0 + tc) * HV + hv];

  // ---- cumulative gate over the chunk, per channel (rows past nrow add 0)
  {
    float acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tok = 16 * w + u;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        acc[e] += tok < nrow ? gx[u][e] : 0.f;
        sG[tok][cl + e] = acc[e];
      }
    }
    __syncthreads();
    float off[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      off[e] = 0.f;
      for (int w2 = 0; w2 < w; ++w2) off[e] += sG[16 * w2 + 15][cl + e];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int e = 0; e < CPL; ++e) sG[16 * w + u][cl + e] += off[e];
    __syncthreads();
  }

  // ---- the block pairs' decay factors (the same for the 16 rows of a
  // block, so computed once here rather than in every lane)
  for (int idx = tid; idx < 10 * DK; idx += 256) {
    const int pr = idx / DK, c = idx - pr * DK;
    const int i = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
    const int jj = pr - tix(i, 0);
    sE[pr][c] = __expf(sG[16 * i][c] - sG[16 * jj + 15][c]);
  }

  // ---- gated operands of this wave's block; row operands kept in registers
  float qa[KS][8], ka[KS][8];  // q, k scaled by exp(G[t] - G[n_w])
  float dmax = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int cb = 32 * s + 8 * grp;
    float qv[8], kv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] = tv ? fq[s].get(e) : 0.f;
      kv[e] = tv ? fk[s].get(e) : 0.f;
    }
    float vq[8], vk[8], vt[8], vc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cb + e;
      const float g = sG[t][c], gn = sG[16 * w][c], gm = sG[16 * w + 15][c], gl = sG[BT - 1][c];
      const float eg = __expf(g);
      const float a = __expf(g - gn);
      qa[s][e] = qv[e] * a;
      ka[s][e] = kv[e] * a;
      vq[e] = qv[e] * eg;
      vk[e] = kv[e] * eg;
      vt[e] = kv[e] * __expf(gl - g);
      vc[e] = kv[e] * __expf(gm - g);
      dmax = fmaxf(dmax, gn - gm);
    }
    if (tv) {
      const size_t oo = ((size_t)(c0 + t) * HV + hv) * DK + cb;
      if constexpr (sizeof(P) == 2) {
        *reinterpret_cast<uint4*>(qg + oo) =
            make_uint4(pack2_bounded<P>(vq[0], vq[1]), pack2_bounded<P>(vq[2], vq[3]),
                       pack2_bounded<P>(vq[4], vq[5]), pack2_bounded<P>(vq[6], vq[7]));
        *reinterpret_cast<uint4*>(kg + oo) =
            make_uint4(pack2_bounded<P>(vk[0], vk[1]), pack2_bounded<P>(vk[2], vk[3]),
                       pack2_bounded<P>(vk[4], vk[5]), pack2_bounded<P>(vk[6], vk[7]));
        *reinterpret_cast<uint4*>(kt + oo) =
            make_uint4(pack2_bounded<P>(vt[0], vt[1]), pack2_bounded<P>(vt[2], vt[3]),
                       pack2_bounded<P>(vt[4], vt[5]), pack2_bounded<P>(vt[6], vt[7]));
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          *reinterpret_cast<float4*>(qg + oo + e) = make_float4(vq[e], vq[e + 1], vq[e + 2], vq[e + 3]);
          *reinterpret_cast<float4*>(kg + oo + e) = make_float4(vk[e], vk[e + 1], vk[e + 2], vk[e + 3]);
          *reinterpret_cast<float4*>(kt + oo + e) = make_float4(vt[e], vt[e + 1], vt[e + 2], vt[e + 3]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sC[t][cb + e] = to_bounded<P>(vc[e]);
  }
  const float Dw = wave_max(dmax);
  __syncthreads();

  // ---- block pairs (w, j), j <= w: fp16 (fp32 for fp32 io) MFMA
  f32x4 QK[4], KK[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) { QK[jb] = zero4(); KK[jb] = zero4(); }
  float opmax = 0.f;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    if (jb > w) continue;  // uniform per wave
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int cb = 32 * s + 8 * grp;
      Frag<P> fa, fb, fc;
      const float4 sv0 = *reinterpret_cast<const float4*>(&sE[tix(w, jb)][cb]);
      const float4 sv1 = *reinterpret_cast<const float4*>(&sE[tix(w, jb)][cb + 4]);
      const float sv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xq = qa[s][e] * sv[e], xk = ka[s][e] * sv[e];
        if (jb == w) opmax = fmaxf(opmax, fmaxf(fabsf(xq), fabsf(xk)));
        set_bounded<P>(fa, e, xq);
        set_bounded<P>(fb, e, xk);
      }
      load8(fc, &sC[16 * jb + row][cb]);
      QK[jb] = mma(fa, fc, QK[jb]);
      KK[jb] = mma(fb, fc, KK[jb]);
    }
  }
  const bool slow = !(Dw <= DIAG_MAX_DECAY) || !(wave_max(opmax) <= DIAG_MAX_OPERAND);
  if (slow) {
    // exact diagonal block: every pair (r, s), s <= r, in fp32
    const int sc = 16 * w + row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * grp + i;
      float aq = 0.f, ak = 0.f;
      if (sc <= r && r < nrow) {
        const T* qr = q + ((size_t)(c0 + r) * Hk + hk) * DK;
        const T* kr = k + ((size_t)(c0 + r) * Hk + hk) * DK;
        const T* ks = k + ((size_t)(c0 + sc) * Hk + hk) * DK;
        for (int c = 0; c < DK; ++c) {
          const float f = expf(sG[r][c] - sG[sc][c]);
          const float kv = to_f(ks[c]) * f;
          aq = fmaf(to_f(qr[c]), kv, aq);
          ak = fmaf(to_f(kr[c]), kv, ak);
        }
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        if (jb == w) {
          QK[jb][i] = aq;
          KK[jb][i] = ak;
        }
    }
  }

  // ---- scale / beta / masks; Aqk and A to LDS (upper blocks zero).  Aqk
  // (fp32) is staged in the cumsum tile, which nothing reads after this
  // barrier (wave 0 keeps the last row for the decay first).
  float dgv[CPL];
  if (w == 0) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) dgv[e] = sG[BT - 1][lane * CPL + e];
  }
  __syncthreads();
  float (*sQ)[AP] = reinterpret_cast<float (*)[AP]>(&sG[0][0]);
  static_assert(sizeof(sG) >= sizeof(float) * BT * AP, "Aqk staging tile");
  float br[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * grp + i;
    br[i] = r < nrow ? braw[i] : 0.f;
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * grp + i, sc = 16 * jb + row;
      const bool in = jb <= w;
      const float aqk = (in && sc <= r) ? scale * QK[jb][i] : 0.f;
      const float akk = (in && sc < r) ? br[i] * KK[jb][i] : 0.f;
      sA[r][sc] = akk;
      sQ[r][sc] = aqk;
    }
  if (grp == 0 && tv) {
    const size_t gs = (size_t)gf_stride(ttot);
    float* gp = GF + (size_t)hv * 4 * gs + c0 + t;
    gp[0] = 1.f;
    gp[gs] = 1.f;
    gp[2 * gs] = bt;
    gp[3 * gs] = 1.f;
  }
  if (w == 0) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = lane * CPL + e;
      DG[((size_t)slot * HV + hv) * DK + c] = __expf(dgv[e]);
    }
  }
  __syncthreads();

  // ---- the tiles to memory in 16-byte row pieces: the Aqk tiles first (waves
  // 2, 3, while wave 0 runs the substitution), then (I + A)^-1 (substitution
  // on wave 0, the merge's three column blocks on waves 0 - 2), half a tile
  // per wave
  if (w == 2) store_tile<P>(sQ, Aqk_ws, c0, nrow, HV, hv, lane);
  if (w == 3 && Aqk_out) store_tile<T>(sQ, Aqk_out, c0, nrow, HV, hv, lane);
  solve_unit_lower_64<4>(sA, lane, w);
  if (w < 2) store_tile<P, 2>(sA, Ainv_ws, c0, nrow, HV, hv, lane, w);
  else if (Akk_out) store_tile<T, 2>(sA, Akk_out, c0, nrow, HV, hv, lane, w - 2);
}

template <typename T, int DK>
hipError_t launch_t(const ChunkArgs& a, const KdaBuffers& kb, hipStream_t s, int NT, int nslots) {
  typedef typename ComputeOf<T>::type P;
  const dim3 grid(intra_blocks(nslots, a.HV));
  hipLaunchKernelGGL((kda_intra_kernel<T, DK>), grid, dim3(256), 0, s, (const T*)a.q, (const T*)a.k,
                     a.gk, a.beta, a.scale, (T*)kb.Aqk_out, (T*)kb.Akk_out, (P*)a.Ainv, (P*)a.Aqk,
                     (P*)kb.qg, (P*)kb.kg, (P*)kb.kt, (float*)a.GF, kb.dg, a.cu_seqlens,
                     a.chunk_off, a.T, a.B * a.T, a.N, NT, nslots, a.Hk, a.HV);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_intra_kda(const ChunkArgs& a, const KdaBuffers& kb, hipStream_t s, int NT,
                            int nslots) {
  if (a.bf16) {
    if (a.K == 128) return launch_t<bf16_t, 128>(a, kb, s, NT, nslots);
    return launch_t<bf16_t, 64>(a, kb, s, NT, nslots);
  }
  if (a.K == 128) return launch_t<float, 128>(a, kb, s, NT, nslots);
  return launch_t<float, 64>(a, kb, s, NT, nslots);
}

}  // namespace gdn
