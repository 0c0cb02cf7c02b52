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
// gfx950 design: 4 waves per work-group, wave w owns 16-token block w; the
// key channels are walked in 32-channel slabs (everything but the pair
// products is independent per channel, and those accumulate over slabs).
// 34 KB of LDS and <= 168 VGPRs give 3 work-groups per CU.
//   * per slab, each wave forms the block-local cumulative gate of its 16
//     tokens (two 8-token runs per channel) and its block's total; every
//     exponent below is a difference of block-local sums plus block totals;
//   * block pair (i, j), j <= i, is one fp16 MFMA product per slab with
//     every factor bounded:
//       row operand  x[t] o exp(G[t] - G[n_i]) o exp(G[n_i] - G[m_j])
//       col operand  k[s] o exp(G[m_j] - G[s])
//     (n_i first row of block i, m_j last row of block j).  For j < i every
//     exponent is <= 0.  The diagonal pair (j = i) carries exp(G[n_i] -
//     G[m_i]) >= 1, the decay inside one 16-token block; when that exceeds
//     10 nats in a slab (or an operand leaves the fp16 range) the wave
//     computes that slab's part of its diagonal block exactly, pair by pair,
//     in fp32;
//   * a slab's global loads are issued while the slab before it is
//     processed; its tiles in LDS are double-buffered, so a slab needs two
//     barriers;
//   * the pairs' decay factors exp(G[n_i] - G[m_j]) are one LDS table per
//     slab built by all threads (they do not depend on the row);
//   * beta / scale / causal masks on the fp32 accumulators; Aqk and A are
//     staged in LDS over the slab tiles, the 64 x 64 solve is the same
//     forward substitution + block merge as the GDN kernel, and the tiles
//     leave in 16-byte row pieces;
//   * the gated planes of bf16 io are written head- and slab-major
//     ([HV][DK / 32][tokens][32]): a chunk's slab is one contiguous 4 KB
//     block, which the chunk scan's movers copy to LDS as it is.  Row-major
//     planes (a 64-byte piece per row at an HV * DK * 2-byte stride) cost
//     the kernel ~20 us more at B=2 T=8192 H=32.

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

// Element `i` of an array whose base is the same for the whole wave, with the
// byte offset formed in 32 bits: the access then takes the scalar-base form
// (one VGPR per address instead of two).
template <typename X>
__device__ __forceinline__ X* at(X* base, uint32_t i) {
  typedef typename std::conditional<std::is_const<X>::value, const char, char>::type B;
  return reinterpret_cast<X*>(reinterpret_cast<B*>(base) + i * (uint32_t)sizeof(X));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// LDS of one work-group.  The key channels are processed in 32-channel
// slabs; a slab's tiles are double-buffered, so that the next slab's
// cumulative sum can start while another wave still reads this one.  After
// the last slab the two 64 x 64 fp32 tiles of the solve overlay them.
constexpr int SG = 32 + 4;   // padded fp32 row of a slab's gate tile
constexpr int SC = 32 + 8;   // padded row of a slab's column-operand tile

template <typename P>
struct SlabTiles {
  float g[BT][SG];    // cumulative gate inside each 16-token block
  float tot[4][32];   // each block's total
  P c[BT][SC];        // column operand k[s] o exp(G[m_j] - G[s])
  float e[10][32];    // exp(G[n_i] - G[m_j]) of block pair (i, j), j <= i
};
struct SolveTiles {
  float a[BT][AP];    // A, then (I + A)^-1
  float q[BT][AP];    // Aqk
};
template <typename P>
union IntraSmem {
  SlabTiles<P> s[2];
  SolveTiles t;
};

// Occupancy: 3 work-groups per CU (<= 168 VGPRs; 34 KB of LDS for bf16 io,
// 42 KB for fp32 io).  A cap of 128 VGPRs for a fourth spills 30 - 57
// registers and about doubles the time.
template <typename T, int DK, typename P = typename ComputeOf<T>::type>
__global__ __launch_bounds__(256, 3) void kda_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ gk,
    const float* __restrict__ beta, float scale, T* __restrict__ Aqk_out,
    T* __restrict__ Akk_out, P* __restrict__ Ainv_ws, P* __restrict__ Aqk_ws,
    P* __restrict__ qg, P* __restrict__ kg, P* __restrict__ kt, float* __restrict__ GF,
    float* __restrict__ DG, const int64_t* __restrict__ cu, const int32_t* __restrict__ coff,
    int Tlen, int ttot, int N, int NT, int nslots, int Hk, int HV) {
  constexpr int NS = DK / 32;  // 32-channel slabs
  __shared__ __attribute__((aligned(16))) IntraSmem<P> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, grp = lane >> 4;
  int slot, hv, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, hv)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int hk = hv / (HV / Hk);

  // lanes of the cumulative sum: slab channel ch, tokens 16w + 8hh + u
  const int ch = lane & 31, hh = lane >> 5;
  // lanes of the operands: token t, slab channels cb .. cb + 7
  const int t = 16 * w + row, cb = 8 * grp;
  const bool tv = t < nrow;
  const int tc = tv ? t : nrow - 1;

  // A slab's global inputs (addresses of rows past nrow are clamped to the
  // last row, the values masked where used); the next slab's are loaded
  // while this one is processed.
  struct In {
    float g[8];
    Frag<T> q, k;
  };
  // (uniform chunk bases and 32-bit lane offsets, so that the loads take the
  // scalar-base form and each address costs one VGPR)
  const float* gkc = gk + ((size_t)c0 * HV + hv) * DK;
  const T* qc = q + ((size_t)c0 * Hk + hk) * DK;
  const T* kc = k + ((size_t)c0 * Hk + hk) * DK;
  const uint32_t gstr = (uint32_t)(HV * DK), qstr = (uint32_t)(Hk * DK);
  // gated planes at the chunk: for bf16 io head- and slab-major
  // ([HV][DK / 32][tokens][32], so that a chunk's slab is one 4 KB block),
  // for fp32 io row-major like q ([tokens][HV][DK])
  constexpr bool SLABS = sizeof(P) == 2;
  const size_t pbase = SLABS ? ((size_t)hv * NS * ttot + c0) * 32 : ((size_t)c0 * HV + hv) * DK;
  P* qgc = qg + pbase;
  P* kgc = kg + pbase;
  P* ktc = kt + pbase;
  auto load_in = [&](int s, In& in) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * w + 8 * hh + u;
      const uint32_t tok = (uint32_t)(r < nrow ? r : nrow - 1);
      in.g[u] = *at(gkc, tok * gstr + (uint32_t)(32 * s + ch));
    }
    const uint32_t qo = (uint32_t)tc * qstr + (uint32_t)(32 * s + cb);
    load8(in.q, at(qc, qo));
    load8(in.k, at(kc, qo));
  };
  In cur, nxt;
  load_in(0, cur);
  const float* bc = beta + (size_t)c0 * HV + hv;
  float braw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * grp + i < nrow ? 16 * w + 4 * grp + i : nrow - 1;
    braw[i] = *at(bc, (uint32_t)r * (uint32_t)HV);
  }
  const float bt = *at(bc, (uint32_t)tc * (uint32_t)HV);

  f32x4 QK[4], KK[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) { QK[jb] = zero4(); KK[jb] = zero4(); }

#pragma unroll
  for (int s = 0; s < NS; ++s) {
    SlabTiles<P>& S = sm.s[s & 1];
    if (s + 1 < NS) load_in(s + 1, nxt);

    // ---- cumulative gate inside the wave's block (rows past nrow add 0)
    {
      float acc = 0.f, part[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc += 16 * w + 8 * hh + u < nrow ? cur.g[u] : 0.f;
        part[u] = acc;
      }
      const float lo = __shfl(acc, ch, 64);  // total of the block's first 8 tokens
      const float add = hh ? lo : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) S.g[16 * w + 8 * hh + u][ch] = part[u] + add;
      if (hh) S.tot[w][ch] = acc + lo;
    }
    __syncthreads();

    // ---- the lane's 8 channels: sums of the block totals before the
    // wave's block and from it on (G[t] = g[t] + before, G_last = before + from)
    float before[8], from[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) before[e] = from[e] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float4 t0 = *reinterpret_cast<const float4*>(&S.tot[b][cb]);
      const float4 t1 = *reinterpret_cast<const float4*>(&S.tot[b][cb + 4]);
      const float tb[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (b < w) before[e] += tb[e];
        else from[e] += tb[e];
      }
    }
    float qa[8], ka[8];  // q, k scaled by exp(G[t] - G[n_w])
    float dmax = 0.f;
    {
      float gt[8], gn[8], gm[8];
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
        const float4 a = *reinterpret_cast<const float4*>(&S.g[t][cb + h]);
        const float4 n = *reinterpret_cast<const float4*>(&S.g[16 * w][cb + h]);
        const float4 m = *reinterpret_cast<const float4*>(&S.g[16 * w + 15][cb + h]);
        gt[h] = a.x; gt[h + 1] = a.y; gt[h + 2] = a.z; gt[h + 3] = a.w;
        gn[h] = n.x; gn[h + 1] = n.y; gn[h + 2] = n.z; gn[h + 3] = n.w;
        gm[h] = m.x; gm[h + 1] = m.y; gm[h + 2] = m.z; gm[h + 3] = m.w;
      }
      float vq[8], vk[8], vt[8], vc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = tv ? cur.q.get(e) : 0.f, kv = tv ? cur.k.get(e) : 0.f;
        const float a = __expf(gt[e] - gn[e]);
        const float eg = __expf(gt[e] + before[e]);
        qa[e] = qv * a;
        ka[e] = kv * a;
        vq[e] = qv * eg;
        vk[e] = kv * eg;
        vt[e] = kv * __expf(from[e] - gt[e]);
        vc[e] = kv * __expf(gm[e] - gt[e]);
        dmax = fmaxf(dmax, gn[e] - gm[e]);
      }
      if (tv) {
        const uint32_t oo = SLABS ? (uint32_t)s * (uint32_t)ttot * 32u + (uint32_t)(t * 32 + cb)
                                  : (uint32_t)t * gstr + (uint32_t)(32 * s + cb);
        if constexpr (sizeof(P) == 2) {
          *reinterpret_cast<uint4*>(at(qgc, oo)) =
              make_uint4(pack2_bounded<P>(vq[0], vq[1]), pack2_bounded<P>(vq[2], vq[3]),
                         pack2_bounded<P>(vq[4], vq[5]), pack2_bounded<P>(vq[6], vq[7]));
          *reinterpret_cast<uint4*>(at(kgc, oo)) =
              make_uint4(pack2_bounded<P>(vk[0], vk[1]), pack2_bounded<P>(vk[2], vk[3]),
                         pack2_bounded<P>(vk[4], vk[5]), pack2_bounded<P>(vk[6], vk[7]));
          *reinterpret_cast<uint4*>(at(ktc, oo)) =
              make_uint4(pack2_bounded<P>(vt[0], vt[1]), pack2_bounded<P>(vt[2], vt[3]),
                         pack2_bounded<P>(vt[4], vt[5]), pack2_bounded<P>(vt[6], vt[7]));
        } else {
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            *reinterpret_cast<float4*>(at(qgc, oo + e)) = make_float4(vq[e], vq[e + 1], vq[e + 2], vq[e + 3]);
            *reinterpret_cast<float4*>(at(kgc, oo + e)) = make_float4(vk[e], vk[e + 1], vk[e + 2], vk[e + 3]);
            *reinterpret_cast<float4*>(at(ktc, oo + e)) = make_float4(vt[e], vt[e + 1], vt[e + 2], vt[e + 3]);
          }
        }
      }
      if constexpr (sizeof(P) == 2) {
        *reinterpret_cast<uint4*>(&S.c[t][cb]) =
            make_uint4(pack2_bounded<P>(vc[0], vc[1]), pack2_bounded<P>(vc[2], vc[3]),
                       pack2_bounded<P>(vc[4], vc[5]), pack2_bounded<P>(vc[6], vc[7]));
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 4)
          *reinterpret_cast<float4*>(&S.c[t][cb + e]) = make_float4(vc[e], vc[e + 1], vc[e + 2], vc[e + 3]);
      }
    }
    // the block pairs' decay factors exp(G[n_i] - G[m_j]) from the
    // block-local sums: the exponent is g[16i] - tot[i] on the diagonal
    // (j = i), and g[16i] plus the totals of the blocks strictly between j
    // and i below it (j < i)
    auto pair_decay = [&](int idx) {
      const int pr = idx >> 5, c = idx & 31;
      const int i = pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0;
      const int j = pr - tix(i, 0);
      float d = S.g[16 * i][c];
      if (j == i) d -= S.tot[i][c];
#pragma unroll
      for (int b = 1; b < 3; ++b)
        if (b > j && b < i) d += S.tot[b][c];
      S.e[pr][c] = __expf(d);
    };
    pair_decay(tid);
    if (tid < 10 * 32 - 256) pair_decay(tid + 256);
    if (w == 0 && hh == 0)
      DG[((size_t)slot * HV + hv) * DK + 32 * s + ch] =
          __expf(S.tot[0][ch] + S.tot[1][ch] + S.tot[2][ch] + S.tot[3][ch]);
    const float Dw = wave_max(dmax);
    __syncthreads();

    // ---- block pairs (w, jb), jb <= w, over the slab's channels: fp16 (fp32
    // for fp32 io) MFMA.  The diagonal pair's operands decide first whether
    // its decay or size leaves the fast path's range; if so, this slab's part
    // of the diagonal block is computed exactly, pair by pair, in fp32.
    bool exact;
    {
      const float4 e0 = *reinterpret_cast<const float4*>(&S.e[tix(w, w)][cb]);
      const float4 e1 = *reinterpret_cast<const float4*>(&S.e[tix(w, w)][cb + 4]);
      const float sv[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
      float opmax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) opmax = fmaxf(opmax, fmaxf(fabsf(qa[e] * sv[e]), fabsf(ka[e] * sv[e])));
      exact = !(Dw <= DIAG_MAX_DECAY) || !(wave_max(opmax) <= DIAG_MAX_OPERAND);
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb > w || (jb == w && exact)) continue;  // uniform per wave
      const float4 e0 = *reinterpret_cast<const float4*>(&S.e[tix(w, jb)][cb]);
      const float4 e1 = *reinterpret_cast<const float4*>(&S.e[tix(w, jb)][cb + 4]);
      const float sv[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
      Frag<P> fa, fb, fc;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        set_bounded<P>(fa, e, qa[e] * sv[e]);
        set_bounded<P>(fb, e, ka[e] * sv[e]);
      }
      load8(fc, &S.c[16 * jb + row][cb]);
      QK[jb] = mma(fa, fc, QK[jb]);
      KK[jb] = mma(fb, fc, KK[jb]);
    }
    if (exact) {
      // pairs (r, sc), sc <= r < nrow, of the diagonal block; the gate
      // difference comes from the block-local sums of one block
      const int sc = 16 * w + row, r0 = 16 * w + 4 * grp;
      float aq[4] = {0.f, 0.f, 0.f, 0.f}, ak[4] = {0.f, 0.f, 0.f, 0.f};
      const uint32_t so = (uint32_t)(sc < nrow ? sc : nrow - 1) * qstr + (uint32_t)(32 * s);
#pragma unroll 1
      for (int c = 0; c < 32; ++c) {
        const float gs = S.g[sc][c];
        const float ks = to_f(*at(kc, so + (uint32_t)c));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          const uint32_t ro = (uint32_t)(r < nrow ? r : nrow - 1) * qstr + (uint32_t)(32 * s + c);
          const float kv = ks * expf(S.g[r][c] - gs);
          aq[i] = fmaf(to_f(*at(qc, ro)), kv, aq[i]);
          ak[i] = fmaf(to_f(*at(kc, ro)), kv, ak[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = sc <= r0 + i && r0 + i < nrow;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          if (jb == w) {
            QK[jb][i] += in ? aq[i] : 0.f;
            KK[jb][i] += in ? ak[i] : 0.f;
          }
      }
    }
    if (s + 1 < NS) cur = nxt;
  }

  // ---- scale / beta / masks; Aqk and A to LDS (upper blocks zero), over
  // the slab tiles once every wave is done with them
  __syncthreads();
  float (*sA)[AP] = sm.t.a;
  float (*sQ)[AP] = sm.t.q;
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
