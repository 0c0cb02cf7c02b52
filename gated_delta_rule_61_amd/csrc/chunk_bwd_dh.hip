// Backward state-gradient scan, gfx950: "fla ops/common/chunk_h.py",
// chunk_bwd_kernel_dh.  Per (sequence, v-head), over the chunks in reverse
// order, with dh (K x V, fp32) the gradient with respect to the state at the
// end of the current chunk:
//
//   start:        dh = dht (or 0)
//   every chunk:  if its index is a multiple of split_size / 64, store dh;
//                 dh <- decay * dh + scale * (Q o e^G)^T dO
//   end:          dh0 = dh
//
// with G the chunk-local cumulative log-gate (scalar per token, the fixed
// per-head gamma, or per key channel), decay = e^{G_last} (per channel for
// the per-channel gate, applied to the key rows).  This is the state
// gradient of the decay-only recurrence h_t = decay_t h_{t-1} + k_t v_t^T,
// o_t = scale q_t^T h_t; the delta rule's erase term is not part of it.
//
// gfx950 design.  Work-group = 256 threads per (sequence, v-head, 32-column
// V tile); wave w holds key rows DK/4 * w .. + DK/4 of dh in fp32 MFMA
// accumulators for the whole scan.  A chunk's q and dO rows are staged in
// LDS transposed (key channel / value column major, tokens contiguous), so
// both operands of the 16x16x32 bf16 product read 8 consecutive tokens with
// one 16-byte LDS read.  The gated operand is split into a bf16 hi + lo pair
// (dO * scale e^{G_t} for a scalar gate, q * scale e^{G_t,c} for the
// per-channel gate); the other operand is the raw bf16 input, exact.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int BT = 64;
constexpr int BVT = 32;        // V columns per work-group
constexpr int TP = BT + 8;     // padded token row of the transposed tiles (bf16)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma_bf(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int DK, bool KDA>
__global__ __launch_bounds__(256) void chunk_bwd_dh_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, const float* __restrict__ g,
    const float* __restrict__ gamma, const float* __restrict__ gk, float scale,
    const float* __restrict__ dht, float* __restrict__ dh, int nts, float* __restrict__ dh0,
    const int64_t* __restrict__ cu, int Tlen, int N, int Hk, int HV) {
  constexpr int DV = DK;
  constexpr int RW = DK / 4;          // key rows per wave
  constexpr int RB = RW / 16;         // 16-row blocks per wave
  constexpr int QU = BT * DK / 8;     // 16-byte q units of a chunk
  constexpr int QPT = QU / 256;       // ... per thread
  __shared__ __attribute__((aligned(16))) bf16_t sAh[DK][TP];   // A operand (q side), hi
  __shared__ __attribute__((aligned(16))) bf16_t sAl[KDA ? DK : 1][TP];   //   lo
  __shared__ __attribute__((aligned(16))) bf16_t sBh[BVT][TP];  // B operand (dO side), hi
  __shared__ __attribute__((aligned(16))) bf16_t sBl[KDA ? 1 : BVT][TP];  //   lo
  __shared__ float sG[KDA ? BT : 1][KDA ? DK + 4 : 1];          // KDA cumulative gates
  __shared__ float sGam[BT + 1];    // GDN: scale e^{G_t}, and e^{G_last} at [BT]
  __shared__ float sDec[KDA ? DK : 1];  // KDA: e^{G_last, c}

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  const int NVT = DV / BVT;
  const int bid = blockIdx.x;
  const int vt = bid % NVT;
  const int sh = bid / NVT;
  if (sh >= N * HV) return;
  const int sq = sh / HV, j = sh - sq * HV;
  const int jk = j / (HV / Hk);
  const int v0 = vt * BVT;
  int bos, eos;
  if (cu) {
    long long b0 = cu[sq], b1 = cu[sq + 1];
    b0 = b0 < 0 ? 0 : (b0 > Tlen ? Tlen : b0);
    b1 = b1 < b0 ? b0 : (b1 > Tlen ? Tlen : b1);
    bos = (int)b0;
    eos = (int)b1;
  } else {
    bos = sq * Tlen;
    eos = bos + Tlen;
  }
  const int NC = (eos - bos + BT - 1) / BT;
  const size_t hbase = (size_t)sh * DV * DK;   // [N, HV, V, K] arrays
  const size_t sbase = dh ? (size_t)snapshot_offset(cu, sq, Tlen, nts * BT) : 0;

  // accumulators: block (rb, cb), lane (n, gq): key row RW w + 16 rb + 4 gq + i, column v0 + 16 cb + n
  f32x4 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (dht) {
        const float4 x = *reinterpret_cast<const float4*>(
            dht + hbase + (size_t)(v0 + 16 * cb + n) * DK + RW * w + 16 * rb + 4 * gq);
        acc[rb][cb] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        *reinterpret_cast<float4*>(dst + (size_t)(v0 + 16 * cb + n) * DK + RW * w + 16 * rb + 4 * gq) =
            make_float4(acc[rb][cb][0], acc[rb][cb][1], acc[rb][cb][2], acc[rb][cb][3]);
  };

  for (int ic = NC - 1; ic >= 0; --ic) {
    const int c0 = bos + ic * BT;
    const int nrow = eos - c0 < BT ? eos - c0 : BT;

    // ---- global loads of the chunk (rows past its end repeat the last row; masked below)
    uint4 qr[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int u = tid + 256 * i, t = u / (DK / 8), cu8 = u % (DK / 8);
      const int tc = t < nrow ? t : nrow - 1;
      qr[i] = *reinterpret_cast<const uint4*>(q + ((size_t)(c0 + tc) * Hk + jk) * DK + 8 * cu8);
    }
    const int dt_ = tid / (BVT / 8), du = tid % (BVT / 8);   // dO unit: token, 8-column group
    const int dtc = dt_ < nrow ? dt_ : nrow - 1;
    const uint4 dr = *reinterpret_cast<const uint4*>(dout + ((size_t)(c0 + dtc) * HV + j) * DV + v0 + 8 * du);

    // ---- chunk-local cumulative gates
    if constexpr (KDA) {
      if (tid < DK) {
        float gv[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          const int tc = t < nrow ? t : nrow - 1;
          gv[t] = gk[((size_t)(c0 + tc) * HV + j) * DK + tid];
        }
        float G = 0.f;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          G += t < nrow ? gv[t] : 0.f;
          sG[t][tid] = G;
        }
        sDec[tid] = __expf(G);
      }
    } else {
      if (w == 0) {
        const int tc = lane < nrow ? lane : nrow - 1;
        float gl = g ? g[(size_t)(c0 + tc) * HV + j] : (gamma ? gamma[j] : 0.f);
        gl = lane < nrow ? gl : 0.f;
        const float G = intra::wave_incl_scan(gl, lane);
        sGam[lane] = lane < nrow ? scale * __expf(G) : 0.f;
        if (lane == nrow - 1) sGam[BT] = __expf(G);
      }
    }
    __syncthreads();

    // ---- transposed operand tiles
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int u = tid + 256 * i, t = u / (DK / 8), cu8 = u % (DK / 8);
      const uint32_t wv[4] = {qr[i].x, qr[i].y, qr[i].z, qr[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * cu8 + e;
        const uint32_t bits = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xFFFFu);
        if constexpr (KDA) {
          const float a = t < nrow ? bf2f((bf16_t)bits) * scale * __expf(sG[t][c]) : 0.f;
          const bf16_t hi = f2bf(a);
          sAh[c][t] = hi;
          sAl[c][t] = f2bf(a - bf2f(hi));
        } else {
          sAh[c][t] = t < nrow ? (bf16_t)bits : (bf16_t)0;
        }
      }
    }
    {
      const uint32_t wv[4] = {dr.x, dr.y, dr.z, dr.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * du + e;
        const uint32_t bits = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xFFFFu);
        if constexpr (KDA) {
          sBh[c][dt_] = dt_ < nrow ? (bf16_t)bits : (bf16_t)0;
        } else {
          const float b = bf2f((bf16_t)bits) * sGam[dt_];   // 0 past the chunk end
          const bf16_t hi = f2bf(b);
          sBh[c][dt_] = hi;
          sBl[c][dt_] = f2bf(b - bf2f(hi));
        }
      }
    }
    __syncthreads();

    // ---- snapshot, decay, accumulate
    if (dh && ic % nts == 0) store_state(dh + ((sbase + ic / nts) * HV + j) * (size_t)DV * DK);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 dec;
#pragma unroll
      for (int i = 0; i < 4; ++i) dec[i] = KDA ? sDec[RW * w + 16 * rb + 4 * gq + i] : sGam[BT];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] *= dec;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const u32x4 ah = *reinterpret_cast<const u32x4*>(&sAh[RW * w + 16 * rb + n][32 * s + 8 * gq]);
        u32x4 al;
        if constexpr (KDA) al = *reinterpret_cast<const u32x4*>(&sAl[RW * w + 16 * rb + n][32 * s + 8 * gq]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const u32x4 bh = *reinterpret_cast<const u32x4*>(&sBh[16 * cb + n][32 * s + 8 * gq]);
          acc[rb][cb] = mma_bf(ah, bh, acc[rb][cb]);
          if constexpr (KDA) {
            acc[rb][cb] = mma_bf(al, bh, acc[rb][cb]);
          } else {
            const u32x4 bl = *reinterpret_cast<const u32x4*>(&sBl[16 * cb + n][32 * s + 8 * gq]);
            acc[rb][cb] = mma_bf(ah, bl, acc[rb][cb]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (dh0) store_state(dh0 + hbase);
}

template <int DK, bool KDA>
hipError_t launch_k(const BwdDhArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.N * a.HV * (DK / BVT);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bwd_dh_kernel<DK, KDA>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.dout, a.g, a.g_gamma, a.gk, a.scale, a.dht, a.dh,
                     a.split_chunks, a.dh0, a.cu_seqlens, a.T, a.N, a.Hk, a.HV);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dh(const BwdDhArgs& a, hipStream_t s) {
  if (a.gk) return a.K == 128 ? launch_k<128, true>(a, s) : launch_k<64, true>(a, s);
  return a.K == 128 ? launch_k<128, false>(a, s) : launch_k<64, false>(a, s);
}

}  // namespace gdn
