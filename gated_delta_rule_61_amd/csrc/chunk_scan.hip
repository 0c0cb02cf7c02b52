// Sequential part of the chunked prefill, gfx950: the chunk-state scan fused
// with the output.  Per (sequence, v-head, V-tile of BV columns), over the
// chunks of the sequence in order, with S^T (K x BV, fp32) the state at the
// chunk start, G the chunk-local cumulative log-gate, Ainv = (I + A)^-1 and
// Aqk from the intra kernel:
//
//   X     = diag(e^G) K S^T                      (state seen by each key)
//   R     = beta * (V - X)
//   Vn    = Ainv R                               (corrected values, "u - w h")
//   O     = scale diag(e^G) Q S^T + Aqk Vn       (inter + intra output)
//   S^T  <- e^{G_last} S^T + K^T diag(e^{G_last - G}) Vn
//
// i.e. v_new = u - w h with u = Ainv (beta V), w = Ainv (beta e^G K); the
// pages' recompute_w_u / chunk_fwd_h / output steps, regrouped so that w and
// u never reach memory ("fla ops/common/chunk_h.py", chunk_fwd_kernel_h:
// sequential chunk loop with an fp32 state, h *= exp(g_last), v scaled by
// exp(g_last - g); "sglang srt/layers/attention/fla/chunk_fwd.py", the
// intra-chunk A consumed by recompute_w_u).  For KDA every scalar e^G becomes
// a per-channel factor inside the contractions (see the KDA variant).
//
// gfx950 design: 4 waves (256 threads) per work-group.
//   * S^T stays in MFMA accumulators: wave w owns key rows
//     [w*DK/4, (w+1)*DK/4) x BV columns; a bf16 copy lives in LDS as the B
//     operand of the next chunk's K S^T and Q S^T;
//   * wave w owns tokens 16w..16w+15 of X, O, R, Vn; its q / k / Ainv / Aqk
//     fragments are prefetched from HBM one chunk ahead into registers;
//   * the key chunk is written to LDS transposed (token-contiguous per key
//     channel) by all 256 threads, as the A operand of K^T Vn;
//   * three block barriers per chunk, no global round trip of any
//     intermediate;
//   * work-groups of one (sequence, head) share an XCD (its L2), and
//     sequences are issued longest first.

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int BT = 64;
constexpr int TP = BT + 8;  // padded token row (elements) of the transposed LDS tiles

// Store 4 consecutive elements of type T (8 or 16 bytes).
template <typename T>
__device__ __forceinline__ void st4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2<T>(a, b), pack2<T>(c, d));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}

__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// raw 8-element row segment of the io type
template <typename T> struct Seg8;
template <> struct Seg8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ bf16_t get(int e) const {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (bf16_t)((e & 1) ? (w >> 16) : (w & 0xFFFF));
  }
};
template <> struct Seg8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0, 0, 0, 0); }
  __device__ __forceinline__ float get(int e) const {
    return e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : e == 3 ? a.w
         : e == 4 ? b.x : e == 5 ? b.y : e == 6 ? b.z : b.w;
  }
};

// Write TPT consecutive tokens of one key channel into the transposed tile
// (element type C).
template <typename C, int TPT>
__device__ __forceinline__ void put_tokens(C* dst, const float (&vals)[TPT]) {
  if constexpr (TPT == 4) {
    st4<C>(dst, vals[0], vals[1], vals[2], vals[3]);
  } else if constexpr (sizeof(C) == 2 && TPT == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack2<C>(vals[0], vals[1]);
  } else {
#pragma unroll
    for (int u = 0; u < TPT; ++u) dst[u] = from_f<C>(vals[u]);
  }
}

template <typename T, int DK, int BV, typename C = typename ComputeOf<T>::type>
struct ScanRegs {
  static constexpr int KS = DK / 32;        // channel slabs
  static constexpr int CB = BV / 16;        // 16-column blocks of the tile
  static constexpr int CG = DK / 8;         // 8-channel groups (loader)
  static constexpr int TG = 256 / CG;       // token groups (loader)
  static constexpr int TPT = BT / TG;       // tokens per loader thread
  Frag<T> kA[KS], qA[KS];                   // rows 16w + row of k, q
  Frag<C> ai[2], aq[2];                     // rows 16w + row of Ainv, Aqk (compute type)
  T vv[CB][4];                              // v[16w + 4grp + i][v0 + 16cb + row], raw
                                            // (converted at use so the prefetch never waits)
  Seg8<T> kt[TPT];                          // loader: tokens TPT*tg + u, channels 8cg..
  float gl, bl;                             // g, beta of token `lane`
};

template <typename T, int DK, int BV, typename C>
__device__ __forceinline__ void load_chunk(ScanRegs<T, DK, BV>& R, const T* __restrict__ q,
                                           const T* __restrict__ k, const T* __restrict__ v,
                                           const float* __restrict__ g,
                                           const float* __restrict__ beta,
                                           const C* __restrict__ Ainv, const C* __restrict__ Aqk,
                                           int c0, int nrow, int Hk, int HV, int V, int jk,
                                           int j, int v0, int w, int lane, int tid) {
  typedef ScanRegs<T, DK, BV> RT;
  const int row = lane & 15, grp = lane >> 4;
  const int r = 16 * w + row;
  if (r < nrow) {
    const size_t qk = ((size_t)(c0 + r) * Hk + jk) * DK + 8 * grp;
#pragma unroll
    for (int s = 0; s < RT::KS; ++s) {
      load8(R.kA[s], k + qk + 32 * s);
      load8(R.qA[s], q + qk + 32 * s);
    }
    const size_t ao = ((size_t)(c0 + r) * HV + j) * BT + 8 * grp;
    load8(R.ai[0], Ainv + ao);
    load8(R.aq[0], Aqk + ao);
    if (w >= 2) {
      load8(R.ai[1], Ainv + ao + 32);
      load8(R.aq[1], Aqk + ao + 32);
    } else {
      R.ai[1].zero();
      R.aq[1].zero();
    }
  } else {
#pragma unroll
    for (int s = 0; s < RT::KS; ++s) { R.kA[s].zero(); R.qA[s].zero(); }
    R.ai[0].zero(); R.aq[0].zero(); R.ai[1].zero(); R.aq[1].zero();
  }
#pragma unroll
  for (int cb = 0; cb < RT::CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * grp + i;
      R.vv[cb][i] = rr < nrow ? v[((size_t)(c0 + rr) * HV + j) * V + v0 + 16 * cb + row] : T(0);
    }
  const int tg = tid / RT::CG, cg = tid % RT::CG;
#pragma unroll
  for (int u = 0; u < RT::TPT; ++u) {
    const int tok = RT::TPT * tg + u;
    if (tok < nrow) R.kt[u].load(k + ((size_t)(c0 + tok) * Hk + jk) * DK + 8 * cg);
    else R.kt[u].zero();
  }
  R.gl = (g && lane < nrow) ? g[(size_t)(c0 + lane) * HV + j] : 0.f;
  R.bl = lane < nrow ? beta[(size_t)(c0 + lane) * HV + j] : 0.f;
}

template <typename T, int DK, int BV, typename C = typename ComputeOf<T>::type>
__global__ __launch_bounds__(256) void gdn_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    const float* __restrict__ h0, float* __restrict__ ht, const C* __restrict__ Ainv,
    const C* __restrict__ Aqk, T* __restrict__ o, const int64_t* __restrict__ cu,
    const int32_t* __restrict__ order, int Tlen, int N, int Hk, int HV, int V) {
  typedef ScanRegs<T, DK, BV> RT;
  constexpr int KS = RT::KS, CB = RT::CB;
  constexpr int WR = DK / 4;        // state rows (key channels) per wave
  constexpr int RB = WR / 16;       // 16-row blocks per wave
  constexpr int KP = DK + 8;        // padded key row of the state copy
  __shared__ __attribute__((aligned(16))) C sKt[DK][TP];         // K^T of the chunk (token-contiguous)
  __shared__ __attribute__((aligned(16))) C sS[BV][KP];          // S (value rows, key-contiguous), io type
  __shared__ __attribute__((aligned(16))) C sR[BV][TP];          // R^T
  __shared__ __attribute__((aligned(16))) C sVn[BV][TP];         // Vn^T
  __shared__ __attribute__((aligned(16))) C sVt[BV][TP];         // (diag(e^{G_last - G}) Vn)^T

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int row = lane & 15, grp = lane >> 4;
  const int NVT = V / BV;

  // ---- work-group -> (sequence, head, V-tile); a (sequence, head) group keeps
  // its NVT tiles on one XCD, groups in order of decreasing sequence length.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, pos = bid >> 3;
  const int vt = pos % NVT;
  const int grpi = (pos / NVT) * 8 + xcd;
  if (grpi >= N * HV) return;
  const int rank = grpi / HV, j = grpi - rank * HV;
  const int n = order ? order[rank] : rank;
  int bos, eos;
  if (cu) {
    long long b0 = cu[n], b1 = cu[n + 1];
    b0 = b0 < 0 ? 0 : (b0 > Tlen ? Tlen : b0);
    b1 = b1 < b0 ? b0 : (b1 > Tlen ? Tlen : b1);
    bos = (int)b0;
    eos = (int)b1;
  } else {
    bos = n * Tlen;
    eos = bos + Tlen;
  }
  const int jk = j / (HV / Hk);
  const int v0 = vt * BV;

  // ---- initial state: St[rb][cb] lane holds S^T[c][v] for
  // c = WR*w + 16rb + 4grp + i, v = v0 + 16cb + row
  f32x4 St[RB][CB];
  const size_t hbase = ((size_t)n * HV + j) * (size_t)V * DK;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (h0) {
        const float4 x = *reinterpret_cast<const float4*>(
            h0 + hbase + (size_t)(v0 + 16 * cb + row) * DK + WR * w + 16 * rb + 4 * grp);
        St[rb][cb] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        St[rb][cb] = zero4();
      }
      st4<C>(&sS[16 * cb + row][WR * w + 16 * rb + 4 * grp], St[rb][cb][0], St[rb][cb][1],
             St[rb][cb][2], St[rb][cb][3]);
    }

  const int NC = (eos - bos + BT - 1) / BT;
  RT nx;
  if (NC > 0)
    load_chunk<T, DK, BV>(nx, q, k, v, g, beta, Ainv, Aqk, bos, eos - bos < BT ? eos - bos : BT,
                          Hk, HV, V, jk, j, v0, w, lane, tid);

  for (int ic = 0; ic < NC; ++ic) {
    const int c0 = bos + ic * BT;
    const int nrow = eos - c0 < BT ? eos - c0 : BT;
    RT cur = nx;
    if (ic + 1 < NC) {
      const int c1 = c0 + BT;
      load_chunk<T, DK, BV>(nx, q, k, v, g, beta, Ainv, Aqk, c1, eos - c1 < BT ? eos - c1 : BT,
                            Hk, HV, V, jk, j, v0, w, lane, tid);
    }
    // K^T into LDS (token-contiguous per channel)
    {
      const int tg = tid / RT::CG, cg = tid % RT::CG;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float vals[RT::TPT];
#pragma unroll
        for (int u = 0; u < RT::TPT; ++u) vals[u] = to_f(cur.kt[u].get(e));
        put_tokens<C, RT::TPT>(&sKt[8 * cg + e][RT::TPT * tg], vals);
      }
    }
    // gates: lane = token
    const float G = wave_incl_scan(cur.gl, lane);
    const float Gl = __shfl(G, nrow - 1, 64);
    float eG[4], eGt[4], br[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * grp + i;
      const float Gr = __shfl(G, rr, 64);
      eG[i] = __expf(Gr);
      eGt[i] = __expf(Gl - Gr);
      br[i] = __shfl(cur.bl, rr, 64);
    }
    const float eGl = __expf(Gl);

    // ---- steps 1-2: X = K S^T, Oi = Q S^T (rows 16w.., all BV columns)
    f32x4 X[CB], Oi[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) { X[cb] = zero4(); Oi[cb] = zero4(); }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Frag<C> kc = conv<C>(cur.kA[s]), qc = conv<C>(cur.qA[s]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        Frag<C> sf;
        load8(sf, &sS[16 * cb + row][32 * s + 8 * grp]);
        X[cb] = mma(kc, sf, X[cb]);
        Oi[cb] = mma(qc, sf, Oi[cb]);
      }
    }
    // ---- step 3: R = beta (v - e^G X) -> LDS (transposed)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rv[i] = br[i] * (to_f(cur.vv[cb][i]) - eG[i] * X[cb][i]);
      st4<C>(&sR[16 * cb + row][16 * w + 4 * grp], rv[0], rv[1], rv[2], rv[3]);
    }
    __syncthreads();

    // ---- step 4: Vn = Ainv R (block lower: slab 1 only for waves 2, 3)
    f32x4 Vn[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      Frag<C> rf;
      load8(rf, &sR[16 * cb + row][8 * grp]);
      Vn[cb] = mma(cur.ai[0], rf, zero4());
      if (w >= 2) {
        load8(rf, &sR[16 * cb + row][32 + 8 * grp]);
        Vn[cb] = mma(cur.ai[1], rf, Vn[cb]);
      }
      st4<C>(&sVn[16 * cb + row][16 * w + 4 * grp], Vn[cb][0], Vn[cb][1], Vn[cb][2], Vn[cb][3]);
      st4<C>(&sVt[16 * cb + row][16 * w + 4 * grp], Vn[cb][0] * eGt[0], Vn[cb][1] * eGt[1],
             Vn[cb][2] * eGt[2], Vn[cb][3] * eGt[3]);
    }
    __syncthreads();

    // ---- step 5: O = scale e^G Oi + Aqk Vn
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Oi[cb][i] * (scale * eG[i]);
      Frag<C> vf;
      load8(vf, &sVn[16 * cb + row][8 * grp]);
      acc = mma(cur.aq[0], vf, acc);
      if (w >= 2) {
        load8(vf, &sVn[16 * cb + row][32 + 8 * grp]);
        acc = mma(cur.aq[1], vf, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * w + 4 * grp + i;
        if (rr < nrow) o[((size_t)(c0 + rr) * HV + j) * V + v0 + 16 * cb + row] = from_f<T>(acc[i]);
      }
    }
    // ---- step 6: S^T = e^{G_last} S^T + K^T diag(e^{G_last - G}) Vn
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        f32x4 acc = St[rb][cb] * eGl;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag<C> af, bfr;
          load8(af, &sKt[WR * w + 16 * rb + row][32 * s + 8 * grp]);
          load8(bfr, &sVt[16 * cb + row][32 * s + 8 * grp]);
          acc = mma(af, bfr, acc);
        }
        St[rb][cb] = acc;
        st4<C>(&sS[16 * cb + row][WR * w + 16 * rb + 4 * grp], acc[0], acc[1], acc[2], acc[3]);
      }
    __syncthreads();
  }

  if (ht) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<float4*>(ht + hbase + (size_t)(v0 + 16 * cb + row) * DK + WR * w + 16 * rb +
                                   4 * grp) =
            make_float4(St[rb][cb][0], St[rb][cb][1], St[rb][cb][2], St[rb][cb][3]);
  }
}

template <typename T, int DK, int BV>
hipError_t launch_scan_t(const ChunkArgs& a, hipStream_t s) {
  typedef typename ComputeOf<T>::type C;
  const int nvt = a.V / BV;
  const int groups = a.N * a.HV;
  const int nblk = ((groups + 7) / 8) * 8 * nvt;
  hipLaunchKernelGGL((gdn_scan_kernel<T, DK, BV>), dim3((unsigned)nblk), dim3(256), 0, s,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, a.scale, a.h0, a.ht,
                     (const C*)a.Ainv, (const C*)a.Aqk, (T*)a.o, a.cu_seqlens, a.seq_order, a.T,
                     a.N, a.Hk, a.HV, a.V);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_gdn(const ChunkArgs& a, hipStream_t s) {
  if (a.bf16) {
    if (a.K == 128) return launch_scan_t<bf16_t, 128, 32>(a, s);
    return launch_scan_t<bf16_t, 64, 32>(a, s);
  }
  if (a.K == 128) return launch_scan_t<float, 128, 32>(a, s);
  return launch_scan_t<float, 64, 32>(a, s);
}

}  // namespace gdn
