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
// intra-chunk A consumed by recompute_w_u).
//
// This kernel serves fp32 io (GDN and KDA); bf16 io runs the LDS-staged
// kernel of chunk_scan_gdn.hip.
//
// gfx950 design: 4 waves (256 threads) per work-group, BV = 16 columns.
//   * S^T stays in fp32 MFMA accumulators: wave w owns key rows
//     [w*DK/4, (w+1)*DK/4); LDS holds S as the B operand of the next chunk's
//     K S^T and Q S^T;
//   * every product is an fp32 16x16x4 MFMA;
//   * wave w owns tokens 16w..16w+15 of X, O, R, Vn; its q / k / Ainv / Aqk
//     fragments, v, and gate factors are prefetched one chunk ahead into one
//     of two register sets used in turn (no copies);
//   * the key chunk is written to LDS transposed (token-contiguous per key
//     channel) by all 256 threads, as the A operand of K^T Vn;
//   * three block barriers per chunk, no global round trip of any
//     intermediate;
//   * work-groups of one (sequence, head) share an XCD (its L2), and
//     sequences are issued longest first.
//
// KDA (one log-gate per key channel) runs the same kernel: every scalar e^G
// becomes a per-channel factor inside the contractions, so the intra kernel
// writes the gated operands K o e^G, Q o e^G and K o e^{G_last - G} (fp32
// for fp32 io) and a per-channel decay e^{G_last}; the scan reads
// those in place of q / k, skips the per-row gate scaling and decays S^T
// row by row ("fla ops/common/chunk_h.py", USE_GK: h *= exp(gk_last)[:, None],
// k *= exp(gk_last - gk)).

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

// Store 4 consecutive values of a computed operand (S, diag(.) Vn); `pl`
// (a lo-part tile) is unused for fp32 operands.
template <typename T>
__device__ __forceinline__ void st4_split(T* ph, T*, float a, float b, float c, float d) {
  st4<T>(ph, a, b, c, d);
}

// raw 8-element row segment of the operand type
template <typename T> struct Seg8;
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

// Channel e of TPT consecutive tokens -> TPT consecutive elements of the
// transposed tile row.
template <int TPT>
__device__ __forceinline__ void put_channel(float* dst, const Seg8<float> (&src)[TPT], int e) {
  if constexpr (TPT == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(src[0].get(e), src[1].get(e), src[2].get(e), src[3].get(e));
  } else {
    *reinterpret_cast<float2*>(dst) = make_float2(src[0].get(e), src[1].get(e));
  }
}

// Types of one scan instantiation.
//   IOT: io type of v and o;  OPT: type of the operand tensors the scan reads
//   (q / k for GDN, the gated operands for KDA);  P: type of the small 64 x 64
//   products (all float here).  SPLIT (computed operands as a hi + lo pair)
//   is off for fp32 operands.
template <typename IOT_, typename OPT_, int DK_, int BV_, bool KDA_>
struct ScanCfg {
  typedef IOT_ IOT;
  typedef OPT_ OPT;
  typedef typename ComputeOf<IOT_>::type P;
  static constexpr int DK = DK_, BV = BV_;
  static constexpr bool KDA = KDA_;
  static constexpr bool SPLIT = __is_same(OPT_, bf16_t);
  static constexpr int KS = DK / 32;        // channel slabs
  static constexpr int CB = BV / 16;        // 16-column blocks of the tile
  static constexpr int WR = DK / 4;         // state rows (key channels) per wave
  static constexpr int RB = WR / 16;        // 16-row blocks per wave
  static constexpr int CG = DK / 8;         // 8-channel groups (loader)
  static constexpr int TG = 256 / CG;       // token groups (loader)
  static constexpr int TPT = BT / TG;       // tokens per loader thread
};

template <typename C>
struct ScanRegs {
  typedef typename C::OPT OPT;
  typedef typename C::P P;
  Frag<OPT> xA[C::KS], oA[C::KS];           // rows 16w + row of the X / O operands (k, q)
  Frag<P> ai[2], aq[2];                     // rows 16w + row of Ainv, Aqk
  typename C::IOT vv[C::CB][4];             // v[16w + 4grp + i][v0 + 16cb + row], raw
  Seg8<OPT> kt[C::TPT];                     // loader: tokens TPT*tg + u, channels 8cg..
                                            // (tg = tid % TG, cg = tid / TG)
  float4 gf[4];                             // gate factors of rows 16w + 4grp + i
  float eGl;                                // GDN: e^{G_last} of the chunk (uniform)
  float4 dg[C::RB];                         // KDA: e^{G_last} of key rows WR*w + 16rb + 4grp + i
};

// Streams the scan reads: work-group-uniform base pointers at the current
// chunk (advanced by scalar adds) plus constant per-lane 32-bit offsets, so
// no per-chunk address arithmetic runs per lane.
template <typename C>
struct ScanStreams {
  typedef typename C::OPT OPT;
  typedef typename C::P P;
  const OPT *x, *op, *t;                    // X operand, O operand, update operand (row-major)
  const typename C::IOT* v;
  const P *ai, *aq;
  const float* gf;                          // gate-factor plane 0 at the chunk
  uint32_t gs;                              // plane stride (floats)
  const float* dg;                          // KDA decay rows of the chunk
  uint32_t oA, oAi, oV[4], oG[4], oK[4], oD;  // element offsets within the chunk
};

// Issue the loads of one chunk.  Full chunks take the unpredicated path; the
// tail chunk of a sequence (nrow < 64) zero-fills rows past its end.  Raw
// values only: nothing here waits on a load.
template <typename C>
__device__ __forceinline__ void load_chunk(ScanRegs<C>& R, const ScanStreams<C>& S, int nrow,
                                           int w, int lane, int tid) {
  typedef typename C::IOT IOT;
  if constexpr (C::KDA) {
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) R.dg[rb] = *reinterpret_cast<const float4*>(S.dg + S.oD + 16 * rb);
  } else {
    R.eGl = S.gf[3 * S.gs];  // row 0 of the chunk is always valid
  }
  if (nrow == BT) {
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      load8(R.xA[s], S.x + S.oA + 32 * s);
      load8(R.oA[s], S.op + S.oA + 32 * s);
    }
    load8(R.ai[0], S.ai + S.oAi);
    load8(R.aq[0], S.aq + S.oAi);
    if (w >= 2) {
      load8(R.ai[1], S.ai + S.oAi + 32);
      load8(R.aq[1], S.aq + S.oAi + 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) R.vv[cb][i] = S.v[S.oV[i] + 16 * cb];
      R.gf[i] = make_float4(S.gf[S.oG[i]], S.gf[S.oG[i] + S.gs], S.gf[S.oG[i] + 2 * S.gs], 0.f);
    }
#pragma unroll
    for (int u = 0; u < C::TPT; ++u) R.kt[u].load(S.t + S.oK[u]);
    return;
  }
  const int row = lane & 15, grp = lane >> 4;
  if (16 * w + row < nrow) {
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      load8(R.xA[s], S.x + S.oA + 32 * s);
      load8(R.oA[s], S.op + S.oA + 32 * s);
    }
    load8(R.ai[0], S.ai + S.oAi);
    load8(R.aq[0], S.aq + S.oAi);
    if (w >= 2) {
      load8(R.ai[1], S.ai + S.oAi + 32);
      load8(R.aq[1], S.aq + S.oAi + 32);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::KS; ++s) { R.xA[s].zero(); R.oA[s].zero(); }
    R.ai[0].zero(); R.aq[0].zero(); R.ai[1].zero(); R.aq[1].zero();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = 16 * w + 4 * grp + i < nrow;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) R.vv[cb][i] = ok ? S.v[S.oV[i] + 16 * cb] : IOT(0);
    R.gf[i] = ok ? make_float4(S.gf[S.oG[i]], S.gf[S.oG[i] + S.gs], S.gf[S.oG[i] + 2 * S.gs], 0.f)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int tg = tid % C::TG;
#pragma unroll
  for (int u = 0; u < C::TPT; ++u) {
    if (C::TPT * tg + u < nrow) R.kt[u].load(S.t + S.oK[u]);
    else R.kt[u].zero();
  }
}

// Operand tensors and chunk tables of one scan launch.
struct ScanArgs {
  const void *x, *op, *t;   // X operand, O operand, update operand
  int op_rows;              // heads per token row of the operand tensors
  int op_head_div;          // operand head of v-head j: j / op_head_div
  const float* dg;          // KDA decay [chunks, HV, K] or nullptr
  const int32_t* coff;      // varlen chunk offsets or nullptr
  int NT;                   // chunks per sequence without varlen
};

template <typename C>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    const typename C::OPT* __restrict__ xop, const typename C::OPT* __restrict__ oop,
    const typename C::OPT* __restrict__ top, int op_rows, int op_head_div,
    const typename C::IOT* __restrict__ v, const float* __restrict__ GF,
    const float* __restrict__ DG, float scale, const float* __restrict__ h0,
    float* __restrict__ ht, void* __restrict__ hs, int nts, int sbf16, long long scap,
    const typename C::P* __restrict__ Ainv,
    const typename C::P* __restrict__ Aqk, typename C::IOT* __restrict__ o,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ coff,
    const int32_t* __restrict__ order, int Tlen, int ttot, int NT, int N, int HV, int V, int dg_rows) {
  typedef ScanRegs<C> RT;
  typedef typename C::OPT OPT;
  typedef typename C::P P;
  typedef typename C::IOT IOT;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int DK = C::DK, BV = C::BV;
  constexpr int KS = C::KS, CB = C::CB, WR = C::WR, RB = C::RB;
  constexpr int KP = DK + 8;              // padded key row of the state copy
  constexpr int NL = SPLIT ? BV : 1;      // rows of the lo-part tiles
  __shared__ __attribute__((aligned(16))) OPT sKt[DK][TP];   // update operand^T (token-contiguous)
  __shared__ __attribute__((aligned(16))) OPT sSh[BV][KP];   // S (value rows, key-contiguous), hi part
  __shared__ __attribute__((aligned(16))) OPT sSl[NL][KP];   //   lo part
  __shared__ __attribute__((aligned(16))) P sR[BV][TP];      // R^T
  __shared__ __attribute__((aligned(16))) P sVn[BV][TP];     // Vn^T
  __shared__ __attribute__((aligned(16))) OPT sVth[BV][TP];  // (diag(e^{G_last - G}) Vn)^T, hi part
  __shared__ __attribute__((aligned(16))) OPT sVtl[NL][TP];  //   lo part

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
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
  int bos, eos, chunk0;
  if (cu) {
    long long b0 = cu[n], b1 = cu[n + 1];
    b0 = b0 < 0 ? 0 : (b0 > Tlen ? Tlen : b0);
    b1 = b1 < b0 ? b0 : (b1 > Tlen ? Tlen : b1);
    bos = (int)b0;
    eos = (int)b1;
    chunk0 = coff ? coff[n] : 0;
  } else {
    bos = n * Tlen;
    eos = bos + Tlen;
    chunk0 = n * NT;
  }
  const int jo = j / op_head_div;  // operand head
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
      const int c = WR * w + 16 * rb + 4 * grp;
      st4_split<OPT>(&sSh[16 * cb + row][c], &sSl[SPLIT ? 16 * cb + row : 0][c], St[rb][cb][0],
                     St[rb][cb][1], St[rb][cb][2], St[rb][cb][3]);
    }

  // ---- streams: uniform bases at chunk 0, per-lane offsets, per-chunk strides
  const uint32_t sQK = (uint32_t)op_rows * DK, sA = (uint32_t)HV * BT, sV = (uint32_t)HV * V,
                 sG = 1;
  // loader: token group varies fastest across lanes, so the transposed
  // writes of a half-wave cover one contiguous 128-byte row segment
  const int tg = tid % C::TG, cg = tid / C::TG;
  ScanStreams<C> St_;
  St_.x = xop + (size_t)bos * sQK + (size_t)jo * DK;
  St_.op = oop + (size_t)bos * sQK + (size_t)jo * DK;
  St_.t = top + (size_t)bos * sQK + (size_t)jo * DK;
  St_.ai = Ainv + (size_t)bos * sA + (size_t)j * BT;
  St_.aq = Aqk + (size_t)bos * sA + (size_t)j * BT;
  St_.v = v + (size_t)bos * sV + (size_t)j * V + v0;
  St_.gs = (uint32_t)gf_stride(ttot);
  St_.gf = GF + (size_t)j * 4 * St_.gs + bos;
  St_.dg = DG ? DG + ((size_t)chunk0 * HV + j) * DK : nullptr;
  St_.oA = (uint32_t)(16 * w + row) * sQK + 8 * grp;
  St_.oAi = (uint32_t)(16 * w + row) * sA + 8 * grp;
  St_.oD = (uint32_t)(WR * w + 4 * grp);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    St_.oV[i] = (uint32_t)(16 * w + 4 * grp + i) * sV + row;
    St_.oG[i] = (uint32_t)(16 * w + 4 * grp + i) * sG;
    St_.oK[i] = (uint32_t)(C::TPT * tg + (i < C::TPT ? i : 0)) * sQK + 8 * cg;
  }
  const size_t cQK = (size_t)BT * sQK, cA = (size_t)BT * sA, cV = (size_t)BT * sV,
               cG = (size_t)BT * sG, cD = (size_t)HV * DK;

  int NC = (eos - bos + BT - 1) / BT;
  // KDA: the decay rows of the sequence's chunks are rows chunk0 .. chunk0 + NC - 1
  // of DG; only non-monotone (invalid) varlen boundaries can reach past its end
  if (C::KDA && chunk0 + NC > dg_rows) NC = dg_rows - chunk0 > 0 ? dg_rows - chunk0 : 0;
  // state snapshots: the state at the start of every nts-th chunk
  const size_t sbase = hs ? (size_t)snapshot_offset(cu, n, Tlen, nts * BT) : 0;

  // One chunk: compute from `cur`, prefetch the next chunk into `nxt`.
  auto step = [&](RT& cur, RT& nxt, int ic) {
    const int c0 = bos + ic * BT;
    const int nrow = eos - c0 < BT ? eos - c0 : BT;
    // (entries past the buffer's capacity are not written)
    if (hs && ic % nts == 0 && (long long)(sbase + ic / nts) < scap) {
      const size_t hp = ((sbase + ic / nts) * HV + j) * (size_t)V * DK;
#pragma unroll
      for (int rb2 = 0; rb2 < RB; ++rb2)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const float x[4] = {St[rb2][cb][0], St[rb2][cb][1], St[rb2][cb][2], St[rb2][cb][3]};
          store_state4(hs, hp + (size_t)(v0 + 16 * cb + row) * DK + WR * w + 16 * rb2 + 4 * grp, x, sbf16 != 0);
        }
    }
    // update operand^T into LDS from the loader registers
#pragma unroll
    for (int e = 0; e < 8; ++e) put_channel<C::TPT>(&sKt[8 * cg + e][C::TPT * tg], cur.kt, e);
    if (ic + 1 < NC) {
      St_.x += cQK; St_.op += cQK; St_.t += cQK; St_.ai += cA; St_.aq += cA; St_.v += cV;
      St_.gf += cG;
      if constexpr (C::KDA) St_.dg += cD;
      const int c1 = c0 + BT;
      load_chunk<C>(nxt, St_, eos - c1 < BT ? eos - c1 : BT, w, lane, tid);
    }
    float eG[4], eGt[4], br[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { eG[i] = cur.gf[i].x; eGt[i] = cur.gf[i].y; br[i] = cur.gf[i].z; }

    // ---- steps 1-2: X = K S^T, Oi = Q S^T (rows 16w.., all BV columns)
    f32x4 X[CB], Oi[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) { X[cb] = zero4(); Oi[cb] = zero4(); }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        Frag<OPT> sf;
        load8(sf, &sSh[16 * cb + row][32 * s + 8 * grp]);
        X[cb] = mma(cur.xA[s], sf, X[cb]);
        Oi[cb] = mma(cur.oA[s], sf, Oi[cb]);
        if constexpr (SPLIT) {
          load8(sf, &sSl[16 * cb + row][32 * s + 8 * grp]);
          X[cb] = mma(cur.xA[s], sf, X[cb]);
          Oi[cb] = mma(cur.oA[s], sf, Oi[cb]);
        }
      }
    }
    // ---- step 3: R = beta (v - e^G X) -> LDS (transposed); KDA: e^G is in the operand
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rv[i] = br[i] * (to_f(cur.vv[cb][i]) - (C::KDA ? X[cb][i] : eG[i] * X[cb][i]));
      st4<P>(&sR[16 * cb + row][16 * w + 4 * grp], rv[0], rv[1], rv[2], rv[3]);
    }
    __syncthreads();

    // ---- step 4: Vn = Ainv R (block lower: slab 1 only for waves 2, 3)
    f32x4 Vn[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      Frag<P> rf;
      load8(rf, &sR[16 * cb + row][8 * grp]);
      Vn[cb] = mma(cur.ai[0], rf, zero4());
      if (w >= 2) {
        load8(rf, &sR[16 * cb + row][32 + 8 * grp]);
        Vn[cb] = mma(cur.ai[1], rf, Vn[cb]);
      }
      st4<P>(&sVn[16 * cb + row][16 * w + 4 * grp], Vn[cb][0], Vn[cb][1], Vn[cb][2], Vn[cb][3]);
      if constexpr (C::KDA) {
        st4_split<OPT>(&sVth[16 * cb + row][16 * w + 4 * grp], &sVtl[SPLIT ? 16 * cb + row : 0][16 * w + 4 * grp],
                       Vn[cb][0], Vn[cb][1], Vn[cb][2], Vn[cb][3]);
      } else {
        st4_split<OPT>(&sVth[16 * cb + row][16 * w + 4 * grp], &sVtl[SPLIT ? 16 * cb + row : 0][16 * w + 4 * grp],
                       Vn[cb][0] * eGt[0], Vn[cb][1] * eGt[1], Vn[cb][2] * eGt[2], Vn[cb][3] * eGt[3]);
      }
    }
    __syncthreads();

    // ---- step 5: O = scale e^G Oi + Aqk Vn
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Oi[cb][i] * (C::KDA ? scale : scale * eG[i]);
      Frag<P> vf;
      load8(vf, &sVn[16 * cb + row][8 * grp]);
      acc = mma(cur.aq[0], vf, acc);
      if (w >= 2) {
        load8(vf, &sVn[16 * cb + row][32 + 8 * grp]);
        acc = mma(cur.aq[1], vf, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * w + 4 * grp + i;
        if (rr < nrow) o[((size_t)(c0 + rr) * HV + j) * V + v0 + 16 * cb + row] = from_f<IOT>(acc[i]);
      }
    }
    // ---- step 6: S^T = e^{G_last} S^T + K^T diag(e^{G_last - G}) Vn
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        f32x4 acc;
        if constexpr (C::KDA) {
          acc = St[rb][cb] * f32x4{cur.dg[rb].x, cur.dg[rb].y, cur.dg[rb].z, cur.dg[rb].w};
        } else {
          acc = St[rb][cb] * cur.eGl;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag<OPT> af, bfr;
          load8(af, &sKt[WR * w + 16 * rb + row][32 * s + 8 * grp]);
          load8(bfr, &sVth[16 * cb + row][32 * s + 8 * grp]);
          acc = mma(af, bfr, acc);
          if constexpr (SPLIT) {
            load8(bfr, &sVtl[16 * cb + row][32 * s + 8 * grp]);
            acc = mma(af, bfr, acc);
          }
        }
        St[rb][cb] = acc;
        const int c = WR * w + 16 * rb + 4 * grp;
        st4_split<OPT>(&sSh[16 * cb + row][c], &sSl[SPLIT ? 16 * cb + row : 0][c], acc[0], acc[1],
                       acc[2], acc[3]);
      }
    __syncthreads();
  };

  RT ra, rb;
  if (NC > 0) load_chunk<C>(ra, St_, eos - bos < BT ? eos - bos : BT, w, lane, tid);
  for (int ic = 0; ic < NC; ic += 2) {
    step(ra, rb, ic);
    if (ic + 1 < NC) step(rb, ra, ic + 1);
  }

  if (ht) {
#pragma unroll
    for (int rb2 = 0; rb2 < RB; ++rb2)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<float4*>(ht + hbase + (size_t)(v0 + 16 * cb + row) * DK + WR * w + 16 * rb2 +
                                   4 * grp) =
            make_float4(St[rb2][cb][0], St[rb2][cb][1], St[rb2][cb][2], St[rb2][cb][3]);
  }
}

template <typename C>
hipError_t launch_scan_c(const ChunkArgs& a, const ScanArgs& sa, hipStream_t s) {
  typedef typename C::OPT OPT;
  typedef typename C::P P;
  typedef typename C::IOT IOT;
  const int nvt = a.V / C::BV;
  const int groups = a.N * a.HV;
  const int nblk = ((groups + 7) / 8) * 8 * nvt;
  hipLaunchKernelGGL((chunk_scan_kernel<C>), dim3((unsigned)nblk), dim3(256), 0, s,
                     (const OPT*)sa.x, (const OPT*)sa.op, (const OPT*)sa.t, sa.op_rows,
                     sa.op_head_div, (const IOT*)a.v, (const float*)a.GF, sa.dg, a.scale, a.h0,
                     a.ht, a.hs, a.split_chunks, a.hs_bf16 ? 1 : 0, a.hs_cap, (const P*)a.Ainv, (const P*)a.Aqk,
                     (IOT*)a.o, a.cu_seqlens, sa.coff, a.seq_order, a.T, a.B * a.T, sa.NT, a.N, a.HV, a.V,
                     a.max_chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_gdn(const ChunkArgs& a, hipStream_t s) {
  ScanArgs sa;
  sa.x = a.k; sa.op = a.q; sa.t = a.k;
  sa.op_rows = a.Hk;
  sa.op_head_div = a.HV / a.Hk;
  sa.dg = nullptr;
  sa.coff = nullptr;
  sa.NT = (a.T + BT - 1) / BT;
  if (a.bf16) return launch_scan_gdn_bf16(a, s);
  if (a.K == 128) return launch_scan_c<ScanCfg<float, float, 128, 16, false>>(a, sa, s);
  return launch_scan_c<ScanCfg<float, float, 64, 16, false>>(a, sa, s);
}

// KDA: operands are the gated tensors written by the KDA intra kernel, one
// per v-head ([tokens, HV, K]), plus the per-chunk decay rows DG.
hipError_t launch_scan_kda(const ChunkArgs& a, const void* qg, const void* kg, const void* kt,
                           const float* dg, hipStream_t s) {
  ScanArgs sa;
  sa.x = kg; sa.op = qg; sa.t = kt;
  sa.op_rows = a.HV;
  sa.op_head_div = 1;
  sa.dg = dg;
  sa.coff = a.chunk_off;
  sa.NT = (a.T + BT - 1) / BT;
  if (a.bf16) return launch_scan_kda_bf16(a, qg, kg, kt, dg, s);
  if (a.K == 128) return launch_scan_c<ScanCfg<float, float, 128, 16, true>>(a, sa, s);
  return launch_scan_c<ScanCfg<float, float, 64, 16, true>>(a, sa, s);
}

}  // namespace gdn
