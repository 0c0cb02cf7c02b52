// Sequential part of the chunked prefill for bf16 io with the scalar gate,
// gfx950.  The mathematics is the one of the generic scan: per (sequence,
// v-head, V-tile), over the chunks in order, with S^T (K x BV, fp32; BV the
// tile's columns) the state at the chunk start and Ainv, Aqk, G from the
// intra kernel,
//
//   X     = diag(e^G) K S^T
//   R     = beta * (V - X)
//   Vn    = Ainv R                               (u - w h)
//   O     = scale diag(e^G) Q S^T + Aqk Vn
//   S^T  <- e^{G_last} S^T + K^T diag(e^{G_last - G}) Vn
//
// ("fla ops/common/chunk_h.py", chunk_fwd_kernel_h: sequential chunk loop,
// fp32 state, h *= exp(g_last), v scaled by exp(g_last - g); "sglang
// srt/layers/attention/fla/chunk_fwd.py": the intra-chunk matrices consumed by
// recompute_w_u and the output step.)
//
// gfx950 design.  Work-group = one (sequence, v-head, 32-column V tile), eight
// waves, two per SIMD (the 64-column form is described at the end):
//   * two state waves, one per 16-column block, keep their S^T (K x 16) in
//     fp32 MFMA accumulators and run the chain of a chunk,
//       X = K S^T  ->  R  ->  Vn = Ainv R  ->  S^T update,
//     without an LDS round trip of their own.  An accumulator lane holds
//     column l % 16 at rows 4 (l / 16) + i; two accumulators give a lane the
//     8 reduction slots of a 32-deep B operand.  The rows of the A operands
//     (tokens of K / Ainv, channels of K^T) are placed so that accumulator
//     pair (2s, 2s + 1) covers exactly reduction slots 32s + 8 (l / 16) + e in
//     natural order: block 2s + h, row 4a + b  <->  index 32s + 8a + 4h + b.
//     S, R and Vn so become B operands in registers, and every A fragment is
//     one 16-byte LDS read;
//   * the K^T operand of the state update comes from the same k tile through
//     gfx950's transposing LDS read (ds_read_b64_tr_b16), after the
//     mid-chunk barrier;
//   * two helper waves compute O (no later step of the chunk needs it) from
//     the S and Vn fragments the state waves publish in LDS;
//   * four mover waves (the second wave on each SIMD) move the data: the next
//     chunk's q / k / Ainv / Aqk / v / gate rows go from global memory to LDS
//     with direct-to-LDS loads (global_load_lds_dwordx4, whole rows, no
//     registers), double buffered; a wave keeps only a few such loads in
//     flight, so four issuing waves move about twice what two do.  The lines
//     of the chunk after next are pulled into L2 ahead of them; O leaves
//     through LDS as 16-byte row stores;
//   * q / k and Ainv / Aqk tiles are stored with a 16-byte-unit XOR swizzle so
//     that the fragment reads and the transposing reads hit distinct banks;
//   * the raw bf16 q / k enter the products exactly; S enters Q S^T and
//     diag(e^{G_last - G}) Vn the state update as hi + lo bf16 pairs (about 16
//     significant bits); K S^T takes S rounded to bf16 (its error enters R
//     below R's own fp16 rounding); the 64 x 64 products (Ainv R, Aqk Vn) run
//     in fp16;
//   * a state wave issues every LDS read of a chunk's first half before its
//     first product, so the chain waits out the LDS latency once;
//   * two barriers per chunk; the work-groups of one (sequence, head) share an
//     XCD (its L2), sequences are issued longest first.
// A CU holds one such work-group at a time (LDS, and two 247-VGPR waves per
// SIMD).  When the 32-column work-groups would not all run at once, the
// scalar-gate scan (K = 128) uses 64-column ones instead: four state waves
// (one per SIMD), two helper waves of two 16-column blocks each, and two
// movers taking load sets {k, Ainv, v} and {q, Aqk, gate rows}.  The o tile
// then lives in the v buffer of the chunk's stage, which the state waves have
// read before the mid-chunk barrier and the movers refill only after the
// mover that loads v has stored o from it.

#include <atomic>

#include "gdn_device.h"
#include "gdn_launch.h"
#include "scan_tiles.h"

namespace gdn {

namespace {

using namespace tiles;

// KDA: the k / q tiles are the gated fp16 operands K o e^G and Q o e^G, a
// third tile holds K o e^{G_last - G} for the state update, the scalar
// gate factors are 1 except beta, and S^T decays row by row by the chunk's
// e^{G_last} (one value per key channel).
template <int DK, bool KDA, int NB>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdn_scan_bf16_kernel(
    const void* __restrict__ qop, const void* __restrict__ kop, const f16_t* __restrict__ ktop,
    const bf16_t* __restrict__ v, const float* __restrict__ GF, const float* __restrict__ DG,
    const f16_t* __restrict__ Ainv, const f16_t* __restrict__ Aqk, float scale,
    const float* __restrict__ h0, float* __restrict__ ht, void* __restrict__ hs, int nts, int sbf16,
    long long scap, bf16_t* __restrict__ o,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ order, const int32_t* __restrict__ coff,
    int Tlen, int ttot, int NT, int N, int Hk, int HV, int V, int dg_rows) {
  typedef Lds<DK> L;
  constexpr int KS = L::KS, KB = L::KB, NQK = L::NQK;
  // NB 16-column blocks per work-group, one state wave each; two helper
  // waves of NB / 2 blocks each; the other 6 - NB waves move data
  static_assert(NB == 2 || (NB == 4 && !KDA), "32 columns, or 64 for the scalar gate");
  constexpr int BVW = 16 * NB;                 // V columns per work-group
  constexpr int NHB = NB / 2;                  // column blocks per helper wave
  constexpr int NMW = 6 - NB;                  // mover waves
  constexpr int VTB = BT * BVW * 2;            // v tile bytes
  constexpr int OROW = BVW * 2 + 16;           // padded o row (bytes) of sO
  // q / k tile sources (GDN: the raw bf16 inputs, one row per q / k head;
  // KDA: the gated fp16 operands, head- and slab-major: [HV][DK / 32][tokens][32])
  const char* const qsrc = reinterpret_cast<const char*>(qop);
  const char* const ksrc = reinterpret_cast<const char*>(kop);
  // two stages of the chunk inputs, separate arrays so that the compiler can
  // tell the stage being filled from the one being read
  __shared__ __attribute__((aligned(16))) char sK0[L::QK], sK1[L::QK], sQ0[L::QK], sQ1[L::QK];
  __shared__ __attribute__((aligned(16))) char sAi0[L::AT], sAi1[L::AT], sAq0[L::AT], sAq1[L::AT];
  __shared__ __attribute__((aligned(16))) char sV0[VTB], sV1[VTB];
  __shared__ __attribute__((aligned(16))) float sG0[4][BT], sG1[4][BT];  // gate-factor planes
  // KDA: K o e^{G_last - G} tiles and the chunk's decay row e^{G_last}
  __shared__ __attribute__((aligned(16))) char sT0[KDA ? L::QK : 16], sT1[KDA ? L::QK : 16];
  __shared__ __attribute__((aligned(16))) float sD0[KDA ? DK : 4], sD1[KDA ? DK : 4];
  // S fragments for the output: GDN fp32 (split there into bf16 hi + lo),
  // KDA fp16 (the B operand itself)
  __shared__ __attribute__((aligned(16))) u32x4 sSF[NB][KS][KDA ? 1 : 2][64];
  __shared__ __attribute__((aligned(16))) u32x4 sVnF[NB][2][64];      // Vn fragments (fp16)
  // o tile; with 64 columns it lives in the v buffer of the chunk's stage
  // (free after the mid-chunk barrier, refilled only after o has left)
  __shared__ __attribute__((aligned(16))) char sO[NB == 2 ? BT * OROW : 16];
  __shared__ __attribute__((aligned(16))) uint32_t sSink[64];          // L2-prefetch landing words

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave roles; wave w runs on SIMD w % 4: state waves on SIMDs 0 and 1,
  // helpers on 2 and 3, one mover on each SIMD (placing both state waves
  // on one SIMD, or a state wave beside the other block's helper, was slower)
  const int role = w < NB ? 0 : w < NB + 2 ? 1 : 2;
  const int ridx = NB == 2 ? (w < 4 ? (w & 1) : w - 4) : (w < NB ? w : w < NB + 2 ? w - NB : w - NB - 2);
  const bool is_state = role == 0;
  const int cb = ridx;                    // 16-column block (state, helper) / mover index
  const int n = lane & 15, g = lane >> 4;
  const int NVT = V / BVW;

  // ---- work-group -> (sequence, head, V-tile).  Work-group ids are dealt
  // round-robin to the 8 XCDs.  The unit is a (sequence, q / k head): its
  // HV / Hk v-heads and their NVT tiles run next to each other on one XCD, so
  // that they share the q / k rows in that XCD's L2 (KDA: one v-head per
  // unit).  Units go in order of decreasing sequence length.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, pos = bid >> 3;
  const int G = KDA ? 1 : HV / Hk;            // v-heads per unit
  const int per = G * NVT;                    // work-groups per unit
  const int unit = (pos / per) * 8 + xcd;
  const int rem = pos - (pos / per) * per;
  const int vt = rem % NVT;
  const int HU = HV / G;                      // units per sequence
  if (unit >= N * HU) return;
  const int rank = unit / HU, j = (unit - rank * HU) * G + rem / NVT;
  const int ns = order ? order[rank] : rank;
  int bos, eos;
  if (cu) {
    long long b0 = cu[ns], b1 = cu[ns + 1];
    b0 = b0 < 0 ? 0 : (b0 > Tlen ? Tlen : b0);
    b1 = b1 < b0 ? b0 : (b1 > Tlen ? Tlen : b1);
    bos = (int)b0;
    eos = (int)b1;
  } else {
    bos = ns * Tlen;
    eos = bos + Tlen;
  }
  const int jo = KDA ? j : j / (HV / Hk);   // row of the q / k tile sources
  const int v0 = vt * BVW;
  int NC = (eos - bos + BT - 1) / BT;
  // KDA: global index of the sequence's first chunk (row of the decay rows);
  // only non-monotone (invalid) varlen boundaries can reach past their end
  const int chunk0 = KDA ? (coff ? coff[ns] : ns * NT) : 0;
  if (KDA && chunk0 + NC > dg_rows) NC = dg_rows - chunk0 > 0 ? dg_rows - chunk0 : 0;
  const size_t hbase = ((size_t)ns * HV + j) * (size_t)V * DK;
  const size_t gs = (size_t)gf_stride(ttot);   // gate-factor plane stride
  const uint32_t qk_row = (uint32_t)(KDA ? HV : Hk) * DK * 2, a_row = (uint32_t)HV * BT * 2,
                 v_row = (uint32_t)HV * V * 2;

  if (is_state) {
    // =================== state wave: the recurrence of 16 columns
    // S^T blocks: block kb, lane: channels perm_row(kb, 4g + i), column 16cb + n
    f32x4 St[KB];
    u32x4 Sh[KS];   // S rounded to bf16 (KDA: fp16), B operand of X = K S^T
    // publish S for the output (GDN: fp32; KDA: its fp16 rounding), keep
    // the rounding
    auto publish_s = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const f32x4 a = St[2 * s], b = St[2 * s + 1];
        if constexpr (KDA) {
          Sh[s] = pack_h(a, b);
          sSF[cb][s][0][lane] = Sh[s];
        } else {
          sSF[cb][s][0][lane] = __builtin_bit_cast(u32x4, a);
          sSF[cb][s][1][lane] = __builtin_bit_cast(u32x4, b);
          Sh[s] = u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]),
                        pack_bf2(b[2], b[3])};
        }
      }
    };
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (h0) {
        const float4 x = *reinterpret_cast<const float4*>(
            h0 + hbase + (size_t)(v0 + 16 * cb + n) * DK + perm_row(kb, 4 * g));
        St[kb] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        St[kb] = zero4();
      }
    }
    publish_s();
    __syncthreads();

    // per-lane LDS byte offsets, the same in every chunk.  The swizzle of row
    // perm_row(blk, n) does not depend on blk, so a tile block adds
    // blk_rows(blk) whole rows to the offsets of block 0.
    int o_kf[KS];                 // K row fragments, slab s
#pragma unroll
    for (int s = 0; s < KS; ++s) o_kf[s] = qk_off<DK>(perm_row(0, n), 4 * s + g);
    const int o_ai0 = a_off(perm_row(0, n), g), o_ai1 = a_off(perm_row(0, n), 4 + g);
    int o_tr[KB / 2][2][2];       // K^T transposing reads [kb / 2][slab][token half]
#pragma unroll
    for (int kh = 0; kh < KB / 2; ++kh)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          o_tr[kh][s][h] = qk_off<DK>(32 * s + 8 * g + (n >> 2) + 4 * h, 4 * kh + (n & 3));

    // state snapshots: the state at the start of every nts-th chunk
    const size_t sbase = hs ? (size_t)snapshot_offset(cu, ns, Tlen, nts * BT) : 0;
    // the state at the start of chunk c, if it is a snapshot chunk (entries
    // past the buffer's capacity are not written); stored at the end of the
    // chunk before, while the wave waits at the barrier
    auto snapshot = [&](int c) __attribute__((always_inline)) {
      if (hs && c < NC && c % nts == 0 && (long long)(sbase + c / nts) < scap) {
        const size_t hp = ((sbase + c / nts) * HV + j) * (size_t)V * DK + (size_t)(v0 + 16 * cb + n) * DK;
        // blocks 2m and 2m + 1 hold keys 32 m + 8 g + [0, 8) of this lane's row
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          const float x[8] = {St[kb][0], St[kb][1], St[kb][2], St[kb][3],
                              St[kb + 1][0], St[kb + 1][1], St[kb + 1][2], St[kb + 1][3]};
          store_state8(hs, hp + perm_row(kb, 4 * g), x, sbf16 != 0);
        }
      }
    };
    snapshot(0);
    auto chunk = [&](auto stg, int c) __attribute__((always_inline)) {
      constexpr bool S1 = decltype(stg)::value;
      const char* sK = S1 ? sK1 : sK0;
      const char* sKt = KDA ? (S1 ? sT1 : sT0) : sK;   // source of the update's K^T
      const char* sAi = S1 ? sAi1 : sAi0;
      const char* sV = S1 ? sV1 : sV0;
      const float (*sG)[BT] = S1 ? sG1 : sG0;
      const float* sD = S1 ? sD1 : sD0;
      const int nrow = eos - (bos + c * BT) < BT ? eos - (bos + c * BT) : BT;

      // ---- every LDS read of the first half, issued up front in the order
      // of use (the compiler would otherwise issue each just before its use
      // and wait out the LDS latency at every step of the chain)
      // K row fragments: block tb, lane: tokens perm_row(tb, 4g + i)
      u32x4 A[KS][4];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) A[s][tb] = ld16(sK + o_kf[s] + blk_rows(tb) * (2 * DK));
      // lane's rows of block tb are the 4 consecutive tokens perm_row(tb, 4g) + i:
      // one 16-byte read per gate plane, one transposing read of the v tile
      // (this lane addresses columns 16cb + 4 (n % 4) .. + 3 of token
      // perm_row(tb, 4g + n / 4))
      f32x4 ex[4], ey[4], bz[4];
      uint2 vr[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int t0 = perm_row(tb, 4 * g);
        ex[tb] = KDA ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&sG[0][t0]);
        bz[tb] = *reinterpret_cast<const f32x4*>(&sG[2][t0]);
        vr[tb] = ld_tr(sV + (perm_row(tb, 4 * g + (n >> 2)) * BVW + 16 * cb + 4 * (n & 3)) * 2);
      }
      u32x4 Ai[6];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) Ai[tb] = ld16(sAi + o_ai0 + blk_rows(tb) * 128);
      Ai[4] = ld16(sAi + o_ai1 + blk_rows(2) * 128);
      Ai[5] = ld16(sAi + o_ai1 + blk_rows(3) * 128);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        ey[tb] = KDA ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&sG[1][perm_row(tb, 4 * g)]);
      const float eGl = KDA ? 1.f : sG[3][0];
      __builtin_amdgcn_sched_barrier(0);

      // ---- X = K S^T with S rounded to bf16 (its rounding error enters R
      // below the fp16 rounding of R itself); KDA: (K o e^G) S^T, fp16
      f32x4 X[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) X[tb] = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) X[tb] = KDA ? mma_h(A[s][tb], Sh[s], X[tb]) : mma_bf(A[s][tb], Sh[s], X[tb]);
      // ---- R = beta (v - e^G X); rows past the end are zero (KDA: e^G is
      // inside X, and e^{G_last - G} inside the update's K^T: ex = ey = 1)
      f32x4 R[4], eGt[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const float vv[4] = {__builtin_bit_cast(float, vr[tb].x << 16), __builtin_bit_cast(float, vr[tb].x & 0xFFFF0000u),
                             __builtin_bit_cast(float, vr[tb].y << 16), __builtin_bit_cast(float, vr[tb].y & 0xFFFF0000u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) R[tb][i] = bz[tb][i] * (vv[i] - ex[tb][i] * X[tb][i]);
        eGt[tb] = ey[tb];
      }
      if (nrow < BT) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = perm_row(tb, 4 * g + i) < nrow;
            R[tb][i] = ok ? R[tb][i] : 0.f;
            eGt[tb][i] = ok ? eGt[tb][i] : 0.f;
          }
      }
      const u32x4 Rf0 = pack_h(R[0], R[1]), Rf1 = pack_h(R[2], R[3]);
      // ---- Vn = Ainv R (block lower triangular in 32-token slabs)
      f32x4 Vn[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) Vn[tb] = mma_h(Ai[tb], Rf0, zero4());
      Vn[2] = mma_h(Ai[4], Rf1, Vn[2]);
      Vn[3] = mma_h(Ai[5], Rf1, Vn[3]);
      // publish Vn for the output; Vt = diag(e^{G_last - G}) Vn (zero past the
      // end) as a bf16 (KDA: fp16) hi + lo pair
      sVnF[cb][0][lane] = pack_h(Vn[0], Vn[1]);
      sVnF[cb][1][lane] = pack_h(Vn[2], Vn[3]);
      u32x4 Vh[2], Vl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (KDA)
          split_h(Vn[2 * s] * eGt[2 * s], Vn[2 * s + 1] * eGt[2 * s + 1], Vh[s], Vl[s]);
        else
          split_bf(Vn[2 * s] * eGt[2 * s], Vn[2 * s + 1] * eGt[2 * s + 1], Vh[s], Vl[s]);
      }
      lds_barrier();

      // ---- K^T fragments: lane (n, g) of block kb holds channel
      // perm_row(kb, n) of tokens 32s + 8g + e, e = 0..7, the slot order of
      // Vt.  Two transposing reads each: this lane addresses channels
      // perm_row(kb, 4 (n % 4)) .. + 3 of token 32s + 8g + n / 4 (+ 4).
      u32x4 Kt[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint2 lo = ld_tr(sKt + o_tr[kb >> 1][s][0] + 8 * (kb & 1));
          const uint2 hi = ld_tr(sKt + o_tr[kb >> 1][s][1] + 8 * (kb & 1));
          Kt[kb][s] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      // KDA: decay of the lane's state rows, channels perm_row(kb, 4g + i)
      f32x4 dk[KDA ? KB : 1];
      if constexpr (KDA) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dk[kb] = *reinterpret_cast<const f32x4*>(sD + perm_row(kb, 4 * g));
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- S^T <- e^{G_last} S^T + K^T Vt  (KDA: diag(e^{G_last}) S^T + K^T Vn)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (KDA)
          St[kb] = St[kb] * dk[kb];
        else
          St[kb] = St[kb] * eGl;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          St[kb] = KDA ? mma_h(Kt[kb][s], Vh[s], St[kb]) : mma_bf(Kt[kb][s], Vh[s], St[kb]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          St[kb] = KDA ? mma_h(Kt[kb][s], Vl[s], St[kb]) : mma_bf(Kt[kb][s], Vl[s], St[kb]);
      }
      publish_s();
      snapshot(c + 1);
      lds_barrier();
    };
    for (int c = 0; c < NC; c += 2) {
      chunk(Stage0{}, c);
      if (c + 1 < NC) chunk(Stage1{}, c + 1);
    }
    if (ht) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        store_nt16(ht + hbase + (size_t)(v0 + 16 * cb + n) * DK + perm_row(kb, 4 * g), St[kb]);
    }
  } else if (role == 1) {
    // =================== helper wave: the output of NB / 2 16-column blocks
    __syncthreads();
    auto chunk = [&](auto stg, int c) __attribute__((always_inline)) {
      constexpr bool S1 = decltype(stg)::value;
      const char* sQ = S1 ? sQ1 : sQ0;
      const char* sAq = S1 ? sAq1 : sAq0;
      const float (*sG)[BT] = S1 ? sG1 : sG0;
      // the o tile: sO, or (64 columns) this stage's v buffer, whose 128-byte
      // rows take a 16-byte-unit XOR swizzle by row / 8
      char* oT = NB == 2 ? sO : const_cast<char*>(S1 ? sV1 : sV0);
      // the state waves' reads at the start of a chunk head the chain; the
      // helpers (which have slack) and the movers stay off the LDS meanwhile
      // (about 500 and 250 cycles; measured at DK = 128)
      if constexpr (DK == 128) __builtin_amdgcn_s_sleep(8);
      // ---- Oi = Q S^T from the published fp32 S (split into bf16 hi + lo);
      // KDA: (Q o e^G) S^T with the published fp16 S
      f32x4 Oi[NHB][4];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) Oi[hb][tb] = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 A[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) A[tb] = ld16(sQ + qk_off<DK>(perm_row(tb, n), 4 * s + g));
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const int cbh = cb * NHB + hb;
          if constexpr (KDA) {
            const u32x4 bs = sSF[cbh][s][0][lane];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) Oi[hb][tb] = mma_h(A[tb], bs, Oi[hb][tb]);
          } else {
            u32x4 bh, bl;
            split_bf(__builtin_bit_cast(f32x4, sSF[cbh][s][0][lane]),
                     __builtin_bit_cast(f32x4, sSF[cbh][s][KDA ? 0 : 1][lane]), bh, bl);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) Oi[hb][tb] = mma_bf(A[tb], bh, Oi[hb][tb]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) Oi[hb][tb] = mma_bf(A[tb], bl, Oi[hb][tb]);
          }
        }
      }
      lds_barrier();

      // ---- O = scale e^G Oi + Aqk Vn -> LDS tile
      u32x4 vf[NHB][2];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        vf[hb][0] = sVnF[cb * NHB + hb][0][lane];
        vf[hb][1] = sVnF[cb * NHB + hb][1][lane];
      }
      u32x4 Aq[6];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) Aq[tb] = ld16(sAq + a_off(perm_row(tb, n), g));
      Aq[4] = ld16(sAq + a_off(perm_row(2, n), 4 + g));
      Aq[5] = ld16(sAq + a_off(perm_row(3, n), 4 + g));
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int cbh = cb * NHB + hb;
        const u32x4 vf0 = vf[hb][0], vf1 = vf[hb][1];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const f32x4 ex = KDA ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&sG[0][perm_row(tb, 4 * g)]);
          f32x4 acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = Oi[hb][tb][i] * (scale * ex[i]);
          acc = mma_h(Aq[tb], vf0, acc);
          if (tb >= 2) acc = mma_h(Aq[tb + 2], vf1, acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = perm_row(tb, 4 * g + i), col = 16 * cbh + n;
            const int ob = NB == 2 ? row * OROW + 2 * col
                                   : row * (2 * BVW) + (((col >> 3) ^ ((row >> 3) & 7)) << 4) + 2 * (col & 7);
            *reinterpret_cast<bf16_t*>(oT + ob) = f2bf(acc[i]);
          }
        }
      }
      lds_barrier();
    };
    for (int c = 0; c < NC; c += 2) {
      chunk(Stage0{}, c);
      if (c + 1 < NC) chunk(Stage1{}, c + 1);
    }
  } else {
    // =================== mover wave: global <-> LDS traffic
    // Direct-to-LDS loads of the next chunk into the other stage; with 32
    // columns each of the four movers also stores a quarter of the o tile.
    // Load sets (mr): GDN: 0 k, 1 q, 2 Ainv and v, 3 Aqk and the gate rows.
    // KDA: 0 K o e^G and v, 1 Q o e^G, the beta row and the decay row,
    // 2 K o e^{G_last - G}, 3 Ainv and Aqk.  With 64 columns two movers
    // take sets {0, 2} and {1, 3}; the one that loads v also stores the
    // whole o tile, which sits in the v buffer its next loads refill.
    const int mv = ridx;
    // load set of this mover: movers 0 and 1 share SIMDs with the state
    // waves, which leave them fewer issue slots, so they take the lighter
    // sets (GDN: Ainv + v, Aqk + gates; KDA: K o e^{G_last - G}, Ainv + Aqk)
    const int mr = NB == 2 ? (mv + 2) & 3 : mv + 2;
    constexpr int NVL = VTB / 1024;              // 1 KB loads per v tile
    // per-lane byte offsets within a full chunk: LDS slot (row, unit')
    // receives global unit unit' ^ swizzle(row)
    uint32_t o_qk[NQK], o_a[8], o_v[NVL];
    // KDA's gated planes are head- and slab-major (a chunk's 32-channel slab
    // is one 4 KB block, the slabs of a head ttot * 64 bytes apart)
    const uint32_t slab_bytes = (uint32_t)ttot * 64u;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int row = i * L::QROWS + lane / (DK / 8);
      o_qk[i] = KDA ? plane_off<DK>(row, lane % (DK / 8), slab_bytes)
                    : (uint32_t)row * qk_row + 16 * ((lane % (DK / 8)) ^ qk_swz<DK>(row));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + lane / 8;
      o_a[i] = (uint32_t)row * a_row + 16 * ((lane % 8) ^ a_swz(row));
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i)
      o_v[i] = (uint32_t)((64 / (BVW / 8)) * i + lane / (BVW / 8)) * v_row + 16 * (lane % (BVW / 8));

    // loads of the chunk at token c0 into the given stage
    auto dma_chunk = [&](int c0, lchar* dK, lchar* dQ, lchar* dT, lchar* dAi, lchar* dAq, lchar* dV,
                         lchar* dG, lchar* dD) __attribute__((always_inline)) {
      const int nr = eos - c0 < BT ? eos - c0 : BT;
      const size_t xo = KDA ? ((size_t)j * (DK / 32) * ttot + c0) * 64 : (size_t)c0 * qk_row + (size_t)jo * DK * 2;
      const char* ac0 = reinterpret_cast<const char*>(Ainv + ((size_t)c0 * HV + j) * BT);
      const char* ac1 = reinterpret_cast<const char*>(Aqk + ((size_t)c0 * HV + j) * BT);
      const char* vc = reinterpret_cast<const char*>(v + ((size_t)c0 * HV + j) * V + v0);
      // gate planes (KDA: only the beta plane is read); KDA decay row
      const int rg = lane < nr ? lane : nr - 1;
      const float* gp = GF + (size_t)j * 4 * gs + c0 + rg;
      if constexpr (KDA) {
        if (mr == 0) {
          dma_plane_tile<DK>(ksrc + xo, o_qk, nr, slab_bytes, dK, lane);
          dma_v_tile(vc, o_v, nr, v_row, dV, lane);
        } else if (mr == 1) {
          dma_plane_tile<DK>(qsrc + xo, o_qk, nr, slab_bytes, dQ, lane);
          dma4(gp + 2 * gs, dG + 512);
          const float* dp = DG + ((size_t)(chunk0 + (c0 - bos) / BT) * HV + j) * DK;
#pragma unroll
          for (int i = 0; i < DK / 64; ++i) dma4(dp + 64 * i + lane, dD + 256 * i);
        } else if (mr == 2) {
          dma_plane_tile<DK>(reinterpret_cast<const char*>(ktop) + xo, o_qk, nr, slab_bytes, dT, lane);
        } else {
          dma_a_tile(ac0, o_a, nr, a_row, dAi, lane);
          dma_a_tile(ac1, o_a, nr, a_row, dAq, lane);
        }
      } else if constexpr (NB == 4) {
        if (mr == 2) {
          dma_qk_tile<DK>(ksrc + xo, o_qk, nr, qk_row, dK, lane);
          dma_a_tile(ac0, o_a, nr, a_row, dAi, lane);
          dma_v_tile<BVW>(vc, o_v, nr, v_row, dV, lane);
        } else {
          dma_qk_tile<DK>(qsrc + xo, o_qk, nr, qk_row, dQ, lane);
          dma_a_tile(ac1, o_a, nr, a_row, dAq, lane);
#pragma unroll
          for (int pl = 0; pl < 4; ++pl) dma4(gp + pl * gs, dG + 256 * pl);
        }
      } else {
        if (mr < 2) {
          dma_qk_tile<DK>(pick(mr == 0, ksrc, qsrc) + xo, o_qk, nr, qk_row, mr == 0 ? dK : dQ, lane);
        } else {
          dma_a_tile(pick(mr == 2, ac0, ac1), o_a, nr, a_row, mr == 2 ? dAi : dAq, lane);
          if (mr == 2) {
            dma_v_tile(vc, o_v, nr, v_row, dV, lane);
          } else {
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) dma4(gp + pl * gs, dG + 256 * pl);
          }
        }
      }
    };

    // pull the lines of the chunk at token c0 into L2 ahead of its
    // direct-to-LDS loads.  The head's q / k / Ainv / Aqk lines are cut into
    // 64-line pieces, one per (work-group, mover) of the head (the others
    // repeat one); movers 2 also take the lines of their v slice, movers 0,
    // 1, 3 the gate rows.  Exactly kTouches instructions per mover.
    auto touch_chunk = [&](int c0) __attribute__((always_inline)) {
      const int nr = eos - c0 < BT ? eos - c0 : BT;
      lchar* sink = (lchar*)sSink;
      constexpr int QKP = DK / 64;               // 64-line pieces per q or k tile
      constexpr int NXT = KDA ? 3 : 2;           // q / k-like tiles of a chunk
      // 64 columns: fewer work-groups per head, so every one of a unit's
      // work-groups takes its own pieces
      const int piece = (NMW * (NB == 2 ? vt : rem) + mv) % (NXT * QKP + 2);
      const char* p;
      if (piece < NXT * QKP) {
        const int t = piece / QKP;
        const char* x = pick(t == 0, qsrc, pick(t == 1, ksrc, reinterpret_cast<const char*>(ktop)));
        if constexpr (KDA) {
          // slabs 2 * (piece % QKP) and the next one: 32 lines (two rows each) per slab
          const int row = 2 * (lane & 31) < nr ? 2 * (lane & 31) : nr - 1;
          p = x + ((size_t)j * (DK / 32) * ttot + c0 + row) * 64 +
              (size_t)(2 * (piece % QKP) + (lane >> 5)) * slab_bytes;
        } else {
          const int row0 = (piece % QKP) * (64 / QKP) + lane / QKP;
          const int row = row0 < nr ? row0 : nr - 1;
          p = x + (size_t)(c0 + row) * qk_row + (size_t)jo * DK * 2 + 128 * (lane % QKP);
        }
      } else {
        const int row = lane < nr ? lane : nr - 1;
        p = reinterpret_cast<const char*>(pick(piece == NXT * QKP, Ainv, Aqk) +
                                          ((size_t)(c0 + row) * HV + j) * BT);
      }
      touch4(p, sink);
      const int rr = lane < nr ? lane : nr - 1;
      if (mr == (KDA ? 0 : 2)) touch4(v + ((size_t)(c0 + rr) * HV + j) * V + v0, sink);
      else if (KDA) touch4(GF + (size_t)j * 4 * gs + 2 * gs + c0 + rr, sink);
      else touch4(GF + (size_t)j * 4 * gs + (lane >> 1 & 3) * gs + c0 + (nr > 32 ? 32 * (lane & 1) : 0), sink);
    };

    // the o rows of the chunk at token c0 from its LDS tile (oT): with 32
    // columns a quarter per mover; with 64 columns all of them, by the mover
    // that loads v (mr 2)
    auto store_o = [&](int c0, const char* oT) __attribute__((always_inline)) {
      const int nr = eos - c0 < BT ? eos - c0 : BT;
      if constexpr (NB == 2) {
        const int qq = mv * 64 + lane;
        const int row = qq / (BVW / 8), u = qq % (BVW / 8);
        if (row < nr)
          store_nt16(o + ((size_t)(c0 + row) * HV + j) * V + v0 + 8 * u,
                     *reinterpret_cast<const uint4*>(oT + row * OROW + 16 * u));
      } else {
        if (mr != 2) return;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int row = 8 * p + (lane >> 3), u = lane & 7;
          if (row < nr)
            store_nt16(o + ((size_t)(c0 + row) * HV + j) * V + v0 + 8 * u,
                       *reinterpret_cast<const uint4*>(oT + row * (2 * BVW) + ((u ^ ((row >> 3) & 7)) << 4)));
        }
      }
    };

    if (NC > 0) {
      dma_chunk(bos, (lchar*)sK0, (lchar*)sQ0, (lchar*)sT0, (lchar*)sAi0, (lchar*)sAq0, (lchar*)sV0,
                (lchar*)sG0, (lchar*)sD0);
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    auto chunk = [&](auto stg, int c) __attribute__((always_inline)) {
      constexpr bool S1 = decltype(stg)::value;
      const int c0 = bos + c * BT;
      if constexpr (DK == 128) __builtin_amdgcn_s_sleep(4);   // see the helper waves
      if (c > 0) store_o(c0 - BT, NB == 2 ? sO : (S1 ? sV0 : sV1));   // the previous chunk's tile
      if (c + 1 < NC) {
        if constexpr (S1)
          dma_chunk(c0 + BT, (lchar*)sK0, (lchar*)sQ0, (lchar*)sT0, (lchar*)sAi0, (lchar*)sAq0, (lchar*)sV0,
                    (lchar*)sG0, (lchar*)sD0);
        else
          dma_chunk(c0 + BT, (lchar*)sK1, (lchar*)sQ1, (lchar*)sT1, (lchar*)sAi1, (lchar*)sAq1, (lchar*)sV1,
                    (lchar*)sG1, (lchar*)sD1);
      }
      if (c + 2 < NC) touch_chunk(c0 + 2 * BT);
      lds_barrier();
      // this mover's loads of the next chunk (and its o store) are done;
      // vector-memory operations complete in issue order, so the L2 prefetch
      // loads issued after them may stay in flight
      if (c + 2 < NC) {
        static_assert(kTouches == 2, "vmcnt below");
        __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2) expcnt(7) lgkmcnt(15)
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      lds_barrier();
    };
    for (int c = 0; c < NC; c += 2) {
      chunk(Stage0{}, c);
      if (c + 1 < NC) chunk(Stage1{}, c + 1);
    }
    if (NC > 0) store_o(bos + (NC - 1) * BT, NB == 2 ? sO : (((NC - 1) & 1) ? sV1 : sV0));
  }
}

template <int DK, bool KDA, int NB>
hipError_t launch_dk(const ChunkArgs& a, const void* qop, const void* kop, const void* ktop,
                     const float* dg, hipStream_t s) {
  const int nvt = a.V / (16 * NB);
  const int G = KDA ? 1 : a.HV / a.Hk;        // v-heads per (sequence, q / k head) unit
  const int units = a.N * (a.HV / G);
  const int nblk = ((units + 7) / 8) * 8 * G * nvt;
  hipLaunchKernelGGL((gdn_scan_bf16_kernel<DK, KDA, NB>), dim3((unsigned)nblk), dim3(NTHR), 0, s, qop, kop,
                     (const f16_t*)ktop, (const bf16_t*)a.v, (const float*)a.GF, dg,
                     (const f16_t*)a.Ainv, (const f16_t*)a.Aqk, a.scale, a.h0, a.ht, a.hs, a.split_chunks,
                     a.hs_bf16 ? 1 : 0, a.hs_cap, (bf16_t*)a.o,
                     a.cu_seqlens, a.seq_order, a.chunk_off, a.T, a.B * a.T, (a.T + BT - 1) / BT, a.N,
                     a.Hk, a.HV, a.V, a.max_chunks);
  return hipGetLastError();
}

// compute units of the current device (queried once per device; calls from
// several host threads may race to fill the cache with the same value)
int cu_count() {
  static std::atomic<int> counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

hipError_t launch_scan_gdn_bf16(const ChunkArgs& a, hipStream_t s) {
  if (a.K == 128) {
    // One work-group per CU runs at a time.  When the 32-column work-groups
    // would not all fit at once, 64-column ones (four state waves) carry
    // twice the columns per CU through each chunk.
    const int G = a.HV / a.Hk;
    const long long wg32 = (long long)((a.N * (a.HV / G) + 7) / 8) * 8 * G * (a.V / 32);
    if (wg32 > cu_count()) return launch_dk<128, false, 4>(a, a.q, a.k, nullptr, nullptr, s);
    return launch_dk<128, false, 2>(a, a.q, a.k, nullptr, nullptr, s);
  }
  return launch_dk<64, false, 2>(a, a.q, a.k, nullptr, nullptr, s);
}

hipError_t launch_scan_kda_bf16(const ChunkArgs& a, const void* qg, const void* kg, const void* kt,
                                const float* dg, hipStream_t s) {
  if (a.K == 128) return launch_dk<128, true, 2>(a, qg, kg, kt, dg, s);
  return launch_dk<64, true, 2>(a, qg, kg, kt, dg, s);
}

}  // namespace gdn
