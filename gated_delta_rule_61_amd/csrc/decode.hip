// GDN decode over a bf16 state pool, gfx950.
//
// Follows "flashinfer gdn_kernels/gdn_decode_bf16_state.py" for what is
// computed (compute_single_gate; normalize_and_store_qk_to_smem; the decay /
// pred / v_delta / update / output sequence; state kept in fp32 across the
// T <= 4 tokens and written back to bf16 once).  The mapping is wave64-native
// rather than the page's 4 x 32-lane-warp layout:
//
//   one work-group of 256 threads per (batch row, v-head), or, with fewer
//   pairs than CUs, four work-groups of 64 threads (32 value rows each;
//   value rows are independent);
//   thread t owns key columns 8*(t%16) .. +7 of the 8 consecutive value rows
//   8*(t/16) .. +7, i.e. 64 fp32 state values in registers;
//   a 16-lane DPP row holds full 128-wide state rows, so pred = S k and
//   o = S q are 4-step in-row DPP reductions -- no LDS, no barriers;
//   every state load / store is a 16-byte access (a wave instruction covers
//   four whole 256-byte rows), v and o of a thread's rows are one 16-byte
//   access each, and all loads of the call are issued before any math.
//
// The state is streamed once per call (read 32 KiB, write 32 KiB per
// (row, head)); the kernel is HBM-bound.  That per-token kernel runs T = 1;
// T = 2 .. 4 run the MFMA form further below, which replaces the T
// sequential rank-1 steps by one pass of products over the state.

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int DK = 128;  // key dim
constexpr int DV = 128;  // value dim

__device__ __forceinline__ void unpack8(const uint4& r, float (&f)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __builtin_bit_cast(float, w[e] << 16);
    f[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
  }
}

template <int NTOK, int TPB>
__global__ __launch_bounds__(TPB) void gdn_decode_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ ga,
    const bf16_t* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, bf16_t* __restrict__ state,
    const int32_t* __restrict__ idx, bf16_t* __restrict__ o,
    int H, int HV, int pool, float scale, float sp_beta, float sp_thr,
    int use_norm, float eps) {
  constexpr int SPL = 256 / TPB;   // work-groups per (batch row, v-head)
  const int bh = blockIdx.x / SPL;
  const int part = blockIdx.x - bh * SPL;
  const int bi = bh / HV;
  const int hv = bh - bi * HV;
  const int hk = hv / (HV / H);
  const int t = threadIdx.x;
  const int rg = part * (TPB / 16) + (t >> 4);   // row group: value rows 8*rg .. 8*rg + 7
  const int cl = t & 15;   // key columns 8*cl .. 8*cl + 7
  const int slot = idx ? idx[bi] : bi;
  const bool valid = slot >= 0 && slot < pool;

  // Issue every load of the call up front (state first), keep raw bits.
  bf16_t* sp = state + ((size_t)(valid ? slot : 0) * HV + hv) * (size_t)(DV * DK) +
               (size_t)(8 * rg) * DK + 8 * cl;
  uint4 raw[8];
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(sp + (size_t)i * DK);
  }
  uint4 qr[NTOK], kr[NTOK], vr[NTOK];
#pragma unroll
  for (int tt = 0; tt < NTOK; ++tt) {
    const size_t tok = (size_t)bi * NTOK + tt;
    qr[tt] = *reinterpret_cast<const uint4*>(q + (tok * H + hk) * DK + 8 * cl);
    kr[tt] = *reinterpret_cast<const uint4*>(k + (tok * H + hk) * DK + 8 * cl);
    vr[tt] = *reinterpret_cast<const uint4*>(v + (tok * HV + hv) * DV + 8 * rg);
  }

  if (!valid) {
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      const size_t tok = (size_t)bi * NTOK + tt;
      if (cl == 0) *reinterpret_cast<uint4*>(o + (tok * HV + hv) * DV + 8 * rg) = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const float A = -expf(A_log[hv]);
  const float bias = dt_bias[hv];

  float S[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(raw[i], S[i]);

#pragma unroll
  for (int tt = 0; tt < NTOK; ++tt) {
    const size_t tok = (size_t)bi * NTOK + tt;
    // gate (compute_single_gate): softplus with threshold, then exp
    const float x = bf2f(ga[tok * HV + hv]) + bias;
    const float bx = sp_beta * x;
    const float spv = (bx <= sp_thr) ? log1pf(expf(bx)) / sp_beta : x;
    const float alpha = expf(A * spv);
    const float beta = 1.0f / (1.0f + expf(-bf2f(gb[tok * HV + hv])));

    float qq[8], kk[8], vv[8];
    unpack8(qr[tt], qq);
    unpack8(kr[tt], kk);
    unpack8(vr[tt], vv);
    float qs = scale, ks = 1.0f;
    if (use_norm) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq = fmaf(qq[e], qq[e], sq);
        sk = fmaf(kk[e], kk[e], sk);
      }
      sq = row16_sum(sq);
      sk = row16_sum(sk);
      qs = scale / sqrtf(sq + eps);
      ks = 1.0f / sqrtf(sk + eps);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qq[e] *= qs;
      kk[e] *= ks;
    }

    // decay, pred = S k (16-lane row reduction)
    float pred[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        S[i][e] *= alpha;
        p = fmaf(S[i][e], kk[e], p);
      }
      pred[i] = p;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) pred[i] = row16_sum(pred[i]);

    // delta update and output o = S q
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = beta * (vv[i] - pred[i]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        S[i][e] = fmaf(d, kk[e], S[i][e]);
        acc = fmaf(S[i][e], qq[e], acc);
      }
      out[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = row16_sum(out[i]);
    if (cl == 0) {
      uint4 w;
      w.x = pack_bf2(out[0], out[1]);
      w.y = pack_bf2(out[2], out[3]);
      w.z = pack_bf2(out[4], out[5]);
      w.w = pack_bf2(out[6], out[7]);
      store_nt16(o + (tok * HV + hv) * DV + 8 * rg, w);
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 w;
    w.x = pack_bf2(S[i][0], S[i][1]);
    w.y = pack_bf2(S[i][2], S[i][3]);
    w.z = pack_bf2(S[i][4], S[i][5]);
    w.w = pack_bf2(S[i][6], S[i][7]);
    store_nt16(sp + (size_t)i * DK, w);
  }
}

// ---------------------------------------------------------------------------
// MFMA form for T = 1 .. 4 tokens.  With G_t = alpha_1 ... alpha_t and
// R_st = G_t / G_s = alpha_{s+1} ... alpha_t (a product, never a quotient),
// the T sequential steps close up as
//
//   w_t = beta_t (v_t - G_t S0 k_t - sum_{s<t} R_st (k_s . k_t) w_s)
//   o_t = G_t S0 q_t + sum_{s<=t} R_st (k_s . q_t) w_s
//   S_T = G_T S0 + sum_s R_sT w_s k_s^T
//
// (the same recurrence unrolled; q and k normalised, q scaled).  One bf16
// MFMA pass over the raw state gives S0 [k_1..k_T q_1..q_T] for every state
// row, a second the Gram matrix of the raw q / k rows (their norms and the
// dot products), the T-step solve runs per state row inside one lane, and a
// fp32 MFMA applies the rank-T update S_T^T = G_T S0^T + K W^T.
//
// Work-group = one (batch row, v-head), 4 waves, or (small batches) one of
// its waves; wave w owns state rows 32w .. 32w + 31 as two 16-row blocks rb
// and shares nothing with the other waves.  Lane (n, g) = (lane % 16,
// lane / 16) holds, for 32-channel block kb, the 8 bf16 state values
// S0[32w + 16rb + n][32kb + 8g .. + 7] (one 16-byte LDS read; the state
// reaches LDS in whole rows): the B operand of the bf16 16x16x32 product
// (k-slots 8g + e, column n).  The update writes them back from two
// 16 x 16 accumulator blocks of S^T whose rows are the channels
// 32kb + 8 (r / 4) + (r % 4) and the same + 4, so that accumulator lane
// (n, g) holds exactly the lane's 8 values again.
typedef short v8i16 __attribute__((ext_vector_type(8)));

// 16 bytes as a plain vector (a copy of HIP's uint4 struct between memory
// spaces becomes a memcpy that keeps arrays of them out of registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma32_bf(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float from_lane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * l, __builtin_bit_cast(int, x)));
}

// At most 128 VGPRs, so that 4 work-groups share a CU (144 without the cap,
// 3 per CU; the cap costs no spills, and the fourth work-group hides more of
// each one's load latency: -4 % at T = 4).
template <int NTOK, int WPB>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(4))) void gdn_decode_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ ga,
    const bf16_t* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, bf16_t* __restrict__ state,
    const int32_t* __restrict__ idx, bf16_t* __restrict__ o,
    int H, int HV, int pool, float scale, float sp_beta, float sp_thr,
    int use_norm, float eps) {
  constexpr int KB = DK / 32;
  // the state rows of the work-group's waves, bf16: rows 16 lw + r of each
  // wave's two 16-row blocks (block 0 in sS0, block 1 in sS1)
  __shared__ uint4 sS0[WPB * 16 * DK / 8], sS1[WPB * 16 * DK / 8];
  constexpr int SPL = 4 / WPB;   // work-groups per (batch row, v-head)
  const int bh = blockIdx.x / SPL;
  const int bi = bh / HV;
  const int hv = bh - bi * HV;
  const int hk = hv / (HV / H);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int lw = threadIdx.x >> 6;                        // wave in the work-group
  const int wv = (blockIdx.x - bh * SPL) * WPB + lw;      // wave of the (row, head)
  const int row0 = 32 * wv;
  const int slot = idx ? idx[bi] : bi;
  const size_t tok0 = (size_t)bi * NTOK;

  if (slot < 0 || slot >= pool) {   // o = 0, the pool is not touched
    if (g == 0) {
#pragma unroll
      for (int tt = 0; tt < NTOK; ++tt)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) o[((tok0 + tt) * HV + hv) * DV + row0 + 16 * rb + n] = 0;
    }
    return;
  }

  // ---- the small loads first: the A operand rows (j = n < 4 -> k of token
  // j, 4 <= j < 8 -> q of token j - 4, other rows zero; loads of row j are
  // clamped to a valid token, then masked), k at the update's channel rows
  // (lane (n, g): token g at the channels of accumulator row n of the two
  // blocks h = 0, 1 of channel block kb), v of the lane's two state rows,
  // and the gate inputs of token lane % 4
  const int jt = n & 3;
  const bool jv = n < 8 && jt < NTOK;
  const bf16_t* srcj = (n < 4 ? k : q) + ((tok0 + (jt < NTOK ? jt : 0)) * H + hk) * DK + 8 * g;
  uint4 kq[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) kq[kb] = *reinterpret_cast<const uint4*>(srcj + 32 * kb);
  const bool gv = g < NTOK;
  const bf16_t* srcg = k + ((tok0 + (gv ? g : 0)) * H + hk) * DK + 8 * (n >> 2) + (n & 3);
  bf16_t kc[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) kc[kb][h] = srcg[32 * kb + 4 * h];
  bf16_t vr[2][NTOK];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) vr[rb][tt] = v[((tok0 + tt) * HV + hv) * DV + row0 + 16 * rb + n];
  const int tl = (lane & 3) < NTOK ? (lane & 3) : 0;
  const bf16_t ga_r = ga[(tok0 + tl) * HV + hv], gb_r = gb[(tok0 + tl) * HV + hv];

  // ---- then the wave's 32 state rows in whole rows, in two 16-row blocks:
  // lane l of load i covers row 4i + l / 16 of the block, 16-byte unit u =
  // (l % 16) ^ (row % 16), stored in LDS slot l % 16, so that the fragment
  // reads (16 rows at one unit) hit distinct banks.  Block 0 goes straight
  // to LDS; block 1 into registers, written to LDS after block 0's math (an
  // LDS read after a direct-to-LDS load waits for every such load in flight).
  bf16_t* sp = state + ((size_t)slot * HV + hv) * (size_t)(DV * DK);
  {
    typedef __attribute__((address_space(1))) const void gvoid;
    typedef __attribute__((address_space(3))) char lchar;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 4 * i + (lane >> 4);
      const int u = (lane & 15) ^ (r & 15);
      __builtin_amdgcn_global_load_lds((gvoid*)(sp + (size_t)r * DK + 8 * u),
                                       (lchar*)(sS0 + (16 * lw + 4 * i) * 16), 16, 0, 0);
    }
  }

  // ---- gates (compute_single_gate: softplus with threshold, then exp),
  // one token per lane, then broadcast; hardware exp / log (a few ulp of
  // fp32, far below the bf16 state's rounding)
  float alpha[NTOK], beta[NTOK];
  {
    const float x = bf2f(ga_r) + dt_bias[hv];
    const float bx = sp_beta * x;
    const float spv = (bx <= sp_thr) ? __logf(1.0f + __expf(bx)) / sp_beta : x;
    const float al = __expf(-__expf(A_log[hv]) * spv);
    const float be = 1.0f / (1.0f + __expf(-bf2f(gb_r)));
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      alpha[tt] = lane_f(al, tt);
      beta[tt] = lane_f(be, tt);
    }
  }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    if (!jv) kq[kb] = make_uint4(0u, 0u, 0u, 0u);

  // ---- Gram matrix of the raw rows (fp32 accumulation of exact bf16
  // products).  Accumulator lane (n, g) holds row 4g + i, column n.
  f32x4 Gm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) Gm = mma32_bf(kq[kb], kq[kb], Gm);

  // ---- per-call scalars: norms, normalised dot products, decay products
  float ks[NTOK], qs[NTOK], kk[NTOK][NTOK], kqd[NTOK][NTOK];
  {
    // lane t < 4 holds Gram[t][t] in reg t, lane 20 + t Gram[4 + t][4 + t]
    // in reg t: one inverse norm per lane, then broadcast
    const int r = lane & 3;
    const float sq = r == 0 ? Gm[0] : r == 1 ? Gm[1] : r == 2 ? Gm[2] : Gm[3];
    const float inv = 1.0f / sqrtf(sq + eps);
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      ks[tt] = use_norm ? lane_f(inv, tt) : 1.0f;
      qs[tt] = use_norm ? scale * lane_f(inv, 20 + tt) : scale;
    }
  }
  {
    // lane t < 4 holds Gram[s][t] (reg s), lane 4 + t holds Gram[s][4 + t]:
    // each lane scales its column, then broadcast
    const int c = lane & 3;
    float cs = 0.f;
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) cs = c == tt ? (lane & 4 ? qs[tt] : ks[tt]) : cs;
#pragma unroll
    for (int s2 = 0; s2 < NTOK; ++s2) {
      const float x = Gm[s2] * (ks[s2] * cs);
#pragma unroll
      for (int tt = 0; tt < NTOK; ++tt) {
        kk[s2][tt] = lane_f(x, tt);
        kqd[s2][tt] = lane_f(x, 4 + tt);
      }
    }
  }
  float Gt[NTOK], Rst[NTOK][NTOK];   // G_t; R_st = alpha_{s+1} .. alpha_t
#pragma unroll
  for (int tt = 0; tt < NTOK; ++tt) {
    Gt[tt] = tt == 0 ? alpha[0] : Gt[tt - 1] * alpha[tt];
    Rst[tt][tt] = 1.0f;
#pragma unroll
    for (int s2 = tt - 1; s2 >= 0; --s2) Rst[s2][tt] = Rst[s2 + 1][tt] * alpha[s2 + 1];
  }

  // ---- the update's constant operands.  S_T^T = G_T S0^T + K W^T:
  // S0^T comes out of a bf16 MFMA of the raw state fragments with a 0 / 1
  // selector (block h's A row r picks k-slot 8 (r / 4) + 4h + r % 4 of the
  // 32-channel block; exact), scaled by G_T in fp32; K W^T is an fp32 MFMA
  // (16x16x4: lane (n, g) holds the A element [channel row n][token g] and
  // the B element [token g][row n]).
  float ksg = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < NTOK; ++s2) ksg = g == s2 ? ks[s2] : ksg;
  const float GT = Gt[NTOK - 1];
  uint4 sel[2];   // [h]: bf16 1.0 in the selected slot
  {
    constexpr uint32_t kOne = 0x3F80u;   // bf16 1.0
    const bool on = g == (n >> 2);
    const int e = n & 3;   // slot 4h + e of the lane's 8
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wds[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int e0 = 2 * d - 4 * h;   // slots 2d, 2d + 1 relative to 4h
        wds[d] = (on && e0 == (e & ~1)) ? (kOne << (16 * (e & 1))) : 0u;
      }
      sel[h] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
  }
  float ak[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) ak[kb][h] = gv ? bf2f(kc[kb][h]) * ksg : 0.f;

  // ---- one 16-row block: S0 [k | q] (accumulator lane (n, g): row 4g + i
  // of [k | q], state row n), the deltas w_t (valid in lanes g = 0, sent to
  // all lanes of the row), o_t (lanes g = 1, returned), the rank-T update
  // written back over the block's LDS rows.  `mid` runs once the block's
  // fragments have been read.
  auto block = [&](int rb, uint4* sb, float (&ov)[NTOK], auto mid) __attribute__((always_inline)) {
    // lane (n, g) of channel block kb: S0[row][32kb + 8g .. + 7]
    auto frag = [&](int kb) __attribute__((always_inline)) -> uint4& {
      return sb[(16 * lw + n) * 16 + ((4 * kb + g) ^ n)];
    };
    uint4 fr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) fr[kb] = frag(kb);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) P = mma32_bf(kq[kb], fr[kb], P);
    float wv2[NTOK], wa[NTOK];
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      float d = bf2f(vr[rb][tt]) - Gt[tt] * (P[tt] * ks[tt]);
#pragma unroll
      for (int s2 = 0; s2 < tt; ++s2) d -= Rst[s2][tt] * kk[s2][tt] * wv2[s2];
      wv2[tt] = beta[tt] * d;
    }
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) wa[tt] = from_lane(wv2[tt], n);
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      float ot = Gt[tt] * (P[tt] * qs[tt]);
#pragma unroll
      for (int s2 = 0; s2 <= tt; ++s2) ot += Rst[s2][tt] * kqd[s2][tt] * wa[s2];
      ov[tt] = ot;
    }
    float bu = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NTOK; ++s2) bu = g == s2 ? Rst[s2][NTOK - 1] * wa[s2] : bu;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 r = fr[kb];
      uint32_t out[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 c = mma32_bf(sel[h], r, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] *= GT;
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kb][h], bu, c, 0, 0, 0);
        out[2 * h] = pack_bf2(c[0], c[1]);
        out[2 * h + 1] = pack_bf2(c[2], c[3]);
      }
      frag(kb) = make_uint4(out[0], out[1], out[2], out[3]);
    }
  };
  // a block's rows back to the pool in whole rows (16-byte unit u of row r
  // from slot u ^ (r % 16)), and its o values
  auto store_block = [&](int rb, const uint4* sb, const float (&ov)[NTOK]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 4 * i + (lane >> 4);   // row within the block
      const int u = lane & 15;
      store_nt16(sp + (size_t)(row0 + 16 * rb + rl) * DK + 8 * u, sb[(16 * lw + rl) * 16 + (u ^ rl)]);
    }
    if (g == 1) {
#pragma unroll
      for (int tt = 0; tt < NTOK; ++tt) o[((tok0 + tt) * HV + hv) * DV + row0 + 16 * rb + n] = f2bf(ov[tt]);
    }
  };

  // block 1's rows are loaded into registers once block 0's fragments are
  // read (the wait before those reads covers every load in flight), so
  // they arrive during block 0's math
  float ov0[NTOK], ov1[NTOK];
  u32x4 raw1[4];
  block(0, sS0, ov0, [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 16 + 4 * i + (lane >> 4);
      const int u = (lane & 15) ^ (r & 15);
      raw1[i] = *reinterpret_cast<const u32x4*>(sp + (size_t)r * DK + 8 * u);
    }
  });
#pragma unroll
  for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4*>(sS1)[(16 * lw + 4 * i) * 16 + lane] = raw1[i];
  store_block(0, sS0, ov0);
  block(1, sS1, ov1, []() {});
  store_block(1, sS1, ov1);
}

// With fewer (batch row, v-head) pairs than the 256 CUs, each pair is split
// over four 64-thread work-groups (measured: -5 % at B = 1, T = 1 and -12 %
// at B = 1, T = 4 with 32 v-heads; no gain from 16 rows of 32 v-heads on).
constexpr long long kSplitBelow = 256;   // (batch row, v-head) pairs

// T = 1 runs the per-token kernel (the rank-1 step has no products worth
// MFMA work and its loads / stores cover whole rows); T = 2 .. 4 the MFMA form.
template <int NTOK>
hipError_t launch_n(const DecodeArgs& a, hipStream_t s) {
  const bool split = (long long)a.B * a.HV < kSplitBelow;
  const dim3 grid((unsigned)(a.B * a.HV * (split ? 4 : 1)));
  void (*kern)(const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*,
               const float*, const float*, bf16_t*, const int32_t*, bf16_t*, int, int, int,
               float, float, float, int, float);
  if constexpr (NTOK == 1)
    kern = split ? gdn_decode_kernel<1, 64> : gdn_decode_kernel<1, 256>;
  else
    kern = split ? gdn_decode_mfma_kernel<NTOK, 1> : gdn_decode_mfma_kernel<NTOK, 4>;
  hipLaunchKernelGGL(kern, grid, dim3(split ? 64 : 256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
                     (const bf16_t*)a.a, (const bf16_t*)a.b, a.A_log, a.dt_bias,
                     (bf16_t*)a.state, a.idx, (bf16_t*)a.o, a.H, a.HV, a.pool,
                     a.scale, a.sp_beta, a.sp_thr, a.use_norm, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (a.T) {
    case 1: return launch_n<1>(a, s);
    case 2: return launch_n<2>(a, s);
    case 3: return launch_n<3>(a, s);
    default: return launch_n<4>(a, s);
  }
}

}  // namespace gdn
