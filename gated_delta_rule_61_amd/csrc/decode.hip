// GDN decode over a bf16 state pool, gfx950.
//
// Follows "flashinfer gdn_kernels/gdn_decode_bf16_state.py" for what is
// computed (compute_single_gate; normalize_and_store_qk_to_smem; the decay /
// pred / v_delta / update / output sequence; state kept in fp32 across the
// T <= 4 tokens and written back to bf16 once).  The mapping is wave64-native
// rather than the page's 4 x 32-lane-warp layout:
//
//   one work-group of 256 threads per (batch row, v-head);
//   thread t owns key columns 8*(t%16) .. +7 of the 8 consecutive value rows
//   8*(t/16) .. +7, i.e. 64 fp32 state values in registers;
//   a 16-lane DPP row holds full 128-wide state rows, so pred = S k and
//   o = S q are 4-step in-row DPP reductions -- no LDS, no barriers;
//   every state load / store is a 16-byte access (a wave instruction covers
//   four whole 256-byte rows), v and o of a thread's rows are one 16-byte
//   access each, and all loads of the call are issued before any math.
//
// The state is streamed once per call (read 32 KiB, write 32 KiB per
// (row, head)); the kernel is HBM-bound.

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

template <int NTOK>
__global__ __launch_bounds__(256) void gdn_decode_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ ga,
    const bf16_t* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, bf16_t* __restrict__ state,
    const int32_t* __restrict__ idx, bf16_t* __restrict__ o,
    int H, int HV, int pool, float scale, float sp_beta, float sp_thr,
    int use_norm, float eps) {
  const int bh = blockIdx.x;
  const int bi = bh / HV;
  const int hv = bh - bi * HV;
  const int hk = hv / (HV / H);
  const int t = threadIdx.x;
  const int rg = t >> 4;   // row group: value rows 8*rg .. 8*rg + 7
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
      *reinterpret_cast<uint4*>(o + (tok * HV + hv) * DV + 8 * rg) = w;
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 w;
    w.x = pack_bf2(S[i][0], S[i][1]);
    w.y = pack_bf2(S[i][2], S[i][3]);
    w.z = pack_bf2(S[i][4], S[i][5]);
    w.w = pack_bf2(S[i][6], S[i][7]);
    *reinterpret_cast<uint4*>(sp + (size_t)i * DK) = w;
  }
}

template <int NTOK>
hipError_t launch_n(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.HV));
  hipLaunchKernelGGL(gdn_decode_kernel<NTOK>, grid, dim3(256), 0, s,
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
