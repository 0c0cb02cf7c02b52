// The scalar-gate intra-chunk step on its own, with w and u, gfx950.  Per
// chunk of 64 tokens and v-head, with G the chunk-local cumulative log-gate:
//
//   A = (I + L)^-1,  L_ts = beta_t (k_t . k_s) e^{G_t - G_s} for s < t
//   w = A diag(beta e^G) K          (64 x K)
//   u = A diag(beta) V              (64 x V)
//
// ("sglang srt/layers/attention/fla/chunk_fwd.py",
// chunk_gated_delta_rule_fwd_intra: the fused beta K K^T + solve, then
// recompute_w_u, which scales the k rows by beta e^G and the v rows by beta
// before the product with A.)  The prefill does not need this step: its scan
// forms Vn = A beta (V - e^G K S^T) = u - w S^T directly.
//
// gfx950 design: one wave per (chunk, v-head), as in the prefill's intra
// kernel:
//   * the ten lower 16 x 16 blocks of K K^T as MFMA straight from global
//     memory (bf16 16x16x32, fp32 io 16x16x4), gate / beta / mask on the
//     accumulators, forward substitution and block merge in LDS (fp32);
//   * A leaves as 16-byte rows in the io dtype;
//   * w and u, 32 columns at a time: the wave scales its k or v rows (lane =
//     token) and stages them in LDS as fp32, column-major ([column][token],
//     so the stores of a column and the operand reads of a 4-token slice
//     both hit distinct banks); the block-lower product with the fp32
//     inverse runs as fp32 MFMA (v_mfma_f32_16x16x4f32, both operands
//     exact); the 64 x 32 result goes back through the same tile into
//     16-byte row stores.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

using namespace intra;

constexpr int XT = 68;   // padded token column of the 32 x 64 staging tile

template <typename T, int DK>
__global__ __launch_bounds__(64) void gdn_intra_wu_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g, int g_cumulative,
    const float* __restrict__ beta, T* __restrict__ Aout, T* __restrict__ wout, T* __restrict__ uout,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ coff, int Tlen, int N, int NT, int nslots,
    int Hk, int HV, int DV) {
  __shared__ __attribute__((aligned(16))) float sA[BT][AP];
  __shared__ __attribute__((aligned(16))) float sX[32][XT];
  const int lane = threadIdx.x;
  int slot, j, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, j)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int jk = j / (HV / Hk);
  const int row = lane & 15, grp = lane >> 4;

  // gate and beta, lane = token (rows past the chunk end: no gate, beta 0)
  const int tl = lane < nrow ? lane : nrow - 1;
  const float g_raw = g ? g[(size_t)(c0 + tl) * HV + j] : 0.f;
  const float b_raw = beta[(size_t)(c0 + tl) * HV + j];
  const float gl = lane < nrow ? g_raw : 0.f;
  const float G = g_cumulative ? gl : wave_incl_scan(gl, lane);
  const float bl = lane < nrow ? b_raw : 0.f;

  // ---- the ten lower blocks of K K^T, one 32-channel slab at a time; rows
  // past the chunk end repeat its last row (they reach A only through beta 0)
  f32x4 KK[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) KK[t] = zero4();
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    Frag<T> kf[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 16 * rb + row < nrow ? 16 * rb + row : nrow - 1;
      load8(kf[rb], k + ((size_t)(c0 + r) * Hk + jk) * DK + 32 * s + 8 * grp);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) KK[tix(rb, cb)] = mma(kf[rb], kf[cb], KK[tix(rb, cb)]);
  }

  // ---- L = beta_r (k_r . k_s) e^{G_r - G_s}, s < r.  Lane holds rows
  // 16 rb + 4 grp + i, column 16 cb + row.
  float Gc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) Gc[cb] = __shfl(G, 16 * cb + row, 64);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * grp + i;
      const float Gr = __shfl(G, r, 64), Br = __shfl(bl, r, 64);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int s = 16 * cb + row;
        float val = 0.f;
        if (cb <= rb && s < r) val = Br * KK[tix(rb, cb < rb ? cb : rb)][i] * __expf(Gr - Gc[cb]);
        sA[r][s] = val;
      }
    }
  __syncthreads();
  solve_unit_lower_64<1>(sA, lane, 0);
  __syncthreads();
  store_tile<T>(sA, Aout, c0, nrow, HV, j, lane);

  // ---- w = A diag(beta e^G) K and u = A diag(beta) V, 32 columns at a time
  auto product = [&](const T* src, size_t src_row, int cols, float f, T* dst, size_t dst_row) {
    for (int c = 0; c < cols; c += 32) {
      __syncthreads();                       // the last readers of sX are done
      // this lane's token row, 32 values, scaled (f = 0 past the chunk end)
      const T* p = src + (size_t)(c0 + tl) * src_row + c;
#pragma unroll
      for (int e8 = 0; e8 < 4; ++e8) {
        Frag<T> x;
        load8(x, p + 8 * e8);
#pragma unroll
        for (int e = 0; e < 8; ++e) sX[8 * e8 + e][lane] = x.get(e) * f;
      }
      __syncthreads();
      f32x4 acc[4][2];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb][0] = zero4();
        acc[rb][1] = zero4();
        // only tokens t < 16 (rb + 1) reach the rows of block rb (A is block
        // lower triangular)
#pragma unroll
        for (int kk = 0; kk < 4 * (rb + 1); ++kk) {
          const float a = sA[16 * rb + row][4 * kk + grp];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sX[16 * cb + row][4 * kk + grp], acc[rb][cb],
                                                               0, 0, 0);
        }
      }
      __syncthreads();                       // every operand read is done
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sX[16 * cb + row][16 * rb + 4 * grp + i] = acc[rb][cb][i];
      __syncthreads();
      if (lane < nrow) {
        T* q = dst + (size_t)(c0 + lane) * dst_row + c;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e8 = 0; e8 < 4; ++e8) {
            uint4 o;
            o.x = pack2<T>(sX[8 * e8 + 0][lane], sX[8 * e8 + 1][lane]);
            o.y = pack2<T>(sX[8 * e8 + 2][lane], sX[8 * e8 + 3][lane]);
            o.z = pack2<T>(sX[8 * e8 + 4][lane], sX[8 * e8 + 5][lane]);
            o.w = pack2<T>(sX[8 * e8 + 6][lane], sX[8 * e8 + 7][lane]);
            *reinterpret_cast<uint4*>(q + 8 * e8) = o;
          }
        } else {
#pragma unroll
          for (int e4 = 0; e4 < 8; ++e4)
            *reinterpret_cast<float4*>(q + 4 * e4) = make_float4(sX[4 * e4][lane], sX[4 * e4 + 1][lane],
                                                                 sX[4 * e4 + 2][lane], sX[4 * e4 + 3][lane]);
        }
      }
    }
  };
  if (wout) product(k + (size_t)jk * DK, (size_t)Hk * DK, DK, bl * __expf(G), wout + (size_t)j * DK, (size_t)HV * DK);
  if (uout) product(v + (size_t)j * DV, (size_t)HV * DV, DV, bl, uout + (size_t)j * DV, (size_t)HV * DV);
}

template <typename T, int DK>
hipError_t launch_t(const IntraArgs& a, hipStream_t s, int NT, int nslots) {
  hipLaunchKernelGGL((gdn_intra_wu_kernel<T, DK>), dim3(intra_blocks(nslots, a.HV)), dim3(64), 0, s,
                     (const T*)a.k, (const T*)a.v, a.g, a.g_cumulative ? 1 : 0, a.beta, (T*)a.A, (T*)a.w,
                     (T*)a.u, a.cu_seqlens, a.chunk_off, a.T, a.N, NT, nslots, a.Hk, a.HV, a.V);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_intra_wu(const IntraArgs& a, hipStream_t s) {
  const int NT = (a.T + 63) / 64;
  const int nslots = a.cu_seqlens ? NT + a.N : a.B * NT;
  if (nslots <= 0 || (long long)a.B * a.T <= 0) return hipSuccess;
  if (a.bf16) return a.K == 128 ? launch_t<bf16_t, 128>(a, s, NT, nslots) : launch_t<bf16_t, 64>(a, s, NT, nslots);
  return a.K == 128 ? launch_t<float, 128>(a, s, NT, nslots) : launch_t<float, 64>(a, s, NT, nslots);
}

}  // namespace gdn
