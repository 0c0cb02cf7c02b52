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
//   * bf16 io: w and u as fp16 MFMA (16x16x32) of the fp16-rounded inverse
//     and the fp16-rounded scaled rows (the page rounds both to bf16; fp16's
//     2^-11 keeps the products within the bf16 storage error at any length).
//     The k fragments of K K^T stay in registers and are reused; the v
//     fragments are loaded after the solve and arrive while w is formed.
//     The inverse's six nonzero 16 x 32 operand blocks sit in registers,
//     which frees the fp32 tile: the transposed staging tile of 64 scaled
//     columns ([column][token], fp16) takes its place in
//     LDS, 17 KB per wave in all.  The products run transposed (X^T A^T),
//     so each lane ends with four consecutive columns of one token row:
//     8-byte stores, no staging of the result.
//   * fp32 io: w and u 32 columns at a time: the wave scales its k or v rows
//     (lane = token) and stages them in LDS as fp32, column-major ([column]
//     [token], so the stores of a column and the operand reads of a 4-token
//     slice both hit distinct banks); the block-lower product with the fp32
//     inverse runs as fp32 MFMA (v_mfma_f32_16x16x4f32, both operands
//     exact); the 64 x 32 result goes back through the same tile into
//     16-byte row stores.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

using namespace intra;

constexpr int XT = 68;   // padded token column of the fp32 32 x 64 staging tile
constexpr int XP = 72;   // padded token row of the fp16 64 x 64 staging tile (144 B)

// Gate scan (G and beta, lane = token, zero past the chunk end), the ten
// lower blocks of K K^T, L = beta_r (k_r . k_s) e^{G_r - G_s} (s < r), its
// unit lower inverse in sA, and A stored.  The k fragments stay in kf (lane
// holds K[16 rb + row][32 s + 8 grp .. + 8], rows past the chunk end repeat
// its last row: they reach A, w and u only through beta 0).
template <typename T, int DK>
__device__ __forceinline__ void intra_inverse(const T* __restrict__ k, const float* __restrict__ g, int g_cumulative,
                                              const float* __restrict__ beta, T* __restrict__ Aout,
                                              float (*sA)[AP], Frag<T> (&kf)[DK / 32][4], int c0, int nrow,
                                              int Hk, int HV, int j, int jk, int lane, float& G, float& bl) {
  const int row = lane & 15, grp = lane >> 4;
  const int tl = lane < nrow ? lane : nrow - 1;
  const float g_raw = g ? g[(size_t)(c0 + tl) * HV + j] : 0.f;
  const float b_raw = beta[(size_t)(c0 + tl) * HV + j];
  const float gl = lane < nrow ? g_raw : 0.f;
  G = g_cumulative ? gl : wave_incl_scan(gl, lane);
  bl = lane < nrow ? b_raw : 0.f;

  f32x4 KK[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) KK[t] = zero4();
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 16 * rb + row < nrow ? 16 * rb + row : nrow - 1;
      load8(kf[s][rb], k + ((size_t)(c0 + r) * Hk + jk) * DK + 32 * s + 8 * grp);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) KK[tix(rb, cb)] = mma(kf[s][rb], kf[s][cb], KK[tix(rb, cb)]);
  }

  // lane holds rows 16 rb + 4 grp + i, column 16 cb + row
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
}

// fp32 io
template <int DK>
__global__ __launch_bounds__(64) void gdn_intra_wu_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ g, int g_cumulative,
    const float* __restrict__ beta, float* __restrict__ Aout, float* __restrict__ wout, float* __restrict__ uout,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ coff, int Tlen, int N, int NT, int nslots,
    int Hk, int HV, int DV) {
  using T = float;
  __shared__ __attribute__((aligned(16))) float sA[BT][AP];
  __shared__ __attribute__((aligned(16))) float sX[32][XT];
  const int lane = threadIdx.x;
  int slot, j, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, j)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int jk = j / (HV / Hk);
  const int row = lane & 15, grp = lane >> 4;
  const int tl = lane < nrow ? lane : nrow - 1;
  float G, bl;
  {
    Frag<T> kf[DK / 32][4];
    intra_inverse<T, DK>(k, g, g_cumulative, beta, Aout, sA, kf, c0, nrow, Hk, HV, j, jk, lane, G, bl);
  }

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
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4)
          *reinterpret_cast<float4*>(q + 4 * e4) = make_float4(sX[4 * e4][lane], sX[4 * e4 + 1][lane],
                                                               sX[4 * e4 + 2][lane], sX[4 * e4 + 3][lane]);
      }
    }
  };
  if (wout) product(k + (size_t)jk * DK, (size_t)Hk * DK, DK, bl * __expf(G), wout + (size_t)j * DK, (size_t)HV * DK);
  if (uout) product(v + (size_t)j * DV, (size_t)HV * DV, DV, bl, uout + (size_t)j * DV, (size_t)HV * DV);
}

// index of the inverse's nonzero 16 x 32 operand block (rb, kk), kk <= rb / 2
__host__ __device__ constexpr int apair(int rb, int kk) { return rb < 2 ? rb : 2 * rb - 2 + kk; }

// Columns 64 H .. 64 H + 63 of w or u for bf16 io: the wave's scaled
// fragments (lane holds X[16 rb + row][32 s + 8 grp .. + 8] of slab s, scale
// f[rb] for its token) go to the staging tile as fp16, column-major; then,
// per 16-column block cb and token block rb, out^T = X^T A^T over the two
// 32-token halves kk (only kk <= rb / 2 meet nonzero entries of A).
template <int H, int NS>
__device__ __forceinline__ void wu_half(const Frag<bf16_t> (&src)[NS][4], const float (&f)[4],
                                        const Frag<f16_t> (&af)[6], uint16_t (*sX)[XP], bf16_t* __restrict__ dst,
                                        size_t dst_row, int c0, int nrow, int lane) {
  const int row = lane & 15, grp = lane >> 4;
  __syncthreads();                           // the last readers of the tile are done
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sX[32 * sl + 8 * grp + e][16 * rb + row] =
            __builtin_bit_cast(uint16_t, from_f<f16_t>(src[2 * H + sl][rb].get(e) * f[rb]));
  __syncthreads();
  Frag<f16_t> xf[4][2];                      // lane holds X[32 kk + 8 grp .. + 8][16 cb + row]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      xf[cb][kk].v = *reinterpret_cast<const f16x8*>(&sX[16 * cb + row][32 * kk + 8 * grp]);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int t = 16 * rb + row;             // this lane's token of the result
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 acc = mma(xf[cb][0], af[apair(rb, 0)], zero4());
      if (rb >= 2) acc = mma(xf[cb][1], af[apair(rb, 1)], acc);
      // acc[i] = out[t][16 cb + 4 grp + i]
      if (t < nrow)
        *reinterpret_cast<uint2*>(dst + (size_t)(c0 + t) * dst_row + 16 * cb + 4 * grp) =
            uint2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
    }
  }
}

// bf16 io
template <int DK, int DV>
__global__ __launch_bounds__(64) void gdn_intra_wu_bf16_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ g, int g_cumulative,
    const float* __restrict__ beta, bf16_t* __restrict__ Aout, bf16_t* __restrict__ wout, bf16_t* __restrict__ uout,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ coff, int Tlen, int N, int NT, int nslots,
    int Hk, int HV) {
  // the fp32 inverse, then (once its operand blocks are in registers) the
  // fp16 staging tile in the same bytes
  __shared__ __attribute__((aligned(16))) union {
    float a[BT][AP];
    uint16_t x[64][XP];
  } sm;
  const int lane = threadIdx.x;
  int slot, j, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, j)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int jk = j / (HV / Hk);
  const int row = lane & 15, grp = lane >> 4;

  Frag<bf16_t> kf[DK / 32][4];
  float G, bl;
  intra_inverse<bf16_t, DK>(k, g, g_cumulative, beta, Aout, sm.a, kf, c0, nrow, Hk, HV, j, jk, lane, G, bl);
  if (!wout && !uout) return;
  // the v fragments arrive while w is formed
  Frag<bf16_t> vf[DV / 32][4];
  if (uout) {
#pragma unroll
    for (int s = 0; s < DV / 32; ++s)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int r = 16 * rb + row < nrow ? 16 * rb + row : nrow - 1;
        load8(vf[s][rb], v + ((size_t)(c0 + r) * HV + j) * DV + 32 * s + 8 * grp);
      }
  }

  // B operands of the products: lane holds A[16 rb + row][32 kk + 8 grp .. + 8]
  Frag<f16_t> af[6];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int kk = 0; kk <= rb / 2; ++kk) {
      const float* a = &sm.a[16 * rb + row][32 * kk + 8 * grp];
      const uint4 pk{pack2<f16_t>(a[0], a[1]), pack2<f16_t>(a[2], a[3]), pack2<f16_t>(a[4], a[5]),
                     pack2<f16_t>(a[6], a[7])};
      af[apair(rb, kk)].v = __builtin_bit_cast(f16x8, pk);
    }

  // per-token scales of the rows: beta e^G for k, beta for v (0 past the end)
  float fk[4], fv[4];
  const float bg = bl * __expf(G);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    fk[rb] = __shfl(bg, 16 * rb + row, 64);
    fv[rb] = __shfl(bl, 16 * rb + row, 64);
  }
  if (wout) {
    bf16_t* w0 = wout + (size_t)j * DK;
    wu_half<0>(kf, fk, af, sm.x, w0, (size_t)HV * DK, c0, nrow, lane);
    if constexpr (DK == 128) wu_half<1>(kf, fk, af, sm.x, w0 + 64, (size_t)HV * DK, c0, nrow, lane);
  }
  if (uout) {
    bf16_t* u0 = uout + (size_t)j * DV;
    wu_half<0>(vf, fv, af, sm.x, u0, (size_t)HV * DV, c0, nrow, lane);
    if constexpr (DV == 128) wu_half<1>(vf, fv, af, sm.x, u0 + 64, (size_t)HV * DV, c0, nrow, lane);
  }
}

template <int DK>
hipError_t launch_f32(const IntraArgs& a, hipStream_t s, int NT, int nslots) {
  hipLaunchKernelGGL((gdn_intra_wu_f32_kernel<DK>), dim3(intra_blocks(nslots, a.HV)), dim3(64), 0, s,
                     (const float*)a.k, (const float*)a.v, a.g, a.g_cumulative ? 1 : 0, a.beta, (float*)a.A,
                     (float*)a.w, (float*)a.u, a.cu_seqlens, a.chunk_off, a.T, a.N, NT, nslots, a.Hk, a.HV, a.V);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bf16(const IntraArgs& a, hipStream_t s, int NT, int nslots) {
  hipLaunchKernelGGL((gdn_intra_wu_bf16_kernel<DK, DV>), dim3(intra_blocks(nslots, a.HV)), dim3(64), 0, s,
                     (const bf16_t*)a.k, (const bf16_t*)a.v, a.g, a.g_cumulative ? 1 : 0, a.beta, (bf16_t*)a.A,
                     (bf16_t*)a.w, (bf16_t*)a.u, a.cu_seqlens, a.chunk_off, a.T, a.N, NT, nslots, a.Hk, a.HV);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_intra_wu(const IntraArgs& a, hipStream_t s) {
  const int NT = (a.T + 63) / 64;
  const int nslots = a.cu_seqlens ? NT + a.N : a.B * NT;
  if (nslots <= 0 || (long long)a.B * a.T <= 0) return hipSuccess;
  if (a.bf16) {
    if (a.K == 128)
      return a.V == 128 ? launch_bf16<128, 128>(a, s, NT, nslots) : launch_bf16<128, 64>(a, s, NT, nslots);
    return a.V == 128 ? launch_bf16<64, 128>(a, s, NT, nslots) : launch_bf16<64, 64>(a, s, NT, nslots);
  }
  return a.K == 128 ? launch_f32<128>(a, s, NT, nslots) : launch_f32<64>(a, s, NT, nslots);
}

}  // namespace gdn
