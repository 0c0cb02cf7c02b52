// Chunk-parallel part of the chunked prefill, gfx950: per (chunk, v-head)
//   Aqk  = scale * (Q K^T  o  Gamma)  on s <= t          (causal, gated)
//   A    = beta_t (K K^T o Gamma)     on s <  t          (strictly lower)
//   Ainv = (I + A)^-1
// with Gamma_ts = exp(G_t - G_s) for GDN (G = chunk-local cumulative log-gate)
// or the per-channel gated dot products for KDA.
//
// What is computed follows "sglang srt/layers/attention/fla/chunk_fwd.py"
// (chunk_gated_delta_rule_fwd_kkt_solve_kernel, steps 1-5: the ten lower
// 16 x 16 blocks of K K^T, gate and beta scaling with the strictly-lower mask
// on the diagonal blocks, forward substitution on the four diagonal blocks,
// the block merge Ai10 = -Ai11 A10 Ai00, ..., Ai30 = -Ai33 (A30 Ai00 + A31
// Ai10 + A32 Ai20)) and, for the per-channel gate, "vLLM kimi_k3 amd ops
// kda/chunk_intra" (chunk_kda_fwd_kernel_inter_solve_fused: off-diagonal
// Aqk / Akk with a reference row, beta on Akk rows, scale on Aqk).
//
// gfx950 design: one wave64 per (chunk, v-head).
//   * the ten lower 16 x 16 blocks of K K^T and Q K^T run as bf16
//     v_mfma_f32_16x16x32 (fp32 io: v_mfma_f32_16x16x4_f32) straight from
//     global memory -- the same k fragment serves as A and B operand;
//   * gate / beta / mask are applied to the fp32 accumulators;
//   * the substitution gives lane (b, j) column j of the inverse of diagonal
//     block b: 16 lanes per block, 4 blocks in parallel, fp32 FMAs on
//     registers with the A rows broadcast from LDS;
//   * the merge runs as fp32 v_mfma_f32_16x16x4 chains inside the wave; an
//     accumulator is reused as the next product's B operand without a trip
//     through LDS (its lane layout equals the B layout up to a permutation of
//     the reduction index, which the A operand mirrors);
//   * results are staged in LDS and written as 16-byte rows.
// Everything is kept in fp32 until the final store in the io dtype.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

using namespace intra;

// -------------------------------------------------------------------------
// GDN intra kernel (scalar gate)
// -------------------------------------------------------------------------
template <typename T, int DK, typename C = typename ComputeOf<T>::type>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void gdn_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ gamma, const float* __restrict__ beta, float scale, C* __restrict__ Ainv,
    C* __restrict__ Aqk, float* __restrict__ GF, const int64_t* __restrict__ cu,
    const int32_t* __restrict__ coff, int Tlen, int ttot, int N, int NT, int nslots, int Hk, int HV) {
  __shared__ __attribute__((aligned(16))) float sA[BT][AP];
  const int lane = threadIdx.x;
  int slot, j, c0, nrow;
  if (!slot_of_block(nslots, HV, slot, j)) return;
  if (!locate_chunk(slot, cu, coff, N, Tlen, NT, c0, nrow)) return;
  const int jk = j / (HV / Hk);
  const int row = lane & 15, grp = lane >> 4;

  // q / k fragments of one 32-channel slab: rows 16rb + row of the chunk;
  // rows past the chunk end repeat its last row (loads stay unconditional,
  // so they are all in flight at once): such rows reach A only through
  // beta = 0, and Aqk only in rows and columns that are never stored
  auto load_slab = [&](int s, Frag<T> (&kf)[4], Frag<T> (&qf)[4]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 16 * rb + row < nrow ? 16 * rb + row : nrow - 1;
      const size_t off = ((size_t)(c0 + r) * Hk + jk) * DK + 32 * s + 8 * grp;
      load8(kf[rb], k + off);
      load8(qf[rb], q + off);
    }
  };
  Frag<T> kf[2][4], qf[2][4];   // two slabs in flight
  load_slab(0, kf[0], qf[0]);

  // chunk-local cumulative gate and beta, lane = token
  // (loads clamped to the chunk, values masked: no branch around a load)
  const int tl = lane < nrow ? lane : nrow - 1;
  // per-token log-gate, or the head's fixed log-decay for every token
  // ("fla ops/common/chunk_h.py", USE_G_GAMMA: G = gamma * (t + 1) in a chunk)
  const float g_raw = g ? g[(size_t)(c0 + tl) * HV + j] : (gamma ? gamma[j] : 0.f);
  const float b_raw = beta[(size_t)(c0 + tl) * HV + j];
  if (DK / 32 > 1) load_slab(1, kf[1], qf[1]);
  const float gl = lane < nrow ? g_raw : 0.f;
  const float G = wave_incl_scan(gl, lane);
  const float bl = lane < nrow ? b_raw : 0.f;
  // per-token gate factors for the scan: e^G, e^{G_last - G}, beta, e^{G_last}
  {
    const float Gl = __shfl(G, nrow - 1, 64);
    if (lane < nrow) {
      const size_t gs = (size_t)gf_stride(ttot);
      float* gp = GF + (size_t)j * 4 * gs + c0 + lane;
      gp[0] = __expf(G);
      gp[gs] = __expf(Gl - G);
      gp[2 * gs] = bl;
      gp[3 * gs] = __expf(Gl);
    }
  }

  // Step 1: ten lower blocks of K K^T and Q K^T
  f32x4 KK[10], QK[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) { KK[t] = zero4(); QK[t] = zero4(); }
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    if (s >= 1 && s + 1 < DK / 32) load_slab(s + 1, kf[(s + 1) & 1], qf[(s + 1) & 1]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) {
        KK[tix(rb, cb)] = mma(kf[s & 1][rb], kf[s & 1][cb], KK[tix(rb, cb)]);
        QK[tix(rb, cb)] = mma(qf[s & 1][rb], kf[s & 1][cb], QK[tix(rb, cb)]);
      }
  }

  // Step 2: gate / beta / mask.  Lane holds rows 16rb + 4grp + i, column 16cb + row.
  float Gr[4][4], Br[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Gr[rb][i] = __shfl(G, 16 * rb + 4 * grp + i, 64);
      Br[rb][i] = __shfl(bl, 16 * rb + 4 * grp + i, 64);
    }
  float Gc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) Gc[cb] = __shfl(G, 16 * cb + row, 64);

  // Aqk -> LDS (upper blocks zero) -> global
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * grp + i, s = 16 * cb + row;
        float val = 0.f;
        if (cb <= rb && s <= r) val = scale * QK[tix(rb, cb < rb ? cb : rb)][i] * __expf(Gr[rb][i] - Gc[cb]);
        sA[r][s] = val;
      }
  __syncthreads();
  store_tile<C>(sA, Aqk, c0, nrow, HV, j, lane);
  __syncthreads();
  // A = beta_r (k_r . k_s) exp(G_r - G_s), s < r
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * grp + i, s = 16 * cb + row;
        float val = 0.f;
        if (cb <= rb && s < r) val = Br[rb][i] * KK[tix(rb, cb < rb ? cb : rb)][i] * __expf(Gr[rb][i] - Gc[cb]);
        sA[r][s] = val;
      }
  __syncthreads();

  // Steps 3-4: substitution + merge
  solve_unit_lower_64<1>(sA, lane, 0);

  // Step 5: store
  store_tile<C>(sA, Ainv, c0, nrow, HV, j, lane);
}

}  // namespace

hipError_t launch_intra_gdn(const ChunkArgs& a, hipStream_t s, int NT, int nslots) {
  const dim3 grid(intra_blocks(nslots, a.HV));
  if (a.bf16) {
    if (a.K == 128)
      hipLaunchKernelGGL((gdn_intra_kernel<bf16_t, 128>), grid, dim3(64), 0, s,
                         (const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.g_gamma, a.beta, a.scale,
                         (f16_t*)a.Ainv, (f16_t*)a.Aqk, (float*)a.GF, a.cu_seqlens, a.chunk_off,
                         a.T, a.B * a.T, a.N, NT, nslots, a.Hk, a.HV);
    else
      hipLaunchKernelGGL((gdn_intra_kernel<bf16_t, 64>), grid, dim3(64), 0, s,
                         (const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.g_gamma, a.beta, a.scale,
                         (f16_t*)a.Ainv, (f16_t*)a.Aqk, (float*)a.GF, a.cu_seqlens, a.chunk_off,
                         a.T, a.B * a.T, a.N, NT, nslots, a.Hk, a.HV);
  } else {
    if (a.K == 128)
      hipLaunchKernelGGL((gdn_intra_kernel<float, 128>), grid, dim3(64), 0, s,
                         (const float*)a.q, (const float*)a.k, a.g, a.g_gamma, a.beta, a.scale,
                         (float*)a.Ainv, (float*)a.Aqk, (float*)a.GF, a.cu_seqlens, a.chunk_off,
                         a.T, a.B * a.T, a.N, NT, nslots, a.Hk, a.HV);
    else
      hipLaunchKernelGGL((gdn_intra_kernel<float, 64>), grid, dim3(64), 0, s,
                         (const float*)a.q, (const float*)a.k, a.g, a.g_gamma, a.beta, a.scale,
                         (float*)a.Ainv, (float*)a.Aqk, (float*)a.GF, a.cu_seqlens, a.chunk_off,
                         a.T, a.B * a.T, a.N, NT, nslots, a.Hk, a.HV);
  }
  return hipGetLastError();
}

}  // namespace gdn
