// The state scans of "fla ops/common/chunk_h.py", gfx950: the backward
// state-gradient scan (chunk_bwd_kernel_dh) and, run forward over (k, v), the
// decay-only state scan (chunk_fwd_kernel_h).  Both keep a K x V fp32
// accumulator per (sequence, v-head, V tile) and apply one chunk per step:
//
//   backward (chunks in reverse order; A = q, B = dO):
//     start dh = dht (or 0); per chunk: if its index is a multiple of
//     split_size / 64, store dh; dh <- decay o dh + scale (A o e^{G_t})^T B;
//     end: dh0 = dh
//   forward (chunks in order; A = k, B = v):
//     start h = h0 (or 0); per chunk: if its index is a multiple of
//     split_size / 64, store h; h <- decay o h + (A o e^{G_last - G_t})^T B;
//     end: ht = h
//
// with G the chunk-local cumulative log-gate: scalar per token (g), the
// fixed per-head gamma, per key channel (gk: a factor of the A rows) or per
// value channel (gv: a factor of the B columns; it may come with g or
// gamma), and decay = e^{G_last} on the matching rows / columns.  The
// backward one is the state gradient of the decay-only recurrence
// h_t = decay_t h_{t-1} + k_t v_t^T, o_t = scale q_t^T h_t; the delta rule's
// erase term is part of neither.  In the code below the buffers keep the
// backward's names: dht = the initial state, dh = the stored states, dh0 =
// the final state.
//
// gfx950 design.  Work-group per (sequence, v-head, V tile); wave w holds key
// rows DK/4 w .. + DK/4 of dh in fp32 MFMA accumulators for the whole scan;
// the gated operand is split into a bf16 hi + lo pair (dO * scale e^{G_t} for
// a scalar gate, q * scale e^{G_t,c} for the per-channel gate; forward: the
// e^{G_last - G_t} factors); the other operand is the raw bf16 input, exact.
// Two kernels:
//   * scalar gate, gamma or no gate (state_scan_ring_kernel, 16-column
//     tiles, two work-groups per CU): a mover wave copies each chunk's rows
//     into a ring of four LDS slots three chunks ahead (direct-to-LDS loads)
//     and four compute waves read both operands out of the raw row-major
//     tiles with transposing LDS reads; one barrier per chunk;
//   * per-channel gate gk, or per-value-channel gate gv (state_scan_gk_kernel,
//     state_scan_kernel; 32-column tiles for gk, 16 for gv): each chunk's q
//     and dO rows are loaded two chunks ahead into registers and staged in
//     LDS transposed (key channel / value column major, tokens contiguous):
//     each thread transposes an 8 x 8 block (8 tokens x 8 channels) in
//     registers and writes 8 rows of 16 bytes, the 8-token units
//     XOR-swizzled by row, so both operands of the 16x16x32 bf16 product read
//     8 consecutive tokens with one 16-byte LDS read.

#include "chunk_common.h"
#include "gdn_device.h"
#include "gdn_launch.h"
#include "scan_tiles.h"

namespace gdn {

namespace {

constexpr int BT = 64;
// V columns per work-group: 16 for the scalar gate (two work-groups per CU
// fit, 512 for B = 4, H = 16), 32 for the per-channel gate (over 256 VGPRs
// per wave: one work-group per CU)
constexpr int BVS = 16, BVK = 32;
static_assert(BVK * 64 / 8 <= 256, "one gating unit per thread");
constexpr int TP = BT + 8;     // padded token row of the transposed tiles (bf16)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// the log-gate of "no gate" (not const: a const array would sit in the constant
// address space, and a pointer that may point to either would load through flat)
__device__ float kNoGate[1] = {0.f};

__device__ __forceinline__ f32x4 mma_bf(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-bit element e (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t elem16(const uint4& r, int e) {
  const uint32_t w = e < 2 ? r.x : e < 4 ? r.y : e < 6 ? r.z : r.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}
__device__ __forceinline__ uint32_t word(const uint4& r, int i) {
  return i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w;
}
// 8 x 8 transpose of 16-bit values: out[e] word p = (row 2p elem e, row 2p + 1 elem e)
__device__ __forceinline__ void transpose8(const uint4 (&R)[8], uint4 (&O)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = __builtin_amdgcn_perm(word(R[2 * p + 1], e >> 1), word(R[2 * p], e >> 1), sel);
    O[e] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// A work-group's accumulators into a [*, HV, V, K] state array: lane (n, gq)
// of a wave holds keys 16 rb + 4 gq + [0, 4) of the wave's key range in
// column 16 cb + n; `base` is the element of (column n, first key of the
// range).  With two 16-key blocks and bf16 storage, lanes gq and gq ^ 1 (lane
// ^ 16) first trade one 4-key half, so that each lane stores 8 consecutive
// keys in one 16-byte store and the four lanes of a column fill 64 contiguous
// bytes (instead of 32-byte pieces).
template <int DK, int RB, int CBN>
__device__ __forceinline__ void store_tile(void* dst, size_t base, const f32x4 (&acc)[RB][CBN], int gq, bool bf) {
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) {
    const size_t row = base + (size_t)16 * cb * DK;
    if constexpr (RB == 2) {
      if (bf) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const bool odd = gq & 1;
        const uint32_t a0 = pack_bf2(acc[0][cb][0], acc[0][cb][1]), a1 = pack_bf2(acc[0][cb][2], acc[0][cb][3]);
        const uint32_t b0 = pack_bf2(acc[1][cb][0], acc[1][cb][1]), b1 = pack_bf2(acc[1][cb][2], acc[1][cb][3]);
        // even gq keeps block 0 and takes the partner's block-0 keys 4 gq + [4, 8);
        // odd gq keeps block 1 and takes the partner's block-1 keys 16 + 4 (gq - 1) + [0, 4)
        const uint32_t r0 = (uint32_t)__shfl_xor((int)(odd ? a0 : b0), 16);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)(odd ? a1 : b1), 16);
        const u4 v = odd ? u4{r0, r1, b0, b1} : u4{a0, a1, r0, r1};
        store_nt16(reinterpret_cast<bf16_t*>(dst) + row + (odd ? 16 + 4 * (gq - 1) : 4 * gq), v);
        continue;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float x[4] = {acc[rb][cb][0], acc[rb][cb][1], acc[rb][cb][2], acc[rb][cb][3]};
      store_state4(dst, row + 16 * rb + 4 * gq, x, bf);
    }
  }
}

// The same accumulators into a key-first [*, HV, K, V] array (V contiguous:
// the state scans' layout without state_v_first): `eb` is the entry's first
// element, key0 the wave's first key, col the lane's first column.  One 4- or
// 2-byte store per element; the 16 lanes of a key row cover 16 consecutive
// columns.
template <int DK, int RB, int CBN>
__device__ __forceinline__ void store_tile_kfirst(void* dst, size_t eb, int key0, int col,
                                                  const f32x4 (&acc)[RB][CBN], int gq, bool bf) {
  constexpr int DV = DK;
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = eb + (size_t)(key0 + 16 * rb + 4 * gq + i) * DV + col + 16 * cb;
        if (bf)
          reinterpret_cast<bf16_t*>(dst)[off] = f2bf(acc[rb][cb][i]);
        else
          reinterpret_cast<float*>(dst)[off] = acc[rb][cb][i];
      }
}

// A work-group's accumulators into entry e of a state array, V-first
// ([*, HV, V, K]) or key-first ([*, HV, K, V]).
template <int DK, int RB, int CBN>
__device__ __forceinline__ void store_state_tile(void* dst, size_t e, int HV, int j, int key0, int col,
                                                 const f32x4 (&acc)[RB][CBN], int gq, bool bf, bool vfirst) {
  const size_t eb = (e * HV + j) * (size_t)DK * DK;
  if (vfirst)
    store_tile<DK, RB, CBN>(dst, eb + (size_t)col * DK + key0, acc, gq, bf);
  else
    store_tile_kfirst<DK, RB, CBN>(dst, eb, key0, col, acc, gq, bf);
}

// The initial state of the accumulators (same lane layout) from entry `sh`
// of a fp32 state array, V-first or key-first.
template <int DK, int RB, int CBN>
__device__ __forceinline__ void load_state_tile(const float* src, size_t sh, int key0, int col,
                                                f32x4 (&acc)[RB][CBN], int gq, bool vfirst) {
  const size_t eb = sh * (size_t)DK * DK;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) {
      if (vfirst) {
        const float4 x = *reinterpret_cast<const float4*>(src + eb + (size_t)(col + 16 * cb) * DK + key0 + 16 * rb +
                                                          4 * gq);
        acc[rb][cb] = f32x4{x.x, x.y, x.z, x.w};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][cb][i] = src[eb + (size_t)(key0 + 16 * rb + 4 * gq + i) * DK + col + 16 * cb];
      }
    }
}

// Per-key-channel gate (gk): the gated operand is the A side (q / k), one
// thread per key channel forms the chunk-local cumulative gates in LDS, the
// value side transposes raw; three barriers per chunk.
template <int DK, bool FWD>
__global__ __launch_bounds__(256) void state_scan_gk_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, const float* __restrict__ gk, float scale,
    const float* __restrict__ dht, void* __restrict__ dh, int nts, int sbf16, long long scap,
    float* __restrict__ dh0, const int64_t* __restrict__ cu, int Tlen, int N, int Hk, int HV, int Hg,
    int vfirst) {
  constexpr int DV = DK;
  constexpr int BVT = BVK, CBN = BVT / 16;
  constexpr int RW = DK / 4;          // key rows per wave
  constexpr int RB = RW / 16;         // 16-row blocks per wave
  constexpr int NQB = BT / 8 * DK / 8;  // 8 x 8 blocks (tokens x channels) of a q tile
  static_assert(NQB + BT / 8 * BVT / 8 <= 256, "one block per thread");
  // transposed tiles: row = key channel / value column, 8-token units XOR-swizzled by row / 8
  __shared__ __attribute__((aligned(16))) bf16_t sAh[DK][TP];   // A operand (q side), hi
  __shared__ __attribute__((aligned(16))) bf16_t sAl[DK][TP];   //   lo
  __shared__ __attribute__((aligned(16))) bf16_t sBh[BVT][TP];  // B operand (dO side), raw
  __shared__ float sG[BT][DK + 4];   // token x channel factors (backward scale e^{G_t,c}, forward e^{G_last,c - G_t,c})
  __shared__ float sDec[DK];         // e^{G_last,c}

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  // work-group -> (sequence, head, V tile): ids are dealt round-robin to the
  // 8 XCDs; the NVT tiles of a (sequence, head), which read the same q rows,
  // share an XCD (its L2)
  const int NVT = DV / BVT;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, pos = bid >> 3;
  const int vt = pos % NVT;
  const int sh = (pos / NVT) * 8 + xcd;
  if (sh >= N * HV) return;
  const int sq = sh / HV, j = sh - sq * HV;
  const int jk = j / (HV / Hk);
  const int jg = j / (HV / Hg);   // gate head: HV / Hg v-heads share one
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
  const size_t sbase = dh ? (size_t)snapshot_offset(cu, sq, Tlen, nts * BT) : 0;

  // accumulators: block (rb, cb), lane (n, gq): key row RW w + 16 rb + 4 gq + i, column v0 + 16 cb + n
  f32x4 acc[RB][CBN];
  if (dht) {
    load_state_tile<DK, RB, CBN>(dht, sh, RW * w, v0 + n, acc, gq, vfirst != 0);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the state into entry `e` of a state array (fp32, or bf16 when `bf`)
  auto store_state = [&](void* dst, size_t e, bool bf) {
    store_state_tile<DK, RB, CBN>(dst, e, HV, j, RW * w, v0 + n, acc, gq, bf, vfirst != 0);
  };

  // this thread's 8 x 8 block: q (waves 0 .. NQB / 64 - 1) or dO (the next
  // wave's first 32 lanes); roles are uniform per wave
  constexpr int QW = NQB / 64;
  static_assert(NQB % 64 == 0, "whole q waves");
  const bool isq = w < QW, isd = w == QW && lane < BT / 8 * BVT / 8;
  const int bq = isq ? tid : tid - NQB;
  const int tb = isq ? bq / (DK / 8) : bq / (BVT / 8);     // token block
  const int cb8 = isq ? bq % (DK / 8) : bq % (BVT / 8);    // channel / column block
  // raw loads of a chunk: the block's 8 rows, and the gate values; two
  // buffers, so that the loads of chunk ic - 2 fly during chunks ic and ic - 1
  uint4 rawA[8], rawB[8];
  float gvA[BT], gvB[BT];
  auto load = [&](int ic, uint4 (&raw)[8], float (&gv)[BT]) __attribute__((always_inline)) {
    const int c0 = bos + ic * BT;
    const int nrow = eos - c0 < BT ? eos - c0 : BT;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int t = 8 * tb + r, tc = t < nrow ? t : nrow - 1;
      if (isq) raw[r] = *reinterpret_cast<const uint4*>(q + ((size_t)(c0 + tc) * Hk + jk) * DK + 8 * cb8);
      else if (isd) raw[r] = *reinterpret_cast<const uint4*>(dout + ((size_t)(c0 + tc) * HV + j) * DV + v0 + 8 * cb8);
    }
    if (tid < DK) {
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        const int tc = t < nrow ? t : nrow - 1;
        gv[t] = gk[((size_t)(c0 + tc) * Hg + jg) * DK + tid];
      }
    }
  };

  // chunk of scan position i (forward: in order, backward: in reverse)
  auto chunk_at = [&](int i) { return FWD ? i : NC - 1 - i; };
  auto step = [&](int ic, int i, uint4 (&raw)[8], float (&gv)[BT]) __attribute__((always_inline)) {
    const int nrow = eos - (bos + ic * BT) < BT ? eos - (bos + ic * BT) : BT;

    // ---- chunk-local cumulative gates, one thread per key channel
    if (tid < DK) {
      if constexpr (FWD) {
        float GL = 0.f;
#pragma unroll
        for (int t = 0; t < BT; ++t) GL += t < nrow ? gv[t] : 0.f;
        float G = 0.f;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          G += t < nrow ? gv[t] : 0.f;
          sG[t][tid] = __expf(GL - G);
        }
        sDec[tid] = __expf(GL);
      } else {
        float G = 0.f;
#pragma unroll
        for (int t = 0; t < BT; ++t) {
          G += t < nrow ? gv[t] : 0.f;
          sG[t][tid] = scale * __expf(G);
        }
        sDec[tid] = __expf(G);
      }
    }
    __syncthreads();

    // ---- the block transposed into its tile: row = channel (column) 8 cb8 + e,
    // 8-token unit tb at position tb ^ (cb8 & 7); tokens past the chunk end are 0.
    // The gated operand (q / k) goes in as a bf16 hi + lo pair, dO / v raw.
    const int col = 8 * (tb ^ (cb8 & 7));
    if (isd) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (8 * tb + r >= nrow) raw[r] = make_uint4(0u, 0u, 0u, 0u);
      uint4 O[8];
      transpose8(raw, O);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *reinterpret_cast<uint4*>(&sBh[8 * cb8 + e][col]) = O[e];
      }
    } else if (isq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * cb8 + e;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          float x[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = 8 * tb + 2 * p2 + h;
            // q * scale e^{G_t,c} (forward: k * e^{G_last,c - G_t,c}); 0 past the end
            const float f = t < nrow ? sG[t][c] : 0.f;
            x[h] = bf2f((bf16_t)elem16(raw[2 * p2 + h], e)) * f;
          }
          const uint32_t h0 = f2bf(x[0]), h1 = f2bf(x[1]);
          hw[p2] = h0 | (h1 << 16);
          lw[p2] = (uint32_t)f2bf(x[0] - bf2f((bf16_t)h0)) | ((uint32_t)f2bf(x[1] - bf2f((bf16_t)h1)) << 16);
        }
        *reinterpret_cast<uint4*>(&sAh[c][col]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&sAl[c][col]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
    __syncthreads();
    // this buffer is free again: the chunk after next
    if (i + 2 < NC) load(chunk_at(i + 2), raw, gv);

    // ---- snapshot, decay, accumulate
    // (entries past the buffer's capacity are not written)
    if (dh && ic % nts == 0 && (long long)(sbase + ic / nts) < scap) store_state(dh, sbase + ic / nts, sbf16 != 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 dec;
#pragma unroll
      for (int e = 0; e < 4; ++e) dec[e] = sDec[RW * w + 16 * rb + 4 * gq + e];
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] *= dec;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int ra = RW * w + 16 * rb + n;
        const int ca = 8 * ((4 * s + gq) ^ ((ra >> 3) & 7));
        const u32x4 ah = *reinterpret_cast<const u32x4*>(&sAh[ra][ca]);
        const u32x4 al = *reinterpret_cast<const u32x4*>(&sAl[ra][ca]);
#pragma unroll
        for (int cb = 0; cb < CBN; ++cb) {
          const int rbv = 16 * cb + n;
          const int cbv = 8 * ((4 * s + gq) ^ ((rbv >> 3) & 7));
          const u32x4 bh = *reinterpret_cast<const u32x4*>(&sBh[rbv][cbv]);
          acc[rb][cb] = mma_bf(ah, bh, acc[rb][cb]);
          acc[rb][cb] = mma_bf(al, bh, acc[rb][cb]);
        }
      }
    }
    __syncthreads();
  };
  if (NC > 0) load(chunk_at(0), rawA, gvA);
  if (NC > 1) load(chunk_at(1), rawB, gvB);
  for (int i = 0; i < NC; i += 2) {
    step(chunk_at(i), i, rawA, gvA);
    if (i + 1 < NC) step(chunk_at(i + 1), i + 1, rawB, gvB);
  }
  if (dh0) store_state(dh0, sq, false);
}

// Scalar gate (g or gamma) and / or the per-value-channel gate (gv): two
// barriers per chunk.  Staging phase: the first DK / 64 waves transpose the
// q (k) block rows (8 x 8 blocks, v_perm_b32), waves 2 and 3 gate dO (v) --
// thread (column c, 8-token unit u) reads its 8 values, scales them by the
// token's factor (and, with gv, by its column's factor: the 8 threads of a
// column are adjacent lanes, so the column's chunk-local cumulative gate is
// a sum over the thread's 8 tokens plus a prefix over the 8 lanes) and
// writes the hi and lo rows.  Product phase: the MFMAs of this chunk, while
// wave 0 forms the next chunk's token factors into the other buffer and the
// loads of the chunk after next are issued.
template <int DK, bool FWD, bool GV, bool ST>
__global__ __launch_bounds__(256) void state_scan_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, const float* __restrict__ g,
    const float* __restrict__ gamma, const float* __restrict__ gvp, float scale,
    const float* __restrict__ dht, void* __restrict__ dh, int nts, int sbf16, long long scap,
    float* __restrict__ dh0, const int64_t* __restrict__ cu, int Tlen, int N, int Hk, int HV, int Hg,
    int vfirst) {
  constexpr int DV = DK;
  constexpr int BVT = BVS, CBN = BVT / 16;
  constexpr int RW = DK / 4;
  constexpr int RB = RW / 16;
  constexpr int QB = BT / 8 * DK / 8;    // q blocks: one per thread of the first QB / 64 waves
  constexpr int QPT = 1;
  // threads 128 .. 128 + ND - 1: one 8-token unit of two adjacent dO columns each
  constexpr int ND = BVT * BT / 16;
  static_assert(QB % 64 == 0 && QB <= 128 && ND % 64 == 0 && ND <= 128, "thread roles");
  __shared__ __attribute__((aligned(16))) bf16_t sAh[DK][TP];
  __shared__ __attribute__((aligned(16))) bf16_t sBh[BVT][TP];
  __shared__ __attribute__((aligned(16))) bf16_t sBl[BVT][TP];
  __shared__ float sF[2][BT + 1];     // token factors of each dO wave; e^{G_last} at [BT]
  __shared__ float sGvL[GV ? BVT : 1];  // gv: e^{Gv_last} of each column of the tile

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  const int NVT = DV / BVT;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, pos = bid >> 3;
  const int vt = pos % NVT;
  const int sh = (pos / NVT) * 8 + xcd;
  if (sh >= N * HV) return;
  const int sq = sh / HV, j = sh - sq * HV;
  const int jk = j / (HV / Hk);
  const int jg = j / (HV / Hg);   // gate head: HV / Hg v-heads share one
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
  const size_t sbase = dh ? (size_t)snapshot_offset(cu, sq, Tlen, nts * BT) : 0;

  f32x4 acc[RB][CBN];
  if (dht) {
    load_state_tile<DK, RB, CBN>(dht, sh, RW * w, v0 + n, acc, gq, vfirst != 0);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the state into entry `e` of a state array (fp32, or bf16 when `bf`)
  auto store_state = [&](void* dst, size_t e, bool bf) {
    store_state_tile<DK, RB, CBN>(dst, e, HV, j, RW * w, v0 + n, acc, gq, bf, vfirst != 0);
  };

  // roles: the first QB / 64 waves -> q blocks; waves 2, 3 -> dO (columns
  // 2 dp and 2 dp + 1, 8-token unit du: one 32-bit word per token, so the
  // loads land in whole registers and stay in flight); with DK = 64 wave 1
  // stages nothing
  const bool isq = tid < QB, isd = tid >= 128 && tid < 128 + ND;
  const int dp = (tid - 128) / (BT / 8), du = (tid - 128) % (BT / 8);
  // raw loads of a chunk (two buffers); gw: the thread's 8 tokens of its two columns (0 past the end);
  // gv: the dO waves' gate value of token `lane`
  constexpr int GVT = GV ? 8 : 1;
  uint4 rqA[QPT][8], rqB[QPT][8];
  uint32_t rdA[8], rdB[8];
  float gwA[2][GVT], gwB[2][GVT];
  float gvA, gvB;
  auto load = [&](int ic, uint4 (&rq)[QPT][8], uint32_t (&rd)[8], float (&gw)[2][GVT], float& gv)
      __attribute__((always_inline)) {
    const int c0 = bos + ic * BT;
    const int nrow = eos - c0 < BT ? eos - c0 : BT;
    if (isq) {
#pragma unroll
      for (int k2 = 0; k2 < QPT; ++k2) {
        const int bq = tid + 128 * k2, tb = bq / (DK / 8), cb8 = bq % (DK / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = 8 * tb + r, tc = t < nrow ? t : nrow - 1;
          rq[k2][r] = *reinterpret_cast<const uint4*>(q + ((size_t)(c0 + tc) * Hk + jk) * DK + 8 * cb8);
        }
      }
    } else if (isd) {
      {
        // one vector load from whichever source applies (a zero for no gate):
        // a branch between a vector and a scalar load would make the compiler
        // wait for every load in flight where the two meet
        const int tc = lane < nrow ? lane : nrow - 1;
        const float* gp = g ? g + (size_t)(c0 + tc) * Hg + jg : (gamma ? gamma + jg : kNoGate);
        gv = *gp;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int t = 8 * du + r, tc = t < nrow ? t : nrow - 1;
        const size_t off = ((size_t)(c0 + tc) * HV + j) * DV + v0 + 2 * dp;
        rd[r] = *reinterpret_cast<const uint32_t*>(dout + off);
        if constexpr (GV) {
          const float2 x = *reinterpret_cast<const float2*>(gvp + ((size_t)(c0 + tc) * Hg + jg) * DV + v0 + 2 * dp);
          gw[0][r] = t < nrow ? x.x : 0.f;
          gw[1][r] = t < nrow ? x.y : 0.f;
        }
      }
    }
  };
  // chunk of scan position i (forward: in order, backward: in reverse)
  auto chunk_at = [&](int i) { return FWD ? i : NC - 1 - i; };

  // (the staging reads this buffer's gate value, the loads then refill it)
  auto step = [&](int ic, int i, uint4 (&rq)[QPT][8], uint32_t (&rd)[8], float (&gw)[2][GVT], float& gv)
      __attribute__((always_inline)) {
    const int nrow = eos - (bos + ic * BT) < BT ? eos - (bos + ic * BT) : BT;
    // ---- staging
    if (isq) {
#pragma unroll
      for (int k2 = 0; k2 < QPT; ++k2) {
        const int bq = tid + 128 * k2, tb = bq / (DK / 8), cb8 = bq % (DK / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (8 * tb + r >= nrow) rq[k2][r] = make_uint4(0u, 0u, 0u, 0u);
        uint4 O[8];
        transpose8(rq[k2], O);
        const int col = 8 * (tb ^ (cb8 & 7));
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(&sAh[8 * cb8 + e][col]) = O[e];
      }
    } else if (isd) {
      // the chunk's token factors, formed by each dO wave from the gate row it
      // loaded with the tile (lane = token): backward scale e^{G_t}, forward
      // e^{G_last - G_t}, 0 past the end; e^{G_last} at [BT]
      float* sFw = sF[w - 2];
      {
        const float G = intra::wave_incl_scan(lane < nrow ? gv : 0.f, lane);
        const float GL = __shfl(G, nrow - 1);
        sFw[lane] = lane < nrow ? (FWD ? __expf(GL - G) : scale * __expf(G)) : 0.f;
        if (lane == 0) sFw[BT] = __expf(GL);
      }
      const int t0 = 8 * du;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * dp + cc;
        // gv: the column's factors at the thread's 8 tokens
        float fv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) fv[r] = 1.f;
        if constexpr (GV) {
          float P[8], run = 0.f;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            run += gw[cc][r];
            P[r] = run;
          }
          // inclusive prefix of the 8 units' sums over the column's lanes (du = lane % 8)
          float inc = run;
#pragma unroll
          for (int d = 1; d < 8; d <<= 1) {
            const float y = __shfl_up(inc, d, 8);
            if (du >= d) inc += y;
          }
          const float base = inc - run, GL = __shfl(inc, 7, 8);
#pragma unroll
          for (int r = 0; r < 8; ++r) fv[r] = FWD ? __expf(GL - (base + P[r])) : __expf(base + P[r]);
          if (du == 0) sGvL[c] = __expf(GL);
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          // column cc of tokens t0 + 2 p2 (+ 1): the low / high half of the word
          const uint32_t w0 = rd[2 * p2], w1 = rd[2 * p2 + 1];
          const float d0 = __builtin_bit_cast(float, cc ? (w0 & 0xFFFF0000u) : (w0 << 16));
          const float d1 = __builtin_bit_cast(float, cc ? (w1 & 0xFFFF0000u) : (w1 << 16));
          const float x0 = d0 * (sFw[t0 + 2 * p2] * fv[2 * p2]);   // 0 past the chunk end
          const float x1 = d1 * (sFw[t0 + 2 * p2 + 1] * fv[2 * p2 + 1]);
          const uint32_t h0 = f2bf(x0), h1 = f2bf(x1);
          hw[p2] = h0 | (h1 << 16);
          lw[p2] = (uint32_t)f2bf(x0 - bf2f((bf16_t)h0)) | ((uint32_t)f2bf(x1 - bf2f((bf16_t)h1)) << 16);
        }
        const int col = 8 * (du ^ ((c >> 3) & 7));
        *reinterpret_cast<uint4*>(&sBh[c][col]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&sBl[c][col]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
    __syncthreads();
    // ---- products; the loads of the chunk after next
    if (i + 2 < NC) load(chunk_at(i + 2), rq, rd, gw, gv);
    // (entries past the buffer's capacity are not written)
    if (ST && ic % nts == 0 && (long long)(sbase + ic / nts) < scap) store_state(dh, sbase + ic / nts, sbf16 != 0);
    const float dec = sF[0][BT];
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) {
      const float decy = GV ? dec * sGvL[16 * cb + n] : dec;   // the lane's column 16 cb + n
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb][cb] *= decy;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int ra = RW * w + 16 * rb + n;
        const u32x4 ah = *reinterpret_cast<const u32x4*>(&sAh[ra][8 * ((4 * s2 + gq) ^ ((ra >> 3) & 7))]);
#pragma unroll
        for (int cb = 0; cb < CBN; ++cb) {
          const int rbv = 16 * cb + n;
          const int cbv = 8 * ((4 * s2 + gq) ^ ((rbv >> 3) & 7));
          acc[rb][cb] = mma_bf(ah, *reinterpret_cast<const u32x4*>(&sBh[rbv][cbv]), acc[rb][cb]);
          acc[rb][cb] = mma_bf(ah, *reinterpret_cast<const u32x4*>(&sBl[rbv][cbv]), acc[rb][cb]);
        }
      }
    }
    __syncthreads();
  };

  // the initial state has landed before the first tile loads: otherwise the
  // compiler waits for it inside the loop, for every load in flight, each step
  __builtin_amdgcn_s_waitcnt(0);
  if (NC > 0) load(chunk_at(0), rqA, rdA, gwA, gvA);
  if (NC > 1) load(chunk_at(1), rqB, rdB, gwB, gvB);
  // scan position 2 m uses buffer A, 2 m + 1 buffer B
  for (int i = 0; i < NC; i += 2) {
    step(chunk_at(i), i, rqA, rdA, gwA, gvA);
    if (i + 1 < NC) step(chunk_at(i + 1), i + 1, rqB, rdB, gwB, gvB);
  }
  if (dh0) store_state(dh0, sq, false);
}

// s_waitcnt vmcnt(n) with the other counters untouched (gfx9 encoding: vmcnt
// bits 3:0 and 15:14)
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

// Inclusive prefix sum over the 64 lanes with DPP: shifts within each
// 16-lane row (0 shifted in), then row 15's total into rows 1 and 3 and lane
// 31's into rows 2 and 3 (row_bcast, a GFX9 DPP form).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_scan_dpp(float x) {
  x += dpp_rows<0x111, 0xF>(x);   // row_shr:1
  x += dpp_rows<0x112, 0xF>(x);   // row_shr:2
  x += dpp_rows<0x114, 0xF>(x);   // row_shr:4
  x += dpp_rows<0x118, 0xF>(x);   // row_shr:8
  x += dpp_rows<0x142, 0xA>(x);   // row_bcast:15 into rows 1, 3
  x += dpp_rows<0x143, 0xC>(x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Scalar gate g, fixed per-head decay gamma, or no gate (no gv).  A mover
// wave copies each chunk's rows from global memory straight into a ring of
// four LDS slots, three chunks ahead of their use (direct-to-LDS loads: no
// registers held, so the lead is not bounded by the register budget); four
// compute waves read both MFMA operands out of the raw row-major tiles
// through transposing reads (ds_read_b64_tr_b16), each lane addressing 4
// consecutive channels of one token:
//   * A (q / k, raw bf16, exact): lane (n, g) of 16-key block rb holds key
//     DK/4 w + 16 rb + n at tokens 32 s + 8 g + e;
//   * B (dO / v times the token factor, bf16 hi + lo): lane (n, g) holds
//     column n at the same tokens.
// Every compute wave forms the chunk's token factors itself (a DPP scan of
// the gate row).  One barrier per chunk: the mover waits for its loads of
// the chunk (vmcnt: only its loads are in flight, in issue order) and the
// barrier publishes them; after it the mover refills the slot the compute
// waves finished reading before it.  The roles run separate loops, and each
// slot is its own array selected at compile time: a wave that reads LDS
// while its own direct-to-LDS loads are in flight, or reads an array the
// compiler cannot tell apart from the one being filled, gets a wait for all
// of them.  16-column V tiles: two work-groups per CU.
template <int DK, bool FWD, bool ST>
__global__ __launch_bounds__(320) void state_scan_ring_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, const float* __restrict__ g,
    const float* __restrict__ gamma, float scale, const float* __restrict__ dht, void* __restrict__ dh,
    int nts, int sbf16, long long scap, float* __restrict__ dh0, const int64_t* __restrict__ cu, int Tlen,
    int N, int Hk, int HV, int Hg, int vfirst) {
  constexpr int DV = DK, BV = BVS, CBN = 1;
  constexpr int RW = DK / 4, RB = RW / 16;
  constexpr int NSL = 4, LEAD = NSL - 1;  // LDS slots; chunks loaded ahead of their use
  constexpr int QT = BT * DK * 2;         // q tile bytes
  constexpr int NQK = QT / 1024;          // 1 KB direct-to-LDS loads per q tile
  constexpr int QROWS = 512 / DK;         // q rows per 1 KB load
  constexpr int VT = BT * BV * 2;         // value tile bytes
  static_assert(VT == 2048, "two 1 KB loads per value tile");
  constexpr int NLD = NQK + 3;            // mover loads per chunk: q tile, value tile, gate row
  static_assert(2 * NLD <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char sQ0[QT], sQ1[QT], sQ2[QT], sQ3[QT];
  __shared__ __attribute__((aligned(16))) char sV0[VT], sV1[VT], sV2[VT], sV3[VT];
  __shared__ __attribute__((aligned(16))) float sG0[BT], sG1[BT], sG2[BT], sG3[BT];  // gate rows
  __shared__ __attribute__((aligned(16))) float sFw[4][BT];    // token factors of each compute wave
  __shared__ __attribute__((aligned(16))) uint32_t sSink[64];  // landing words of an L2 touch

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  constexpr int NVT = DV / BV;
  // work-group -> (sequence, head, V tile): the NVT tiles of a (sequence,
  // head), which read the same q rows, share an XCD (its L2)
  const int bid = blockIdx.x;
  const int xcd = bid & 7, pos = bid >> 3;
  const int vt = pos % NVT;
  const int sh = (pos / NVT) * 8 + xcd;
  if (sh >= N * HV) return;
  const int sq = sh / HV, j = sh - sq * HV;
  const int jk = j / (HV / Hk);
  const int jg = j / (HV / Hg);
  const int v0 = vt * BV;
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
  auto chunk_at = [&](int i) { return FWD ? i : NC - 1 - i; };
  auto slot_q = [&](auto S) -> char* {
    if constexpr (decltype(S)::value == 0) return sQ0;
    else if constexpr (decltype(S)::value == 1) return sQ1;
    else if constexpr (decltype(S)::value == 2) return sQ2;
    else return sQ3;
  };
  auto slot_v = [&](auto S) -> char* {
    if constexpr (decltype(S)::value == 0) return sV0;
    else if constexpr (decltype(S)::value == 1) return sV1;
    else if constexpr (decltype(S)::value == 2) return sV2;
    else return sV3;
  };
  auto slot_g = [&](auto S) -> float* {
    if constexpr (decltype(S)::value == 0) return sG0;
    else if constexpr (decltype(S)::value == 1) return sG1;
    else if constexpr (decltype(S)::value == 2) return sG2;
    else return sG3;
  };

  if (w == 4) {
    // =================== mover wave
    // one chunk into a slot: the q tile (LDS row r, 16-byte unit u' receives
    // global unit u' ^ swizzle(r); rows past the sequence end repeat its last
    // row), the value tile (32-byte rows), the gate row (or an L2 touch, so
    // that every chunk takes NLD loads)
    const uint32_t q_row = (uint32_t)Hk * DK * 2;
    auto load_chunk = [&](int ic, auto S) __attribute__((always_inline)) {
      const int c0 = bos + ic * BT;
      const int nr = eos - c0 < BT ? eos - c0 : BT;
      const char* qc = reinterpret_cast<const char*>(q + ((size_t)c0 * Hk + jk) * DK);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        const int row = i * QROWS + lane / (DK / 8);
        const int rr = row < nr ? row : nr - 1;
        tiles::dma16(qc + (uint32_t)rr * q_row + 16 * ((lane % (DK / 8)) ^ tiles::qk_swz<DK>(row)),
                     (tiles::lchar*)slot_q(S) + 1024 * i);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * i + (lane >> 1);
        const int rr = row < nr ? row : nr - 1;
        tiles::dma16(dout + ((size_t)(c0 + rr) * HV + j) * DV + v0 + 8 * (lane & 1),
                     (tiles::lchar*)slot_v(S) + 1024 * i);
      }
      if (g) {
        const int rr = lane < nr ? lane : nr - 1;
        tiles::dma4(g + (size_t)(c0 + rr) * Hg + jg, (tiles::lchar*)slot_g(S));
      } else {
        tiles::touch4(dout + ((size_t)c0 * HV + j) * DV + v0, (tiles::lchar*)sSink);
      }
    };
    if (NC > 0) load_chunk(chunk_at(0), tiles::Int<0>{});
    if (NC > 1) load_chunk(chunk_at(1), tiles::Int<1>{});
    if (NC > 2) load_chunk(chunk_at(2), tiles::Int<2>{});
    auto mstep = [&](auto S, int i) __attribute__((always_inline)) {
      constexpr int SL = decltype(S)::value;
      // this chunk's loads have landed: only the next two chunks' may be in flight
      const int ahead = (i + 1 < NC) + (i + 2 < NC);
      if (ahead == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NLD));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      tiles::lds_barrier();
      if (i + LEAD < NC) load_chunk(chunk_at(i + LEAD), tiles::Int<(SL + LEAD) % NSL>{});
    };
    for (int i = 0; i < NC; i += NSL) {
      mstep(tiles::Int<0>{}, i);
      if (i + 1 < NC) mstep(tiles::Int<1>{}, i + 1);
      if (i + 2 < NC) mstep(tiles::Int<2>{}, i + 2);
      if (i + 3 < NC) mstep(tiles::Int<3>{}, i + 3);
    }
    return;
  }

  // =================== compute waves
  const size_t sbase = ST ? (size_t)snapshot_offset(cu, sq, Tlen, nts * BT) : 0;
  // accumulators: lane (n, gq) of block rb holds keys DK/4 w + 16 rb + 4 gq + i, column v0 + n
  f32x4 acc[RB][CBN];
  if (dht) {
    load_state_tile<DK, RB, CBN>(dht, sh, RW * w, v0 + n, acc, gq, vfirst != 0);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float gam = (!g && gamma) ? gamma[jg] : 0.f;
  auto store_state = [&](void* dst, size_t e, bool bf) {
    store_state_tile<DK, RB, CBN>(dst, e, HV, j, RW * w, v0 + n, acc, gq, bf, vfirst != 0);
  };
  // A-fragment byte offsets within a q tile: block rb, slab s, token half h
  int o_a[RB][2][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 32 * s2 + 8 * gq + 4 * h + (n >> 2);
        const int key = RW * w + 16 * rb + 4 * (n & 3);
        o_a[rb][s2][h] = tiles::qk_off<DK>(t, key >> 3) + 2 * (key & 7);
      }

  auto cstep = [&](auto S, int i) __attribute__((always_inline)) {
    const int ic = chunk_at(i);
    const int nrow = eos - (bos + ic * BT) < BT ? eos - (bos + ic * BT) : BT;
    tiles::lds_barrier();
    // LDS returns in order: the gate value first, then the tile reads (they do
    // not depend on the gate); then the token factors (lane = token):
    // backward scale e^{G_t}, forward e^{G_last - G_t}, 0 past the end; the
    // state decays by e^{G_last}
    const float graw = g ? slot_g(S)[lane] : gam;
    const char* qs = slot_q(S);
    const char* vs = slot_v(S);
    uint2 ra[RB][2][2], rv[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int t0 = 32 * s2 + 8 * gq;
#pragma unroll
      for (int h = 0; h < 2; ++h) rv[s2][h] = tiles::ld_tr(vs + (t0 + 4 * h + (n >> 2)) * (2 * BV) + 8 * (n & 3));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) ra[rb][s2][h] = tiles::ld_tr(qs + o_a[rb][s2][h]);
    }
    const float G = wave_scan_dpp(lane < nrow ? graw : 0.f);
    const float GL = __shfl(G, nrow - 1);
    sFw[w][lane] = lane < nrow ? (FWD ? __expf(GL - G) : scale * __expf(G)) : 0.f;
    const float dec = __expf(GL);

    // B fragments: column n of the value tile at tokens 32 s + 8 gq + e, scaled, bf16 hi + lo
    u32x4 Bh[2], Bl[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int t0 = 32 * s2 + 8 * gq;
      const uint2 d0 = rv[s2][0], d1 = rv[s2][1];
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sFw[w][t0]);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sFw[w][t0 + 4]);
      const f32x4 x0 = {bf2f((bf16_t)(d0.x & 0xFFFFu)) * f0[0], bf2f((bf16_t)(d0.x >> 16)) * f0[1],
                        bf2f((bf16_t)(d0.y & 0xFFFFu)) * f0[2], bf2f((bf16_t)(d0.y >> 16)) * f0[3]};
      const f32x4 x1 = {bf2f((bf16_t)(d1.x & 0xFFFFu)) * f1[0], bf2f((bf16_t)(d1.x >> 16)) * f1[1],
                        bf2f((bf16_t)(d1.y & 0xFFFFu)) * f1[2], bf2f((bf16_t)(d1.y >> 16)) * f1[3]};
      tiles::split_bf(x0, x1, Bh[s2], Bl[s2]);
    }
    // the state before this chunk, stored after the products are issued
    // (entries past the capacity are not written)
    const bool st = ST && ic % nts == 0 && (long long)(sbase + ic / nts) < scap;
    f32x4 prev[RB][CBN];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) prev[rb][0] = acc[rb][0];
    // the products: the two 32-token halves accumulate separately, so that
    // each product's accumulator was last written 2 RB products earlier
    f32x4 p1[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc[rb][0] *= dec;
      p1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 a[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        a[rb][s2] = u32x4{ra[rb][s2][0].x, ra[rb][s2][0].y, ra[rb][s2][1].x, ra[rb][s2][1].y};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = mma_bf(a[rb][0], Bh[0], acc[rb][0]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) p1[rb] = mma_bf(a[rb][1], Bh[1], p1[rb]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = mma_bf(a[rb][0], Bl[0], acc[rb][0]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) p1[rb] = mma_bf(a[rb][1], Bl[1], p1[rb]);
    if (st) store_state_tile<DK, RB, CBN>(dh, sbase + ic / nts, HV, j, RW * w, v0 + n, prev, gq, sbf16 != 0,
                                          vfirst != 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] += p1[rb];
  };
  for (int i = 0; i < NC; i += NSL) {
    cstep(tiles::Int<0>{}, i);
    if (i + 1 < NC) cstep(tiles::Int<1>{}, i + 1);
    if (i + 2 < NC) cstep(tiles::Int<2>{}, i + 2);
    if (i + 3 < NC) cstep(tiles::Int<3>{}, i + 3);
  }
  if (dh0) store_state(dh0, sq, false);
}

template <int DK, bool FWD>
hipError_t launch_k(const BwdDhArgs& a, hipStream_t s) {
  const long long blocks = ((long long)a.N * a.HV + 7) / 8 * 8 * (DK / BVK);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((state_scan_gk_kernel<DK, FWD>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.dout, a.gk, a.scale, a.dht, a.dh,
                     a.split_chunks, a.dh_bf16 ? 1 : 0, a.dh_cap, a.dh0, a.cu_seqlens, a.T, a.N, a.Hk, a.HV,
                     a.Hg, a.v_first ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

template <int DK, bool FWD, bool GV>
hipError_t launch_gdn(const BwdDhArgs& a, hipStream_t s) {
  const long long blocks = ((long long)a.N * a.HV + 7) / 8 * 8 * (DK / BVS);
  if (blocks == 0) return hipSuccess;
  if constexpr (!GV) {
    auto ring = a.dh ? state_scan_ring_kernel<DK, FWD, true> : state_scan_ring_kernel<DK, FWD, false>;
    hipLaunchKernelGGL(ring, dim3((unsigned)blocks), dim3(320), 0, s, (const bf16_t*)a.q, (const bf16_t*)a.dout,
                       a.g, a.g_gamma, a.scale, a.dht, a.dh, a.split_chunks, a.dh_bf16 ? 1 : 0, a.dh_cap, a.dh0,
                       a.cu_seqlens, a.T, a.N, a.Hk, a.HV, a.Hg, a.v_first ? 1 : 0);
    return hipGetLastError();
  }
  // without stored states the loop issues no stores, so the waits for the
  // loads of earlier chunks stay partial (the compiler waits for every
  // memory operation in flight wherever loads and stores may both be pending)
  auto kern = a.dh ? state_scan_kernel<DK, FWD, GV, true> : state_scan_kernel<DK, FWD, GV, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.dout, a.g, a.g_gamma, a.gv, a.scale, a.dht, a.dh,
                     a.split_chunks, a.dh_bf16 ? 1 : 0, a.dh_cap, a.dh0, a.cu_seqlens, a.T, a.N, a.Hk, a.HV,
                     a.Hg, a.v_first ? 1 : 0);
  return hipGetLastError();
}

template <bool FWD>
hipError_t launch_dir(const BwdDhArgs& a, hipStream_t s) {
  if (a.gk) return a.K == 128 ? launch_k<128, FWD>(a, s) : launch_k<64, FWD>(a, s);
  if (a.gv) return a.K == 128 ? launch_gdn<128, FWD, true>(a, s) : launch_gdn<64, FWD, true>(a, s);
  return a.K == 128 ? launch_gdn<128, FWD, false>(a, s) : launch_gdn<64, FWD, false>(a, s);
}

hipError_t launch_bwd_dh(const BwdDhArgs& a, hipStream_t s) {
  return a.fwd ? launch_dir<true>(a, s) : launch_dir<false>(a, s);
}

}  // namespace gdn
