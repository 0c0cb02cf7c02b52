// LDS tiles, MFMA fragment helpers and direct-to-LDS copies shared by the
// bf16 chunk scan (chunk_scan_gdn.hip), gfx950.
//
// Conventions: a chunk is 64 tokens; a work-group covers a 32-column V tile.
// 16 x 16 accumulator blocks are renumbered so that accumulator pair
// (2s, 2s + 1) covers reduction slots 32 s + 8 (l / 16) + e in natural order
// (perm_row), which makes two accumulators the B operand of the next 32-deep
// product without a trip through LDS.  q / k tiles (rows of 2 DK bytes) and
// 64 x 64 fp16 tiles (rows of 128 bytes) are stored with a 16-byte-unit XOR
// swizzle by row, so both row-fragment reads and the transposing reads of
// ds_read_b64_tr_b16 are free of bank conflicts.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace tiles {

constexpr int BT = 64;     // chunk length
constexpr int BV = 32;     // V columns per work-group (the 64-column form doubles it)
constexpr int NTHR = 512;  // eight waves per work-group

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lchar;  // LDS byte pointer

// compile-time stage selectors of the double-buffered chunk inputs
struct Stage0 { static constexpr bool value = false; };
struct Stage1 { static constexpr bool value = true; };

// compile-time loop: f(Int<I>{}) for I = 0 .. N - 1
template <int I> struct Int { static constexpr int value = I; };
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

// Row (token or channel) of block `blk`, row r of a 16-row MFMA tile.
__device__ __forceinline__ int perm_row(int blk, int r) {
  return 32 * (blk >> 1) + 8 * (r >> 2) + 4 * (blk & 1) + (r & 3);
}
// perm_row(blk, r) - perm_row(0, r)
__device__ __forceinline__ constexpr int blk_rows(int blk) { return 32 * (blk >> 1) + 4 * (blk & 1); }

// 16-byte-unit XOR swizzles of the q / k tiles (rows of 2 DK bytes) and the
// Ainv / Aqk tiles (rows of 128 bytes).  Bank-conflict free for (a) the row
// fragment reads, 16 rows perm_row(blk, 0..15) at one unit, and (b) the
// transposing reads of K^T, rows t0 + {0..3} at units u0 + {0..3}.
template <int DK>
__device__ __forceinline__ int qk_swz(int t) {
  if constexpr (DK == 128) return ((t & 3) << 2) | ((t >> 3) & 3);
  else return (((t >> 1) & 1) << 2) | ((t >> 3) & 3);
}
__device__ __forceinline__ int a_swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 3) & 3); }

// byte offset of 16-byte unit u of row t
template <int DK>
__device__ __forceinline__ int qk_off(int t, int u) {
  return t * (2 * DK) + ((u ^ qk_swz<DK>(t)) << 4);
}
__device__ __forceinline__ int a_off(int t, int u) { return t * 128 + ((u ^ a_swz(t)) << 4); }

// select by value (a conditional over two captured lvalues would select their
// addresses and keep the lambda's captures in memory)
template <typename T>
__device__ __forceinline__ T pick(bool c, T a, T b) { return c ? a : b; }

__device__ __forceinline__ u32x4 ld16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives element i % 4 of the 4-element (8-byte) rows addressed by lanes
// i / 4 + 4k, k = 0..3.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_tr(const char* p) {
  typedef __attribute__((address_space(3))) v4i16 lv4i16;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4i16*)p));
}

// Work-group barrier ordering LDS only: this wave's LDS writes have completed
// (lgkmcnt) before the barrier.  Unlike __syncthreads() it does not wait for
// the direct-to-LDS loads in flight, which the wave that issued them waits for
// before the barrier that publishes their data.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 mma_bf(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_h(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two accumulators -> one B fragment (slots 0..3 from `a`, 4..7 from `b`),
// as a bf16 hi + lo pair (x ~= hi + lo).
__device__ __forceinline__ void split_bf(f32x4 a, f32x4 b, u32x4& hi, u32x4& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t h = pack_bf2(x[2 * p], x[2 * p + 1]);
    hi[p] = h;
    lo[p] = pack_bf2(x[2 * p] - __builtin_bit_cast(float, h << 16),
                     x[2 * p + 1] - __builtin_bit_cast(float, h & 0xFFFF0000u));
  }
}
// ... as fp16 (saturating)
__device__ __forceinline__ u32x4 pack_h(f32x4 a, f32x4 b) {
  return u32x4{pack2<f16_t>(a[0], a[1]), pack2<f16_t>(a[2], a[3]), pack2<f16_t>(b[0], b[1]),
               pack2<f16_t>(b[2], b[3])};
}
// fp16 (low 16 bits of w) -> fp32 as its own instruction.  Written as a
// C++ conversion inside x - hi, the compiler fuses it into a mixed-precision
// FMA with an f16 operand, and that form left hi unsubtracted here (lo came
// out equal to x).
__device__ __forceinline__ float h16_to_f(uint32_t w) {
  float f;
  asm("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(w));
  return f;
}
// ... as an fp16 hi + lo pair (about 22 significant bits)
__device__ __forceinline__ void split_h(f32x4 a, f32x4 b, u32x4& hi, u32x4& lo) {
  hi = pack_h(a, b);
  f32x4 ra, rb;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ra[2 * i] = a[2 * i] - h16_to_f(hi[i]);
    ra[2 * i + 1] = a[2 * i + 1] - h16_to_f(hi[i] >> 16);
    rb[2 * i] = b[2 * i] - h16_to_f(hi[2 + i]);
    rb[2 * i + 1] = b[2 * i + 1] - h16_to_f(hi[2 + i] >> 16);
  }
  lo = pack_h(ra, rb);
}

// 16 bytes per lane, global -> LDS; lane l's bytes land at lds + 16 l
__device__ __forceinline__ void dma16(const void* src, lchar* lds) {
  typedef __attribute__((address_space(1))) const void gvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)src, lds, 16, 0, 0);
}
// 4 bytes per lane, global -> LDS; lane l's bytes land at lds + 4 l
__device__ __forceinline__ void dma4(const void* src, lchar* lds) {
  typedef __attribute__((address_space(1))) const void gvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)src, lds, 4, 0, 0);
}
// one dword per lane into a landing area nobody reads: pulls the line into L2
__device__ __forceinline__ void touch4(const void* src, lchar* sink) {
  typedef __attribute__((address_space(1))) const void gvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)src, sink, 4, 0, 0);
}

// vector-memory operations a helper leaves in flight across the chunk's last
// barrier: the L2 prefetch loads issued after the chunk's data loads
constexpr int kTouches = 2;

template <int DK>
struct Lds {
  static constexpr int QK = BT * DK * 2;        // one q or k tile (bytes)
  static constexpr int AT = BT * BT * 2;        // one Ainv or Aqk tile (fp16)
  static constexpr int VT = BT * BV * 2;        // v tile
  static constexpr int OROW = BV * 2 + 16;      // padded o row (bytes)
  static constexpr int KS = DK / 32, KB = DK / 16;
  static constexpr int NQK = DK / 8;            // 1 KB loads per q / k tile
  static constexpr int QROWS = 512 / DK;        // q / k rows per 1 KB load
};

// Direct-to-LDS copies of one chunk's tiles (per-lane offsets precomputed;
// in the last chunk of a sequence, rows past its end repeat its last row).
template <int DK>
__device__ __forceinline__ void dma_qk_tile(const char* xc, const uint32_t* o_qk, int nr, uint32_t qk_row,
                                            lchar* dX, int lane) {
  typedef Lds<DK> L;
  if (nr == BT) {
#pragma unroll
    for (int i = 0; i < L::NQK; ++i) dma16(xc + o_qk[i], dX + 1024 * i);
  } else {
#pragma unroll
    for (int i = 0; i < L::NQK; ++i) {
      const int row = i * L::QROWS + lane / (DK / 8);
      const int rr = row < nr ? row : nr - 1;
      dma16(xc + (uint32_t)rr * qk_row + 16 * ((lane % (DK / 8)) ^ qk_swz<DK>(row)), dX + 1024 * i);
    }
  }
}
// A q / k-like tile stored head- and slab-major: for each 32-channel slab a
// block of [tokens][32] rows (64 bytes each), the slabs `slab_bytes` apart.
// Byte offset of the global unit that lands in LDS slot (row t, unit u): the
// unit u ^ swizzle(t) of row t, as for the row-major tiles.
template <int DK>
__device__ __forceinline__ uint32_t plane_off(int t, int u, uint32_t slab_bytes) {
  const int gu = u ^ qk_swz<DK>(t);
  return (uint32_t)(gu >> 2) * slab_bytes + (uint32_t)(t * 64 + ((gu & 3) << 4));
}
template <int DK>
__device__ __forceinline__ void dma_plane_tile(const char* xc, const uint32_t* o_pl, int nr,
                                               uint32_t slab_bytes, lchar* dX, int lane) {
  typedef Lds<DK> L;
  if (nr == BT) {
#pragma unroll
    for (int i = 0; i < L::NQK; ++i) dma16(xc + o_pl[i], dX + 1024 * i);
  } else {
#pragma unroll
    for (int i = 0; i < L::NQK; ++i) {
      const int row = i * L::QROWS + lane / (DK / 8);
      const int rr = row < nr ? row : nr - 1;
      // the unit of the clamped row at the position the swizzle of `row` selects
      const uint32_t off = plane_off<DK>(row, lane % (DK / 8), slab_bytes) - (uint32_t)(row - rr) * 64u;
      dma16(xc + off, dX + 1024 * i);
    }
  }
}
__device__ __forceinline__ void dma_a_tile(const char* ac, const uint32_t* o_a, int nr, uint32_t a_row,
                                           lchar* dA, int lane) {
  if (nr == BT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(ac + o_a[i], dA + 1024 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + lane / 8;
      const int rr = row < nr ? row : nr - 1;
      dma16(ac + (uint32_t)rr * a_row + 16 * ((lane % 8) ^ a_swz(row)), dA + 1024 * i);
    }
  }
}
// v tile of BVC columns: rows of 2 BVC bytes, BVC / 8 lanes per row
template <int BVC = BV>
__device__ __forceinline__ void dma_v_tile(const char* vc, const uint32_t* o_v, int nr, uint32_t v_row,
                                           lchar* dV, int lane) {
  constexpr int LPR = BVC / 8, RPL = 64 / LPR, NVL = BT / RPL;
  if (nr == BT) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) dma16(vc + o_v[i], dV + 1024 * i);
  } else {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int row = RPL * i + lane / LPR;
      const int rr = row < nr ? row : nr - 1;
      dma16(vc + (uint32_t)rr * v_row + 16 * (lane % LPR), dV + 1024 * i);
    }
  }
}


}  // namespace tiles
}  // namespace gdn
