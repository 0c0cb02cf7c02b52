// Device helpers shared by the intra-chunk kernels (GDN and KDA): chunk
// location for dense and packed batches, the 64 x 64 unit-lower solve
// (forward substitution on the four 16 x 16 diagonal blocks, then the block
// merge), and 16-byte row stores of a 64 x 64 LDS tile.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace intra {

constexpr int BT = 64;
constexpr int AP = 68;  // padded fp32 row of the 64 x 64 LDS tile

__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Work-group -> (chunk slot, v-head).  Work-group ids are dealt round-robin
// to the 8 XCDs, each with its own L2.  The order below puts the HV heads of
// a chunk slot on one XCD, next to each other in time, so that per-token
// arrays with the head innermost ([tokens, HV] gates and beta) come from HBM
// about once instead of once per head.  Returns false for padding ids.
__device__ __forceinline__ bool slot_of_block(int nslots, int HV, int& slot, int& j) {
  const int id = blockIdx.x;
  const int rest = id >> 3;
  j = rest % HV;
  slot = (rest / HV) * 8 + (id & 7);
  return slot < nslots;
}
inline unsigned intra_blocks(int nslots, int HV) { return (unsigned)(((nslots + 7) / 8) * 8 * HV); }

// Locate chunk slot c: sets [c0, c0 + nrow) and returns false when the slot
// is past the last chunk.
__device__ __forceinline__ bool locate_chunk(int c, const int64_t* __restrict__ cu,
                                             const int32_t* __restrict__ coff,
                                             int N, int T, int NT, int& c0, int& nrow) {
  int bos, eos, it;
  if (cu) {
    if (c >= coff[N]) return false;
    int lo = 0, hi = N;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (coff[mid] <= c) lo = mid; else hi = mid;
    }
    long long b0 = cu[lo], b1 = cu[lo + 1];
    b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
    b1 = b1 < b0 ? b0 : (b1 > T ? T : b1);
    bos = (int)b0;
    eos = (int)b1;
    it = c - coff[lo];
  } else {
    const int b = c / NT;
    it = c - b * NT;
    bos = b * T;
    eos = bos + T;
  }
  c0 = bos + BT * it;
  nrow = eos - c0 < BT ? eos - c0 : BT;
  return nrow > 0;
}

// Store the 64 x 64 fp32 LDS tile as rows of an [tokens, HV, 64] io-dtype
// array (rows >= nrow skipped), 16 bytes per lane and access.
// (part `part` of NPART: rows part * BT / NPART .. of the tile)
template <typename T, int NPART = 1>
__device__ __forceinline__ void store_tile(const float (*sA)[AP], T* __restrict__ out,
                                          int c0, int nrow, int HV, int j, int lane, int part = 0) {
  constexpr int PER = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int SEGS = BT / PER;             // vectors per row
  constexpr int ITS = BT * SEGS / 64 / NPART;
  static_assert(BT * SEGS % (64 * NPART) == 0, "whole iterations per part");
#pragma unroll
  for (int it = part * ITS; it < (part + 1) * ITS; ++it) {
    const int idx = it * 64 + lane;
    const int r = idx / SEGS, sg = idx % SEGS;
    if (r < nrow) {
      T* p = out + ((size_t)(c0 + r) * HV + j) * BT + sg * PER;
      if constexpr (sizeof(T) == 2) {
        uint4 w;
        const float* s = &sA[r][sg * 8];
        w.x = pack2<T>(s[0], s[1]);
        w.y = pack2<T>(s[2], s[3]);
        w.z = pack2<T>(s[4], s[5]);
        w.w = pack2<T>(s[6], s[7]);
        store_nt16(p, w);   // streaming: the scan reads these rows once, from memory anyway
      } else {
        const float* s = &sA[r][sg * 4];
        *reinterpret_cast<float4*>(p) = make_float4(s[0], s[1], s[2], s[3]);
      }
    }
  }
}

// tile index of lower block (rb, cb), cb <= rb
__host__ __device__ constexpr int tix(int rb, int cb) { return rb * (rb + 1) / 2 + cb; }

// -------------------------------------------------------------------------
// Solve (I + A)^-1 for the strictly lower 64 x 64 fp32 matrix held in sA and
// leave the inverse (unit lower, zero upper part) in sA.  Wave 0 does the
// forward substitution on the diagonal blocks.  The block merge has three
// independent column blocks (0: X10 -> X20 -> X30, 1: X21 -> X31, 2: X32);
// with NW = 1 wave 0 does all of them, with NW >= 3 waves 0, 1, 2 one each.
// Every wave of the work-group must call it (it holds block barriers).
// -------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ void solve_unit_lower_64(float (*sA)[AP], int lane, int wave) {
  static_assert(NW == 1 || NW >= 3, "one wave, or one wave per column block");
  const bool active = wave == 0;
  const int b = lane >> 4, jj = lane & 15;
  // forward substitution, column jj of diagonal block b
  float X[16];
  if (active) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* arow = &sA[16 * b + i][16 * b];
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int m = 0; m < i; m += 2) {
        acc0 = fmaf(arow[m], X[m], acc0);
        if (m + 1 < i) acc1 = fmaf(arow[m + 1], X[m + 1], acc1);
      }
      X[i] = (i == jj) ? 1.0f : ((i < jj) ? 0.0f : -(acc0 + acc1));
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[16 * b + i][16 * b + jj] = X[i];
  }
  __syncthreads();

  // block merge: X_rc = -X_rr * sum_{m=c}^{r-1} A_rm X_mc, fp32 MFMA 16x16x4.
  const int row = lane & 15, grp = lane >> 4;
  // A operand of block (br, bc): lane holds M[16br + row][16bc + 4grp + s]
  auto mmA = [&](int br, int bc, const f32x4& Bv, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * br + row][16 * bc + 4 * grp + s], Bv[s], c, 0, 0, 0);
    return c;
  };
  // B operand of diagonal block d from LDS, in accumulator layout
  auto diagB = [&](int d) {
    f32x4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = sA[16 * d + 4 * grp + s][16 * d + row];
    return r;
  };
  f32x4 X10, X20, X30, X21, X31, X32;
  auto put = [&](int br, int bc, const f32x4& Xv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sA[16 * br + 4 * grp + i][16 * bc + row] = Xv[i];
  };
  if constexpr (NW == 1) {
    if (active) {
      const f32x4 X00 = diagB(0), X11 = diagB(1), X22 = diagB(2);
      f32x4 P;
      // column block 0
      P = mmA(1, 0, X00, zero4());
      X10 = -mmA(1, 1, P, zero4());
      P = mmA(2, 0, X00, zero4());
      P = mmA(2, 1, X10, P);
      X20 = -mmA(2, 2, P, zero4());
      P = mmA(3, 0, X00, zero4());
      P = mmA(3, 1, X10, P);
      P = mmA(3, 2, X20, P);
      X30 = -mmA(3, 3, P, zero4());
      // column block 1
      P = mmA(2, 1, X11, zero4());
      X21 = -mmA(2, 2, P, zero4());
      P = mmA(3, 1, X11, zero4());
      P = mmA(3, 2, X21, P);
      X31 = -mmA(3, 3, P, zero4());
      // column block 2
      P = mmA(3, 2, X22, zero4());
      X32 = -mmA(3, 3, P, zero4());
    }
    __syncthreads();
    if (active) {
      put(1, 0, X10); put(2, 0, X20); put(3, 0, X30);
      put(2, 1, X21); put(3, 1, X31); put(3, 2, X32);
    }
  } else {
    // one column block per wave (the same products, in the same order)
    f32x4 P;
    if (wave == 0) {
      const f32x4 X00 = diagB(0);
      P = mmA(1, 0, X00, zero4());
      X10 = -mmA(1, 1, P, zero4());
      P = mmA(2, 0, X00, zero4());
      P = mmA(2, 1, X10, P);
      X20 = -mmA(2, 2, P, zero4());
      P = mmA(3, 0, X00, zero4());
      P = mmA(3, 1, X10, P);
      P = mmA(3, 2, X20, P);
      X30 = -mmA(3, 3, P, zero4());
    } else if (wave == 1) {
      const f32x4 X11 = diagB(1);
      P = mmA(2, 1, X11, zero4());
      X21 = -mmA(2, 2, P, zero4());
      P = mmA(3, 1, X11, zero4());
      P = mmA(3, 2, X21, P);
      X31 = -mmA(3, 3, P, zero4());
    } else if (wave == 2) {
      const f32x4 X22 = diagB(2);
      P = mmA(3, 2, X22, zero4());
      X32 = -mmA(3, 3, P, zero4());
    }
    __syncthreads();
    if (wave == 0) {
      put(1, 0, X10); put(2, 0, X20); put(3, 0, X30);
    } else if (wave == 1) {
      put(2, 1, X21); put(3, 1, X31);
    } else if (wave == 2) {
      put(3, 2, X32);
    }
  }
  __syncthreads();
}


}  // namespace intra
}  // namespace gdn
