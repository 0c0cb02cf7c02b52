// Prefill -> decode handoff, gfx950: the final fp32 states of a chunked
// prefill ([N, HV, V, K], K contiguous: "fla ops/common/chunk_h.py" ht in its
// state-V-first layout) are written into slots of the bf16 decode state pool
// ([pool, HV, V, K]: "flashinfer gdn_kernels/gdn_decode_bf16_state.py",
// initial_state_source indexed by initial_state_indices), each value rounded
// to the nearest bf16 (ties to even), as the decode step itself stores it.
//
// HBM-bound: 4 bytes read and 2 written per element, nothing else.  A
// work-group of 256 threads covers 2048 ITEMS consecutive elements of one
// (sequence, head) state; per 8 elements a thread reads two 16-byte fp32
// vectors and writes one 16-byte bf16 vector (each wave instruction touches
// 1 KiB of contiguous memory), all of its loads issued before its stores.
// Both directions are streaming accesses (each byte is touched once).

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int ITEMS = 1;                       // 8-element vectors per thread
constexpr int PER_BLOCK = 256 * 8 * ITEMS;     // elements per work-group

__global__ __launch_bounds__(256) void state_to_pool_kernel(
    const float* __restrict__ ht, const int32_t* __restrict__ idx, bf16_t* __restrict__ pool_state,
    int HV, long long VK, int blocks_per_state, int pool) {
  const int bid = blockIdx.x;
  const int sh = bid / blocks_per_state;          // (sequence, head)
  const int part = bid - sh * blocks_per_state;
  const int n = sh / HV, hv = sh - n * HV;
  const int slot = idx ? idx[n] : n;
  if (slot < 0 || slot >= pool) return;           // skipped, pool untouched
  const float* src = ht + (size_t)sh * VK;
  bf16_t* dst = pool_state + ((size_t)slot * HV + hv) * VK;
  // all loads first, then the stores; vector i of the thread covers elements
  // part * PER_BLOCK + 2048 i + 8 tid .. + 7
  float4 a[ITEMS], b[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const long long e0 = (long long)part * PER_BLOCK + 2048 * i + 8 * threadIdx.x;
    if (e0 < VK) {
      typedef float f4 __attribute__((ext_vector_type(4)));
      // read once: streaming (nontemporal) loads
      const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + e0));
      const f4 y = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + e0 + 4));
      a[i] = make_float4(x[0], x[1], x[2], x[3]);
      b[i] = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const long long e0 = (long long)part * PER_BLOCK + 2048 * i + 8 * threadIdx.x;
    if (e0 < VK) {
      uint4 w;
      w.x = pack_bf2(a[i].x, a[i].y);
      w.y = pack_bf2(a[i].z, a[i].w);
      w.z = pack_bf2(b[i].x, b[i].y);
      w.w = pack_bf2(b[i].z, b[i].w);
      store_nt16(dst + e0, w);
    }
  }
}

}  // namespace

hipError_t launch_state_to_pool(const float* ht, const int32_t* idx, void* pool_state, int N, int HV,
                                int K, int V, int pool, hipStream_t s) {
  const long long VK = (long long)V * K;
  const int per = (int)((VK + PER_BLOCK - 1) / PER_BLOCK);
  const long long blocks = (long long)N * HV * per;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(state_to_pool_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ht, idx,
                     (bf16_t*)pool_state, HV, VK, per, pool);
  return hipGetLastError();
}

}  // namespace gdn
