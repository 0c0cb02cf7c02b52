// Host-side launch helpers of the gfx950 kernels (internal to the library).
// Arguments have been validated by the C-ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Per-stage event timing (enabled through gdn_profile_enable).
void prof_begin(int stage, hipStream_t s);
void prof_end(int stage, hipStream_t s);

struct DecodeArgs {
  const void *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  void* state;
  const int32_t* idx;
  void* o;
  int B, T, H, HV, K, V, pool;
  float scale, sp_beta, sp_thr, eps;
  int use_norm;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// the state scans (bf16 io): backward state gradient (fwd = false; q, dout)
// or the forward decay-only state scan (fwd = true; k in q, v in dout, h0 in
// dht, the stored states in dh, ht in dh0)
struct BwdDhArgs {
  const void *q, *dout;
  const float *g, *g_gamma, *gk;   // at most one; Hg gate heads
  const float* gv;                 // [B*T, Hg, V] or nullptr; not with gk
  bool fwd;
  float scale;
  const float* dht;                // [N, HV, V, K] (v_first) or [N, HV, K, V], or nullptr
  void* dh;                        // [splits, HV, V, K] or [splits, HV, K, V], fp32 or bf16 (dh_bf16), or nullptr
  bool dh_bf16;
  long long dh_cap;                // entries of dh; later entries are not written
  int split_chunks;
  float* dh0;                      // [N, HV, V, K] or [N, HV, K, V], or nullptr
  bool v_first;                    // state layout: V-first (K contiguous) or key-first (V contiguous)
  const int64_t* cu_seqlens;
  int N, B, T, Hk, HV, K, V;
  int Hg;                          // gate heads (HV % Hg == 0)
};
hipError_t launch_bwd_dh(const BwdDhArgs& a, hipStream_t s);

// prefill -> decode handoff: fp32 [N, HV, V, K] into bf16 pool slots
hipError_t launch_state_to_pool(const float* ht, const int32_t* idx, void* pool_state, int N, int HV,
                                int K, int V, int pool, hipStream_t s);

// One chunked prefill problem (GDN: gk == nullptr; KDA: g == nullptr).
struct ChunkArgs {
  const void *q, *k, *v;
  const float *g, *gk, *beta;
  const float* g_gamma;  // [HV] fixed per-head log-decay per token (GDN) or nullptr
  float scale;
  const float* h0;
  float* ht;
  void* hs;              // [splits, HV, V, K] state snapshots (fp32, or bf16 when hs_bf16) or nullptr
  bool hs_bf16;
  long long hs_cap;      // entries of hs; later entries are not written
  int split_chunks;      // chunks per snapshot (split_size / 64)
  const int64_t* cu_seqlens;
  int N;                 // sequences (B without cu_seqlens)
  int B, T, Hk, HV, K, V;
  int bf16;              // 1 = bf16 io, 0 = fp32 io
  void* o;
  void* Ainv;            // [B*T, HV, 64] compute dtype: (I + A)^-1 rows
  void* Aqk;             // [B*T, HV, 64] compute dtype: scale * gated causal Q K^T rows
  void* GF;              // float [HV][4][B*T]: planes e^G, e^{G_last - G}, beta, e^{G_last}
                         // per token (head-major)
  int32_t* chunk_off;    // [N + 1] varlen chunk offsets (workspace) or nullptr
  int32_t* seq_order;    // [N] sequences, longest first (workspace) or nullptr
  int max_chunks;        // upper bound of the total chunk count
};
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t s);
// Token stride of a gate-factor plane.
__host__ __device__ inline long long gf_stride(long long tokens) { return tokens; }

// First state snapshot of sequence n: a sequence of L tokens has
// ceil(L / S) snapshots (S = split tokens), stored back to back in sequence
// order.  Varlen boundaries are clamped as the scans clamp them.  Called by
// all 64 lanes of a wave with the same arguments: lane l sums sequences
// l, l + 64, ..., so the loads of 64 sequences are in flight together, and
// the partial sums are combined across the wave.
__device__ inline long long snapshot_offset(const int64_t* cu, int n, int Tlen, int S) {
  if (!cu) return (long long)n * ((Tlen + S - 1) / S);
  long long acc = 0;
  for (int m = (int)(threadIdx.x & 63); m < n; m += 64) {
    long long b0 = cu[m], b1 = cu[m + 1];
    b0 = b0 < 0 ? 0 : (b0 > Tlen ? Tlen : b0);
    b1 = b1 < b0 ? b0 : (b1 > Tlen ? Tlen : b1);
    acc += (b1 - b0 + S - 1) / S;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  return acc;
}
// bf16 GDN and KDA scans (direct-to-LDS staging, state / helper / mover waves);
// KDA reads the gated operands and decay rows of KdaBuffers
hipError_t launch_scan_gdn_bf16(const ChunkArgs& a, hipStream_t s);
hipError_t launch_scan_kda_bf16(const ChunkArgs& a, const void* qg, const void* kg, const void* kt,
                                const float* dg, hipStream_t s);

// Extra buffers of the KDA path.
struct KdaBuffers {
  void* Aqk_out;         // [B*T, HV, 64] io dtype output or nullptr
  void* Akk_out;         // [B*T, HV, 64] io dtype output or nullptr
  void *qg, *kg, *kt;    // [B*T, HV, K] compute dtype: Q o e^G, K o e^G, K o e^{G_last - G}
  float* dg;             // [chunks, HV, K] e^{G_last}
};
hipError_t launch_kda_fwd(const ChunkArgs& a, const KdaBuffers& kb, hipStream_t s);

// The scalar-gate intra-chunk step on its own: A = (I + L)^-1, w, u.
struct IntraArgs {
  const void *k, *v;               // [B*T, Hk, K], [B*T, HV, V] io dtype
  const float* g;                  // [B*T, HV] log-gates or their chunk-local sums, or nullptr
  bool g_cumulative;               // g holds chunk-local cumulative sums
  const float* beta;               // [B*T, HV]
  void *A, *w, *u;                 // [B*T, HV, 64], [B*T, HV, K], [B*T, HV, V] io dtype; w, u optional
  const int64_t* cu_seqlens;
  int32_t* chunk_off;              // [N + 1] varlen chunk offsets (workspace) or nullptr
  int N, B, T, Hk, HV, K, V;
  int bf16;
};
hipError_t launch_intra_wu(const IntraArgs& a, hipStream_t s);

// Workspace layout shared by the size query and the launcher.
struct ChunkWorkspace {
  size_t ainv_off, aqk_off, gf_off, coff_off, order_off;
  size_t qg_off, kg_off, kt_off, dg_off;  // KDA only
  size_t total;
};
ChunkWorkspace chunk_workspace_layout(long long tokens, int HV, int K, int N, int max_chunks,
                                      int elem_bytes, bool kda);

}  // namespace gdn
