// C ABI of the library: argument validation (host only, before any HIP call),
// workspace layout, and the launch sequence of each entry point.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "gdn61.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

hipError_t launch_intra_gdn(const ChunkArgs& a, hipStream_t s, int NT, int nslots);
hipError_t launch_scan_gdn(const ChunkArgs& a, hipStream_t s);
hipError_t launch_intra_kda(const ChunkArgs& a, const KdaBuffers& kb, hipStream_t s, int NT,
                            int nslots);
hipError_t launch_scan_kda(const ChunkArgs& a, const void* qg, const void* kg, const void* kt,
                           const float* dg, hipStream_t s);

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return GDN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr size_t ALIGN = 256;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Chunk tables for packed variable-length batches: chunk offsets (exclusive
// prefix of ceil(len / 64)) and the sequence order by decreasing length.
// One work-group; N up to any size for the offsets, the order is sorted for
// N <= 1024 and left as the identity beyond.  For N <= 1024 the (clamped)
// lengths are read from global memory once, one per thread, and kept in LDS,
// so the ranking loop does not wait out a memory round trip per sequence.
__global__ __launch_bounds__(1024) void varlen_tables_kernel(const int64_t* __restrict__ cu, int N,
                                                              int T, int32_t* __restrict__ coff,
                                                              int32_t* __restrict__ order) {
  __shared__ int32_t part[1024];
  __shared__ int32_t slen[1024];
  const int t = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int lo = t * per, hi = lo + per < N ? lo + per : N;
  auto len_g = [&](int i) {
    long long b0 = cu[i], b1 = cu[i + 1];
    b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
    b1 = b1 < b0 ? b0 : (b1 > T ? T : b1);
    return (int)(b1 - b0);
  };
  const bool staged = N <= 1024;   // uniform
  if (staged) {
    if (t < N) slen[t] = len_g(t);
    __syncthreads();
  }
  auto len = [&](int i) { return staged ? slen[i] : len_g(i); };
  int s = 0;
  for (int i = lo; i < hi; ++i) s += (len(i) + 63) / 64;
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    coff[i] = run;
    run += (len(i) + 63) / 64;
  }
  if (t == 1023) coff[N] = part[1023];
  if (N <= 1024) {
    if (t < N) {
      const int li = len(t);
      int rank = 0;
      for (int m = 0; m < N; ++m) {
        const int lm = len(m);
        rank += (lm > li) || (lm == li && m < t);
      }
      order[rank] = t;
    }
  } else {
    for (int i = t; i < N; i += 1024) order[i] = i;
  }
}

struct Problem {
  int B, T, Hk, HV, K, V, N;
};

// Checks of the stored-state arguments shared by the prefill and the state
// scans: split size, dtype, capacity (dense batches: every entry must fit).
int check_states(const void* snaps, int split_size, long long entries, int state_dtype, bool varlen,
                 int B, int T, const char* name) {
  if (!snaps) return GDN_OK;
  if (split_size <= 0 || split_size % 64 != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "split_size must be a positive multiple of 64 (got %d)", split_size);
  if (state_dtype != GDN_DTYPE_F32 && state_dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown state dtype code %d", state_dtype);
  if (entries < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s entries must be >= 0", name);
  const long long need = (long long)B * ((T + split_size - 1) / split_size);
  if (!varlen && entries < need)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s holds %lld entries, %lld needed", name, entries, need);
  return GDN_OK;
}

int check_chunk(const void* q, const void* k, const void* v, const float* gate,
                bool gate_required, const float* beta, const float* h0, float* ht,
                const void* h_snap, int split_size, long long snap_entries, int state_dtype,
                const int64_t* cu, int num_seqs, int B, int T, int Hk, int HV, int K, int V,
                int chunk_size, int dtype, const void* o, Problem& P) {
  if (B < 0 || T < 0 || Hk <= 0 || HV <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be positive (B, T >= 0): B=%d T=%d Hk=%d HV=%d K=%d V=%d",
                B, T, Hk, HV, K, V);
  if (HV % Hk != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "HV (%d) must be a multiple of Hk (%d)", HV, Hk);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown dtype code %d", dtype);
  if (chunk_size != 64)
    return fail(GDN_ERR_UNSUPPORTED, "chunk_size must be 64 (got %d)", chunk_size);
  if (!((K == 64 && V == 64) || (K == 128 && V == 128)))
    return fail(GDN_ERR_UNSUPPORTED, "supported head dims are K = V in {64, 128} (got K=%d V=%d)", K, V);
  if ((long long)B * T >= (1LL << 31) / 64)
    return fail(GDN_ERR_UNSUPPORTED, "B*T too large (got %lld tokens)", (long long)B * T);
  if (cu) {
    if (B != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
    if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
    P.N = num_seqs;
  } else {
    P.N = B;
  }
  {
    // the launches index chunk slots, (sequence, head) pairs and their
    // tiles (at most 8 per pair) with 32-bit integers
    const long long slots = cu ? (long long)(T + 63) / 64 + P.N : (long long)B * ((T + 63) / 64);
    if ((slots + 8) * HV * 8 >= (1LL << 31) || ((long long)P.N * HV + 8) * 8 >= (1LL << 31))
      return fail(GDN_ERR_UNSUPPORTED, "too many chunks or sequences x heads for one launch (N=%d HV=%d)", P.N,
                  HV);
  }
  const bool work = (long long)B * T > 0;
  if (work && (!q || !k || !v || !beta || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, beta and o are required");
  if (work && gate_required && !gate) return fail(GDN_ERR_INVALID_ARGUMENT, "gk is required");
  {
    const int st = check_states(h_snap, split_size, snap_entries, state_dtype, cu != nullptr, B, T, "h_snap");
    if (st != GDN_OK) return st;
  }
  const void* ptrs[] = {q, k, v, gate, beta, h0, ht, h_snap, o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDN_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  P.B = B; P.T = T; P.Hk = Hk; P.HV = HV; P.K = K; P.V = V;
  return GDN_OK;
}

}  // namespace

// ---------------------------------------------------------------- profiler
namespace {
struct ProfRec {
  int stage;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;     // recorded, not yet read
std::vector<hipEvent_t> g_prof_free;  // reusable events
hipEvent_t prof_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
thread_local hipEvent_t t_open[GDN_STAGE_COUNT];
}  // namespace

void prof_begin(int stage, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  hipEvent_t e = prof_event();
  if (e && hipEventRecord(e, s) == hipSuccess) t_open[stage] = e;
}

void prof_end(int stage, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || !t_open[stage]) return;
  hipEvent_t e = prof_event();
  if (e && hipEventRecord(e, s) == hipSuccess) g_prof_recs.push_back({stage, t_open[stage], e});
  t_open[stage] = nullptr;
}

ChunkWorkspace chunk_workspace_layout(long long tokens, int HV, int K, int N, int max_chunks,
                                      int elem_bytes, bool kda) {
  ChunkWorkspace w;
  const size_t mat = (size_t)tokens * HV * 64 * elem_bytes;
  w.ainv_off = 0;
  w.aqk_off = up(mat);
  w.gf_off = w.aqk_off + up(mat);
  w.coff_off = w.gf_off + up((size_t)gf_stride(tokens) * HV * 16);
  w.order_off = w.coff_off + up((size_t)(N + 1) * 4);
  size_t end = w.order_off + up((size_t)(N > 0 ? N : 1) * 4);
  w.qg_off = w.kg_off = w.kt_off = w.dg_off = 0;
  if (kda) {
    const size_t op = (size_t)tokens * HV * K * elem_bytes;
    w.qg_off = end;
    w.kg_off = w.qg_off + up(op);
    w.kt_off = w.kg_off + up(op);
    w.dg_off = w.kt_off + up(op);
    end = w.dg_off + up((size_t)(max_chunks > 0 ? max_chunks : 1) * HV * K * 4);
  }
  w.total = end;
  return w;
}

hipError_t launch_kda_fwd(const ChunkArgs& a, const KdaBuffers& kb, hipStream_t s) {
  if (a.cu_seqlens) {
    prof_begin(GDN_STAGE_VARLEN_TABLES, s);
    hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.N, a.T,
                       a.chunk_off, a.seq_order);
    hipError_t e = hipGetLastError();
    prof_end(GDN_STAGE_VARLEN_TABLES, s);
    if (e != hipSuccess) return e;
  }
  const int NT = (a.T + 63) / 64;
  const int nslots = a.cu_seqlens ? NT + a.N : a.B * NT;
  if (nslots > 0 && (long long)a.B * a.T > 0) {
    prof_begin(GDN_STAGE_INTRA, s);
    hipError_t e = launch_intra_kda(a, kb, s, NT, nslots);
    prof_end(GDN_STAGE_INTRA, s);
    if (e != hipSuccess) return e;
  }
  prof_begin(GDN_STAGE_SCAN, s);
  const hipError_t e = launch_scan_kda(a, kb.qg, kb.kg, kb.kt, kb.dg, s);
  prof_end(GDN_STAGE_SCAN, s);
  return e;
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t s) {
  if (a.cu_seqlens) {
    prof_begin(GDN_STAGE_VARLEN_TABLES, s);
    hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.N, a.T,
                       a.chunk_off, a.seq_order);
    hipError_t e = hipGetLastError();
    prof_end(GDN_STAGE_VARLEN_TABLES, s);
    if (e != hipSuccess) return e;
  }
  const int NT = (a.T + 63) / 64;
  const int nslots = a.cu_seqlens ? NT + a.N : a.B * NT;
  if (nslots > 0 && (long long)a.B * a.T > 0) {
    prof_begin(GDN_STAGE_INTRA, s);
    hipError_t e = launch_intra_gdn(a, s, NT, nslots);
    prof_end(GDN_STAGE_INTRA, s);
    if (e != hipSuccess) return e;
  }
  prof_begin(GDN_STAGE_SCAN, s);
  const hipError_t e = launch_scan_gdn(a, s);
  prof_end(GDN_STAGE_SCAN, s);
  return e;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

const char* gdn_version(void) { return "gdn61 0.1 gfx950"; }

size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int Hk, int HV, int K, int V, int num_seqs,
                                     int dtype) {
  if (B < 0 || T < 0 || Hk <= 0 || HV <= 0 || K <= 0 || V <= 0 || num_seqs < 0) return 0;
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return 0;
  const int N = num_seqs > B ? num_seqs : B;
  const int maxc = (T + 63) / 64 * B + N;
  return chunk_workspace_layout((long long)B * T, HV, K, N, maxc, dtype == GDN_DTYPE_BF16 ? 2 : 4,
                                false).total;
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int Hk, int HV, int K, int V, int num_seqs,
                                     int dtype) {
  if (B < 0 || T < 0 || Hk <= 0 || HV <= 0 || K <= 0 || V <= 0 || num_seqs < 0) return 0;
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return 0;
  const int N = num_seqs > B ? num_seqs : B;
  const int maxc = (T + 63) / 64 * B + N;
  return chunk_workspace_layout((long long)B * T, HV, K, N, maxc, dtype == GDN_DTYPE_BF16 ? 2 : 4,
                                true).total;
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* g_gamma, const float* beta, float scale, const float* h0, float* ht,
                  void* h_snap, int split_size, long long snap_entries, int state_dtype,
                  const int64_t* cu_seqlens,
                  int num_seqs, int B, int T, int Hk, int HV, int K, int V, int chunk_size,
                  int dtype, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  Problem P;
  int st = check_chunk(q, k, v, g, false, beta, h0, ht, h_snap, split_size, snap_entries, state_dtype,
                       cu_seqlens, num_seqs, B, T, Hk, HV, K, V, chunk_size, dtype, o, P);
  if (st != GDN_OK) return st;
  if (g && g_gamma) return fail(GDN_ERR_INVALID_ARGUMENT, "pass g or g_gamma, not both");
  const int eb = dtype == GDN_DTYPE_BF16 ? 2 : 4;
  const ChunkWorkspace L = chunk_workspace_layout((long long)B * T, HV, K, P.N,
                                                  (T + 63) / 64 * B + P.N, eb, false);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (P.N == 0) return ok();
  char* ws = (char*)workspace;
  ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.g_gamma = g_gamma; a.gk = nullptr; a.beta = beta; a.scale = scale;
  a.h0 = h0; a.ht = ht; a.cu_seqlens = cu_seqlens; a.N = P.N;
  a.hs = h_snap; a.split_chunks = h_snap ? split_size / 64 : 1;
  a.hs_bf16 = h_snap && state_dtype == GDN_DTYPE_BF16;
  a.hs_cap = h_snap ? snap_entries : 0;
  a.B = B; a.T = T; a.Hk = Hk; a.HV = HV; a.K = K; a.V = V;
  a.bf16 = dtype == GDN_DTYPE_BF16;
  a.o = o;
  a.Ainv = ws + L.ainv_off;
  a.Aqk = ws + L.aqk_off;
  a.GF = ws + L.gf_off;
  a.chunk_off = cu_seqlens ? (int32_t*)(ws + L.coff_off) : nullptr;
  a.seq_order = cu_seqlens ? (int32_t*)(ws + L.order_off) : nullptr;
  a.max_chunks = (T + 63) / 64 * B + (cu_seqlens ? P.N : 0);
  const hipError_t e = launch_chunk_fwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t gdn_chunk_intra_workspace_bytes(int num_seqs) {
  if (num_seqs < 0) return 0;
  return ((2 * (size_t)num_seqs + 1) * sizeof(int32_t) + 255) / 256 * 256;   // chunk offsets, order
}

int gdn_chunk_intra(const void* k, const void* v, const float* g, int g_cumulative, const float* beta,
                    const int64_t* cu_seqlens, int num_seqs, int B, int T, int Hk, int HV, int K, int V,
                    int chunk_size, int dtype, void* A, void* w, void* u, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || Hk <= 0 || HV <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be positive (B, T >= 0): B=%d T=%d Hk=%d HV=%d K=%d V=%d",
                B, T, Hk, HV, K, V);
  if (HV % Hk != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "HV (%d) must be a multiple of Hk (%d)", HV, Hk);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown dtype code %d", dtype);
  if (g_cumulative != 0 && g_cumulative != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "g_cumulative must be 0 or 1 (got %d)", g_cumulative);
  if (chunk_size != 64) return fail(GDN_ERR_UNSUPPORTED, "chunk_size must be 64 (got %d)", chunk_size);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(GDN_ERR_UNSUPPORTED, "supported head dims are K, V in {64, 128} (got K=%d V=%d)", K, V);
  if ((long long)B * T >= (1LL << 31) / 64)
    return fail(GDN_ERR_UNSUPPORTED, "B*T too large (got %lld tokens)", (long long)B * T);
  int N = B;
  if (cu_seqlens) {
    if (B != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
    if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
    N = num_seqs;
  }
  {
    const long long slots = cu_seqlens ? (long long)(T + 63) / 64 + N : (long long)B * ((T + 63) / 64);
    if ((slots + 8) * HV * 8 >= (1LL << 31))
      return fail(GDN_ERR_UNSUPPORTED, "too many chunks x heads for one launch (HV=%d)", HV);
  }
  const bool work = (long long)B * T > 0 && N > 0;
  if (work && (!k || !beta || !A)) return fail(GDN_ERR_INVALID_ARGUMENT, "k, beta and A are required");
  if (work && u && !v) return fail(GDN_ERR_INVALID_ARGUMENT, "v is required for u");
  const void* ptrs[] = {k, v, A, w, u};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDN_ERR_INVALID_ARGUMENT, "k, v, A, w and u must be 16-byte aligned");
  if (cu_seqlens) {
    const size_t need = gdn_chunk_intra_workspace_bytes(N);
    if (!workspace || workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  if (!work) return ok();
  IntraArgs a;
  a.k = k; a.v = v; a.g = g; a.g_cumulative = g_cumulative != 0; a.beta = beta;
  a.A = A; a.w = w; a.u = u; a.cu_seqlens = cu_seqlens;
  a.chunk_off = cu_seqlens ? (int32_t*)workspace : nullptr;
  a.N = N; a.B = B; a.T = T; a.Hk = Hk; a.HV = HV; a.K = K; a.V = V;
  a.bf16 = dtype == GDN_DTYPE_BF16;
  const hipStream_t s = (hipStream_t)stream;
  prof_begin(GDN_STAGE_INTRA, s);
  hipError_t e = hipSuccess;
  if (cu_seqlens) {
    hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(1024), 0, s, cu_seqlens, N, T, a.chunk_off,
                       a.chunk_off + N + 1);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = launch_intra_wu(a, s);
  prof_end(GDN_STAGE_INTRA, s);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ------------------------------------------------ no-allocation prefill entry
namespace {
// Scratch of gdn_chunk_fwd_noalloc: the workspace of gdn_chunk_fwd, one copy
// per GPU, held until the process ends.  On the host this name is only a
// stand-in, never an address: host code uses the per-device address that
// scratch_address() looks up.
constexpr size_t kScratchBytes = (size_t)96 << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device of `stream` (which must be the
// current device), looked up once per device.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(GDN_ERR_INVALID_ARGUMENT, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "device %d is beyond the %d devices the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GDN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}
}  // namespace

extern "C" {

size_t gdn_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const float* g_gamma, const float* beta, float scale, const float* h0, float* ht,
                          void* h_snap, int split_size, long long snap_entries, int state_dtype,
                          const int64_t* cu_seqlens,
                          int num_seqs, int B, int T, int Hk, int HV, int K, int V, int chunk_size,
                          int dtype, void* o, void* stream) {
  const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, Hk, HV, K, V, num_seqs, dtype);
  if (need > kScratchBytes)
    return fail(GDN_ERR_UNSUPPORTED,
                "the call needs %zu bytes of scratch; the no-allocation entry point holds %zu (use gdn_chunk_fwd "
                "with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  const int st = scratch_address((hipStream_t)stream, &ws);
  if (st != GDN_OK) return st;
  return gdn_chunk_fwd(q, k, v, g, g_gamma, beta, scale, h0, ht, h_snap, split_size, snap_entries, state_dtype,
                       cu_seqlens, num_seqs, B, T, Hk, HV, K, V, chunk_size, dtype, o, ws, kScratchBytes, stream);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* gk, const float* beta,
                  float scale, const float* h0, float* ht,
                  void* h_snap, int split_size, long long snap_entries, int state_dtype,
                  const int64_t* cu_seqlens,
                  int num_seqs, int B, int T, int Hk, int HV, int K, int V, int chunk_size,
                  int dtype, void* o, void* Aqk, void* Akk_inv, void* workspace,
                  size_t workspace_bytes, void* stream) {
  Problem P;
  int st = check_chunk(q, k, v, gk, true, beta, h0, ht, h_snap, split_size, snap_entries, state_dtype,
                       cu_seqlens, num_seqs, B, T, Hk, HV, K, V, chunk_size, dtype, o, P);
  if (st != GDN_OK) return st;
  if ((Aqk && !aligned16(Aqk)) || (Akk_inv && !aligned16(Akk_inv)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  // the gated planes of one head span B*T*K*2 bytes, addressed with 32-bit offsets
  if ((long long)B * T * K * 2 >= (1LL << 32))
    return fail(GDN_ERR_UNSUPPORTED, "B*T too large for KDA (got %lld tokens)", (long long)B * T);
  const int eb = dtype == GDN_DTYPE_BF16 ? 2 : 4;
  const ChunkWorkspace L = chunk_workspace_layout((long long)B * T, HV, K, P.N,
                                                  (T + 63) / 64 * B + P.N, eb, true);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (P.N == 0) return ok();
  char* ws = (char*)workspace;
  ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.g = nullptr; a.g_gamma = nullptr; a.gk = gk; a.beta = beta; a.scale = scale;
  a.h0 = h0; a.ht = ht; a.cu_seqlens = cu_seqlens; a.N = P.N;
  a.hs = h_snap; a.split_chunks = h_snap ? split_size / 64 : 1;
  a.hs_bf16 = h_snap && state_dtype == GDN_DTYPE_BF16;
  a.hs_cap = h_snap ? snap_entries : 0;
  a.B = B; a.T = T; a.Hk = Hk; a.HV = HV; a.K = K; a.V = V;
  a.bf16 = dtype == GDN_DTYPE_BF16;
  a.o = o;
  a.Ainv = ws + L.ainv_off;
  a.Aqk = ws + L.aqk_off;
  a.GF = ws + L.gf_off;
  a.chunk_off = cu_seqlens ? (int32_t*)(ws + L.coff_off) : nullptr;
  a.seq_order = cu_seqlens ? (int32_t*)(ws + L.order_off) : nullptr;
  a.max_chunks = (T + 63) / 64 * B + P.N;
  KdaBuffers kb;
  kb.Aqk_out = Aqk;
  kb.Akk_out = Akk_inv;
  kb.qg = ws + L.qg_off;
  kb.kg = ws + L.kg_off;
  kb.kt = ws + L.kt_off;
  kb.dg = (float*)(ws + L.dg_off);
  const hipError_t e = launch_kda_fwd(a, kb, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

int gdn_decode(const void* q, const void* k, const void* v, const void* a, const void* b,
               const float* A_log, const float* dt_bias, void* state,
               const int32_t* state_indices, void* o, int B, int T, int H, int HV, int K, int V,
               int pool, float scale, float softplus_beta, float softplus_threshold,
               int use_qk_l2norm, float eps, void* stream) {
  if (B < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || pool < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be positive: B=%d H=%d HV=%d K=%d V=%d pool=%d",
                B, H, HV, K, V, pool);
  if (T < 1 || T > 4) return fail(GDN_ERR_INVALID_ARGUMENT, "decode supports T = 1..4 (got T=%d)", T);
  if (HV % H != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "HV (%d) must be a multiple of H (%d)", HV, H);
  if (K != 128 || V != 128)
    return fail(GDN_ERR_UNSUPPORTED, "decode supports K = V = 128 (got K=%d V=%d)", K, V);
  if (!state_indices && pool < B)
    return fail(GDN_ERR_INVALID_ARGUMENT, "identity slots need pool >= B (pool=%d B=%d)", pool, B);
  if (!(softplus_beta > 0.f)) return fail(GDN_ERR_INVALID_ARGUMENT, "softplus_beta must be > 0");
  if (!(eps >= 0.f)) return fail(GDN_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (B == 0) return ok();
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state || !o)
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, a, b, A_log, dt_bias, state and o are required");
  const void* ptrs[] = {q, k, v, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, state and o must be 16-byte aligned");
  if ((long long)pool * HV * V * K >= (1LL << 40)) return fail(GDN_ERR_UNSUPPORTED, "state pool too large");
  // up to four work-groups per (batch row, v-head), indexed with 32-bit integers
  if ((long long)B * HV * 4 >= (1LL << 31))
    return fail(GDN_ERR_UNSUPPORTED, "too many batch rows x heads for one launch (B=%d HV=%d)", B, HV);
  DecodeArgs d;
  d.q = q; d.k = k; d.v = v; d.a = a; d.b = b; d.A_log = A_log; d.dt_bias = dt_bias;
  d.state = state; d.idx = state_indices; d.o = o;
  d.B = B; d.T = T; d.H = H; d.HV = HV; d.K = K; d.V = V; d.pool = pool;
  d.scale = scale; d.sp_beta = softplus_beta; d.sp_thr = softplus_threshold; d.eps = eps;
  d.use_norm = use_qk_l2norm != 0;
  prof_begin(GDN_STAGE_DECODE, (hipStream_t)stream);
  const hipError_t e = launch_decode(d, (hipStream_t)stream);
  prof_end(GDN_STAGE_DECODE, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

// checks and launch shared by the two state scans; a = A operand (q / k),
// b = B operand (dout / v), init / snaps / fin = dht, dh, dh0 (h0, h, ht)
static int state_scan(bool fwd, int stage, const void* a_op, const void* b_op, const float* g,
                      const float* g_gamma, const float* gk, const float* gv, int num_gate_heads,
                      float scale, const float* init, void* snaps, int split_size, long long entries,
                      int state_dtype, int state_v_first, float* fin,
                      const int64_t* cu_seqlens, int num_seqs, int B, int T, int Hk, int HV, int K, int V,
                      int chunk_size, int dtype, void* stream) {
  const char* an = fwd ? "k" : "q";
  const char* bn = fwd ? "v" : "dout";
  if (B < 0 || T < 0 || Hk <= 0 || HV <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be positive (B, T >= 0): B=%d T=%d Hk=%d HV=%d K=%d V=%d",
                B, T, Hk, HV, K, V);
  if (HV % Hk != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "HV (%d) must be a multiple of Hk (%d)", HV, Hk);
  const int Hg = num_gate_heads == 0 ? HV : num_gate_heads;
  if (Hg < 0 || HV % Hg != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "HV (%d) must be a multiple of the gate heads (%d)", HV, Hg);
  if (dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_UNSUPPORTED, "the state scans take bf16 io only");
  if (chunk_size != 64) return fail(GDN_ERR_UNSUPPORTED, "chunk_size must be 64 (got %d)", chunk_size);
  if (!((K == 64 && V == 64) || (K == 128 && V == 128)))
    return fail(GDN_ERR_UNSUPPORTED, "supported head dims are K = V in {64, 128} (got K=%d V=%d)", K, V);
  if ((g != nullptr) + (g_gamma != nullptr) + (gk != nullptr) > 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "pass at most one of g, g_gamma and gk");
  if (gk && gv) return fail(GDN_ERR_UNSUPPORTED, "gk together with gv is not supported");
  if (state_v_first != 0 && state_v_first != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "state_v_first must be 0 or 1 (got %d)", state_v_first);
  if ((long long)B * T >= (1LL << 31) / 64)
    return fail(GDN_ERR_UNSUPPORTED, "B*T too large (got %lld tokens)", (long long)B * T);
  {
    const int st = check_states(snaps, split_size, entries, state_dtype, cu_seqlens != nullptr, B, T,
                                fwd ? "h" : "dh");
    if (st != GDN_OK) return st;
  }
  int N = B;
  if (cu_seqlens) {
    if (B != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
    if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
    N = num_seqs;
  }
  // the launch indexes (sequence, head) pairs and their tiles (at most 8 per
  // pair) with 32-bit integers
  if (((long long)N * HV + 8) * 8 >= (1LL << 31))
    return fail(GDN_ERR_UNSUPPORTED, "too many sequences x heads for one launch (N=%d HV=%d)", N, HV);
  if ((long long)B * T > 0 && (!a_op || !b_op))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s and %s are required", an, bn);
  const void* ptrs[] = {a_op, b_op, g, g_gamma, gk, gv, init, snaps, fin};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDN_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if (N == 0 || (!snaps && !fin)) return ok();
  BwdDhArgs a;
  a.q = a_op; a.dout = b_op; a.g = g; a.g_gamma = g_gamma; a.gk = gk; a.gv = gv; a.fwd = fwd;
  a.scale = scale; a.dht = init; a.dh = snaps; a.split_chunks = snaps ? split_size / 64 : 1; a.dh0 = fin;
  a.dh_bf16 = snaps && state_dtype == GDN_DTYPE_BF16;
  a.dh_cap = snaps ? entries : 0;
  a.cu_seqlens = cu_seqlens; a.N = N; a.B = B; a.T = T; a.Hk = Hk; a.HV = HV; a.K = K; a.V = V;
  a.Hg = Hg;
  a.v_first = state_v_first != 0;
  prof_begin(stage, (hipStream_t)stream);
  const hipError_t e = launch_bwd_dh(a, (hipStream_t)stream);
  prof_end(stage, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

int gdn_chunk_bwd_dh(const void* q, const void* dout, const float* g, const float* g_gamma,
                     const float* gk, const float* gv, int num_gate_heads, float scale,
                     const float* dht, void* dh, int split_size, long long dh_entries, int state_dtype,
                     int state_v_first, float* dh0, const int64_t* cu_seqlens, int num_seqs, int B, int T,
                     int Hk, int HV, int K, int V, int chunk_size, int dtype, void* stream) {
  return state_scan(false, GDN_STAGE_BWD_DH, q, dout, g, g_gamma, gk, gv, num_gate_heads, scale, dht, dh,
                    split_size, dh_entries, state_dtype, state_v_first, dh0, cu_seqlens, num_seqs, B, T, Hk,
                    HV, K, V, chunk_size, dtype, stream);
}

int gdn_chunk_fwd_h(const void* k, const void* v, const float* g, const float* g_gamma,
                    const float* gk, const float* gv, int num_gate_heads, const float* h0, void* h,
                    int split_size, long long h_entries, int state_dtype, int state_v_first, float* ht,
                    const int64_t* cu_seqlens, int num_seqs, int B, int T, int Hk, int HV,
                    int K, int V, int chunk_size, int dtype, void* stream) {
  return state_scan(true, GDN_STAGE_FWD_H, k, v, g, g_gamma, gk, gv, num_gate_heads, 1.f, h0, h, split_size,
                    h_entries, state_dtype, state_v_first, ht, cu_seqlens, num_seqs, B, T, Hk, HV, K, V,
                    chunk_size, dtype, stream);
}

int gdn_state_to_pool(const float* ht, const int32_t* indices, void* pool_state, int N, int HV,
                      int K, int V, int pool, void* stream) {
  if (N < 0 || HV <= 0 || K <= 0 || V <= 0 || pool < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be positive: N=%d HV=%d K=%d V=%d pool=%d", N,
                HV, K, V, pool);
  if (((long long)V * K) % 8 != 0)
    return fail(GDN_ERR_UNSUPPORTED, "V * K must be a multiple of 8 (got V=%d K=%d)", V, K);
  if (!indices && pool < N)
    return fail(GDN_ERR_INVALID_ARGUMENT, "identity slots need pool >= N (pool=%d N=%d)", pool, N);
  if ((long long)(N > pool ? N : pool) * HV * V * K >= (1LL << 40))
    return fail(GDN_ERR_UNSUPPORTED, "state arrays too large");
  if (N == 0) return ok();
  if (!ht || !pool_state) return fail(GDN_ERR_INVALID_ARGUMENT, "ht and pool_state are required");
  if (!aligned16(ht) || !aligned16(pool_state))
    return fail(GDN_ERR_INVALID_ARGUMENT, "ht and pool_state must be 16-byte aligned");
  prof_begin(GDN_STAGE_HANDOFF, (hipStream_t)stream);
  const hipError_t e = launch_state_to_pool(ht, indices, pool_state, N, HV, K, V, pool, (hipStream_t)stream);
  prof_end(GDN_STAGE_HANDOFF, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

int gdn_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return GDN_OK;
}

int gdn_profile_read(double* ms, int* counts) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof_recs);
  }
  int status = GDN_OK;
  for (const ProfRec& r : recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      status = fail(GDN_ERR_LAUNCH, "event timing failed");
      continue;
    }
    if (ms) ms[r.stage] += t;
    if (counts) counts[r.stage] += 1;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : recs) {
    g_prof_free.push_back(r.a);
    g_prof_free.push_back(r.b);
  }
  return status;
}

}  // extern "C"
