/*
 * gdn61.h -- C ABI of the MI355X (gfx950) gated-delta-rule library.
 *
 * The library computes, for each (sequence, value head), the gated delta rule
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,
 *
 * with the state S held "V-first" as a V x K matrix (row = value channel,
 * column = key channel, K contiguous).  GDN uses one log-gate g_t per token
 * and v-head; KDA uses one per token, v-head and key channel, replacing
 * exp(g_t) S by S diag(exp(gk_t)).  Sources, by page and section:
 *   - "sglang srt/layers/attention/fla/chunk_fwd.py":
 *     chunk_gated_delta_rule_fwd_intra (arguments k, v, g, beta, cu_seqlens,
 *     chunk_size; A of shape [B, T, H, BT]) and the fused beta*K K^T +
 *     solve_tril kernel;
 *   - "fla ops/common/chunk_h.py": chunk_fwd_h (h0, output_final_state,
 *     state_v_first, cu_seqlens; final state fp32);
 *   - "vLLM kimi_k3 amd ops kda/chunk_intra": the KDA Aqk / Akk_inv outputs
 *     (row-per-token layout [B, T, HV, BT], Aqk scaled by `scale`);
 *   - "flashinfer gdn_kernels/gdn_decode_bf16_state.py": the public
 *     gated_delta_rule entry (A_log, a, dt_bias, softplus_beta,
 *     softplus_threshold, q, k, v, b, state pool [pool, HV, V, K] bf16
 *     updated in place, per-batch slot indices int32, use_qk_l2norm,
 *     scale; T = 1..4).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller, contiguous
 *     and row-major in the stated shape, aligned to 16 bytes (the library
 *     reads and writes 16-byte vectors).  The library allocates nothing,
 *     keeps no state between calls and never synchronises the host.
 *   - `stream` is a hipStream_t (NULL = the null stream); all work is queued
 *     on it asynchronously, in stream order.
 *   - Outputs must not alias inputs (the decode state, updated in place, is
 *     the one exception).
 *   - Every argument check runs on the host before any HIP call; a failed
 *     check returns GDN_ERR_INVALID_ARGUMENT or GDN_ERR_UNSUPPORTED and
 *     queues nothing.  gdn_last_error() then describes the failure.
 *   - A launch failure reported by the HIP runtime returns GDN_ERR_LAUNCH; a
 *     missing or too small workspace GDN_ERR_WORKSPACE (the one code added
 *     to the four of the plan: it tells the caller to query the size).
 *   - io dtype codes: GDN_DTYPE_F32 (0) or GDN_DTYPE_BF16 (1).
 *   - Size limits (GDN_ERR_UNSUPPORTED beyond them): B * T below 2^25
 *     tokens; the kernels index work-groups with 32-bit integers, so
 *     (sequences x v-heads + 8) x 8 and, for the prefill, (chunk slots + 8)
 *     x v-heads x 8 stay below 2^31 (decode: B x HV x 4); tensor offsets
 *     are 64-bit.
 *   - Stored states (prefill snapshots, the state scans' h / dh) are kept in
 *     fp32 or bf16 as the caller chooses (state_dtype; "fla ops/common/
 *     chunk_h.py", chunk_fwd_h / chunk_bwd_dh: states in the input dtype
 *     unless states_in_fp32).  A bf16 state is the fp32 state rounded to
 *     nearest, ties to even.  Initial and final states (h0, ht, dht, dh0)
 *     are always fp32.  A stored-state buffer comes with its capacity in
 *     entries of [HV, V, K]: without cu_seqlens a buffer smaller than the
 *     call needs is rejected (GDN_ERR_INVALID_ARGUMENT); with cu_seqlens
 *     (whose values the host never reads) entries at or past the capacity
 *     are not written.  sum_n ceil(L_n / split_size) <= ceil(T / split_size)
 *     + N bounds the entries a varlen call needs.
 */
#ifndef GDN61_H
#define GDN61_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad size, bad layout */
  GDN_ERR_UNSUPPORTED = 2,      /* valid request outside the compiled set     */
  GDN_ERR_LAUNCH = 3,           /* the HIP runtime rejected a kernel launch   */
  GDN_ERR_WORKSPACE = 4         /* workspace missing or smaller than needed   */
} gdn_status_t;

enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };

/* Static text for a status code. */
const char* gdn_status_string(int status);

/* Detail message of the last failing call made by this host thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* gdn_last_error(void);

/* Library version, e.g. "gdn61 0.1 gfx950". */
const char* gdn_version(void);

/*
 * Workspace needed by gdn_chunk_fwd / kda_chunk_fwd, in bytes, for the
 * given problem (num_seqs = N of cu_seqlens, or B without it).  Returns 0
 * when the arguments are invalid.  The workspace holds the per-chunk
 * (I + A)^-1 and masked, gated Q K^T blocks ([B*T, HV, 64] each; fp16 for
 * bf16 io, fp32 for fp32 io), the per-token gate factors and the varlen
 * chunk tables (KDA: also its gated operands and decay rows).
 */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int Hk, int HV, int K, int V,
                                     int num_seqs, int dtype);
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int Hk, int HV, int K, int V,
                                     int num_seqs, int dtype);

/*
 * GDN chunked prefill forward (scalar gate).
 *
 *   q, k        [B, T, Hk, K]   io dtype
 *   v           [B, T, HV, V]   io dtype
 *   g           [B, T, HV]      fp32 per-token natural-log gate (the chunk-
 *                               local cumulative sum is taken inside), or
 *                               NULL
 *   g_gamma     [HV]            fp32 fixed per-head natural-log decay applied
 *                               at every token, or NULL ("fla ops/common/
 *                               chunk_h.py", USE_G_GAMMA: the chunk-local
 *                               cumulative gate is gamma * (t + 1)); the
 *                               same as g[b, t, h] = g_gamma[h].  At most one
 *                               of g and g_gamma; neither means no decay
 *   beta        [B, T, HV]      fp32
 *   scale       output scale (callers usually pass K^-0.5)
 *   h0          [N, HV, V, K]   fp32 initial state, or NULL for zeros
 *   ht          [N, HV, V, K]   fp32 final state out, or NULL to skip
 *   h_snap      [S, HV, V, K]   state snapshots out (fp32 or bf16, state_dtype),
 *                               or NULL to skip:
 *                               the state before the first token of every
 *                               split of split_size tokens of a sequence
 *                               ("fla ops/common/chunk_h.py",
 *                               chunk_fwd_kernel_h: h is stored at every
 *                               chunk whose index is a multiple of
 *                               split_size / chunk_size, before that chunk's
 *                               update).  Sequence n of length L_n owns
 *                               ceil(L_n / split_size) consecutive entries,
 *                               after those of sequences 0..n-1, so
 *                               S = sum_n ceil(L_n / split_size)
 *                               (B * ceil(T / split_size) without
 *                               cu_seqlens); its first entry is h0 (or
 *                               zeros).  The caller sizes the buffer.
 *   split_size  tokens per snapshot, a positive multiple of 64; read only
 *               when h_snap is not NULL
 *   snap_entries  capacity of h_snap in [HV, V, K] entries (see above)
 *   state_dtype   GDN_DTYPE_F32 or GDN_DTYPE_BF16: dtype of h_snap
 *   cu_seqlens  [N + 1]         int64 device array of packed sequence
 *                               boundaries, or NULL.  With it B must be 1 and
 *                               num_seqs = N; the values must satisfy
 *                               0 = cu[0] <= cu[1] <= ... <= cu[N] = T
 *                               (values outside [0, T] are clamped, and
 *                               non-monotone values only shorten what is
 *                               computed, so no access leaves the buffers;
 *                               results are then unspecified).  Without it
 *                               num_seqs is ignored and N = B.
 *   o           [B, T, HV, V]   io dtype output
 *   workspace   device buffer of at least gdn_chunk_fwd_workspace_bytes()
 *
 * q/k head of v-head j is j / (HV / Hk) (HV must be a multiple of Hk).
 * Supported: K = V in {64, 128}, chunk_size = 64, T >= 0.
 * T = 0 (or all sequences empty) is valid: ht = h0 (or zeros) is written.
 */
int gdn_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* g, const float* g_gamma, const float* beta, float scale,
                  const float* h0, float* ht,
                  void* h_snap, int split_size, long long snap_entries, int state_dtype,
                  const int64_t* cu_seqlens, int num_seqs,
                  int B, int T, int Hk, int HV, int K, int V,
                  int chunk_size, int dtype,
                  void* o, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * gdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as gdn_chunk_fwd; the workspace is a scratch array inside the
 * library (one per GPU, gdn_chunk_fwd_noalloc_max_bytes() = 96 MiB, held
 * until the process ends; looked up once per device, on the first call).
 * A call needing more (gdn_chunk_fwd_workspace_bytes() > that) returns
 * GDN_ERR_UNSUPPORTED and queues nothing.  `stream` must belong to the
 * current device.  Every call on a GPU shares that GPU's scratch, so calls
 * that overlap on one GPU (different streams, or host threads) race; calls
 * in one stream are ordered.  Calls no hipMalloc, hipFree or allocating
 * library routine.
 */
size_t gdn_chunk_fwd_noalloc_max_bytes(void);
int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                          const float* g, const float* g_gamma, const float* beta, float scale,
                          const float* h0, float* ht,
                          void* h_snap, int split_size, long long snap_entries, int state_dtype,
                          const int64_t* cu_seqlens, int num_seqs,
                          int B, int T, int Hk, int HV, int K, int V,
                          int chunk_size, int dtype, void* o, void* stream);

/*
 * KDA chunked prefill forward (one log-gate per key channel).
 *
 * As gdn_chunk_fwd, with
 *   gk          [B, T, HV, K]   fp32 per-token, per-channel natural-log gate
 *                               (required)
 *   Aqk         [B, T, HV, 64]  io dtype out, or NULL: row t holds
 *                               scale * sum_c q_t,c k_s,c exp(G_t,c - G_s,c)
 *                               for the tokens s <= t of t's chunk, at column
 *                               s - chunk_start; 0 elsewhere
 *   Akk_inv     [B, T, HV, 64]  io dtype out, or NULL: row t holds row
 *                               (t - chunk_start) of (I + A)^-1, where
 *                               A_ts = beta_t sum_c k_t,c k_s,c
 *                               exp(G_t,c - G_s,c) for s < t in the chunk;
 *                               0 above the diagonal and past the chunk end
 * (G = cumulative log-gate from the chunk start).
 * B * T * K * 2 must stay below 2^32 (16.7 M tokens at K = 128): the
 * workspace's gated operands of one head are addressed with 32-bit offsets;
 * larger calls return GDN_ERR_UNSUPPORTED.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* gk, const float* beta, float scale,
                  const float* h0, float* ht,
                  void* h_snap, int split_size, long long snap_entries, int state_dtype,
                  const int64_t* cu_seqlens, int num_seqs,
                  int B, int T, int Hk, int HV, int K, int V,
                  int chunk_size, int dtype,
                  void* o, void* Aqk, void* Akk_inv,
                  void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * The scalar-gate intra-chunk step on its own ("sglang srt/layers/attention/
 * fla/chunk_fwd.py", chunk_gated_delta_rule_fwd_intra: the fused beta K K^T
 * + solve, then recompute_w_u).  Per chunk of 64 tokens (restarting at every
 * sequence start) and v-head, with G the chunk-local cumulative log-gate:
 *   A = (I + L)^-1,  L_ts = beta_t (k_t . k_s) e^{G_t - G_s} for s < t
 *   w = A diag(beta e^G) K,   u = A diag(beta) V
 * (gdn_chunk_fwd never forms w and u: its scan computes u - w S^T in one
 * step.)  With h = S^T the state after a chunk is
 * e^{G_last} h + (K o e^{G_last - G})^T (u - w h).
 *
 *   k            [B, T, Hk, K]  io dtype (key head of v-head j: j / (HV / Hk))
 *   v            [B, T, HV, V]  io dtype, read when u is requested
 *   g            [B, T, HV]     fp32: per-token log-gates (g_cumulative = 0)
 *                or their chunk-local cumulative sums, as the page's
 *                wrapper takes them (g_cumulative = 1); NULL = no gate
 *   beta         [B, T, HV]     fp32
 *   A            [B, T, HV, 64] io dtype out: row t holds row (t - chunk
 *                start) of the chunk's A (entries past the chunk end 0)
 *   w            [B, T, HV, K]  io dtype out, or NULL (not formed)
 *   u            [B, T, HV, V]  io dtype out, or NULL (not formed)
 *   cu_seqlens, num_seqs, B, T, Hk, HV, chunk_size, dtype  as in gdn_chunk_fwd
 *   workspace    device buffer of at least gdn_chunk_intra_workspace_bytes(N)
 *                bytes, 256-byte aligned, with cu_seqlens (the chunk
 *                tables); unused (NULL allowed) without
 * Supported: K, V in {64, 128}, chunk_size = 64, bf16 or fp32 io.  A is
 * formed in fp32 (forward substitution and block merge) and stored once in
 * the io dtype.  w and u are products of that inverse with the scaled rows,
 * accumulated in fp32: with fp32 io from fp32 operands, with bf16 io from
 * the inverse and the scaled rows rounded to fp16 (saturating at +-65504;
 * the page rounds both to bf16).  Errors and pointer rules as in
 * gdn_chunk_fwd.  Asynchronous on `stream`.
 */
size_t gdn_chunk_intra_workspace_bytes(int num_seqs);
int gdn_chunk_intra(const void* k, const void* v, const float* g, int g_cumulative,
                    const float* beta, const int64_t* cu_seqlens, int num_seqs,
                    int B, int T, int Hk, int HV, int K, int V,
                    int chunk_size, int dtype, void* A, void* w, void* u,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * GDN decode step over a bf16 state pool, T = 1..4 tokens per call.
 *
 *   q, k           [B, T, H, K]    bf16 (normalised in-kernel when
 *                                  use_qk_l2norm != 0:
 *                                  q * scale / sqrt(sum q^2 + eps),
 *                                  k / sqrt(sum k^2 + eps))
 *   v              [B, T, HV, V]   bf16
 *   a, b           [B, T, HV]      bf16 gate inputs
 *   A_log, dt_bias [HV]            fp32
 *   state          [pool, HV, V, K] bf16, read and written IN PLACE: slot
 *                                  indices[b] (or b when indices is NULL)
 *                                  holds the state of batch row b
 *   state_indices  [B] int32 device array, or NULL for the identity
 *                  (then pool >= B is required).  A slot outside [0, pool)
 *                  leaves the pool untouched and writes o = 0 for that row.
 *                  Two rows naming the same slot race (undefined result).
 *   o              [B, T, HV, V]   bf16 output
 *
 * Per token: x = a + dt_bias; softplus(x) = log(1 + exp(sb*x))/sb if
 * sb*x <= threshold else x (sb = softplus_beta); alpha = exp(-exp(A_log)
 * * softplus(x)); beta = sigmoid(b); S <- alpha S; delta = beta (v - S k);
 * S <- S + delta k^T; o = S q.  The state is carried in fp32 across the T
 * tokens and rounded to bf16 (nearest-even) once, after the last token.
 * q/k head of v-head j is j / (HV / H).
 * Supported: K = V = 128, T in 1..4.
 */
int gdn_decode(const void* q, const void* k, const void* v,
               const void* a, const void* b,
               const float* A_log, const float* dt_bias,
               void* state, const int32_t* state_indices,
               void* o,
               int B, int T, int H, int HV, int K, int V, int pool,
               float scale, float softplus_beta, float softplus_threshold,
               int use_qk_l2norm, float eps,
               void* stream);

/*
 * Backward state-gradient scan ("fla ops/common/chunk_h.py",
 * chunk_bwd_kernel_dh), bf16 io.  Per sequence and v-head, over the chunks of
 * 64 tokens in reverse order, with dh [V, K] the gradient with respect to the
 * state at the end of the current chunk:
 *   start:       dh = dht (or zeros)
 *   each chunk:  if its index is a multiple of split_size / 64, store dh;
 *                dh <- decay * dh + scale * sum_t e^{G_t} do_t q_t^T
 *                (per-key-channel gate gk: the key column c of every term
 *                and of the decay carries e^{G_t,c} / e^{G_last,c} instead;
 *                per-value-channel gate gv: the value row i carries in
 *                addition e^{Gv_t,i} / e^{Gv_last,i})
 *   end:         dh0 = dh
 * G = chunk-local cumulative log-gate, decay = e^{G_last}.  This is the
 * state gradient of the decay-only recurrence h_t = decay_t h_{t-1} +
 * (terms free of h), o_t = scale q_t . h_t; the delta rule's erase term is
 * not part of it.
 *
 *   q            [B, T, Hk, K]  bf16 (query head of v-head j: j / (HV / Hk))
 *   dout         [B, T, HV, V]  bf16 gradient of the output
 *   num_gate_heads  Hg, the heads of the gate arrays (0 = HV); HV must be a
 *                multiple of it and v-head j takes gate head j / (HV / Hg).
 *                The page's grouped form (HQ query / output heads sharing
 *                the gates of H = HQ / NG heads, one dh per query head) is
 *                Hk = HV = HQ with Hg = H
 *   g [B,T,Hg] | g_gamma [Hg] | gk [B,T,Hg,K]   fp32 log-gates, at most
 *                one (none = no decay); as in gdn_chunk_fwd / kda_chunk_fwd
 *   gv           [B, T, Hg, V]  fp32 per-value-channel log-gates, or NULL;
 *                may come with g or g_gamma, not with gk (GDN_ERR_UNSUPPORTED)
 *   dht          [N, HV, V, K]  fp32 gradient of the final state, or NULL
 *   dh           [S, HV, V, K]  out (fp32 or bf16, state_dtype), or NULL:
 *                sequence n of length L_n owns ceil(L_n / split_size)
 *                entries after those of sequences 0..n-1 (entry s = the
 *                gradient at the end of chunk s * split_size / 64)
 *   split_size   a positive multiple of 64, read when dh is not NULL
 *   dh_entries   capacity of dh in [HV, V, K] entries (see the conventions)
 *   state_dtype  GDN_DTYPE_F32 or GDN_DTYPE_BF16: dtype of dh
 *   state_v_first  layout of dht, dh and dh0 (the page's state_v_first):
 *                1 = [*, HV, V, K] (K contiguous, as documented here and as
 *                the prefill and decode keep their states; the fast layout),
 *                0 = [*, HV, K, V] (V contiguous, the page's default)
 *   dh0          [N, HV, V, K]  fp32 out (gradient of the initial state), or NULL
 *   cu_seqlens, num_seqs, B, T, Hk, HV, K, V, chunk_size  as in gdn_chunk_fwd
 * Supported: dtype = GDN_DTYPE_BF16, K = V in {64, 128}, chunk_size = 64.
 * Allocates nothing; asynchronous on `stream`.
 */
int gdn_chunk_bwd_dh(const void* q, const void* dout,
                     const float* g, const float* g_gamma, const float* gk,
                     const float* gv, int num_gate_heads, float scale,
                     const float* dht, void* dh, int split_size,
                     long long dh_entries, int state_dtype,
                     int state_v_first, float* dh0,
                     const int64_t* cu_seqlens, int num_seqs,
                     int B, int T, int Hk, int HV, int K, int V,
                     int chunk_size, int dtype, void* stream);

/*
 * Forward decay-only chunk-state scan ("fla ops/common/chunk_h.py",
 * chunk_fwd_kernel_h, either state layout), bf16 io.  Per sequence
 * and v-head, over the chunks of 64 tokens in order, with h [V, K] the state
 * at the start of the current chunk:
 *   start:       h = h0 (or zeros)
 *   each chunk:  if its index is a multiple of split_size / 64, store h;
 *                h <- e^{G_last} h + sum_t e^{G_last - G_t} v_t k_t^T
 *                (gk: key column c carries e^{G_last,c} and
 *                e^{G_last,c - G_t,c}; gv: value row i carries in addition
 *                e^{Gv_last,i} and e^{Gv_last,i - Gv_t,i})
 *   end:         ht = h
 * G = chunk-local cumulative log-gate.  Token by token this is
 * S_t = diag(e^{gv_t}) S_{t-1} diag(e^{gk_t}) e^{g_t} + v_t k_t^T: the
 * linear-attention state without the delta rule's erase term.
 *
 *   k            [B, T, Hk, K]  bf16 (key head of v-head j: j / (HV / Hk))
 *   v            [B, T, HV, V]  bf16
 *   num_gate_heads, g, g_gamma, gk, gv   as in gdn_chunk_bwd_dh
 *   h0           [N, HV, V, K]  fp32 initial state, or NULL (zeros)
 *   h            [S, HV, V, K]  out (fp32 or bf16, state_dtype), or NULL:
 *                sequence n of length L_n owns ceil(L_n / split_size)
 *                entries after those of sequences 0..n-1 (entry s = the
 *                state at the start of chunk s * split_size / 64)
 *   split_size   a positive multiple of 64, read when h is not NULL
 *   h_entries    capacity of h in [HV, V, K] entries (see the conventions)
 *   state_dtype  GDN_DTYPE_F32 or GDN_DTYPE_BF16: dtype of h
 *   state_v_first  layout of h0, h and ht, as in gdn_chunk_bwd_dh (1 =
 *                [*, HV, V, K] as documented here, 0 = [*, HV, K, V])
 *   ht           [N, HV, V, K]  fp32 out (final state), or NULL
 *   cu_seqlens, num_seqs, B, T, Hk, HV, K, V, chunk_size  as in gdn_chunk_fwd
 * Supported: dtype = GDN_DTYPE_BF16, K = V in {64, 128}, chunk_size = 64.
 * Errors and pointer rules as in gdn_chunk_bwd_dh.  Allocates nothing;
 * asynchronous on `stream`.
 */
int gdn_chunk_fwd_h(const void* k, const void* v,
                    const float* g, const float* g_gamma, const float* gk,
                    const float* gv, int num_gate_heads, const float* h0,
                    void* h, int split_size, long long h_entries,
                    int state_dtype, int state_v_first, float* ht,
                    const int64_t* cu_seqlens, int num_seqs,
                    int B, int T, int Hk, int HV, int K, int V,
                    int chunk_size, int dtype, void* stream);

/*
 * Prefill -> decode handoff: write final prefill states into a bf16 decode
 * state pool (the prefill's ht fp32 layout and the decode pool's layout are
 * both [*, HV, V, K], K contiguous: "fla ops/common/chunk_h.py" ht with the
 * state-V-first layout; "flashinfer gdn_kernels/gdn_decode_bf16_state.py"
 * initial_state_source / initial_state_indices).
 *
 *   ht          [N, HV, V, K]    fp32, caller-owned device memory (read)
 *   indices     [N] int32 device array: pool slot of sequence n, or NULL
 *               for slot n (then pool >= N is required).  A slot outside
 *               [0, pool) is skipped.  Two sequences naming the same slot
 *               race (undefined result).
 *   pool_state  [pool, HV, V, K] bf16, written IN PLACE at the named slots
 *               only; each value is rounded to nearest bf16, ties to even
 *
 * Both arrays must be 16-byte aligned and V * K a multiple of 8.  Errors:
 * GDN_ERR_INVALID_ARGUMENT (sizes, NULL or misaligned pointers),
 * GDN_ERR_UNSUPPORTED (V * K not a multiple of 8), GDN_ERR_LAUNCH.  Runs
 * asynchronously on `stream`; allocates nothing.
 */
int gdn_state_to_pool(const float* ht, const int32_t* indices, void* pool_state,
                      int N, int HV, int K, int V, int pool, void* stream);

/*
 * Per-stage timing for measurement tools.  While enabled, every call of the
 * entry points above records a pair of HIP events on the caller's stream
 * around each kernel it launches (stage ids below); this adds two event
 * records per kernel and nothing else.  gdn_profile_read() waits for the
 * recorded events, adds their elapsed times per stage into ms[stage] and
 * counts[stage] (arrays of at least GDN_STAGE_COUNT entries, caller-owned
 * host memory), then forgets them.  Returns GDN_OK, or GDN_ERR_LAUNCH if the
 * HIP runtime fails.  Not meant to be toggled while calls are in flight on
 * other host threads.
 */
enum {
  GDN_STAGE_VARLEN_TABLES = 0, /* varlen chunk tables                         */
  GDN_STAGE_INTRA = 1,         /* per-chunk (I + A)^-1 and Aqk                 */
  GDN_STAGE_SCAN = 2,          /* chunk-state scan fused with the output       */
  GDN_STAGE_DECODE = 3,        /* decode step                                  */
  GDN_STAGE_HANDOFF = 4,       /* prefill state -> decode pool (bf16)          */
  GDN_STAGE_BWD_DH = 5,        /* backward state-gradient scan                 */
  GDN_STAGE_FWD_H = 6,         /* forward decay-only state scan                */
  GDN_STAGE_COUNT = 7
};
int gdn_profile_enable(int on);
int gdn_profile_read(double* ms, int* counts);

#ifdef __cplusplus
}
#endif

#endif /* GDN61_H */
