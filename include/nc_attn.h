/*
 * nc_attn.h -- C ABI of the MI355X (gfx950) causal self-attention block
 * forward of the nanochat GPT: RoPE, parameter-free QK RMSNorm after RoPE,
 * GQA attention with a per-layer sliding window, and a one-token decode step
 * over a contiguous per-layer KV cache.
 *
 * Sources (page title, section):
 *   [S5.4]  "从文本到聊天模型" (onehacker.top), §5.4 Attention: Q (B,T,H,D),
 *           K and V (B,T,Hkv,D); score = Q K^T, softmax, weighted sum of V.
 *   [S5.5]  same page, §5.5 Causal Attention: causal mask.
 *   [S5.6]  same page, §5.6 RoPE: rotate q and k by position.
 *   [S10]   same page, §10.2-10.4: per-layer KV cache of shape
 *           (batch, seq_len, heads, head_dim); decode computes the new token's
 *           q, k, v, appends k and v to the cache, then attends to all of it.
 *   [TBL]   "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io), §1 model
 *           architecture table and notes: RoPE, RMSNorm without parameters,
 *           QK-norm after RoPE, GQA, SSSL sliding window (short = 1/4 context).
 *
 * Value-embedding gate ([TBL] notes, value residual: v = v + gate * ve). The
 * three cache entry points (nc_attn_prefill, nc_attn_decode,
 * nc_attn_decode_shared) take an optional pair ve (shaped like the values)
 * and ve_gate (one value per token and K/V head, the values' shape without
 * the head dim), both in the call's element type: the values written to the
 * cache and attended to are v' = v + ve_gate * ve, formed in fp32 and rounded
 * once to the element type. Both NULL: v unchanged. The ungated forward
 * nc_attn_fwd equals nc_attn_prefill at pos_offset 0 with Tmax = T bit for
 * bit, so a gated forward is that call with the pair.
 *
 * Conventions fixed by this library where the pages are silent:
 *   RoPE rotates adjacent pairs (x[2i], x[2i+1]) by +p*theta_i with
 *   theta_i = rope_base^(-2i/D) and 0-based positions p = pos_offset + t;
 *   QK-norm is y = x / sqrt(mean(x^2) + 1e-6); scores are scaled by 1/sqrt(D);
 *   key j is visible to query i iff 0 <= i - j < window (window >= T is full
 *   causal attention); query head h reads K/V head h / (H / Hkv).
 *
 * Memory and ownership, for every entry point:
 *   - every tensor argument is a caller-owned DEVICE pointer to a contiguous,
 *     row-major array, 16-byte aligned;
 *   - element type is bfloat16 (NC_BF16) or float32 (NC_F32) for all float
 *     tensors of one call; arithmetic is float32 (bf16 MFMA operands with
 *     float32 accumulation on the bf16 path);
 *   - ws is a caller-owned device workspace of at least the size reported by
 *     the matching *_workspace_bytes query (it may be NULL when that is 0);
 *     its contents on entry do not matter and are clobbered;
 *   - stream is a hipStream_t (NULL = the default stream); all work is
 *     enqueued asynchronously on it and nothing is allocated, freed or
 *     synchronised; the library keeps no state between calls and is
 *     thread-safe;
 *   - inputs are not modified, except the two caches of nc_attn_decode and
 *     nc_attn_decode_shared (exactly one row per sequence and K/V head) and
 *     of nc_attn_prefill (exactly the chunk's T rows per sequence and K/V
 *     head).
 *
 * Errors: arguments are validated on the host before any HIP call. A non-OK
 * status means nothing was enqueued. NC_ERR_INVALID: bad pointer, size,
 * alignment, window, offset, base, dtype or workspace. NC_ERR_UNSUPPORTED:
 * head dim other than 32, 64 or 128, or more query heads per K/V head than
 * supported. NC_ERR_HIP: a launch failed (nc_last_error() has the HIP
 * message). Faults inside kernels surface from the caller's next sync.
 * nc_last_error() returns a thread-local description of the last failure of
 * the calling thread. No function aborts, throws or prints.
 */
#ifndef NC_ATTN_H
#define NC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two enumerations span the whole int range (the _MIN_ and _MAX_
 * members), so that any int a caller passes is a value of the type: unknown
 * codes are reported as such (nc_status_string) or rejected (NC_ERR_INVALID),
 * never undefined. Both are int-sized. */
typedef enum {
  NC_OK = 0,
  NC_ERR_INVALID = 1,
  NC_ERR_UNSUPPORTED = 2,
  NC_ERR_HIP = 3,
  NC_STATUS_MIN_ = -2147483647 - 1,
  NC_STATUS_MAX_ = 2147483647
} nc_status;

typedef enum {
  NC_BF16 = 0,
  NC_F32 = 1,
  NC_DTYPE_MIN_ = -2147483647 - 1,
  NC_DTYPE_MAX_ = 2147483647
} nc_dtype;

/* RMSNorm epsilon inside QK-norm. */
#define NC_QKNORM_EPS 1e-6

/* ABI version of this header (bumped on any signature change). */
#define NC_ABI_VERSION 10
int nc_abi_version(void);

/* Static description of a status code. Never NULL. */
const char* nc_status_string(nc_status status);

/* Detail of the calling thread's last failure ("" if none). Never NULL. */
const char* nc_last_error(void);

/*
 * nc_rope_qknorm -- RoPE then parameter-free RMSNorm on q and k
 * ([S5.6] rotation by position; [TBL] QK-norm after RoPE).
 *
 *   q      (B, T, H,   D)  input rows; position of row t is pos_offset + t
 *   k      (B, T, Hkv, D)
 *   q_out  (B, T, H,   D)  norm(rope(q)); may alias q exactly (in place)
 *   k_out  (B, T, Hkv, D)  norm(rope(k)); may alias k exactly
 * Any other overlap between inputs and outputs is undefined.
 * Requires B, T, H, Hkv >= 1, D in {32, 64, 128}, pos_offset >= 0,
 * pos_offset + T <= 2^30, rope_base finite and > 0.
 */
size_t nc_rope_qknorm_workspace_bytes(int T, int D, int pos_offset);
nc_status nc_rope_qknorm(const void* q, const void* k, void* q_out, void* k_out,
                         int B, int T, int H, int Hkv, int D,
                         double rope_base, int pos_offset, nc_dtype dtype,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * nc_qkv_rope_qknorm -- the bias-free q, k, v projections of the block input
 * followed by RoPE and QK-norm on q and k, in one kernel ("从文本到聊天模型"
 * §5.4: q = c_q(x), k = c_k(x), v = c_v(x), viewed as (B, T, H, D) and
 * (B, T, Hkv, D); "Nanochat与nanoGPT对比：关键升级" §1 table: no bias, QK-norm
 * after RoPE).
 *
 *   x      (B, T, C)     block input (after the block's pre-norm)
 *   w_q    (H*D, C)      weights in the linear-layer layout (out, in): output
 *   w_k    (Hkv*D, C)    column h*D + d is element d of head h; the element
 *   w_v    (Hkv*D, C)    type of the call (fp32 master weights are cast by
 *                        the caller)
 *   q_out  (B, T, H, D)   norm(rope(x w_q^T)) at positions pos_offset + t
 *   k_out  (B, T, Hkv, D) norm(rope(x w_k^T))
 *   v_out  (B, T, Hkv, D) x w_v^T
 * q_out and k_out equal nc_rope_qknorm applied to the plain projections, but
 * formed from the fp32 accumulators with one rounding to the element type.
 * Requires C >= 64 and C % 64 == 0 (else NC_ERR_UNSUPPORTED), the sizes of
 * nc_rope_qknorm, outputs disjoint from each other and from the inputs.
 * Workspace (nc_qkv_rope_qknorm_workspace_bytes): the (cos, sin) table of the
 * T positions.
 */
size_t nc_qkv_rope_qknorm_workspace_bytes(int T, int D, nc_dtype dtype);
nc_status nc_qkv_rope_qknorm(const void* x, const void* w_q, const void* w_k, const void* w_v,
                             void* q_out, void* k_out, void* v_out,
                             int B, int T, int C, int H, int Hkv, int D,
                             double rope_base, int pos_offset, nc_dtype dtype,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_fwd -- prefill forward of one attention layer from RAW q, k, v
 * ([S5.4] scores, softmax, weighted sum; [S5.5] causal mask; [S5.6] RoPE;
 * [TBL] QK-norm after RoPE, GQA, sliding window).
 *
 *   q  (B, T, H,   D)  raw query projections
 *   k  (B, T, Hkv, D)  raw key projections
 *   v  (B, T, Hkv, D)  values
 *   o  (B, T, H,   D)  output, o[b,t,h] = sum_j softmax_j(q'.k'_j / sqrt(D)) v_j
 *                      over keys j with 0 <= t - j < window, q' and k' the
 *                      rotated (positions pos_offset + t) and normalised rows
 * Requires H % Hkv == 0, window >= 1 (window >= T: full causal), the sizes
 * of nc_rope_qknorm, T * Hkv * D * sizeof(element) < 2^32 (one sequence's K
 * or V is addressed with 32-bit byte offsets), and o not overlapping any input.
 * Workspace (nc_attn_fwd_workspace_bytes, which depends on B, T, H, Hkv, D
 * and dtype): the (cos, sin) table of the T positions, k' = norm(rope(k)),
 * and, for bf16 launches too small to fill the device (few sequences and
 * heads), room for per-slice partial output rows: the key tiles of each query
 * tile are then cut into slices run by separate workgroups, and a second
 * kernel adds the slices' unnormalised sums and divides by their row sums
 * (QK-norm bounds the scores, so the slices share one exponent scale). Calls
 * that overlap in time must not share a workspace.
 * nc_attn_fwd(...) is exactly nc_attn_prep followed by nc_attn_core on the
 * same workspace.
 */
size_t nc_attn_fwd_workspace_bytes(int B, int T, int H, int Hkv, int D, int pos_offset,
                                   nc_dtype dtype);
nc_status nc_attn_fwd(const void* q, const void* k, const void* v, void* o,
                      int B, int T, int H, int Hkv, int D, int window,
                      double rope_base, int pos_offset, nc_dtype dtype,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_fwd_normed -- the attention of nc_attn_fwd from rows that are
 * already rotated and normalised ([S5.4] scores, softmax, weighted sum; [S5.5]
 * causal mask; [TBL] GQA and window), e.g. the outputs of nc_qkv_rope_qknorm
 * or nc_rope_qknorm: no input stage runs, q' and k' are read as given.
 *
 *   q  (B, T, H,   D)  q' = norm(rope(q))
 *   k  (B, T, Hkv, D)  k' = norm(rope(k))
 *   v  (B, T, Hkv, D)  values
 *   o  (B, T, H,   D)  o[b,t,h] = sum_j softmax_j(q'_t . k'_j / sqrt(D)) v_j over
 *                      0 <= t - j < window
 * The bound on stored rows of nc_attn_prefill applies to q and k (RMS at
 * most 4; the library's own rows have RMS 1). Sizes and errors as for
 * nc_attn_fwd. Workspace (nc_attn_fwd_normed_workspace_bytes, possibly 0):
 * the partial rows of a launch cut into key-tile slices.
 */
size_t nc_attn_fwd_normed_workspace_bytes(int B, int T, int H, int Hkv, int D, nc_dtype dtype);
nc_status nc_attn_fwd_normed(const void* q, const void* k, const void* v, void* o,
                             int B, int T, int H, int Hkv, int D, int window, nc_dtype dtype,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_fwd_lse -- nc_attn_fwd that also writes the row log-sum-exp the
 * backward pass starts from (a training step runs the forward, then
 * backpropagates: "从文本到聊天模型" (onehacker.top) §6.5).
 *
 *   lse  (B, T, H) float32  lse[b,t,h] = ln sum_j exp(q'_t . k'_j / sqrt(D))
 *                           over the visible keys j (natural log); o and the
 *                           other arguments as for nc_attn_fwd
 * lse must be 4-byte aligned and must not overlap any other argument. o may
 * differ from nc_attn_fwd's in the last bit (at D = 128 the call runs the
 * two-wave attention kernel, whose registers leave room for the extra output).
 * Workspace: nc_attn_fwd_workspace_bytes.
 */
nc_status nc_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int T, int H, int Hkv, int D, int window,
                          double rope_base, int pos_offset, nc_dtype dtype,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_bwd -- gradients of the prefill forward with respect to its RAW
 * inputs q, k, v ("从文本到聊天模型" §6.5, the training step's backward
 * pass; "Nanochat与nanoGPT对比：关键升级" §1 table: the training attention
 * runs forward and backward). The chain rule through nc_attn_fwd's
 * definition: with P = exp(q'k'^T/sqrt(D) - lse) on the band and
 * Delta_t = dO_t . o_t,
 *   dv[g] = sum over g's query heads of P^T dO,  dS = P (dO v^T - Delta),
 *   dq' = dS k' / sqrt(D),  dk'[g] = sum over g's query heads of dS^T q' / sqrt(D),
 * then through the RMSNorm (dx = r (dy - y mean(dy y)), y = x r) and the
 * RoPE rotation (rotated back by -p theta_i).
 *
 *   q, k, v   the forward's raw inputs, layouts as for nc_attn_fwd
 *   o         (B, T, H, D)   the forward's output for them
 *   dout      (B, T, H, D)   dL/do
 *   lse       (B, T, H) f32  the forward's row log-sum-exp (nc_attn_fwd_lse)
 *   dq        (B, T, H, D)   dL/dq      written, element type of the inputs
 *   dk, dv    (B, T, Hkv, D) dL/dk, dL/dv (sums over each K/V head's group)
 * window, rope_base and pos_offset must be the forward's. Requires the sizes
 * of nc_attn_fwd and T * H * D * sizeof(element) < 2^32; dq, dk, dv must not
 * overlap each other or any input; lse 4-byte aligned.
 * Workspace (nc_attn_bwd_workspace_bytes): the (cos, sin) table, k', and for
 * bf16 the prepared MFMA operands (q' scaled, transposed copies of q', dO and
 * k' in tiles of 32 positions) and per-row lse and dO.o; calls that overlap in
 * time must not share a workspace.
 */
size_t nc_attn_bwd_workspace_bytes(int B, int T, int H, int Hkv, int D, nc_dtype dtype);
nc_status nc_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      int B, int T, int H, int Hkv, int D, int window,
                      double rope_base, int pos_offset, nc_dtype dtype,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_fwd_noalloc -- nc_attn_fwd for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, result and kernels
 * as nc_attn_fwd minus the workspace: the workspace lives in a static 64 MiB
 * device array of the library (one per GPU, held from module load until the
 * process ends), on the CURRENT device (hipGetDevice), where q, k, v, o and
 * stream must be. Nothing is allocated or freed, and nothing needs clearing
 * (every byte the kernels read is written earlier in the same call).
 * Errors: NC_ERR_INVALID when nc_attn_fwd_workspace_bytes for the sizes
 * exceeds 64 MiB (k' alone takes B*T*Hkv*D*sizeof(element): B = 8, T = 2048,
 * Hkv = 6, D = 128 in bf16 needs 25.7 MB in all, B = 32 does not fit),
 * otherwise as nc_attn_fwd. Calls that overlap in time on one GPU (several
 * streams or threads) share the array and race: serialise them.
 */
nc_status nc_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                              int B, int T, int H, int Hkv, int D, int window,
                              double rope_base, int pos_offset, nc_dtype dtype, void* stream);

/*
 * nc_attn_prep / nc_attn_core -- the two stages of nc_attn_fwd, for callers
 * that schedule them separately (for instance to overlap one layer's prep with
 * another layer's attention on a second stream).
 *   nc_attn_prep writes into ws the (cos, sin) pairs of angles
 *     (pos_offset + t) * rope_base^(-2i/D), t < T, i < D/2, each formed and
 *     reduced modulo 2*pi in fp64 and stored as two fp16 (dtype bf16: the
 *     rounding, at most 2^-11 relative, is a quarter of the bf16 rounding of
 *     the rotated q that follows) or two fp32 values (dtype fp32), and
 *     k' = norm(rope(k)) in k's layout and element type. Arguments as for
 *     nc_attn_fwd.
 *   nc_attn_core computes o from raw q, the k' and table in ws (read, not
 *     modified), and v; it may write the partial rows after them. B, T, Hkv,
 *     D and dtype must be those of the nc_attn_prep call that filled ws, which
 *     must complete (same stream or an event) first; ws must hold
 *     nc_attn_fwd_workspace_bytes for the call's H.
 * nc_attn_prep needs only the table and k' part of that size.
 */
nc_status nc_attn_prep(const void* k, int B, int T, int Hkv, int D, double rope_base,
                       int pos_offset, nc_dtype dtype, void* ws, size_t ws_bytes,
                       void* stream);
nc_status nc_attn_core(const void* q, const void* v, void* o, int B, int T, int H, int Hkv,
                       int D, int window, nc_dtype dtype, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * nc_attn_prefill -- prefill of a chunk of T tokens into a contiguous KV cache,
 * the step before nc_attn_decode; called with increasing pos_offset it is a
 * chunked prefill ([S10] the new tokens' K and V are appended to the per-layer
 * cache, then their queries attend to the cache; [S5.5] causal mask; [TBL]
 * QK-norm after RoPE, GQA, sliding window).
 *
 *   q        (B, T, H,   D)     raw queries of the chunk's tokens, which sit at
 *                               positions pos_offset .. pos_offset + T - 1
 *   k, v     (B, T, Hkv, D)     their raw keys and values
 *   k_cache  (B, Tmax, Hkv, D)  rows 0 .. pos_offset-1 hold rotated, normalised
 *                               keys (from earlier calls or decode steps) and
 *                               are used as stored (see the bound below); rows pos_offset .. +T-1 are
 *                               overwritten with norm(rope(k)); later rows are
 *                               neither read nor written
 *   v_cache  (B, Tmax, Hkv, D)  likewise; rows pos_offset .. +T-1 receive v
 *   o        (B, T, H, D)       o[b,t,h]: softmax over cache rows j with
 *                               0 <= pos_offset + t - j < window of
 *                               q'.k_cache[b,j] / sqrt(D), applied to v_cache
 * Bound on stored rows: the attention kernels exponentiate the scores with a
 * fixed scale instead of a running maximum (QK-norm bounds the scores of the
 * rows this library writes, whose RMS is 1). That is exact for stored key rows
 * of RMS at most 4: the scores then lie within +-4*sqrt(D), their exponentials
 * and the row sums stay inside the fp32 and bf16 ranges. Rows of larger RMS
 * are outside the contract (their exponentials may overflow); nc_attn_decode,
 * which keeps a running maximum, has no such bound.
 * With pos_offset = 0 and Tmax = T, o equals nc_attn_fwd's. One pos_offset
 * serves the whole batch. The caches are written by a first kernel and read by
 * a second one on the same stream.
 * Requires pos_offset + T <= Tmax, the sizes of nc_attn_fwd with Tmax in place
 * of T for the caches (Tmax * Hkv * D * sizeof(element) < 2^32), and q, k, v,
 * o pairwise disjoint and disjoint from the caches.
 * Workspace (nc_attn_prefill_workspace_bytes): the (cos, sin) table of the
 * chunk's positions, as in nc_attn_prep, and room for partial output rows of
 * a launch cut into key-tile slices, as in nc_attn_fwd (a chunk at a large
 * offset has long key ranges for few query tiles). Calls that overlap in time
 * must not share a workspace.
 */
size_t nc_attn_prefill_workspace_bytes(int B, int T, int Tmax, int H, int Hkv, int D,
                                       nc_dtype dtype);
/* ve (B, T, Hkv, D), ve_gate (B, T, Hkv): optional value-embedding pair (above). */
nc_status nc_attn_prefill(const void* q, const void* k, const void* v, const void* ve,
                          const void* ve_gate, void* k_cache, void* v_cache, void* o,
                          int B, int T, int Tmax, int H, int Hkv, int D, int window,
                          double rope_base, int pos_offset, nc_dtype dtype,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_decode -- one decode step per sequence over a contiguous KV cache
 * ([S10] append the new token's K/V, then attend; cache per layer of shape
 * (batch, seq_len, heads, head_dim)).
 *
 *   q        (B, H,   D)        raw query of the new token
 *   k_new    (B, Hkv, D)        raw key of the new token
 *   v_new    (B, Hkv, D)        value of the new token
 *   k_cache  (B, Tmax, Hkv, D)  rows 0 .. L-2 hold rotated, normalised keys;
 *                               row L-1 is overwritten with norm(rope(k_new))
 *   v_cache  (B, Tmax, Hkv, D)  row L-1 is overwritten with v_new
 *   seqlens  (B,) int32 DEVICE array, L = seqlens[b] in [1, Tmax] counts the
 *                               new token, whose position is L-1
 *   o        (B, H, D)          softmax over keys max(0, L-window) .. L-1
 * seqlens values outside [1, Tmax] are a precondition violation: the kernels
 * clamp them to that range instead of reading out of bounds.
 * Workspace: the key range of a sequence is split into chunks processed in
 * parallel; ws holds each chunk's softmax state until a second kernel merges
 * them. Calls that overlap in time must not share a workspace.
 * Requires H % Hkv == 0, H / Hkv <= 64, window >= 1, Tmax >= 1, D in
 * {32, 64, 128}; q, k_new, v_new and o must not overlap the caches.
 */
size_t nc_attn_decode_workspace_bytes(int B, int Tmax, int H, int Hkv, int D, int window);
/* ve_new (B, Hkv, D), ve_gate (B, Hkv): optional value-embedding pair of the
 * new token (above); the appended value is v_new + ve_gate * ve_new. */
nc_status nc_attn_decode(const void* q, const void* k_new, const void* v_new,
                         const void* ve_new, const void* ve_gate,
                         void* k_cache, void* v_cache, const int32_t* seqlens,
                         void* o, int B, int Tmax, int H, int Hkv, int D,
                         int window, double rope_base, nc_dtype dtype,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * nc_attn_decode_shared -- one decode step for B samples continuing one
 * prompt, over a single shared copy of the prompt's cache ([S10] §10.6: the
 * prompt is prefilled once at batch 1 and every sample generates from its
 * cache; here the samples read the one prompt cache instead of copies of it).
 *
 *   q         (B, H,   D)        raw query of each sample's new token
 *   k_new     (B, Hkv, D)        raw key of the new token
 *   v_new     (B, Hkv, D)        value of the new token
 *   k_prompt  (Lp, Hkv, D)       rotated, normalised keys of prompt positions
 *                                0 .. Lp-1 (for instance written by
 *                                nc_attn_prefill with B = 1); only read
 *   v_prompt  (Lp, Hkv, D)       their values; only read
 *   k_cache   (B, Tgen, Hkv, D)  row r of sample b holds position Lp + r;
 *                                rows before L-1-Lp are used as stored, row
 *                                L-1-Lp is overwritten with norm(rope(k_new))
 *   v_cache   (B, Tgen, Hkv, D)  row L-1-Lp is overwritten with v_new
 *   seqlens   (B,) int32 DEVICE array, L = seqlens[b] in [Lp+1, Lp+Tgen]
 *                                counts the prompt, the sample's earlier
 *                                tokens and the new token (position L-1)
 *   o         (B, H, D)          softmax over positions max(0, L-window) ..
 *                                L-1, prompt positions from the shared cache
 * The result equals nc_attn_decode over per-sample caches holding the prompt
 * rows followed by the sample's rows. seqlens values outside [Lp+1, Lp+Tgen]
 * are clamped to that range. Workspace as for nc_attn_decode (a sample's keys
 * are processed in chunks that lie wholly in the prompt or wholly in its own
 * rows). Requires Lp >= 1, Tgen >= 1, the sizes of nc_attn_decode, and q,
 * k_new, v_new, o not overlapping any cache.
 */
size_t nc_attn_decode_shared_workspace_bytes(int B, int Lp, int Tgen, int H, int Hkv, int D,
                                             int window);
/* ve_new, ve_gate: as for nc_attn_decode. */
nc_status nc_attn_decode_shared(const void* q, const void* k_new, const void* v_new,
                                const void* ve_new, const void* ve_gate,
                                const void* k_prompt, const void* v_prompt, int Lp,
                                void* k_cache, void* v_cache, const int32_t* seqlens,
                                void* o, int B, int Tgen, int H, int Hkv, int D,
                                int window, double rope_base, nc_dtype dtype,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NC_ATTN_H */
