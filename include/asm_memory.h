/*
 * attention-state memory (ASM) on MI355X (gfx950): the library's C ABI.
 *
 * The method (sources cited by page title and section):
 *   [TS]   "Context Memorization for Efficient Long Context Generation",
 *          technical summary (gist.science): Metodología; Fase de
 *          Calibración Offline (Recolección, Agrupamiento, Agregación,
 *          Eficiencia); Fase de Inferencia Online (Recuperación, Fusión).
 *   [NEWS] "Búsqueda de Memoria Reemplaza Atención Lineal en Prefijos
 *          Largos" (aiexpert.news), the paragraph on how the method works.
 *
 * A long fixed prefix is replaced by a table of K entries per query head.
 * Entry k holds a centroid query c_k and the attention state (a_k, lse_k)
 * that summarises attention over the prefix: a is the softmax-weighted mean
 * of the values and lse = log Z, Z = sum_j exp(scale * q.k_j) ([TS]
 * Metodología).  The empty state is (a = 0, lse = -inf).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed in
 *     the layout given (the local KV of asm_decode_step takes strides).
 *     Shapes and scalars are host values.
 *   - dtype selects the element type of the "void*" tensors: ASM_BF16
 *     (uint16 bf16 bit patterns) or ASM_F32.  States (a, lse), inverse
 *     norms and outputs are always float32.
 *   - The caller owns every buffer, including the workspace `ws` whose size
 *     the matching *_ws() function returns (0 means ws may be NULL).  The
 *     library allocates no memory and keeps no state between calls except a
 *     thread-local error message and, for asm_decode_step_noalloc only, one
 *     fixed scratch array per GPU (see there).
 *   - Calls validate their arguments on the host before any launch, enqueue
 *     their kernels on `stream` and return without synchronising.  A
 *     negative status means nothing was enqueued (or, for ASM_ERR_HIP, that
 *     a launch failed); asm_last_error() then describes the problem.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - bf16 tensors must be 16-byte aligned; every row length and stride
 *     counted in elements must be a multiple of 8.
 *   - Outputs must not overlap inputs unless an entry point says so.
 *   - Two calls that share a workspace must not run concurrently.
 *   - Launch shapes and workspace sizes depend only on the arguments and
 *     the device (its compute-unit count); nothing is read from the
 *     environment.
 */
#ifndef ASM_MEMORY_H
#define ASM_MEMORY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum asm_status_code {
  ASM_OK = 0,
  ASM_ERR_NULL = -1,      /* a required pointer is NULL */
  ASM_ERR_SHAPE = -2,     /* a shape or scalar is out of the supported range */
  ASM_ERR_DTYPE = -3,     /* unknown dtype */
  ASM_ERR_ALIGN = -4,     /* pointer or stride misaligned for bf16 vector loads */
  ASM_ERR_WORKSPACE = -5, /* ws_bytes smaller than the *_ws() size, or ws NULL */
  ASM_ERR_HIP = -6        /* a HIP launch failed; see asm_last_error() */
};

enum asm_dtype { ASM_BF16 = 0, ASM_F32 = 1 };

/* ABI version of this header (bumped on any signature change). */
#define ASM_ABI_VERSION 9
int asm_abi_version(void);

/* Static text for a status code. */
const char* asm_status_str(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* asm_last_error(void);

/*
 * asm_centroid_inv_norms -- cinv[h,k] = 1/|C[h,k,:]|, or 0 for a zero row.
 * Retrieval scores a query against centroid k by cosine similarity ([TS]
 * Recuperación); the kernels use q.c_k * cinv_k, which orders centroids as
 * the cosine does for a fixed query.
 *   C    [H, K, d] dtype;  cinv [H, K] float32 (output).
 *   1 <= d <= 256 (multiple of 8 for bf16); H, K >= 0.
 */
int asm_centroid_inv_norms(int dtype, int H, int K, int d, const void* C, float* cinv,
                           hipStream_t stream);

/*
 * asm_decode_step -- one decode step against the memory ([TS] Recuperación
 * and Fusión; [NEWS]).  For every sequence b and query head h:
 *   1. idx[b,h] = the k maximising q[b,h].C[h,k] * cinv[h,k] (the cosine
 *      order), the lowest such k on exact float32 ties;
 *   2. the memory state (Abar[h,idx], LSEbar[h,idx]) is gathered;
 *   3. the local state: attention of q[b,h] over the sequence's local
 *      (non-prefix) tokens t = 0..kv_len[b]-1 of kv head g = h / (Hq/Hkv),
 *      with scores scale * q.k_t;
 *   4. out, out_lse = the online-softmax merge of the two states:
 *      a = (Z1 a1 + Z2 a2)/(Z1 + Z2), lse = log(Z1 + Z2).
 *   Prefix tokens are never read.
 * Arguments:
 *   B >= 1 sequences; Hq query heads, Hkv kv heads, Hq % Hkv == 0;
 *   d in {64, 128} for bf16 (any 1..256 for float32); K >= 1 entries.
 *   q      [B, Hq, d] dtype
 *   C      [Hq, K, d] dtype          cinv [Hq, K] float32 (see above)
 *   Abar   [Hq, K, d] float32        LSEbar [Hq, K] float32 (-inf = empty)
 *   Kl, Vl dtype; local key/value of (kv head g, token slot p) starts at
 *          element g*kv_head_stride + p*kv_tok_stride, d contiguous values.
 *          Sequence b occupies slots kv_start[b] .. kv_start[b]+kv_len[b]-1.
 *   kv_capacity  number of token slots addressable per kv head.
 *   kv_start, kv_len  [B] int32, device memory.
 *   max_kv_len   host-side upper bound on every kv_len[b] (sizes the grid).
 *   out    [B, Hq, d] float32; out_lse [B, Hq] float32 (nullable);
 *   out_idx [B, Hq] int32 (nullable).
 * A sequence whose kv_len/kv_start is negative, exceeds max_kv_len or runs
 * past kv_capacity is not read: its outputs are NaN (idx still written).
 * kv_len[b] == 0 gives the memory state itself.
 * Reproducibility: idx is the same on every run.  When the step has more
 * work units (64 centroids of a head, or 32 local tokens of a kv head) than
 * the persistent grid has waves, pairs of waves split their units at run
 * time, so out and out_lse may differ between runs in the last bits (the
 * local state's grouping changes; see the parity tolerance of the tests).
 * Smaller steps give one unit per wave and identical results every run.
 */
size_t asm_decode_step_ws(int dtype, int B, int Hq, int Hkv, int d, int K, int max_kv_len);
int asm_decode_step(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                    const void* q, const void* C, const float* cinv, const float* Abar,
                    const float* LSEbar, const void* Kl, const void* Vl,
                    int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                    const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                    float* out, float* out_lse, int32_t* out_idx,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_decode_step_begin, asm_decode_step_finish -- asm_decode_step as its
 * two launches, for callers that place other work, or a timer, between
 * them ([TS] Fase de Inferencia Online: Recuperación and the local
 * attention in the first, Fusión in the second).
 *   _begin  the main grid: the centroid scoring (the per-unit argmax keys)
 *           and the split-K attention over the local tokens (the partial
 *           states), both into the workspace; out is not touched.
 *   _finish the merge: the index from the keys, the gather of the memory
 *           state and the online-softmax merge with the partial states into
 *           out, out_lse and out_idx.
 * Both take exactly the arguments of asm_decode_step.  Called on one
 * stream, _begin then _finish, with the same arguments and workspace (and
 * nothing writing the workspace or the inputs in between), they compute
 * what asm_decode_step computes, with the same reproducibility.  _finish on
 * a workspace that no _begin of this shape filled gives unspecified
 * outputs, but reads nothing outside the workspace and the inputs.
 * Only for steps on the MFMA path in one launch: bf16, d in {64, 128},
 * Hq/Hkv in {1, 2, 4, 8}, each sequence's KV rows within 2 GiB, at most 2048
 * sequences; otherwise ASM_ERR_SHAPE before any launch.  The workspace size
 * is asm_decode_step_ws.
 */
int asm_decode_step_begin(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                          const void* q, const void* C, const float* cinv, const float* Abar,
                          const float* LSEbar, const void* Kl, const void* Vl,
                          int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                          const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                          float* out, float* out_lse, int32_t* out_idx,
                          void* ws, size_t ws_bytes, hipStream_t stream);
int asm_decode_step_finish(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                           const void* q, const void* C, const float* cinv, const float* Abar,
                           const float* LSEbar, const void* Kl, const void* Vl,
                           int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                           const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                           float* out, float* out_lse, int32_t* out_idx,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_decode_step_noalloc -- asm_decode_step without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * step's scratch (argmax keys, tile prefix, partial states) lives in one
 * array of ASM_NOALLOC_SCRATCH_BYTES bytes per GPU, part of the library's
 * code object: each GPU the library runs on holds it until the process
 * ends.  The call allocates nothing; the caller still passes every input
 * and output, with the meaning, layout and results of asm_decode_step.
 *   - The current HIP device must be the device of `stream`
 *     (ASM_ERR_SHAPE otherwise).  The first call on a device looks up the
 *     array's address there (hipGetSymbolAddress, which may load the
 *     library's device code on that device) and keeps it: make that first
 *     call outside graph capture; later calls may be captured.
 *   - A step that needs more scratch than the array holds (what
 *     asm_decode_step_ws reports for its shape, up to the layout this call
 *     uses) returns ASM_ERR_WORKSPACE before any launch; asm_decode_step
 *     with a workspace serves it.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; nothing in it needs to start at zero.  Calls that
 *     overlap on one GPU (other streams, other threads, two replays of a
 *     captured graph in flight) race on it: order them.
 */
#define ASM_NOALLOC_SCRATCH_BYTES (16u << 20)
int asm_decode_step_noalloc(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                            const void* q, const void* C, const float* cinv, const float* Abar,
                            const float* LSEbar, const void* Kl, const void* Vl,
                            int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                            const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                            float* out, float* out_lse, int32_t* out_idx, hipStream_t stream);

/*
 * asm_attend_step -- full attention of one decode step, without memory: the
 * baseline the method is timed against ([TS] Resultados Experimentales,
 * latency against full attention over the prefix; [ABS]).  For every
 * sequence b and query head h, the attention state of q[b,h] over the
 * sequence's tokens t = 0..kv_len[b]-1 of kv head g = h / (Hq/Hkv) -- for
 * the comparison, the prefix followed by the local tokens, one KV cache --
 * with scores scale * q.k_t:
 *   out[b,h] = sum_t softmax(s)_t v_t, out_lse[b,h] = log sum_t exp(s_t).
 * It runs the split-K attention and merge of asm_decode_step with the lookup
 * switched off and the merge started from the empty state.  Arguments as
 * asm_decode_step (Kc, Vc take the place of Kl, Vl); kv_len[b] == 0 gives
 * (0, -inf).  Needs bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}, each
 * sequence's rows within 2 GiB and min(B, 2048) * Hkv * ceil(max_kv_len / 32)
 * below 2^30; otherwise ASM_ERR_SHAPE (and _ws returns 0).
 */
size_t asm_attend_step_ws(int dtype, int B, int Hq, int Hkv, int d, int max_kv_len);
int asm_attend_step(int dtype, int B, int Hq, int Hkv, int d, float scale, const void* q,
                    const void* Kc, const void* Vc, int64_t kv_head_stride, int64_t kv_tok_stride,
                    int64_t kv_capacity, const int32_t* kv_start, const int32_t* kv_len,
                    int max_kv_len, float* out, float* out_lse, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * asm_decode_step_hier -- the decode step with the two-level lookup of an
 * index built by asm_build_index ([TS] Complejidad: the lookup grows with
 * the logarithm of the memory size through a hierarchical index; two levels
 * are used).  Per (b, h): the S super-centroids of head h are scored as in
 * step 1 of asm_decode_step (q.SC * scinv); the p best supers with members
 * are probed (lowest index on exact ties); idx[b,h] is the member entry k of
 * a probed super maximising q.C[h,k] * cinv[h,k] (lowest k on exact ties).
 * Steps 2-4 of asm_decode_step follow unchanged.  With p >= the number of
 * non-empty supers this is the flat search.
 *   bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}; 1 <= S <= min(K, 1024);
 *   1 <= p <= 32.
 *   SC [Hq, S, d] bf16; scinv [Hq, S]; offsets [Hq, S+1]; members [Hq, K]
 *   int32: as written by asm_build_index.
 *   Cg [Hq, K, d] bf16 and cginv [Hq, K] (both NULL, or both given): the
 *   entry table grouped by super, as written by asm_index_group_rows from
 *   C, cinv and members.  Given, the probed members' rows are read from Cg
 *   at their member positions, one dependent load round fewer than through
 *   members into C; the results are the same.
 *   out_probes [B, Hq, p] int32 (nullable): the probed supers, best first,
 *   -1 past the number of non-empty supers.  The probes of rank p-1 and
 *   below that tie exactly in score resolve to the lower super index.
 *   Other arguments as asm_decode_step; the workspace size comes from
 *   asm_decode_step_hier_ws.
 */
size_t asm_decode_step_hier_ws(int dtype, int B, int Hq, int Hkv, int d, int K, int S, int p,
                               int max_kv_len);
int asm_decode_step_hier(int dtype, int B, int Hq, int Hkv, int d, int K, int S, int p,
                         float scale, const void* q, const void* C, const float* cinv,
                         const void* SC, const float* scinv, const int32_t* offsets,
                         const int32_t* members, const void* Cg, const float* cginv,
                         const float* Abar, const float* LSEbar,
                         const void* Kl, const void* Vl, int64_t kv_head_stride,
                         int64_t kv_tok_stride, int64_t kv_capacity, const int32_t* kv_start,
                         const int32_t* kv_len, int max_kv_len, float* out, float* out_lse,
                         int32_t* out_idx, int32_t* out_probes, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Whitening at retrieval ([TS] Recuperación: the cosine lookup may run
 * after a whitening transform).  The transform of head h is
 * x -> W[h] (x - mu[h]), fit on that head's calibration queries:
 *   mu = mean of the rows, Sigma = their population covariance plus
 *   ridge * trace(Sigma) / d on the diagonal, W = Sigma^-1/2 (symmetric).
 * Whitened rows are rounded once, to nearest-even, to the row type.
 * d in {64, 128}; bf16 or float32 rows.
 *
 * asm_whiten_fit -- mu [H, d] and W [H, d, d] (float64) from X [H, N, d].
 *   The inverse square root is the coupled Newton-Schulz iteration in
 *   float64 (at most 100 rounds); resid [H] (float64, nullable) receives
 *   |Z Y - I|_F at exit, about 1e-14 when it converged.  Needs N >= 1 and
 *   ridge >= 0.  A head whose iteration does not converge (resid >= 1e-6 or NaN,
 *   e.g. a singular covariance with ridge = 0, or a constant corpus whose
 *   covariance is zero) gets W filled with NaN; the call itself still
 *   returns ASM_OK, since the outcome is only known on the device.
 *   Workspace: asm_whiten_fit_ws bytes.
 * asm_whiten_rows -- Yw = round(W[h] (Y - mu[h])) for M rows of each of H
 *   heads.  Row r of head h starts at element h*head_stride + r*row_stride
 *   of Y and of Yw (the same layout); d contiguous elements per row.  Yw
 *   must not overlap Y; W must be 16-byte aligned.  Whitening the memory table C [H, K, d] is
 *   (M = K, head_stride = K*d, row_stride = d); its inverse norms come from
 *   asm_centroid_inv_norms on the whitened table.
 * asm_decode_step_whitened -- asm_decode_step whose lookup scores the
 *   whitened query against the whitened table: q is whitened into the
 *   workspace (as asm_whiten_rows), idx[b,h] = argmax_k qw.Cw[h,k] *
 *   cwinv[h,k]; the local attention and the merge use the raw q.
 *   Cw, cwinv: the whitened table and its inverse norms; other arguments as
 *   asm_decode_step; workspace: asm_decode_step_whitened_ws bytes.
 */
size_t asm_whiten_fit_ws(int dtype, int H, int N, int d);
int asm_whiten_fit(int dtype, int H, int N, int d, const void* X, double ridge, double* mu,
                   double* W, double* resid, void* ws, size_t ws_bytes, hipStream_t stream);
int asm_whiten_rows(int dtype, int H, int64_t M, int d, const void* Y, int64_t head_stride,
                    int64_t row_stride, const double* mu, const double* W, void* Yw,
                    hipStream_t stream);
size_t asm_decode_step_whitened_ws(int dtype, int B, int Hq, int Hkv, int d, int K,
                                   int max_kv_len);
int asm_decode_step_whitened(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                             const void* q, const double* mu, const double* W, const void* Cw,
                             const float* cwinv, const float* Abar, const float* LSEbar,
                             const void* Kl, const void* Vl, int64_t kv_head_stride,
                             int64_t kv_tok_stride, int64_t kv_capacity, const int32_t* kv_start,
                             const int32_t* kv_len, int max_kv_len, float* out, float* out_lse,
                             int32_t* out_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_build_states -- prefix attention states of the calibration queries
 * ([TS] Recolección), chunk by chunk ([TS] Eficiencia: the prefix may be cut
 * into chunks encoded independently and merged with the online-softmax
 * identity).  For query head h (kv head g = h / (Hq/Hkv)) and query i:
 *   chunk c covers prefix tokens [c*chunk, min(L, (c+1)*chunk));
 *   (a_c, lse_c) = attention state of Q[h,i] over that chunk;
 *   the merged state is the running merge over c = 0, 1, ... in order.
 * Arguments:
 *   Q [Hq, N, d] dtype; Kp, Vp [Hkv, L, d] dtype; chunk >= 1.
 *   A_chunks [nc, Hq, N, d], LSE_chunks [nc, Hq, N] float32, nullable
 *     (nc = ceil(L/chunk)): per-chunk states, written when non-NULL.
 *   A [Hq, N, d], LSE [Hq, N] float32: merged states.  With accumulate != 0
 *     the incoming (A, LSE) are merged with this call's prefix states (a
 *     prefix streamed in pieces); otherwise they are overwritten.
 *   d in {64, 128} for bf16 (any 1..256 for float32).
 *   bf16 builds with d in {64, 128} and Hq/Hkv in {1, 2, 4, 8} convert Vp
 *   to fp16 once per call into the workspace (asm_build_states_ws bytes:
 *   Hkv*L*d*2 rounded up to 256, plus 256 for a flag) and take the
 *   probability-value products in fp16 with float32 accumulation.  If some
 *   finite Vp value has no fp16 form (magnitude 65520 or more), the
 *   conversion raises the flag and the whole call computes every state on
 *   the exact bf16 path instead (float32 vector arithmetic, much slower);
 *   the results stay finite and correct.  Other shapes need no workspace.
 */
size_t asm_build_states_ws(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk);
int asm_build_states(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk, float scale,
                     const void* Q, const void* Kp, const void* Vp,
                     float* A_chunks, float* LSE_chunks, float* A, float* LSE, int accumulate,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_build_states_streamed -- asm_build_states (A_chunks = LSE_chunks =
 * NULL) for a prefix held in host memory ([TS] Eficiencia: chunks are
 * encoded independently and merged, so the prefix need not be resident).
 * Chunk c (prefix tokens [c*chunk, min(L, (c+1)*chunk)) of every kv head) is
 * copied into one of two device staging slots on copy_stream while `stream`
 * encodes the previous chunk; each chunk then runs as one asm_build_states
 * call that merges into (A, LSE) (the first one with the caller's
 * `accumulate`).  The results equal asm_build_states on the same prefix
 * with the same chunk bit for bit: the chunk-end merge is the same
 * arithmetic.
 *   Kp_host, Vp_host [Hkv, L, d] dtype in host memory.  Pinned memory
 *   (hipHostMalloc) lets the copies overlap the compute; pageable memory
 *   works, with copies that do not overlap.  The host buffers must stay
 *   valid and unchanged until `stream` has passed this call's work.
 *   Q, A, LSE, scale, accumulate: as asm_build_states (device memory).
 *   ws: asm_build_states_streamed_ws bytes of device memory (four staging
 *   slots of Hkv*chunk*d elements, then asm_build_states' workspace).
 *   copy_stream: a stream distinct from `stream` for the copies; passing
 *   `stream` itself (or the same NULL stream) serialises copies and compute.
 *   On return all work is enqueued; `stream` is ordered after every copy and
 *   encode, copy_stream after the copies only.  Returns ASM_ERR_HIP if an
 *   event, copy or launch fails (work enqueued before the failure stays
 *   enqueued).
 */
size_t asm_build_states_streamed_ws(int dtype, int Hq, int Hkv, int N, int d, int chunk);
int asm_build_states_streamed(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk,
                              float scale, const void* Q, const void* Kp_host,
                              const void* Vp_host, float* A, float* LSE, int accumulate,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              hipStream_t copy_stream);

/*
 * asm_kmeans_assign -- nearest centroid by cosine for every collected query
 * ([TS] Agrupamiento clusters the queries; the metric is the retrieval
 * cosine of [TS] Recuperación).
 *   idx[h,i] = argmax_k X[h,i,:].C[h,k,:] * cinv[h,k], lowest k on ties.
 *   X [H, N, d] dtype; C [H, K, d] dtype; cinv [H, K] float32;
 *   idx [H, N] int32; best [H, N] float32 (nullable): the winning
 *   X.C * cinv (cosine times |x|).
 */
size_t asm_kmeans_assign_ws(int dtype, int H, int N, int K, int d);
int asm_kmeans_assign(int dtype, int H, int N, int K, int d, const void* X, const void* C,
                      const float* cinv, int32_t* idx, float* best,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_aggregate -- one memory-table update from an assignment ([TS]
 * Agregación).  Per head h and cluster k with members M = {i : idx[h,i]=k},
 * n = |M|:
 *   count[h,k] = n;
 *   n > 0: C[h,k] = mean of X[h,i] over M, summed in float64 and rounded
 *          once (nearest-even) to dtype;  n == 0: C[h,k] unchanged;
 *   cinv[h,k] = 1/|C[h,k]| (0 for a zero row), after the update;
 *   if Abar/LSEbar are non-NULL (then A and LSE must be too):
 *     Abar[h,k] = sum_M Z_i A[h,i] / sum_M Z_i,  Z_i = exp(LSE[h,i]),
 *     LSEbar[h,k] = log(mean_M Z_i);  (0, -inf) for an empty cluster.
 *   X [H, N, d] dtype; idx [H, N] int32 with 0 <= idx < K (others ignored);
 *   A [H, N, d], LSE [H, N] float32; C [H, K, d] dtype (in/out);
 *   cinv [H, K] float32; count [H, K] int32; Abar [H, K, d], LSEbar [H, K].
 */
size_t asm_aggregate_ws(int dtype, int H, int N, int K, int d);
int asm_aggregate(int dtype, int H, int N, int K, int d, const void* X, const int32_t* idx,
                  const float* A, const float* LSE, void* C, float* cinv, int32_t* count,
                  float* Abar, float* LSEbar, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * asm_build_memory -- the whole table build ([TS] Agrupamiento then
 * Agregación) in one call: C[h] = X[h, :K] (first-K initialisation), its
 * inverse norms, then `iters` rounds of asm_kmeans_assign and the mean step
 * of asm_aggregate; the last round also aggregates the states when A and
 * LSE are given.  The same results as that sequence of calls.
 *   X [H, N, d] dtype with N >= K; A [H, N, d], LSE [H, N] float32
 *   (nullable together with Abar, LSEbar).
 *   Outputs: C [H, K, d] dtype; cinv [H, K] float32; count [H, K] int32 (of
 *   the last partition); idx [H, N] int32 (the last partition); Abar
 *   [H, K, d], LSEbar [H, K] float32.
 *   Workspace: asm_build_memory_ws bytes.
 */
size_t asm_build_memory_ws(int dtype, int H, int N, int K, int d);
int asm_build_memory(int dtype, int H, int N, int K, int d, int iters, const void* X,
                     const float* A, const float* LSE, void* C, float* cinv, float* Abar,
                     float* LSEbar, int32_t* count, int32_t* idx, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * asm_build_index -- the two-level index used by asm_decode_step_hier.  For
 * every head the K entry queries C[h] are clustered into S super-centroids
 * with the build's cosine k-means (asm_kmeans_assign and the mean step of
 * asm_aggregate): first-S initialisation (SC[h] = C[h, :S]), then `iters`
 * rounds of assignment and mean.  The partition is the last assignment,
 * whose means are SC.
 *   C [H, K, d] dtype; 1 <= S <= K; iters >= 1.
 *   Outputs: SC [H, S, d] dtype; scinv [H, S] float32 (1/|SC|, 0 for a zero
 *   row); counts [H, S] int32; offsets [H, S+1] int32 (exclusive prefix of
 *   counts per head); members [H, K] int32: the entries of super s are
 *   members[h, offsets[h,s] .. offsets[h,s+1]), in unspecified order.
 *   Workspace: asm_build_index_ws bytes.
 */
size_t asm_build_index_ws(int dtype, int H, int K, int S, int d);
int asm_build_index(int dtype, int H, int K, int S, int d, int iters, const void* C, void* SC,
                    float* scinv, int32_t* counts, int32_t* offsets, int32_t* members, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * asm_index_group_rows -- the entry table grouped by super, for
 * asm_decode_step_hier ([TS] Complejidad: the members of a probed super are
 * then contiguous).  Cg[h, i, :] = C[h, members[h, i], :] and
 * cginv[h, i] = cinv[h, members[h, i]] for every head h and i < K; a member
 * outside [0, K) gives a zero row and 0.  Rebuild it whenever C, cinv or
 * the index change.
 *   dtype bf16 or float32; d in {64, 128}; C, Cg [H, K, d] 16-byte aligned,
 *   not overlapping; cinv, cginv [H, K] float32; members [H, K] int32.
 *   No workspace.
 */
int asm_index_group_rows(int dtype, int H, int K, int d, const void* C, const float* cinv,
                         const int32_t* members, void* Cg, float* cginv, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ASM_MEMORY_H */
