/*
 * libtxl — relative-positional self-attention over a cached memory, the hot path
 * of Dai et al., "Transformer-XL: Attentive Language Models Beyond a
 * Fixed-Length Context", for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership  Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *            library keeps no pointer after a call returns and allocates no
 *            device memory: temporaries live in a caller-provided workspace
 *            whose size the matching *_workspace_bytes() query returns.
 * Streams    `stream` is a hipStream_t (NULL = the default stream).  Work is
 *            enqueued asynchronously; returning TXL_OK means "enqueued".
 * Errors     Every argument is validated before anything is enqueued.  On an
 *            error nothing is launched, in/out arguments (mem_start) are left
 *            untouched and txl_last_error() holds a message for this thread.
 *            A failing HIP launch returns TXL_ERR_HIP.
 * Dtypes     One storage dtype per call (TXL_F32 or TXL_BF16) for every tensor
 *            argument; accumulation is always fp32; conversions to bf16 round
 *            to nearest even.  The bf16 path requires d_head <= 64.
 * Layouts    Row-major, no padding, no strides:
 *              h        [B][L][d_model]          current segment
 *              mem      [B][M][d_model]          memory ring: logical row p
 *                                                (oldest first) is physical
 *                                                slot (mem_start + p) mod M
 *              W_q, W_kE, W_v  [H*d_head][d_model]  (out x in; q = h W_q^T)
 *              W_kR     [H*d_head][d_pos]
 *              u, v     [H][d_head]
 *              R        [M+L][d_pos]             row delta = distance delta
 *              Rk       [M+L][H][d_head]         Rk[delta] = W_kR R_delta
 *              out      [B][L][H][d_head]        heads concatenated
 *            Head h owns rows h*d_head .. (h+1)*d_head-1 of each W and R is
 *            shared by all heads.
 * Indices    Query i in [0,L), key j in [0,M+L) over [memory ; segment],
 *            distance delta = M + i - j; key j is visible to query i iff
 *            j <= M + i (every memory slot plus the causal part of the segment).
 */
#ifndef TXL_H
#define TXL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TXL_ABI_VERSION 1

typedef enum {
  TXL_OK = 0,
  TXL_ERR_NULL_ARG = 1,             /* a required pointer is NULL              */
  TXL_ERR_BAD_SHAPE = 2,            /* a size is out of range or inconsistent  */
  TXL_ERR_BAD_DTYPE = 3,            /* dtype is not TXL_F32 / TXL_BF16         */
  TXL_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes below the query result  */
  TXL_ERR_UNSUPPORTED = 5,          /* valid but not implemented (e.g. bf16
                                       with d_head > 64)                       */
  TXL_ERR_HIP = 6                   /* a HIP runtime call or launch failed     */
} txl_status_t;

typedef enum { TXL_F32 = 0, TXL_BF16 = 1 } txl_dtype_t;

/* Shape of one relative-attention call (one layer, one segment). */
typedef struct {
  int32_t batch;     /* B >= 1                                             */
  int32_t seg_len;   /* L >= 1                                             */
  int32_t mem_len;   /* M >= 0 (0 = no memory: plain causal attention)     */
  int32_t d_model;   /* width of h and mem                                 */
  int32_t n_heads;   /* H >= 1                                             */
  int32_t d_head;    /* per-head width                                     */
  int32_t d_pos;     /* width of R (d_model in the paper)                  */
  int32_t dtype;     /* txl_dtype_t                                        */
  float scale;       /* multiplies the sum of the four score terms;
                        <= 0 selects 1/sqrt(d_head)                        */
} txl_attn_shape_t;

/* ABI version of the loaded library (TXL_ABI_VERSION of its build). */
int txl_abi_version(void);

/* Static text for a status code. */
const char* txl_status_str(txl_status_t status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* txl_last_error(void);

/*
 * Relative position table (Sec. 3.3: R is a sinusoid encoding matrix without
 * learnable parameters, row delta encodes distance delta).  Writes
 * R[n_pos][d_pos] with R[delta][2k] = sin(delta / 10000^(2k/d_pos)) and
 * R[delta][2k+1] = cos(delta / 10000^(2k/d_pos)), evaluated in fp64 and
 * rounded once to `dtype`.
 * Errors: NULL R; n_pos < 1 or d_pos < 1; bad dtype; HIP failure.
 */
txl_status_t txl_sinusoid_pos(void* R, int32_t n_pos, int32_t d_pos, int32_t dtype,
                              void* stream);

/*
 * Position keys for every distance (App. B: the matrix Q holds W_kR R_delta for
 * delta = M+L-1 .. 0; here they are stored in natural order):
 *   Rk[delta][h][c] = sum_x W_kR[h*d_head + c][x] * R[delta][x]
 * R [n_pos][d_pos], W_kR [n_heads*d_head][d_pos], Rk [n_pos][n_heads][d_head].
 * The result depends only on the weights and R, so a caller streaming segments
 * may compute it once per layer and pass it to txl_rel_attn_fwd as Rk.
 * `workspace` may be NULL when txl_rel_proj_workspace_bytes() returns 0.
 * Errors: NULL pointers; sizes < 1; bad dtype; workspace too small; HIP.
 */
size_t txl_rel_proj_workspace_bytes(int32_t n_pos, int32_t d_pos, int32_t n_heads,
                                    int32_t d_head, int32_t dtype);
txl_status_t txl_rel_proj(const void* R, const void* W_kR, void* Rk, int32_t n_pos,
                          int32_t d_pos, int32_t n_heads, int32_t d_head, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * One relative-attention forward over a cached memory (Sec. 3.3, the per-layer
 * summary equations, with H heads):
 *   h~  = [mem (logical order) ; h]
 *   q   = h W_q^T,  k = h~ W_kE^T,  val = h~ W_v^T          (per head)
 *   A_ij = scale * ( q_i.k_j + q_i.Rk[M+i-j] + u.k_j + v.Rk[M+i-j] )
 *   out_i = sum_j softmax_j(A_ij masked to j <= M+i) val_j
 * Rk: if non-NULL, the caller's position keys [M+L][H][d_head] (e.g. from
 * txl_rel_proj) and W_kR, R are not read (may be NULL); if NULL, Rk is computed
 * from W_kR and R (R needs >= M+L rows) inside the call.
 * mem may be NULL iff M == 0; mem_start must lie in [0, M) (0 when M == 0).
 * The memory is only read; advancing it is txl_mem_update's job.
 * Errors: NULL pointers; sizes out of range; scale NaN; bad dtype; bf16 with
 * d_head > 64 (TXL_ERR_UNSUPPORTED); workspace too small; HIP.
 */
size_t txl_rel_attn_workspace_bytes(const txl_attn_shape_t* shape);
txl_status_t txl_rel_attn_fwd(const txl_attn_shape_t* shape, const void* h, const void* mem,
                              int32_t mem_start, const void* W_q, const void* W_kE,
                              const void* W_kR, const void* W_v, const void* u, const void* v,
                              const void* R, const void* Rk, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * txl_rel_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same result and errors.  The
 * temporaries live in a static device array of TXL_STATIC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends.  A shape whose
 * txl_rel_attn_workspace_bytes() exceeds that returns
 * TXL_ERR_WORKSPACE_TOO_SMALL before anything is launched.  The call makes no
 * device allocation (and records no timing events).  All calls on one GPU
 * share its array and leave their contents in it: calls that overlap on one
 * GPU (different streams or threads) race, so the caller must order them.
 */
#define TXL_STATIC_SCRATCH_BYTES (96u << 20)
txl_status_t txl_rel_attn_fwd_static(const txl_attn_shape_t* shape, const void* h,
                                     const void* mem, int32_t mem_start, const void* W_q,
                                     const void* W_kE, const void* W_kR, const void* W_v,
                                     const void* u, const void* v, const void* R, const void* Rk,
                                     void* out, void* stream);

/*
 * Backward of txl_rel_attn_fwd (bf16 inputs; fp32 gradients).  Gradients flow
 * within the segment only: Sec. 3.2 puts a stop-gradient on the cached
 * memory, so nothing is returned for `mem`, while the keys and values computed
 * from it are ordinary tensors and receive gradients.  With s_ij = scale *
 * A_ij (Sec. 3.3 summary equations), P = Masked-Softmax(s), out = P val and
 * G = d_out:
 *   d_val_j  = sum_i P_ij G_i
 *   dS_ij    = P_ij (G_i . val_j - G_i . out_i)
 *   d_q_i    = scale sum_j dS_ij (k_j + Rk[M+i-j])        terms (a), (b)
 *   d_k_j    = scale sum_i dS_ij (q_i + u)                terms (a), (c)
 *   d_u      = scale sum_{b,i,j} dS_ij k_j                term (c)
 *   d_v      = scale sum_{b,i,j} dS_ij Rk[M+i-j]          term (d)
 *   d_Rk[delta] = scale sum over pairs with M+i-j = delta of dS_ij (q_i + v)
 *   d_W_kR   = sum_delta d_Rk[delta] (x) R_delta          (optional)
 * Inputs as txl_rel_attn_fwd (the forward is recomputed inside), plus d_out
 * [B][L][H][d_head] bf16.  Outputs (device, fp32, overwritten):
 *   d_q [B][L][H][d_head]; d_k, d_val [B][M+L][H][d_head] (memory rows first);
 *   d_u, d_v [H][d_head]; d_Rk [M+L][H][d_head]; d_W_kR [H*d_head][d_pos] or
 *   NULL (only allowed when Rk is NULL, i.e. computed from W_kR and R).
 * Workspace: txl_rel_attn_bwd_workspace_bytes() (0 for unsupported shapes).
 * Errors: fp32 (TXL_ERR_UNSUPPORTED); the errors of txl_rel_attn_fwd; NULL
 * gradient pointers; d_W_kR with a caller Rk (TXL_ERR_BAD_SHAPE).
 */
size_t txl_rel_attn_bwd_workspace_bytes(const txl_attn_shape_t* shape);
txl_status_t txl_rel_attn_bwd(const txl_attn_shape_t* shape, const void* h, const void* mem,
                              int32_t mem_start, const void* W_q, const void* W_kE,
                              const void* W_kR, const void* W_v, const void* u, const void* v,
                              const void* R, const void* Rk, const void* d_out, float* d_q,
                              float* d_k, float* d_val, float* d_u, float* d_v, float* d_Rk,
                              float* d_W_kR, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The same backward split at the forward, for training loops that run the
 * forward anyway: no recompute.
 * txl_rel_attn_fwd_train: txl_rel_attn_fwd's arguments and output (bf16
 * only), with a workspace of txl_rel_attn_bwd_workspace_bytes() in which it
 * leaves what the backward reads (projected q, K, V, Rk in the kernels'
 * layouts and each row's log-sum-exp).
 * txl_rel_attn_bwd_saved: the gradients of txl_rel_attn_bwd from that state.
 * `workspace` must be the one the forward used, unchanged since; `out` the
 * forward's output, unchanged; u, v the forward's; rk_given nonzero iff the
 * forward was passed a caller Rk; R (the forward's sinusoid table) is read
 * only for d_W_kR.  Outputs and their conditions as txl_rel_attn_bwd.
 * Errors: fp32 (TXL_ERR_UNSUPPORTED); NULL u, v, out, d_out, workspace or
 * gradient pointers; d_W_kR with rk_given or without R (TXL_ERR_BAD_SHAPE);
 * misaligned out, d_out, R (TXL_ERR_UNSUPPORTED); workspace too small.
 */
txl_status_t txl_rel_attn_fwd_train(const txl_attn_shape_t* shape, const void* h, const void* mem,
                                    int32_t mem_start, const void* W_q, const void* W_kE,
                                    const void* W_kR, const void* W_v, const void* u,
                                    const void* v, const void* R, const void* Rk, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream);
txl_status_t txl_rel_attn_bwd_saved(const txl_attn_shape_t* shape, const void* u, const void* v,
                                    const void* R, int32_t rk_given, const void* out,
                                    const void* d_out, float* d_q, float* d_k, float* d_val,
                                    float* d_u, float* d_v, float* d_Rk, float* d_W_kR,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Carried projected-K/V memory for evaluation (bf16 only, seg_len % 32 == 0).
 * Sec. 3.2 extends each segment with the cached hidden states,
 * h~ = [SG(m) ; h], and Sec. 3.3 projects k = h~ W_kE^T, val = h~ W_v^T row by
 * row.  With W_kE and W_v fixed (evaluation), the key and value of a memory
 * row are exactly those computed when that row was in the segment, so a ring
 * of projected keys and values can stand in for the hidden-state memory and a
 * step then projects only its L new rows.  The attention itself is unchanged:
 * same keys, values, position keys, mask and result as txl_rel_attn_fwd over
 * the hidden-state memory the ring was built from.
 *
 * Ring (one per layer, caller-owned device memory, txl_kv_ring_bytes()):
 * C = txl_kv_ring_slots() = round_up(M, 32) + L slots holding K
 * [B][H][C][64] followed by V^T in 32-slot tiles [B][C/32][H][64][32], bf16,
 * head width zero-padded to 64.  At ring start s, the G = round_up(M,32) - M
 * slots s .. s+G-1 (mod C) are unused, the next M hold the memory oldest
 * first, and the last L receive the segment's keys and values.  The layout is
 * internal to the library; only these functions read or write it.
 *
 * txl_kv_ring_init projects a hidden-state memory mem [B][M][d_model]
 * (logical row p at slot (mem_start + p) mod M, as in txl_rel_attn_fwd) into
 * the ring and sets *ring_start (HOST pointer) to 0.  mem may be NULL iff
 * M == 0.
 * txl_rel_attn_fwd_kv computes txl_rel_attn_fwd's output for the segment h
 * with the memory held by the ring, writes the segment's keys and values into
 * the ring (so it is also the memory update) and advances *ring_start (HOST
 * pointer, in/out, a multiple of 32 in [0, C)) by L mod C on success.
 * Ring calls of one layer must be stream-ordered.  Both take a workspace of
 * txl_kv_ring_workspace_bytes(); ring_bytes is the size of `ring`.
 * Errors: fp32 or seg_len % 32 != 0 (TXL_ERR_UNSUPPORTED); NULL pointers;
 * ring too small or *ring_start invalid (TXL_ERR_BAD_SHAPE); the errors of
 * txl_rel_attn_fwd.  The query functions return 0 for unsupported shapes.
 */
int32_t txl_kv_ring_slots(const txl_attn_shape_t* shape);
size_t txl_kv_ring_bytes(const txl_attn_shape_t* shape);
size_t txl_kv_ring_workspace_bytes(const txl_attn_shape_t* shape);
txl_status_t txl_kv_ring_init(const txl_attn_shape_t* shape, const void* mem, int32_t mem_start,
                              const void* W_kE, const void* W_v, void* ring, size_t ring_bytes,
                              int32_t* ring_start, void* workspace, size_t workspace_bytes,
                              void* stream);
txl_status_t txl_rel_attn_fwd_kv(const txl_attn_shape_t* shape, const void* h, const void* W_q,
                                 const void* W_kE, const void* W_kR, const void* W_v,
                                 const void* u, const void* v, const void* R, const void* Rk,
                                 void* ring, size_t ring_bytes, int32_t* ring_start, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Memory update (Sec. 3.2: the memory caches the M most recent hidden states,
 * possibly spanning several segments).  New logical memory = last M rows of
 * [memory ; h].  If L < M the L oldest ring slots are overwritten with h and
 * *mem_start advances by L (mod M); if L >= M the ring receives the last M
 * rows of h in order and *mem_start becomes 0.  M == 0 is a no-op.
 * mem [B][M][d_model] (device), mem_start (HOST pointer, in/out, written only
 * on success), h [B][L][d_model] (device).  Must be ordered after every read of
 * the old memory (same stream).
 * Errors: NULL pointers; sizes out of range; *mem_start outside [0, M); HIP.
 */
txl_status_t txl_mem_update(void* mem, int32_t* mem_start, const void* h, int32_t batch,
                            int32_t mem_len, int32_t seg_len, int32_t d_model, int32_t dtype,
                            void* stream);

/*
 * One layer of a segment step.  Required: W_q, W_kE, W_v, u, v, mem (if M > 0)
 * and either Rk or W_kR.  The rest of the layer (Sec. 3.3 summary equations:
 * o = LayerNorm(Linear(a) + h), then a position-wise feed-forward block) is
 * present iff W_o is non-NULL, and then W_ff1 [d_inner][d_model] and
 * W_ff2 [d_model][d_inner] are required:
 *   o  = LN(a W_o^T + h),  h' = LN(o + ReLU(o W_ff1^T) W_ff2^T)
 * with LN over d_model, eps 1e-5, no affine parameters.  Without W_o the layer
 * output is the attention output itself and H*d_head must equal d_model when
 * another layer follows.  W_o is [d_model][H*d_head].
 */
typedef struct {
  const void* W_q;
  const void* W_kE;
  const void* W_kR;
  const void* W_v;
  const void* u;
  const void* v;
  const void* Rk;     /* optional cached position keys [M+L][H][d_head]     */
  const void* W_o;    /* optional: NULL = attention-only layer              */
  const void* W_ff1;
  const void* W_ff2;
  void* mem;          /* this layer's memory ring [B][M][d_model]           */
} txl_layer_t;

/*
 * One segment through n_layers layers (Sec. 3.3 summary, for n = 1..N), with the
 * memory update of Sec. 3.2: layer n attends over [mem_n ; h^{n-1}] and then
 * mem_n receives h^{n-1} (its own input).  All layers share *mem_start (HOST
 * pointer, in/out), advanced once on success.  h_in [B][L][d_model];
 * h_out [B][L][d_out] with d_out = d_model if the last layer has W_o, else
 * H*d_head.  R (>= M+L rows) is needed by every layer whose Rk is NULL.
 * d_inner is the feed-forward width (ignored when no layer has W_o).
 * Errors: as txl_rel_attn_fwd, plus n_layers < 1 and layer pointer checks.
 */
size_t txl_segment_workspace_bytes(const txl_attn_shape_t* shape, int32_t n_layers,
                                   int32_t d_inner);
txl_status_t txl_segment_step(const txl_attn_shape_t* shape, int32_t n_layers, int32_t d_inner,
                              const txl_layer_t* layers, const void* R, const void* h_in,
                              void* h_out, int32_t* mem_start, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * txl_segment_step over per-layer K/V rings (evaluation; see txl_kv_ring_init):
 * rings[n] (ring_bytes each, txl_kv_ring_bytes()) carries layer n's projected
 * keys and values and replaces layers[n].mem, which is not read.  Every ring
 * must have been initialised (txl_kv_ring_init, from that layer's memory) and
 * all share *ring_start (HOST pointer, in/out), advanced by L mod C once on
 * success.  Same result as txl_segment_step on the hidden-state memories the
 * rings were built from.  Workspace: txl_segment_kv_workspace_bytes() (also
 * enough for txl_kv_ring_init).
 * Errors: as txl_segment_step and txl_rel_attn_fwd_kv.
 */
size_t txl_segment_kv_workspace_bytes(const txl_attn_shape_t* shape, int32_t n_layers,
                                      int32_t d_inner);
txl_status_t txl_segment_step_kv(const txl_attn_shape_t* shape, int32_t n_layers,
                                 int32_t d_inner, const txl_layer_t* layers,
                                 void* const* rings, size_t ring_bytes, const void* R,
                                 const void* h_in, void* h_out, int32_t* ring_start,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing (diagnostics, off by default).  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on its launch
 * stream.  txl_timing_read() waits for the recorded events, accumulates their
 * elapsed times per kernel kind, and fills up to `capacity` entries of names
 * (static strings), counts (launches) and total_ms; it returns the number of
 * kinds.  txl_timing_reset() drops everything accumulated.  Enabling adds two
 * event records per launch; keep it off for headline timings.
 */
txl_status_t txl_timing_enable(int32_t on);
void txl_timing_reset(void);
int32_t txl_timing_read(int32_t capacity, const char** names, int64_t* counts, double* total_ms);

/*
 * Matrix-core probe (diagnostics; no part of the attention path).  Measures the
 * bf16 matrix-core rate the chip sustains on given operand data, against which
 * the projection GEMM's throughput can be read.  Launches n_wg workgroups of
 * eight waves on `stream`; every wave issues `iters` rounds of 16 independent
 * 32x32x16 bf16 products (2 * 32 * 32 * 16 * 16 * iters * 8 * n_wg FLOP in
 * all), with operands taken from `operands`:
 *   operands  device, 16-byte aligned, n_wg * 512 * 24 units of 16 bytes (eight
 *             bf16 values each); thread t of workgroup w reads units
 *             (w * 512 + t) * 24 .. +23.  Caller-owned, read only.
 *   clocks    device, 2 * n_wg + 1 uint64 entries, caller-owned: entry 2w gets
 *             the shader-clock cycles and entry 2w + 1 the 100 MHz reference
 *             ticks of the product loop of workgroup w's first wave (their ratio
 *             times 100 MHz is the clock the matrix cores ran at); the last entry
 *             is scratch.
 * n_wg in [1, 65536], iters even and >= 2; TXL_ERR_NULL_ARG / TXL_ERR_BAD_SHAPE /
 * TXL_ERR_UNSUPPORTED (misaligned operands) before any launch.  Asynchronous:
 * time it with events on `stream`.
 */
txl_status_t txl_probe_mfma(const void* operands, int32_t n_wg, int32_t iters, uint64_t* clocks,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TXL_H */
