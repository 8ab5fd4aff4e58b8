/*
 * kata.h - C ABI of the MI355X (gfx950) KATA causal linear-attention library.
 *
 * The method: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
 * Cones" (Ghriss & Chakraborty, arXiv 2607.17419). Each query and key is projected onto
 * the unit sphere and lifted to the rank-one PSD feature psi(u) = u u^T (arXiv HTML page,
 * rank-one lift display after Eq. (8)); the feature is stored in n = p(p+1)/2 packed
 * coordinates (Eq. (8)); the output is the normalized causal readout
 *     o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t,  S_t = sum_{s<=t} psi(k_s) v_s^T,
 *     Z_t = sum_{s<=t} psi(k_s)
 * (normalized-readout paragraph; feature-value state display). Equivalently
 *     o_t = sum_{s<=t} (q_hat_t . k_hat_s)^2 v_s / sum_{s<=t} (q_hat_t . k_hat_s)^2.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory, allocated and owned by the caller, contiguous
 *     row-major, 16-byte aligned. The library never allocates, never frees, never
 *     synchronises and keeps no mutable global state; calls only enqueue work on
 *     `stream` and return. Results are valid once the stream has executed the work.
 *     One exception, by design: kata_chunked_fwd_noalloc keeps its workspace in a fixed
 *     device array of the library (one per GPU, shared by every call on that GPU).
 *   - Arguments are validated on the host before any HIP call. A call with a zero-sized
 *     problem (rows, B, H, T or N equal to 0) does nothing and returns KATA_OK; its
 *     pointers may then be NULL.
 *   - Packed feature order: row-major upper triangle including the diagonal,
 *     idx(i,j) = i*p - i*(i-1)/2 + (j-i) for 0 <= i <= j < p; off-diagonal entries carry
 *     a factor sqrt(2) so that <psi(a), psi(b)> = (a_hat . b_hat)^2 and ||psi(a)|| = 1.
 *   - A zero input vector lifts to zero (no epsilon); a zero denominator gives a zero
 *     output row (no epsilon). Causality is inclusive (s <= t). NaN/Inf propagate.
 *   - dtype: KATA_DTYPE_F32 (float) or KATA_DTYPE_BF16 (bfloat16, stored as uint16).
 *     bf16 inputs are computed with bf16 MFMA operands and fp32 accumulation; fp32 inputs
 *     are computed in fp32 throughout.
 *   - Errors are reported only through the returned status; KATA_ERR_HIP means the
 *     kernel launch failed (hipGetLastError) and the outputs are unspecified.
 *   - The [B, H, T, *] forwards address one sequence with 32-bit byte offsets:
 *     T * max(p, dv) * 4 must stay below 2^31 (KATA_ERR_SHAPE otherwise).
 */
#ifndef KATA_H
#define KATA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* kata_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum { KATA_DTYPE_F32 = 0, KATA_DTYPE_BF16 = 1 } kata_dtype_t;

typedef enum {
  /* The inter-chunk prefix is one sequential pass over all chunks: one workgroup per
   * (b,h) carries the state through every chunk (depth N_C; the pages' sequential
   * chunk traversal, chunked-forward paragraph). Needs no workspace. */
  KATA_SCAN_SEQUENTIAL = 0,
  /* Chunks are grouped into segments; per-segment state summaries are combined by a
   * log-depth (Hillis-Steele) associative scan, then every segment runs its chunks from
   * its exclusive prefix (chunked-forward paragraph: the prefix over chunks is an
   * associative vector-space cumulative sum). Needs the workspace. */
  KATA_SCAN_ASSOCIATIVE = 1
} kata_scan_t;

typedef enum {
  KATA_OK = 0,
  KATA_ERR_NULL = 1,        /* a required pointer is NULL */
  KATA_ERR_SHAPE = 2,       /* a size is negative, zero where it must be positive, or too large */
  KATA_ERR_DTYPE = 3,       /* a dtype argument is not a kata_dtype_t value */
  KATA_ERR_UNSUPPORTED = 4, /* valid but not implemented (p, dv, C combination) */
  KATA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  KATA_ERR_ALIAS = 6,       /* an output overlaps an input or another output */
  KATA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than kata_chunked_workspace_bytes */
  KATA_ERR_HIP = 8,         /* a HIP launch failed */
  KATA_ERR_SCAN = 9,        /* scan is not a kata_scan_t value */
  KATA_ERR_PASS = 10,       /* passes is not a non-empty combination of kata_pass_t bits */
  KATA_ERR_FEATURE = 11,    /* feature family not a kata_feature_t value, or g does not divide p */
  KATA_ERR_SCRATCH = 12     /* kata_chunked_fwd_noalloc: the call needs more workspace than
                             * KATA_NOALLOC_SCRATCH_BYTES */
} kata_status_t;

/* PSD feature families (reduced PSD families paragraph of the HTML page). The projected
 * query or key, normalised to the unit sphere, is split into g consecutive blocks of
 * m = p / g components u = (u_1, ..., u_g):
 *   FULL  : psi(u) = u u^T (g = 1), n = p(p+1)/2, weight (q.k)^2;
 *   SIGMA : KATA-Sigma g, psi(u) = sum_a u_a u_a^T, n = m(m+1)/2,
 *           weight sum_{a,b} (q_a . k_b)^2;
 *   BLOCK : KATA-M g, psi(u) = (u_1 u_1^T, ..., u_g u_g^T), n = g m(m+1)/2,
 *           weight sum_a (q_a . k_a)^2.
 * Packing inside an m x m block is the full map's (row-major upper triangle, sqrt(2) off
 * the diagonal); BLOCK concatenates the blocks, block 1 first. At g = 1 both reduced
 * families are the full map. */
typedef enum { KATA_FEAT_FULL = 0, KATA_FEAT_SIGMA = 1, KATA_FEAT_BLOCK = 2 } kata_feature_t;

/* The three passes of the chunked forward (bit mask). */
typedef enum {
  KATA_PASS_SUMMARIES = 1, /* per-segment state summaries into the workspace */
  KATA_PASS_SCAN = 2,      /* in-place associative scan of the summaries over the segments */
  KATA_PASS_SEGMENTS = 4,  /* every segment's chunks from its prefix: writes o */
  KATA_PASS_ALL = 7
} kata_pass_t;

/* n = p(p+1)/2 (Eq. (8)); -1 if p < 1. */
int64_t kata_packed_dim(int p);

/* Packed feature width n of a family (see kata_feature_t); -1 if p < 1, g does not divide
 * p, or fam is FULL with g != 1. */
int64_t kata_feature_dim(int p, kata_feature_t fam, int g);

/* Static, human-readable name of a status code (never NULL). */
const char* kata_status_string(kata_status_t s);

/*
 * kata_lift - packed rank-one lift of each row (rank-one lift display after Eq. (8)).
 *   u   : [rows, p] in u_dt.           psi : [rows, n] in psi_dt, n = p(p+1)/2.
 *   psi[r, idx(i,j)] = c_ij * u_hat[r,i] * u_hat[r,j], c_ii = 1, c_ij = sqrt(2) (i<j),
 *   u_hat = u / ||u|| computed in fp32 (zero row -> zero lift).
 *   Supported: 1 <= p <= 128. psi must not overlap u (KATA_ERR_ALIAS).
 */
kata_status_t kata_lift(const void* u, kata_dtype_t u_dt, int64_t rows, int p,
                        void* psi, kata_dtype_t psi_dt, kata_stream_t stream);

/*
 * Workspace bytes kata_chunked_fwd needs for these arguments (0 if none). Depends only
 * on its arguments, not on the device. Returns 0 for arguments kata_chunked_fwd would
 * reject. in_dt is needed because the segment summaries' layout depends on the kernel the
 * input dtype selects (fp32 VALU, or bf16 MFMA with fp16 or bf16 operands).
 */
size_t kata_chunked_workspace_bytes(int B, int H, int T, int p, int dv, int C,
                                    kata_scan_t scan, kata_dtype_t in_dt);

/*
 * kata_chunked_fwd - exact O(T) chunked-state forward (chunked-forward paragraph).
 *   q, k : [B, H, T, p] in in_dt.   v : [B, H, T, dv] in in_dt.   o : [B, H, T, dv] in o_dt.
 *   Per chunk of C tokens: the intra-chunk causal block (q_hat . k_hat)^2 over s <= t in
 *   the chunk, plus the readout psi(q_t)^T [S | Z] of the state accumulated over all
 *   earlier chunks; then the chunk's psi(K)^T [V | 1] is added to the state.
 *   T need not be a multiple of C (the tail chunk is zero-padded; zero keys add nothing).
 *   workspace: device buffer of at least kata_chunked_workspace_bytes(...) bytes,
 *   owned by the caller; its contents on entry are ignored and on exit unspecified.
 *   It may be NULL when that size is 0.
 *   Supported: p in {16, 32}; dv in {16, 32, 64}; C in {32, 64, 128}, for both input
 *   dtypes (fp32 inputs at p = 32, dv = 64, whose state does not fit in LDS at once, run in
 *   two halves of the value columns; each output column has the same denominator, so the
 *   split is exact).
 *   o must not overlap q, k, v or the workspace.
 */
kata_status_t kata_chunked_fwd(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                               void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                               int C, kata_scan_t scan, void* workspace,
                               size_t workspace_bytes, kata_stream_t stream);

/*
 * kata_chunked_fwd_passes - kata_chunked_fwd split into its passes (chunked-forward
 * paragraph: chunk summaries, the associative prefix over them, then every chunk from
 * its prefix). passes is a mask of kata_pass_t bits; the enabled passes run in the order
 * SUMMARIES, SCAN, SEGMENTS. Calls with masks 1, 2 and 4, issued in that order on one
 * stream with the same arguments and workspace, enqueue exactly the kernels of one
 * kata_chunked_fwd call and give the same o, bit for bit; mask 7 is kata_chunked_fwd.
 * The workspace carries the summaries between the calls and must not be touched in
 * between. With one segment (KATA_SCAN_SEQUENTIAL, or a single chunk) SUMMARIES and SCAN
 * enqueue nothing. Uses: timing the passes separately, and placing work between them
 * (for instance combining summaries of sequence shards held elsewhere). Arguments,
 * validation and errors as kata_chunked_fwd, plus KATA_ERR_PASS for a bad mask.
 */
kata_status_t kata_chunked_fwd_passes(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B, int H,
                                      int T, int p, int dv, int C, kata_scan_t scan,
                                      void* workspace, size_t workspace_bytes, int passes,
                                      kata_stream_t stream);

/* Size of the library's fixed device scratch array used by kata_chunked_fwd_noalloc. */
#define KATA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * kata_chunked_fwd_noalloc - kata_chunked_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * caller passes inputs and outputs only; the workspace kata_chunked_fwd would take is a
 * static device array of KATA_NOALLOC_SCRATCH_BYTES (64 MiB) owned by the library. Each GPU
 * the library runs on holds its own copy from the first call on that device (whose address is
 * resolved then, with hipGetSymbolAddress, while that device is current) until the process
 * ends. The call allocates and frees nothing, and no library routine it calls does.
 *   Arguments, validation, results and errors as kata_chunked_fwd (bit-identical output);
 *   the current device must be the one holding q, k, v, o and the stream. Arguments are
 *   validated before any HIP call; then a call whose workspace would exceed
 *   KATA_NOALLOC_SCRATCH_BYTES returns KATA_ERR_SCRATCH without enqueueing anything (every
 *   supported shape needs at most about 36 MB). The summaries in the array are written
 *   before they are read, so no call depends on what a previous one left there.
 *   Concurrency: every call on one GPU shares that GPU's array; calls whose work overlaps on
 *   one GPU (different streams, or different host threads without ordering) race on it and
 *   give unspecified results. Calls ordered on one stream are safe.
 */
kata_status_t kata_chunked_fwd_noalloc(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                       void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                       int C, kata_scan_t scan, kata_stream_t stream);

/*
 * kata_chunked_fwd_state - kata_chunked_fwd that also returns the recurrent state after the
 * last token of every sequence (feature-value state display: S_T = sum_{s<=T} psi(k_s) v_s^T
 * and Z_T = sum_{s<=T} psi(k_s), psi the packed lift above), in the layout kata_decode_step
 * reads and updates, so decoding continues from a chunked prefill:
 *   S : [B, H, n, dv] float32 and Z : [B, H, n] float32, packed order; written, not
 *   accumulated (T = 0 writes zeros). The state is the forward's own: built from bf16
 *   products with fp32 accumulation for bf16 inputs, in fp32 for fp32 inputs.
 *   Arguments, validation and errors as kata_chunked_fwd; S and Z must be non-NULL (when
 *   B * H > 0), 16-byte aligned, and must not overlap each other, q, k, v, o or the
 *   workspace (KATA_ERR_NULL, KATA_ERR_ALIGN, KATA_ERR_ALIAS).
 */
kata_status_t kata_chunked_fwd_state(const void* q, const void* k, const void* v,
                                     kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B, int H,
                                     int T, int p, int dv, int C, kata_scan_t scan,
                                     void* workspace, size_t workspace_bytes, float* S, float* Z,
                                     kata_stream_t stream);

/*
 * kata_quadratic_fwd - flash-attention-style forward without a state (abstract: the
 * flash-attention-style operating point). For each query block the kernel walks the key
 * blocks s <= t, accumulating sum_s (q_hat . k_hat_s)^2 [v_s | 1] on chip, and divides
 * once at the end. Weights lie in [0, 1], so no running maximum or rescaling is needed.
 *   q, k : [B, H, T, p] in in_dt.   v, o : [B, H, T, dv] (o in o_dt).
 *   Supported: p in {16, 32, 64}; dv in {16, 32, 64}. o must not overlap q, k, v.
 */
kata_status_t kata_quadratic_fwd(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                 void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                 kata_stream_t stream);

/*
 * kata_decode_step - one recurrent inference step per sequence and head (abstract:
 * constant-time recurrent inference; feature-value state display): update, then read out
 *     S += psi(k) v^T,  Z += psi(k),  o = psi(q)^T S / psi(q)^T Z.
 *   q, k : [N, H, p] in in_dt.   v : [N, H, dv] in in_dt.   o : [N, H, dv] in o_dt.
 *   S : [N, H, n, dv] float32 and Z : [N, H, n] float32, packed order above; both are
 *   read and updated IN PLACE (they are the complete recurrent state: saving them is a
 *   checkpoint, resuming from them continues bit for bit).
 *   Supported: 1 <= p <= 64; 1 <= dv <= 64 with dv % 4 == 0.
 *   o, S and Z must not overlap each other or q, k, v.
 */
kata_status_t kata_decode_step(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                               float* S, float* Z, void* o, kata_dtype_t o_dt, int N, int H,
                               int p, int dv, kata_stream_t stream);

/*
 * The forms above for any feature family (kata_feature_t, block count g). FULL with g = 1
 * is exactly the corresponding entry point above (same kernels). SIGMA and BLOCK run VALU
 * kernels (fp32 arithmetic for fp32 or bf16 inputs); the readout, denominator, state and
 * chunk algebra are the full map's with psi replaced by the family's map, and the weights
 * of the intra-chunk and quadratic forms are the family's block dot products.
 * Arguments, layouts, ownership and errors are those of the entry point without the
 * suffix, with n = kata_feature_dim(p, fam, g) for the state and the lift, plus
 * KATA_ERR_FEATURE for a bad (fam, g). kata_chunked_fwd_family also takes the optional
 * final-state outputs of kata_chunked_fwd_state: S [B,H,n,dv] and Z [B,H,n] fp32, both
 * NULL for none (one NULL alone is KATA_ERR_NULL). Supported for SIGMA / BLOCK: lift 1 <= p <= 128;
 * decode p <= 64, dv <= 64; quadratic p <= 64, dv <= 64; chunked p <= 64, dv <= 64,
 * C in {32, 64, 128} while its LDS state fits (160 KB).
 */
kata_status_t kata_lift_family(const void* u, kata_dtype_t u_dt, int64_t rows, int p,
                               kata_feature_t fam, int g, void* psi, kata_dtype_t psi_dt,
                               kata_stream_t stream);
size_t kata_chunked_workspace_bytes_family(int B, int H, int T, int p, int dv, int C,
                                           kata_scan_t scan, kata_dtype_t in_dt,
                                           kata_feature_t fam, int g);
kata_status_t kata_chunked_fwd_family(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int T, int p, int dv, int C, kata_scan_t scan,
                                      kata_feature_t fam, int g, void* workspace,
                                      size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream);
/*
 * kata_chunked_fwd_ragged - kata_chunked_fwd_family over sequences of different lengths in
 * the padded layout: sequence b uses its first lens[b] tokens of q, k, v ([B, H, T, *] as
 * above); lens is a device array of B int32 (16-byte aligned), values clamped to [0, T].
 * Output rows t >= lens[b] are not written (they keep what o held). With S, Z (both or
 * neither) the state after token lens[b] - 1 of every sequence is written (zero for an
 * empty sequence). Each sequence's result equals a call on that sequence alone (up to the
 * fp32 summation order of the segments: the segment plan is that of T). Errors as
 * kata_chunked_fwd_family; lens NULL is KATA_ERR_NULL when B * H * T > 0.
 */
kata_status_t kata_chunked_fwd_ragged(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int T, int p, int dv, int C, kata_scan_t scan,
                                      kata_feature_t fam, int g, const int32_t* lens,
                                      void* workspace, size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream);
/*
 * kata_chunked_fwd_varlen - kata_chunked_fwd_family over B sequences packed without padding
 * in the token-major layout: q, k are [total, H, p] and v, o are [total, H, dv] (row-major;
 * token cu_seqlens[b] + t of sequence b, head h, is row (cu_seqlens[b] + t) * H + h).
 * cu_seqlens is a device array of B + 1 int32 (4-byte aligned) with cu_seqlens[0] = 0,
 * non-decreasing, cu_seqlens[B] <= total; max_len must be at least every length
 * cu_seqlens[b + 1] - cu_seqlens[b] (longer sequences are cut at max_len). The kernels clamp
 * offsets to [0, total] and lengths to [0, max_len], so invalid contents give unspecified
 * results but no access outside the tensors. The workspace is that of the padded call with
 * T = max_len (kata_chunked_workspace_bytes_family(B, H, max_len, ...)). With S, Z (both or
 * neither) the state after each sequence's last token is written, [B, H, n, dv] and
 * [B, H, n] as for kata_chunked_fwd_state (zero for an empty sequence). Rows outside every
 * sequence are not written. bf16 KATA-Sigma 2 at p = 64, dv = 64, C in {64, 128} runs the
 * fp16 two-block kernels here as in the padded call; the virtual-row MFMA path of the other
 * bf16 Sigma 2 shapes takes the padded layout only, so those run here on the VALU family
 * kernel where its LDS fits (else KATA_ERR_UNSUPPORTED). Each sequence's result equals the
 * padded call on that sequence
 * alone (up to the fp32 summation order of the segments: the plan is that of max_len).
 * Errors as kata_chunked_fwd_family; KATA_ERR_NULL for cu_seqlens NULL when B * H > 0;
 * KATA_ERR_SHAPE for negative total / max_len or max_len * H * max(p, dv) * 4 >= 2^31.
 */
kata_status_t kata_chunked_fwd_varlen(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int total, int max_len, int p, int dv, int C,
                                      kata_scan_t scan, kata_feature_t fam, int g,
                                      const int32_t* cu_seqlens, void* workspace,
                                      size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream);
/*
 * kata_quadratic_fwd_varlen - kata_quadratic_fwd_family over B sequences packed without
 * padding, in the token-major layout of kata_chunked_fwd_varlen: q, k are [total, H, p] and
 * v, o are [total, H, dv]; token cu_seqlens[b] + t of sequence b, head h, is row
 * (cu_seqlens[b] + t) * H + h. Every sequence attends causally to its own tokens only
 * (abstract: flash-attention-style operating point; normalized-readout paragraph).
 * cu_seqlens is a device array of B + 1 int32 (4-byte aligned), cu_seqlens[0] = 0,
 * non-decreasing, cu_seqlens[B] <= total; max_len must be at least every length (longer
 * sequences are cut at max_len). Offsets are clamped to [0, total] and lengths to
 * [0, max_len], so invalid contents give unspecified results but no access outside the
 * tensors. No workspace, no state. Rows outside every sequence are not written. Each
 * sequence's rows equal, bit for bit, kata_quadratic_fwd_family on that sequence alone.
 *   Supported: the shapes of kata_quadratic_fwd_family (else KATA_ERR_UNSUPPORTED): the full
 *   map with p, dv in {16, 32, 64}, or KATA-Sigma g / KATA-M g (reduced PSD families
 *   paragraph) with p, dv <= 64; bf16 or fp32 inputs. bf16 runs the MFMA kernels (full map;
 *   KATA-Sigma 2 / KATA-M 2 at p = 64 with dv in {16, 32, 64}), every other case the VALU
 *   kernels (fp32 full map; the other families and fp32 families); fam, g as for
 *   kata_quadratic_fwd_family (KATA_ERR_FEATURE when g does not fit the family); o in o_dt,
 *   must not overlap q, k, v (KATA_ERR_ALIAS).
 *   Errors: KATA_ERR_NULL for a NULL tensor or cu_seqlens when B * H, total and max_len are
 *   all positive (otherwise nothing is done); KATA_ERR_ALIGN for a tensor not 16-byte or
 *   cu_seqlens not 4-byte aligned; KATA_ERR_SHAPE for negative sizes or
 *   (max_len + 512) * H * max(p, dv) * 4 >= 2^31.
 */
kata_status_t kata_quadratic_fwd_varlen(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                        void* o, kata_dtype_t o_dt, int B, int H, int total, int max_len,
                                        int p, int dv, kata_feature_t fam, int g, const int32_t* cu_seqlens,
                                        kata_stream_t stream);
kata_status_t kata_quadratic_fwd_family(const void* q, const void* k, const void* v,
                                        kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                        int H, int T, int p, int dv, kata_feature_t fam, int g,
                                        kata_stream_t stream);
kata_status_t kata_decode_step_family(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, kata_feature_t fam, int g, float* S,
                                      float* Z, void* o, kata_dtype_t o_dt, int N, int H, int p,
                                      int dv, kata_stream_t stream);

/*
 * Higher even-order lifts (HTML page, psi_2r display): psi_2r(u) = u_hat^(x 2r), packed over
 * the multisets i_1 <= ... <= i_2r of range(p) in lexicographic order with coordinate
 * sqrt((2r)! / prod multiplicity!) prod u_hat_i, so <psi_2r(q), psi_2r(k)> = (q_hat . k_hat)^(2r)
 * (r = 1: the rank-one lift above). The state binom(p + 2r - 1, 2r) x dv outgrows chip memory
 * already at r = 2 (the pages use r = 1), so the higher orders come as the lift and the
 * stateless quadratic form only.
 *   kata_order_dim: binom(p + 2r - 1, 2r); -1 if p < 1 or r outside 1..4 (or it overflows).
 *   kata_lift_order: as kata_lift with n = kata_order_dim(p, r); 1 <= p <= 128, r <= 4.
 *   kata_quadratic_fwd_order: as kata_quadratic_fwd with weights (q_hat . k_hat)^(2r);
 *   r = 1 is kata_quadratic_fwd; bf16 inputs with r = 2 and (p, dv) of the full map run the
 *   MFMA kernel, the rest a VALU kernel (p <= 64, dv <= 64). KATA_ERR_FEATURE for r outside 1..4.
 */
int64_t kata_order_dim(int p, int r);
kata_status_t kata_lift_order(const void* u, kata_dtype_t u_dt, int64_t rows, int p, int r, void* psi,
                              kata_dtype_t psi_dt, kata_stream_t stream);
kata_status_t kata_quadratic_fwd_order(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                       void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv, int r,
                                       kata_stream_t stream);

/*
 * kata_quadratic_bwd - gradients of the causal forward (any feature family) with respect to
 * q, k and v, given grad_o = dL/do. The pages describe no backward pass; this is the calculus
 * of the forward they define (normalized readout, the family's weights, the projection onto
 * the unit sphere): with D_t = sum_{s<=t} w_ts and delta_t = grad_o_t . o_t,
 *   dv_s = sum_{t>=s} (w_ts / D_t) grad_o_t,  dw_ts = (grad_o_t . v_s - delta_t) / D_t,
 *   and dw_ts through the block dot products and the normalisation to dq and dk (zero rows
 *   and rows with D_t = 0 get zero gradients).
 *   q, k : [B, H, T, p] and v, grad_o : [B, H, T, dv] in in_dt; dq, dk : [B, H, T, p] and
 *   dv_out : [B, H, T, dv] float32, written. workspace: at least
 *   kata_quadratic_bwd_workspace_bytes(B, H, T) bytes (D_t and delta_t per row).
 *   Flash-style O(T^2) VALU kernels (a reference for training, not a tuned kernel).
 *   Supported: p <= 64, dv <= 64, at most 16 block pairs (Sigma g: g <= 4). Outputs must not
 *   overlap each other, the inputs or the workspace.
 */
size_t kata_quadratic_bwd_workspace_bytes(int B, int H, int T);
kata_status_t kata_quadratic_bwd(const void* q, const void* k, const void* v, const void* grad_o,
                                 kata_dtype_t in_dt, int B, int H, int T, int p, int dv,
                                 kata_feature_t fam, int g, float* dq, float* dk, float* dv_out,
                                 void* workspace, size_t workspace_bytes, kata_stream_t stream);

/*
 * kata_quadratic_bwd_varlen - kata_quadratic_bwd for the full map over B sequences packed
 * without padding in the token-major layout of kata_quadratic_fwd_varlen: q, k, dq, dk are
 * [total, H, p] and v, grad_o, dv_out are [total, H, dv] (token cu_seqlens[b] + t of sequence
 * b, head h, is row (cu_seqlens[b] + t) * H + h). cu_seqlens: device int32 [B + 1], 4-byte
 * aligned, read on the device (offsets clamped to [0, total]); max_len bounds every length
 * (longer sequences are cut). Each sequence's gradients equal kata_quadratic_bwd's on that
 * sequence alone; rows outside every sequence are not written. bf16 inputs with p and dv in
 * {32, 64} run the bf16 MFMA kernels; bf16 or fp32 inputs with other p, dv <= 64 the VALU
 * kernels (else KATA_ERR_UNSUPPORTED). workspace: at least
 * kata_quadratic_bwd_varlen_workspace_bytes(B, H, total) bytes (D_t and delta_t per packed
 * row); 0 means unsupported arguments. Errors as kata_quadratic_bwd; KATA_ERR_NULL for
 * cu_seqlens NULL when B H > 0; KATA_ERR_SHAPE for negative sizes or
 * (max_len + 512) * H * max(p, dv) * 4 >= 2^31.
 */
size_t kata_quadratic_bwd_varlen_workspace_bytes(int B, int H, int total);
kata_status_t kata_quadratic_bwd_varlen(const void* q, const void* k, const void* v, const void* grad_o,
                                        kata_dtype_t in_dt, int B, int H, int total, int max_len, int p, int dv,
                                        const int32_t* cu_seqlens, float* dq, float* dk, float* dv_out,
                                        void* workspace, size_t workspace_bytes, kata_stream_t stream);

/*
 * kata_chunked_bwd - the same gradients as kata_quadratic_bwd for the full map, in O(T):
 * the state form of the forward (feature-value state display, normalized readout, chunked
 * forward paragraph of the HTML page) differentiated. A forward-time pass over the chunks
 * carries [S | Z] and gives D_t, delta_t and dq; a reverse-time pass carries
 * [R | r] = sum_{t>=s} psi(q_hat_t) [g_t / D_t | -delta_t / D_t] and gives dk and dv. Both
 * passes are split into segments whose summaries are scanned like the forward's (scan).
 *   q, k : [B, H, T, p] and v, grad_o : [B, H, T, dv] in in_dt; dq, dk : [B, H, T, p] and
 *   dv_out : [B, H, T, dv] float32, written. workspace: at least
 *   kata_chunked_bwd_workspace_bytes(B, H, T, p, dv, C, scan) bytes (D_t, delta_t per row and
 *   the two sets of segment summaries); 0 means unsupported arguments.
 *   bf16 inputs with p in {16, 32} and dv in {32, 64} run bf16 MFMA kernels: the bf16
 *   chunked forward (o in fp32 and its segment prefixes, in the workspace), then 32-token
 *   chunks whose state contractions, lift and lift transpose stay on chip; C only has to be
 *   in {16, 32, 64} there, and states, lifted features and per-pair weights are rounded to bf16
 *   before fp32 accumulation as in the forward (normwise error about 2e-3 to 3e-3 against the
 *   exact gradients). Other shapes and
 *   fp32 inputs run fp32 VALU kernels with the state n (dv + 1) fp32 and the chunk's rows
 *   within 160 KB of LDS (p <= 64, dv <= 64; p = 32, dv = 64 needs C = 16). Otherwise
 *   KATA_ERR_UNSUPPORTED. The workspace size depends on the shape, not on in_dt, and covers
 *   both paths. Outputs must not overlap each other, the inputs or the workspace.
 */
size_t kata_chunked_bwd_workspace_bytes(int B, int H, int T, int p, int dv, int C, kata_scan_t scan);
kata_status_t kata_chunked_bwd(const void* q, const void* k, const void* v, const void* grad_o, kata_dtype_t in_dt,
                               int B, int H, int T, int p, int dv, int C, kata_scan_t scan, float* dq, float* dk,
                               float* dv_out, void* workspace, size_t workspace_bytes, kata_stream_t stream);

/*
 * kata_chunked_bwd_varlen - kata_chunked_bwd over B sequences packed without padding in the
 * token-major layout of kata_chunked_fwd_varlen: q, k, dq, dk are [total, H, p] and v,
 * grad_o, dv_out are [total, H, dv] (token cu_seqlens[b] + t of sequence b, head h, is row
 * (cu_seqlens[b] + t) * H + h). cu_seqlens: device int32 [B + 1], 4-byte aligned, as for the
 * forward; max_len bounds every length (longer sequences are cut). Each sequence's gradients
 * equal the padded call's on that sequence alone; rows outside every sequence are not
 * written. bf16 inputs with p in {16, 32} and dv in {32, 64} run the bf16 MFMA state form;
 * fp32 inputs and the other shapes the fp32 VALU state form, at the largest chunk of 64, 32
 * and 16 whose state and rows fit LDS (p, dv <= 64; else KATA_ERR_UNSUPPORTED). workspace:
 * kata_chunked_bwd_varlen_workspace_bytes (D_t and delta_t of the total H rows and the
 * segment summaries of the plan of max_len; the larger of the two paths' needs, whatever the
 * input dtype); 0 means unsupported arguments. Errors as kata_chunked_bwd; KATA_ERR_NULL for
 * cu_seqlens NULL when B H > 0;
 * KATA_ERR_SHAPE for negative sizes or max_len * H * max(p, dv) * 4 >= 2^31.
 */
size_t kata_chunked_bwd_varlen_workspace_bytes(int B, int H, int total, int max_len, int p, int dv, kata_scan_t scan);
kata_status_t kata_chunked_bwd_varlen(const void* q, const void* k, const void* v, const void* grad_o,
                                      kata_dtype_t in_dt, int B, int H, int total, int max_len, int p, int dv,
                                      kata_scan_t scan, const int32_t* cu_seqlens, float* dq, float* dk,
                                      float* dv_out, void* workspace, size_t workspace_bytes, kata_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KATA_H */
