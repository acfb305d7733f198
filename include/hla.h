/*
 * hla.h -- C ABI of the masked second-order Higher-order Linear Attention
 * (HLA) forward, its decode step, the unmasked variant and the asymmetric
 * variant AHLA, for AMD Instinct MI355X (gfx950).
 *
 * The method (summaries of "Higher-order Linear Attention", arXiv 2510.27258,
 * gist.science, Japanese and French pages):
 *   - method section 1 (second-order HLA): per (batch, head) the prefix
 *     moments S_t = sum_{i<=t} k_i k_i^T, C_t = sum_{i<=t} q_i v_i^T,
 *     m_t = sum_{i<=t} q_i and the cross summaries G_t, h_t that remove the
 *     future terms of S_t C_t; the output o_t = q_t^T (S_t C_t - G_t) and a
 *     ratio-normalised variant divided by a masked denominator;
 *   - method section 4 (parallel training by associative scans): segment
 *     summaries joined by an associative semidirect-product operator whose
 *     cross term is S_B C_A, and an exclusive Blelloch scan of the summaries
 *     that reproduces the serial activations exactly;
 *   - key contribution 2: the same operators with exponential decay;
 *   - results and claims: O(d^2 + d dv) work and memory per token.
 *
 * Readings used where the pages are silent (decay gamma per head, in [0, 1]):
 *   G_t = g^2 G_{t-1} + g k_t (k_t^T C_{t-1}),  h_t = g^2 h_{t-1} + g k_t (k_t^T m_{t-1}),
 *   S_t = g S_{t-1} + k_t k_t^T,  C_t = g C_{t-1} + q_t v_t^T,  m_t = g m_{t-1} + q_t,
 *   num_t = q_t^T (S_t C_t - G_t),  den_t = q_t^T (S_t m_t - h_t),
 *   o_t = num_t (unnormalised) or num_t / (den_t + eps) (ratio-normalised).
 * Equivalently num_t = sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) (q_t.k_i)(q_j.k_i) v_j.
 * Segment combine (A then B, a = g^(length of B)):
 *   S = a S_A + S_B, C = a C_A + C_B, m = a m_A + m_B,
 *   G = a^2 G_A + G_B + a S_B C_A, h = a^2 h_A + h_B + a S_B m_A.
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer (memory of the current HIP device)
 *     unless stated otherwise; struct arguments are HOST pointers read during
 *     the call only.  The caller owns every buffer; the library allocates no
 *     device memory and keeps no pointer after it returns.
 *   - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t
 *     passed as void*; NULL = the default stream).  The caller synchronises.
 *   - All arguments are validated on the host before anything is enqueued;
 *     on any error nothing is launched and a non-zero hla_status is
 *     returned.  A HIP launch/runtime failure returns HLA_ERR_HIP.  No C++
 *     exception crosses the ABI.
 *   - Layouts are dense row-major (C order).  Every device pointer must be
 *     16-byte aligned (HLA_ERR_MISALIGNED).
 *   - Numerical conditions (den + eps = 0, NaN/Inf inputs) are not errors and
 *     follow IEEE arithmetic.
 *   - An empty problem (B, H, T or N equal to 0) is valid once its sizes and
 *     options pass validation: nothing is launched, pointers are not
 *     checked (they may be NULL) and HLA_OK is returned.
 *   - Supported head sizes: d, dv in {16, 32, 64, 128} with d/dv in
 *     {1/2, 1, 2}; fp32 inputs need d, dv <= 64 (HLA_ERR_UNSUPPORTED).
 *   - Calls on one device that share output or state buffers must be
 *     ordered by the caller (same stream or events); apart from the scratch
 *     array of hla_fwd_noalloc (below) the library holds no global mutable
 *     state, so distinct calls are otherwise independent.
 */
#ifndef HLA_H
#define HLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HLA_OK = 0,
  HLA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  HLA_ERR_BAD_SHAPE = 2,          /* negative size, T % chunk != 0, chunk <= 0 */
  HLA_ERR_BAD_DTYPE = 3,          /* in_dtype is not an hla_dtype */
  HLA_ERR_MISALIGNED = 4,         /* a device pointer is not 16-byte aligned */
  HLA_ERR_UNSUPPORTED = 5,        /* d / dv / dtype combination not built */
  HLA_ERR_WORKSPACE_TOO_SMALL = 6,
  HLA_ERR_ALIASING = 7,           /* an output overlaps an input it must not */
  HLA_ERR_HIP = 8,                /* no usable device, or a HIP call failed */
  HLA_ERR_BAD_VALUE = 9           /* eps not finite, normalize not 0/1, sizes too large */
} hla_status;

typedef enum { HLA_F32 = 0, HLA_BF16 = 1 } hla_dtype;

/* One forward problem: q, k [B, H, T, d], v [B, H, T, dv] of in_dtype. */
typedef struct {
  int32_t B, H, T, d, dv;
  int32_t chunk;        /* tokens per segment summary; T % chunk == 0 */
  int32_t in_dtype;     /* hla_dtype of q, k, v */
  int32_t normalize;    /* 0: o = num; 1: o = num / (den + eps) */
  float eps;            /* used when normalize == 1; must be finite */
  const float* gamma;   /* device [H] per-head decay in [0, 1]; NULL means 1.
                           Values are not range-checked (they live on the device). */
} hla_problem;

/* Struct of device arrays, fp32.  For segment summaries / prefixes:
 *   S [B, H, n, d, d], C [B, H, n, d, dv], m [B, H, n, d], G [B, H, n, d, dv],
 *   h [B, H, n, d] with n = T / chunk.
 * For decode state the leading dims are [N, H] instead of [B, H, n]. */
typedef struct { float *S, *C, *m, *G, *h; } hla_state;

/* Human-readable name of a status code (static string, never NULL). */
const char* hla_status_string(hla_status s);

/* Library version string (static). */
const char* hla_version(void);

/*
 * Segment summaries (method section 4: the summary of a token segment; its
 * moments and cross summaries are those of method section 1).  For every
 * (b, h) and every segment s of `chunk` tokens, writes the state the serial
 * recurrence reaches from the zero state after that segment's tokens:
 *   S = sum_i g^(c-i) k_i k_i^T, C = sum_j g^(c-j) q_j v_j^T, m = sum_j g^(c-j) q_j,
 *   G = sum_{j<i} g^((c-i)+(c-j)) k_i (k_i.q_j) v_j^T, h = the same without v_j
 * (1-based positions i, j inside the segment, c = chunk).
 * `out` fields are all required ([B,H,n,...] as above) and must not overlap
 * q, k or v.
 */
hla_status hla_fwd_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                   const void* v, const hla_state* out, void* stream);

/* Bytes of scratch hla_scan needs for this problem: 0 with at most 16
 * segments per (b, h); otherwise the run totals and the tree's padding slots,
 * B*H*N summaries of (d*d + 2*d*dv + 2*d) floats, N the power of two >= the
 * number of runs.  Host-only; returns 0 for an invalid problem. */
size_t hla_scan_workspace_bytes(const hla_problem* p);

/*
 * Exclusive scan (method section 4: the exclusive Blelloch scan of segment
 * summaries under the semidirect-product combine with cross term S_B C_A;
 * decay per key contribution 2 as read above), in its blocked two-level form:
 * runs of consecutive segments are reduced in order, the run totals go through
 * the Blelloch tree, and each run is rescanned from its prefix; the result is
 * the same up to fp32 rounding order.  In place: on entry `inout`
 * holds the n segment summaries of every (b, h); on return it holds the
 * exclusive prefixes P_s = s_0 (+) ... (+) s_{s-1} (P_0 = 0).  If
 * `total_out` is non-NULL, each of its non-NULL fields receives the
 * inclusive total of all n segments ([B, H, ...], the state after T tokens).
 * `workspace` must hold hla_scan_workspace_bytes(p) bytes (may be NULL when
 * that is 0, i.e. with at most 16 segments per (b, h)).
 */
hla_status hla_scan(const hla_problem* p, const hla_state* inout, const hla_state* total_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The exclusive scan of hla_scan (method section 4, as above) out of place:
 * `summaries` (as hla_fwd_chunk_summaries writes them) is only read, and
 * `prefixes_out` ([B, H, n, ...], all fields required, overlapping neither
 * `summaries` nor `workspace`) receives what hla_scan would leave in `inout`,
 * bit for bit.  With the segments left alone, the rescan writes every prefix
 * itself: in place, C and m of a segment are still read by other workgroups
 * when its prefix is known, so hla_scan rewrites them in a launch of its own.
 * total_out, workspace (hla_scan_workspace_bytes(p) bytes) and errors as for
 * hla_scan.
 */
hla_status hla_scan_into(const hla_problem* p, const hla_state* summaries,
                         const hla_state* prefixes_out, const hla_state* total_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Segments per run of the blocked scan: n when n <= 16, else the smallest
 * power of two R with R*R >= n (n = T / chunk).  Host-only; 0 for an
 * invalid problem. */
int32_t hla_scan_run_length(const hla_problem* p);

/* Bytes of scratch hla_scan_runs needs: the tree's padding slots, B*H*(N -
 * runs) summaries of (d*d + 2*d*dv + 2*d) floats (0 with a single run).
 * Host-only; returns 0 for an invalid problem. */
size_t hla_scan_runs_workspace_bytes(const hla_problem* p);

/*
 * The scan of method section 4 stopped at the run level: the n segments of
 * every (b, h) are cut into runs of R = hla_scan_run_length(p) consecutive
 * segments (the last run may be shorter), each run is reduced in order and
 * the run totals go through the exclusive Blelloch tree.  `run_prefix_out`
 * ([B, H, runs, ...], runs = ceil(n / R), all fields required, no overlap
 * with `summaries`) receives for run r the exclusive prefix at its first
 * segment, P_{rR} = s_0 (+) ... (+) s_{rR-1} (zero for r = 0).
 * `summaries` (as hla_fwd_chunk_summaries writes them) is only read.
 * When R divides n, hla_fwd_output called with chunk' = R * chunk and these
 * prefixes gives the outputs of hla_scan + hla_fwd_output at `chunk`: inside
 * a run the output kernel carries the state from one segment to the next
 * itself, so the prefixes of the other segments are never written.
 * `workspace` must hold hla_scan_runs_workspace_bytes(p) bytes and overlap
 * neither argument.
 */
hla_status hla_scan_runs(const hla_problem* p, const hla_state* summaries,
                         const hla_state* run_prefix_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of scratch hla_fwd_output needs (0 today; kept for ABI stability). */
size_t hla_fwd_output_workspace_bytes(const hla_problem* p);

/*
 * Outputs from the exclusive prefixes (method section 1: o_t = q_t^T (S_t C_t
 * - G_t) and the ratio-normalised variant; section 4: each segment continues
 * from its exclusive prefix).  o [B, H, T, dv] fp32 receives num (normalize
 * == 0) or num / (den + eps) (normalize == 1).  den [B, H, T] fp32 is
 * optional (NULL to skip) and receives the denominator before eps is added.
 * `prefixes` is what hla_scan leaves in `inout`.
 */
hla_status hla_fwd_output(const hla_problem* p, const void* q, const void* k, const void* v,
                          const hla_state* prefixes, float* o, float* den,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch hla_fwd needs: the n summaries plus hla_scan's scratch. */
size_t hla_fwd_workspace_bytes(const hla_problem* p);

/* Bytes of the segment-local p for segments of p->chunk tokens: bf16,
 * [B, H, n, ceil(chunk / 64), d / 16, 4, 64, 4]: per 64-token tile, for
 * column block cb (columns 16 cb .. 16 cb + 15) and row block r (tokens
 * 16 r .. 16 r + 15 of the tile), 64 groups of 4 values, group l holding
 * tokens 16 r + 4 (l / 16) + [0, 4) of column 16 cb + (l % 16) (the MFMA
 * accumulator's lane order); tokens past the segment end are zero.  Only
 * bf16 inputs with d = dv = 128 have this path: 0 otherwise, and 0 for an
 * invalid or empty problem.  Host-only. */
size_t hla_fwd_p_bytes(const hla_problem* p);

/*
 * hla_fwd_chunk_summaries that also writes the segment-local p (method
 * section 1: p_t = S_t q_t with the state S_t of method section 4 formed
 * from zero at each segment's start), which the summary kernel forms for
 * every token anyway, to `plocal` (hla_fwd_p_bytes(p) bytes, 16-byte
 * aligned, no overlap with q, k, v or `out`).  bf16 inputs with d = dv = 128
 * only (HLA_ERR_UNSUPPORTED otherwise).
 */
hla_status hla_fwd_chunk_summaries_p(const hla_problem* p, const void* q, const void* k,
                                     const void* v, const hla_state* out, void* plocal,
                                     void* stream);

/*
 * hla_fwd_output from the segment-local p (as hla_fwd_chunk_summaries_p
 * writes it) instead of k: with the segment's exclusive prefix S_P the state
 * at position j of the segment is g^(j+1) S_P + S^loc_j (decay per key
 * contribution 2), so p_j = g^(j+1) S_P q_j + p^loc_j and the outputs follow
 * without the S recurrence.  Same prefixes, outputs and errors as
 * hla_fwd_output (up to rounding); bf16 inputs with d = dv = 128 only.
 */
hla_status hla_fwd_output_from_p(const hla_problem* p, const void* q, const void* v,
                                 const void* plocal, const hla_state* prefixes, float* o,
                                 float* den, void* stream);

/* Bytes of workspace for hla_fwd's fastest plan.  With the summaries and
 * the scan's scratch (hla_fwd_workspace_bytes(p)) rounded up to 256 bytes,
 * then hla_fwd_p_bytes at chunk' = R * chunk, hla_fwd also keeps the
 * segment-local p of its spans and computes the outputs from it
 * (hla_fwd_chunk_summaries_p + hla_fwd_output_from_p); with room for the
 * n / R exclusive prefixes as well, it scans out of place (hla_scan_into)
 * instead of in place.  That room is found inside hla_fwd_workspace_bytes(p)
 * when spans of several chunks leave enough of it (it is sized for one
 * summary per chunk); otherwise it comes last, rounded up to 256 bytes.
 * Host-only; 0 for an invalid or empty problem. */
size_t hla_fwd_p_workspace_bytes(const hla_problem* p);

/*
 * Chunks per span of hla_fwd (a power of two R dividing n = T / chunk): each
 * workgroup of hla_fwd's summary and output kernels walks R consecutive
 * chunks, forming their summaries and combining them in order as it goes
 * (the first level of the scan of method section 4, fused with forming the
 * chunk summaries).  R is the smallest that leaves at most 16 span totals per
 * (b, h) while keeping at least 256 workgroups, else the largest that keeps
 * 256 workgroups.  Host-only; 0 for an invalid problem, 1 for an empty one.
 */
int32_t hla_fwd_span_chunks(const hla_problem* p);

/*
 * The whole chunk-parallel forward (method section 4): segment summaries,
 * exclusive scan, outputs -- the three calls above on one stream, with
 * chunk' = R * chunk, R = hla_fwd_span_chunks(p): hla_fwd_chunk_summaries
 * writes the n / R span totals (each the combine, in order, of R chunk
 * summaries), hla_scan turns them into exclusive prefixes, and
 * hla_fwd_output walks each span from its prefix.  The summaries are kept in
 * `workspace` (at least hla_fwd_workspace_bytes(p) bytes; with
 * hla_fwd_p_workspace_bytes(p) bytes the fastest plan: for the shapes that
 * have it, the summary kernel also keeps the segment-local p there and the
 * outputs come from it, hla_fwd_chunk_summaries_p and hla_fwd_output_from_p,
 * and the scan runs out of place, hla_scan_into).  o and den as in
 * hla_fwd_output; the results equal those of the three calls at `chunk` up
 * to fp32 rounding order.  If `final_state` is non-NULL its non-NULL fields
 * receive the state after all T tokens ([B, H, ...]), ready for
 * hla_decode_step.
 */
hla_status hla_fwd(const hla_problem* p, const void* q, const void* k, const void* v,
                   float* o, float* den, const hla_state* final_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * hla_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments (minus the workspace), results and errors as
 * hla_fwd, with the summaries and the scan's scratch kept in a device array
 * that the library owns.  That array has a fixed size,
 * hla_fwd_noalloc_max_workspace_bytes() = 64 MiB, per device: a problem with
 * hla_fwd_workspace_bytes(p) above it returns HLA_ERR_WORKSPACE_TOO_SMALL
 * before anything is enqueued.  Each device the library runs this on holds
 * its own copy of the array until the process ends; the call allocates and
 * frees nothing.  Every call on one device shares that device's array, which
 * keeps the last call's contents: calls on one device whose executions
 * overlap (different streams without ordering, or host threads) race on it
 * and must be ordered by the caller.
 */
size_t hla_fwd_noalloc_max_workspace_bytes(void);
hla_status hla_fwd_noalloc(const hla_problem* p, const void* q, const void* k, const void* v,
                           float* o, float* den, const hla_state* final_state, void* stream);

/*
 * The unmasked second-order variant (method section 1: the plain product
 * S^K_t C^QV_t, whose future terms -- key index after value index -- the
 * cross summaries G, h remove in the masked operator; key contribution 2:
 * the associative operators of the unmasked setting, with and without decay;
 * method section 4: segment summaries joined by an exclusive scan):
 *   num_t = q_t^T S_t C_t = sum_{i<=t} sum_{j<=t} g^((t-i)+(t-j)) (q_t.k_i)(k_i.q_j) v_j,
 *   den_t = q_t^T S_t m_t,
 * with S, C, m decayed as above and o = num or num / (den + eps).  Only the
 * S, C and m fields of an hla_state are used (G and h are ignored and may be
 * NULL); problem fields, o, den, errors and layouts are as for the masked
 * calls of the same name.
 *
 * hla_unmasked_chunk_summaries: per segment, the moments the recurrence
 *   reaches from zero: S = sum_i g^(c-i) k_i k_i^T, C = sum_j g^(c-j) q_j v_j^T,
 *   m = sum_j g^(c-j) q_j ([B, H, n, ...], must not overlap q, k, v).
 * hla_unmasked_scan: in place, the exclusive prefixes under the unmasked
 *   combine S = a S_A + S_B, C = a C_A + C_B, m = a m_A + m_B (a = g^(length
 *   of B); no cross term): P_s = sum_{r<s} a^(s-1-r) X_r with a = g^chunk.
 * hla_unmasked_output: o (and den) from those prefixes.
 * hla_unmasked_fwd: the three on one stream, the moments kept in `workspace`
 *   (hla_unmasked_fwd_workspace_bytes(p) = B*H*n*(d*d + d*dv + d) floats, not
 *   overlapping q, k or v).
 * hla_unmasked_decode_step: one token per unit applied to the state S, C, m
 *   ([N, H, ...] fp32, in place; results and claims: constant work per
 *   token), o = C'^T S' q (or divided by q^T S' m' + eps), den optional;
 *   arguments and errors as for hla_decode_step.  The state after a prefix
 *   is the moments hla_unmasked_chunk_summaries writes with chunk = T.
 */
hla_status hla_unmasked_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                        const void* v, const hla_state* out, void* stream);
hla_status hla_unmasked_scan(const hla_problem* p, const hla_state* inout, void* stream);
hla_status hla_unmasked_output(const hla_problem* p, const void* q, const void* k, const void* v,
                               const hla_state* prefixes, float* o, float* den, void* stream);
size_t hla_unmasked_fwd_workspace_bytes(const hla_problem* p);
hla_status hla_unmasked_fwd(const hla_problem* p, const void* q, const void* k, const void* v,
                            float* o, float* den, void* workspace, size_t workspace_bytes,
                            void* stream);
hla_status hla_unmasked_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                                    int32_t normalize, float eps, const float* gamma,
                                    const void* q, const void* k, const void* v,
                                    const hla_state* state, float* o, float* den, void* stream);

/*
 * The asymmetric variant AHLA (method section 2: the operator
 * Q (K^T Q)(K^T V), whose single path runs through an intermediate key index,
 * with the streaming summaries P^KV, m^K, E, n; method section 4: segment
 * summaries and an exclusive scan).  Reading of the causal form:
 *   num_t = sum_{i<=t} sum_{j<=i} g^(t-j) (q_t.k_i)(q_i.k_j) v_j,  den_t the same with v = 1,
 * i.e. P_t = g P_{t-1} + k_t v_t^T, m_t = g m_{t-1} + k_t, r_t = P_t^T q_t,
 * E_t = g E_{t-1} + k_t r_t^T, n_t = g n_{t-1} + k_t (q_t.m_t), num_t = E_t^T q_t,
 * den_t = q_t.n_t.  A segment summary also carries X = sum_i k_i q_i^T (no
 * decay); the combine (A then B, a = g^(length of B)) is P = a P_A + P_B,
 * m = a m_A + m_B, E = a E_A + E_B + a X_B P_A, n = a n_A + n_B + a X_B m_A.
 * State arrays (fp32, all required): P [B,H,n,d,dv], m [B,H,n,d],
 * E [B,H,n,d,dv], n [B,H,n,d], X [B,H,n,d,d].  Problem fields, o, den and
 * errors as for the masked calls of the same name.
 *
 * hla_ahla_chunk_summaries: per segment, the state reached from zero and X.
 * hla_ahla_scan: in place, the exclusive prefixes of P, m, E, n (X only
 *   read), walking each unit's segments in order.
 * hla_ahla_output: o (and den) from those prefixes.
 * hla_ahla_fwd: the three on one stream, the summaries kept in `workspace`
 *   (hla_ahla_fwd_workspace_bytes(p) = B*H*n*(2 d dv + 2 d + d d) floats, not
 *   overlapping q, k or v).
 * hla_ahla_decode_step: one token per unit applied in place to P, m, E, n
 *   ([N, H, ...] fp32; X is not used and may be NULL); o = E'^T q (or divided
 *   by q.n' + eps), den optional; arguments and errors as for hla_decode_step.
 *   The state after a prefix is what hla_ahla_chunk_summaries writes with
 *   chunk = T.
 */
typedef struct { float *P, *m, *E, *n, *X; } hla_ahla_state;
hla_status hla_ahla_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                    const void* v, const hla_ahla_state* out, void* stream);
hla_status hla_ahla_scan(const hla_problem* p, const hla_ahla_state* inout, void* stream);
hla_status hla_ahla_output(const hla_problem* p, const void* q, const void* k, const void* v,
                           const hla_ahla_state* prefixes, float* o, float* den, void* stream);
size_t hla_ahla_fwd_workspace_bytes(const hla_problem* p);
hla_status hla_ahla_fwd(const hla_problem* p, const void* q, const void* k, const void* v,
                        float* o, float* den, void* workspace, size_t workspace_bytes,
                        void* stream);
hla_status hla_ahla_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                                int32_t normalize, float eps, const float* gamma, const void* q,
                                const void* k, const void* v, const hla_ahla_state* state,
                                float* o, float* den, void* stream);

/*
 * Third-order HLA (method section 3: the masked interaction A A^T A with
 * A = Q K^T, its prefix moments S^K, S^Q, P^KV and cross summaries; method
 * section 4: the third-order scan, whose associative operator carries the
 * segment-level linear maps M^KQP, M^KQm; key contribution 3: online update,
 * streaming kernel, exact chunk-parallel algorithm).  Reading of the masked
 * output (decay g per head as for the second order):
 *   num_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} g^((t-i)+(t-j)+(t-l)) (q_t.k_i)(q_j.k_i)(q_j.k_l) v_l,
 *   den_t the same with v = 1, o = num or num / (den + eps);
 * equivalently num_t = q_t^T R_t with R_t = sum_{j<=t} g^(3(t-j)) p_j u_j^T,
 * p_j = S_j q_j, u_j = P_j^T q_j (S = sum g^(..) k k^T, P = sum g^(..) k v^T),
 * and den_t = q_t . r_t with u_j -> q_j . m_j (m = sum g^(..) k).
 *
 * A segment summary (from the zero state, 1-based positions j in a segment of
 * c tokens, a = g^c): the moments S, Q = sum g^(c-j) q_j q_j^T, P, m and the
 * cross summaries V = sum g^(2(c-j)) p_j q_j^T, Z = sum g^(2(c-j)) q_j u_j^T,
 * z = sum g^(2(c-j)) (q_j.m_j) q_j, R = sum g^(3(c-j)) p_j u_j^T,
 * r = sum g^(3(c-j)) (q_j.m_j) p_j (p, u, m local to the segment).  Combine
 * (A then B): moments X = a X_A + X_B; R = a^3 R_A + R_B + a S_A Z_B + M P_A,
 * r = a^3 r_A + r_B + a S_A z_B + M m_A with the segment map
 * M = a^2 S_A Q_B + a V_B.
 *
 * hla3_summary holds fp32 [B, H, n, ...] arrays: S, Q, V [d, d]; P, Z, R [d, dv];
 * m, z, r [d].  hla3_state holds fp32 S [.., d, d], P [.., d, dv], m [.., d],
 * R [.., d, dv], r [.., d] with leading [B, H] (final state) or [N, H]
 * (decode state).  Problem fields, layouts of q, k, v, o, den, errors and the
 * supported head sizes are those of the second-order calls.
 *
 * hla3_workspace_bytes: scratch of hla3_chunk_summaries and hla3_fwd (the
 *   unit channel, p, u and q.m per token in the input dtype, the summaries
 *   with m, z, r 16 floats wide, den 16 wide, a 16-wide total of m); 0 for
 *   an invalid or empty problem.
 * hla3_chunk_summaries: every segment's summary into `out` (all fields
 *   required, no overlap with q, k, v or the workspace).
 * hla3_scan: in place, the exclusive prefixes of S, P, m, R, r (Q, V, Z, z
 *   only read): the moments by a decayed running sum, R and r by the combine
 *   with the segment map, walking each (b, h)'s segments in order; the
 *   non-NULL fields of `total_out` ([B, H, ...]) receive the inclusive totals.
 * hla3_fwd: summaries, scan and outputs on one stream (the outputs continue
 *   p, u and q.m from the moments' prefixes and num, den from R's and r's);
 *   o [B, H, T, dv] fp32, den [B, H, T] (optional, before eps); the
 *   non-NULL fields of `final_state` receive the state after T tokens, ready
 *   for hla3_decode_step.  Precision as in the second order (bf16 inputs:
 *   bf16 MFMA operands, p, u and q.m stored as bf16, fp32 accumulation, state
 *   and scan; fp32 inputs: fp32 throughout).
 * hla3_decode_step: one token per unit applied in place to `state` ([N, H,
 *   ...], all fields required), o [N, H, dv] (num or num / (den + eps)) and the
 *   optional den [N, H]; arguments and errors as for hla_decode_step.
 */
typedef struct { float *S, *Q, *P, *m, *V, *Z, *z, *R, *r; } hla3_summary;
typedef struct { float *S, *P, *m, *R, *r; } hla3_state;
size_t hla3_workspace_bytes(const hla_problem* p);
hla_status hla3_chunk_summaries(const hla_problem* p, const void* q, const void* k, const void* v,
                                const hla3_summary* out, void* workspace, size_t workspace_bytes,
                                void* stream);
hla_status hla3_scan(const hla_problem* p, const hla3_summary* inout, const hla3_state* total_out,
                     void* stream);
hla_status hla3_fwd(const hla_problem* p, const void* q, const void* k, const void* v, float* o,
                    float* den, const hla3_state* final_state, void* workspace,
                    size_t workspace_bytes, void* stream);
hla_status hla3_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                            int32_t normalize, float eps, const float* gamma, const void* q,
                            const void* k, const void* v, const hla3_state* state, float* o,
                            float* den, void* stream);

/*
 * One streaming decode step (method section 1: the online update of the
 * prefix state; results and claims: constant work and memory per token).
 * For each of the N*H units: applies one token (q, k [N, H, d], v [N, H, dv]
 * of in_dtype) to `state` ([N, H, ...] fp32, updated in place) and writes
 * o [N, H, dv] fp32 (num, or num / (den + eps) when normalize == 1) and the
 * optional den [N, H] fp32 (before eps).  gamma: device [H] or NULL.
 */
hla_status hla_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                           int32_t normalize, float eps, const float* gamma,
                           const void* q, const void* k, const void* v,
                           const hla_state* state, float* o, float* den, void* stream);

/*
 * Backward pass of the masked forward.  The method section on parallel
 * training by associative scans motivates it; the pages give no formula, so
 * it is the plain gradient of the closed form
 *   num_t = sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) (q_t.k_i)(q_j.k_i) v_j
 * (den_t the same with v = 1) with respect to q, k and v, for an upstream
 * gradient dout = dL/do ([B, H, T, dv] fp32), o = num (normalize == 0) or
 * o = num / (den + eps) (normalize == 1, method section 1's ratio-normalised
 * variant).  gamma is not differentiated.
 *
 * With p_t = S_t q_t the forward is o_t = sum_{j<=t} g^(2(t-j)) (q_t.p_j) v_j,
 * and the gradient is seven first-order decayed sums over the tokens (p; the
 * others over the future tokens: dp, dv, dk, or the past: dq), each computed
 * chunk-parallel: segment states of `chunk` tokens, an exclusive decayed
 * running sum over the segments, then the outputs per segment.  For the
 * ratio-normalised output the forward's num and den are recomputed first,
 * and the gradient is that of the numerator with the value channel v = 1
 * appended and upstream gradient [dout / (den + eps), -(dout . num) /
 * (den + eps)^2]: two more first-order sums (the v = 1 channel's terms of dp
 * and dq).
 *
 * hla_bwd: writes dq, dk [B, H, T, d] and dv [B, H, T, dv] (fp32; they must
 *   not overlap each other, the inputs or the workspace).  Problem fields as
 *   for hla_fwd.  Precision as in the forward: bf16 inputs contract in bf16
 *   (the intermediates p and dp are stored as bf16, the upstream gradients
 *   are rounded to bf16 as MFMA operands) with fp32 accumulation and state;
 *   fp32 inputs stay fp32 throughout.
 * hla_bwd_workspace_bytes: the workspace hla_bwd needs (p and dp, fp32
 *   [B, H, T, d] each, of which bf16 inputs use half; the segment states,
 *   B*H*n*max(d, dv)^2 floats; the prefixes of the k k^T states,
 *   B*H*n*d*d floats, which p = S q and S dp share; with bf16 inputs, dout
 *   rounded to bf16, B*H*T*dv values; with normalize == 1 also the
 *   recomputed num and den, the two upstream gradients, the v = 1 channel,
 *   dp rounded to bf16 and hla_fwd's workspace); 0 for an invalid or empty
 *   problem.
 */
size_t hla_bwd_workspace_bytes(const hla_problem* p);
hla_status hla_bwd(const hla_problem* p, const void* q, const void* k, const void* v,
                   const float* dout, float* dq, float* dk, float* dv,
                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H */
