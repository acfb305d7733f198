// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hla.h"

namespace hla {

// Arguments of the chunk kernels (segment summaries and outputs).  All
// pointers are device pointers; sizes are validated by the ABI layer.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;  // [H] or nullptr
  int H, T, chunk, nspan, normalize;
  float eps;
  // summaries (written by the summary kernel) or exclusive prefixes (read by
  // the output kernel): [units, nspan, ...]
  float *S, *C, *m, *G, *h;
  float* o;    // [units, T, dv]
  float* den;  // [units, T] or nullptr
  // the segment-local p_t = S_t q_t (S from zero at the segment start), bf16,
  // [units, nspan, tiles, d, 64] (token-contiguous 64-token tiles), written
  // by the bf16 d = dv = 128 summary kernel when set; nullptr otherwise
  void* pl;
};

// One tree scan over slots (used for the run totals of the two-level scan).
struct ScanArgs {
  float *S, *C, *m, *G, *h;             // [units, n, ...] in place
  float *wS, *wC, *wm, *wG, *wh;        // padding slots [units, N - n, ...]
  const float* gamma;
  int H, n, N, chunk;
  int seg, nseg;                        // slot i holds segments [i seg, (i+1) seg) of nseg
  int step;                             // tree distance 2^level
  int d, dv;
};

// The whole exclusive scan of one problem, or (rS set) only the exclusive
// prefixes at the starts of the runs.
struct ScanPlan {
  float *S, *C, *m, *G, *h;             // [units, n, ...] in place (read only with rS)
  float *tS, *tC, *tm, *tG, *th;        // inclusive totals [units, ...], each may be nullptr
  float *rS, *rC, *rm, *rG, *rh;        // run prefixes [units, runs, ...], or all nullptr
  float* ws;                            // scan_workspace_floats(...) floats (nullptr if 0),
                                        // scan_runs_workspace_floats(...) with rS
  const float* gamma;
  int units, H, n, chunk, d, dv;
  // With oS set: the exclusive prefixes go to oS, oC, om, oG, oh ([units,
  // n, ...], disjoint from the segments, all set) and the segments are only
  // read; the rescan then writes every prefix itself (no separate C, m pass).
  float *oS = nullptr, *oC = nullptr, *om = nullptr, *oG = nullptr, *oh = nullptr;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  float *S, *C, *m, *G, *h;
  float* o;
  float* den;
  int H, normalize;
  float eps;
};

// Returns hipSuccess or the launch error.
hipError_t launch_chunk_summaries(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                  hipStream_t s);
// Outputs from the segment-local p (ChunkArgs::pl) instead of the S
// recurrence: bf16 inputs with d = dv = 128 only.
bool outp_supported(int dtype, int d, int dv);
// Bytes of the segment-local p for `units` units of T tokens in segments of `chunk`.
size_t outp_plocal_bytes(int64_t units, int64_t T, int chunk, int d);
hipError_t launch_outputs_from_p(int units, const ChunkArgs& a, hipStream_t s);
hipError_t launch_chunk_outputs(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                hipStream_t s);
bool chunk_shape_supported(int dtype, int d, int dv);

// Segments per run of the two-level scan, and the scratch it needs (run
// totals and the tree's padding slots; 0 with a single run).
int scan_run_length(int n);
size_t scan_workspace_floats(int64_t units, int n, int d, int dv);
// Scratch of the run-prefix scan: the tree's padding slots only.
size_t scan_runs_workspace_floats(int64_t units, int n, int d, int dv);
// Runs the whole exclusive scan (every launch, in order, on stream s).
hipError_t launch_scan(const ScanPlan& p, hipStream_t s);

// The unmasked variant: segment moments (S, C, m; G and h unused), the
// exclusive decayed running sum over a unit's segments (in place on S, C, m),
// and the outputs from the prefixes.
hipError_t launch_unmasked_summaries(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                     hipStream_t s);
hipError_t launch_unmasked_scan(const ChunkArgs& a, int units, int d, int dv, hipStream_t s);
hipError_t launch_unmasked_outputs(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                   hipStream_t s);
// One decode step of the unmasked variant (S, C, m of `a`; G and h unused).
hipError_t launch_unmasked_decode(int dtype, int d, int dv, int units, const DecodeArgs& a,
                                  hipStream_t s);

// The asymmetric variant AHLA: summaries P [units, n, d, dv], m [units, n, d],
// E [units, n, d, dv], n [units, n, d], X [units, n, d, d].
struct AhlaArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  int H, T, chunk, nspan, normalize;
  float eps;
  float *P, *m, *E, *n, *X;
  float* o;
  float* den;
};
hipError_t launch_ahla_summaries(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s);
hipError_t launch_ahla_scan(int d, int dv, int units, const AhlaArgs& a, hipStream_t s);
hipError_t launch_ahla_outputs(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s);
hipError_t launch_ahla_decode(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s);

hipError_t launch_decode(int dtype, int d, int dv, int units, const DecodeArgs& a, hipStream_t s);

// Third order: the scan of R and r over a unit's segments (in place:
// summaries in, exclusive prefixes out), given the moments' exclusive
// prefixes Sp, Pp, mp and the segments' Q, V, Z, z.  m, z, r arrays have row
// stride ldm (16 in the first-order-sum layout, 1 for plain [.., d]).
struct R3ScanArgs {
  const float *Sp, *Pp, *mp, *Q, *V, *Z, *z;
  float *R, *r;
  float *tR, *tr;        // inclusive totals [units, d, dv] and [units, d], or null
  const float* gamma;
  int H, seg, nseg, ldm, units;
};
struct Decode3Args {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  float *S, *P, *m, *R, *r;
  float* o;
  float* den;
  int H, normalize;
  float eps;
};
// Exclusive decayed running sum (a = gamma^seg) over each unit's nseg
// segments of elems[i] floats of x[i] (up to three arrays, a null x[i]
// skipped), in place, in one launch; totals [units, elems[i]] to total[i]
// when not null.
hipError_t launch_moments_scan(float* const x[3], float* const total[3], const int elems[3],
                               const float* gamma, int H, int seg, int nseg, int units, hipStream_t s);
hipError_t launch_r_scan(int d, int dv, int units, const R3ScanArgs& a, hipStream_t s);
// den[t] = den16[t][0] (den may be null); with normalize, o[t] /= den + eps.
hipError_t launch_finish3(float* o, const float* den16, float* den, size_t tokens, int dv,
                          int normalize, float eps, hipStream_t s);
// y[i] = x[16 i] for i < n.
hipError_t launch_gather_col0(const float* x, float* y, size_t n, hipStream_t s);
hipError_t launch_decode3(int dtype, int d, int dv, int units, const Decode3Args& a, hipStream_t s);

// hla_fwd in two parts (both host code, in the ABI layer): the argument
// checks (with check_ws, also those of a caller's workspace of
// workspace_bytes bytes), and the launches of the whole forward with the
// summaries and the scan's scratch in `workspace` (workspace_bytes >=
// hla_fwd_workspace_bytes; with at least hla_fwd_p_workspace_bytes, and a
// shape that has it, the segment-local p path; called only for a validated,
// non-empty problem).
hla_status fwd_validate(const hla_problem* p, const void* q, const void* k, const void* v,
                        float* o, float* den, const hla_state* final_state, const void* workspace,
                        size_t workspace_bytes, bool check_ws);
hla_status fwd_enqueue(const hla_problem* p, const void* q, const void* k, const void* v,
                       float* o, float* den, const hla_state* final_state, void* workspace,
                       size_t workspace_bytes, void* stream);

// First-order decayed sum y_t = sum_{s<=t} lam^(t-s) (a_t.b_s) c_s over the
// walk order (tokens 0..T-1, or T-1..0 when reverse), the building block of
// the backward pass.  Operands are [unit][T][width] rows, bf16 or fp32.
struct LaOperand {
  const void* p;
  int bf16;
};
struct LaArgs {
  LaOperand a, b, c;      // a, b: width Da; c: width Dc
  float* y;               // [unit][T][Dc] fp32 (bf16 with y_bf16), written or accumulated
  float* Hp;              // segment states [unit][nseg][Da][Dc] (workspace)
  const float* gamma;     // [H] or null (gamma = 1)
  int H, gexp;            // lam = gamma[unit % H] ^ gexp, gexp in {1, 2, 3}
  int T, seg, nseg;       // tokens per unit, tokens per segment, segments
  int reverse, accumulate;
  int mfma_bf16;          // contract in bf16 (fp32 accumulate) rather than fp32
  // add the mirrored pair: y_t = sum lam^(t-s) [(a_t.b_s) c_s + (a_t.c_s) b_s],
  // one state sum (b c^T + c b^T); needs Da == Dc, at least one MFMA K step
  int sym = 0;
  // Hp holds the transposed states ([Dc][Da] per segment): the prefixes of an
  // earlier sum with the same lam whose b and c are this one's c and b
  int hp_transposed = 0;
  // y is bf16 (an intermediate that is only ever read back as a bf16 MFMA
  // operand); not with accumulate
  int y_bf16 = 0;
  // when set (bf16 MFMA, fp32 b): the first pass that stages b also writes
  // it, rounded to bf16, here ([unit][T][Da]); after a summary pass the
  // output pass reads this copy instead of b
  void* b_copy = nullptr;
  // when set (output pass): the state after each segment's last tile, from
  // the state the segment started from, [unit][nseg][Da][Dc] (with Hp null:
  // the segment's own state, the same values a summary pass writes)
  float* Hout = nullptr;
  // with ch (summary passes only): a second sum with the same a, b and lam
  // whose value is the scalar in column 0 of the 16-wide rows of c2 (c2.p
  // null: the unit channel), formed by every thread beside the main one; its
  // segment states go to Hp2, [unit][nseg][Da][16], column 0 (the rest
  // written zero).  Not with sym, reverse or b_copy.
  int ch = 0;
  LaOperand c2{nullptr, 0};
  float* Hp2 = nullptr;
};
// prefixes_ready: Hp already holds this sum's exclusive segment prefixes (the
// same b, c and lam as an earlier call), so only the output pass runs; with
// Hp null every segment starts from the zero state.
hipError_t launch_first_order_sum(int Da, int Dc, int units, const LaArgs& a, hipStream_t s,
                                  bool prefixes_ready = false);
// The segment states alone: Hp[unit][s] = sum over segment s of
// lam^(L-1-i) b_i c_i^T (i local to the segment), from the zero state; a is
// not read.
hipError_t launch_first_order_states(int Da, int Dc, int units, const LaArgs& a, hipStream_t s);

// The prefix terms of three first-order sums that share a and lam and whose
// segment-local parts y already hold (every segment from the zero state):
//   y_i[t] += lam^(t - s0 + 1) a_t^T Hp_i[seg]     (s0 = the segment's first token)
// for outputs of widths Da (i = 0), E (1) and 16 (2); Hp_i the exclusive
// segment prefixes [unit][nseg][Da][width] (fp32); y_i [unit][T][width] in
// the MFMA operand type (bf16 with mfma_bf16, else fp32), updated in place.
struct PrefixTermArgs {
  LaOperand a;
  void* y[3];
  const float* Hp[3];
  const float* gamma;
  int H, gexp, T, seg, nseg;
  int mfma_bf16;
};
hipError_t launch_prefix_terms(int Da, int E, int units, const PrefixTermArgs& a, hipStream_t s);

// Upstream gradients of the ratio-normalised output from the unnormalised
// num [tokens, dv] and den [tokens] (fp32): g_num [tokens, dv] = dO / (den +
// eps); g_den [tokens, 16] holds -(dO . num) / (den + eps)^2 in column 0 and
// zeros elsewhere; one [tokens, 16] holds 1 in column 0 and zeros elsewhere.
// The three outputs are bf16 (bf16 != 0) or fp32.
hipError_t launch_norm_grad(int bf16, const float* num, const float* den, const float* dout,
                            float eps, size_t tokens, int dv, void* g_num, void* g_den, void* one,
                            hipStream_t s);
// y[i] = bf16(x[i]) for i < n.
hipError_t launch_to_bf16(const float* x, void* y, size_t n, hipStream_t s);

}  // namespace hla
