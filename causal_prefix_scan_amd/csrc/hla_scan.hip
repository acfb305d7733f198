// Exclusive scan of segment summaries under the semidirect-product combine
// ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 4 -- associative operator with cross term
// S_B C_A, exclusive Blelloch scan equal to the serial activations; key
// contribution 2 -- decayed operators).
//
// Combine of A followed by B with a = gamma^(tokens in B):
//   S = a S_A + S_B, C = a C_A + C_B, m = a m_A + m_B,
//   G = a^2 G_A + G_B + a S_B C_A, h = a^2 h_A + h_B + a S_B m_A.
// The identity is all zeros with length 0 (a = 1).
//
// Two levels.  The n segments of a (b, h) unit are cut into runs of R
// consecutive segments (one run when n is small):
//   1. run reduce:  each run's total, walking its segments in order;
//   2. run scan:    exclusive Blelloch scan of the run totals, in place: the
//                   up-sweep below the root, the top level (root = identity),
//                   then each down-sweep level in one launch that both moves
//                   the parent prefix left and combines it with the left sum;
//   3. run rescan:  each run walks its segments again from the run's
//                   exclusive prefix and overwrites every segment with its
//                   own exclusive prefix (rows of S, G, h);
//   4. C, m pass:   the same for C and m, elementwise.
// Steps 1-2 are skipped with a single run.  Each segment is read twice and
// written once, in four launches; the tree's levels only see the run totals.
// The run-prefix form stops after step 2 (the run totals reduced into the
// caller's run-prefix arrays and scanned there; segments only read): a
// forward pass whose output kernel walks whole runs needs nothing more, as it
// carries the state from one segment of a run to the next itself.  The
// out-of-place form writes every prefix to arrays of its own and leaves the
// segments as they were, so step 3 also writes C's and m's prefixes and
// step 4 is not needed.
//
// Steps 1 and 3 split a run's state over workgroups by 16-row blocks: a
// workgroup owns rows [r0, r0 + 16) of S, G and h, and keeps the whole
// running C and m, which its rows of the cross terms S_B C_A, S_B m_A need.
// In place, C and m are therefore only read in step 3 (every workgroup of the
// run reads them) and rewritten in step 4.  The cross term runs on fp32 MFMA
// with the running C as the B operand straight from registers.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int SCAN_THR = 256;
constexpr int SCAN_WAVES = SCAN_THR / 64;
constexpr int SCAN_RB = 16;      // state rows per combine workgroup

struct Slot {
  float *S, *C, *m, *G, *h;
};

__device__ __forceinline__ Slot slot_ptr(const ScanArgs& a, int unit, int idx) {
  const int d = a.d, dv = a.dv;
  Slot s;
  if (idx < a.n) {
    const size_t k = (size_t)unit * a.n + idx;
    s.S = a.S + k * d * d; s.C = a.C + k * d * dv; s.m = a.m + k * d;
    s.G = a.G + k * d * dv; s.h = a.h + k * d;
  } else {
    const size_t k = (size_t)unit * (a.N - a.n) + (idx - a.n);
    s.S = a.wS + k * d * d; s.C = a.wC + k * d * dv; s.m = a.wm + k * d;
    s.G = a.wG + k * d * dv; s.h = a.wh + k * d;
  }
  return s;
}

// Tokens in the slot range [lo, hi]: slot i holds segments
// [i seg, (i + 1) seg) of the nseg real ones, each of `chunk` tokens.
__device__ __forceinline__ int slot_tokens(const ScanArgs& a, int lo, int hi) {
  const int s0 = lo * a.seg;
  if (s0 >= a.nseg) return 0;
  const int s1 = (hi + 1) * a.seg < a.nseg ? (hi + 1) * a.seg : a.nseg;
  return (s1 - s0) * a.chunk;
}

// Up-sweep level: x[j] <- x[i] (+) x[j] for every pair; blockIdx.x = pair *
// (D/RB) + row block; a = gamma^(tokens in x[j]'s subtree).
template <int D, int E>
__global__ __launch_bounds__(SCAN_THR) void scan_combine_kernel(ScanArgs a) {
  constexpr int LDC = E + 4, LDS_ = D + 4, ET = E / 16, NRB = D / SCAN_RB;
  __shared__ __attribute__((aligned(16))) float sC[D * LDC];
  __shared__ __attribute__((aligned(16))) float sS[SCAN_RB * LDS_];
  __shared__ float sm[D];

  const int unit = blockIdx.y;
  const int step = a.step;
  const int pair = blockIdx.x / NRB, rb = blockIdx.x % NRB;
  const int j = (pair + 1) * 2 * step - 1;
  const int i = j - step;
  if (i - step + 1 >= a.n) return;   // both subtrees are padding: identity (+) identity
  const Slot A = slot_ptr(a, unit, i), B = slot_ptr(a, unit, j);
  const int lenB = slot_tokens(a, j - step + 1, j);
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), lenB);
  const float al2 = al * al;
  const int r0 = rb * SCAN_RB;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = tid; t < D * E / 4; t += SCAN_THR) {
    const int r = (4 * t) / E, c = (4 * t) % E;
    *reinterpret_cast<f32x4*>(sC + r * LDC + c) = reinterpret_cast<const f32x4*>(A.C)[t];
  }
  for (int t = tid; t < SCAN_RB * D / 4; t += SCAN_THR) {
    const int r = (4 * t) / D, c = (4 * t) % D;
    *reinterpret_cast<f32x4*>(sS + r * LDS_ + c) =
        reinterpret_cast<const f32x4*>(B.S + (size_t)r0 * D)[t];
  }
  for (int t = tid; t < D; t += SCAN_THR) sm[t] = A.m[t];
  __syncthreads();

  // G rows [r0, r0 + 16): a^2 G_A + G_B + a S_B C_A
  for (int et = wave; et < ET; et += SCAN_WAVES) {
    const f32x4 acc = gemm_f32_tile<D>(sS, LDS_, sC, LDC, 0, 16 * et, lane, zero4());
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t e = (size_t)(r0 + 4 * (lane >> 4) + q) * E + 16 * et + (lane & 15);
      B.G[e] = al2 * A.G[e] + B.G[e] + al * acc[q];
    }
  }
  // h rows: a^2 h_A + h_B + a S_B m_A
  for (int r = tid; r < SCAN_RB; r += SCAN_THR) {
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc += sS[r * LDS_ + c] * sm[c];
    B.h[r0 + r] = al2 * A.h[r0 + r] + B.h[r0 + r] + al * acc;
  }
  // S, C, m rows: a X_A + X_B
  for (int t = tid; t < SCAN_RB * D / 4; t += SCAN_THR) {
    const size_t e = (size_t)r0 * D / 4 + t;
    reinterpret_cast<f32x4*>(B.S)[e] = reinterpret_cast<const f32x4*>(A.S)[e] * al +
                                       reinterpret_cast<const f32x4*>(B.S)[e];
  }
  for (int t = tid; t < SCAN_RB * E / 4; t += SCAN_THR) {
    const size_t e = (size_t)r0 * E / 4 + t;
    reinterpret_cast<f32x4*>(B.C)[e] = reinterpret_cast<const f32x4*>(A.C)[e] * al +
                                       reinterpret_cast<const f32x4*>(B.C)[e];
  }
  for (int t = tid; t < SCAN_RB; t += SCAN_THR) B.m[r0 + t] = al * A.m[r0 + t] + B.m[r0 + t];
}

// Top of the tree: the up-sweep stops below the root, whose value (the total)
// the exclusive scan never uses; the down-sweep's first level, with the root
// reset to the identity, is then x[N-1] <- x[N/2-1], x[N/2-1] <- identity.
// blockIdx.x = unit * parts + part; one f32x4 of (S | C | G | m | h) per thread.
__global__ __launch_bounds__(256) void scan_top_kernel(ScanArgs a, int parts) {
  const int unit = blockIdx.x / parts, part = blockIdx.x % parts;
  const Slot x = slot_ptr(a, unit, a.N / 2 - 1), y = slot_ptr(a, unit, a.N - 1);
  const int nS = a.d * a.d / 4, nC = a.d * a.dv / 4, nm = a.d / 4;
  for (int t = part * 256 + threadIdx.x; t < nS + 2 * nC + 2 * nm; t += parts * 256) {
    f32x4 *px, *py;
    int o;
    if (t < nS) { px = reinterpret_cast<f32x4*>(x.S); py = reinterpret_cast<f32x4*>(y.S); o = t; }
    else if (t < nS + nC) { px = reinterpret_cast<f32x4*>(x.C); py = reinterpret_cast<f32x4*>(y.C); o = t - nS; }
    else if (t < nS + 2 * nC) { px = reinterpret_cast<f32x4*>(x.G); py = reinterpret_cast<f32x4*>(y.G); o = t - nS - nC; }
    else if (t < nS + 2 * nC + nm) { px = reinterpret_cast<f32x4*>(x.m); py = reinterpret_cast<f32x4*>(y.m); o = t - nS - 2 * nC; }
    else { px = reinterpret_cast<f32x4*>(x.h); py = reinterpret_cast<f32x4*>(y.h); o = t - nS - 2 * nC - nm; }
    py[o] = px[o];
    px[o] = zero4();
  }
}

// One down-sweep level below the top, one workgroup (16 waves) per pair
// (i, j = i + step): with A = x[j] (the parent's prefix) and B = x[i] (the left
// subtree's sum), x[i] <- A and x[j] <- A (+) B, a = gamma^(tokens in the left
// subtree).  C_A, m_A and all of S_B are staged in LDS before anything is
// written; every other element is read and then written by the same thread,
// so the pair needs no second launch for the swap.  Groups of 4 waves take the
// 16-row blocks round robin
// (two groups at d = 128, where the 128 registers of a 16-wave workgroup
// would not hold the row block's GEMM)
template <int D>
struct DownThreads {
  static constexpr int value = D == 128 ? 2 * SCAN_THR : 4 * SCAN_THR;
};
template <int D, int E>
__global__ __launch_bounds__(DownThreads<D>::value) void scan_down_kernel(ScanArgs a) {
  constexpr int DOWN_THR = DownThreads<D>::value, DOWN_GROUPS = DOWN_THR / SCAN_THR;
  constexpr int LDC = E + 4, LDS_ = D + 4, ET = E / 16, NRB = D / SCAN_RB;
  __shared__ __attribute__((aligned(16))) float sC[D * LDC];
  __shared__ __attribute__((aligned(16))) float sS[D * LDS_];
  __shared__ float sm[D];

  const int unit = blockIdx.y;
  const int step = a.step;
  const int j = (blockIdx.x + 1) * 2 * step - 1;
  const int i = j - step;
  if (i - step + 1 >= a.n) return;   // the left subtree is padding: nothing reads these prefixes
  const Slot X = slot_ptr(a, unit, i), Y = slot_ptr(a, unit, j);
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), slot_tokens(a, i - step + 1, i));
  const float al2 = al * al;
  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = tid / SCAN_THR, gt = tid % SCAN_THR, gw = gt >> 6;

  for (int t = tid; t < D * E / 4; t += DOWN_THR) {
    const int r = (4 * t) / E, c = (4 * t) % E;
    *reinterpret_cast<f32x4*>(sC + r * LDC + c) = reinterpret_cast<const f32x4*>(Y.C)[t];
  }
  for (int t = tid; t < D * D / 4; t += DOWN_THR) {
    const int r = (4 * t) / D, c = (4 * t) % D;
    *reinterpret_cast<f32x4*>(sS + r * LDS_ + c) = reinterpret_cast<const f32x4*>(X.S)[t];
  }
  for (int t = tid; t < D; t += DOWN_THR) sm[t] = Y.m[t];
  __syncthreads();

  for (int rb = grp; rb < NRB; rb += DOWN_GROUPS) {
    const int r0 = rb * SCAN_RB;
    // G rows: a^2 G_A + G_B + a S_B C_A
    for (int et = gw; et < ET; et += SCAN_WAVES) {
      const f32x4 acc = gemm_f32_tile<D>(sS, LDS_, sC, LDC, r0, 16 * et, lane, zero4());
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t e = (size_t)(r0 + 4 * (lane >> 4) + q) * E + 16 * et + (lane & 15);
        const float gA = Y.G[e], gB = X.G[e];
        X.G[e] = gA;
        Y.G[e] = al2 * gA + gB + al * acc[q];
      }
    }
    // h rows: a^2 h_A + h_B + a S_B m_A
    for (int r = gt; r < SCAN_RB; r += SCAN_THR) {
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc += sS[(r0 + r) * LDS_ + c] * sm[c];
      const float hA = Y.h[r0 + r], hB = X.h[r0 + r];
      X.h[r0 + r] = hA;
      Y.h[r0 + r] = al2 * hA + hB + al * acc;
    }
    // S and C rows: a X_A + X_B (S_B and C_A from LDS)
    for (int t = gt; t < SCAN_RB * D / 4; t += SCAN_THR) {
      const int r = (4 * t) / D, c = (4 * t) % D;
      const size_t e = (size_t)r0 * D / 4 + t;
      const f32x4 sA = reinterpret_cast<const f32x4*>(Y.S)[e];
      const f32x4 sB = *reinterpret_cast<const f32x4*>(sS + (r0 + r) * LDS_ + c);
      reinterpret_cast<f32x4*>(X.S)[e] = sA;
      reinterpret_cast<f32x4*>(Y.S)[e] = sA * al + sB;
    }
    for (int t = gt; t < SCAN_RB * E / 4; t += SCAN_THR) {
      const int r = (4 * t) / E, c = (4 * t) % E;
      const size_t e = (size_t)r0 * E / 4 + t;
      const f32x4 cA = *reinterpret_cast<const f32x4*>(sC + (r0 + r) * LDC + c);
      const f32x4 cB = reinterpret_cast<const f32x4*>(X.C)[e];
      reinterpret_cast<f32x4*>(X.C)[e] = cA;
      reinterpret_cast<f32x4*>(Y.C)[e] = cA * al + cB;
    }
  }
  for (int t = tid; t < D; t += DOWN_THR) {
    const float mA = sm[t], mB = X.m[t];
    X.m[t] = mA;
    Y.m[t] = al * mA + mB;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, size_t count) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += stride) p[t] = 0.f;
}

// ---- runs ----------------------------------------------------------------------

struct RunArgs {
  float *S, *C, *m, *G, *h;        // segments [units, n, ...]
  float *aS, *aC, *am, *aG, *ah;   // run totals / exclusive run prefixes [units, runs, ...]
  float *tS, *tC, *tm, *tG, *th;   // inclusive totals [units, ...], each may be nullptr
  float *oS, *oC, *om, *oG, *oh;   // exclusive prefixes [units, n, ...] (side-by-side rescan
                                   // with its prefixes out of place), else nullptr
  const float* gamma;
  int H, n, R, runs, chunk, units;
  int from_prefix;                 // rescan starts from a*[run] (else from the identity)
};

// Row tiles (16 rows) per workgroup of steps 1 and 3: one up to d = 64, two at
// d = 128.  Each step of a run is a chain (this segment's products, then its
// prefix out, then the running state in): fewer rows per workgroup shortens
// every link and puts more workgroups on the walk, at the cost of every
// workgroup reading the whole running C each step (measured: 16 segments per
// head at d = 64, 54 -> 28 us with one row tile instead of four; at d = 128 two
// row tiles beat one and four).
template <int D>
struct RunRT {
  static constexpr int value = D <= 64 ? 1 : 2;
};

// Steps 1 (REDUCE) and 3: one workgroup per (unit, run, block of 16 RT rows),
// E/16 waves; wave w owns column block w of C and G.  blockIdx.x is laid out
// so that the row blocks of one (unit, run) share blockIdx.x mod 8 and so run
// on one XCD, where the C and m they all read stay in one L2.  With PO (step 3
// out of place) every prefix goes to the arrays of RunArgs::oS.. and the
// segments are only read, so each workgroup also writes its rows of C's and
// m's prefixes (it carries the whole running C and m) and step 4 is not
// needed.
template <int D, int E, bool REDUCE, bool PO>
__global__ __launch_bounds__(64 * (E / 16)) void run_rows_kernel(RunArgs a) {
  static_assert(!(REDUCE && PO), "the reduce step writes run totals only");
  constexpr int RT = RunRT<D>::value, RB = 16 * RT;
  constexpr int NW = E / 16, NT = 64 * NW, DT = D / 16, NRB = D / RB, LS = D + 4;
  constexpr int SV = RB * D / 4;            // f32x4 in RB rows of S
  constexpr int SPT = (SV + NT - 1) / NT;
  constexpr int PH = NT / RB;               // lanes per row of the S m product
  static_assert(PH >= 1 && (PH & (PH - 1)) == 0 && PH <= 64, "rows per workgroup");
  // one workgroup per run: nobody else reads the run's C and m, so step 3
  // writes their prefixes too and step 4 is not needed
  constexpr bool CM = !REDUCE && NRB == 1;
  __shared__ __attribute__((aligned(16))) float sS[RB * LS];
  __shared__ float sm[2][D];

  const int bid = blockIdx.x, xcd = bid & 7, qb = bid >> 3;
  const int grp = xcd + 8 * (qb / NRB), rb = qb % NRB;
  if (grp >= a.units * a.runs) return;
  const int unit = grp / a.runs, run = grp % a.runs;
  const int k0 = run * a.R;
  const int len = (a.n - k0) < a.R ? (a.n - k0) : a.R;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg4 = lane >> 4;
  const int r0 = RB * rb;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), a.chunk), al2 = al * al;

  // running state: C column block (rows 16 t + 4 lg4 + j), G row tiles x
  // column block (tile q: rows r0 + 16 q + 4 lg4 + j), S rows (f32x4 e = tid +
  // NT i: row e / (D/4), columns 4 (e % (D/4))), h row hrow in the first of
  // the row's PH lanes (hown); m in LDS
  f32x4 Cb[DT], Gb[RT], Sb[SPT];
  float hb = 0.f;
  const int hrow = tid / PH, hpart = tid % PH;
  const bool hown = hpart == 0;
  const bool pre = !REDUCE && a.from_prefix;
  const size_t pr = (size_t)unit * a.runs + run;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Cb[t][j] = pre ? a.aC[pr * D * E + (size_t)(16 * t + 4 * lg4 + j) * E + 16 * w + lr] : 0.f;
#pragma unroll
  for (int q = 0; q < RT; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Gb[q][j] = pre ? a.aG[pr * D * E + (size_t)(r0 + 16 * q + 4 * lg4 + j) * E + 16 * w + lr] : 0.f;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int e = tid + NT * i;
    Sb[i] = zero4();
    if (pre && e < SV)
      Sb[i] = reinterpret_cast<const f32x4*>(a.aS + pr * D * D + (size_t)r0 * D)[e];
  }
  if (pre && hown) hb = a.ah[pr * D + r0 + hrow];
  for (int t = tid; t < D; t += NT) sm[0][t] = pre ? a.am[pr * D + t] : 0.f;

  // loads of one segment
  f32x4 xC[DT], xG[RT], xS[SPT];
  float xh = 0.f, xm = 0.f;
  auto load = [&](int k) {
    const size_t sl = (size_t)unit * a.n + k0 + k;
    const float* pC = a.C + sl * D * E;
    const float* pG = a.G + sl * D * E;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xC[t][j] = pC[(16 * t + 4 * lg4 + j) * E + 16 * w + lr];
#pragma unroll
    for (int q = 0; q < RT; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) xG[q][j] = pG[(r0 + 16 * q + 4 * lg4 + j) * E + 16 * w + lr];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = tid + NT * i;
      xS[i] = e < SV ? reinterpret_cast<const f32x4*>(a.S + sl * D * D + (size_t)r0 * D)[e] : zero4();
    }
    xh = hown ? a.h[sl * D + r0 + hrow] : 0.f;
    xm = tid < D ? a.m[sl * D + tid] : 0.f;
  };

  // The running state after a run's last segment is written only as a total
  // (step 1's run totals, or the last run's inclusive total when asked for);
  // otherwise that segment is neither loaded nor combined: the walk's last
  // step only writes its prefix.
  const bool keep_last =
      REDUCE || (run == a.runs - 1 && (a.tS || a.tC || a.tm || a.tG || a.th));
  const int walk = (keep_last || len == 0) ? len : len - 1;
  int cur = 0;
  if (walk > 0) load(0);
  __syncthreads();
  for (int k = 0; k < len; ++k) {
    const bool comb = k < walk;   // uniform
    // S rows of segment k to LDS: the A operand of S_B C_A and S_B m_A
    if (comb) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int e = tid + NT * i;
        if (e < SV) *reinterpret_cast<f32x4*>(sS + (e / (D / 4)) * LS + 4 * (e % (D / 4))) = xS[i];
      }
    }
    __syncthreads();
    if (!REDUCE) {
      // the segment's own rows become its exclusive prefix, the running state
      // before this segment (in place, each thread overwrites the elements it
      // read a step earlier)
      const size_t sl = (size_t)unit * a.n + k0 + k;
      float* const dG = PO ? a.oG : a.G;
      float* const dS = PO ? a.oS : a.S;
      float* const dh = PO ? a.oh : a.h;
#pragma unroll
      for (int q = 0; q < RT; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dG[sl * D * E + (size_t)(r0 + 16 * q + 4 * lg4 + j) * E + 16 * w + lr] = Gb[q][j];
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int e = tid + NT * i;
        if (e < SV) reinterpret_cast<f32x4*>(dS + sl * D * D + (size_t)r0 * D)[e] = Sb[i];
      }
      if (hown) dh[sl * D + r0 + hrow] = hb;
      if constexpr (PO) {
        // this workgroup's rows of C's and m's prefixes
#pragma unroll
        for (int t = 0; t < DT; ++t)
          if (16 * t >= r0 && 16 * t < r0 + RB) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              a.oC[sl * D * E + (size_t)(16 * t + 4 * lg4 + j) * E + 16 * w + lr] = Cb[t][j];
          }
        if (tid < RB) a.om[sl * D + r0 + tid] = sm[cur][r0 + tid];
      } else if constexpr (CM) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a.C[sl * D * E + (size_t)(16 * t + 4 * lg4 + j) * E + 16 * w + lr] = Cb[t][j];
        if (tid < D) a.m[sl * D + tid] = sm[cur][tid];
      }
    }
    if (!comb) break;
    // the segment's S, G and h enter the running state now, its C after the
    // product, which reads the running C before this segment
#pragma unroll
    for (int i = 0; i < SPT; ++i) Sb[i] = Sb[i] * al + xS[i];
#pragma unroll
    for (int q = 0; q < RT; ++q) Gb[q] = Gb[q] * al2 + xG[q];
    hb = al2 * hb + xh;
    const float cm = xm;
    f32x4 cS[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) cS[t] = xC[t];
    if (k + 1 < walk) load(k + 1);

    // G rows += a S_B C_A (C_A = running C, before this segment); RT
    // independent accumulator chains (two when RT = 1)
    f32x4 acc[RT], acc1 = zero4();
#pragma unroll
    for (int q = 0; q < RT; ++q) acc[q] = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) {
      const float bk = Frag<float>::acc_b(Cb, kk);
#pragma unroll
      for (int q = 0; q < RT; ++q) {
        const float ak = sS[(16 * q + lr) * LS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)];
        if (RT == 1 && (kk & 1)) acc1 = MM<float>::mma(ak, bk, acc1);
        else acc[q] = MM<float>::mma(ak, bk, acc[q]);
      }
    }
    if (RT == 1) acc[0] += acc1;
    // h rows += a S_B m_A: PH lanes per row, D / PH products each
    float hm = 0.f;
#pragma unroll
    for (int c = hpart; c < D; c += PH) hm += sS[hrow * LS + c] * sm[cur][c];
#pragma unroll
    for (int off = 1; off < PH; off *= 2) hm += __shfl_xor(hm, off, 64);

#pragma unroll
    for (int q = 0; q < RT; ++q) Gb[q] = Gb[q] + acc[q] * al;
    hb = hb + al * hm;
#pragma unroll
    for (int t = 0; t < DT; ++t) Cb[t] = Cb[t] * al + cS[t];
    if (tid < D) sm[cur ^ 1][tid] = al * sm[cur][tid] + cm;
    cur ^= 1;
    __syncthreads();
  }

  // run total (step 1) or, for the last run, the inclusive total (step 3)
  float *oS = nullptr, *oC = nullptr, *om = nullptr, *oG = nullptr, *oh = nullptr;
  if (REDUCE) {
    oS = a.aS + pr * D * D; oC = a.aC + pr * D * E; om = a.am + pr * D;
    oG = a.aG + pr * D * E; oh = a.ah + pr * D;
  } else if (run == a.runs - 1) {
    const size_t u = unit;
    if (a.tS) oS = a.tS + u * D * D;
    if (a.tC) oC = a.tC + u * D * E;
    if (a.tm) om = a.tm + u * D;
    if (a.tG) oG = a.tG + u * D * E;
    if (a.th) oh = a.th + u * D;
  }
  if (oS) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = tid + NT * i;
      if (e < SV) reinterpret_cast<f32x4*>(oS + (size_t)r0 * D)[e] = Sb[i];
    }
  }
  if (oG) {
#pragma unroll
    for (int q = 0; q < RT; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) oG[(size_t)(r0 + 16 * q + 4 * lg4 + j) * E + 16 * w + lr] = Gb[q][j];
  }
  if (oh && hown) oh[r0 + hrow] = hb;
  if (rb == 0) {
    if (oC) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) oC[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * w + lr] = Cb[t][j];
    }
    if (om && tid < D) om[tid] = sm[cur][tid];
  }
}

// Step 4: C and m (and, after the side-by-side rescan, S) of every segment
// become their exclusive prefixes: elementwise decayed running sums.  One
// thread per f32x4 of (S | C | m) per (unit, run); blockIdx.x = (unit * runs +
// run) * NBLK + block.
template <int D, int E, bool WITH_S>
__global__ __launch_bounds__(256) void run_cm_kernel(RunArgs a) {
  constexpr int VS = WITH_S ? D * D / 4 : 0, VC = D * E / 4, VM = D / 4;
  constexpr int NBLK = (VS + VC + VM + 255) / 256;
  const int grp = blockIdx.x / NBLK;
  const int e = (blockIdx.x % NBLK) * 256 + threadIdx.x;
  if (e >= VS + VC + VM) return;
  const int unit = grp / a.runs, run = grp % a.runs;
  const int k0 = run * a.R;
  const int len = (a.n - k0) < a.R ? (a.n - k0) : a.R;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), a.chunk);
  const int fld = e < VS ? 0 : e < VS + VC ? 1 : 2;   // S, C, m
  const int o = fld == 0 ? e : fld == 1 ? e - VS : e - VS - VC;
  const size_t per = fld == 0 ? (size_t)D * D : fld == 1 ? (size_t)D * E : (size_t)D;
  f32x4* base = reinterpret_cast<f32x4*>(fld == 0 ? a.S : fld == 1 ? a.C : a.m);
  f32x4 p = zero4();
  if (a.from_prefix) {
    const float* pa = fld == 0 ? a.aS : fld == 1 ? a.aC : a.am;
    p = reinterpret_cast<const f32x4*>(pa + ((size_t)unit * a.runs + run) * per)[o];
  }
  constexpr int BATCH = 8;
  for (int k = 0; k < len; k += BATCH) {
    f32x4 x[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (k + b < len) x[b] = base[((size_t)unit * a.n + k0 + k + b) * (per / 4) + o];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (k + b < len) {
        base[((size_t)unit * a.n + k0 + k + b) * (per / 4) + o] = p;
        p = p * al + x[b];
      }
  }
  if (run == a.runs - 1) {
    float* t = fld == 0 ? a.tS : fld == 1 ? a.tC : a.tm;
    if (t) reinterpret_cast<f32x4*>(t + (size_t)unit * per)[o] = p;
  }
}

// Step 3 with a run's segments side by side (runs of at most 16 segments).
// Over a run the exclusive prefixes obey
//   C_P(k+1) = a C_P(k) + C_k      (m and S likewise),
//   G_P(k+1) = a^2 G_P(k) + X_k,   X_k = G_k + a S_k C_P(k),
//   h_P(k+1) = a^2 h_P(k) + y_k,   y_k = h_k + a S_k m_P(k),
// so the products S_k C_P(k) and S_k m_P(k) need only the elementwise
// prefixes of C and m and do not depend on one another: every segment's
// product runs at once instead of one link of a chain per segment.  One
// workgroup per (unit, run, 16-row block, 16-column block) and one wave per
// segment: the waves load their segments together, the C column block's and
// m's prefixes are formed across the slots in LDS, each wave forms its X
// block (and y rows in the column block 0 workgroups) on fp32 MFMA, and the G
// (h) prefixes are formed across the slots and written in place.  S, C and m
// are only read here (every workgroup of the run reads them), so in place
// run_cm_kernel<.., true> rewrites them afterwards.  With PO every prefix
// goes to arrays of their own instead, the segments are only read, and this
// launch is the whole rescan: the workgroup of (row block rb, column block
// cb) writes that block of G's and C's prefixes (its rows of the column block
// it forms anyway), S's blocks (rb, cb + k E/16) (its slot's blocks staged in
// LDS once the products are done) and, in the column block 0 workgroups, its
// rows of h's and m's.  The workgroups of one (unit, run) share blockIdx.x
// mod 8, i.e. one XCD and its L2.
template <int D, int E, int RM, bool PO>
// (at most 64 VGPRs: two 16-wave workgroups per CU)
__global__ __launch_bounds__(64 * RM) __attribute__((amdgpu_waves_per_eu(8))) void run_flat_kernel(RunArgs a) {
  static_assert(!PO || RM == 16, "prefixes out of place: 16 waves");
  constexpr int NT = 64 * RM, DT = D / 16, NCB = E / 16, NP = (D / 16) * NCB;
  constexpr int LC = D + 4;   // floats per column of a slot's C block
  constexpr int NSB = (DT + NCB - 1) / NCB;   // (PO) S blocks per workgroup, at most 2
  constexpr int SO = 272;     // (PO) the slot's S blocks, after X and y
  constexpr int SLOT = PO && 16 * LC < SO + 256 * NSB ? SO + 256 * NSB : 16 * LC;
  static_assert(!PO || 256 + 256 * NSB + 16 <= NT, "threads for the S, G and h walks");
  // slot w: the C block's prefix, then (once wave w has read it) X's block in
  // its first 256 floats and y in the next 16; only wave w touches its slot
  // between the barriers
  __shared__ __attribute__((aligned(16))) float sC[RM][SLOT];
  __shared__ float sm[RM][D];

  const int bid = blockIdx.x, xcd = bid & 7, qb = bid >> 3;
  const int grp = xcd + 8 * (qb / NP), part = qb % NP;
  if (grp >= a.units * a.runs) return;
  const int rb = part / NCB, cb = part % NCB;
  const int unit = grp / a.runs, run = grp % a.runs;
  const int k0 = run * a.R;
  const int len = (a.n - k0) < a.R ? (a.n - k0) : a.R;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg4 = lane >> 4;
  const int r0 = 16 * rb, c0 = 16 * cb;
  const bool hw = cb == 0;    // this workgroup also carries h, which needs m
  const bool live = w < len;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), a.chunk), al2 = al * al;
  const size_t pr = (size_t)unit * a.runs + run;
  const size_t sl = (size_t)unit * a.n + k0 + w;
  const bool last = run == a.runs - 1;

  // 1. this wave's segment: C column block (rows 16 t + 4 lg4 + j, column
  // c0 + lr), S rows r0 + lr as the A operand (columns 16 c + 4 lg4 .. + 3),
  // G block (rows r0 + 4 lg4 + j, column c0 + lr), h row r0 + lr, m
  f32x4 xC[DT], xS[DT], xG = zero4();
  float xh = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t) xC[t] = xS[t] = zero4();
  if (live) {
    const float* pC = a.C + sl * D * E;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xC[t][j] = pC[(size_t)(16 * t + 4 * lg4 + j) * E + c0 + lr];
    const f32x4* pS = reinterpret_cast<const f32x4*>(a.S + sl * D * D + (size_t)(r0 + lr) * D);
#pragma unroll
    for (int t = 0; t < DT; ++t) xS[t] = pS[4 * t + lg4];
    const float* pG = a.G + sl * D * E;
#pragma unroll
    for (int j = 0; j < 4; ++j) xG[j] = pG[(size_t)(r0 + 4 * lg4 + j) * E + c0 + lr];
    if (hw) {
      xh = a.h[sl * D + r0 + lr];
      for (int t = lane; t < D; t += 64) sm[w][t] = a.m[sl * D + t];
    }
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
    *reinterpret_cast<f32x4*>(&sC[w][lr * LC + 16 * t + 4 * lg4]) = xC[t];
  __syncthreads();

  // 2. exclusive prefixes of the C column block and of m across the run
  for (int e = tid; e < 16 * D; e += NT) {
    const int row = e >> 4, col = e & 15;
    float p = a.from_prefix ? a.aC[pr * D * E + (size_t)row * E + c0 + col] : 0.f;
    // every slot is read and written (slots past the run's end are never
    // used): no branch, so the reads issue together
    float v[RM];
#pragma unroll
    for (int s = 0; s < RM; ++s) v[s] = sC[s][col * LC + row];
#pragma unroll
    for (int s = 0; s < RM; ++s) {
      sC[s][col * LC + row] = p;
      const float nx = p * al + v[s];
      p = !PO || s < len ? nx : p;   // (PO) the run's total stops at its end
    }
    if (PO && last && a.tC && (row >> 4) == rb) a.tC[(size_t)unit * D * E + (size_t)row * E + c0 + col] = p;
  }
  if (hw) {
    for (int e = tid; e < D; e += NT) {
      float p = a.from_prefix ? a.am[pr * D + e] : 0.f;
      const bool mine = PO && (e >> 4) == rb;
      float v[RM];
#pragma unroll
      for (int s = 0; s < RM; ++s) v[s] = sm[s][e];
#pragma unroll
      for (int s = 0; s < RM; ++s) {
        sm[s][e] = p;
        if (mine && s < len) a.om[((size_t)unit * a.n + k0 + s) * D + e] = p;
        const float nx = p * al + v[s];
        p = !PO || s < len ? nx : p;
      }
      if (mine && last && a.tm) a.tm[(size_t)unit * D + e] = p;
    }
  }
  __syncthreads();

  // 3. X = G_k + a S_k C_P(k) for the block, y = h_k + a S_k m_P(k)
  if (live) {
    f32x4 cp[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) cp[t] = *reinterpret_cast<const f32x4*>(&sC[w][lr * LC + 16 * t + 4 * lg4]);
    if constexpr (PO) {
      // this slot's C prefix, rows r0 + 4 lg4 + j of column c0 + lr
      f32x4 cb4 = cp[0];
#pragma unroll
      for (int t = 1; t < DT; ++t)
        if (t == rb) cb4 = cp[t];
      float* pc = a.oC + sl * D * E + c0 + lr;
#pragma unroll
      for (int j = 0; j < 4; ++j) pc[(size_t)(r0 + 4 * lg4 + j) * E] = cb4[j];
    }
    f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) {
      const float ak = xS[kk >> 2][kk & 3], bk = Frag<float>::acc_b(cp, kk);
      if (kk & 1) acc1 = MM<float>::mma(ak, bk, acc1);
      else acc0 = MM<float>::mma(ak, bk, acc0);
    }
    *reinterpret_cast<f32x4*>(&sC[w][4 * lane]) = xG + (acc0 + acc1) * al;
    if (hw) {
      float hp = 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) hp += xS[t][i] * sm[w][16 * t + 4 * lg4 + i];
      hp += __shfl_xor(hp, 16, 64);
      hp += __shfl_xor(hp, 32, 64);
      if (lg4 == 0) sC[w][256 + lr] = xh + al * hp;
    }
  }
  __syncthreads();
  if constexpr (PO) {
    // every wave has read its C prefix: the slot's S blocks (rows r0 + lr,
    // columns 16 sb + 4 lg4 + j, sb = cb + NCB i) go after X and y
    if (live) {
#pragma unroll
      for (int i = 0; i < NSB; ++i) {
        const int sbk = cb + NCB * i;
        f32x4 sv = xS[0];
#pragma unroll
        for (int t = 1; t < DT; ++t)
          if (t == sbk) sv = xS[t];
        if (sbk < DT) *reinterpret_cast<f32x4*>(&sC[w][SO + 256 * i + 16 * lr + 4 * lg4]) = sv;
      }
    }
    __syncthreads();
    // exclusive prefixes of the S blocks across the run, on threads 256 ..
    // 256 + 256 NSB - 1 (those of G on 0..255 and of h after the S threads
    // below, at the same time)
    const int se = tid - 256, sbk = cb + NCB * (se >> 8);
    if (se >= 0 && se < 256 * NSB && sbk < DT) {
      const int row = (se & 255) >> 4, col = se & 15;
      const size_t so = (size_t)(r0 + row) * D + 16 * sbk + col;
      float p = a.from_prefix ? a.aS[pr * D * D + so] : 0.f;
      float v[RM], o[RM];
#pragma unroll
      for (int s = 0; s < RM; ++s) v[s] = sC[s][SO + se];
#pragma unroll
      for (int s = 0; s < RM; ++s) {
        o[s] = p;
        if (s < len) p = p * al + v[s];
      }
      float* pS = a.oS + ((size_t)unit * a.n + k0) * D * D + so;
#pragma unroll
      for (int s = 0; s < RM; ++s)
        if (s < len) pS[(size_t)s * D * D] = o[s];
      if (last && a.tS) a.tS[(size_t)unit * D * D + so] = p;
    }
  }

  // 4. exclusive prefixes of the G block and of h across the run, in place;
  // the last run's inclusive totals
  for (int e = tid; e < 256; e += NT) {
    const int row = e >> 4, col = e & 15;
    const int li = 4 * (16 * (row >> 2) + col) + (row & 3);   // lane 16 (row/4) + col, element row % 4
    const size_t go = (size_t)(r0 + row) * E + c0 + col;
    float p = a.from_prefix ? a.aG[pr * D * E + go] : 0.f;
    float v[RM], o[RM];
#pragma unroll
    for (int s = 0; s < RM; ++s) v[s] = sC[s][li];
#pragma unroll
    for (int s = 0; s < RM; ++s) {
      o[s] = p;
      if (s < len) p = p * al2 + v[s];
    }
    float* pG = (PO ? a.oG : a.G) + ((size_t)unit * a.n + k0) * D * E + go;
#pragma unroll
    for (int s = 0; s < RM; ++s)
      if (s < len) pG[(size_t)s * D * E] = o[s];
    if (last && a.tG) a.tG[(size_t)unit * D * E + go] = p;
  }
  const int ht = PO ? tid - (256 + 256 * NSB) : tid;
  if (hw && ht >= 0 && ht < 16) {
    float p = a.from_prefix ? a.ah[pr * D + r0 + ht] : 0.f;
    float v[RM], o[RM];
#pragma unroll
    for (int s = 0; s < RM; ++s) v[s] = sC[s][256 + ht];
#pragma unroll
    for (int s = 0; s < RM; ++s) {
      o[s] = p;
      if (s < len) p = p * al2 + v[s];
    }
    float* ph = (PO ? a.oh : a.h) + ((size_t)unit * a.n + k0) * D + r0 + ht;
#pragma unroll
    for (int s = 0; s < RM; ++s)
      if (s < len) ph[(size_t)s * D] = o[s];
    if (last && a.th) a.th[(size_t)unit * D + r0 + ht] = p;
  }
}

int scan_run_length(int n) {
  if (n <= 16) return n > 0 ? n : 1;
  int r = 1;
  while (r * r < n) r *= 2;
  return r;
}


size_t scan_workspace_floats(int64_t units, int n, int d, int dv) {
  const int R = scan_run_length(n);
  const int runs = (n + R - 1) / R;
  if (runs <= 1) return 0;
  int N = 1;
  while (N < runs) N *= 2;
  const size_t per = (size_t)d * d + 2 * (size_t)d * dv + 2 * (size_t)d;
  return (size_t)units * (size_t)N * per;   // run totals, then the tree's padding slots
}

size_t scan_runs_workspace_floats(int64_t units, int n, int d, int dv) {
  const int R = scan_run_length(n);
  const int runs = (n + R - 1) / R;
  if (runs <= 1) return 0;
  int N = 1;
  while (N < runs) N *= 2;
  const size_t per = (size_t)d * d + 2 * (size_t)d * dv + 2 * (size_t)d;
  return (size_t)units * (size_t)(N - runs) * per;   // the tree's padding slots
}

template <int D, int E>
static hipError_t run_scan(const ScanPlan& p, hipStream_t s) {
  constexpr int NRB = D / 16, VEC = (D * D + 2 * D * E + 2 * D) / 4;
  constexpr int NRR = D / (16 * RunRT<D>::value);   // row blocks of the run kernels
  const int units = p.units;
  if (p.oS && (p.rS || !p.oC || !p.om || !p.oG || !p.oh)) return hipErrorInvalidValue;
  RunArgs r;
  r.S = p.S; r.C = p.C; r.m = p.m; r.G = p.G; r.h = p.h;
  r.tS = p.tS; r.tC = p.tC; r.tm = p.tm; r.tG = p.tG; r.th = p.th;
  r.oS = p.oS; r.oC = p.oC; r.om = p.om; r.oG = p.oG; r.oh = p.oh;
  r.gamma = p.gamma; r.H = p.H; r.n = p.n; r.chunk = p.chunk; r.units = units;
  r.R = scan_run_length(p.n);
  r.runs = (p.n + r.R - 1) / r.R;
  r.from_prefix = r.runs > 1;
  const size_t cnt = (size_t)units * r.runs;
  // run prefixes only: the run totals are reduced straight into the output
  // arrays and scanned there; the segments are only read
  const bool runs_only = p.rS != nullptr;
  r.aS = r.aC = r.am = r.aG = r.ah = nullptr;
  if (runs_only) {
    r.aS = p.rS; r.aC = p.rC; r.am = p.rm; r.aG = p.rG; r.ah = p.rh;
    if (r.runs == 1) {   // one run: its exclusive prefix is the identity
      float* const outs[5] = {p.rS, p.rC, p.rm, p.rG, p.rh};
      const size_t per[5] = {(size_t)D * D, (size_t)D * E, (size_t)D, (size_t)D * E, (size_t)D};
      for (int i = 0; i < 5; ++i) {
        const size_t count = cnt * per[i];
        size_t blocks = (count + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, outs[i], count);
        if (hipError_t e = hipGetLastError()) return e;
      }
      return hipSuccess;
    }
  } else if (r.runs > 1) {
    r.aS = p.ws; r.aC = r.aS + cnt * D * D; r.am = r.aC + cnt * D * E; r.aG = r.am + cnt * D;
    r.ah = r.aG + cnt * D * E;
  }
  const unsigned groups8 = (unsigned)((cnt + 7) / 8 * 8);
  if (r.runs > 1) {
    hipLaunchKernelGGL((run_rows_kernel<D, E, true, false>), dim3(groups8 * NRR), dim3(64 * (E / 16)), 0, s, r);
    if (hipError_t e = hipGetLastError()) return e;
    // exclusive Blelloch scan of the run totals; padding slots follow them
    ScanArgs a;
    a.S = r.aS; a.C = r.aC; a.m = r.am; a.G = r.aG; a.h = r.ah;
    a.n = r.runs;
    a.N = 1;
    while (a.N < a.n) a.N *= 2;
    const size_t pad = (size_t)units * (a.N - a.n);
    a.wS = runs_only ? p.ws : r.ah + cnt * D;
    a.wC = a.wS + pad * D * D; a.wm = a.wC + pad * D * E;
    a.wG = a.wm + pad * D; a.wh = a.wG + pad * D * E;
    a.gamma = p.gamma; a.H = p.H; a.chunk = p.chunk; a.seg = r.R; a.nseg = p.n;
    a.d = D; a.dv = E;
    if (pad > 0) {
      const size_t count = pad * (size_t)(4 * VEC);
      size_t blocks = (count + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.wS, count);
      if (hipError_t e = hipGetLastError()) return e;
    }
    // up-sweep below the root, the top level, then the down-sweep
    for (int step = 1; step < a.N / 2; step *= 2) {
      a.step = step;
      hipLaunchKernelGGL((scan_combine_kernel<D, E>), dim3(a.N / (2 * step) * NRB, units),
                         dim3(SCAN_THR), 0, s, a);
      if (hipError_t e = hipGetLastError()) return e;
    }
    constexpr int TOP_PARTS = (VEC + 1023) / 1024;
    hipLaunchKernelGGL(scan_top_kernel, dim3(units * TOP_PARTS), dim3(256), 0, s, a, TOP_PARTS);
    if (hipError_t e = hipGetLastError()) return e;
    for (int step = a.N / 4; step >= 1; step /= 2) {
      a.step = step;
      hipLaunchKernelGGL((scan_down_kernel<D, E>), dim3(a.N / (2 * step), units),
                         dim3(DownThreads<D>::value), 0, s, a);
      if (hipError_t e = hipGetLastError()) return e;
    }
  }
  if (runs_only) return hipSuccess;
  if (r.oS) {
    // out of place: the side-by-side rescan (d <= 64, runs of at most 16
    // segments, as in place) or the walk, each writing every prefix itself
    if constexpr (D <= 64) {
      if (r.R <= 16) {
        hipLaunchKernelGGL((run_flat_kernel<D, E, 16, true>), dim3(groups8 * (D / 16) * (E / 16)), dim3(1024),
                           0, s, r);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((run_rows_kernel<D, E, false, true>), dim3(groups8 * NRR), dim3(64 * (E / 16)), 0, s, r);
    return hipGetLastError();
  }
  if constexpr (D <= 64) {
    if (r.R <= 16) {
      // runs of at most 16 segments: the segments of a run side by side, then S,
      // C and m elementwise (measured at d = 64 with 16 segments per head: 25 ->
      // 17 us and 32 -> 25 us; at d = 128, 4 segments per head, the walk below
      // stays faster: 37 against 56 us)
      constexpr int NP = (D / 16) * (E / 16);
      if (r.R <= 4)
        hipLaunchKernelGGL((run_flat_kernel<D, E, 4, false>), dim3(groups8 * NP), dim3(256), 0, s, r);
      else
        hipLaunchKernelGGL((run_flat_kernel<D, E, 16, false>), dim3(groups8 * NP), dim3(1024), 0, s, r);
      if (hipError_t e = hipGetLastError()) return e;
      constexpr int VSCM = (D * D + D * E + D) / 4;
      hipLaunchKernelGGL((run_cm_kernel<D, E, true>), dim3((unsigned)(cnt * ((VSCM + 255) / 256))),
                         dim3(256), 0, s, r);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((run_rows_kernel<D, E, false, false>), dim3(groups8 * NRR), dim3(64 * (E / 16)), 0, s, r);
  if (hipError_t e = hipGetLastError()) return e;
  if (NRR == 1) return hipSuccess;   // the rescan wrote C and m
  constexpr int VCM = (D * E + D) / 4;
  hipLaunchKernelGGL((run_cm_kernel<D, E, false>), dim3((unsigned)(cnt * ((VCM + 255) / 256))), dim3(256),
                     0, s, r);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanPlan& p, hipStream_t s) {
#define HLA_CASE(D, E) \
  if (p.d == D && p.dv == E) return run_scan<D, E>(p, s);
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hla
