// C ABI of the masked second-order HLA forward (declarations and the
// contract of every entry point are in include/hla.h).
//
// This layer validates every argument on the host, sizes workspaces and
// enqueues the kernels; it owns no memory and keeps no state between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "hla.h"
#include "hla_internal.h"

namespace {

using hla::ChunkArgs;
using hla::DecodeArgs;

constexpr int64_t kMaxGrid = 2147483647;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (both non-empty)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t dtype_size(int dt) { return dt == HLA_BF16 ? 2 : 4; }

bool head_ok(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }

// Shape/dtype validation shared by the forward entry points.
hla_status check_problem(const hla_problem* p) {
  if (!p) return HLA_ERR_NULL_POINTER;
  if (p->B < 0 || p->H < 0 || p->T < 0 || p->d <= 0 || p->dv <= 0) return HLA_ERR_BAD_SHAPE;
  if (p->chunk <= 0) return HLA_ERR_BAD_SHAPE;
  if (p->T % p->chunk != 0) return HLA_ERR_BAD_SHAPE;
  if (p->in_dtype != HLA_F32 && p->in_dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (p->normalize != 0 && p->normalize != 1) return HLA_ERR_BAD_VALUE;
  if (!std::isfinite(p->eps)) return HLA_ERR_BAD_VALUE;
  if (!head_ok(p->d) || !head_ok(p->dv)) return HLA_ERR_UNSUPPORTED;
  if (!hla::chunk_shape_supported(p->in_dtype, p->d, p->dv)) return HLA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)p->B * p->H;
  const int64_t n = p->T / p->chunk;
  if (units * n > kMaxGrid) return HLA_ERR_BAD_VALUE;
  if (units > 65535) return HLA_ERR_BAD_VALUE;   // grid.y of the scan levels
  // a segment's rows are addressed with 32-bit byte offsets
  const int64_t row_bytes = (int64_t)(p->d > p->dv ? p->d : p->dv) * (int64_t)dtype_size(p->in_dtype);
  if ((int64_t)p->chunk * row_bytes > 2147483647) return HLA_ERR_BAD_VALUE;
  if (p->gamma && !aligned16(p->gamma)) return HLA_ERR_MISALIGNED;
  return HLA_OK;
}

bool empty_problem(const hla_problem* p) { return p->B == 0 || p->H == 0 || p->T == 0; }

hla_status device_ready() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return HLA_ERR_HIP;
  }
  return HLA_OK;
}

hla_status from_hip(hipError_t e) {
  if (e == hipSuccess) return HLA_OK;
  (void)hipGetLastError();
  return HLA_ERR_HIP;
}

struct Sizes {
  int64_t units, n, N;
  size_t qk_bytes, v_bytes, o_bytes, den_bytes;
  size_t S, C, m;   // floats per summary field
};

Sizes sizes_of(const hla_problem* p) {
  Sizes s;
  s.units = (int64_t)p->B * p->H;
  s.n = p->T / p->chunk;
  s.N = 1;
  while (s.N < s.n) s.N *= 2;
  const size_t tok = (size_t)s.units * (size_t)p->T;
  s.qk_bytes = tok * p->d * dtype_size(p->in_dtype);
  s.v_bytes = tok * p->dv * dtype_size(p->in_dtype);
  s.o_bytes = tok * p->dv * 4;
  s.den_bytes = tok * 4;
  s.S = (size_t)p->d * p->d;
  s.C = (size_t)p->d * p->dv;
  s.m = (size_t)p->d;
  return s;
}

hla_status check_state(const hla_state* st, bool all_required, int64_t count, const Sizes& z,
                       const void* const* inputs, const size_t* in_bytes, int n_inputs) {
  if (!st) return HLA_ERR_NULL_POINTER;
  float* f[5] = {st->S, st->C, st->m, st->G, st->h};
  const size_t per[5] = {z.S, z.C, z.m, z.C, z.m};
  for (int i = 0; i < 5; ++i) {
    if (!f[i]) {
      if (all_required) return HLA_ERR_NULL_POINTER;
      continue;
    }
    if (!aligned16(f[i])) return HLA_ERR_MISALIGNED;
    const size_t bytes = (size_t)count * per[i] * 4;
    for (int j = 0; j < n_inputs; ++j)
      if (overlap(f[i], bytes, inputs[j], in_bytes[j])) return HLA_ERR_ALIASING;
    for (int j = 0; j < i; ++j)
      if (f[j] && overlap(f[i], bytes, f[j], (size_t)count * per[j] * 4)) return HLA_ERR_ALIASING;
  }
  return HLA_OK;
}

hla_status check_qkv(const void* q, const void* k, const void* v) {
  if (!q || !k || !v) return HLA_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return HLA_ERR_MISALIGNED;
  return HLA_OK;
}

ChunkArgs chunk_args(const hla_problem* p, const void* q, const void* k, const void* v,
                     const hla_state* st, float* o, float* den) {
  ChunkArgs a;
  a.q = q; a.k = k; a.v = v;
  a.gamma = p->gamma;
  a.H = p->H; a.T = p->T; a.chunk = p->chunk; a.nspan = p->T / p->chunk;
  a.normalize = p->normalize; a.eps = p->eps;
  a.S = st->S; a.C = st->C; a.m = st->m; a.G = st->G; a.h = st->h;
  a.o = o; a.den = den;
  a.pl = nullptr;
  return a;
}

size_t scan_ws_bytes(const hla_problem* p) {
  const Sizes z = sizes_of(p);
  return hla::scan_workspace_floats(z.units, (int)z.n, p->d, p->dv) * 4;
}

// The exclusive scan of `inout`'s segments, in place; with prefix_out the
// prefixes go there instead and `inout` is only read.
hla_status do_scan(const hla_problem* p, const hla_state* inout, const hla_state* total,
                   void* ws, hipStream_t s, const hla_state* prefix_out = nullptr) {
  const Sizes z = sizes_of(p);
  hla::ScanPlan a;
  a.S = inout->S; a.C = inout->C; a.m = inout->m; a.G = inout->G; a.h = inout->h;
  a.tS = total ? total->S : nullptr; a.tC = total ? total->C : nullptr;
  a.tm = total ? total->m : nullptr; a.tG = total ? total->G : nullptr;
  a.th = total ? total->h : nullptr;
  a.rS = a.rC = a.rm = a.rG = a.rh = nullptr;
  a.ws = static_cast<float*>(ws);
  a.gamma = p->gamma;
  a.units = (int)z.units; a.H = p->H; a.n = (int)z.n; a.chunk = p->chunk;
  a.d = p->d; a.dv = p->dv;
  if (prefix_out) {
    a.oS = prefix_out->S; a.oC = prefix_out->C; a.om = prefix_out->m;
    a.oG = prefix_out->G; a.oh = prefix_out->h;
  }
  return from_hip(hla::launch_scan(a, s));
}

// Consecutive chunks that each workgroup of hla_fwd's summary and output
// kernels walks (a power of two dividing n).  Inside a workgroup the chunk
// summaries of its span are formed and combined in order as its tiles go by
// (the first level of the scan, fused with forming them); the span totals
// then go through hla_scan.  Preferred: the fewest chunks per span that leave
// at most 16 span totals per (b, h) (a single-run scan: one launch), as long
// as that keeps at least 256 workgroups (one per CU with 8-wave kernels, or
// two with 4-wave kernels); otherwise the most chunks per span that keep 256
// workgroups.
int64_t fwd_span_chunks(const hla_problem* p) {
  const Sizes z = sizes_of(p);
  const int64_t row_bytes = (int64_t)(p->d > p->dv ? p->d : p->dv) * (int64_t)dtype_size(p->in_dtype);
  auto fits = [&](int64_t R) {
    return z.n % R == 0 && (int64_t)p->chunk * R * row_bytes <= 2147483647;
  };
  const int64_t want_wg = 256;
  int64_t R1 = 1;
  while (z.n / R1 > 16 && fits(R1 * 2)) R1 *= 2;
  if (z.n / R1 <= 16 && z.units * (z.n / R1) >= want_wg) return R1;
  int64_t R = 1;
  while (fits(R * 2) && z.units * (z.n / (R * 2)) >= want_wg) R *= 2;
  return R;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// One segment's p blocks (64-token tiles of d bf16 rows) stay within the
// 32-bit byte range of the kernels' buffer addressing.
bool plocal_fits(int64_t chunk, int d) { return (chunk + 63) / 64 * 64 * (int64_t)d * 2 <= 2147483647; }

// Bytes of the segment-local p over hla_fwd's spans (0 for shapes without
// the path that uses it).
size_t fwd_span_p_bytes(const hla_problem* p) {
  if (!hla::outp_supported(p->in_dtype, p->d, p->dv)) return 0;
  const int64_t span = (int64_t)p->chunk * fwd_span_chunks(p);
  if (!plocal_fits(span, p->d)) return 0;
  return hla::outp_plocal_bytes(sizes_of(p).units, p->T, (int)span, p->d);
}

// Where hla_fwd keeps what in a workspace of workspace_bytes (byte offsets
// from its start).  The summaries of the spans and the scan's scratch come
// first, in the room of hla_fwd_workspace_bytes(p), which is sized for one
// summary per chunk; then the segment-local p, when the shape has that path
// and the workspace holds it; the exclusive prefixes go out of place (the
// scan then forms them without a separate C, m pass) into the rest of that
// first room when spans of several chunks leave enough of it, else after p
// when the workspace holds them, else the scan runs in place.
struct FwdPlan {
  size_t base;       // hla_fwd_workspace_bytes(p)
  size_t scan_ws;    // the scan's scratch, after the span summaries
  size_t p_off;      // the segment-local p, or 0 (none)
  size_t po_off;     // the out-of-place prefixes, or 0 (scan in place)
  size_t end;        // bytes used
};

FwdPlan fwd_plan(const hla_problem* p, size_t workspace_bytes) {
  FwdPlan f;
  f.base = hla_fwd_workspace_bytes(p);
  hla_problem ps = *p;
  ps.chunk = (int32_t)(p->chunk * fwd_span_chunks(p));
  const Sizes z = sizes_of(&ps);
  const size_t cnt = (size_t)z.units * (size_t)z.n;
  const size_t summ = cnt * (z.S + 2 * z.C + 2 * z.m) * 4;
  f.scan_ws = summ;
  const size_t in_base = summ + scan_ws_bytes(&ps);
  const size_t pb = fwd_span_p_bytes(p);
  f.p_off = 0;
  f.end = f.base;
  if (pb && workspace_bytes >= align256(f.base) + pb) {
    f.p_off = align256(f.base);
    f.end = f.p_off + pb;
  }
  f.po_off = 0;
  if (in_base + summ <= f.base) {
    f.po_off = in_base;
  } else if (workspace_bytes >= align256(f.end) + summ) {
    f.po_off = align256(f.end);
    f.end = f.po_off + summ;
  }
  return f;
}

// The bytes of hla_fwd's fastest plan: the segment-local p where the shape
// has it, the prefixes out of place.
size_t fwd_full_bytes(const hla_problem* p) {
  return fwd_plan(p, ~(size_t)0).end;
}

}  // namespace

extern "C" {

const char* hla_status_string(hla_status s) {
  switch (s) {
    case HLA_OK: return "HLA_OK";
    case HLA_ERR_NULL_POINTER: return "HLA_ERR_NULL_POINTER: a required pointer is NULL";
    case HLA_ERR_BAD_SHAPE: return "HLA_ERR_BAD_SHAPE: negative size, chunk <= 0 or T % chunk != 0";
    case HLA_ERR_BAD_DTYPE: return "HLA_ERR_BAD_DTYPE: in_dtype is not HLA_F32 or HLA_BF16";
    case HLA_ERR_MISALIGNED: return "HLA_ERR_MISALIGNED: a device pointer is not 16-byte aligned";
    case HLA_ERR_UNSUPPORTED: return "HLA_ERR_UNSUPPORTED: head sizes / dtype not built";
    case HLA_ERR_WORKSPACE_TOO_SMALL: return "HLA_ERR_WORKSPACE_TOO_SMALL";
    case HLA_ERR_ALIASING: return "HLA_ERR_ALIASING: an output overlaps an input";
    case HLA_ERR_HIP: return "HLA_ERR_HIP: no usable HIP device or a HIP call failed";
    case HLA_ERR_BAD_VALUE: return "HLA_ERR_BAD_VALUE: eps/normalize invalid or sizes too large";
  }
  return "HLA_ERR_UNKNOWN";
}

const char* hla_version(void) { return "hla-mi355x 0.1 (gfx950)"; }

hla_status hla_fwd_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                   const void* v, const hla_state* out, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {z.qk_bytes, z.qk_bytes, z.v_bytes};
  if (hla_status e = check_state(out, true, z.units * z.n, z, ins, inb, 3)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = device_ready()) return e;
  const ChunkArgs a = chunk_args(p, q, k, v, out, nullptr, nullptr);
  return from_hip(hla::launch_chunk_summaries(p->in_dtype, p->d, p->dv, (int)z.units, a,
                                              static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

size_t hla_scan_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  return scan_ws_bytes(p);
}

hla_status hla_scan(const hla_problem* p, const hla_state* inout, const hla_state* total_out,
                    void* workspace, size_t workspace_bytes, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_state(inout, true, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  if (total_out) {
    const void* ins[5] = {inout->S, inout->C, inout->m, inout->G, inout->h};
    const size_t inb[5] = {z.units * z.n * z.S * 4, z.units * z.n * z.C * 4,
                           z.units * z.n * z.m * 4, z.units * z.n * z.C * 4,
                           z.units * z.n * z.m * 4};
    if (hla_status e = check_state(total_out, false, z.units, z, ins, inb, 5)) return e;
  }
  const size_t need = empty_problem(p) ? 0 : scan_ws_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0) {
    if (!workspace) return HLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  }
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = device_ready()) return e;
  return do_scan(p, inout, total_out, workspace, static_cast<hipStream_t>(stream));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_scan_into(const hla_problem* p, const hla_state* summaries,
                         const hla_state* prefixes_out, const hla_state* total_out, void* workspace,
                         size_t workspace_bytes, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_state(summaries, true, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  const size_t per[5] = {z.S * 4, z.C * 4, z.m * 4, z.C * 4, z.m * 4};
  const void* ins[5] = {summaries->S, summaries->C, summaries->m, summaries->G, summaries->h};
  size_t inb[5];
  for (int j = 0; j < 5; ++j) inb[j] = z.units * z.n * per[j];
  if (hla_status e = check_state(prefixes_out, true, z.units * z.n, z, ins, inb, 5)) return e;
  const void* outs[5] = {prefixes_out->S, prefixes_out->C, prefixes_out->m, prefixes_out->G,
                         prefixes_out->h};
  if (total_out) {
    const void* both[10];
    size_t bb[10];
    for (int j = 0; j < 5; ++j) {
      both[j] = ins[j]; bb[j] = inb[j];
      both[5 + j] = outs[j]; bb[5 + j] = inb[j];
    }
    if (hla_status e = check_state(total_out, false, z.units, z, both, bb, 10)) return e;
  }
  const size_t need = scan_ws_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0) {
    if (!workspace) return HLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
    for (int j = 0; j < 5; ++j)
      if (overlap(workspace, need, ins[j], inb[j]) || overlap(workspace, need, outs[j], inb[j]))
        return HLA_ERR_ALIASING;
  }
  if (hla_status e = device_ready()) return e;
  return do_scan(p, summaries, total_out, workspace, static_cast<hipStream_t>(stream), prefixes_out);
} catch (...) {
  return HLA_ERR_HIP;
}

int32_t hla_scan_run_length(const hla_problem* p) {
  if (check_problem(p) != HLA_OK) return 0;
  return hla::scan_run_length((int)(p->T / p->chunk));
}

int32_t hla_fwd_span_chunks(const hla_problem* p) {
  if (check_problem(p) != HLA_OK) return 0;
  if (empty_problem(p)) return 1;
  return (int32_t)fwd_span_chunks(p);
}

size_t hla_scan_runs_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  const Sizes z = sizes_of(p);
  return hla::scan_runs_workspace_floats(z.units, (int)z.n, p->d, p->dv) * 4;
}

hla_status hla_scan_runs(const hla_problem* p, const hla_state* summaries,
                         const hla_state* run_prefix_out, void* workspace, size_t workspace_bytes,
                         void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  const int64_t R = hla::scan_run_length((int)z.n), runs = (z.n + R - 1) / R;
  if (hla_status e = check_state(summaries, true, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  const void* ins[5] = {summaries->S, summaries->C, summaries->m, summaries->G, summaries->h};
  const size_t inb[5] = {z.units * z.n * z.S * 4, z.units * z.n * z.C * 4, z.units * z.n * z.m * 4,
                         z.units * z.n * z.C * 4, z.units * z.n * z.m * 4};
  if (hla_status e = check_state(run_prefix_out, true, z.units * runs, z, ins, inb, 5)) return e;
  const size_t need = hla_scan_runs_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0) {
    if (!workspace) return HLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
    const size_t pb[5] = {z.units * runs * z.S * 4, z.units * runs * z.C * 4, z.units * runs * z.m * 4,
                          z.units * runs * z.C * 4, z.units * runs * z.m * 4};
    const void* outs[5] = {run_prefix_out->S, run_prefix_out->C, run_prefix_out->m,
                           run_prefix_out->G, run_prefix_out->h};
    for (int j = 0; j < 5; ++j)
      if (overlap(workspace, need, ins[j], inb[j]) || overlap(workspace, need, outs[j], pb[j]))
        return HLA_ERR_ALIASING;
  }
  if (hla_status e = device_ready()) return e;
  hla::ScanPlan a;
  a.S = summaries->S; a.C = summaries->C; a.m = summaries->m; a.G = summaries->G; a.h = summaries->h;
  a.tS = a.tC = a.tm = a.tG = a.th = nullptr;
  a.rS = run_prefix_out->S; a.rC = run_prefix_out->C; a.rm = run_prefix_out->m;
  a.rG = run_prefix_out->G; a.rh = run_prefix_out->h;
  a.ws = static_cast<float*>(workspace);
  a.gamma = p->gamma;
  a.units = (int)z.units; a.H = p->H; a.n = (int)z.n; a.chunk = p->chunk;
  a.d = p->d; a.dv = p->dv;
  return from_hip(hla::launch_scan(a, static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

size_t hla_fwd_output_workspace_bytes(const hla_problem* p) {
  (void)p;
  return 0;
}

hla_status hla_fwd_output(const hla_problem* p, const void* q, const void* k, const void* v,
                          const hla_state* prefixes, float* o, float* den, void* workspace,
                          size_t workspace_bytes, void* stream) try {
  (void)workspace;
  (void)workspace_bytes;
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den))) return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_state(prefixes, true, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  const void* ins[8] = {q, k, v, prefixes->S, prefixes->C, prefixes->m, prefixes->G, prefixes->h};
  const size_t inb[8] = {z.qk_bytes, z.qk_bytes, z.v_bytes,
                         z.units * z.n * z.S * 4, z.units * z.n * z.C * 4, z.units * z.n * z.m * 4,
                         z.units * z.n * z.C * 4, z.units * z.n * z.m * 4};
  for (int j = 0; j < 8; ++j) {
    if (overlap(o, z.o_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, z.den_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, z.o_bytes, den, z.den_bytes)) return HLA_ERR_ALIASING;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = device_ready()) return e;
  const ChunkArgs a = chunk_args(p, q, k, v, prefixes, o, den);
  return from_hip(hla::launch_chunk_outputs(p->in_dtype, p->d, p->dv, (int)z.units, a,
                                            static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

size_t hla_fwd_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  const Sizes z = sizes_of(p);
  const size_t summ = (size_t)z.units * (size_t)z.n * (z.S + 2 * z.C + 2 * z.m) * 4;
  return summ + scan_ws_bytes(p);
}

size_t hla_fwd_p_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  return fwd_full_bytes(p);
}

size_t hla_fwd_p_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  if (!hla::outp_supported(p->in_dtype, p->d, p->dv) || !plocal_fits(p->chunk, p->d)) return 0;
  return hla::outp_plocal_bytes(sizes_of(p).units, p->T, p->chunk, p->d);
}

hla_status hla_fwd_chunk_summaries_p(const hla_problem* p, const void* q, const void* k,
                                     const void* v, const hla_state* out, void* plocal,
                                     void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (!hla::outp_supported(p->in_dtype, p->d, p->dv)) return HLA_ERR_UNSUPPORTED;
  if (!plocal_fits(p->chunk, p->d)) return HLA_ERR_BAD_VALUE;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!plocal) return HLA_ERR_NULL_POINTER;
  if (!aligned16(plocal)) return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  const size_t pb = hla_fwd_p_bytes(p);
  const void* ins[4] = {q, k, v, plocal};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, pb};
  for (int j = 0; j < 3; ++j)
    if (overlap(plocal, pb, ins[j], inb[j])) return HLA_ERR_ALIASING;
  if (hla_status e = check_state(out, true, z.units * z.n, z, ins, inb, 4)) return e;
  if (hla_status e = device_ready()) return e;
  ChunkArgs a = chunk_args(p, q, k, v, out, nullptr, nullptr);
  a.pl = plocal;
  return from_hip(hla::launch_chunk_summaries(p->in_dtype, p->d, p->dv, (int)z.units, a,
                                              static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_fwd_output_from_p(const hla_problem* p, const void* q, const void* v,
                                 const void* plocal, const hla_state* prefixes, float* o,
                                 float* den, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (!hla::outp_supported(p->in_dtype, p->d, p->dv)) return HLA_ERR_UNSUPPORTED;
  if (!plocal_fits(p->chunk, p->d)) return HLA_ERR_BAD_VALUE;
  if (!q || !v || !plocal || !o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(v) || !aligned16(plocal) || !aligned16(o) || (den && !aligned16(den)))
    return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_state(prefixes, true, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  const void* ins[8] = {q, v, plocal, prefixes->S, prefixes->C, prefixes->m, prefixes->G, prefixes->h};
  const size_t inb[8] = {z.qk_bytes, z.v_bytes, hla_fwd_p_bytes(p),
                         z.units * z.n * z.S * 4, z.units * z.n * z.C * 4, z.units * z.n * z.m * 4,
                         z.units * z.n * z.C * 4, z.units * z.n * z.m * 4};
  for (int j = 0; j < 8; ++j) {
    if (overlap(o, z.o_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, z.den_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, z.o_bytes, den, z.den_bytes)) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  ChunkArgs a = chunk_args(p, q, nullptr, v, prefixes, o, den);
  a.pl = const_cast<void*>(plocal);
  return from_hip(hla::launch_outputs_from_p((int)z.units, a, static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_fwd(const hla_problem* p, const void* q, const void* k, const void* v, float* o,
                   float* den, const hla_state* final_state, void* workspace,
                   size_t workspace_bytes, void* stream) try {
  if (hla_status e = hla::fwd_validate(p, q, k, v, o, den, final_state, workspace,
                                        workspace_bytes, true))
    return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = device_ready()) return e;
  return hla::fwd_enqueue(p, q, k, v, o, den, final_state, workspace, workspace_bytes, stream);
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"

namespace hla {

// Host-side checks of hla_fwd's arguments.  With check_ws the workspace must
// be present (when the problem needs one), aligned and disjoint from the
// inputs and outputs; without it the caller supplies a workspace of its own.
hla_status fwd_validate(const hla_problem* p, const void* q, const void* k, const void* v,
                        float* o, float* den, const hla_state* final_state, const void* workspace,
                        size_t workspace_bytes, bool check_ws) {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den))) return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  const size_t minimum = check_ws ? hla_fwd_workspace_bytes(p) : 0;
  if (workspace_bytes < minimum) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (minimum > 0) {
    if (!workspace) return HLA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  }
  // the part of the workspace the chosen plan uses
  const size_t need = check_ws ? fwd_plan(p, workspace_bytes).end : 0;
  const void* ins[4] = {q, k, v, workspace};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need};
  for (int j = 0; j < 4; ++j) {
    if (overlap(o, z.o_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, z.den_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, z.o_bytes, den, z.den_bytes)) return HLA_ERR_ALIASING;
  if (final_state) {
    const void* fins[6] = {q, k, v, workspace, o, den};
    const size_t finb[6] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need, z.o_bytes,
                            den ? z.den_bytes : 0};
    if (hla_status e = check_state(final_state, false, z.units, z, fins, finb, 6)) return e;
  }
  return HLA_OK;
}

// Enqueues the whole forward on `stream` with the summaries and the scan's
// scratch in `workspace` (workspace_bytes >= hla_fwd_workspace_bytes(p); the
// segment-local p path when it also holds hla_fwd_p_workspace_bytes(p); the
// arguments have passed fwd_validate and the problem is not empty).
hla_status fwd_enqueue(const hla_problem* p, const void* q, const void* k, const void* v,
                       float* o, float* den, const hla_state* final_state, void* workspace,
                       size_t workspace_bytes, void* stream) {
  // spans of R chunks: summaries of the spans, the scan over them, outputs
  hla_problem ps = *p;
  ps.chunk = (int32_t)(p->chunk * fwd_span_chunks(p));
  const Sizes z = sizes_of(&ps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* w = static_cast<float*>(workspace);
  const size_t cnt = (size_t)z.units * (size_t)z.n;
  hla_state sm;
  sm.S = w; sm.C = sm.S + cnt * z.S; sm.m = sm.C + cnt * z.C; sm.G = sm.m + cnt * z.m;
  sm.h = sm.G + cnt * z.C;
  const FwdPlan f = fwd_plan(p, workspace_bytes);
  char* const wb = static_cast<char*>(workspace);
  void* scan_ws = wb + f.scan_ws;
  // the exclusive prefixes out of place when the workspace has room for them
  hla_state po{};
  const hla_state* prefix_out = nullptr;
  if (f.po_off) {
    po.S = reinterpret_cast<float*>(wb + f.po_off); po.C = po.S + cnt * z.S; po.m = po.C + cnt * z.C;
    po.G = po.m + cnt * z.m; po.h = po.G + cnt * z.C;
    prefix_out = &po;
  }
  // the segment-local p, when the workspace holds it: the output kernel then
  // carries no S recurrence
  void* plocal = f.p_off ? wb + f.p_off : nullptr;
  ChunkArgs a1 = chunk_args(&ps, q, k, v, &sm, nullptr, nullptr);
  a1.pl = plocal;
  if (hla_status e = from_hip(hla::launch_chunk_summaries(p->in_dtype, p->d, p->dv, (int)z.units, a1, s)))
    return e;
  if (hla_status e = do_scan(&ps, &sm, final_state, scan_ws, s, prefix_out)) return e;
  if (prefix_out) sm = po;
  ChunkArgs a3 = chunk_args(&ps, q, k, v, &sm, o, den);
  if (plocal) {
    a3.pl = plocal;
    return from_hip(hla::launch_outputs_from_p((int)z.units, a3, s));
  }
  return from_hip(hla::launch_chunk_outputs(p->in_dtype, p->d, p->dv, (int)z.units, a3, s));
}

}  // namespace hla

namespace {

// S, C, m of `st` (G and h are not used by the unmasked variant) for `count`
// segments: present, aligned, disjoint from each other and from the inputs.
hla_status check_moments(const hla_state* st, int64_t count, const Sizes& z,
                         const void* const* inputs, const size_t* in_bytes, int n_inputs) {
  if (!st) return HLA_ERR_NULL_POINTER;
  if (!st->S || !st->C || !st->m) return HLA_ERR_NULL_POINTER;
  hla_state mo = *st;
  mo.G = mo.h = nullptr;
  return check_state(&mo, false, count, z, inputs, in_bytes, n_inputs);
}

hla_status unmasked_summaries(const hla_problem* p, const void* q, const void* k, const void* v,
                              const hla_state* st, hipStream_t s) {
  const Sizes z = sizes_of(p);
  hla_state mo = *st;
  mo.G = mo.h = nullptr;
  const ChunkArgs a = chunk_args(p, q, k, v, &mo, nullptr, nullptr);
  return from_hip(hla::launch_unmasked_summaries(p->in_dtype, p->d, p->dv, (int)z.units, a, s));
}

hla_status unmasked_scan(const hla_problem* p, const hla_state* st, hipStream_t s) {
  const Sizes z = sizes_of(p);
  hla_state mo = *st;
  mo.G = mo.h = nullptr;
  const ChunkArgs a = chunk_args(p, nullptr, nullptr, nullptr, &mo, nullptr, nullptr);
  return from_hip(hla::launch_unmasked_scan(a, (int)z.units, p->d, p->dv, s));
}

hla_status unmasked_outputs(const hla_problem* p, const void* q, const void* k, const void* v,
                            const hla_state* st, float* o, float* den, hipStream_t s) {
  const Sizes z = sizes_of(p);
  hla_state mo = *st;
  mo.G = mo.h = nullptr;
  const ChunkArgs a = chunk_args(p, q, k, v, &mo, o, den);
  return from_hip(hla::launch_unmasked_outputs(p->in_dtype, p->d, p->dv, (int)z.units, a, s));
}

// o and den against the inputs (ins / inb) and each other
hla_status check_outputs(const Sizes& z, float* o, float* den, const void* const* ins,
                         const size_t* inb, int n) {
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den))) return HLA_ERR_MISALIGNED;
  for (int j = 0; j < n; ++j) {
    if (overlap(o, z.o_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, z.den_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, z.o_bytes, den, z.den_bytes)) return HLA_ERR_ALIASING;
  return HLA_OK;
}

}  // namespace

extern "C" {

hla_status hla_unmasked_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                        const void* v, const hla_state* out, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {z.qk_bytes, z.qk_bytes, z.v_bytes};
  if (hla_status e = check_moments(out, z.units * z.n, z, ins, inb, 3)) return e;
  if (hla_status e = device_ready()) return e;
  return unmasked_summaries(p, q, k, v, out, static_cast<hipStream_t>(stream));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_unmasked_scan(const hla_problem* p, const hla_state* inout, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_moments(inout, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  if (hla_status e = device_ready()) return e;
  return unmasked_scan(p, inout, static_cast<hipStream_t>(stream));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_unmasked_output(const hla_problem* p, const void* q, const void* k, const void* v,
                               const hla_state* prefixes, float* o, float* den, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_moments(prefixes, z.units * z.n, z, nullptr, nullptr, 0)) return e;
  const void* ins[6] = {q, k, v, prefixes->S, prefixes->C, prefixes->m};
  const size_t inb[6] = {z.qk_bytes, z.qk_bytes, z.v_bytes, z.units * z.n * z.S * 4,
                         z.units * z.n * z.C * 4, z.units * z.n * z.m * 4};
  if (hla_status e = check_outputs(z, o, den, ins, inb, 6)) return e;
  if (hla_status e = device_ready()) return e;
  return unmasked_outputs(p, q, k, v, prefixes, o, den, static_cast<hipStream_t>(stream));
} catch (...) {
  return HLA_ERR_HIP;
}

size_t hla_unmasked_fwd_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  const Sizes z = sizes_of(p);
  return (size_t)z.units * (size_t)z.n * (z.S + z.C + z.m) * 4;
}

hla_status hla_unmasked_fwd(const hla_problem* p, const void* q, const void* k, const void* v,
                            float* o, float* den, void* workspace, size_t workspace_bytes,
                            void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  const Sizes z = sizes_of(p);
  const size_t need = hla_unmasked_fwd_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return HLA_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  const void* ins[4] = {q, k, v, workspace};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need};
  if (hla_status e = check_outputs(z, o, den, ins, inb, 4)) return e;
  for (int j = 0; j < 3; ++j)
    if (overlap(workspace, need, ins[j], inb[j])) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t cnt = (size_t)z.units * (size_t)z.n;
  hla_state sm;
  sm.S = static_cast<float*>(workspace);
  sm.C = sm.S + cnt * z.S;
  sm.m = sm.C + cnt * z.C;
  sm.G = sm.h = nullptr;
  if (hla_status e = unmasked_summaries(p, q, k, v, &sm, s)) return e;
  if (hla_status e = unmasked_scan(p, &sm, s)) return e;
  return unmasked_outputs(p, q, k, v, &sm, o, den, s);
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"

namespace {

struct AhlaSizes {
  size_t P, m, X;   // floats per segment of P (= E), m (= n), X
};

AhlaSizes ahla_sizes(const hla_problem* p) {
  return AhlaSizes{(size_t)p->d * p->dv, (size_t)p->d, (size_t)p->d * p->d};
}

// every field present, aligned, disjoint from the others and from the inputs
hla_status check_ahla_state(const hla_ahla_state* st, int64_t count, const hla_problem* p,
                            const void* const* inputs, const size_t* in_bytes, int n_inputs) {
  if (!st) return HLA_ERR_NULL_POINTER;
  const AhlaSizes z = ahla_sizes(p);
  float* f[5] = {st->P, st->m, st->E, st->n, st->X};
  const size_t per[5] = {z.P, z.m, z.P, z.m, z.X};
  for (int i = 0; i < 5; ++i) {
    if (!f[i]) return HLA_ERR_NULL_POINTER;
    if (!aligned16(f[i])) return HLA_ERR_MISALIGNED;
    const size_t bytes = (size_t)count * per[i] * 4;
    for (int j = 0; j < n_inputs; ++j)
      if (overlap(f[i], bytes, inputs[j], in_bytes[j])) return HLA_ERR_ALIASING;
    for (int j = 0; j < i; ++j)
      if (overlap(f[i], bytes, f[j], (size_t)count * per[j] * 4)) return HLA_ERR_ALIASING;
  }
  return HLA_OK;
}

hla::AhlaArgs ahla_args(const hla_problem* p, const void* q, const void* k, const void* v,
                        const hla_ahla_state* st, float* o, float* den) {
  hla::AhlaArgs a;
  a.q = q; a.k = k; a.v = v; a.gamma = p->gamma;
  a.H = p->H; a.T = p->T; a.chunk = p->chunk; a.nspan = p->T / p->chunk;
  a.normalize = p->normalize; a.eps = p->eps;
  a.P = st->P; a.m = st->m; a.E = st->E; a.n = st->n; a.X = st->X;
  a.o = o; a.den = den;
  return a;
}

size_t ahla_summary_bytes(const hla_problem* p) {
  const Sizes z = sizes_of(p);
  const AhlaSizes a = ahla_sizes(p);
  return (size_t)z.units * (size_t)z.n * (2 * a.P + 2 * a.m + a.X) * 4;
}

}  // namespace

extern "C" {

hla_status hla_ahla_chunk_summaries(const hla_problem* p, const void* q, const void* k,
                                    const void* v, const hla_ahla_state* out, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {z.qk_bytes, z.qk_bytes, z.v_bytes};
  if (hla_status e = check_ahla_state(out, z.units * z.n, p, ins, inb, 3)) return e;
  if (hla_status e = device_ready()) return e;
  return from_hip(hla::launch_ahla_summaries(p->in_dtype, p->d, p->dv, (int)z.units,
                                             ahla_args(p, q, k, v, out, nullptr, nullptr),
                                             static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_ahla_scan(const hla_problem* p, const hla_ahla_state* inout, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_ahla_state(inout, z.units * z.n, p, nullptr, nullptr, 0)) return e;
  if (hla_status e = device_ready()) return e;
  return from_hip(hla::launch_ahla_scan(p->d, p->dv, (int)z.units,
                                        ahla_args(p, nullptr, nullptr, nullptr, inout, nullptr, nullptr),
                                        static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_ahla_output(const hla_problem* p, const void* q, const void* k, const void* v,
                           const hla_ahla_state* prefixes, float* o, float* den, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_ahla_state(prefixes, z.units * z.n, p, nullptr, nullptr, 0)) return e;
  const AhlaSizes a = ahla_sizes(p);
  const size_t cnt = (size_t)z.units * (size_t)z.n;
  const void* ins[7] = {q, k, v, prefixes->P, prefixes->m, prefixes->E, prefixes->n};
  const size_t inb[7] = {z.qk_bytes, z.qk_bytes, z.v_bytes, cnt * a.P * 4, cnt * a.m * 4,
                         cnt * a.P * 4, cnt * a.m * 4};
  if (hla_status e = check_outputs(z, o, den, ins, inb, 7)) return e;
  if (hla_status e = device_ready()) return e;
  return from_hip(hla::launch_ahla_outputs(p->in_dtype, p->d, p->dv, (int)z.units,
                                           ahla_args(p, q, k, v, prefixes, o, den),
                                           static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

size_t hla_ahla_fwd_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  return ahla_summary_bytes(p);
}

hla_status hla_ahla_fwd(const hla_problem* p, const void* q, const void* k, const void* v,
                        float* o, float* den, void* workspace, size_t workspace_bytes,
                        void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  const Sizes z = sizes_of(p);
  const size_t need = hla_ahla_fwd_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return HLA_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  const void* ins[4] = {q, k, v, workspace};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need};
  if (hla_status e = check_outputs(z, o, den, ins, inb, 4)) return e;
  for (int j = 0; j < 3; ++j)
    if (overlap(workspace, need, ins[j], inb[j])) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AhlaSizes a = ahla_sizes(p);
  const size_t cnt = (size_t)z.units * (size_t)z.n;
  hla_ahla_state st;
  st.P = static_cast<float*>(workspace);
  st.E = st.P + cnt * a.P;
  st.X = st.E + cnt * a.P;
  st.m = st.X + cnt * a.X;
  st.n = st.m + cnt * a.m;
  if (hla_status e = from_hip(hla::launch_ahla_summaries(p->in_dtype, p->d, p->dv, (int)z.units,
                                                         ahla_args(p, q, k, v, &st, nullptr, nullptr), s)))
    return e;
  if (hla_status e = from_hip(hla::launch_ahla_scan(p->d, p->dv, (int)z.units,
                                                    ahla_args(p, q, k, v, &st, nullptr, nullptr), s)))
    return e;
  return from_hip(hla::launch_ahla_outputs(p->in_dtype, p->d, p->dv, (int)z.units,
                                           ahla_args(p, q, k, v, &st, o, den), s));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_ahla_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                                int32_t normalize, float eps, const float* gamma, const void* q,
                                const void* k, const void* v, const hla_ahla_state* state,
                                float* o, float* den, void* stream) try {
  if (N < 0 || H < 0) return HLA_ERR_BAD_SHAPE;
  if (in_dtype != HLA_F32 && in_dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (normalize != 0 && normalize != 1) return HLA_ERR_BAD_VALUE;
  if (!std::isfinite(eps)) return HLA_ERR_BAD_VALUE;
  if (!head_ok(d) || !head_ok(dv) || d > 2 * dv || dv > 2 * d) return HLA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)N * H;
  if (units > kMaxGrid) return HLA_ERR_BAD_VALUE;
  if (units == 0) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den)) || (gamma && !aligned16(gamma)))
    return HLA_ERR_MISALIGNED;
  if (!state) return HLA_ERR_NULL_POINTER;
  // P, m, E, n are used (X is not): check them as a masked-style state S, C, m, G, h
  Sizes z;
  z.S = (size_t)d * dv; z.C = (size_t)d * dv; z.m = (size_t)d;
  hla_state as{state->P, state->E, state->m, nullptr, state->n};
  if (!as.S || !as.C || !as.m || !as.h) return HLA_ERR_NULL_POINTER;
  const size_t es = dtype_size(in_dtype);
  const size_t uu = (size_t)units;
  const void* ins[5] = {q, k, v, o, den};
  const size_t inb[5] = {uu * d * es, uu * d * es, uu * dv * es, uu * dv * 4, den ? uu * 4 : 0};
  if (hla_status e = check_state(&as, false, units, z, ins, inb, 5)) return e;
  for (int j = 0; j < 3; ++j) {
    if (overlap(o, inb[3], ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, inb[4], ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, inb[3], den, inb[4])) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  hla::AhlaArgs a;
  a.q = q; a.k = k; a.v = v; a.gamma = gamma;
  a.H = H; a.T = 0; a.chunk = 0; a.nspan = 0; a.normalize = normalize; a.eps = eps;
  a.P = state->P; a.m = state->m; a.E = state->E; a.n = state->n; a.X = nullptr;
  a.o = o; a.den = den;
  return from_hip(hla::launch_ahla_decode(in_dtype, d, dv, (int)units, a,
                                          static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_unmasked_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                                    int32_t normalize, float eps, const float* gamma,
                                    const void* q, const void* k, const void* v,
                                    const hla_state* state, float* o, float* den,
                                    void* stream) try {
  if (N < 0 || H < 0) return HLA_ERR_BAD_SHAPE;
  if (in_dtype != HLA_F32 && in_dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (normalize != 0 && normalize != 1) return HLA_ERR_BAD_VALUE;
  if (!std::isfinite(eps)) return HLA_ERR_BAD_VALUE;
  if (!head_ok(d) || !head_ok(dv) || d > 2 * dv || dv > 2 * d) return HLA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)N * H;
  if (units > kMaxGrid) return HLA_ERR_BAD_VALUE;
  if (units == 0) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den)) || (gamma && !aligned16(gamma)))
    return HLA_ERR_MISALIGNED;
  Sizes z;
  z.S = (size_t)d * d; z.C = (size_t)d * dv; z.m = (size_t)d;
  const size_t es = dtype_size(in_dtype);
  const size_t uu = (size_t)units;
  const void* ins[5] = {q, k, v, o, den};
  const size_t inb[5] = {uu * d * es, uu * d * es, uu * dv * es, uu * dv * 4, den ? uu * 4 : 0};
  if (hla_status e = check_moments(state, units, z, ins, inb, 5)) return e;
  for (int j = 0; j < 3; ++j) {
    if (overlap(o, inb[3], ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, inb[4], ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, inb[3], den, inb[4])) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.gamma = gamma;
  a.S = state->S; a.C = state->C; a.m = state->m; a.G = nullptr; a.h = nullptr;
  a.o = o; a.den = den; a.H = H; a.normalize = normalize; a.eps = eps;
  return from_hip(hla::launch_unmasked_decode(in_dtype, d, dv, (int)units, a,
                                              static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                           int32_t normalize, float eps, const float* gamma, const void* q,
                           const void* k, const void* v, const hla_state* state, float* o,
                           float* den, void* stream) try {
  if (N < 0 || H < 0) return HLA_ERR_BAD_SHAPE;
  if (in_dtype != HLA_F32 && in_dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (normalize != 0 && normalize != 1) return HLA_ERR_BAD_VALUE;
  if (!std::isfinite(eps)) return HLA_ERR_BAD_VALUE;
  if (!head_ok(d) || !head_ok(dv) || d > 2 * dv || dv > 2 * d) return HLA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)N * H;
  if (units > kMaxGrid) return HLA_ERR_BAD_VALUE;
  if (units == 0) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den)) || (gamma && !aligned16(gamma)))
    return HLA_ERR_MISALIGNED;
  Sizes z;
  z.S = (size_t)d * d; z.C = (size_t)d * dv; z.m = (size_t)d;
  const size_t es = dtype_size(in_dtype);
  const void* ins[5] = {q, k, v, o, den};
  const size_t uu = (size_t)units;
  const size_t inb[5] = {uu * d * es, uu * d * es, uu * dv * es, uu * dv * 4,
                         den ? (size_t)units * 4 : 0};
  if (hla_status e = check_state(state, true, units, z, ins, inb, 5)) return e;
  for (int j = 0; j < 3; ++j) {
    if (overlap(o, inb[3], ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, inb[4], ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, inb[3], den, inb[4])) return HLA_ERR_ALIASING;
  if (units == 0) return HLA_OK;
  if (hla_status e = device_ready()) return e;
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.gamma = gamma;
  a.S = state->S; a.C = state->C; a.m = state->m; a.G = state->G; a.h = state->h;
  a.o = o; a.den = den; a.H = H; a.normalize = normalize; a.eps = eps;
  return from_hip(hla::launch_decode(in_dtype, d, dv, (int)units, a, static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"

namespace {

size_t bwd_state_floats(const hla_problem* p, const Sizes& z) {
  const size_t w = (size_t)(p->d > p->dv ? p->d : p->dv);
  return (size_t)z.units * (size_t)z.n * w * w;
}

size_t bwd_core_bytes(const hla_problem* p, const Sizes& z) {
  const size_t do16 = p->in_dtype == HLA_BF16 ? (size_t)z.units * (size_t)p->T * (size_t)p->dv * 2 : 0;
  return (2 * (size_t)z.units * (size_t)p->T * (size_t)p->d + bwd_state_floats(p, z) +
          (size_t)z.units * (size_t)z.n * (size_t)p->d * (size_t)p->d) * 4 + do16;
}

// Extra workspace of the ratio-normalised backward, after the core's: the
// unnormalised num [tok, dv] and den [tok] (fp32), the upstream gradients
// g_num [tok, dv], g_den [tok, 16] and the unit channel [tok, 16] (in the
// MFMA operand type), dp rounded to bf16 [tok, d] (bf16 inputs), and the
// forward's own workspace; every part 16-byte aligned.
struct NormWs {
  size_t num, den, gnum, gden, one, dp16, fwd, total;
};

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

NormWs norm_ws(const hla_problem* p, const Sizes& z) {
  NormWs w;
  const size_t tok = (size_t)z.units * (size_t)p->T;
  const size_t es = p->in_dtype == HLA_BF16 ? 2 : 4;
  w.num = align16(bwd_core_bytes(p, z));
  w.den = w.num + align16(tok * p->dv * 4);
  w.gnum = w.den + align16(tok * 4);
  w.gden = w.gnum + align16(tok * p->dv * es);
  w.one = w.gden + align16(tok * 16 * es);
  w.dp16 = w.one + align16(tok * 16 * es);
  w.fwd = w.dp16 + align16(p->in_dtype == HLA_BF16 ? tok * p->d * 2 : 0);
  hla_problem pf = *p;
  pf.normalize = 0;
  w.total = w.fwd + hla_fwd_workspace_bytes(&pf);
  return w;
}

}  // namespace

extern "C" {

size_t hla_bwd_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  const Sizes z = sizes_of(p);
  return p->normalize ? norm_ws(p, z).total : bwd_core_bytes(p, z);
}

hla_status hla_bwd(const hla_problem* p, const void* q, const void* k, const void* v,
                   const float* dout, float* dq, float* dk, float* dv, void* workspace,
                   size_t workspace_bytes, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!dout || !dq || !dk || !dv) return HLA_ERR_NULL_POINTER;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  const size_t need = hla_bwd_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return HLA_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  const size_t tok = (size_t)z.units * (size_t)p->T;
  const size_t gq = tok * p->d * 4, gv = tok * p->dv * 4;
  const void* ins[5] = {q, k, v, dout, workspace};
  const size_t inb[5] = {z.qk_bytes, z.qk_bytes, z.v_bytes, z.o_bytes, need};
  float* outs[3] = {dq, dk, dv};
  const size_t outb[3] = {gq, gq, gv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j])) return HLA_ERR_ALIASING;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return HLA_ERR_ALIASING;
  }
  for (int j = 0; j < 4; ++j)
    if (overlap(workspace, need, ins[j], inb[j])) return HLA_ERR_ALIASING;
  if (hla_status e = device_ready()) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);

  float* pbuf = static_cast<float*>(workspace);
  float* dpbuf = pbuf + tok * p->d;
  float* hbuf = dpbuf + tok * p->d;
  // prefixes of the states sum g^(..) k k^T, shared by p = S q and S dp
  float* hkk = hbuf + bwd_state_floats(p, z);
  const int bf = p->in_dtype == HLA_BF16 ? 1 : 0;
  // with bf16 inputs p and dp are only ever read back as bf16 MFMA operands,
  // so they are stored as bf16 (the same rounding, half the traffic)
  const hla::LaOperand Q{q, bf}, K{k, bf}, V{v, bf}, DO{dout, 0}, P{pbuf, bf}, DP{dpbuf, bf};
  auto run = [&](hla::LaOperand a, hla::LaOperand b, hla::LaOperand c, int Da, int Dc, int gexp,
                 int reverse, float* y, int accumulate, float* states = nullptr,
                 bool ready = false, int sym = 0, int hp_t = 0, int y_bf16 = 0,
                 void* b_copy = nullptr) -> hla_status {
    hla::LaArgs la;
    la.a = a; la.b = b; la.c = c;
    la.y = y; la.Hp = states ? states : hbuf; la.gamma = p->gamma;
    la.H = p->H; la.gexp = gexp;
    la.T = p->T; la.seg = p->chunk; la.nseg = (int)z.n;
    la.reverse = reverse; la.accumulate = accumulate;
    la.mfma_bf16 = bf;
    la.sym = sym;
    la.hp_transposed = hp_t;
    la.y_bf16 = y_bf16;
    la.b_copy = b_copy;
    return from_hip(hla::launch_first_order_sum(Da, Dc, (int)z.units, la, s, ready));
  };
  const int d = p->d, e = p->dv;
  // with bf16 inputs the dp sum writes dO rounded to bf16 as it stages it (the
  // rounding every later use applies anyway); dv and dq read that copy
  void* do16 = bf ? static_cast<void*>(hkk + (size_t)z.units * (size_t)z.n * (size_t)d * (size_t)d)
                  : nullptr;
  const hla::LaOperand DOb = bf ? hla::LaOperand{do16, 1} : DO;
  if (p->normalize) {
    // o = num / (den + eps): the gradient is that of the numerator with the
    // value channel v = 1 appended (den is num with v = 1) and the upstream
    // gradient [dO / (den + eps), -(dO . num) / (den + eps)^2].  The v = 1
    // channel adds one term to dp and one to dq: two more first-order sums
    // whose operands carry the scalar in column 0 of 16.
    const NormWs nw = norm_ws(p, z);
    char* wb = static_cast<char*>(workspace);
    float* num = reinterpret_cast<float*>(wb + nw.num);
    float* den = reinterpret_cast<float*>(wb + nw.den);
    void* gnum = wb + nw.gnum;
    void* gden = wb + nw.gden;
    void* one = wb + nw.one;
    void* dp16 = wb + nw.dp16;
    hla_problem pf = *p;
    pf.normalize = 0;
    if (hla_status r = hla::fwd_enqueue(&pf, q, k, v, num, den, nullptr, wb + nw.fwd,
                                        hla_fwd_workspace_bytes(&pf), stream))
      return r;
    if (hla_status r = from_hip(hla::launch_norm_grad(bf, num, den, dout, p->eps, tok, e, gnum, gden,
                                                      one, s)))
      return r;
    const hla::LaOperand G{gnum, bf}, GD{gden, bf}, ONE{one, bf};
    const hla::LaOperand DPn = bf ? hla::LaOperand{dp16, 1} : hla::LaOperand{dpbuf, 0};
    if (hla_status r = run(Q, K, K, d, d, 1, 0, pbuf, 0, hkk, false, 0, 0, bf)) return r;
    // dp = sum_{t>=j} g^2(t-j) (v_j.G_t + g_t) q_t, accumulated in fp32
    if (hla_status r = run(V, G, Q, e, d, 2, 1, dpbuf, 0)) return r;
    if (hla_status r = run(P, Q, G, d, e, 2, 1, dv, 0, nullptr, true, 0, 1)) return r;
    if (hla_status r = run(ONE, GD, Q, 16, d, 2, 1, dpbuf, 1)) return r;
    if (bf) {
      if (hla_status r = from_hip(hla::launch_to_bf16(dpbuf, dp16, tok * d, s))) return r;
    }
    // dq = sum_{j<=t} g^2(t-j) (G_t.v_j + g_t) p_j + S_t dp_t
    if (hla_status r = run(G, V, P, e, d, 2, 0, dq, 0)) return r;
    if (hla_status r = run(GD, ONE, P, 16, d, 2, 0, dq, 1)) return r;
    if (hla_status r = run(DPn, K, K, d, d, 1, 0, dq, 1, hkk, true)) return r;
    if (d >= (bf ? 32 : 4)) return run(K, Q, DPn, d, d, 1, 1, dk, 0, nullptr, false, 1);
    if (hla_status r = run(K, Q, DPn, d, d, 1, 1, dk, 0)) return r;
    return run(K, DPn, Q, d, d, 1, 1, dk, 1);
  }
  // p = S q; dp, dv over the future tokens (weights g^2); dq = M dO + S dp;
  // dk from the future tokens' q and dp (weights g): one sum over the
  // symmetric states g^(..) (q dp^T + dp q^T) when d spans whole MFMA steps
  if (hla_status r = run(Q, K, K, d, d, 1, 0, pbuf, 0, hkk, false, 0, 0, bf)) return r;
  // (dv's states g^(..) q dO^T are the transposes of dp's: its output pass
  // starts from dp's prefixes)
  if (hla_status r = run(V, DO, Q, e, d, 2, 1, dpbuf, 0, nullptr, false, 0, 0, bf, do16)) return r;
  if (hla_status r = run(P, Q, DOb, d, e, 2, 1, dv, 0, nullptr, true, 0, 1)) return r;
  if (hla_status r = run(DOb, V, P, e, d, 2, 0, dq, 0)) return r;
  if (hla_status r = run(DP, K, K, d, d, 1, 0, dq, 1, hkk, true)) return r;
  if (d >= (bf ? 32 : 4)) return run(K, Q, DP, d, d, 1, 1, dk, 0, nullptr, false, 1);
  if (hla_status r = run(K, Q, DP, d, d, 1, 1, dk, 0)) return r;
  return run(K, DP, Q, d, d, 1, 1, dk, 1);
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"

// ---- third-order HLA ------------------------------------------------------------

namespace {

// Workspace of the third-order calls: p, u and u_m (local, then global; the
// MFMA operand type), the segment summaries (fp32; m, z, r in the 16-wide
// layout), den16 and the 16-wide total of m.
struct Ws3 {
  size_t p, u, um, S, Q, V, P, Z, R, m, z, r, den16, tm16, total;
};

Ws3 ws3_of(const hla_problem* p) {
  const Sizes z = sizes_of(p);
  const size_t tok = (size_t)z.units * (size_t)p->T, es = dtype_size(p->in_dtype);
  const size_t cnt = (size_t)z.units * (size_t)z.n, d = p->d, e = p->dv;
  Ws3 w;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align16(bytes); return at; };
  w.p = take(tok * d * es);
  w.u = take(tok * e * es);
  w.um = take(tok * 16 * es);
  w.S = take(cnt * d * d * 4);
  w.Q = take(cnt * d * d * 4);
  w.V = take(cnt * d * d * 4);
  w.P = take(cnt * d * e * 4);
  w.Z = take(cnt * d * e * 4);
  w.R = take(cnt * d * e * 4);
  w.m = take(cnt * d * 16 * 4);
  w.z = take(cnt * d * 16 * 4);
  w.r = take(cnt * d * 16 * 4);
  w.den16 = take(tok * 16 * 4);
  w.tm16 = take((size_t)z.units * d * 16 * 4);
  w.total = off;
  return w;
}

struct Third {
  const hla_problem* p;
  Sizes z;
  hipStream_t s;
  int bf;
  hla::LaOperand Q, K, V, ONE, Pq, U, UM;
  // the scalar channel of a summary pass: a second sum with the same a, b
  // and lam whose value is column 0 of c2 (16 wide), its segment states Hp2
  // (16 wide)
  struct Channel {
    hla::LaOperand c2{nullptr, 0};
    float* Hp2 = nullptr;
  };
  // one first-order sum over this problem's segments (with `ch`, a summary
  // pass, its channel in the same pass)
  hla_status sum(hla::LaOperand a, hla::LaOperand b, hla::LaOperand c, int Da, int Dc, int gexp,
                 float* y, int y_bf16, float* Hp, bool states_only, float* Hout = nullptr,
                 const Channel* ch = nullptr) const {
    hla::LaArgs la;
    la.a = a; la.b = b; la.c = c;
    if (ch) {
      la.ch = 1;
      la.c2 = ch->c2; la.Hp2 = ch->Hp2;
    }
    la.y = y; la.Hp = Hp; la.Hout = Hout; la.gamma = p->gamma;
    la.H = p->H; la.gexp = gexp;
    la.T = p->T; la.seg = p->chunk; la.nseg = (int)z.n;
    la.reverse = 0; la.accumulate = 0;
    la.mfma_bf16 = bf;
    la.y_bf16 = y_bf16;
    if (states_only) return from_hip(hla::launch_first_order_states(Da, Dc, (int)z.units, la, s));
    return from_hip(hla::launch_first_order_sum(Da, Dc, (int)z.units, la, s, true));
  }
};

// Segment summaries into the workspace arrays of `w` (S, Q, V, P, Z, R as
// [units, n, ...], m, z, r 16 wide), through the local p, u, u_m.
hla_status third_summaries(const Third& t, char* wb, const Ws3& w, float* S, float* Qm, float* V,
                           float* P, float* Z, float* R) {
  const int d = t.p->d, e = t.p->dv;
  float* m = reinterpret_cast<float*>(wb + w.m);
  float* z = reinterpret_cast<float*>(wb + w.z);
  float* r = reinterpret_cast<float*>(wb + w.r);
  float* py = reinterpret_cast<float*>(wb + w.p);
  float* uy = reinterpret_cast<float*>(wb + w.u);
  float* umy = reinterpret_cast<float*>(wb + w.um);
  // local p, u, u_m: every segment from the zero state; the same passes leave
  // the segment states of their sums, the summaries S^K, P^KV and m^K
  if (hla_status x = t.sum(t.Q, t.K, t.K, d, d, 1, py, t.bf, nullptr, false, S)) return x;
  if (hla_status x = t.sum(t.Q, t.K, t.V, d, e, 1, uy, t.bf, nullptr, false, P)) return x;
  if (hla_status x = t.sum(t.Q, t.K, t.ONE, d, 16, 1, umy, t.bf, nullptr, false, m)) return x;
  // the other summaries as segment states; z and r ride on Z's and R's
  // passes (the same a, b and lam) as their scalar channels
  if (hla_status x = t.sum(t.Q, t.Q, t.Q, d, d, 1, nullptr, 0, Qm, true)) return x;
  if (hla_status x = t.sum(t.Q, t.Pq, t.Q, d, d, 2, nullptr, 0, V, true)) return x;
  Third::Channel cz;
  cz.c2 = t.UM; cz.Hp2 = z;
  if (hla_status x = t.sum(t.Q, t.Q, t.U, d, e, 2, nullptr, 0, Z, true, nullptr, &cz)) return x;
  Third::Channel cr;
  cr.c2 = t.UM; cr.Hp2 = r;
  return t.sum(t.Q, t.Pq, t.U, d, e, 3, nullptr, 0, R, true, nullptr, &cr);
}

hla_status third_setup(const hla_problem* p, const void* q, const void* k, const void* v,
                       void* workspace, void* stream, Third& t, Ws3& w) {
  t.p = p;
  t.z = sizes_of(p);
  t.s = static_cast<hipStream_t>(stream);
  t.bf = p->in_dtype == HLA_BF16 ? 1 : 0;
  w = ws3_of(p);
  char* wb = static_cast<char*>(workspace);
  t.Q = {q, t.bf}; t.K = {k, t.bf}; t.V = {v, t.bf};
  t.ONE = {nullptr, t.bf};   // the unit channel, formed by the kernels
  t.Pq = {wb + w.p, t.bf}; t.U = {wb + w.u, t.bf};
  t.UM = {wb + w.um, t.bf};
  return HLA_OK;
}

hla_status check_state3(const hla3_state* st, bool all_required, int64_t count, const hla_problem* p,
                        const void* const* ins, const size_t* inb, int nin) {
  if (!st) return HLA_ERR_NULL_POINTER;
  float* f[5] = {st->S, st->P, st->m, st->R, st->r};
  const size_t d = p->d, e = p->dv;
  const size_t per[5] = {d * d, d * e, d, d * e, d};
  for (int i = 0; i < 5; ++i) {
    if (!f[i]) {
      if (all_required) return HLA_ERR_NULL_POINTER;
      continue;
    }
    if (!aligned16(f[i])) return HLA_ERR_MISALIGNED;
    const size_t b = (size_t)count * per[i] * 4;
    for (int j = 0; j < nin; ++j)
      if (overlap(f[i], b, ins[j], inb[j])) return HLA_ERR_ALIASING;
    for (int j = 0; j < i; ++j)
      if (f[j] && overlap(f[i], b, f[j], (size_t)count * per[j] * 4)) return HLA_ERR_ALIASING;
  }
  return HLA_OK;
}

hla_status check_summary3(const hla3_summary* sm, int64_t count, const hla_problem* p,
                          const void* const* ins, const size_t* inb, int nin) {
  if (!sm) return HLA_ERR_NULL_POINTER;
  float* f[9] = {sm->S, sm->Q, sm->P, sm->m, sm->V, sm->Z, sm->z, sm->R, sm->r};
  const size_t d = p->d, e = p->dv;
  const size_t per[9] = {d * d, d * d, d * e, d, d * d, d * e, d, d * e, d};
  for (int i = 0; i < 9; ++i) {
    if (!f[i]) return HLA_ERR_NULL_POINTER;
    if (!aligned16(f[i])) return HLA_ERR_MISALIGNED;
    const size_t b = (size_t)count * per[i] * 4;
    for (int j = 0; j < nin; ++j)
      if (overlap(f[i], b, ins[j], inb[j])) return HLA_ERR_ALIASING;
    for (int j = 0; j < i; ++j)
      if (overlap(f[i], b, f[j], (size_t)count * per[j] * 4)) return HLA_ERR_ALIASING;
  }
  return HLA_OK;
}

}  // namespace

extern "C" {

size_t hla3_workspace_bytes(const hla_problem* p) {
  if (check_problem(p) != HLA_OK || empty_problem(p)) return 0;
  return ws3_of(p).total;
}

hla_status hla3_chunk_summaries(const hla_problem* p, const void* q, const void* k, const void* v,
                                const hla3_summary* out, void* workspace, size_t workspace_bytes,
                                void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  const Sizes z = sizes_of(p);
  const size_t need = hla3_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return HLA_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  const void* ins[4] = {q, k, v, workspace};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need};
  for (int j = 0; j < 3; ++j)
    if (overlap(workspace, need, ins[j], inb[j])) return HLA_ERR_ALIASING;
  if (hla_status e = check_summary3(out, z.units * z.n, p, ins, inb, 4)) return e;
  if (hla_status e = device_ready()) return e;
  Third t;
  Ws3 w;
  third_setup(p, q, k, v, workspace, stream, t, w);
  char* wb = static_cast<char*>(workspace);
  if (hla_status e = third_summaries(t, wb, w, out->S, out->Q, out->V, out->P, out->Z, out->R)) return e;
  const size_t cnt = (size_t)z.units * (size_t)z.n * (size_t)p->d;
  if (hla_status e = from_hip(hla::launch_gather_col0(reinterpret_cast<float*>(wb + w.m), out->m, cnt, t.s)))
    return e;
  if (hla_status e = from_hip(hla::launch_gather_col0(reinterpret_cast<float*>(wb + w.z), out->z, cnt, t.s)))
    return e;
  return from_hip(hla::launch_gather_col0(reinterpret_cast<float*>(wb + w.r), out->r, cnt, t.s));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla3_scan(const hla_problem* p, const hla3_summary* inout, const hla3_state* total_out,
                     void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  const Sizes z = sizes_of(p);
  if (hla_status e = check_summary3(inout, z.units * z.n, p, nullptr, nullptr, 0)) return e;
  if (total_out) {
    const float* f[9] = {inout->S, inout->Q, inout->P, inout->m, inout->V, inout->Z, inout->z,
                         inout->R, inout->r};
    const size_t d = p->d, e = p->dv, cnt = (size_t)z.units * (size_t)z.n;
    const size_t per[9] = {d * d, d * d, d * e, d, d * d, d * e, d, d * e, d};
    const void* ins[9];
    size_t inb[9];
    for (int i = 0; i < 9; ++i) { ins[i] = f[i]; inb[i] = cnt * per[i] * 4; }
    if (hla_status x = check_state3(total_out, false, z.units, p, ins, inb, 9)) return x;
  }
  if (hla_status e = device_ready()) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = p->d, e = p->dv, units = (int)z.units, n = (int)z.n;
  const hla3_state* t = total_out;
  {
    float* const xs[3] = {inout->S, inout->P, inout->m};
    float* const ts[3] = {t ? t->S : nullptr, t ? t->P : nullptr, t ? t->m : nullptr};
    const int el[3] = {d * d, d * e, d};
    if (hla_status x = from_hip(hla::launch_moments_scan(xs, ts, el, p->gamma, p->H, p->chunk, n, units, s)))
      return x;
  }
  hla::R3ScanArgs a;
  a.Sp = inout->S; a.Pp = inout->P; a.mp = inout->m; a.Q = inout->Q; a.V = inout->V;
  a.Z = inout->Z; a.z = inout->z; a.R = inout->R; a.r = inout->r;
  a.tR = t ? t->R : nullptr; a.tr = t ? t->r : nullptr;
  a.gamma = p->gamma; a.H = p->H; a.seg = p->chunk; a.nseg = n; a.ldm = 1; a.units = (int)units;
  return from_hip(hla::launch_r_scan(d, e, units, a, s));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla3_fwd(const hla_problem* p, const void* q, const void* k, const void* v, float* o,
                    float* den, const hla3_state* final_state, void* workspace,
                    size_t workspace_bytes, void* stream) try {
  if (hla_status e = check_problem(p)) return e;
  if (empty_problem(p)) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den))) return HLA_ERR_MISALIGNED;
  const Sizes z = sizes_of(p);
  const size_t need = hla3_workspace_bytes(p);
  if (workspace_bytes < need) return HLA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return HLA_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return HLA_ERR_MISALIGNED;
  const void* ins[4] = {q, k, v, workspace};
  const size_t inb[4] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need};
  for (int j = 0; j < 4; ++j) {
    if (overlap(o, z.o_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, z.den_bytes, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (j < 3 && overlap(workspace, need, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (den && overlap(o, z.o_bytes, den, z.den_bytes)) return HLA_ERR_ALIASING;
  if (final_state) {
    const void* fins[6] = {q, k, v, workspace, o, den};
    const size_t finb[6] = {z.qk_bytes, z.qk_bytes, z.v_bytes, need, z.o_bytes, den ? z.den_bytes : 0};
    if (hla_status e = check_state3(final_state, false, z.units, p, fins, finb, 6)) return e;
  }
  if (hla_status e = device_ready()) return e;
  Third t;
  Ws3 w;
  third_setup(p, q, k, v, workspace, stream, t, w);
  char* wb = static_cast<char*>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(wb + off); };
  const int d = p->d, e = p->dv, units = (int)z.units, n = (int)z.n;
  if (hla_status x = third_summaries(t, wb, w, F(w.S), F(w.Q), F(w.V), F(w.P), F(w.Z), F(w.R))) return x;
  // the scan: the moments elementwise, then R and r with the segment map
  const hla3_state* fs = final_state;
  const bool want_m = fs && fs->m;
  {
    float* const xs[3] = {F(w.S), F(w.P), F(w.m)};
    float* const ts[3] = {fs ? fs->S : nullptr, fs ? fs->P : nullptr, want_m ? F(w.tm16) : nullptr};
    const int el[3] = {d * d, d * e, d * 16};
    if (hla_status x = from_hip(hla::launch_moments_scan(xs, ts, el, p->gamma, p->H, p->chunk, n, units, t.s)))
      return x;
  }
  if (want_m) {
    if (hla_status x = from_hip(hla::launch_gather_col0(F(w.tm16), fs->m, (size_t)units * d, t.s))) return x;
  }
  hla::R3ScanArgs a;
  a.Sp = F(w.S); a.Pp = F(w.P); a.mp = F(w.m); a.Q = F(w.Q); a.V = F(w.V); a.Z = F(w.Z); a.z = F(w.z);
  a.R = F(w.R); a.r = F(w.r);
  a.tR = fs ? fs->R : nullptr; a.tr = fs ? fs->r : nullptr;
  a.gamma = p->gamma; a.H = p->H; a.seg = p->chunk; a.nseg = n; a.ldm = 16; a.units = (int)units;
  if (hla_status x = from_hip(hla::launch_r_scan(d, e, units, a, t.s))) return x;
  // outputs: p, u, u_m are their segment-local parts (left in the workspace by
  // the summaries) plus the prefix terms lam^(t-s0+1) q_t^T (S, P, m prefix);
  // then num and den from R, r
  if (n > 1) {
    hla::PrefixTermArgs pa;
    pa.a = t.Q;
    pa.y[0] = wb + w.p; pa.y[1] = wb + w.u; pa.y[2] = wb + w.um;
    pa.Hp[0] = F(w.S); pa.Hp[1] = F(w.P); pa.Hp[2] = F(w.m);
    pa.gamma = p->gamma; pa.H = p->H; pa.gexp = 1; pa.T = p->T; pa.seg = p->chunk; pa.nseg = n;
    pa.mfma_bf16 = t.bf;
    if (hla_status x = from_hip(hla::launch_prefix_terms(d, e, units, pa, t.s))) return x;
  }
  if (hla_status x = t.sum(t.Q, t.Pq, t.U, d, e, 3, o, 0, F(w.R), false)) return x;
  if (hla_status x = t.sum(t.Q, t.Pq, t.UM, d, 16, 3, F(w.den16), 0, F(w.r), false)) return x;
  return from_hip(hla::launch_finish3(o, F(w.den16), den, (size_t)units * p->T, e, p->normalize,
                                      p->eps, t.s));
} catch (...) {
  return HLA_ERR_HIP;
}

hla_status hla3_decode_step(int32_t N, int32_t H, int32_t d, int32_t dv, int32_t in_dtype,
                            int32_t normalize, float eps, const float* gamma, const void* q,
                            const void* k, const void* v, const hla3_state* state, float* o,
                            float* den, void* stream) try {
  if (N < 0 || H < 0) return HLA_ERR_BAD_SHAPE;
  if (in_dtype != HLA_F32 && in_dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (normalize != 0 && normalize != 1) return HLA_ERR_BAD_VALUE;
  if (!std::isfinite(eps)) return HLA_ERR_BAD_VALUE;
  if (!head_ok(d) || !head_ok(dv) || d > 2 * dv || dv > 2 * d) return HLA_ERR_UNSUPPORTED;
  if ((int64_t)N * H > kMaxGrid) return HLA_ERR_BAD_VALUE;
  if (N == 0 || H == 0) return HLA_OK;
  if (hla_status e = check_qkv(q, k, v)) return e;
  if (!o) return HLA_ERR_NULL_POINTER;
  if (!aligned16(o) || (den && !aligned16(den)) || (gamma && !aligned16(gamma))) return HLA_ERR_MISALIGNED;
  const size_t units = (size_t)N * (size_t)H;
  const size_t es = in_dtype == HLA_BF16 ? 2 : 4;
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {units * d * es, units * d * es, units * dv * es};
  hla_problem pd{};
  pd.d = d; pd.dv = dv;
  if (hla_status e = check_state3(state, true, (int64_t)units, &pd, ins, inb, 3)) return e;
  const void* outs_in[5] = {state->S, state->P, state->m, state->R, state->r};
  const size_t outs_b[5] = {units * d * d * 4, units * d * dv * 4, units * d * 4, units * d * dv * 4,
                            units * d * 4};
  for (int j = 0; j < 5; ++j) {
    if (overlap(o, units * dv * 4, outs_in[j], outs_b[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, units * 4, outs_in[j], outs_b[j])) return HLA_ERR_ALIASING;
  }
  for (int j = 0; j < 3; ++j) {
    if (overlap(o, units * dv * 4, ins[j], inb[j])) return HLA_ERR_ALIASING;
    if (den && overlap(den, units * 4, ins[j], inb[j])) return HLA_ERR_ALIASING;
  }
  if (hla_status e = device_ready()) return e;
  hla::Decode3Args a;
  a.q = q; a.k = k; a.v = v; a.gamma = gamma;
  a.S = state->S; a.P = state->P; a.m = state->m; a.R = state->R; a.r = state->r;
  a.o = o; a.den = den; a.H = H; a.normalize = normalize; a.eps = eps;
  return from_hip(hla::launch_decode3(in_dtype, d, dv, (int)units, a, static_cast<hipStream_t>(stream)));
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"
