// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
};

struct ScanArgs {
  float *S, *C, *m, *G, *h;             // [units, n, ...] in place
  float *wS, *wC, *wm, *wG, *wh;        // padding slots [units, N - n, ...]
  const float* gamma;
  int H, n, N, chunk;
  int step;                             // tree distance 2^level
  int d, dv;
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
hipError_t launch_chunk_outputs(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                hipStream_t s);
bool chunk_shape_supported(int dtype, int d, int dv);

// Runs the whole exclusive scan (all levels).  t* (each may be nullptr)
// receive the inclusive totals [units, ...].  The padding slots w* must be
// one contiguous region laid out S | C | m | G | h.
hipError_t launch_scan(int units, int d, int dv, const ScanArgs& a, float* tS, float* tC, float* tm,
                       float* tG, float* th, hipStream_t s);

hipError_t launch_decode(int dtype, int d, int dv, int units, const DecodeArgs& a, hipStream_t s);

}  // namespace hla
