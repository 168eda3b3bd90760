// Arguments of the streamed window scan (ssd_scan.hip) and its launch.
#pragma once
#include <hip/hip_runtime.h>

namespace m2 {

struct ScanArgs {
  int B, L, H, G, Q, nchunks;
  const _Float16* x;   // x rows: token stride xstride elements
  const _Float16* Bm;  // B rows: token stride gstride elements
  const _Float16* Cm;  // C rows: token stride gstride elements
  int xstride, gstride;
  const _Float16* dt;
  long long dtld;      // dt rows: token stride in elements
  const float* A;
  const float* D;
  const float* state_in;
  float* state_out;
  const int* seqlens;
  const int* cu;       // packed layout: row offsets (B+1), else null
  int T;               // packed layout: rows of the per-token tensors
  int xpk;             // x, B, C rows follow the packed rows (else padded b * L + t)
  _Float16* y;
  unsigned* ctrl;      // claim counters, done counter, generation, error
  unsigned long long* flags;   // per item: decay bits << 32 | generation tag | 1 once published
  float* agg;          // per item: segment aggregate state (private tile layout)
  int nseg;            // segments per sequence
  int cps;             // chunks per segment
  int tree_lg;         // log2 of the radix of the segment tree
  int pair;            // two segments: the second computes the first's local state itself (no hand-off)
  int dt_sp;
  const float* dt_bias;
  const _Float16* Blo;   // fused conv: B's binary16 remainder, rows of gn elements (else null)
  int gn;
};

// Launches the scan for binary16 x, B, C and dt, N = 128, P = 64 (the
// caller checks those); the workspace pointers (ctrl, flags, agg) follow the
// window workspace layout.  a.nseg = 0 lets the launch choose the segments.
hipError_t launch_ssd_scan(const ScanArgs& a, int cus, hipStream_t st);

// Launches the column scan (colscan.hip): one workgroup per (sequence, head,
// half of the head dim) over the whole sequence, the state split over n
// between its waves; no workspace.  Same argument contract as
// launch_ssd_scan without the B remainder (a.Blo must be null).
hipError_t launch_ssd_colscan(const ScanArgs& a, hipStream_t st);

}  // namespace m2
