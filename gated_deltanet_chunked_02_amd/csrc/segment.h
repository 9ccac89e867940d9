// Launchers of the segmented variant's packed-batch table and of the segment scan over
// per-sequence segment ranges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Segments of a packed batch: sequence n (tokens [cu[n], cu[n+1]), clamped to [0, Ttot])
// is cut into ceil(len / Ls) segments of Ls tokens, the last one ragged.  Writes
// seg_first[n] = index of n's first segment (seg_first[N] = the total) and the segments'
// packed table cu_seg[0 .. nseg] (entries past the total repeat the end of the token range).
// One workgroup.
hipError_t launch_segment_table_packed(const int32_t* cu, int32_t* cu_seg, int32_t* seg_first,
                                       int N, int Ttot, int Ls, int nseg, hipStream_t st);

// h_in(s + 1) = M_s h_in(s) + b_s over the segments of each sequence: those of sequence n are
// seg_first[n] .. seg_first[n + 1] - 1, or n S .. n S + S - 1 when seg_first is null.
hipError_t launch_segment_scan_ranges(const float* M, const float* b, const float* h0,
                                      float* h_in, float* ht, const int32_t* seg_first, int N,
                                      int S, int H, int D, hipStream_t st);

// The backward's composition, in reverse: for the segments of each sequence from last to
// first, dh_end[s] = x and then x <- M_s^T x + e[s], from x = dht (zero when absent); dh0 (if
// not null) receives the final x.  D = 64 or 128.
hipError_t launch_segment_rscan(const float* M, const float* e, const float* dht,
                                float* dh_end, float* dh0, const int32_t* seg_first, int N,
                                int S, int H, int D, hipStream_t st);

// seg_chunks[j] = the chunk-table index of segment j's first chunk (cps chunks per segment,
// segments of sequence n as in launch_segment_scan_ranges); seg_chunks[nseg] = the total.
hipError_t launch_segment_chunks(const int32_t* seq_chunks, const int32_t* seg_first,
                                 int32_t* seg_chunks, int N, int S, int cps, int nseg,
                                 hipStream_t st);

}  // namespace gdn
