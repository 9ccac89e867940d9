// Host-side view of one call, shared by the C ABI (api.cpp) and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct Problem {
  int B, T, N, H, Hg, D, C;  // D = Dk = Dv
  int Ttot;                  // B * T tokens on the packed axis
  int max_chunks;            // ceil(Ttot / C) + N: bound on the number of chunks
  bool f32;                  // q, k, v, o are fp32 (else bf16)
  bool beta_f32;             // beta is fp32 (else bf16)
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;
  void* o;
  float* ht;
};

// Intermediates of the staged variant (device pointers inside the caller's workspace).
struct Stages {
  int32_t* table;       // [max_chunks][4]
  int32_t* seq_chunks;  // [N + 1]
  float* g_cum;         // [Ttot][H]
  float* g_t;           // [H][Ttot]
  void* beta_t;         // [H][Ttot]
  float* A;             // [Ttot][H][C]
  void* Tinv;           // [Ttot][H][C]
  void* W;              // [Ttot][H][D]
  void* U;              // [Ttot][H][D]
  void* h_c;            // [max_chunks][H][D][D]
  void* v_new;          // [Ttot][H][D]
};

hipError_t launch_staged(const Problem& p, const Stages& s, int stop_after, hipStream_t st);
bool fused_supported(const Problem& p);
hipError_t launch_fused(const Problem& p, hipStream_t st);

}  // namespace gdn
