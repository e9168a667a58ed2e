// Internal interface of the AoH labeller kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace has {

struct LabelArgs {
  int L, Hq, Hkv, dm, d;
  bool bf16;
  const void* w_q;
  const void* w_k;
  int n_retrieval;
  float threshold;
  float* er_head;   // may be null
  float* er_group;  // may be null
  uint8_t* labels;
  void* ws;
};

size_t label_workspace_bytes(int L, int Hq, int Hkv, int dm, int d);
hipError_t launch_label(const LabelArgs& a, hipStream_t s);

}  // namespace has
