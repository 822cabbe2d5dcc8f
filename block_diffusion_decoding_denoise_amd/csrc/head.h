// Tied-embedding head with fused row statistics and p.E -- internal interface.
#pragma once
#include "common.h"

namespace dlm {
size_t head_ws_bytes(int dtype, int rows, int d, int V);
int head_launch(int dtype, const void* h, const void* E, const uint8_t* committed, int rows, int d,
                int V, float* lse, float* ent, float* maxp, int32_t* amax, float* pe,
                float* logits_dbg, void* ws, const int32_t* cont_dev, hipStream_t st);
}  // namespace dlm
