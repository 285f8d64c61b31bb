// The matrix-core path of mdt_medusa_heads for batches (see heads_mfma.hip).
#pragma once

#include "common.h"

// Smallest batch that takes the matrix-core path (below it the GEMV path streams the
// weights once with every activation vector in LDS).
constexpr int kHeadsMfmaMinB = 4;

// Whether the bf16 heads of B sequences of hidden size d take the matrix-core path.
bool mdt_heads_mfma_applies(int B, int d);

// Both launches; ws holds K*2B*d bf16 values (a_hi, a_lo per head).  Arguments checked
// by the caller.
mdt_status mdt_heads_mfma(hipStream_t s, int B, int d, int V, int K, const void* h, const void* W1, const void* W2,
                          const void* Wlm, float* logits, void* ws);
