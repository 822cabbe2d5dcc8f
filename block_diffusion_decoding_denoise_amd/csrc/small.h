// Small kernels of the round -- internal interface.
#pragma once
#include "common.h"
#include "gemm.h"

namespace dlm {
// x: f32 [rows, d] residual stream; when ps is non-null and holds partial sums, x is first
// completed with them (x += sum of partials, written back), then normalised into out.
int rmsnorm(float* x, const void* g, void* out, int rows, int d, int bf16, int packed, float eps,
            const int32_t* cont_dev, hipStream_t st, const PartialSrc* ps = nullptr);
int commit_launch(const dlm_commit_rule& rule, int rows, const float* maxp, const int32_t* amax,
                  const float* lse, const float* ent, uint8_t* committed, int32_t* tokens,
                  dlm_round_state* state, hipStream_t st);
int block_reset(int rows, uint8_t* committed, int32_t* tokens, dlm_round_state* state, float* pe,
                int pe_elems, hipStream_t st);
int selfcond_prep(const float* pe, const uint8_t* committed, void* xsc, int rows, int d, int bf16,
                  const int32_t* cont_dev, hipStream_t st);
int embed(const int32_t* tokens, const void* E, float* x, int rows, int d, int V, int bf16, hipStream_t st);
int len_add(int32_t* len, int add, hipStream_t st);
int pack_rows_bf16(const void* x, int rows, int k, void* out, hipStream_t st);
}  // namespace dlm
