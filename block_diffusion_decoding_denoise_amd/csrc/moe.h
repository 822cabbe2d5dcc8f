// Routed-expert FFN (MXFP4 weights) -- internal interface.
#pragma once
#include "common.h"

namespace dlm {
size_t moe_ws_bytes(const dlm_model_desc& d);
// h += MoE(xn): xn bf16 [rows, d] (normed), h f32 [rows, d].
int moe_ffn(const dlm_model_desc& d, const dlm_layer_weights& L, const void* xn, float* h, int rows, void* ws,
            const int32_t* cont_dev, hipStream_t st);
}  // namespace dlm
