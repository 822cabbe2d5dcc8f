// Routed-expert FFN (MXFP4 expert weights, MXFP8 activations) -- internal interface.
#pragma once
#include "common.h"
#include "gemm.h"

namespace dlm {

// Shapes of one MoE layer.  Experts 0..E-1 are routed, E..E+S-1 shared; every row has
// NS = top_k + S output slots (routed ranks 0..top_k-1, then the shared experts).
struct MoeDims {
  int d, F, E, S, top_k, NS, rows;
  size_t w13_bytes() const { return (size_t)2 * F * d / 2; }     // e2m1 codes per expert
  size_t w13_scale_bytes() const { return (size_t)2 * F * d / 32; }
  size_t w2_bytes() const { return (size_t)d * F / 2; }
  size_t w2_scale_bytes() const { return (size_t)d * F / 32; }
  size_t expert_bytes() const { return w13_bytes() + w13_scale_bytes() + w2_bytes() + w2_scale_bytes(); }
};
MoeDims moe_dims(const dlm_model_desc& d);

// Packed bytes of one layer's experts (router excluded).
size_t moe_layer_packed_bytes(const MoeDims& m);
// Repack one layer's experts from the natural MXFP4 layout given in dlm_layer_weights into dst
// (moe_layer_packed_bytes bytes).
int moe_pack_layer(const MoeDims& m, const dlm_layer_weights& L, void* dst, hipStream_t st);

size_t moe_ws_bytes(const dlm_model_desc& d);
// Pointers into a MoE workspace (test views).
void moe_views(const MoeDims& m, void* ws, dlm_decode_views* out);
// f: bf16 normed rows in the packed activation order; router_packed: the router matrix packed
// for the stream-K GEMM (router_plan); experts: the layer's packed experts.  Writes each row's
// weighted expert outputs to per-slot rows that *out describes (the next RMSNorm adds them).
// Each call adds its number of distinct experts hit to a per-layer counter in ws (statistics).
int moe_ffn(const MoeDims& m, int layer, const void* f, const void* router_packed, GemmPlan router_plan,
            const void* experts, void* ws, void* gemm_ws, const int32_t* cont_dev, PartialSrc* out,
            hipStream_t st);

}  // namespace dlm
