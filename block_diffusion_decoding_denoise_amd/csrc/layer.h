// Fused layer kernels: one launch per sublayer, XCD-local synchronisation -- internal interface.
#pragma once
#include "attn.h"
#include "attn_body.h"
#include "gemm.h"

namespace dlm {

// The fused path serves dense bf16 models whose kv heads map one to one onto the 8 XCDs of
// the chip (hkv = 8), with 4 query heads of 128 per kv head, 32-row blocks, d % 512 == 0 and
// F % 256 == 0 (every workgroup then owns an even number of rows of each matrix, and a wave's
// share of a d-long contraction is a whole number of ring turns).
bool layer_fused_ok(int dtype, int n_experts, int d, int hq, int hkv, int D, int F, int block);

// Rows per workgroup of each packed matrix in the fused layout.
struct FusedDims {
  int d, F, hq, hkv, D;
  int rq;    // QKV rows per workgroup: (G + 2) D / 32
  int ro;    // attention-output rows (output features) per workgroup: d / 32
  int ko;    // attention-output K-slice per XCD: G D
  int rg;    // gate/up rows per workgroup: 2 F / 256
  int kd;    // FFN-down K-slice per XCD: F / 8
};
FusedDims fused_dims(int d, int F, int hq, int hkv, int D);

// Packed-row -> logical-row map of the QKV matrix in the fused layout (host side): XCD x's
// 32 workgroups own its kv head's rows -- the q rows of query heads G x .. G x + G - 1, then
// the kv head's k rows, then its v rows, q and k rows pair-interleaved for RoPE as in the
// per-op layout.
void build_xqkv_row_map(int hq, int hkv, int D, int32_t* out);

// One pass of the residual stream through the attention or FFN sublayer.  mb: 1 (32 rows) or
// 2 (64 rows).  Residual in: base_in [32 mb][d] plus, when part_in is non-null, the 8 XCD
// partial sums part_in[row][8][d] (added in XCD order); the completed residual is written to
// base_out, this sublayer's own output as 8 XCD partials to part_out.
struct LayerIO {
  const float* base_in;
  const float* part_in;
  float* base_out;
  float* part_out;
};

struct LayerBufs {
  uint16_t* xn;        // [8][64 x d] packed normed rows (one copy per XCD)
  uint16_t* q;         // [64][hq][D]
  uint16_t* o;         // packed [64][hq D]
  uint16_t* act;       // packed [64][F]
  void* attn_ws;       // split partials (attn_ws_bytes with 2 query blocks)
  unsigned* bar;       // [8][64] barrier counters (zero before the first use; stay multiples of 32)
  int* err;            // 9 x 128 bytes: word 0 sync error flags (0: none), word 32 (1 + g) the
                       // XCC id group g ran on in the last launch
};

// Attention sublayer: norm, QKV + RoPE + K/V write, attention, split combine, attention
// output.  last_kv_only: stop after the K/V write (commit pass, last layer).
int fused_attn_sublayer(const FusedDims& fd, int mb, const uint16_t* wqkv, const uint16_t* wo_slices,
                        const void* gain, float eps, const LayerIO& io, const LayerBufs& b, const EpiParams& qkv_epi,
                        AttnPlan plan, float softmax_scale, AttnKv kvf, int last_kv_only, const int32_t* cont_dev,
                        hipStream_t st);
// The attention (32 key splits per kv head), its split combine and the attention-output
// projection in one launch, for the per-op path of the models the fused path serves: q
// [32 mb][hq][D] and the K/V cache as the QKV launch before left them; o_packed receives the
// attention output (packed 32-row panels); the projection leaves 8 XCD partials,
// part_out[row][8][d], for the next RMSNorm to add in XCD order.  wo_slices: the
// attention-output matrix as 8 column slices in the row-owned layout (as the fused path packs it).
int attn_out_xcd(const FusedDims& fd, int mb, const uint16_t* wo_slices, const uint16_t* q, const void* k_cache,
                 const void* v_cache, uint16_t* o_packed, void* attn_ws, float* part_out, unsigned* bar, int* err,
                 int cap, const int32_t* len_dev, AttnPlan plan, float softmax_scale, AttnKv kvf,
                 const int32_t* cont_dev, hipStream_t st);
// FFN sublayer: norm, gate/up + SwiGLU, down.
int fused_ffn_sublayer(const FusedDims& fd, int mb, const uint16_t* wgu, const uint16_t* wd_slices, const void* gain,
                       float eps, const LayerIO& io, const LayerBufs& b, const int32_t* cont_dev, hipStream_t st);

}  // namespace dlm
