// Skinny GEMM (M <= 64 block rows) with fused epilogues -- internal interface.
#pragma once
#include "common.h"

namespace dlm {

enum EpiKind {
  EPI_STORE_F32 = 0,   // out[m][n] = acc
  EPI_RESID = 1,       // out[m][n] += acc            (residual stream, f32)
  EPI_QKV_ROPE = 2,    // q/k rotated at position L + m, q -> q_out, k/v -> caches at row L + m
  EPI_SWIGLU = 3,      // act[m][j] = silu(gate_j) * up_j
  EPI_SELFCOND = 4,    // out[m][n] = committed[m] ? E[tok[m]][n] : mask[n] + acc
  EPI_PARTIAL = 5,     // deferred: each workgroup stores its partial sums; a consumer adds them
};

// Where a deferred GEMM left its partial sums: tile t (32 output columns) has contributors
// c = 0 .. cnt(t)-1, with cnt(t) from the stream-K split (see contributors()), and value
// (m, n) of contributor c at base[(t * cmax + c) * mstride + m * 32 + n % 32], where
// mstride = 32 x (the GEMM's row count rounded up to 32).  A consumer that works on rows
// row0 .. of the GEMM's rows reads its row r as GEMM row row0 + r.
struct PartialSrc {
  const float* base;   // nullptr: no partials
  int tiles, KT, NW, cmax, mstride, row0;
  size_t bytes;        // size of the partial area
  // alternatively (base == nullptr): per-row output slots, value (m, n) of slot j at
  // slots[(m * nslot + j) * d + n], added in slot order (routed experts)
  const float* slots;
  int nslot;
};

// Logical row orders of the fused matrices (packed row order is described in gemm.hip):
//   QKV: rows [0, hq*D) = Wq, then Wk (hkv*D rows), then Wv (hkv*D rows).
//   GU:  rows [0, F) = Wg, then Wu.
enum RowMapKind { MAP_IDENTITY = 0, MAP_QKV = 1, MAP_GU = 2 };

struct EpiParams {
  int kind;
  int M;                  // valid activation rows (<= 64; more than 32 only for the row-owned
                          // kinds and EPI_PARTIAL)
  int bf16_out;           // activations / caches are bf16 (else f32)
  // f32 outputs
  float* out;             // STORE_F32 / RESID / SELFCOND: [M, ld_out]
  int ld_out;
  // QKV
  void* q_out;            // [M, hq*D]
  void* k_cache;          // [hkv, cap, D]
  void* v_cache;
  int hq, hkv, D, cap;
  const int32_t* len_dev; // prefix length L (device) ...
  int len_host;           // ... or host value when len_dev == nullptr
  double rope_r;          // base^(-2/D)
  int kv8;                // the caches hold FP8 e4m3 codes of (bf16 value) / k_scale (v_scale)
  float k_scale, v_scale;
  // SWIGLU
  void* act_out;          // [M, F]
  int F;
  // SELFCOND
  const void* mask_emb;   // [d] (model dtype)
  const void* emb;        // [V, d]
  const int32_t* tokens;
  const uint8_t* committed;
  int vocab;
  // predication: when non-null and *cont_dev == 0 the kernel does nothing
  const int32_t* cont_dev;
};

struct GemmPlan {
  int tpw;      // (unused, 1)
  int splits;   // number of workgroups
  int R;        // row-owned mode: output rows per workgroup (weights packed for it); 0: stream-K
};

// Packed-row -> logical-row map used when packing (host side).
void build_row_map(int kind, int n_rows, int hq, int hkv, int D, int F, int32_t* out);

// bf16 path.  W: packed [N, K] (N % 32 == 0, K % 16 == 0); X: bf16, M <= 32 rows as one
// 32 x K panel in the packed operand order (xpk_index; rows >= M are read but ignored), or
// 32 < M <= 64 rows as two such panels (xpk_index_m).  The SwiGLU epilogue writes its bf16
// output in the same packed order (it feeds the down projection).
// partial/counters: workspace (counters zero before the first use; left zero); mrows: the
// largest M the workspace serves.
size_t gemm_ws_bytes(int N, int K, GemmPlan plan, int mrows = 32);
GemmPlan gemm_plan(int N, int K);
// Row-owned plan when N splits into equal even row blocks over enough workgroups (the weights
// must then be packed with pack_bf16_owned and this plan's R), else the stream-K plan.
GemmPlan gemm_plan_owned(int N, int K);
int gemm_bf16(const void* W, const void* X, int N, int K, int map_kind, const EpiParams& ep,
              GemmPlan plan, void* ws, hipStream_t st);
// Partial sums left in ws by a gemm_bf16 call with kind EPI_PARTIAL (valid until the next GEMM
// on the same workspace).
PartialSrc gemm_partials(int N, int K, GemmPlan plan, void* ws, int M = 32);

// f32 path (natural [out, in] weights).  Up to 3 source matrices make the logical rows.
struct F32Mats {
  const float* w[3];
  int rows[3];
};
int gemm_f32(const F32Mats& W, const float* X, int N, int K, int map_kind, const EpiParams& ep,
             hipStream_t st);

// Pack rows row_map[i] of the virtual concatenation of up to 3 bf16 matrices into dst.
int pack_bf16(const void* const* srcs, const int* src_rows, int n_src, int n_rows, int k,
              const int32_t* row_map_dev, void* dst, hipStream_t st);
// The same rows in the row-owned layout of a plan with R rows per workgroup.  ld: row stride
// of the sources in elements (0: k); with ld > k the k columns at each source pointer are a
// column slice of a wider matrix.
int pack_bf16_owned(const void* const* srcs, const int* src_rows, int n_src, int n_rows, int k,
                    const int32_t* row_map_dev, int R, void* dst, hipStream_t st, int ld = 0);

}  // namespace dlm
