// Block attention (prefix + bidirectional block) -- internal interface.
#pragma once
#include "common.h"

namespace dlm {

struct AttnPlan {
  int chunk;       // keys per split (multiple of 32)
  int nsplit_max;  // splits per kv head at the largest prefix
};

// K/V cache storage: bf16, or FP8 e4m3 codes with one scale per cache (stored value =
// scale * e4m3(code))
struct AttnKv {
  int fp8 = 0;
  float k_scale = 1.f, v_scale = 1.f;
};

AttnPlan attn_plan(int hq, int hkv, int D, int B, int max_len);
// nqb query blocks (1, or 2 of B = 32 rows: the second block also attends to the first's keys,
// which sit at L .. L + 31; see attn.hip)
size_t attn_ws_bytes(int hq, int hkv, int D, AttnPlan pl, int nqb = 1);
// xsync (optional): barrier counters and sync words of the XCD-local split combine (xcd.h;
// zero before the first use).  With them, one query block of 32 rows and exactly 8 groups of
// (kv head, query heads of one workgroup), the splits are merged inside the attention launch
// (attn_xcd_combine_ok); otherwise, and always without them, by a second kernel.
struct AttnXSync {
  unsigned* bar = nullptr;   // 8 x 64 words
  int* err = nullptr;        // 9 x 128 bytes
};
bool attn_xcd_combine_ok(int hq, int hkv, int B, int nqb);
int attn_bf16(const void* q, const void* k, const void* v, void* out, int hq, int hkv, int D,
              int B, int nqb, int cap, float scale, const int32_t* len_dev, int len_host,
              const int32_t* cont_dev, AttnPlan pl, void* ws, int out_packed, hipStream_t st,
              AttnKv kvf = AttnKv(), AttnXSync xs = AttnXSync());
int attn_f32(const float* q, const float* k, const float* v, float* out, int hq, int hkv, int D,
             int B, int cap, float scale, const int32_t* len_dev, int len_host,
             const int32_t* cont_dev, hipStream_t st);

}  // namespace dlm
