// Internal declarations shared by the host API (ls_api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "ls_replay.h"

namespace ls {

constexpr int kPage = 256;       // prompt tokens per page (only size supported)
constexpr int kBN = 32;          // keys per inner block (one 32-row MFMA tile)
constexpr int kFwdWaves = 8;     // waves per forward workgroup (two per SIMD)
constexpr int kFwdRows = 32 * kFwdWaves;  // query rows per forward workgroup (32 per wave)
constexpr int kBwdRows = 128;    // query rows per dQ workgroup (4 score + 4 dQ waves, 32 rows each)
constexpr int kTargetWGs = 256;  // one workgroup per CU on MI355X (256 CUs)
constexpr int kMaxChunks = 64;   // cap on internal sub-splits per split
constexpr int kStages = 4;       // LDS ring depth of K/V blocks in the key loops

// Source of keys for one launch: the paged prompt pool (via the page table) or
// the contiguous response K/V (causal).
struct AttnArgs {
  const uint16_t* q;      // bf16 [Hq, R, d]
  const uint16_t* k;      // bf16 pool [phys, Hkv, 256, d]  or response [Hkv, R, d]
  const uint16_t* v;
  const int32_t* l2p;     // device page map (paged only)
  const int32_t* order;   // device split-major page list (paged only)
  const int32_t* offs;    // device split offsets (paged only)
  const int32_t* phys;    // device physical slot of each page of `order` (-1: bad id)
  const int32_t* moffs;   // device member row offsets [nmembers + 1] (response block;
  int32_t nmembers;       //   null: one member): keys are visible only inside a member
  int64_t prompt_len;
  int32_t num_pages, num_phys, chunks, chunk_pages;
  int32_t hq, hkv, R, mtiles;
  // response keys: the rows are response tokens qoff .. qoff+R-1 and see keys
  // j <= qoff + i; k/v (response) and dk/dv have kvr rows per KV head, of
  // which the first RK = qoff + R are used; kv_accum: dk/dv += instead of =
  int32_t qoff, RK, kvr, kv_accum;
  // causal response block whose tiles each stay inside one query head (R a
  // multiple of the tile rows, one member): dispatch the tiles longest key
  // range first (lpt != 0)
  int32_t lpt;
  float s2;               // scale * log2(e)
  float scale;
  // forward outputs (slot arrays): o [slots, Hq*R, d], m/l [slots, Hq*R]
  float* o;
  float* m;
  float* l;
  int32_t slot_base;
  // backward inputs/outputs
  const uint16_t* d_o;    // bf16 [Hq, R, d]
  const float* lse;       // fp32 [Hq, R]
  const float* dvals;     // fp32 [Hq, R]  D = <dO, O>
  float* dq_slots;        // fp32 [slots, Hq*R, d]
  float* dk;              // fp32 [Hkv, R, d]
  float* dv;
  float* kv_part;         // fp32 [2][g][Hkv][RK][d] per-query-head dV (0) / dK (1) partials
};

// Host checks of a forward call's shape, table and pointers (no HIP call);
// the workspace bytes a forward needs when the chunk partials of its launch
// plan may take at most part_cap bytes (SIZE_MAX: the plan that fills the
// chip); and the checked forward under that cap.
ls_status fwd_check_args(const ls_attn_shape* sh, const ls_page_table* pt, const void* q,
                         const void* k_pool, const void* v_pool, const void* k_resp,
                         const void* v_resp, const float* part_o, const float* part_m,
                         const float* part_l);
size_t fwd_ws_need(const ls_attn_shape& sh, const ls_page_table& pt, size_t part_cap);
ls_status fwd_launch(const ls_attn_shape* sh, const ls_page_table* pt, int32_t nmem,
                     const int32_t* moffs_dev, const void* q, const void* k_pool, const void* v_pool,
                     const void* k_resp, const void* v_resp, float* part_o, float* part_m,
                     float* part_l, void* ws, size_t ws_bytes, size_t part_cap, hipStream_t stream);
// bytes of the resolved page list at the start of a workspace
size_t ws_phys_bytes(const ls_page_table& pt);

hipError_t launch_fwd(const AttnArgs& a, int head_dim, bool resp, int grid, hipStream_t s);
hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, bool resp, int grid, hipStream_t s);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t s);
// dv[kv][j] (=, or += when accum) sum_h kv_part[0][h][kv][j], dk likewise from
// kv_part[1], heads in order; j < rk, output rows strided by kvr
hipError_t launch_kv_reduce(int g, int hkv, int rk, int kvr, int head_dim, bool accum,
                            const float* part, float* dv, float* dk, hipStream_t s);

// Merge `nper` consecutive parts per group: group c reads parts
// [c*nper, (c+1)*nper).  final=true writes bf16 O and natural-log LSE;
// final=false writes a combined fp32 partial (o, m, l) per group.
hipError_t launch_merge(int groups, int nper, int64_t rows, int head_dim, const float* po,
                        const float* pm, const float* pl, bool final, void* out_o,
                        float* out_m, float* out_l, hipStream_t s);
hipError_t launch_bwd_dot(int64_t rows, int head_dim, const uint16_t* d_o, const uint16_t* o,
                          float* dvals, hipStream_t s);
// phys[i] = l2p[order[i]] for i < num_pages, -1 where either id is out of range.
hipError_t launch_resolve_pages(int32_t num_pages, int32_t num_phys, const int32_t* order,
                                const int32_t* l2p, int32_t* phys, hipStream_t s);
hipError_t launch_page_append(int hkv, int head_dim, int tokens, int num_phys,
                              const void* k_chunk, const void* v_chunk, const int32_t* slots,
                              void* k_pool, void* v_pool, hipStream_t s);
hipError_t launch_dq_reduce(int nslots, int64_t elems, const float* slots, float* dq,
                            hipStream_t s);

}  // namespace ls
