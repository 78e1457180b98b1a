// Host side of the C ABI (include/ls_replay.h): argument validation, launch
// planning, the page-split builder and kernel timing.  Every check runs
// before the first HIP call, so a validation error means nothing was
// enqueued; LS_ERR_HIP may follow launches the same call already made.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "ls_internal.hpp"
#include "ls_replay.h"

using namespace ls;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bytes of the forward's chunk partials (o, m, l) for `units` split chunks
size_t chunk_part_bytes(const ls_attn_shape& sh, size_t units) {
  const size_t rows = (size_t)sh.num_q_heads * sh.resp_len;
  return round_up(units * rows * sh.head_dim * 4, 256) + 2 * round_up(units * rows * 4, 256);
}

// ---------------------------------------------------------------- planning
// Internal sub-splitting ("chunks") of every split so that the grid fills the
// chip: items = S * chunks * Hkv * mtiles workgroups, one per CU at a time.
// The chunk count minimises ceil(items / kTargetWGs) * pages_per_chunk, the
// critical path in page-steps of one workgroup (ties -> fewer chunks).
struct Plan {
  int chunks = 1;
  int chunk_pages = 1;
  int mtiles = 0;
  int units = 0;  // S * chunks
};

// part_cap: largest number of bytes the chunk partials may take (chunk counts
// whose partials exceed it are not considered; one chunk needs none).
Plan plan_prompt(const ls_attn_shape& sh, const ls_page_table& pt, int rows_per_wg,
                 size_t part_cap = SIZE_MAX) {
  Plan p;
  const int g = sh.num_q_heads / sh.num_kv_heads;
  const int64_t gr = (int64_t)g * sh.resp_len;
  p.mtiles = (int)((gr + rows_per_wg - 1) / rows_per_wg);
  int maxp = 0;
  for (int c = 0; c < pt.num_splits; ++c)
    maxp = std::max(maxp, pt.split_offsets_host[c + 1] - pt.split_offsets_host[c]);
  if (maxp <= 0) {
    p.chunks = 1;
    p.chunk_pages = 1;
  } else {
    const int64_t base = (int64_t)pt.num_splits * sh.num_kv_heads * p.mtiles;
    int64_t best = -1;
    for (int c = 1; c <= kMaxChunks && c <= maxp; ++c) {
      const int cp = (maxp + c - 1) / c;
      const int chunks = (maxp + cp - 1) / cp;  // chunks actually needed at this size
      if (chunks != c) continue;
      if (chunks > 1 && chunk_part_bytes(sh, (size_t)pt.num_splits * chunks) > part_cap) continue;
      const int64_t items = base * chunks;
      const int64_t cost = ((items + kTargetWGs - 1) / kTargetWGs) * cp;
      if (best < 0 || cost < best) {
        best = cost;
        p.chunks = chunks;
        p.chunk_pages = cp;
      }
    }
  }
  p.units = pt.num_splits * p.chunks;
  return p;
}

ls_status check_shape(const ls_attn_shape* sh) {
  if (!sh) return LS_ERR_INVALID_ARG;
  if (sh->num_q_heads < 1 || sh->num_kv_heads < 1 || sh->resp_len < 1 || sh->prompt_len < 0)
    return LS_ERR_INVALID_ARG;
  if (sh->num_q_heads % sh->num_kv_heads != 0) return LS_ERR_INVALID_ARG;
  if (!(sh->scale > 0.f) || !std::isfinite(sh->scale)) return LS_ERR_INVALID_ARG;
  if (sh->head_dim != 128 && sh->head_dim != 256) return LS_ERR_UNSUPPORTED;
  if (sh->page_size != kPage) return LS_ERR_UNSUPPORTED;
  const int64_t elems = (int64_t)sh->num_q_heads * sh->resp_len * sh->head_dim;
  if (elems >= (int64_t(1) << 31)) return LS_ERR_UNSUPPORTED;
  if (sh->q_offset < 0 || sh->kv_rows < 0) return LS_ERR_INVALID_ARG;
  if (sh->flags & ~LS_ACCUMULATE_KV) return LS_ERR_INVALID_ARG;
  const int64_t rk = (int64_t)sh->q_offset + sh->resp_len;
  if (sh->kv_rows != 0 && sh->kv_rows < rk) return LS_ERR_INVALID_ARG;
  const int64_t kvr = sh->kv_rows != 0 ? sh->kv_rows : rk;
  if ((int64_t)sh->num_kv_heads * kvr * sh->head_dim >= (int64_t(1) << 31)) return LS_ERR_UNSUPPORTED;
  if ((int64_t)sh->num_q_heads * rk * sh->head_dim >= (int64_t(1) << 31)) return LS_ERR_UNSUPPORTED;
  return LS_OK;
}

ls_status check_table(const ls_attn_shape* sh, const ls_page_table* pt) {
  if (!pt) return LS_ERR_INVALID_ARG;
  const int64_t need = (sh->prompt_len + kPage - 1) / kPage;
  if (pt->num_pages != need) return LS_ERR_INVALID_ARG;
  if (pt->num_splits < 1 || pt->num_phys_pages < pt->num_pages) return LS_ERR_INVALID_ARG;
  if (!pt->split_offsets_host || !pt->split_offsets) return LS_ERR_INVALID_ARG;
  if (pt->num_pages > 0 && (!pt->l2p || !pt->order)) return LS_ERR_INVALID_ARG;
  const int32_t* o = pt->split_offsets_host;
  if (o[0] != 0 || o[pt->num_splits] != pt->num_pages) return LS_ERR_INVALID_ARG;
  for (int c = 0; c < pt->num_splits; ++c)
    if (o[c + 1] < o[c]) return LS_ERR_INVALID_ARG;
  return LS_OK;
}

// ---------------------------------------------------------------- timing
struct TimingRec {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  int32_t launches = 0;
  double total_ms = 0.0;
};
bool g_timing = false;
std::map<std::string, TimingRec> g_recs;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Run one launch function, bracketed by events when timing is enabled.
template <class F>
ls_status run(const char* name, hipStream_t st, F&& f) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (g_timing) {
    e0 = take_event();
    e1 = take_event();
    if (e0 && e1) hipEventRecord(e0, st);
  }
  const hipError_t err = f();
  if (g_timing && e0 && e1) {
    hipEventRecord(e1, st);
    g_recs[name].pending.emplace_back(e0, e1);
  }
  return err == hipSuccess ? LS_OK : LS_ERR_HIP;
}

AttnArgs base_args(const ls_attn_shape& sh, const ls_page_table& pt, const void* q,
                   const void* k_pool, const void* v_pool) {
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.v = static_cast<const uint16_t*>(v_pool);
  a.l2p = pt.l2p;
  a.order = pt.order;
  a.offs = pt.split_offsets;
  a.prompt_len = sh.prompt_len;
  a.num_pages = pt.num_pages;
  a.num_phys = pt.num_phys_pages;
  a.hq = sh.num_q_heads;
  a.hkv = sh.num_kv_heads;
  a.R = sh.resp_len;
  a.qoff = sh.q_offset;
  a.RK = sh.q_offset + sh.resp_len;
  a.kvr = sh.kv_rows != 0 ? sh.kv_rows : a.RK;
  a.kv_accum = (sh.flags & LS_ACCUMULATE_KV) != 0;
  a.scale = sh.scale;
  a.s2 = sh.scale * 1.4426950408889634f;
  return a;
}

// Workspace layouts (each piece 256-byte aligned):
//   forward:  phys [num_pages] int32 | (chunks > 1) o, m, l partials per unit
//   backward: phys [num_pages] int32 | D [rows] | dQ partials [units + 1]
//             | response dV/dK partials per query head [2][g][Hkv][q_offset + R][d]
size_t phys_bytes(const ls_page_table& pt) { return round_up((size_t)pt.num_pages * 4, 256); }

size_t kv_part_bytes(const ls_attn_shape& sh) {
  return round_up((size_t)2 * sh.num_q_heads * ((size_t)sh.q_offset + sh.resp_len) * sh.head_dim * 4,
                  256);
}

size_t fwd_ws_bytes(const ls_attn_shape& sh, const ls_page_table& pt, size_t part_cap = SIZE_MAX) {
  const Plan p = plan_prompt(sh, pt, kFwdRows, part_cap);
  size_t n = phys_bytes(pt);
  if (p.chunks > 1) n += chunk_part_bytes(sh, (size_t)p.units);
  return n;
}

size_t bwd_ws_bytes(const ls_attn_shape& sh, const ls_page_table& pt) {
  const Plan p = plan_prompt(sh, pt, kBwdRows);
  const size_t rows = (size_t)sh.num_q_heads * sh.resp_len;
  const size_t slots = (size_t)p.units + 1;
  return phys_bytes(pt) + round_up(rows * 4, 256) + round_up(slots * rows * sh.head_dim * 4, 256) +
         kv_part_bytes(sh);
}

}  // namespace

size_t ls::ws_phys_bytes(const ls_page_table& pt) { return phys_bytes(pt); }

// Host checks of a forward call's shape, table and pointers (no HIP call).
ls_status ls::fwd_check_args(const ls_attn_shape* sh, const ls_page_table* pt, const void* q,
                             const void* k_pool, const void* v_pool, const void* k_resp,
                             const void* v_resp, const float* part_o, const float* part_m,
                             const float* part_l) {
  ls_status st = check_shape(sh);
  if (st != LS_OK) return st;
  if ((st = check_table(sh, pt)) != LS_OK) return st;
  if (!q || !k_resp || !v_resp || !part_o || !part_m || !part_l) return LS_ERR_INVALID_ARG;
  if (pt->num_pages > 0 && (!k_pool || !v_pool)) return LS_ERR_INVALID_ARG;
  for (const void* p : {q, k_pool, v_pool, k_resp, v_resp, (const void*)part_o,
                        (const void*)part_m, (const void*)part_l})
    if (p && !aligned16(p)) return LS_ERR_INVALID_ARG;
  return LS_OK;
}

size_t ls::fwd_ws_need(const ls_attn_shape& sh, const ls_page_table& pt, size_t part_cap) {
  return fwd_ws_bytes(sh, pt, part_cap);
}

ls_status ls::fwd_launch(const ls_attn_shape* sh, const ls_page_table* pt, int32_t nmem,
                         const int32_t* moffs_dev, const void* q, const void* k_pool,
                         const void* v_pool, const void* k_resp, const void* v_resp,
                         float* part_o, float* part_m, float* part_l, void* ws, size_t ws_bytes,
                         size_t part_cap, hipStream_t stream) {
  ls_status st = fwd_check_args(sh, pt, q, k_pool, v_pool, k_resp, v_resp, part_o, part_m, part_l);
  if (st != LS_OK) return st;
  if (ws && !aligned16(ws)) return LS_ERR_INVALID_ARG;
  const size_t need = fwd_ws_bytes(*sh, *pt, part_cap);
  if (need > 0 && (!ws || ws_bytes < need)) return LS_ERR_WORKSPACE;
  if (need == 0) ws = nullptr;

  const Plan plan = plan_prompt(*sh, *pt, kFwdRows, part_cap);
  const size_t rows = (size_t)sh->num_q_heads * sh->resp_len;
  const int d = sh->head_dim;
  AttnArgs a = base_args(*sh, *pt, q, k_pool, v_pool);
  a.chunks = plan.chunks;
  a.chunk_pages = plan.chunk_pages;
  a.mtiles = plan.mtiles;

  char* w = static_cast<char*>(ws);
  int32_t* phys = reinterpret_cast<int32_t*>(w);
  w += phys_bytes(*pt);
  a.phys = phys;
  if (pt->num_pages > 0) {
    st = run("resolve_pages", stream, [&] {
      return launch_resolve_pages(pt->num_pages, pt->num_phys_pages, pt->order, pt->l2p, phys,
                                  stream);
    });
    if (st != LS_OK) return st;
  }
  float *wo = part_o, *wm = part_m, *wl = part_l;
  if (plan.chunks > 1) {
    wo = reinterpret_cast<float*>(w);
    w += round_up((size_t)plan.units * rows * d * 4, 256);
    wm = reinterpret_cast<float*>(w);
    w += round_up((size_t)plan.units * rows * 4, 256);
    wl = reinterpret_cast<float*>(w);
  }
  // prompt splits (or their chunks)
  a.o = wo;
  a.m = wm;
  a.l = wl;
  a.slot_base = 0;
  const int grid = plan.units * sh->num_kv_heads * plan.mtiles;
  st = run("fwd_prompt", stream, [&] { return launch_fwd(a, d, false, grid, stream); });
  if (st != LS_OK) return st;
  if (plan.chunks > 1) {
    st = run("fwd_combine", stream, [&] {
      return launch_merge(pt->num_splits, plan.chunks, (int64_t)rows, d, wo, wm, wl, false,
                          part_o, part_m, part_l, stream);
    });
    if (st != LS_OK) return st;
  }
  // causal response block -> part S
  AttnArgs r = a;
  r.k = static_cast<const uint16_t*>(k_resp);
  r.v = static_cast<const uint16_t*>(v_resp);
  r.o = part_o;
  r.m = part_m;
  r.l = part_l;
  r.slot_base = pt->num_splits;
  r.moffs = nmem > 1 ? moffs_dev : nullptr;
  r.nmembers = nmem;
  r.lpt = (nmem <= 1 && sh->resp_len % kFwdRows == 0) ? 1 : 0;
  const int rgrid = sh->num_kv_heads * plan.mtiles;
  return run("fwd_resp", stream, [&] { return launch_fwd(r, d, true, rgrid, stream); });
}

namespace {

ls_status fwd_impl(const ls_attn_shape* sh, const ls_page_table* pt, int32_t nmem,
                   const int32_t* moffs_dev, const void* q, const void* k_pool,
                   const void* v_pool, const void* k_resp, const void* v_resp, float* part_o,
                   float* part_m, float* part_l, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_launch(sh, pt, nmem, moffs_dev, q, k_pool, v_pool, k_resp, v_resp, part_o, part_m,
                    part_l, ws, ws_bytes, SIZE_MAX, stream);
}

}  // namespace

extern "C" {

const char* ls_status_string(ls_status s) {
  switch (s) {
    case LS_OK: return "ok";
    case LS_ERR_INVALID_ARG: return "invalid argument";
    case LS_ERR_UNSUPPORTED: return "unsupported shape";
    case LS_ERR_PAGE_RANGE: return "page id out of range or repeated";
    case LS_ERR_WORKSPACE: return "workspace too small";
    case LS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int32_t ls_version(void) { return 102; }

ls_status ls_kv_page_table(int32_t num_pages, int32_t page_size, int64_t prompt_len,
                           const int32_t* l2p, int32_t num_phys_pages, int32_t num_splits,
                           int32_t policy, int32_t block_pages, const int32_t* owner,
                           int32_t* order_out, int32_t* split_offsets_out) {
  if (num_pages < 0 || num_splits < 1 || num_phys_pages < 0 || prompt_len < 0)
    return LS_ERR_INVALID_ARG;
  if (!split_offsets_out || (num_pages > 0 && !order_out)) return LS_ERR_INVALID_ARG;
  if (page_size != kPage) return LS_ERR_UNSUPPORTED;
  if ((prompt_len + page_size - 1) / page_size != num_pages) return LS_ERR_INVALID_ARG;
  if (policy != LS_SPLIT_CONTIGUOUS && policy != LS_SPLIT_BLOCK_CYCLIC &&
      policy != LS_SPLIT_EXPLICIT)
    return LS_ERR_INVALID_ARG;
  if (policy == LS_SPLIT_BLOCK_CYCLIC && block_pages < 1) return LS_ERR_INVALID_ARG;
  if (policy == LS_SPLIT_EXPLICIT && num_pages > 0 && !owner) return LS_ERR_INVALID_ARG;
  // the page map: in range, no physical slot used twice
  if (l2p) {
    std::vector<char> used((size_t)num_phys_pages, 0);
    for (int p = 0; p < num_pages; ++p) {
      const int32_t ph = l2p[p];
      if (ph < 0 || ph >= num_phys_pages || used[(size_t)ph]) return LS_ERR_PAGE_RANGE;
      used[(size_t)ph] = 1;
    }
  } else if (num_phys_pages < num_pages) {
    return LS_ERR_PAGE_RANGE;
  }
  // owner of every page
  std::vector<int32_t> own((size_t)num_pages);
  if (policy == LS_SPLIT_CONTIGUOUS) {
    const int a = num_pages / num_splits, b = num_pages % num_splits;
    int p = 0;
    for (int c = 0; c < num_splits; ++c)
      for (int n = 0; n < a + (c < b ? 1 : 0); ++n) own[(size_t)p++] = c;
  } else if (policy == LS_SPLIT_BLOCK_CYCLIC) {
    for (int p = 0; p < num_pages; ++p) own[(size_t)p] = (p / block_pages) % num_splits;
  } else {
    for (int p = 0; p < num_pages; ++p) {
      if (owner[p] < 0 || owner[p] >= num_splits) return LS_ERR_INVALID_ARG;
      own[(size_t)p] = owner[p];
    }
  }
  // counting sort by owner, increasing logical order inside a split
  std::vector<int32_t> count((size_t)num_splits + 1, 0);
  for (int p = 0; p < num_pages; ++p) ++count[(size_t)own[(size_t)p] + 1];
  for (int c = 0; c < num_splits; ++c) count[(size_t)c + 1] += count[(size_t)c];
  for (int c = 0; c <= num_splits; ++c) split_offsets_out[c] = count[(size_t)c];
  for (int p = 0; p < num_pages; ++p) order_out[count[(size_t)own[(size_t)p]]++] = p;
  return LS_OK;
}

size_t ls_replay_attn_fwd_workspace(const ls_attn_shape* sh, const ls_page_table* pt) {
  if (check_shape(sh) != LS_OK || check_table(sh, pt) != LS_OK) return 0;
  return fwd_ws_bytes(*sh, *pt);
}

size_t ls_replay_attn_bwd_workspace(const ls_attn_shape* sh, const ls_page_table* pt) {
  if (check_shape(sh) != LS_OK || check_table(sh, pt) != LS_OK) return 0;
  return bwd_ws_bytes(*sh, *pt);
}

ls_status ls_replay_attn_fwd(const ls_attn_shape* sh, const ls_page_table* pt, const void* q,
                             const void* k_pool, const void* v_pool, const void* k_resp,
                             const void* v_resp, float* part_o, float* part_m, float* part_l,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(sh, pt, 1, nullptr, q, k_pool, v_pool, k_resp, v_resp, part_o, part_m, part_l,
                  ws, ws_bytes, stream);
}

ls_status ls_replay_attn_fwd_members(const ls_attn_shape* sh, const ls_page_table* pt,
                                     int32_t num_members, const int32_t* member_offsets,
                                     const int32_t* member_offsets_dev, const void* q,
                                     const void* k_pool, const void* v_pool, const void* k_resp,
                                     const void* v_resp, float* part_o, float* part_m,
                                     float* part_l, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (!sh || num_members < 1 || !member_offsets) return LS_ERR_INVALID_ARG;
  if (num_members > 1 && !member_offsets_dev) return LS_ERR_INVALID_ARG;
  if (sh->q_offset != 0) return LS_ERR_INVALID_ARG;  // members are whole responses
  if (member_offsets[0] != 0 || member_offsets[num_members] != sh->resp_len)
    return LS_ERR_INVALID_ARG;
  for (int32_t k = 0; k < num_members; ++k)
    if (member_offsets[k + 1] <= member_offsets[k]) return LS_ERR_INVALID_ARG;
  return fwd_impl(sh, pt, num_members, member_offsets_dev, q, k_pool, v_pool, k_resp, v_resp,
                  part_o, part_m, part_l, ws, ws_bytes, stream);
}

ls_status ls_kv_page_append(int32_t num_kv_heads, int32_t head_dim, int32_t tokens,
                            const void* k_chunk, const void* v_chunk, const int32_t* slots_host,
                            const int32_t* slots_dev, void* k_pool, void* v_pool,
                            int32_t num_phys_pages, hipStream_t stream) {
  if (num_kv_heads < 1 || tokens < 1 || num_phys_pages < 1) return LS_ERR_INVALID_ARG;
  if (head_dim != 128 && head_dim != 256) return LS_ERR_UNSUPPORTED;
  if (!slots_host || !slots_dev) return LS_ERR_INVALID_ARG;
  for (const void* p : {k_chunk, v_chunk, static_cast<const void*>(k_pool),
                        static_cast<const void*>(v_pool)})
    if (!p || !aligned16(p)) return LS_ERR_INVALID_ARG;
  if ((int64_t)num_kv_heads * tokens * head_dim >= (int64_t(1) << 31)) return LS_ERR_UNSUPPORTED;
  const int32_t npages = (tokens + kPage - 1) / kPage;
  std::vector<char> seen(num_phys_pages, 0);
  for (int32_t p = 0; p < npages; ++p) {
    const int32_t sl = slots_host[p];
    if (sl < 0 || sl >= num_phys_pages || seen[sl]) return LS_ERR_PAGE_RANGE;
    seen[sl] = 1;
  }
  return run("page_append", stream, [&] {
    return launch_page_append(num_kv_heads, head_dim, tokens, num_phys_pages, k_chunk, v_chunk,
                              slots_dev, k_pool, v_pool, stream);
  });
}

ls_status ls_lse_merge(int32_t num_parts, int64_t rows, int32_t head_dim, const float* part_o,
                       const float* part_m, const float* part_l, void* o_bf16, float* lse,
                       hipStream_t stream) {
  if (num_parts < 1 || rows < 1) return LS_ERR_INVALID_ARG;
  if (head_dim != 128 && head_dim != 256) return LS_ERR_UNSUPPORTED;
  if (!part_o || !part_m || !part_l || !o_bf16 || !lse) return LS_ERR_INVALID_ARG;
  for (const void* p : {(const void*)part_o, (const void*)part_m, (const void*)part_l,
                        (const void*)o_bf16, (const void*)lse})
    if (!aligned16(p)) return LS_ERR_INVALID_ARG;
  if (rows >= (int64_t(1) << 31) / head_dim) return LS_ERR_UNSUPPORTED;
  return run("lse_merge", stream, [&] {
    return launch_merge(1, num_parts, rows, head_dim, part_o, part_m, part_l, true, o_bf16, lse,
                        nullptr, stream);
  });
}

ls_status ls_replay_attn_bwd(const ls_attn_shape* sh, const ls_page_table* pt, const void* q,
                             const void* k_pool, const void* v_pool, const void* k_resp,
                             const void* v_resp, const void* o, const float* lse,
                             const void* d_o, float* dq, float* dk_resp, float* dv_resp,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  ls_status st = check_shape(sh);
  if (st != LS_OK) return st;
  if ((st = check_table(sh, pt)) != LS_OK) return st;
  if (!q || !k_resp || !v_resp || !o || !lse || !d_o || !dq || !dk_resp || !dv_resp)
    return LS_ERR_INVALID_ARG;
  if (pt->num_pages > 0 && (!k_pool || !v_pool)) return LS_ERR_INVALID_ARG;
  for (const void* p : {q, k_pool, v_pool, k_resp, v_resp, o, (const void*)lse, d_o,
                        (const void*)dq, (const void*)dk_resp, (const void*)dv_resp,
                        (const void*)ws})
    if (p && !aligned16(p)) return LS_ERR_INVALID_ARG;
  const size_t need = bwd_ws_bytes(*sh, *pt);
  if (!ws || ws_bytes < need) return LS_ERR_WORKSPACE;

  const Plan plan = plan_prompt(*sh, *pt, kBwdRows);
  const size_t rows = (size_t)sh->num_q_heads * sh->resp_len;
  const int d = sh->head_dim;
  char* w = static_cast<char*>(ws);
  int32_t* phys = reinterpret_cast<int32_t*>(w);
  w += phys_bytes(*pt);
  float* dvals = reinterpret_cast<float*>(w);
  float* slots = reinterpret_cast<float*>(w + round_up(rows * 4, 256));
  float* kv_part = reinterpret_cast<float*>(w + round_up(rows * 4, 256) +
                                            round_up(((size_t)plan.units + 1) * rows * d * 4, 256));

  AttnArgs a = base_args(*sh, *pt, q, k_pool, v_pool);
  a.chunks = plan.chunks;
  a.chunk_pages = plan.chunk_pages;
  a.mtiles = plan.mtiles;
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.dvals = dvals;
  a.dq_slots = slots;
  a.dk = dk_resp;
  a.dv = dv_resp;
  a.kv_part = kv_part;
  a.phys = phys;

  if (pt->num_pages > 0) {
    st = run("resolve_pages", stream, [&] {
      return launch_resolve_pages(pt->num_pages, pt->num_phys_pages, pt->order, pt->l2p, phys,
                                  stream);
    });
    if (st != LS_OK) return st;
  }
  st = run("bwd_dot", stream, [&] {
    return launch_bwd_dot((int64_t)rows, d, a.d_o, static_cast<const uint16_t*>(o), dvals, stream);
  });
  if (st != LS_OK) return st;
  a.slot_base = 0;
  const int grid = plan.units * sh->num_kv_heads * plan.mtiles;
  st = run("bwd_prompt_dq", stream, [&] { return launch_bwd_dq(a, d, false, grid, stream); });
  if (st != LS_OK) return st;
  AttnArgs r = a;
  r.k = static_cast<const uint16_t*>(k_resp);
  r.v = static_cast<const uint16_t*>(v_resp);
  r.slot_base = plan.units;
  r.lpt = (sh->resp_len % kBwdRows == 0) ? 1 : 0;
  const int rgrid = sh->num_kv_heads * plan.mtiles;
  st = run("bwd_resp_dq", stream, [&] { return launch_bwd_dq(r, d, true, rgrid, stream); });
  if (st != LS_OK) return st;
  st = run("bwd_resp_dkdv", stream, [&] { return launch_bwd_dkdv(r, d, stream); });
  if (st != LS_OK) return st;
  st = run("kv_reduce", stream, [&] {
    return launch_kv_reduce(sh->num_q_heads / sh->num_kv_heads, sh->num_kv_heads, r.RK, r.kvr, d,
                            r.kv_accum != 0, kv_part, dv_resp, dk_resp, stream);
  });
  if (st != LS_OK) return st;
  return run("dq_reduce", stream, [&] {
    return launch_dq_reduce(plan.units + 1, (int64_t)rows * d, slots, dq, stream);
  });
}

ls_status ls_timing_enable(int32_t on) {
  g_timing = on != 0;
  return LS_OK;
}

ls_status ls_timing_reset(void) {
  for (auto& kv : g_recs) {
    for (auto& pr : kv.second.pending) {
      hipEventSynchronize(pr.second);
      g_free_events.push_back(pr.first);
      g_free_events.push_back(pr.second);
    }
    kv.second = TimingRec();
  }
  return LS_OK;
}

ls_status ls_timing_read(const char* kernel, int32_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return LS_ERR_INVALID_ARG;
  auto it = g_recs.find(kernel);
  if (it == g_recs.end()) {
    *launches = 0;
    *total_ms = 0.0;
    return LS_OK;
  }
  TimingRec& rec = it->second;
  for (auto& pr : rec.pending) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return LS_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return LS_ERR_HIP;
    rec.total_ms += ms;
    rec.launches += 1;
    g_free_events.push_back(pr.first);
    g_free_events.push_back(pr.second);
  }
  rec.pending.clear();
  *launches = rec.launches;
  *total_ms = rec.total_ms;
  return LS_OK;
}

}  // extern "C"
