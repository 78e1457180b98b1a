/*
 * ls_replay.h -- C ABI of the response-replay attention library (MI355X, gfx950).
 *
 * The operator: exact attention of one short response branch (R rows, causal
 * within the response) over a long, detached prompt whose K/V live in fixed
 * size pages, for a grouped-query attention layer (Hq query heads sharing Hkv
 * K/V heads).  This is the full-attention layer of the LongStraw "Qwen path":
 * compact prompt K/V pages owned by context-parallel ranks, a global
 * log-sum-exp merge of the per-rank partial attention, and a response-only
 * backward that all-reduces only the query gradient (LongStraw review page,
 * section 2 "core method", items 2-3, and the section 7 mind map,
 * "Qwen3.6-27B implementation"; LongStraw abstract on cortexa.online: exact
 * attention composition, response-only objective, detached prompt state).
 *
 * On one GPU each context-parallel rank is emulated by a "split": a list of
 * prompt pages.  The forward writes one partial (max-shift m, sum-exp l,
 * normalised output o) per split plus one for the causal response block;
 * ls_lse_merge composes them exactly.  The backward returns dQ (over prompt and
 * response keys, summed over splits in a fixed order) and dK/dV for the
 * response keys only.  No prompt K/V gradient exists anywhere in this API: the
 * prompt state is stopgrad (DeepRead summary page, "Method").
 *
 * Conventions for every call
 *   - Pointers marked "device" are HIP device pointers; "host" are CPU memory.
 *   - The caller allocates and owns every buffer, including workspaces.  The
 *     library allocates no device memory and keeps no pointer after a call
 *     returns.  Prompt pools are read-only: nothing ever writes them.
 *   - Device pointers must be 16-byte aligned; tensors are dense row-major in
 *     the layouts stated below.  bf16 = IEEE bfloat16 (1-8-7).
 *   - GPU work is enqueued asynchronously on `stream` (0 = null stream).  A
 *     device fault surfaces at the caller's next synchronisation.
 *   - All argument checks happen before any HIP call: a call that returns
 *     LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_PAGE_RANGE or
 *     LS_ERR_WORKSPACE has enqueued nothing.  LS_ERR_HIP reports a failed
 *     launch or runtime call and may follow launches the same call already
 *     enqueued; the outputs are then undefined.
 *   - Supported: head_dim in {128, 256}; page_size == 256; Hq % Hkv == 0;
 *     resp_len >= 1; prompt_len >= 0; Hq*resp_len*head_dim < 2^31;
 *     Hkv*kv_rows*head_dim < 2^31.
 */
#ifndef LS_REPLAY_H
#define LS_REPLAY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ls_status {
  LS_OK = 0,
  LS_ERR_INVALID_ARG = -1, /* null pointer, bad count, misaligned pointer     */
  LS_ERR_UNSUPPORTED = -2, /* head_dim / page_size / shape this build lacks  */
  LS_ERR_PAGE_RANGE = -3,  /* page id out of range or physical page reused   */
  LS_ERR_WORKSPACE = -4,   /* workspace smaller than the size query returned */
  LS_ERR_HIP = -5          /* a HIP launch or runtime call failed            */
} ls_status;

/* Page-split policies for ls_kv_page_table (one split = one emulated
 * context-parallel rank). */
enum {
  LS_SPLIT_CONTIGUOUS = 0,  /* S consecutive page ranges, sizes differ by <= 1, longer first */
  LS_SPLIT_BLOCK_CYCLIC = 1,/* logical page p -> split (p / block_pages) % S (the pages' CP8 rule) */
  LS_SPLIT_EXPLICIT = 2     /* logical page p -> split owner[p] */
};

/* Flags of ls_attn_shape.flags. */
enum {
  LS_ACCUMULATE_KV = 1  /* ls_replay_attn_bwd adds into dk_resp / dv_resp instead of writing */
};

/* Shape of one replay-attention call.
 *   num_q_heads  Hq;  num_kv_heads Hkv, Hq % Hkv == 0; query head h reads
 *                K/V head h / (Hq/Hkv) (contiguous GQA groups).
 *   head_dim     d in {128, 256}.
 *   page_size    prompt tokens per page; must be 256.
 *   prompt_len   P >= 0 prompt positions; all are visible to every response row.
 *   resp_len     R >= 1 response rows; row i sees response keys 0..q_offset+i.
 *   scale        softmax scale applied to q.k (normally 1/sqrt(d)).
 *   q_offset     >= 0.  0 for a whole response.  Otherwise the R rows are the
 *                response tokens q_offset .. q_offset+R-1, one token block of
 *                a longer response replayed on its own (the pages replay a
 *                response in four blocks, in reverse; LongStraw review page,
 *                section 7 mind map, and the cortexa abstract): the response
 *                keys are its first q_offset + R tokens.
 *   kv_rows      rows per KV head of k_resp, v_resp, dk_resp and dv_resp
 *                ([Hkv, kv_rows, d]); 0 means q_offset + R, else it must be
 *                >= q_offset + R and rows past q_offset + R are neither read
 *                nor written (so one buffer of the whole response serves
 *                every block).
 *   flags        0 or LS_ACCUMULATE_KV.
 * Zero-initialising the last three fields gives the whole-response call. */
typedef struct ls_attn_shape {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int64_t prompt_len;
  int32_t resp_len;
  float scale;
  int32_t q_offset;
  int32_t kv_rows;
  int32_t flags;
} ls_attn_shape;

/* Page table of one prompt, as built by ls_kv_page_table and copied to the
 * device by the caller.
 *   l2p                 device int32 [num_pages]: logical page -> physical slot
 *                       in the pools (slots in [0, num_phys_pages), no repeats).
 *   order               device int32 [num_pages]: logical page ids, split-major.
 *   split_offsets       device int32 [num_splits + 1]: CSR offsets into order.
 *   split_offsets_host  host copy of split_offsets (used to size the launch).
 * Logical page p holds prompt positions [p*page_size, (p+1)*page_size); only
 * the last page may be partial (positions >= prompt_len are masked).  The
 * kernels trust the device copies to match what ls_kv_page_table validated;
 * a corrupted device table gives wrong values but never an out-of-bounds
 * access (a page whose id is out of range is read as pool block 0 by the
 * unmasked key loop and skipped by the masked one). */
typedef struct ls_page_table {
  const int32_t* l2p;
  const int32_t* order;
  const int32_t* split_offsets;
  const int32_t* split_offsets_host;
  int32_t num_pages;
  int32_t num_splits;
  int32_t num_phys_pages;
} ls_page_table;

/* Text for a status code (static storage; never NULL). */
const char* ls_status_string(ls_status status);

/* Library ABI version (major*100 + minor). */
int32_t ls_version(void);

/* ls_kv_page_table -- host only, pure (no HIP call).
 * Validates the logical->physical page map of one prompt and deals its pages
 * to num_splits splits (emulated context-parallel ranks; LongStraw review page,
 * section 7 mind map: CP8 page ownership, block-cyclic).  Inside a split pages
 * are listed in increasing logical order.
 *   num_pages           >= 0, must equal ceil(prompt_len / page_size).
 *   page_size           256.
 *   logical_to_physical host [num_pages] or NULL (= identity, then
 *                       num_phys_pages >= num_pages).
 *   num_phys_pages      pool slots; every map entry must lie in [0, num_phys_pages)
 *                       and no slot may appear twice (a compact page is its own
 *                       allocation, never a view shared with another page).
 *   num_splits          >= 1.
 *   policy              LS_SPLIT_*; block_pages >= 1 is used by BLOCK_CYCLIC;
 *                       owner (host [num_pages], values in [0, num_splits)) by
 *                       EXPLICIT, else ignored (may be NULL).
 *   order_out           host [num_pages]    (written on success).
 *   split_offsets_out   host [num_splits+1] (written on success).
 * Errors: LS_ERR_INVALID_ARG (counts, NULL outputs, prompt_len inconsistent
 * with num_pages, unknown policy, bad owner), LS_ERR_UNSUPPORTED (page_size),
 * LS_ERR_PAGE_RANGE (map entry out of range or repeated).  Splits may be empty. */
ls_status ls_kv_page_table(int32_t num_pages, int32_t page_size, int64_t prompt_len,
                           const int32_t* logical_to_physical, int32_t num_phys_pages,
                           int32_t num_splits, int32_t policy, int32_t block_pages,
                           const int32_t* owner, int32_t* order_out,
                           int32_t* split_offsets_out);

/* Workspace bytes the forward / backward need for this shape and table
 * (0 on invalid arguments).  Pure host functions. */
size_t ls_replay_attn_fwd_workspace(const ls_attn_shape* shape, const ls_page_table* pt);
size_t ls_replay_attn_bwd_workspace(const ls_attn_shape* shape, const ls_page_table* pt);

/* ls_replay_attn_fwd -- per-split partial attention (the forward of one
 * replayed response; LongStraw review page, section 7 mind map: forward
 * composition by global LSE over CP ranks).
 * For every row (h, i) (row index h*R + i) and every part c in [0, S]:
 *   parts c < S   cover the prompt pages of split c (all positions visible);
 *   part  c == S  covers the response keys j <= q_offset + i (causal, diagonal
 *                 included).
 *   x_j = scale * <q[h,i], k_j>;  part_m[c,row] = m, part_l[c,row] = sum_j exp(x_j - m),
 *   part_o[c,row,:] = sum_j exp(x_j - m) v_j / part_l[c,row].
 * m is a shift chosen by the kernel, the largest score of the split's first
 * key block, or the split's maximum when a later score exceeds that by more
 * than 32*ln2: so max_j x_j - 32*ln2 <= m <= max_j x_j (32*ln2 ~ 22.2), up to
 * fp32 rounding, and l <= 2^32 * (number of keys).  The pair (m, l) is what
 * is defined: m + ln l is the split's log-sum-exp.  An empty split gives
 * m = -inf, l = 0, o = 0.
 *   q                 device bf16 [Hq, R, d]
 *   k_pool, v_pool    device bf16 [num_phys_pages, Hkv, page_size, d]
 *   k_resp, v_resp    device bf16 [Hkv, kv_rows, d] (rows < q_offset + R are read)
 *   part_o            device fp32 [S+1, Hq, R, d]
 *   part_m, part_l    device fp32 [S+1, Hq, R]
 *   workspace         device, >= ls_replay_attn_fwd_workspace() bytes (may be
 *                     NULL when that is 0).
 * Errors: LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP. */
ls_status ls_replay_attn_fwd(const ls_attn_shape* shape, const ls_page_table* pt,
                             const void* q, const void* k_pool, const void* v_pool,
                             const void* k_resp, const void* v_resp,
                             float* part_o, float* part_m, float* part_l,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ls_replay_attn_fwd_members -- the same forward for a group of G response
 * branches of one prompt in a single pass over the prompt pages (graph-free
 * scoring of the whole group: the pages score every member against the one
 * captured prompt before the per-member replay; DeepRead summary page,
 * "Method"; LongStraw review page, section 2, item 3).  Members are stacked
 * along the response axis: member k owns response rows
 * [member_offsets[k], member_offsets[k+1]) of every head, so q is
 * [Hq, R, d], k_resp / v_resp are [Hkv, R, d] and the partials are laid out
 * exactly as for ls_replay_attn_fwd with R = shape->resp_len = the total.
 * Every prompt key is visible to every row; response key j is visible to row
 * i only when both lie in the same member and j <= i.  Part S is the response
 * block, parts c < S the prompt splits, as above; ls_lse_merge then gives each
 * member's O and LSE in its rows.
 *   num_members          G >= 1
 *   member_offsets       host int32 [G+1]: 0 = offs[0] < offs[1] < ... < offs[G] = R
 *   member_offsets_dev   device copy of member_offsets (may be NULL when G == 1)
 * Other arguments, workspace and errors as ls_replay_attn_fwd; offsets that
 * are not strictly increasing from 0 to R, or a nonzero q_offset, give
 * LS_ERR_INVALID_ARG. */
ls_status ls_replay_attn_fwd_members(const ls_attn_shape* shape, const ls_page_table* pt,
                                     int32_t num_members, const int32_t* member_offsets,
                                     const int32_t* member_offsets_dev, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const void* k_resp, const void* v_resp,
                                     float* part_o, float* part_m, float* part_l,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Bytes of the device scratch ls_replay_attn_fwd_noalloc uses (64 MiB). */
#define LS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ls_replay_attn_fwd_noalloc -- ls_replay_attn_fwd without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Neither this call nor anything it calls allocates memory.
 *   Arguments, layouts, outputs and errors are those of ls_replay_attn_fwd
 *   without workspace / workspace_bytes.
 *   The workspace is the library's own static device array of
 *   LS_NOALLOC_SCRATCH_BYTES; each GPU the library runs on holds one copy
 *   until the process ends.  The first call on a device looks up its address
 *   (host side, once per device).
 *   The launch plan keeps its internal sub-split partials within the scratch:
 *   where ls_replay_attn_fwd would use more, this call uses fewer sub-splits
 *   (same result up to fp32 rounding order, possibly slower).
 *   LS_ERR_WORKSPACE: the prompt's resolved page list (4 bytes per page,
 *   rounded up to 256) does not fit in the scratch (over ~16.7M pages).
 *   Every call on a GPU shares that GPU's scratch, which keeps the last call's
 *   contents: calls that overlap on one GPU (two streams, two host threads)
 *   race, and the caller must order them.  Nothing in the scratch needs to
 *   start at zero: a call reads only bytes it wrote earlier in the same call. */
ls_status ls_replay_attn_fwd_noalloc(const ls_attn_shape* shape, const ls_page_table* pt,
                                     const void* q, const void* k_pool, const void* v_pool,
                                     const void* k_resp, const void* v_resp, float* part_o,
                                     float* part_m, float* part_l, hipStream_t stream);

/* ls_kv_page_append -- the capture-side page writer: stores the K and V of
 * T freshly prefilled prompt tokens as compact pages of the pool (the shared
 * prompt is prefilled once without a graph and only the per-token K/V of the
 * full-attention layers is kept, in pages; DeepRead summary page, "Method";
 * LongStraw review page, section 2, items 1 and 2; the prefill runs in
 * 4096-token chunks, LongStraw review page, section 3).  The chunk's first
 * token is the first row of a page, so token t of the chunk lands in pool
 * slot slots[t / 256], row t % 256, for every KV head:
 *   k_pool[slots[t/256], h, t%256, :] = k_chunk[h, t, :]   (same for v).
 * Rows of the chunk's last page past T are left untouched (the page table's
 * prompt_len masks them).
 *   num_kv_heads    Hkv >= 1;  head_dim d in {128, 256};  tokens T >= 1
 *   k_chunk, v_chunk   device bf16 [Hkv, T, d], 16-byte aligned
 *   slots_host      host int32 [ceil(T/256)]: pool slot of each new page
 *   slots_dev       device copy of slots_host (read by the kernel)
 *   k_pool, v_pool  device bf16 [num_phys_pages, Hkv, 256, d], 16-byte aligned
 *   num_phys_pages  pool slots; every slot must lie in [0, num_phys_pages)
 *                   and appear once (a compact page is its own allocation).
 * Nothing is allocated; the copy is enqueued on stream.  The caller records
 * the new pages in the logical->physical map it passes to ls_kv_page_table.
 * Errors: LS_ERR_INVALID_ARG (counts, NULL or misaligned pointers),
 * LS_ERR_UNSUPPORTED (d, or Hkv*T*d >= 2^31), LS_ERR_PAGE_RANGE (slot out of
 * range or repeated), LS_ERR_HIP. */
ls_status ls_kv_page_append(int32_t num_kv_heads, int32_t head_dim, int32_t tokens,
                            const void* k_chunk, const void* v_chunk, const int32_t* slots_host,
                            const int32_t* slots_dev, void* k_pool, void* v_pool,
                            int32_t num_phys_pages, hipStream_t stream);

/* ls_lse_merge -- exact composition of partial attention (the pages' global
 * LSE/output merge of the CP8 shards; LongStraw review page, section 7 mind map).
 * For each row: M = max_c m_c, w_c = l_c * exp(m_c - M), L = sum_c w_c,
 *   o[row,:] = bf16_rne( sum_c w_c * part_o[c,row,:] / L ),  lse[row] = M + ln L.
 * Parts are combined in index order; the result does not depend on how the
 * keys were partitioned.  A row with L == 0 gets o = 0, lse = -inf.
 *   num_parts >= 1; rows >= 1; head_dim in {128, 256}
 *   part_o  device fp32 [num_parts, rows, head_dim]; part_m, part_l [num_parts, rows]
 *   o_bf16  device bf16 [rows, head_dim];  lse device fp32 [rows] (natural log).
 * Errors: LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_HIP. */
ls_status ls_lse_merge(int32_t num_parts, int64_t rows, int32_t head_dim,
                       const float* part_o, const float* part_m, const float* part_l,
                       void* o_bf16, float* lse, hipStream_t stream);

/* ls_replay_attn_bwd -- response-only backward of the replayed response.
 * With P = exp(x - lse) recomputed from the saved natural-log lse and
 * D = <dO, O> over the stored bf16 O:
 *   dq[h,i,:]      = scale * sum_j P_ij (<dO_i, v_j> - D_i) k_j   over prompt AND
 *                    response keys; the per-split terms are summed in split
 *                    order, the response term last (this replaces the pages'
 *                    dQ all-reduce across CP ranks; LongStraw review page,
 *                    section 2: only the query gradient is all-reduced);
 *   dk_resp[kv,j,:] = scale * sum_{h in group kv} sum_{i : q_offset+i >= j} dS_ij q[h,i,:]
 *   dv_resp[kv,j,:] =         sum_{h in group kv} sum_{i : q_offset+i >= j} P_ij  dO[h,i,:]
 * for the response keys j < q_offset + R: the contribution of these R rows
 * (all of dK_r, dV_r for a whole response).  With LS_ACCUMULATE_KV it is added
 * to what dk_resp / dv_resp hold, so the blocks of a response replayed one
 * after another sum to the whole response's gradient.
 * No gradient of the prompt K/V is formed (stopgrad; DeepRead summary,
 * "Method"), and the pools are never written.
 *   q, d_o, o      device bf16 [Hq, R, d] (o as written by ls_lse_merge)
 *   lse            device fp32 [Hq, R]
 *   k_pool, v_pool, k_resp, v_resp as in the forward
 *   dq             device fp32 [Hq, R, d]
 *   dk_resp, dv_resp device fp32 [Hkv, kv_rows, d]; rows >= q_offset + R untouched
 *   workspace      device, >= ls_replay_attn_bwd_workspace() bytes.
 * Errors: LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP. */
ls_status ls_replay_attn_bwd(const ls_attn_shape* shape, const ls_page_table* pt,
                             const void* q, const void* k_pool, const void* v_pool,
                             const void* k_resp, const void* v_resp,
                             const void* o, const float* lse, const void* d_o,
                             float* dq, float* dk_resp, float* dv_resp,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Kernel timing (measurement aid).  While enabled, every kernel the library
 * launches is bracketed by a pair of hipEvents recorded on the launch stream.
 * ls_timing_read synchronises those events and returns, for the named kernel,
 * the number of launches and their summed duration since the last reset.
 * Kernel names: "resolve_pages", "fwd_prompt", "fwd_combine", "fwd_resp",
 * "lse_merge", "bwd_dot", "bwd_prompt_dq", "bwd_resp_dq", "bwd_resp_dkdv",
 * "kv_reduce", "dq_reduce", "page_append".
 * ls_timing_enable(0) stops recording; ls_timing_reset drops all records.
 * Not thread-safe; calls overlapping on several host threads race. */
ls_status ls_timing_enable(int32_t on);
ls_status ls_timing_reset(void);
ls_status ls_timing_read(const char* kernel, int32_t* launches, double* total_ms);

/* MFMA calibration probe (measurement aid, not part of the method).  Runs
 * `workgroups` workgroups of 512 threads (two waves per SIMD), each wave doing
 * `iters` steps of 4 x 32768 bf16 flop, with random operands cycled every
 * MFMA and no global memory traffic but one float per thread stored to `out`:
 *   mode 0: v_mfma_f32_32x32x16_bf16, register operands;
 *   mode 1: v_mfma_f32_16x16x32_bf16, register operands;
 *   mode 2: 32x32x16 with the A operand read from LDS, 1 KiB per MFMA (the
 *           attention kernels' ratio of LDS bytes to flops);
 *   mode 3: 16x16x32 with the A operand read from LDS, one read per two MFMAs
 *           (the same bytes per flop).
 * Timed by the caller (events on `stream`), it gives the rate the part
 * sustains under its power limit with and without an LDS operand stream.
 *   out       device float [workgroups * 512], written (values meaningless).
 *   flops     host: set to the floating-point operations of the launch.
 * LS_ERR_INVALID_ARG for mode outside 0..3, workgroups < 1, iters < 8 or not
 * a multiple of 8, or a null pointer (nothing launched); LS_ERR_HIP if the
 * launch fails. */
ls_status ls_calib_mfma(int32_t mode, int32_t workgroups, int32_t iters, float* out,
                        double* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LS_REPLAY_H */
