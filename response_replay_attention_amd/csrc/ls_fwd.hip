// Forward of replay attention: one partial (m, l, o) per (query-row tile,
// key range).  Key range = a chunk of one split's prompt pages (paged mode) or
// the causal response block (response mode).
//
// Statistics follow the pages' exact composition: each split produces its own
// shift m, sum-exp l and normalised output o, and the global LSE merge combines
// them (LongStraw review page, section 7 mind map, "Qwen3.6-27B
// implementation": forward composition through a global LSE).
//
// gfx950 mapping (per workgroup: 8 waves, two per SIMD, 256 query rows of one
// KV-head group):
//   * the query heads of a KV group are packed into the M dimension, so every
//     K/V byte staged in LDS serves 256 query rows;
//   * each wave owns 32 query rows as two halves of 16; its Q stays in
//     registers as the B operand;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows read from LDS, each
//     read serving both query halves) puts two queries and 8 of the block's 32
//     keys per lane in registers, so a query's statistics are spread over the
//     four lanes l, l^16, l^32, l^48;
//   * P^T (bf16) is the B operand of O^T = V^T P^T straight from registers; the
//     V^T operand comes from the V tile by transpose reads gathering exactly
//     the keys a lane holds; O^T keeps the lane's two queries, so the shifts
//     and the final 1/l are per-lane scalars;
//   * K and V tiles are stored chunk-major (Lanes16), so each operand read is
//     a base register plus an immediate;
//   * full prompt blocks stream through a 4-stage LDS ring filled by
//     buffer->LDS copies issued three blocks ahead; the second wave on each
//     SIMD covers one wave's waits.  Masked blocks (the partial last prompt
//     page, the causal response block) go through the same ring in a loop of
//     their own;
//   * the exp2 shift is fixed at the first block's max instead of following
//     the running max, so no accumulator is ever rescaled; an input whose
//     scores later exceed the shift by more than 2^32 is detected and its key
//     range recomputed with the true max as the shift.
#include "ls_device.hpp"

namespace ls {

// One step over a full key block b: S(b) = K(b) Q^T, P(b) = exp2(S s log2e -
// mu) on the VALU, O^T += V(b)^T P(b), and the copies of block b+3.  Two
// waves share each SIMD, so the hardware interleaves one wave's LDS waits
// with the other's MFMAs; inside a wave the step is still a fixed sequence of
// sched_barrier-fenced micro-segments (one operand read, the two MFMAs of
// the fragment PF reads earlier, one copy instruction every CEV PV fragments),
// which keeps the wave's LDS read stream steady.
//
// The wave's 32 queries are two halves qh of 16 (v_mfma_f32_16x16x32_bf16);
// lane l (n = l % 16, G = l / 16) holds S^T[16kh + 4G + r][16qh + n], i.e. two
// queries and eight of the block's keys, and every statistic is per (lane, qh).
// The exp2 shift mu is fixed for the whole key range (set from the first
// block's max when first[qh]), so the softmax needs no per-block maximum: the
// lane's running maximum of raw scores (mlane) is checked against the shift
// once the range is done.
// MASK: only the keys at row offsets lo..hi of the lane's own key rows are
// visible (rows 4G + 16kh + r of the block; the caller folds the block's
// valid length, the row's own position and its member start into per-lane
// thresholds for each query half); COPY: issue the block copies.
template <int D, bool MASK, bool COPY>
__device__ __forceinline__ void fwd_step(const Lanes16<D>& tl,
                                         const BlockLoaderCM<D, kFwdWaves>& ldr,
                                         const uint16_t* kt, const uint16_t* vt,
                                         const bf16x8 (&qr)[2][D / 32], f32x4 (&acc)[D / 16][2],
                                         float s2, bool first0, bool first1, float (&mu)[2],
                                         float (&mlane)[2], float (&lsum)[2], uint32_t kdst,
                                         i32x4 kdesc, uint32_t vdst, i32x4 vdesc, int hi0 = kBN,
                                         int hi1 = kBN, int lo0 = 0, int lo1 = 0) {
  constexpr int NF = D / 16;  // K fragments per block = V^T fragments per block
  constexpr int PF = 2;       // LDS prefetch distance, in fragments
  constexpr int NIW = BlockLoaderCM<D, kFwdWaves>::NIW;
  constexpr int CEV = NF / (2 * NIW);
  static_assert(CEV * 2 * NIW == NF, "copy instructions spread evenly over the PV fragments");
  bf16x8 kf[NF], vf[NF];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = tl.krow(kt, i);
  f32x4 s[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[kh][qh][r] = 0.f;
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int kk = i >> 1, kh = i & 1;
    s[kh][0] = mfma16(kf[i], qr[0][kk], s[kh][0]);
    s[kh][1] = mfma16(kf[i], qr[1][kk], s[kh][1]);
    if (i + PF < NF) kf[i + PF] = tl.krow(kt, i + PF);
    else vf[i + PF - NF] = tl.vcol(vt, i + PF - NF);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  if (MASK) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * kh + r;
        s[kh][0][r] = (c <= hi0 && c >= lo0) ? s[kh][0][r] : -kInf;
        s[kh][1][r] = (c <= hi1 && c >= lo1) ? s[kh][1][r] : -kInf;
      }
  }
  if (first0) {
    float mx = fmaxf(fmaxf(s[0][0][0], s[0][0][1]), fmaxf(s[0][0][2], s[0][0][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s[1][0][0], s[1][0][1]), fmaxf(s[1][0][2], s[1][0][3])));
    mu[0] = quad_max(mx) * s2;
  }
  if (first1) {
    float mx = fmaxf(fmaxf(s[0][1][0], s[0][1][1]), fmaxf(s[0][1][2], s[0][1][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s[1][1][0], s[1][1][1]), fmaxf(s[1][1][2], s[1][1][3])));
    mu[1] = quad_max(mx) * s2;
  }
  bf16x8 pb[2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    float mx = mlane[qh], ls = 0.f;
    const float mus = (MASK && mu[qh] == -kInf) ? 0.f : mu[qh];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = s[kh][qh][r];
        mx = fmaxf(mx, x);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, s2, -mus));
        ls += p;
        pb[qh][4 * kh + r] = to_bf16(p);
      }
    mlane[qh] = mx;
    lsum[qh] += ls;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    acc[j][0] = mfma16(vf[j], pb[0], acc[j][0]);
    acc[j][1] = mfma16(vf[j], pb[1], acc[j][1]);
    if (j + PF < NF) vf[j + PF] = tl.vcol(vt, j + PF);
    if (COPY && j % CEV == 0) ldr.issue(j / CEV, kdst, kdesc, vdst, vdesc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool RESP>
__global__ void __launch_bounds__(64 * kFwdWaves, 1) k_fwd(const AttnArgs a) {
  constexpr int TILE = kBN * D;                     // elements of one K or V block
  constexpr int NST = kStages;                      // ring depth (4)
  constexpr int NLD = 2 * BlockLoaderCM<D, kFwdWaves>::NIW;  // copy instructions per wave per block
  // One array per ring stage: distinct LDS objects let the compiler tell the
  // stages apart, so a read of one stage does not wait for the copies still
  // in flight into the others.
  __shared__ __attribute__((aligned(1024))) uint16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
  uint16_t* const kst[NST] = {k0, k1, k2, k3};
  uint16_t* const vst[NST] = {v0, v1, v2, v3};
  static_assert(NST == 4, "the ring has four stages");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 4, n = lane & 15;

  const int w = RESP ? tile_item(a, kFwdRows, blockIdx.x, gridDim.x) : xcd_remap(blockIdx.x, gridDim.x);
  const int per_unit = a.mtiles * a.hkv;
  const int unit = w / per_unit;
  const int rem = w - unit * per_unit;
  const int kv = rem / a.mtiles;
  const int mtile = rem - kv * a.mtiles;
  const int GR = (a.hq / a.hkv) * a.R;
  const int m0 = mtile * kFwdRows;
  const int mq[2] = {m0 + 32 * wave + n, m0 + 32 * wave + 16 + n};  // this lane's two query rows
  const size_t row0 = (size_t)kv * GR;
  const KeyWalk<D, RESP> walk(a, kv, unit, m0, kFwdRows);
  const int nblocks = walk.nblocks;
  // leading blocks that need no mask: the full prompt pages of the range or,
  // in the response block of one response when the tile stays in one query
  // head, the keys that even the tile's first row sees (KeyWalk)
  const int nfull = walk.nfull;
  const int slot = a.slot_base + unit;

  // Q (B operand of query half qh): column = query mq[qh], k = 32*kk + 8G + e.
  // Rows past the group are computed on a copy of its last row and never
  // stored.  Masked blocks: the row sees response keys [member start, qoff +
  // qi]; as thresholds relative to the lane's first key row 4G (keys past the
  // block's valid rows lie beyond qoff + qi, so the bounds cover them).
  bf16x8 qr[2][D / 32];
  int lane_hi[2], lane_lo[2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int qi = mq[qh] % a.R;
    lane_hi[qh] = RESP ? qi + a.qoff - 4 * G : -4 * G;
    lane_lo[qh] = RESP ? member_start(a, qi) - 4 * G : -4 * G;
    const uint16_t* qp = a.q + (row0 + min(mq[qh], GR - 1)) * D + 8 * G;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qr[qh][kk] = ld_bf16x8(qp + 32 * kk);
  }
  Lanes16<D> tl(lane);
  const BlockLoaderCM<D, kFwdWaves> ldr(wave, lane);

  f32x4 acc[D / 16][2];
  float mref[2] = {-kInf, -kInf};   // exp2 shift of each query (log2 units)
  float mtrue[2] = {-kInf, -kInf};  // running max of each query's scaled scores
  float lsum[2] = {0.f, 0.f};

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][qh][r] = 0.f;
    lsum[0] = lsum[1] = 0.f;
    if (pass == 1) {
      mref[0] = mtrue[0];
      mref[1] = mtrue[1];
    }
    bool unsafe = false;
    const bool pass0 = pass == 0;

    // ---- loop over the full (unmasked) blocks through the 4-stage ring.
    // Step b waits for K(b) and V(b), computes block b and starts the copies
    // of block b+3 into the stage block b-1 used.  Every step issues exactly
    // NLD copies (blocks past the range re-read block 0), so "at most two
    // steps' copies in flight" is a fixed vmcnt.
    if (nfull > 0) {
      wait_loads_le<0>();  // Q has landed (the copies below are invisible to the compiler)
      constexpr size_t kBlk = (size_t)kBN * D;
      constexpr unsigned kBlkBytes = kBN * D * 2;
      constexpr int BPP = kPage / kBN;  // blocks per page
      const int npg = nfull / BPP;      // full pages of this range
      // pool offsets of page pn and pn+1, and the id of page pn+2 (loaded one
      // page ahead of its use); copies address block j through page j / BPP
      int pn = 0;
      size_t base0 = 0, base1 = 0;
      int id2 = -1;
      if (!RESP) {
        base0 = walk.page_base(walk.page_id(0));
        base1 = npg > 1 ? walk.page_base(walk.page_id(1)) : 0;
        id2 = npg > 2 ? walk.page_id(2) : -1;
      }
      // (response keys are contiguous: block j is rows [32j, 32j+32) of this KV head)
#define LS_BLOCK_OFF(j)                                                              \
  ((j) < nfull ? (RESP ? ((size_t)kv * a.kvr + (size_t)(j) * kBN) * D                 \
                       : (((j) / BPP == pn) ? base0 : base1) + ((j) % BPP) * kBlk)      \
               : (size_t)0)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const size_t off = LS_BLOCK_OFF(j);
        load_block_cm<false>(ldr, kst[j], a.k + off, kBN);
        load_block_cm<true>(ldr, vst[j], a.v + off, kBN);
      }
      float mlane[2] = {-kInf, -kInf};  // running max of this lane's raw scores in the range
      // Values the loop reads that may have been reloaded from scratch: make
      // them resident here, so the loop body never waits on a pending reload
      // (such a wait would also drain the ring's copies).
      asm volatile("" ::"v"(mref[0]), "v"(lsum[0]), "v"(mtrue[0]), "v"(mref[1]), "v"(lsum[1]),
                   "v"(mtrue[1]));
#define LS_FWD_STEP(ST)                                                                  \
  if (b + (ST) < nfull) {                                                                \
    /* K(b), V(b) landed; stage (ST+3)%4 (block b-1) is free */                         \
    ring_barrier<2 * NLD>();                                                             \
    tl.refresh();                                                                        \
    constexpr int SC = ((ST) + 3) % NST;                                                 \
    const size_t off = LS_BLOCK_OFF(b + (ST) + 3);                                       \
    /* pass 0 starts with no shift: its first block sets it */                          \
    fwd_step<D, false, true>(tl, ldr, kst[ST], vst[ST], qr, acc, a.s2,                 \
                pass0 && b + (ST) == 0, pass0 && b + (ST) == 0, mref, mlane, lsum,       \
                lds_addr(kst[SC]),                                                       \
                block_desc(a.k + off, kBlkBytes), lds_addr(vst[SC]),                     \
                block_desc(a.v + off, kBlkBytes));                                       \
  }
      for (int b = 0; b < nfull; b += NST) {
        // the copies of this iteration (blocks b+3 .. b+6) reach page (b+6)/BPP
        if (!RESP && (b + 6) / BPP > pn + 1 && b + 6 < nfull) {
          ++pn;
          base0 = base1;
          base1 = walk.page_base(id2);
          id2 = pn + 2 < npg ? walk.page_id(pn + 2) : -1;
        }
        LS_FWD_STEP(0)
        LS_FWD_STEP(1)
        LS_FWD_STEP(2)
        LS_FWD_STEP(3)
      }
#undef LS_FWD_STEP
#undef LS_BLOCK_OFF
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float mb = quad_max(mlane[qh]) * a.s2;
        mtrue[qh] = fmaxf(mtrue[qh], mb);
        if (pass0) unsafe = unsafe || (mb > mref[qh] + kShiftSlack);
      }
      wait_loads_le<0>();  // drain the look-ahead copies before LDS is reused
      __syncthreads();
    }

    // ---- masked blocks (partial last prompt page; the causal response
    // block) through the same 4-stage ring, three blocks ahead: step j waits
    // for block j, starts the copies of block j+3 into the stage block j-1
    // used and computes block j.  Every step issues one block's copies (a
    // block past the range gets a zero-length copy, which reads nothing and
    // is never computed), so "at most two blocks in flight" is a fixed vmcnt.
    {
      float mlane[2] = {-kInf, -kInf};
      int jb = max(nfull, walk.jfirst);
      // opaque per pass, so that the block addresses below are computed here
      // rather than hoisted out of the pass loop and kept live across it
      asm volatile("" : "+s"(jb));
      if (jb < nblocks) {
        // Q and any reloaded lane thresholds have landed: the compiler then
        // has no load of its own pending in the loop and adds no wait there
        // that would drain the copies
        asm volatile("" ::"v"(lane_hi[0]), "v"(lane_lo[0]), "v"(lane_hi[1]), "v"(lane_lo[1]));
        wait_loads_le<0>();
#define LS_ISSUE(J)                                                                       \
  {                                                                                       \
    const int s_ = ((J) - jb) & (NST - 1);                                                \
    int nv_ = 0, key0_ = 0;                                                               \
    const size_t off_ = (J) < nblocks ? walk.block((J), nv_, key0_) : 0;                  \
    /* the clamp may be done on the vector unit: bring it back to a scalar */            \
    nv_ = __builtin_amdgcn_readfirstlane(max(nv_, 0));                                    \
    load_block_cm<false>(ldr, s_ == 0 ? k0 : s_ == 1 ? k1 : s_ == 2 ? k2 : k3, a.k + off_, \
                           nv_);                                                          \
    load_block_cm<true>(ldr, s_ == 0 ? v0 : s_ == 1 ? v1 : s_ == 2 ? v2 : v3, a.v + off_,  \
                          nv_);                                                           \
  }
        LS_ISSUE(jb)
        LS_ISSUE(jb + 1)
        LS_ISSUE(jb + 2)
        for (int j = jb; j < nblocks; ++j) {
          ring_barrier<2 * NLD>();  // block j landed; the stage of block j-1 is free
          LS_ISSUE(j + 3)
          const int s = (j - jb) & (NST - 1);
          int nv, key0;
          walk.block(j, nv, key0);
          if (nv > 0) {
            tl.refresh();
            const i32x4 none = {0, 0, 0, 0};
            fwd_step<D, true, false>(tl, ldr, s == 0 ? k0 : s == 1 ? k1 : s == 2 ? k2 : k3,
                                       s == 0 ? v0 : s == 1 ? v1 : s == 2 ? v2 : v3, qr, acc,
                                       a.s2, pass0 && mref[0] == -kInf, pass0 && mref[1] == -kInf,
                                       mref, mlane, lsum, 0, none, 0, none,
                                       RESP ? lane_hi[0] - key0 : lane_hi[0] + nv - 1,
                                       RESP ? lane_hi[1] - key0 : lane_hi[1] + nv - 1,
                                       lane_lo[0] - key0, lane_lo[1] - key0);
          }
        }
#undef LS_ISSUE
        wait_loads_le<0>();  // no copy into LDS outlives the loop
      }
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float mb = quad_max(mlane[qh]) * a.s2;
        mtrue[qh] = fmaxf(mtrue[qh], mb);
        if (pass0) unsafe = unsafe || (mb > mref[qh] + kShiftSlack);
      }
    }

    if (!pass0 || !__syncthreads_or(unsafe ? 1 : 0)) break;
  }

  // ---- epilogue: o = O^T / l, m in natural-log units
  const size_t rows_total = (size_t)a.hq * a.R;
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float lt = quad_sum(lsum[qh]);
    if (mq[qh] < GR) {
      const size_t row = row0 + mq[qh];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* op = a.o + ((size_t)slot * rows_total + row) * D + 4 * G;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        float4 v;
        v.x = acc[dt][qh][0] * inv;
        v.y = acc[dt][qh][1] * inv;
        v.z = acc[dt][qh][2] * inv;
        v.w = acc[dt][qh][3] * inv;
        *reinterpret_cast<float4*>(op + 16 * dt) = v;
      }
      if (G == 0) {
        a.m[(size_t)slot * rows_total + row] = lt > 0.f ? mref[qh] * kLn2 : -kInf;
        a.l[(size_t)slot * rows_total + row] = lt;
      }
    }
  }
}

hipError_t launch_fwd(const AttnArgs& a, int head_dim, bool resp, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), b(64 * kFwdWaves);
  if (head_dim == 256) {
    if (resp) hipLaunchKernelGGL((k_fwd<256, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_fwd<256, false>), g, b, 0, s, a);
  } else {
    if (resp) hipLaunchKernelGGL((k_fwd<128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_fwd<128, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ls
