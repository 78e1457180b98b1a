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
//   * each wave owns 32 query rows; its Q stays in registers as the B operand;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows read from LDS) puts
//     one query per lane and 16 of the block's 32 keys per lane in registers,
//     so the softmax statistics need one exchange between lanes l and l^32;
//   * P^T (bf16) is the B operand of O^T = V^T P^T straight from registers; the
//     V^T operand comes from the V tile by transpose reads; O^T keeps one query
//     per lane, so the shift and the final 1/l are per-lane scalars;
//   * K and V tiles are stored chunk-major (LanesCM), so each operand read is
//     a base register plus an immediate offset;
//   * full prompt blocks stream through a 4-stage LDS ring filled by
//     buffer->LDS copies issued three blocks ahead; the second wave on each
//     SIMD covers one wave's waits.  Masked blocks (the partial last prompt
//     page, the causal response block) take a simple loop of their own;
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
// sched_barrier-fenced micro-segments (one MFMA, the LDS read its MFMA PF
// segments later needs, one copy instruction every CEV PV MFMAs), which keeps
// the wave's LDS read stream steady.
//
// The exp2 shift mu is fixed for the whole key range (set from the first
// block's max when `first`), so the softmax needs no per-block maximum: the
// lane's running maximum of raw scores (mlane) is checked against the shift
// once the range is done.
// MASK: only the keys at row offsets lo..hi of the lane's own key rows are
// visible (lane rows 4*hf + 8*(r/4) + r%4 of the block; the caller folds the
// block's valid length, the row's own position and its member start into the
// two per-lane thresholds); COPY: issue the block copies.
template <int D, bool MASK, bool COPY>
__device__ __forceinline__ void fwd_step(const LanesCM<D>& tl, const BlockLoaderCM<D, kFwdWaves>& ldr,
                                         const uint16_t* kt, const uint16_t* vt,
                                         const bf16x8 (&qr)[D / 16], f32x16 (&acc)[D / 32],
                                         float s2, bool first, float& mu, float& mlane,
                                         float& lsum, uint32_t kdst, i32x4 kdesc, uint32_t vdst,
                                         i32x4 vdesc, int hi = kBN, int lo = 0) {
  constexpr int NS = D / 16;   // score MFMAs per step = PV MFMAs per step
  constexpr int NMT = D / 32;  // 32-wide d tiles of O^T
  constexpr int PF = 2;        // LDS prefetch distance, in MFMAs (3 spills in the loop)
  constexpr int NIW = BlockLoaderCM<D, kFwdWaves>::NIW;
  constexpr int CEV = NS / (2 * NIW);  // PV segments per copy instruction
  static_assert(CEV * 2 * NIW == NS, "copy instructions spread evenly over the PV MFMAs");
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = tl.row8(kt, i);
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  // the score MFMAs form one dependent chain; they win issue ties against the
  // other wave's PV MFMAs (about 3 % faster than equal priorities)
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    s = mfma32(kf[i], qr[i], s);
    if (i + PF < NS) {
      kf[i + PF] = tl.row8(kt, i + PF);
    } else {
      const int j = i + PF - NS;
      vf[j] = tl.col8(vt, j / NMT, j % NMT);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  if (MASK) {
    // compile-time row offsets against the per-lane thresholds, so no key
    // index is kept in a register
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 8 * (r >> 2) + (r & 3);
      s[r] = (c <= hi && c >= lo) ? s[r] : -kInf;
    }
  }
  if (first) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mu = wave_max_halves(mx) * s2;
  }
  bf16x8 pb[2];
  float mx = mlane, ls = 0.f;
  // a fully masked first block leaves no shift (masked blocks only)
  const float mus = (MASK && mu == -kInf) ? 0.f : mu;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float x = s[r];
    mx = fmaxf(mx, x);
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, s2, -mus));
    ls += p;
    pb[r >> 3][r & 7] = to_bf16(p);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    acc[j % NMT] = mfma32(vf[j], pb[j / NMT], acc[j % NMT]);
    if (j + PF < NS) vf[j + PF] = tl.col8(vt, (j + PF) / NMT, (j + PF) % NMT);
    if (COPY && j % CEV == 0) ldr.issue(j / CEV, kdst, kdesc, vdst, vdesc);
    __builtin_amdgcn_sched_barrier(0);
  }
  mlane = mx;
  lsum += ls;
}

template <int D, bool RESP>
__global__ void __launch_bounds__(64 * kFwdWaves, 1) k_fwd(const AttnArgs a) {
  constexpr int NMT = D / 32;
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
  const int hf = lane >> 5, lq = lane & 31;

  const int w = RESP ? tile_item(a, kFwdRows, blockIdx.x, gridDim.x) : xcd_remap(blockIdx.x, gridDim.x);
  const int per_unit = a.mtiles * a.hkv;
  const int unit = w / per_unit;
  const int rem = w - unit * per_unit;
  const int kv = rem / a.mtiles;
  const int mtile = rem - kv * a.mtiles;
  const int GR = (a.hq / a.hkv) * a.R;
  const int m0 = mtile * kFwdRows;
  const int m = m0 + 32 * wave + lq;     // this lane's query row within the group
  const size_t row0 = (size_t)kv * GR;
  const KeyWalk<D, RESP> walk(a, kv, unit, m0, kFwdRows);
  const int nblocks = walk.nblocks;
  // leading blocks that need no mask: the full prompt pages of the range or,
  // in the response block of one response when the tile stays in one query
  // head, the keys that even the tile's first row sees (KeyWalk)
  const int nfull = walk.nfull;
  const int slot = a.slot_base + unit;

  // Q (B operand): column = query m, k = 16*kk + 8*hf + e.  Rows past the
  // group are computed on a copy of its last row and never stored.
  bf16x8 qr[D / 16];
  const int qi = m % a.R;
  // masked blocks: the row sees response keys [member start, qoff + qi]; as
  // thresholds relative to the lane's first key row 4*hf (keys past the
  // block's valid rows lie beyond qoff + qi, so the bounds cover them)
  const int lane_hi = RESP ? qi + a.qoff - 4 * hf : -4 * hf;
  const int lane_lo = RESP ? member_start(a, qi) - 4 * hf : -4 * hf;
  {
    const uint16_t* qp = a.q + (row0 + min(m, GR - 1)) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qr[kk] = ld_bf16x8(qp + 16 * kk);
  }
  LanesCM<D> tl(hf, lq);
  const BlockLoaderCM<D, kFwdWaves> ldr(wave, lane);

  f32x16 acc[NMT];
  float mref = -kInf;   // exp2 shift of this query (log2 units)
  float mtrue = -kInf;  // running max of this query's scaled scores
  float lsum = 0.f;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
    lsum = 0.f;
    if (pass == 1) mref = mtrue;
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
      float mlane = -kInf;  // running max of this lane's raw scores in the range
      // Values the loop reads that may have been reloaded from scratch: make
      // them resident here, so the loop body never waits on a pending reload
      // (such a wait would also drain the ring's copies).
      asm volatile("" ::"v"(mref), "v"(lsum), "v"(mtrue));
#define LS_FWD_STEP(ST)                                                                  \
  if (b + (ST) < nfull) {                                                                \
    /* K(b), V(b) landed; stage (ST+3)%4 (block b-1) is free */                         \
    ring_barrier<2 * NLD>();                                                             \
    tl.refresh();                                                                        \
    constexpr int SC = ((ST) + 3) % NST;                                                 \
    const size_t off = LS_BLOCK_OFF(b + (ST) + 3);                                       \
    /* pass 0 starts with no shift: its first block sets it */                          \
    fwd_step<D, false, true>(tl, ldr, kst[ST], vst[ST], qr, acc, a.s2,                   \
                pass0 && b + (ST) == 0, mref, mlane, lsum, lds_addr(kst[SC]),            \
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
      const float mb = wave_max_halves(mlane) * a.s2;
      mtrue = fmaxf(mtrue, mb);
      if (pass0) unsafe = unsafe || (mb > mref + kShiftSlack);
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
      float mlane = -kInf;
      int jb = max(nfull, walk.jfirst);
      // opaque per pass, so that the block addresses below are computed here
      // rather than hoisted out of the pass loop and kept live across it
      asm volatile("" : "+s"(jb));
      if (jb < nblocks) {
        // Q and any reloaded lane thresholds have landed: the compiler then
        // has no load of its own pending in the loop and adds no wait there
        // that would drain the copies
        asm volatile("" ::"v"(lane_hi), "v"(lane_lo));
        wait_loads_le<0>();
#define LS_ISSUE(J)                                                                       \
  {                                                                                       \
    const int s_ = ((J) - jb) & (NST - 1);                                                \
    int nv_ = 0, key0_ = 0;                                                               \
    const size_t off_ = (J) < nblocks ? walk.block((J), nv_, key0_) : 0;                  \
    /* the clamp may be done on the vector unit: bring it back to a scalar */            \
    nv_ = __builtin_amdgcn_readfirstlane(max(nv_, 0));                                    \
    load_block_cm<false>(ldr, s_ == 0 ? k0 : s_ == 1 ? k1 : s_ == 2 ? k2 : k3, a.k + off_, \
                         nv_);                                                            \
    load_block_cm<true>(ldr, s_ == 0 ? v0 : s_ == 1 ? v1 : s_ == 2 ? v2 : v3, a.v + off_,  \
                        nv_);                                                             \
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
                                     a.s2, pass0 && mref == -kInf, mref, mlane, lsum, 0, none, 0,
                                     none, RESP ? lane_hi - key0 : lane_hi + nv - 1,
                                     lane_lo - key0);
          }
        }
#undef LS_ISSUE
        wait_loads_le<0>();  // no copy into LDS outlives the loop
      }
      const float mb = wave_max_halves(mlane) * a.s2;
      mtrue = fmaxf(mtrue, mb);
      if (pass0) unsafe = unsafe || (mb > mref + kShiftSlack);
    }

    if (!pass0 || !__syncthreads_or(unsafe ? 1 : 0)) break;
  }

  // ---- epilogue: o = O^T / l, m in natural-log units
  const float lt = lsum + __shfl_xor(lsum, 32);
  if (m < GR) {
    const size_t rows_total = (size_t)a.hq * a.R;
    const size_t row = row0 + m;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* op = a.o + ((size_t)slot * rows_total + row) * D + 4 * hf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc[mt][4 * r4 + 0] * inv;
        v.y = acc[mt][4 * r4 + 1] * inv;
        v.z = acc[mt][4 * r4 + 2] * inv;
        v.w = acc[mt][4 * r4 + 3] * inv;
        *reinterpret_cast<float4*>(op + 32 * mt + 8 * r4) = v;
      }
    }
    if (hf == 0) {
      a.m[(size_t)slot * rows_total + row] = lt > 0.f ? mref * kLn2 : -kInf;
      a.l[(size_t)slot * rows_total + row] = lt;
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
