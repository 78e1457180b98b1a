// Forward of replay attention: one partial (m, l, o) per (query-row tile,
// key range).  Key range = a chunk of one split's prompt pages (paged mode) or
// the causal response block (response mode).
//
// Statistics follow the pages' exact composition: each split produces its own
// shift m, sum-exp l and normalised output o, and the global LSE merge combines
// them (LongStraw review page, section 7 mind map, "Qwen3.6-27B
// implementation": forward composition through a global LSE).
//
// gfx950 mapping (per workgroup: 4 waves, 128 query rows of one KV-head group):
//   * the query heads of a KV group are packed into the M dimension, so every
//     K/V byte staged in LDS serves 128 query rows;
//   * each wave owns 32 query rows; its Q stays in registers as the B operand;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows read from LDS) puts
//     one query per lane and 16 of the block's 32 keys per lane in registers,
//     so the softmax statistics need one exchange between lanes l and l^32;
//   * P^T (bf16) is the B operand of O^T = V^T P^T straight from registers; the
//     V^T operand comes from the row-major V tile by transpose reads; O^T keeps
//     one query per lane, so the shift and the final 1/l are per-lane scalars;
//   * full prompt blocks stream through a 4-stage LDS ring filled by
//     buffer->LDS copies issued three blocks ahead, and the loop is software
//     pipelined: the softmax of block b runs on the VALU while the MFMAs
//     compute the scores of block b+1.  Masked blocks (the partial last prompt
//     page, the causal response block) take a simple loop of their own;
//   * the exp2 shift is fixed at the first block's max instead of following
//     the running max, so no accumulator is ever rescaled; an input whose
//     scores later exceed the shift by more than 2^32 is detected and its key
//     range recomputed with the true max as the shift.
#include "ls_device.hpp"

namespace ls {

// S^T[key][query] = sum_d K[key][d] Q[query][d] for the block in tile kt.
template <int D>
__device__ __forceinline__ f32x16 block_scores(const Lanes32<D>& tl, const uint16_t* kt,
                                               const bf16x8 (&qr)[D / 16]) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) s = mfma32(tl.row8(kt, kk), qr[kk], s);
  return s;
}

// Softmax numerators of one block for this lane's query: x = raw scores
// (masked ones -inf), returns P^T as two bf16 B operands (register 8*ks + e
// is k-element e of k-step ks), adds their fp32 sum to lsum.  Pass 0 fixes the
// shift at the first block's max and flags scores that exceed it by more than
// 2^kShiftSlack.
__device__ __forceinline__ void block_probs(const float (&x)[16], float s2, bool pass0,
                                            float& mref, float& mtrue, float& lsum,
                                            bool& unsafe, bf16x8 (&pb)[2]) {
  float mx = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
  const float mb = wave_max_halves(mx) * s2;
  mtrue = fmaxf(mtrue, mb);
  if (pass0) {
    mref = (mref == -kInf) ? mb : mref;
    unsafe = unsafe || (mb > mref + kShiftSlack);
  }
  const float mu = (mref == -kInf) ? 0.f : mref;
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], s2, -mu));
    ls += p;
    pb[r >> 3][r & 7] = to_bf16(p);
  }
  lsum += ls;
}

// O^T[d][query] += sum_key V[key][d] P^T[key][query] for the block in tile vt.
template <int D>
__device__ __forceinline__ void block_pv(f32x16 (&acc)[D / 32], const Lanes32<D>& tl,
                                         const uint16_t* vt, const bf16x8 (&pb)[2]) {
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma32(tl.col8(vt, ks, mt), pb[ks], acc[mt]);
  }
}

// One pipelined step: S(b+1) = K(b+1) Q^T and O^T += V(b)^T P(b), with the
// softmax of S(b) on the VALU and the copies of two blocks three ahead.
//
// A single wave per SIMD pulls LDS operands at a bounded rate, so a step moves
// as fast as its LDS read stream and the MFMAs only keep up if that stream
// never stops.  The step is therefore cut into fixed micro-segments
// (sched_barrier 0 between them): each issues one MFMA, the LDS read its
// MFMA PF segments later needs, and its share of the other work -- one
// softmax element per score MFMA, one copy instruction every second PV MFMA
// (copies issued in a burst stall the wave behind the address unit).
//
// The exp2 shift mu is fixed for the whole key range, so the softmax needs no
// per-block maximum: the lane's running maximum of raw scores (mlane) is only
// checked against the shift once the range is done.
template <int D>
__device__ __forceinline__ void fwd_step(const Lanes32<D>& tl, const BlockLoader<D>& ldr,
                                         const uint16_t* kt, const uint16_t* vt,
                                         const bf16x8 (&qr)[D / 16], f32x16& s_cur,
                                         f32x16 (&acc)[D / 32], float s2, float mu,
                                         float& mlane, float& lsum, uint32_t kdst,
                                         i32x4 kdesc, uint32_t vdst, i32x4 vdesc) {
  constexpr int NS = D / 16;   // score MFMAs per step = PV MFMAs per step
  constexpr int NMT = D / 32;  // 32-wide d tiles of O^T
  constexpr int PF = 4;        // LDS prefetch distance, in MFMAs
  constexpr int NIW = BlockLoader<D>::NIW;
  static_assert(2 * NIW * 2 == NS, "one copy instruction every second PV MFMA");
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = tl.row8(kt, i);
  f32x16 s_next;
#pragma unroll
  for (int r = 0; r < 16; ++r) s_next[r] = 0.f;
  bf16x8 pb[2];
  float mx = mlane, ls = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    s_next = mfma32(kf[i], qr[i], s_next);
    if (i + PF < NS) {
      kf[i + PF] = tl.row8(kt, i + PF);
    } else {
      const int j = i + PF - NS;
      vf[j] = tl.col8(vt, j / NMT, j % NMT);
    }
#pragma unroll
    for (int r = i * 16 / NS; r < (i + 1) * 16 / NS; ++r) {
      const float x = s_cur[r];
      mx = fmaxf(mx, x);
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, s2, -mu));
      ls += p;
      pb[r >> 3][r & 7] = to_bf16(p);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    acc[j % NMT] = mfma32(vf[j], pb[j / NMT], acc[j % NMT]);
    if (j + PF < NS) vf[j + PF] = tl.col8(vt, (j + PF) / NMT, (j + PF) % NMT);
    if ((j & 1) == 0) {
      const int c = j >> 1;
      if (c < NIW) copy16_to_lds(kdst + ldr.lds0 + c * 1024, ldr.voff[c], kdesc);
      else copy16_to_lds(vdst + ldr.lds0 + (c - NIW) * 1024, ldr.voff[c - NIW], vdesc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  mlane = mx;
  lsum += ls;
  s_cur = s_next;
}

template <int D, bool RESP>
__global__ void __launch_bounds__(256, 1) k_fwd(const AttnArgs a) {
  constexpr int NMT = D / 32;
  constexpr int TILE = kBN * D;                     // elements of one K or V block
  constexpr int NST = kStages;                      // ring depth (4)
  constexpr int NLD = 2 * BlockLoader<D>::NIW;      // load instructions per wave per block
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

  const int w = xcd_remap(blockIdx.x, gridDim.x);
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
  const int nfull = walk.nfull;          // leading blocks that need no mask
  const int slot = a.slot_base + unit;

  // Q (B operand): column = query m, k = 16*kk + 8*hf + e.  Rows past the
  // group are computed on a copy of its last row and never stored.
  bf16x8 qr[D / 16];
  const int qi = m % a.R;
  {
    const uint16_t* qp = a.q + (row0 + min(m, GR - 1)) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qr[kk] = ld_bf16x8(qp + 16 * kk);
  }
  const Lanes32<D> tl(hf, lq);
  const BlockLoader<D> ldr(wave, lane);

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

    // ---- pipelined loop over the full (unmasked) blocks.  Iteration b waits
    // for K(b+1) and V(b), starts K(b+4) and V(b+3), computes S(b+1) while
    // turning S(b) into P(b), then accumulates V(b)^T P(b).  Every iteration
    // issues exactly NLD loads (blocks past the range re-read block 0), so
    // "at most two iterations' loads in flight" is a fixed vmcnt.
    if (nfull > 0) {
      wait_loads_le<0>();  // Q has landed (the copies below are invisible to the compiler)
      // All K copies of one loop iteration (blocks b+4 .. b+7) fall in one page,
      // whose pool offset is looked up one iteration ahead.
      constexpr size_t kBlk = (size_t)kBN * D;
      constexpr unsigned kBlkBytes = kBN * D * 2;
      int ph_next = walk.page_id(0);          // page of the blocks the next iteration copies
      size_t pcur = walk.page_base(ph_next);  // offset of the page this iteration copies from
      size_t koff[NST];  // source offset (elements) of the block held by each K stage
#define LS_ISSUE_K(j, st)                                          \
  do {                                                             \
    koff[st] = (j) < nfull ? pcur + ((j) & 7) * kBlk : 0;          \
    load_block(ldr, kst[st], a.k + koff[st], kBN);                 \
  } while (0)
#define LS_ISSUE_V(st) load_block(ldr, vst[st], a.v + koff[st], kBN)
      LS_ISSUE_K(0, 0);
      LS_ISSUE_K(1, 1);
      LS_ISSUE_V(0);
      LS_ISSUE_K(2, 2);
      LS_ISSUE_V(1);
      LS_ISSUE_K(3, 3);
      LS_ISSUE_V(2);  // V(j) always goes to stage j % NST, after K(j)
      ring_barrier<3 * NLD>();  // K(0) landed
      f32x16 s_cur = block_scores<D>(tl, kst[0], qr);
      // the first block fixes the shift of pass 0
      if (pass0 && mref == -kInf) {
        float mx = s_cur[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
        mref = wave_max_halves(mx) * a.s2;
      }
      float mlane = -kInf;  // running max of this lane's raw scores in the loop
#define LS_FWD_STEP(ST)                                                                 \
  if (b + (ST) < nfull) {                                                               \
    /* K(b+1), V(b) landed; stages ST (K) and ST-1 (V) are free */                    \
    ring_barrier<2 * NLD>();                                                            \
    constexpr int SV = ((ST) + NST - 1) % NST; /* V(b+3) goes where V(b-1) was */       \
    const int jk = b + (ST) + NST;             /* K(b+4) goes where K(b) was */         \
    koff[ST] = jk < nfull ? pcur + (jk & 7) * kBlk : 0;                                 \
    fwd_step<D>(tl, ldr, kst[((ST) + 1) % NST], vst[ST], qr, s_cur, acc, a.s2, mref,    \
                mlane, lsum, lds_addr(kst[ST]), block_desc(a.k + koff[ST], kBlkBytes),  \
                lds_addr(vst[SV]), block_desc(a.v + koff[SV], kBlkBytes));              \
  }
      for (int b = 0; b < nfull; b += NST) {
        pcur = walk.page_base(ph_next);
        ph_next = b + 8 < nfull ? walk.page_id((b + 8) >> 3) : -1;
        LS_FWD_STEP(0)
        LS_FWD_STEP(1)
        LS_FWD_STEP(2)
        LS_FWD_STEP(3)
      }
#undef LS_FWD_STEP
#undef LS_ISSUE_V
#undef LS_ISSUE_K
      const float mb = wave_max_halves(mlane) * a.s2;
      mtrue = fmaxf(mtrue, mb);
      if (pass0) unsafe = unsafe || (mb > mref + kShiftSlack);
      wait_loads_le<0>();  // drain the look-ahead loads before LDS is reused
      __syncthreads();
    }

    // ---- masked blocks (partial last prompt page; the causal response block)
    for (int j = nfull; j < nblocks; ++j) {
      int nv, key0;
      const size_t off = walk.block(j, nv, key0);
      if (nv > 0) {
        load_block(ldr, k0, a.k + off, nv);
        load_block(ldr, v0, a.v + off, nv);
      }
      wait_loads_le<0>();
      __syncthreads();
      if (nv > 0) {
        const f32x16 s = block_scores<D>(tl, k0, qr);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = crow(r, hf);
          bool ok = key < nv;
          if (RESP) ok = ok && (key0 + key <= qi);
          x[r] = ok ? s[r] : -kInf;
        }
        bf16x8 pb[2];
        block_probs(x, a.s2, pass0, mref, mtrue, lsum, unsafe, pb);
        block_pv<D>(acc, tl, v0, pb);
      }
      __syncthreads();  // tiles are rewritten by the next block
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
  dim3 g(grid), b(256);
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
