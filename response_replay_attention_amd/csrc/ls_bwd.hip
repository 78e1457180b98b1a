// Response-only backward of replay attention.
//
// The prompt state is stopgrad (DeepRead summary page, "Method"): no gradient
// is formed for the prompt K/V.  What remains (LongStraw review page,
// section 2 and the section 7 mind map):
//   * dQ over the prompt keys of each split, recomputing P = exp(x - LSE) from
//     the saved LSE -- one partial per split, later summed in split order (the
//     one-GPU stand-in for the pages' dQ all-reduce across CP ranks);
//   * dQ over the causal response block (one more partial);
//   * dK, dV of the response keys (key-stationary, one partial per query head,
//     summed over the heads of each KV group in head order by k_kv_reduce, so
//     no atomics are needed).
//
// dQ kernel mapping (32 query rows per score wave and per dQ wave): per key block
//   S^T  = K Q^T      (A = K rows from LDS, B = Q in the score wave's registers)
//   dP^T = V dO^T     (A = V rows from LDS, B = dO in the score wave's registers)
//   dS^T = P^T (dP^T - D)                    with P^T = exp2(S^T*s*log2e - LSE*log2e)
//   dQ^T += K^T dS^T  (A = K^T gathered from the same K tile, B = dS^T that the
//                      score wave stored to LDS, in the dQ wave)
// so dQ^T keeps one query per lane, like O^T in the forward.
#include "ls_device.hpp"

namespace ls {

// dS^T of one block as two bf16 B operands: x = raw scores (masked ones
// -inf), dp = dP^T, lse2 = LSE*log2(e), dval = D of this lane's query.
__device__ __forceinline__ void block_ds(const float (&x)[16], const f32x16& dp, float s2,
                                         float lse2, float dval, bf16x8 (&dsb)[2]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], s2, -lse2));
    dsb[r >> 3][r & 7] = to_bf16(p * (dp[r] - dval));
  }
}

// S^T = K Q^T and dP^T = V dO^T for the block in tiles kt, vt.
template <int D>
__device__ __forceinline__ void block_sdp(const Lanes32<D>& tl, const uint16_t* kt,
                                          const uint16_t* vt, const bf16x8 (&qr)[D / 16],
                                          const bf16x8 (&dor)[D / 16], f32x16& s, f32x16& dp) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    s = mfma32(tl.row8(kt, kk), qr[kk], s);
    dp = mfma32(tl.row8(vt, kk), dor[kk], dp);
  }
}

// dQ^T[d][query] += sum_key K[key][d] dS^T[key][query] for the block in kt.
template <int D>
__device__ __forceinline__ void block_dq(f32x16 (&acc)[D / 32], const Lanes32<D>& tl,
                                         const uint16_t* kt, const bf16x8 (&dsb)[2]) {
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma32(tl.col8(kt, ks, mt), dsb[ks], acc[mt]);
  }
}

// One block of a score wave: S^T = K Q^T (two chains, over even and odd
// k-steps), then dP^T = V dO^T with the exponential of one score placed
// between consecutive dP MFMAs (P = exp2(S s log2e - LSE log2e)), so that
// after the last MFMA only dS^T = P^T (dP^T - D) remains; dS^T is stored to dsw
// as the two bf16 B operands of the dQ product, in this lane's register order
// ([ks][lane][8] elements), for the dQ wave of the same rows.  Each operand is
// read PF MFMAs ahead.
template <int D>
__device__ __forceinline__ void score_block(const Lanes32<D>& tl, const uint16_t* kt,
                                            const uint16_t* vt, const bf16x8 (&qr)[D / 16],
                                            const bf16x8 (&dor)[D / 16], float s2, float lse2,
                                            float dval, uint16_t* dsw) {
  constexpr int NS = D / 16;  // S MFMAs = dP MFMAs per block
  constexpr int PF = 4;       // LDS prefetch distance, in MFMAs
  static_assert(16 % NS == 0, "scores spread evenly over the dP MFMAs");
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = tl.row8(kt, i);
  f32x16 sa, sb, dp;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sa[r] = 0.f;
    sb[r] = 0.f;
    dp[r] = -dval;  // the accumulation starts at -D: it ends at dP - D
  }
  __builtin_amdgcn_sched_barrier(0);
  // S = K Q^T over even (sa) and odd (sb) k-steps; the last reads fetch V
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i & 1) sb = mfma32(kf[i], qr[i], sb);
    else sa = mfma32(kf[i], qr[i], sa);
    if (i + PF < NS) kf[i + PF] = tl.row8(kt, i + PF);
    else vf[i + PF - NS] = tl.row8(vt, i + PF - NS);
    __builtin_amdgcn_sched_barrier(0);
  }
  // dP^T = V dO^T, with P = exp2(S s log2e - LSE log2e) of one score per MFMA
  float p[16];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    dp = mfma32(vf[i], dor[i], dp);
    if (i + PF < NS) vf[i + PF] = tl.row8(vt, i + PF);
#pragma unroll
    for (int r = i * (16 / NS); r < (i + 1) * (16 / NS); ++r) {
      p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r] + sb[r], s2, -lse2));
      asm volatile("" : "+v"(p[r]));  // computed here, between the MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 dsb[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dsb[r >> 3][r & 7] = to_bf16(p[r] * dp[r]);
  *reinterpret_cast<bf16x8*>(dsw) = dsb[0];
  *reinterpret_cast<bf16x8*>(dsw + 64 * 8) = dsb[1];
}

// One step of a dQ wave: dQ^T += K^T dS^T for the block whose K tile is kc and
// whose dS^T the score wave stored at dsr (when mma), and this wave's share of
// the copies of two ring blocks (K into kdst, V into vdst), one copy
// instruction every second MFMA.
template <int D>
__device__ __forceinline__ void dq_block(const Lanes32<D>& tl, const BlockLoader<D>& ldr,
                                         const uint16_t* kc, const uint16_t* dsr,
                                         f32x16 (&acc)[D / 32], bool mma, uint32_t kdst,
                                         i32x4 kdesc, uint32_t vdst, i32x4 vdesc) {
  constexpr int NS = D / 16;  // dQ MFMAs per block
  constexpr int NMT = D / 32;
  constexpr int PF = 4;
  constexpr int NIW = BlockLoader<D>::NIW;
  static_assert(2 * NIW * 2 == NS, "one copy instruction every second dQ MFMA");
  if (mma) {
    bf16x8 dsb[2], cf[NS];
    dsb[0] = *reinterpret_cast<const bf16x8*>(dsr);
    dsb[1] = *reinterpret_cast<const bf16x8*>(dsr + 64 * 8);
#pragma unroll
    for (int j = 0; j < PF; ++j) cf[j] = tl.col8(kc, j / NMT, j % NMT);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      acc[j % NMT] = mfma32(cf[j], dsb[j / NMT], acc[j % NMT]);
      if (j + PF < NS) cf[j + PF] = tl.col8(kc, (j + PF) / NMT, (j + PF) % NMT);
      if ((j & 1) == 0) {
        const int c = j >> 1;
        if (c < NIW) copy16_to_lds(kdst + ldr.lds0 + c * 1024, ldr.voff[c], kdesc);
        else copy16_to_lds(vdst + ldr.lds0 + (c - NIW) * 1024, ldr.voff[c - NIW], vdesc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 2 * NIW; ++c) {
      if (c < NIW) copy16_to_lds(kdst + ldr.lds0 + c * 1024, ldr.voff[c], kdesc);
      else copy16_to_lds(vdst + ldr.lds0 + (c - NIW) * 1024, ldr.voff[c - NIW], vdesc);
    }
  }
}

// The score waves' side of k_bwd_dq (the barrier sequence matches dq_role's).
template <int D, bool RESP>
__device__ __forceinline__ void score_role(const AttnArgs& a, const KeyWalk<D, RESP>& walk,
                                           const Lanes32<D>& tl, uint16_t* const (&kst)[kStages],
                                           uint16_t* const (&vst)[kStages], uint16_t* dsw,
                                           size_t row, bool rvalid, int qi, int hf) {
  constexpr int NKK = D / 16;
  constexpr int NIW = BlockLoader<D>::NIW;
  constexpr int DSX = 2 * 64 * 8;
  const int nblocks = walk.nblocks, nfull = walk.nfull;
  // Q and dO as B operands (column = query m, k = 16*kk + 8*hf + e)
  bf16x8 qr[NKK], dor[NKK];
  {
    const uint16_t* qp = a.q + row * D + 8 * hf;
    const uint16_t* dp = a.d_o + row * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qr[kk] = ld_bf16x8(qp + 16 * kk);
      dor[kk] = ld_bf16x8(dp + 16 * kk);
    }
  }
  // invalid rows: P = exp2(x - inf) = 0, so they contribute nothing
  const float lse2 = rvalid ? a.lse[row] * kLog2e : kInf;
  const float dval = rvalid ? a.dvals[row] : 0.f;

  if (nfull > 0) {
    wait_loads_le<0>();
#define LS_SCORE_STEP(ST)                                                                   \
  if (b + (ST) <= nfull) {                                                                  \
    ring_barrier<3 * NIW>();                                                                \
    if (b + (ST) < nfull)                                                                   \
      score_block<D>(tl, kst[ST], vst[ST], qr, dor, a.s2, lse2, dval,                       \
                     dsw + ((ST) & 1) * 4 * DSX);                                           \
  }
    for (int b = 0; b <= nfull; b += kStages) {
      LS_SCORE_STEP(0)
      LS_SCORE_STEP(1)
      LS_SCORE_STEP(2)
      LS_SCORE_STEP(3)
    }
#undef LS_SCORE_STEP
    wait_loads_le<0>();
    __syncthreads();
  }

  // masked blocks (partial last prompt page; the causal response block)
  for (int j = nfull; j < nblocks; ++j) {
    int nv, key0;
    walk.block(j, nv, key0);
    wait_loads_le<0>();
    __syncthreads();  // the dQ waves' copies of block j have landed
    if (nv > 0) {
      f32x16 s, dp;
      block_sdp<D>(tl, kst[0], vst[0], qr, dor, s, dp);
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = crow(r, hf);
        bool ok = key < nv;
        if (RESP) ok = ok && (key0 + key <= qi + a.qoff);
        x[r] = ok ? s[r] : -kInf;
      }
      bf16x8 dsb[2];
      block_ds(x, dp, a.s2, lse2, dval, dsb);
      *reinterpret_cast<bf16x8*>(dsw) = dsb[0];
      *reinterpret_cast<bf16x8*>(dsw + 64 * 8) = dsb[1];
    }
    __syncthreads();  // dS of block j is stored
    __syncthreads();  // the dQ waves have read it and the tiles
  }
}

// The dQ waves' side of k_bwd_dq: the copies, dQ^T += K^T dS^T one block
// behind the score waves, and the dQ partial of the 32 rows.
template <int D, bool RESP>
__device__ __forceinline__ void dq_role(const AttnArgs& a, const KeyWalk<D, RESP>& walk,
                                        const Lanes32<D>& tl, uint16_t* const (&kst)[kStages],
                                        uint16_t* const (&vst)[kStages], const uint16_t* dsr,
                                        int w4, int lane, float* dq_out, bool rvalid) {
  constexpr int NMT = D / 32;
  constexpr int NST = kStages;
  constexpr int NIW = BlockLoader<D>::NIW;
  constexpr int DSX = 2 * 64 * 8;
  const int nblocks = walk.nblocks, nfull = walk.nfull;
  f32x16 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
  const BlockLoader<D> ldr(w4, lane);
  // the copies and this wave's MFMAs win ties for issue against the score
  // wave on the same SIMD (about 3% faster than equal priorities)
  __builtin_amdgcn_s_setprio(3);

  if (nfull > 0) {
    constexpr size_t kBlk = (size_t)kBN * D;
    constexpr unsigned kBlkBytes = kBN * D * 2;
    // The V copies of loop iteration b (blocks b+3 .. b+6) touch at most two
    // pages; their slots are looked up one iteration ahead.  A page is looked
    // up only if a block of it inside the range is copied.
    // (response keys are contiguous: block j is rows [32j, 32j+32) of this KV head)
    int pa_next = RESP ? -1 : walk.page_id(0), pb_next = pa_next;
    size_t koff[NST];  // source offset of block j, kept from V(j)'s copy to K(j)'s
    {
      const size_t p0 = RESP ? 0 : walk.page_base(pa_next);
#pragma unroll
      for (int j = 0; j < 3; ++j)
        koff[j] = j < nfull ? (RESP ? ((size_t)walk.kv * a.kvr + (size_t)j * kBN) * D : p0 + j * kBlk)
                            : 0;
      // V(0), K(0), V(1), K(1), V(2): the copies of steps -3 .. -1
      load_block(ldr, vst[0], a.v + koff[0], kBN);
      load_block(ldr, kst[0], a.k + koff[0], kBN);
      load_block(ldr, vst[1], a.v + koff[1], kBN);
      load_block(ldr, kst[1], a.k + koff[1], kBN);
      load_block(ldr, vst[2], a.v + koff[2], kBN);
    }
#define LS_DQ_STEP(ST)                                                                      \
  if (b + (ST) <= nfull) {                                                                  \
    /* K(b+ST), V(b+ST) landed; the stages of K(b+ST-2), V(b+ST-1) are free */               \
    ring_barrier<3 * NIW>();                                                                \
    constexpr int SK = ((ST) + 2) % NST, SV = ((ST) + 3) % NST;                             \
    const int jv = b + (ST) + 3;                                                            \
    const size_t pv = ((jv >> 3) == ((b + 3) >> 3)) ? pa : pb;                              \
    koff[SV] = jv >= nfull ? 0                                                              \
               : RESP ? ((size_t)walk.kv * a.kvr + (size_t)jv * kBN) * D                    \
                      : pv + (jv & 7) * kBlk;                                               \
    dq_block<D>(tl, ldr, kst[((ST) + 3) % NST], dsr + (((ST) + 1) & 1) * 4 * DSX, acc,      \
                b + (ST) >= 1, lds_addr(kst[SK]), block_desc(a.k + koff[SK], kBlkBytes),    \
                lds_addr(vst[SV]), block_desc(a.v + koff[SV], kBlkBytes));                  \
  }
    for (int b = 0; b <= nfull; b += NST) {
      const size_t pa = RESP ? 0 : walk.page_base(pa_next);  // page of block b+3
      const size_t pb = RESP ? 0 : walk.page_base(pb_next);  // page of block b+6
      const int ga = b + 7, gb = max(b + 7, ((b + 10) >> 3) << 3);
      pa_next = (!RESP && ga < nfull) ? walk.page_id(ga >> 3) : -1;
      pb_next = (!RESP && gb < nfull) ? walk.page_id(gb >> 3) : -1;
      LS_DQ_STEP(0)
      LS_DQ_STEP(1)
      LS_DQ_STEP(2)
      LS_DQ_STEP(3)
    }
#undef LS_DQ_STEP
    wait_loads_le<0>();  // drain the look-ahead copies before LDS is reused
    __syncthreads();
  }

  // masked blocks (partial last prompt page; the causal response block)
  for (int j = nfull; j < nblocks; ++j) {
    int nv, key0;
    const size_t off = walk.block(j, nv, key0);
    if (nv > 0) {
      load_block(ldr, kst[0], a.k + off, nv);
      load_block(ldr, vst[0], a.v + off, nv);
    }
    wait_loads_le<0>();
    __syncthreads();  // block j's tiles are visible
    __syncthreads();  // the score waves have stored its dS
    if (nv > 0) {
      bf16x8 dsb[2];
      dsb[0] = *reinterpret_cast<const bf16x8*>(dsr);
      dsb[1] = *reinterpret_cast<const bf16x8*>(dsr + 64 * 8);
      block_dq<D>(acc, tl, kst[0], dsb);
    }
    __syncthreads();  // tiles and dS are rewritten by the next block
  }

  if (rvalid) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc[mt][4 * r4 + 0] * a.scale;
        v.y = acc[mt][4 * r4 + 1] * a.scale;
        v.z = acc[mt][4 * r4 + 2] * a.scale;
        v.w = acc[mt][4 * r4 + 3] * a.scale;
        *reinterpret_cast<float4*>(dq_out + 32 * mt + 8 * r4) = v;
      }
    }
  }
}

// dQ of 128 query rows of one KV group over one key range, by two kinds of
// wave.  Waves 0-3 (score waves) own 32 rows each and hold their Q and dO as
// MFMA B operands; per key block b they form S(b), dP(b) and dS(b) and store
// dS(b) to LDS.  Waves 4-7 (dQ waves) own the same rows one to one, hold the
// dQ^T accumulators, and one block behind accumulate K(b-1)^T dS(b-1); they
// also issue every K/V copy.  With 512 threads a SIMD runs two waves, normally
// one of each kind, so the score wave's exp/VALU work and its waits overlap the
// dQ wave's MFMAs instead of idling the matrix unit; each kind needs half the
// registers of a wave that does both.
//
// Ring (four K stages, four V stages; block j in stage j % 4): step b starts
// with one barrier, after which K(b), V(b) have landed; the score waves read
// K(b), V(b), the dQ waves K(b-1), and the dQ waves copy K(b+2) and V(b+3)
// into the stages of K(b-2) and V(b-1), both last read before that barrier.
// Per step every dQ wave issues the same copies (blocks past the range
// re-read block 0), so each wait is a fixed vmcnt: K(b) was issued two steps
// and V(b) three steps before step b, and only V(b+1), K(b+1), V(b+2) may
// still be in flight.  dS goes through two LDS buffers (dS(b) in buffer
// b % 2).  Step nfull only drains the last dQ.
template <int D, bool RESP>
__global__ void __launch_bounds__(512, 1) k_bwd_dq(const AttnArgs a) {
  constexpr int TILE = kBN * D;
  constexpr int DSX = 2 * 64 * 8;  // elements of one wave's dS^T block
  static_assert(kStages == 4, "the ring has four stages");
  // one array per ring stage (distinct LDS objects; see the forward kernel)
  __shared__ __attribute__((aligned(1024))) uint16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t dsx[2 * 4 * DSX];  // [buffer][wave][ks][lane][8]
  uint16_t* const kst[kStages] = {k0, k1, k2, k3};
  uint16_t* const vst[kStages] = {v0, v1, v2, v3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3;
  const int hf = lane >> 5, lq = lane & 31;

  const int w = RESP ? tile_item(a, kBwdRows, blockIdx.x, gridDim.x) : xcd_remap(blockIdx.x, gridDim.x);
  const int per_unit = a.mtiles * a.hkv;
  const int unit = w / per_unit;
  const int rem = w - unit * per_unit;
  const int kv = rem / a.mtiles;
  const int mtile = rem - kv * a.mtiles;
  const int GR = (a.hq / a.hkv) * a.R;
  const int m0 = mtile * kBwdRows;
  const int m = m0 + 32 * w4 + lq;
  const bool rvalid = m < GR;
  const size_t row0 = (size_t)kv * GR;

  const KeyWalk<D, RESP> walk(a, kv, unit, m0, kBwdRows);
  const Lanes32<D> tl(hf, lq);
  uint16_t* const ds_lane = dsx + w4 * DSX + lane * 8;  // this lane's dS^T, buffer 0
  if (wave < 4) {
    score_role<D, RESP>(a, walk, tl, kst, vst, ds_lane, row0 + min(m, GR - 1), rvalid, m % a.R, hf);
  } else {
    const size_t rows_total = (size_t)a.hq * a.R;
    float* op = a.dq_slots + ((size_t)(a.slot_base + unit) * rows_total + row0 + m) * D + 4 * hf;
    dq_role<D, RESP>(a, walk, tl, kst, vst, ds_lane, w4, lane, op, rvalid);
  }
}

// dK or dV of 4 x 32 response keys of KV head kv from the query head
// kv*g + hh, key-stationary: wave w owns keys [j0, j0+32), j0 = 32*(kb0+w),
// and the workgroup loops over the query rows of that head that see any of
// its keys (qoff + i >= 32*kb0, in blocks of 32), accumulating
//   DV:  dV^T[d][key] += sum_query dO[query][d] P[query][key]
//   DK:  dK^T[d][key] += sum_query Q[query][d]  dS[query][key]
// with S = Q K^T and dP = dO V^T recomputed in the (query x key) orientation.
// The four waves share the Q and dO tiles of each query block, which they copy
// a quarter each into the second of two LDS buffers while the current block is
// computed; each wave's K (and V) rows stay in registers as the B operands of
// S (and dP), loaded once from HBM.  Every LDS operand is read four MFMAs ahead
// of its use (fenced, as in the prompt kernels); one barrier per block hands
// the buffers over.  A wave skips the MFMAs of query blocks that see none of
// its keys.  Each head writes its own fp32 partial (k_kv_reduce sums the g
// heads of a group in head order), so no atomics are needed.
template <int D, bool DK>
__device__ __forceinline__ void resp_kv_block(const AttnArgs& a, int kv, int hh, int kb0,
                                              uint16_t* smem, float (&s_lse2)[2][kBN],
                                              float (&s_dval)[2][kBN], int wave, int lane) {
  constexpr int NKK = D / 16;
  constexpr int NMT = D / 32;
  constexpr int TILE = kBN * D;
  constexpr int PF = 4;                   // LDS prefetch distance, in MFMAs
  constexpr int NA = DK ? 2 * NKK : NKK;  // S (and dP) MFMAs per block, two chains
  constexpr int NC = 2 * NMT;             // accumulation MFMAs per block
  const int hf = lane >> 5, lq = lane & 31;
  const int g = a.hq / a.hkv;
  const int h = kv * g + hh;
  // Four tiles: Q of buffer b at smem + b TILE, dO of buffer b at
  // smem + (2 + b) TILE (offsets from the one LDS array, so every access stays
  // an LDS access).
  const BlockLoader<D, 4> ldr(wave, lane);
  const Lanes32<D> tl(hf, lq);

  const int j0 = (kb0 + wave) * kBN;      // this wave's first key
  const bool has_keys = j0 < a.RK;
  const int key = j0 + lq;                // this lane's key column
  const int ib = max(0, kb0 * kBN - a.qoff);  // first query row of the loop
  const int nblk = ib < a.R ? (a.R - ib + kBN - 1) / kBN : 0;

  // K (and V) rows of this wave's keys as B operands: row key, 16-byte chunk
  // 2*kk + hf (keys past the response re-read its last row; they are masked)
  bf16x8 kr[NKK], vr[DK ? NKK : 1];
  {
    const size_t r = (size_t)kv * a.kvr + min(key, a.RK - 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kr[kk] = ld_bf16x8(a.k + r * D + 16 * kk + 8 * hf);
      if (DK) vr[kk] = ld_bf16x8(a.v + r * D + 16 * kk + 8 * hf);
    }
  }
  // Q, dO tiles of block t into buffer t & 1 (a quarter per wave); wave 0's
  // lanes < 32 load LSE*log2(e) and D of query ib + 32t + lane
  auto issue = [&](int t, float& l2, float& dv) {
    const int i0 = ib + t * kBN, nq = min(kBN, a.R - i0);
    if (wave == 0) {
      const bool ok = lane < nq;
      const size_t r = (size_t)h * a.R + i0 + (ok ? lane : 0);
      l2 = ok ? a.lse[r] * kLog2e : kInf;
      dv = ok ? a.dvals[r] : 0.f;
    }
    const size_t qo = ((size_t)h * a.R + i0) * D;
    load_block(ldr, smem + (t & 1) * TILE, a.q + qo, nq);
    load_block(ldr, smem + (2 + (t & 1)) * TILE, a.d_o + qo, nq);
  };

  f32x16 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  float l2n = kInf, dvn = 0.f;
  if (nblk > 0) issue(0, l2n, dvn);
  if (wave == 0 && lane < kBN) {
    s_lse2[0][lane] = l2n;
    s_dval[0][lane] = dvn;
  }
  ring_barrier<0>();  // block 0 and its LSE, D are in LDS

  for (int t = 0; t < nblk; ++t) {
    const int cb = t & 1;
    if (t + 1 < nblk) issue(t + 1, l2n, dvn);
    const int i0 = ib + t * kBN, nq = min(kBN, a.R - i0);
    // the block's last query sees this wave's first key
    if (has_keys && a.qoff + i0 + nq - 1 >= j0) {
      const uint16_t* q = smem + cb * TILE;
      const uint16_t* d_o = smem + (2 + cb) * TILE;
      // this lane's 16 queries crow(r, hf) = 8*(r/4) + 4*hf + r%4: four runs of 4
      f32x4 lse4[4], dv4[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        lse4[r4] = *reinterpret_cast<const f32x4*>(&s_lse2[cb][8 * r4 + 4 * hf]);
        if (DK) dv4[r4] = *reinterpret_cast<const f32x4*>(&s_dval[cb][8 * r4 + 4 * hf]);
      }

      // S[query][key] = sum_d Q[query][d] K[key][d] (DV: two chains over even
      // and odd k-steps; DK: one chain, interleaved with dP = dO V^T)
      auto aop = [&](int i) -> bf16x8 {
        if (DK) return (i & 1) ? tl.row8(d_o, i >> 1) : tl.row8(q, i >> 1);
        return tl.row8(q, i >> 1 | (i & 1) * (NKK / 2));
      };
      bf16x8 rf[NA];
#pragma unroll
      for (int i = 0; i < PF; ++i) rf[i] = aop(i);
      f32x16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = 0.f;
        s1[r] = 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (DK) {
          if (i & 1) s1 = mfma32(rf[i], vr[i >> 1], s1);
          else s0 = mfma32(rf[i], kr[i >> 1], s0);
        } else {
          const int kk = i >> 1 | (i & 1) * (NKK / 2);
          if (i & 1) s1 = mfma32(rf[i], kr[kk], s1);
          else s0 = mfma32(rf[i], kr[kk], s0);
        }
        if (i + PF < NA) rf[i + PF] = aop(i + PF);
        __builtin_amdgcn_sched_barrier(0);
      }
      // X^T operand of the accumulation (dO^T for dV, Q^T for dK), first reads
      const uint16_t* xt = DK ? q : d_o;
      bf16x8 cf[NC];
#pragma unroll
      for (int j = 0; j < PF; ++j) cf[j] = tl.col8(xt, j / NMT, j % NMT);

      // P (or dS) as the B operand: register 8*ks + e holds query kperm(ks,hf,e)
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // masked scores enter the exponential as -inf (P = 0): no branch
        const int qr = crow(r, hf);
        const bool ok = (qr < nq) & (key < a.RK) & (key <= a.qoff + i0 + qr);
        const float sc = ok ? (DK ? s0[r] : s0[r] + s1[r]) : -kInf;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc, a.s2, -lse4[r >> 2][r & 3]));
        pb[r >> 3][r & 7] = to_bf16(DK ? p * (s1[r] - dv4[r >> 2][r & 3]) : p);
      }
      __builtin_amdgcn_sched_barrier(0);

      // dV^T (or dK^T)[d][key] += sum_query X^T[d][query] pb[query][key]
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        acc[j % NMT] = mfma32(cf[j], pb[j / NMT], acc[j % NMT]);
        if (j + PF < NC) cf[j + PF] = tl.col8(xt, (j + PF) / NMT, (j + PF) % NMT);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the next block's LSE and D, then: block t+1 has landed and every read of
    // buffer cb has returned
    if (t + 1 < nblk && wave == 0 && lane < kBN) {
      s_lse2[cb ^ 1][lane] = l2n;
      s_dval[cb ^ 1][lane] = dvn;
    }
    ring_barrier<0>();
  }

  if (has_keys && key < a.RK) {
    const float mul = DK ? a.scale : 1.f;
    float* op = a.kv_part + ((((size_t)(DK ? g : 0) + hh) * a.hkv + kv) * a.RK + key) * D + 4 * hf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc[mt][4 * r4 + 0] * mul;
        v.y = acc[mt][4 * r4 + 1] * mul;
        v.z = acc[mt][4 * r4 + 2] * mul;
        v.w = acc[mt][4 * r4 + 3] * mul;
        *reinterpret_cast<float4*>(op + 32 * mt + 8 * r4) = v;
      }
    }
  }
}

// Response dV and dK in one launch, one workgroup (four waves) per (KV head,
// query head of the group, kind, four key blocks), key blocks fastest: the dV
// and dK partials run side by side.  Work items are dealt to the XCDs in
// contiguous ranges, so the items of a query head -- which all copy that
// head's Q and dO tiles -- share one XCD's L2.  64 KiB of LDS per workgroup.
template <int D>
__global__ void __launch_bounds__(256, 1) k_bwd_resp_kv(const AttnArgs a) {
  constexpr int TILE = kBN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];  // Q x2, dO x2
  __shared__ __attribute__((aligned(16))) float s_lse2[2][kBN], s_dval[2][kBN];
  const int g = a.hq / a.hkv;
  const int nkb4 = ((a.RK + kBN - 1) / kBN + 3) / 4;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int kb4 = w % nkb4;
  const int rest = w / nkb4;
  const int dk = rest & 1;
  const int hh = (rest >> 1) % g;
  const int kv = (rest >> 1) / g;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (!dk) resp_kv_block<D, false>(a, kv, hh, 4 * kb4, smem, s_lse2, s_dval, wave, lane);
  else resp_kv_block<D, true>(a, kv, hh, 4 * kb4, smem, s_lse2, s_dval, wave, lane);
}

hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, bool resp, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), b(512);
  if (head_dim == 256) {
    if (resp) hipLaunchKernelGGL((k_bwd_dq<256, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dq<256, false>), g, b, 0, s, a);
  } else {
    if (resp) hipLaunchKernelGGL((k_bwd_dq<128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_bwd_dq<128, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int head_dim, hipStream_t s) {
  const int nkb4 = ((a.RK + kBN - 1) / kBN + 3) / 4;
  dim3 g(nkb4 * a.hkv * 2 * (a.hq / a.hkv)), b(256);
  if (head_dim == 256) hipLaunchKernelGGL((k_bwd_resp_kv<256>), g, b, 0, s, a);
  else hipLaunchKernelGGL((k_bwd_resp_kv<128>), g, b, 0, s, a);
  return hipGetLastError();
}

}  // namespace ls
