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
// dQ kernel mapping (4 waves x 32 query rows): per key block
//   S^T  = K Q^T      (A = K rows from LDS, B = Q in registers)
//   dP^T = V dO^T     (A = V rows from LDS, B = dO in registers)
//   dS^T = P^T (dP^T - D)                    with P^T = exp2(S^T*s*log2e - LSE*log2e)
//   dQ^T += K^T dS^T  (A = K^T gathered from the same K tile, B = dS^T in registers)
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

// One pipelined step of the prompt dQ loop: S(b+1) = K(b+1) Q^T and
// dP(b+1) = V(b+1) dO^T, dS(b) on the VALU, then dQ^T += K(b)^T dS(b)^T, and
// the copies of K(b+3) and V(b+4).  As in the forward, the step is a fixed
// sequence of sched_barrier-fenced micro-segments that keeps the wave's LDS
// read stream continuous: one MFMA each, the operand read PF MFMAs ahead, one
// dS element every second score segment, one copy every second dQ segment.
template <int D>
__device__ __forceinline__ void bwd_step(const Lanes32<D>& tl, const BlockLoader<D>& ldr,
                                         const uint16_t* kn, const uint16_t* vn,
                                         const uint16_t* kc, const bf16x8 (&qr)[D / 16],
                                         const bf16x8 (&dor)[D / 16], f32x16& s_cur,
                                         f32x16& dp_cur, f32x16 (&acc)[D / 32], float s2,
                                         float lse2, float dval, uint32_t kdst, i32x4 kdesc,
                                         uint32_t vdst, i32x4 vdesc) {
  constexpr int NS = D / 16;   // k-steps of the score products = dQ MFMAs per step
  constexpr int NA = 2 * NS;   // score + dP MFMAs per step
  constexpr int NMT = D / 32;
  constexpr int PF = 4;        // LDS prefetch distance, in MFMAs
  constexpr int NIW = BlockLoader<D>::NIW;
  static_assert(2 * NIW * 2 == NS, "one copy instruction every second dQ MFMA");
  bf16x8 rf[NA], cf[NS];
#pragma unroll
  for (int i = 0; i < PF; ++i) rf[i] = (i & 1) ? tl.row8(vn, i >> 1) : tl.row8(kn, i >> 1);
  f32x16 s_next, dp_next;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s_next[r] = 0.f;
    dp_next[r] = 0.f;
  }
  bf16x8 dsb[2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    if (i & 1) dp_next = mfma32(rf[i], dor[i >> 1], dp_next);
    else s_next = mfma32(rf[i], qr[i >> 1], s_next);
    if (i + PF < NA) {
      const int n = i + PF;
      rf[n] = (n & 1) ? tl.row8(vn, n >> 1) : tl.row8(kn, n >> 1);
    } else {
      const int j = i + PF - NA;
      cf[j] = tl.col8(kc, j / NMT, j % NMT);
    }
    if (i & 1) {
#pragma unroll
      for (int r = (i >> 1) * 16 / NS; r < ((i >> 1) + 1) * 16 / NS; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], s2, -lse2));
        dsb[r >> 3][r & 7] = to_bf16(p * (dp_cur[r] - dval));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
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
  s_cur = s_next;
  dp_cur = dp_next;
}

template <int D, bool RESP>
__global__ void __launch_bounds__(256, 1) k_bwd_dq(const AttnArgs a) {
  constexpr int NKK = D / 16;
  constexpr int NMT = D / 32;
  constexpr int TILE = kBN * D;
  constexpr int NST = kStages;
  constexpr int NIW = BlockLoader<D>::NIW;  // copy instructions per wave per tile
  static_assert(NST == 4, "the ring has four stages");
  // one array per ring stage (distinct LDS objects; see the forward kernel)
  __shared__ __attribute__((aligned(1024))) uint16_t k0[TILE], k1[TILE], k2[TILE], k3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0[TILE], v1[TILE], v2[TILE], v3[TILE];
  uint16_t* const kst[NST] = {k0, k1, k2, k3};
  uint16_t* const vst[NST] = {v0, v1, v2, v3};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, lq = lane & 31;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int per_unit = a.mtiles * a.hkv;
  const int unit = w / per_unit;
  const int rem = w - unit * per_unit;
  const int kv = rem / a.mtiles;
  const int mtile = rem - kv * a.mtiles;
  const int GR = (a.hq / a.hkv) * a.R;
  const int m0 = mtile * kBwdRows;
  const int m = m0 + 32 * wave + lq;
  const bool rvalid = m < GR;
  const size_t row0 = (size_t)kv * GR;
  const size_t row = row0 + min(m, GR - 1);
  const int qi = m % a.R;

  const KeyWalk<D, RESP> walk(a, kv, unit, m0, kBwdRows);
  const int nblocks = walk.nblocks;
  const int nfull = walk.nfull;
  const int slot = a.slot_base + unit;

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

  f32x16 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  const Lanes32<D> tl(hf, lq);
  const BlockLoader<D> ldr(wave, lane);

  // ---- pipelined loop over the full (unmasked) blocks.  Step b waits for
  // K(b+1) and V(b+1), starts K(b+3) and V(b+4), computes S(b+1) and dP(b+1)
  // while turning S(b), dP(b) into dS(b), then accumulates K(b)^T dS(b).  K(b)
  // stays resident for two steps (scores, then dQ), so K runs three blocks
  // ahead and V four.  Every step issues the same number of copies (blocks
  // past the range re-read block 0), so each wait is a fixed vmcnt.
  if (nfull > 0) {
    wait_loads_le<0>();  // Q, dO, LSE, D have landed (the copies are invisible to the compiler)
    // All V copies of one loop iteration (blocks b+4 .. b+7) fall in one page,
    // whose pool offset is looked up one iteration ahead.
    constexpr size_t kBlk = (size_t)kBN * D;
    constexpr unsigned kBlkBytes = kBN * D * 2;
    int ph_next = walk.page_id(0);          // page of the blocks the next iteration copies
    size_t pcur = walk.page_base(ph_next);  // offset of the page this iteration copies from
    size_t koff[NST];      // source offset of block j, kept from V(j)'s copy to K(j)'s
#define LS_ISSUE_V(j, st)                                    \
  do {                                                       \
    koff[st] = (j) < nfull ? pcur + ((j) & 7) * kBlk : 0;    \
    load_block(ldr, vst[st], a.v + koff[st], kBN);           \
  } while (0)
#define LS_ISSUE_K(st) load_block(ldr, kst[st], a.k + koff[st], kBN)
    LS_ISSUE_V(0, 0);
    LS_ISSUE_K(0);
    LS_ISSUE_V(1, 1);
    LS_ISSUE_K(1);
    LS_ISSUE_V(2, 2);
    LS_ISSUE_K(2);
    LS_ISSUE_V(3, 3);
    ring_barrier<5 * NIW>();  // V(0), K(0) landed
    f32x16 s_cur, dp_cur;
    block_sdp<D>(tl, kst[0], vst[0], qr, dor, s_cur, dp_cur);
#define LS_BWD_STEP(ST)                                                                  \
  if (b + (ST) < nfull) {                                                                \
    /* K(b+1), V(b+1) landed; K stage ST-1 and V stage ST are free */                   \
    ring_barrier<3 * NIW>();                                                             \
    constexpr int SK = ((ST) + 3) % NST; /* K(b+3) goes where K(b-1) was */              \
    const int jv = b + (ST) + 4;         /* V(b+4) goes where V(b) was */                \
    koff[ST] = jv < nfull ? pcur + (jv & 7) * kBlk : 0;                                  \
    bwd_step<D>(tl, ldr, kst[((ST) + 1) % NST], vst[((ST) + 1) % NST], kst[ST], qr, dor,  \
                s_cur, dp_cur, acc, a.s2, lse2, dval, lds_addr(kst[SK]),                 \
                block_desc(a.k + koff[SK], kBlkBytes), lds_addr(vst[ST]),                \
                block_desc(a.v + koff[ST], kBlkBytes));                                  \
  }
    for (int b = 0; b < nfull; b += NST) {
      pcur = walk.page_base(ph_next);
      ph_next = b + 8 < nfull ? walk.page_id((b + 8) >> 3) : -1;
      LS_BWD_STEP(0)
      LS_BWD_STEP(1)
      LS_BWD_STEP(2)
      LS_BWD_STEP(3)
    }
#undef LS_BWD_STEP
#undef LS_ISSUE_K
#undef LS_ISSUE_V
    wait_loads_le<0>();  // drain the look-ahead copies before LDS is reused
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
      f32x16 s, dp;
      block_sdp<D>(tl, k0, v0, qr, dor, s, dp);
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
      block_dq<D>(acc, tl, k0, dsb);
    }
    __syncthreads();  // tiles are rewritten by the next block
  }

  if (rvalid) {
    const size_t rows_total = (size_t)a.hq * a.R;
    float* op = a.dq_slots + ((size_t)slot * rows_total + row0 + m) * D + 4 * hf;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = acc[mt][4 * r4 + 0] * a.scale;
        v.y = acc[mt][4 * r4 + 1] * a.scale;
        v.z = acc[mt][4 * r4 + 2] * a.scale;
        v.w = acc[mt][4 * r4 + 3] * a.scale;
        *reinterpret_cast<float4*>(op + 32 * mt + 8 * r4) = v;
      }
    }
  }
}

// dK or dV of 32 response keys [j0, j0+32) of KV head kv from the query head
// kv*g + blockIdx.z, one wave per workgroup, key-stationary: loops over the
// query rows i of that head that see the keys (qoff + i >= j0, in blocks of
// 32 from i = max(0, j0 - qoff)), accumulating
//   DV:  dV^T[d][key] += sum_query dO[query][d] P[query][key]
//   DK:  dK^T[d][key] += sum_query Q[query][d]  dS[query][key]
// with S = Q K^T and dP = dO V^T recomputed in the (query x key) orientation.
// Each head writes its own fp32 partial (k_kv_reduce sums the g heads of a
// group in head order), so the launch has g times more workgroups than key
// blocks and needs no atomics.  dV and dK are separate launches so each needs
// only one 128-register accumulator set.
template <int D, bool DK>
__global__ void __launch_bounds__(64, 1) k_bwd_resp_kv(const AttnArgs a) {
  constexpr int NKK = D / 16;
  constexpr int NMT = D / 32;
  constexpr int TILE = kBN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];  // K_r, V_r, Q, dO
  __shared__ float s_lse2[kBN], s_dval[kBN];

  const int lane = threadIdx.x, hf = lane >> 5, lq = lane & 31;
  const int kv = blockIdx.y;
  const int hh = blockIdx.z;  // query head within the group
  const int j0 = blockIdx.x * kBN;
  const int g = a.hq / a.hkv;
  uint16_t* kt = smem;
  uint16_t* vt = smem + TILE;
  uint16_t* qt = smem + 2 * TILE;
  uint16_t* dt = smem + 3 * TILE;

  const int nkeys = min(kBN, a.RK - j0);
  {
    const size_t off = ((size_t)kv * a.kvr + j0) * D;
    tile_load_async<D, 1>(kt, a.k + off, nkeys, 0, lane);
    if (DK) tile_load_async<D, 1>(vt, a.v + off, nkeys, 0, lane);
  }
  const Lanes32<D> tl(hf, lq);
  const int key = j0 + lq;  // this lane's key column

  f32x16 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  {
    const int h = kv * g + hh;
    for (int i0 = max(0, j0 - a.qoff); i0 < a.R; i0 += kBN) {
      const int nq = min(kBN, a.R - i0);
      const size_t qoff = ((size_t)h * a.R + i0) * D;
      __syncthreads();  // previous block's reads of qt/dt and s_* are done
      tile_load_async<D, 1>(qt, a.q + qoff, nq, 0, lane);
      tile_load_async<D, 1>(dt, a.d_o + qoff, nq, 0, lane);
      if (lane < kBN) {
        const bool ok = lane < nq;
        const size_t r = (size_t)h * a.R + i0 + (ok ? lane : 0);
        s_lse2[lane] = ok ? a.lse[r] * kLog2e : kInf;
        s_dval[lane] = ok ? a.dvals[r] : 0.f;
      }
      wait_async_loads();
      __syncthreads();

      // S[query][key] = sum_d Q[query][d] K[key][d]; dP likewise with dO, V
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma32(tl.row8(qt, kk), tl.row8(kt, kk), s);
        if (DK) dp = mfma32(tl.row8(dt, kk), tl.row8(vt, kk), dp);
      }

      // P (or dS) as the B operand: register 8*ks + e holds query kperm(ks,hf,e)
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = crow(r, hf);
        const bool ok = (q < nq) && (key < a.RK) && (key <= a.qoff + i0 + q);
        const float p = ok ? __builtin_amdgcn_exp2f(s[r] * a.s2 - s_lse2[q]) : 0.f;
        const float val = DK ? p * (dp[r] - s_dval[q]) : p;
        pb[r >> 3][r & 7] = to_bf16(val);
      }

      // dV^T (or dK^T)[d][key] += sum_query X^T[d][query] pb[query][key]
      const uint16_t* xt = DK ? qt : dt;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma32(tl.col8(xt, ks, mt), pb[ks], acc[mt]);
      }
    }
  }

  if (key < a.RK) {
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

hipError_t launch_bwd_dq(const AttnArgs& a, int head_dim, bool resp, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), b(256);
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
  dim3 g((a.RK + kBN - 1) / kBN, a.hkv, a.hq / a.hkv), b(64);
  if (head_dim == 256) {
    hipLaunchKernelGGL((k_bwd_resp_kv<256, false>), g, b, 0, s, a);
    hipLaunchKernelGGL((k_bwd_resp_kv<256, true>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_bwd_resp_kv<128, false>), g, b, 0, s, a);
    hipLaunchKernelGGL((k_bwd_resp_kv<128, true>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ls
