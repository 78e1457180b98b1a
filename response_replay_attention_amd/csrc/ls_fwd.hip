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
//     V^T operand is gathered from the row-major V tile; O^T keeps one query
//     per lane, so the rescale and the final 1/l are per-lane scalars;
//   * K/V blocks of 32 keys are double-buffered in LDS, filled by direct
//     global->LDS copies issued one block ahead;
//   * the exp2 shift is fixed at the first block's max instead of being
//     raised as the running max grows, so no accumulator is ever rescaled; an
//     input whose scores later exceed the shift by more than 2^32 is detected
//     and its key range recomputed with the true max as the shift.
#include "ls_device.hpp"

namespace ls {

template <int D, bool RESP>
__global__ void __launch_bounds__(256, 1) k_fwd(const AttnArgs a) {
  constexpr int NKK = D / 16;           // 16-deep k-steps over head_dim for S
  constexpr int NMT = D / 32;           // 32-wide head_dim tiles of O^T
  constexpr int TILE = kBN * D;         // elements of one K or V block
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];  // [buf][K,V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, lq = lane & 31;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int per_unit = a.mtiles * a.hkv;
  const int unit = w / per_unit;
  const int rem = w - unit * per_unit;
  const int kv = rem / a.mtiles;
  const int mtile = rem - kv * a.mtiles;
  const int g = a.hq / a.hkv;
  const int GR = g * a.R;
  const int m0 = mtile * kFwdRows;
  const int m = m0 + 32 * wave + lq;     // this lane's query row within the group
  const size_t row0 = (size_t)kv * GR;

  const KeyWalk<D, RESP> walk(a, kv, unit, m0, kFwdRows);
  const int nblocks = walk.nblocks;
  const int slot = a.slot_base + unit;

  // ---- Q (B operand): column = query m, k = 16*kk + 8*hf + e.  Rows past the
  // group are computed on a copy of its last row and never stored.
  bf16x8 qr[NKK];
  const int qi = m % a.R;
  {
    const uint16_t* qp = a.q + (row0 + min(m, GR - 1)) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qr[kk] = ld_bf16x8(qp + 16 * kk);
  }

  auto issue = [&](int b, int buf, int& nvalid, int& key0) {
    walk.issue(b, smem + buf * 2 * TILE, smem + buf * 2 * TILE + TILE, wave, lane, nvalid, key0);
  };

  f32x16 acc[NMT];
  float mref = -kInf;   // exp2 shift of this query (log2 units)
  float mtrue = -kInf;  // running max of this query's scores
  float lsum = 0.f;
  const Lanes32<D> tl(hf, lq);

  // Pass 0 fixes the shift at the first block's max and never rescales the
  // accumulators; a score more than 2^kShiftSlack above the shift marks the
  // pass as unsafe (fp32 overflow risk) and pass 1 redoes the key range with
  // the true max as the shift.  Keeping the accumulators free of any VALU
  // access inside the loop lets them stay in AGPRs.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
    lsum = 0.f;
    if (pass == 1) mref = mtrue;
    bool unsafe = false;

    int cur_nv = 0, cur_k0 = 0;
    if (nblocks > 0) issue(0, 0, cur_nv, cur_k0);
    wait_async_loads();
    __syncthreads();

    // one key block; BUF is a compile-time buffer index so LDS offsets are immediates
    auto step = [&](int b, auto buf_tag) {
      constexpr int BUF = decltype(buf_tag)::value;
      int nx_nv = 0, nx_k0 = 0;
      // the other buffer was last read in block b-1, before the barrier that ended it
      if (b + 1 < nblocks) issue(b + 1, BUF ^ 1, nx_nv, nx_k0);

      if (cur_nv > 0) {
        const uint16_t* kl = smem + BUF * 2 * TILE;
        const uint16_t* vl = kl + TILE;

        // S^T[key][query] = sum_d K[key][d] Q[query][d]
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) s = mfma32(tl.row8(kl, kk), qr[kk], s);

        // scale to log2 units, mask, block max of this query (lanes l, l^32)
        float mx = -kInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = crow(r, hf);
          bool ok = key < cur_nv;
          if (RESP) ok = ok && (cur_k0 + key <= qi);
          const float x = ok ? s[r] * a.s2 : -kInf;
          s[r] = x;
          mx = fmaxf(mx, x);
        }
        const float mb = wave_max_halves(mx);
        mtrue = fmaxf(mtrue, mb);
        if (pass == 0) {
          if (mref == -kInf) mref = mb;
          unsafe = unsafe || (mb > mref + kShiftSlack);
        }

        // P^T = exp2(x - m) -> bf16 B operands (register 8*ks + e -> k-element e)
        bf16x8 pb[2];
        const float mu = (mref == -kInf) ? 0.f : mref;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[r] - mu);
          ls += p;
          pb[r >> 3][r & 7] = to_bf16(p);
        }
        lsum += ls;

        // O^T[d][query] += sum_key V[key][d] P^T[key][query]
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma32(tl.col8(vl, ks, mt), pb[ks], acc[mt]);
        }
      }

      cur_nv = nx_nv;
      cur_k0 = nx_k0;
      wait_async_loads();
      __syncthreads();
    };

    for (int b = 0; b < nblocks; b += 2) {
      step(b, IntC<0>{});
      if (b + 1 < nblocks) step(b + 1, IntC<1>{});
    }
    if (pass == 0 && !__syncthreads_or(unsafe ? 1 : 0)) break;
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
        const f32x4 x = read_acc4(acc[mt], r4);
        float4 v;
        v.x = x[0] * inv;
        v.y = x[1] * inv;
        v.z = x[2] * inv;
        v.w = x[3] * inv;
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
