// Small HBM-bound kernels of the replay path:
//   * the exact log-sum-exp merge of partial attention (the pages' global
//     LSE/output composition across CP ranks; LongStraw review page, section 7
//     mind map, "Qwen3.6-27B implementation"), also used to fold internal
//     sub-splits of one split back into that split's partial;
//   * D = rowsum(dO * O) for the backward;
//   * the ordered sum of the per-split dQ partials (the one-GPU stand-in for
//     the pages' dQ all-reduce; review page, section 2).
// All are streaming kernels: one pass over their inputs with 16-byte accesses.
#include "ls_device.hpp"

namespace ls {

// One row per D/4 threads; thread e4 owns elements [4*e4, 4*e4 + 4).
template <int D, bool FINAL>
__global__ void __launch_bounds__(256) k_merge(int nper, int64_t rows, const float* __restrict__ po,
                                               const float* __restrict__ pm,
                                               const float* __restrict__ pl, void* out_o,
                                               float* out_m, float* out_l) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int grp = blockIdx.y;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int e4 = threadIdx.x % TPR;
  if (row >= rows) return;
  const int c0 = grp * nper;

  // Parts are taken in batches of NB whose loads are all issued together (one
  // memory phase per batch).  Within a batch the weights are l_c e^{m_c - big}
  // with big the running maximum of m over the non-empty parts so far; when a
  // batch raises it, what was summed before is rescaled.  Parts are added in
  // index order; a part whose weight is 0 (empty, or underflowed) adds
  // nothing.  With at most NB parts this is the two-pass formula with the
  // global maximum, term for term.
  constexpr int NB = 12;
  float big = -kInf, tot = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int cb = 0; cb < nper; cb += NB) {
    float4 o[NB];
    float m[NB], l[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (cb + u < nper) {
        const size_t i = (size_t)(c0 + cb + u) * rows + row;
        o[u] = *reinterpret_cast<const float4*>(po + i * D + 4 * e4);
        m[u] = pm[i];
        l[u] = pl[i];
      } else {
        l[u] = 0.f;
      }
    }
    float bm = big;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (l[u] > 0.f) bm = fmaxf(bm, m[u]);
    if (bm > big) {
      if (big != -kInf) {
        const float r = expf(big - bm);
        tot *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
      }
      big = bm;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float w = l[u] > 0.f ? l[u] * expf(m[u] - big) : 0.f;
      if (w > 0.f) {
        tot += w;
        acc.x += w * o[u].x;
        acc.y += w * o[u].y;
        acc.z += w * o[u].z;
        acc.w += w * o[u].w;
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  if (FINAL) {
    __bf16* o = reinterpret_cast<__bf16*>(out_o) + row * D + 4 * e4;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v = {to_bf16(acc.x), to_bf16(acc.y), to_bf16(acc.z), to_bf16(acc.w)};
    *reinterpret_cast<bf16x4*>(o) = v;
    if (e4 == 0) out_m[row] = tot > 0.f ? big + logf(tot) : -kInf;  // LSE
  } else {
    const size_t i = (size_t)grp * rows + row;
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out_o) + i * D + 4 * e4) = acc;
    if (e4 == 0) {
      out_m[i] = tot > 0.f ? big : -kInf;
      out_l[i] = tot;
    }
  }
}

// D[row] = sum_d dO[row][d] * O[row][d]; D/8 lanes per row, 8 elements each.
template <int D>
__global__ void __launch_bounds__(256) k_bwd_dot(int64_t rows, const uint16_t* __restrict__ d_o,
                                                 const uint16_t* __restrict__ o,
                                                 float* __restrict__ dvals) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int e8 = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const u16x8 a = *reinterpret_cast<const u16x8*>(d_o + row * D + 8 * e8);
    const u16x8 b = *reinterpret_cast<const u16x8*>(o + row * D + 8 * e8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sum += __uint_as_float((uint32_t)a[e] << 16) * __uint_as_float((uint32_t)b[e] << 16);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (row < rows && e8 == 0) dvals[row] = sum;
}

// dq[e] = sum_{s < nslots} slots[s][e], in slot order (deterministic).
__global__ void __launch_bounds__(256) k_dq_reduce(int nslots, int64_t n4,
                                                   const float4* __restrict__ slots,
                                                   float4* __restrict__ dq) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 acc = slots[i];
    for (int s = 1; s < nslots; ++s) {
      const float4 v = slots[(size_t)s * n4 + i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    dq[i] = acc;
  }
}

// Physical slot of every page of the split-major list, resolved once per call
// so that the key loops read one table entry per page instead of a dependent
// pair of lookups.
__global__ void __launch_bounds__(256) k_resolve_pages(int32_t num_pages, int32_t num_phys,
                                                       const int32_t* __restrict__ order,
                                                       const int32_t* __restrict__ l2p,
                                                       int32_t* __restrict__ phys) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_pages) return;
  const int lp = order[i];
  int ph = -1;
  if (lp >= 0 && lp < num_pages) {
    const int t = l2p[lp];
    if (t >= 0 && t < num_phys) ph = t;
  }
  phys[i] = ph;
}

hipError_t launch_resolve_pages(int32_t num_pages, int32_t num_phys, const int32_t* order,
                                const int32_t* l2p, int32_t* phys, hipStream_t s) {
  if (num_pages <= 0) return hipSuccess;
  dim3 g((unsigned)((num_pages + 255) / 256)), b(256);
  hipLaunchKernelGGL(k_resolve_pages, g, b, 0, s, num_pages, num_phys, order, l2p, phys);
  return hipGetLastError();
}

// dv = sum over the g query heads of part[0], dk = sum of part[1], in head
// order (deterministic); part is [2][g][elems].
// Partials are [2][g][Hkv][rk][d]; element i of one [Hkv][rk][d] set goes to
// output row (kv, j) of a [Hkv][kvr][d] tensor.
__global__ void __launch_bounds__(256) k_kv_reduce(int g, int64_t n4, int64_t head4, int64_t ostride4,
                                                   int accum, const float4* __restrict__ part,
                                                   float4* __restrict__ dv, float4* __restrict__ dk) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kv = i / head4;
    const int64_t o = kv * ostride4 + (i - kv * head4);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const float4* p = part + (size_t)w * g * n4 + i;
      float4 acc = p[0];
      for (int h = 1; h < g; ++h) {
        const float4 v = p[(size_t)h * n4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      float4* out = (w == 0 ? dv : dk) + o;
      if (accum) {
        const float4 prev = *out;
        acc.x = prev.x + acc.x;
        acc.y = prev.y + acc.y;
        acc.z = prev.z + acc.z;
        acc.w = prev.w + acc.w;
      }
      *out = acc;
    }
  }
}

hipError_t launch_kv_reduce(int g, int hkv, int rk, int kvr, int head_dim, bool accum,
                            const float* part, float* dv, float* dk, hipStream_t s) {
  const int64_t head4 = (int64_t)rk * head_dim / 4;
  const int64_t n4 = hkv * head4;
  if (n4 <= 0) return hipSuccess;
  const int64_t want = (n4 + 255) / 256;
  dim3 gr((unsigned)(want < 4096 ? want : 4096)), b(256);
  hipLaunchKernelGGL(k_kv_reduce, gr, b, 0, s, g, n4, head4, (int64_t)kvr * head_dim / 4,
                     accum ? 1 : 0, reinterpret_cast<const float4*>(part),
                     reinterpret_cast<float4*>(dv), reinterpret_cast<float4*>(dk));
  return hipGetLastError();
}

// Page writer: K and V of one chunk of T captured tokens ([Hkv, T, d], row
// stride d) into pool slots ([phys, Hkv, 256, d]); token t of the chunk goes to
// slot slots[t / 256], row t % 256.  16-byte units, grid-stride; positions
// past T in the chunk's last page are not written, nor is a page whose slot
// lies outside the pool.
__global__ void __launch_bounds__(256) k_page_append(int hkv, int d8, int tokens, int64_t n16,
                                                     int num_phys,
                                                     const uint4* __restrict__ kc,
                                                     const uint4* __restrict__ vc,
                                                     const int32_t* __restrict__ slots,
                                                     uint4* __restrict__ kp, uint4* __restrict__ vp) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n16;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(u % d8);
    const int64_t r = u / d8;             // source row kv * T + t
    const int t = (int)(r % tokens);
    const int kv = (int)(r / tokens);
    const int slot = slots[t >> 8];
    if (slot < 0 || slot >= num_phys) continue;
    const int64_t dst = (((int64_t)slot * hkv + kv) * 256 + (t & 255)) * d8 + c;
    kp[dst] = kc[u];
    vp[dst] = vc[u];
  }
}

hipError_t launch_page_append(int hkv, int head_dim, int tokens, int num_phys,
                              const void* k_chunk, const void* v_chunk, const int32_t* slots,
                              void* k_pool, void* v_pool, hipStream_t s) {
  const int d8 = head_dim / 8;
  const int64_t n16 = (int64_t)hkv * tokens * d8;
  if (n16 <= 0) return hipSuccess;
  const int64_t want = (n16 + 255) / 256;
  dim3 g((unsigned)(want < 8192 ? want : 8192)), b(256);
  hipLaunchKernelGGL(k_page_append, g, b, 0, s, hkv, d8, tokens, n16, num_phys,
                     static_cast<const uint4*>(k_chunk), static_cast<const uint4*>(v_chunk), slots,
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool));
  return hipGetLastError();
}

hipError_t launch_merge(int groups, int nper, int64_t rows, int head_dim, const float* po,
                        const float* pm, const float* pl, bool final, void* out_o, float* out_m,
                        float* out_l, hipStream_t s) {
  if (rows <= 0 || groups <= 0) return hipSuccess;
  const int rpb = 256 / (head_dim / 4);
  dim3 g((unsigned)((rows + rpb - 1) / rpb), groups), b(256);
  if (head_dim == 256) {
    if (final) hipLaunchKernelGGL((k_merge<256, true>), g, b, 0, s, nper, rows, po, pm, pl, out_o, out_m, out_l);
    else hipLaunchKernelGGL((k_merge<256, false>), g, b, 0, s, nper, rows, po, pm, pl, out_o, out_m, out_l);
  } else {
    if (final) hipLaunchKernelGGL((k_merge<128, true>), g, b, 0, s, nper, rows, po, pm, pl, out_o, out_m, out_l);
    else hipLaunchKernelGGL((k_merge<128, false>), g, b, 0, s, nper, rows, po, pm, pl, out_o, out_m, out_l);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dot(int64_t rows, int head_dim, const uint16_t* d_o, const uint16_t* o,
                          float* dvals, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int rpb = 256 / (head_dim / 8);
  dim3 g((unsigned)((rows + rpb - 1) / rpb)), b(256);
  if (head_dim == 256) hipLaunchKernelGGL((k_bwd_dot<256>), g, b, 0, s, rows, d_o, o, dvals);
  else hipLaunchKernelGGL((k_bwd_dot<128>), g, b, 0, s, rows, d_o, o, dvals);
  return hipGetLastError();
}

hipError_t launch_dq_reduce(int nslots, int64_t elems, const float* slots, float* dq,
                            hipStream_t s) {
  const int64_t n4 = elems / 4;
  if (n4 <= 0) return hipSuccess;
  const int64_t want = (n4 + 255) / 256;
  dim3 g((unsigned)(want < 4096 ? want : 4096)), b(256);
  hipLaunchKernelGGL(k_dq_reduce, g, b, 0, s, nslots, n4, reinterpret_cast<const float4*>(slots),
                     reinterpret_cast<float4*>(dq));
  return hipGetLastError();
}

}  // namespace ls
