// Device helpers for the gfx950 kernels: bf16 MFMA operand types, the
// 32x32x16 MFMA, operand/accumulator lane layouts, and the XCD-aware
// workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ls_internal.hpp"

namespace ls {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();
// Largest score excess over the exp2 shift (log2 units) accepted without a
// recompute: p = exp2(x - m) <= 2^32 keeps every fp32 sum over up to 2^31
// keys finite for |v| < 2^60.
constexpr float kShiftSlack = 32.0f;

// D += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Operand layout (lane l, half hf = l/32, element t = 0..7):
//   A: row l%32, k = 8*hf + t;   B: column l%32, k = 8*hf + t.
// Accumulator layout: register r holds row crow(r, hf), column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ constexpr int crow(int r, int hf) {
  return 8 * (r >> 2) + 4 * hf + (r & 3);
}

// When an accumulator tile whose rows are keys (or queries) is fed back as the
// B operand of a second MFMA contracting over those rows, register 8*ks + t
// of lane half hf becomes k-element 8*hf + t of k-step ks.  The row it holds
// is kperm(ks, hf, t); the matching A operand must be gathered with the same
// map so both sides of the contraction agree on the order.
__device__ __forceinline__ constexpr int kperm(int ks, int hf, int t) {
  return 16 * ks + 8 * (t >> 2) + 4 * hf + (t & 3);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

// ---- LDS tiles of 32 rows x D bf16 (one K or V block), unpadded.
// 16-byte chunk c of row r is stored at chunk position c ^ swf(r), where swf
// swaps the two 2-bit halves of r & 15.  Rows are 512 B (d = 256) or 256 B
// apart, so without a swizzle every row starts in the same LDS bank; with this
// one, on the 64 x 4-byte banks of gfx950,
//   * a row-operand read (16 B per lane, 16 consecutive rows per bank pass)
//     hits 16 distinct 16-byte bank groups, and
//   * a transpose read (8 B per lane; each 32-lane pass reads the same 64-byte
//     column range of 4 consecutive rows, for 2 lane halves) lands the 4 rows
//     in 4 distinct 64-byte bank groups,
// so both are free of bank conflicts; and a wave can still fill 1 KB of the
// tile with one direct global->LDS copy.
__device__ __forceinline__ constexpr int swf(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 3) ^ swf(row))) << 3) + (col & 7);
}

// ---- 32x32x16 tiles (a wave owns 32 query rows)
// Lane-dependent parts of the swizzled LDS addresses, computed once per kernel
// so that every tile access inside the key loop is "base register +
// compile-time immediate" (otherwise the compiler hoists one address register
// per access out of the loop and runs out of registers).
//
// Row operand of k-step kk: row lq, 16-byte chunk 2*kk + hf:
//     lq*D + 8*((2*kk + hf) ^ swf(lq))  =  rb[kk & 7] + 128*(kk >> 3)
//
// Column operand of (ks, mt): column 32*mt + lq at rows kperm(ks, hf, 0..7),
// read with ds_read_b64_tr_b16.  That instruction works on groups of 16 lanes:
// lane i of a group receives, as element e, the 16-bit word (i & 3) of the
// 8 bytes addressed by lane 4*e + (i >> 2) of the same group.  So lane
// L = 4*e' + j' (L = lane & 15) supplies, for read c (elements 4c..4c+3), the
// address of row 16*ks + 8*c + 4*hf + e' and columns
// 32*mt + 16*((lane >> 4) & 1) + 4*j' + [0, 4).  Under the swizzle
// (swf of that row = 4*e' + 2*c + hf) this is
//     tb[c][mt & 3] + (16*ks + 8*c)*D + 128*(mt >> 2).
template <int D>
struct Lanes32 {
  int rb[8];
  int tb[2][4];
  __device__ __forceinline__ Lanes32(int hf, int lq) {
#pragma unroll
    for (int k7 = 0; k7 < 8; ++k7) rb[k7] = lq * D + 8 * ((2 * k7 + hf) ^ swf(lq));
    const int L = lq & 15, g1 = (lq >> 4) & 1, e = L >> 2;
    const int b0 = ((L >> 1) & 1) ^ hf;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int m3 = 0; m3 < 4; ++m3)
        tb[c][m3] = (4 * hf + e) * D + 8 * (b0 + 2 * (g1 ^ c) + 4 * (m3 ^ e)) + 4 * (L & 1);
  }
  // 16-byte row operand of k-step kk: row lq, elements [16*kk + 8*hf, +8).
  __device__ __forceinline__ bf16x8 row8(const uint16_t* tile, int kk) const {
    return ld_bf16x8(tile + rb[kk & 7] + 128 * (kk >> 3));
  }
  // 8 values of column 32*mt + lq at rows kperm(ks, hf, 0..7).
  __device__ __forceinline__ bf16x8 col8(const uint16_t* tile, int ks, int mt) const {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint16_t* base = tile + 16 * ks * D + 128 * (mt >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + tb[0][mt & 3]));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * D + tb[1][mt & 3]));
    const s16x4 v[2] = {lo, hi};
    u16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (unsigned short)v[t >> 2][t & 3];
    return __builtin_bit_cast(bf16x8, r);
  }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Asynchronous copy of a [32][D] bf16 block at `g` (row stride D) into an LDS
// tile, spread over the NW waves of the workgroup (global_load_lds_dwordx4:
// lane i of a wave instruction lands at LDS base + 16*i).  Rows >= nvalid
// (nvalid >= 1) re-read row nvalid-1, so the tile always holds finite data;
// callers mask those rows.  Completion: s_waitcnt vmcnt(0) + barrier.
template <int D, int NW = 4>
__device__ __forceinline__ void tile_load_async(uint16_t* tile, const uint16_t* g, int nvalid,
                                                int wave, int lane) {
  constexpr int NIW = (kBN * D * 2 / 1024) / NW;  // wave instructions per wave
  static_assert(NIW * NW * 1024 == kBN * D * 2, "tile must split evenly over the waves");
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int blk = wave * NIW + j;
    const int e = blk * 512 + 8 * lane;           // element offset this lane fills
    const int row = e / D;
    const int c = ((e % D) >> 3) ^ swf(row);       // logical chunk stored there
    const int rr = row < nvalid ? row : nvalid - 1;
    __builtin_amdgcn_global_load_lds(g + (size_t)rr * D + c * 8, (lds_ptr_t)(tile + blk * 512),
                                     16, 0, 0);
  }
}

// Keys seen by one work item, in blocks of kBN: either a chunk of one split's
// prompt pages (walked through the page table) or the causal response block.
// Page ids out of range are skipped (treated as empty), so a corrupted device
// page table can never make a kernel read outside the pools.
template <int D, bool RESP>
struct KeyWalk {
  const AttnArgs& a;
  int kv, p0, nblocks;
  // unit = split*chunks + chunk (paged); rows [m0, m0 + rows) of the group
  __device__ __forceinline__ KeyWalk(const AttnArgs& args, int kv_, int unit, int m0, int rows)
      : a(args), kv(kv_), p0(0), nblocks(0) {
    const int GR = (a.hq / a.hkv) * a.R;
    if (RESP) {
      const int mlast = min(m0 + rows, GR) - 1;
      const int imax = (m0 / a.R != mlast / a.R) ? a.R - 1 : mlast % a.R;
      nblocks = (imax + kBN) / kBN;
    } else {
      const int c = unit / a.chunks, k = unit - c * a.chunks;
      int s0 = a.offs[c], s1 = a.offs[c + 1];
      s0 = min(max(s0, 0), a.num_pages);
      s1 = min(max(s1, s0), a.num_pages);
      p0 = s0 + k * a.chunk_pages;
      const int p1 = min(s1, p0 + a.chunk_pages);
      nblocks = max(0, p1 - p0) * (kPage / kBN);
    }
  }
  // block b: base pointers of its K and V rows, number of valid keys, index of
  // its first key (response mode; 0 for prompt pages)
  __device__ __forceinline__ void src(int b, const uint16_t*& kb, const uint16_t*& vb, int& nvalid,
                                      int& key0) const {
    if (RESP) {
      key0 = b * kBN;
      nvalid = min(kBN, a.R - key0);
      const size_t off = ((size_t)kv * a.R + key0) * D;
      kb = a.k + off;
      vb = a.v + off;
    } else {
      key0 = 0;
      nvalid = 0;
      kb = vb = a.k;
      const int lp = a.order[p0 + b / (kPage / kBN)];
      const int tok = (b % (kPage / kBN)) * kBN;
      if (lp >= 0 && lp < a.num_pages) {
        const int ph = a.l2p[lp];
        if (ph >= 0 && ph < a.num_phys) {
          const int64_t left = a.prompt_len - (int64_t)lp * kPage - tok;
          nvalid = (int)(left < 0 ? 0 : (left > kBN ? kBN : left));
          const size_t off = (((size_t)ph * a.hkv + kv) * kPage + tok) * D;
          kb = a.k + off;
          vb = a.v + off;
        }
      }
    }
  }
  // start the asynchronous copy of block b's K and V into tiles kt, vt
  __device__ __forceinline__ void issue(int b, uint16_t* kt, uint16_t* vt, int wave, int lane,
                                        int& nvalid, int& key0) const {
    const uint16_t *kb, *vb;
    src(b, kb, vb, nvalid, key0);
    if (nvalid > 0) {
      tile_load_async<D>(kt, kb, nvalid, wave, lane);
      tile_load_async<D>(vt, vb, nvalid, wave, lane);
    }
  }
};

__device__ __forceinline__ void wait_async_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// acc *= alpha for an accumulator tile that lives in AGPRs.  Plain C++ would
// make the compiler give the loop-carried accumulators VGPR class (VALU cannot
// read AGPRs) and copy every one of them AGPR<->VGPR on every iteration; the
// in-place read/multiply/write keeps them in AGPRs.  Only used on the rare
// rescale path, long after the MFMAs that wrote these registers.
__device__ __forceinline__ void scale_acc(f32x4& acc, float alpha) {
  float x0 = acc[0], x1 = acc[1], x2 = acc[2], x3 = acc[3], t;
  asm volatile(
      "v_accvgpr_read_b32 %4, %0\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %4, %1\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %1, %4\n\t"
      "v_accvgpr_read_b32 %4, %2\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %2, %4\n\t"
      "v_accvgpr_read_b32 %4, %3\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %3, %4"
      : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(t)
      : "v"(alpha));
  acc = f32x4{x0, x1, x2, x3};
}
// Zero an accumulator tile directly in AGPRs (see scale_acc).
__device__ __forceinline__ void zero_acc(f32x4& acc) {
  float x0, x1, x2, x3;
  asm volatile(
      "v_accvgpr_write_b32 %0, 0\n\t"
      "v_accvgpr_write_b32 %1, 0\n\t"
      "v_accvgpr_write_b32 %2, 0\n\t"
      "v_accvgpr_write_b32 %3, 0"
      : "=a"(x0), "=a"(x1), "=a"(x2), "=a"(x3));
  acc = f32x4{x0, x1, x2, x3};
}
// Copy an AGPR accumulator tile to ordinary registers (see scale_acc).
__device__ __forceinline__ f32x4 read_acc(const f32x4& acc) {
  float x0 = acc[0], x1 = acc[1], x2 = acc[2], x3 = acc[3], y0, y1, y2, y3;
  asm volatile(
      "v_accvgpr_read_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %1, %5\n\t"
      "v_accvgpr_read_b32 %2, %6\n\t"
      "v_accvgpr_read_b32 %3, %7"
      : "=v"(y0), "=v"(y1), "=v"(y2), "=v"(y3)
      : "a"(x0), "a"(x1), "a"(x2), "a"(x3));
  return f32x4{y0, y1, y2, y3};
}
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 part = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    scale_acc(part, alpha);
    acc[4 * q] = part[0];
    acc[4 * q + 1] = part[1];
    acc[4 * q + 2] = part[2];
    acc[4 * q + 3] = part[3];
  }
}

__device__ __forceinline__ f32x4 read_acc4(const f32x16& acc, int q) {
  const f32x4 part = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  return read_acc(part);
}

// fp32 -> bf16 with round-to-nearest-even.
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// The hardware deals workgroups to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  Give XCD x the contiguous range of work items
// [x*q + min(x, r), ...) so that neighbouring items -- which read the same K/V
// pages -- share one XCD's L2.  Bijective for any n.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, x = bid & 7, s = bid >> 3;
  return x * q + (x < r ? x : r) + s;
}

__device__ __forceinline__ float wave_max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace ls
