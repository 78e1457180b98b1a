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

// Forward tiles in chunk-major layouts.  K keeps the 16-byte chunk c (elements
// [8c, 8c+8)) of key row r in 16-byte slot c*32 + r; V keeps chunk C of row r
// in slot C*32 + (r ^ 4*(C & 3)).  With these, every operand read is one
// per-lane base register plus an immediate, so no address arithmetic sits
// between an MFMA and the read it waits for:
//   K row read, k-step kk:            kb + 1024*kk bytes
//   V transposed read (ks, mt, half): vb[half] + 2048*mt + 256*ks bytes
// and both are free of LDS bank conflicts for their own read pattern (64 banks
// of 4 bytes; checked on the CPU for every lane and read, together with the
// copies, at d = 128 and 256).  The registers the reads fill are the same as
// with the row-major swizzled tiles (row8 / col8 above).
template <int D>
struct LanesCM {
  int kb, vb0, vb1;  // byte offsets inside a tile
  __device__ __forceinline__ LanesCM(int hf, int lq) {
    kb = 512 * hf + 16 * lq;
    const int L = lq & 15, g1 = lq >> 4, q = 2 * g1 + ((L >> 1) & 1);
    vb0 = 512 * q + 16 * ((4 * hf + (L >> 2)) ^ (4 * q)) + 8 * (L & 1);
    vb1 = 512 * q + 16 * ((8 + 4 * hf + (L >> 2)) ^ (4 * q)) + 8 * (L & 1);
  }
  __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(kb), "+v"(vb0), "+v"(vb1)); }
  __device__ __forceinline__ bf16x8 row8(const uint16_t* tile, int kk) const {
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(tile) + kb + 1024 * kk));
  }
  __device__ __forceinline__ bf16x8 col8(const uint16_t* tile, int ks, int mt) const {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* base = reinterpret_cast<const char*>(tile) + 2048 * mt + 256 * ks;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + vb0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + vb1));
    const s16x4 v[2] = {lo, hi};
    u16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (unsigned short)v[t >> 2][t & 3];
    return __builtin_bit_cast(bf16x8, r);
  }
};

// Block copies through the buffer path: buffer_load_dwordx4 ... lds with a
// raw descriptor whose base is the block's first row (uniform, in SGPRs) and a
// per-lane byte offset that never changes, so a copy costs no per-lane address
// arithmetic.  The descriptor's record count is the block's valid bytes:
// reads past it return zero (hardware range check), which keeps the tail rows
// of a partial block finite without clamping.  Lane i of an instruction lands
// at M0 + 16*i.
//
// The copies are issued from inline asm on purpose: the compiler's own
// tracking of LDS DMA cannot tell the stages of a ring apart and makes reads
// of one stage wait for copies still in flight into another.  Ordering is
// explicit instead: a copy into a stage is issued only after a ring_barrier
// that follows the last read of that stage, and a stage is read only after a
// ring_barrier whose vmcnt covers its copy.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 block_desc(const void* base, unsigned nbytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)addr;
  r.y = (int)((addr >> 32) & 0xffffu);  // stride 0: raw buffer, byte records
  r.z = (int)nbytes;
  r.w = 0x00020000;                      // 32-bit data format, no swizzle
  return r;
}

// one wave instruction: 64 lanes x 16 bytes from desc+voff into LDS at lds
// (M0 is saved and restored around the copy)
__device__ __forceinline__ void copy16_to_lds(uint32_t lds, int voff, i32x4 desc) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(desc));
}

template <int D, int NW = 4>
struct BlockLoader {
  static constexpr int NIW = (kBN * D * 2 / 1024) / NW;  // wave instructions per block
  static_assert(NIW * NW * 1024 == kBN * D * 2, "tile must split evenly over the waves");
  int voff[NIW];  // byte offset of this lane's 16 bytes inside the source block
  int lds0;       // byte offset of this wave's first 1 KB piece inside a tile (uniform)
  __device__ __forceinline__ BlockLoader(int wave, int lane)
      : lds0(__builtin_amdgcn_readfirstlane(wave) * NIW * 1024) {
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int e = (wave * NIW + j) * 512 + 8 * lane;  // element position this lane fills
      const int row = e / D;
      voff[j] = 2 * (row * D + ((((e % D) >> 3) ^ swf(row)) << 3));
    }
  }
};

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Copy rows [0, nvalid) of the block at `src` (row stride D) into `tile`;
// rows past nvalid arrive as zeros.
template <int D, int NW>
__device__ __forceinline__ void load_block(const BlockLoader<D, NW>& L, uint16_t* tile,
                                           const uint16_t* src, int nvalid) {
  const i32x4 desc = block_desc(src, (unsigned)(nvalid * D * 2));
  const uint32_t base = lds_addr(tile) + L.lds0;
#pragma unroll
  for (int j = 0; j < BlockLoader<D, NW>::NIW; ++j) copy16_to_lds(base + j * 1024, L.voff[j], desc);
}

// Copies of [32][D] bf16 blocks into the chunk-major tiles of LanesCM, spread
// over NW waves: copy instruction j of wave w fills slots (w*NIW + j)*64 + lane,
// so lane (hl = lane / 32) reads the 16 bytes of chunk c = 2*(w*NIW + j) + hl of
// row lane % 32 (K; V: of row (lane % 32) ^ 4*(c & 3)).  The source offsets of
// copy 0 are kept; copy j adds 32*j bytes (the next chunk pair), and for V an
// odd j also flips row bit 3 (c & 3 differs by 2).
template <int D, int NW>
struct BlockLoaderCM {
  static constexpr int NIW = (kBN * D * 2 / 1024) / NW;  // wave instructions per block
  static_assert(NIW * NW * 1024 == kBN * D * 2 && NIW <= 2, "tile must split evenly over the waves");
  int vk, vv;  // byte offset of this lane's 16 bytes in the source block, copy 0 of K and of V
  int lds0;    // byte offset of this wave's first 1 KB piece inside a tile (uniform)
  __device__ __forceinline__ BlockLoaderCM(int wave, int lane)
      : lds0(__builtin_amdgcn_readfirstlane(wave) * NIW * 1024) {
    const int hl = lane >> 5;
    vk = (lane & 31) * 2 * D + 16 * hl + 32 * wave * NIW;
    vv = vk ^ (8 * D * ((wave * NIW * 2 + hl) & 3));
  }
  __device__ __forceinline__ int koff(int j) const { return vk + 32 * j; }
  __device__ __forceinline__ int voff(int j) const { return ((j & 1) ? (vv ^ (16 * D)) : vv) + 32 * j; }
  // copy instruction c of a step: K pieces first, then V
  __device__ __forceinline__ void issue(int c, uint32_t kdst, i32x4 kdesc, uint32_t vdst,
                                        i32x4 vdesc) const {
    if (c < NIW) copy16_to_lds(kdst + lds0 + c * 1024, koff(c), kdesc);
    else copy16_to_lds(vdst + lds0 + (c - NIW) * 1024, voff(c - NIW), vdesc);
  }
};

// Rows [0, nvalid) of the block at `src` into a chunk-major tile (K or V
// layout); bytes past the valid rows arrive as zeros.
template <bool V, int D, int NW>
__device__ __forceinline__ void load_block_cm(const BlockLoaderCM<D, NW>& L, uint16_t* tile,
                                              const uint16_t* src, int nvalid) {
  const i32x4 desc = block_desc(src, (unsigned)(nvalid * D * 2));
  const uint32_t base = lds_addr(tile) + L.lds0;
#pragma unroll
  for (int j = 0; j < BlockLoaderCM<D, NW>::NIW; ++j)
    copy16_to_lds(base + j * 1024, V ? L.voff(j) : L.koff(j), desc);
}

// Page-table entries are read through the constant address space: the tables
// never change while a kernel runs, and a uniform load from that space becomes
// a scalar load instead of a vector load followed by a full vmcnt wait.
__device__ __forceinline__ int ld_table(const int32_t* t, int i) {
  return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(t))[i];
}

// Keys seen by one work item, in blocks of kBN: either a chunk of one split's
// prompt pages (walked through the page table) or the causal response block.
// Inside a split pages are in increasing logical order, so the only partial
// prompt page (the last logical page, when prompt_len % 256 != 0) can only be
// the last page of a chunk: blocks [0, nfull) need no mask, [nfull, nblocks)
// do.  A page id out of range reads block 0 of the pool in the unmasked loop
// and is skipped in the masked one, so a corrupted device page table gives
// wrong numbers but never an out-of-bounds access.
// First response row of the member that holds response row i (members are
// consecutive row ranges; one member when there is no offset table).
__device__ __forceinline__ int member_start(const AttnArgs& a, int i) {
  int s = 0;
  if (a.moffs)
    for (int k = 1; k < a.nmembers; ++k) {
      const int o = ld_table(a.moffs, k);
      s = (i >= o) ? o : s;
    }
  return s;
}

template <int D, bool RESP>
struct KeyWalk {
  const AttnArgs& a;
  int kv, p0, nblocks, nfull, jfirst;
  // unit = split*chunks + chunk (paged); rows [m0, m0 + rows) of the group
  __device__ __forceinline__ KeyWalk(const AttnArgs& args, int kv_, int unit, int m0, int rows)
      : a(args), kv(kv_), p0(0), nblocks(0), nfull(0), jfirst(0) {
    const int GR = (a.hq / a.hkv) * a.R;
    if (RESP) {
      // keys [first key of the first row's member, qoff + last row] cover
      // every row of the tile when it stays inside one query head; else all
      const int mlast = min(m0 + rows, GR) - 1;
      const bool one_head = m0 / a.R == mlast / a.R;
      const int imax = one_head ? mlast % a.R : a.R - 1;
      nblocks = (a.qoff + imax + kBN) / kBN;
      jfirst = one_head ? member_start(a, m0 % a.R) / kBN : 0;
      // in the response of one member, when the tile stays in one query head,
      // the keys that even its first row sees need no mask: they stream
      // through the ring like prompt blocks
      nfull = (one_head && !a.moffs) ? min((a.qoff + m0 % a.R + 1) / kBN, nblocks) : 0;
    } else {
      const int c = unit / a.chunks, k = unit - c * a.chunks;
      int s0 = ld_table(a.offs, c), s1 = ld_table(a.offs, c + 1);
      s0 = min(max(s0, 0), a.num_pages);
      s1 = min(max(s1, s0), a.num_pages);
      p0 = s0 + k * a.chunk_pages;
      const int p1 = min(s1, p0 + a.chunk_pages);
      const int npages = max(0, p1 - p0);
      nblocks = npages * (kPage / kBN);
      nfull = nblocks;
      if (npages > 0 && (a.prompt_len % kPage) != 0 && ld_table(a.order, p1 - 1) == a.num_pages - 1)
        nfull = nblocks - kPage / kBN;
    }
  }
  // Pool offset of a page of this chunk, in two halves so that the load can
  // be issued well before the offset is needed: page_id(pg) reads the page's
  // physical slot (one scalar load), page_base(ph) turns it into the element
  // offset of the page's first row (0 for a slot out of range).
  __device__ __forceinline__ int page_id(int pg) const { return ld_table(a.phys, p0 + pg); }
  __device__ __forceinline__ size_t page_base(int ph) const {
    return (ph >= 0 && ph < a.num_phys) ? ((size_t)ph * a.hkv + kv) * kPage * D : 0;
  }
  // any block: element offset of its first row (pool or response tensors),
  // number of valid keys (0 = skip) and, for the response, its first key index
  __device__ __forceinline__ size_t block(int b, int& nvalid, int& key0) const {
    if (RESP) {
      key0 = b * kBN;
      nvalid = min(kBN, a.RK - key0);
      return ((size_t)kv * a.kvr + key0) * D;
    }
    key0 = 0;
    nvalid = 0;
    const int lp = ld_table(a.order, p0 + b / (kPage / kBN));
    const int tok = (b % (kPage / kBN)) * kBN;
    if (lp >= 0 && lp < a.num_pages) {
      const int ph = ld_table(a.l2p, lp);
      if (ph >= 0 && ph < a.num_phys) {
        const int64_t left = a.prompt_len - (int64_t)lp * kPage - tok;
        nvalid = (int)(left < 0 ? 0 : (left > kBN ? kBN : left));
        return (((size_t)ph * a.hkv + kv) * kPage + tok) * D;
      }
    }
    return 0;
  }
};

// Wait until at most N of this wave's vector-memory loads (including the
// direct global->LDS copies) are still in flight.
// s_waitcnt immediate for "at most N vector-memory ops in flight" (gfx9
// encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14), with
// expcnt and, unless LGKM0, lgkmcnt left at their maxima (no wait).
template <int N, bool LGKM0>
constexpr int waitcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8) | ((N >> 4) << 14);
}

// Wait until at most N of this wave's vector-memory ops are in flight.  The
// builtin (not asm) lets the compiler see the wait, so it does not add waits
// of its own for loads this one already covers.
template <int N>
__device__ __forceinline__ void wait_loads_le() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<N, false>());
}

__device__ __forceinline__ void wait_async_loads() { wait_loads_le<0>(); }

// Ring-buffer handoff: wait until at most N of this wave's copies are in
// flight and its LDS reads have returned, then meet the other waves.  No
// fence: __syncthreads()'s workgroup release would also wait for every copy
// still in flight, which is what the ring exists to avoid.  The barrier is an
// asm statement with a memory clobber so that no LDS access moves across it.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<N, true>());
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// Work item of workgroup `bid` for a launch over (KV head, row tile) items,
// item index = kv * mtiles + mtile.  Normally the XCD-aware remap above.  For
// the causal response block (lpt) every tile stays inside one query head and
// tile t of a head sees t + 1 tiles' worth of keys, so the items go out
// longest first: workgroup i takes tile t = T-1 - i / (Hkv*g) of head-slot
// i % (Hkv*g).  The hardware deals workgroup i to XCD i % 8, so every XCD
// gets the same mix of lengths, each in decreasing order.  Bijective.
__device__ __forceinline__ int tile_item(const AttnArgs& a, int rows_per_tile, int bid, int n) {
  if (!a.lpt) return xcd_remap(bid, n);
  const int g = a.hq / a.hkv, heads = a.hkv * g, T = a.R / rows_per_tile;
  const int t = T - 1 - bid / heads, r = bid - (bid / heads) * heads;
  return (r / g) * a.mtiles + (r % g) * T + t;
}

// max of x over the lane pair (l, l ^ 32): v_permlane32_swap exchanges the two
// half-waves in registers (no LDS traffic); for lane l < 32 the partner value
// comes back in the second result, for l >= 32 in the first.
__device__ __forceinline__ float wave_max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace ls
