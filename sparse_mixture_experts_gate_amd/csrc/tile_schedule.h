// Device-side tile scheduler of the persistent grouped GEMMs.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace dsmoe {

// Per tile: group g, row range, m-tile and column tile n of a grouped GEMM.
struct TileCoord {
  int g, rows, rbase, m, n;
  bool shared;
};

constexpr int kMaxGroups = 513;  // 512 routed experts + the shared expert

// LDS copy of the device-built tile schedule (group g owns tiles
// [tiles[g], tiles[g+1]); the shared expert is group E), for tile loops that
// must issue no global loads of their own (their vector-memory waits are
// counted by hand). gnext[i] is the first tile of group i + 1 (i < E) and
// INT_MAX beyond, so the group of a tile is the number of entries <= tile;
// off holds the row offsets of the routed groups. Tiles are numbered
// (group, n, m) with m fastest: the tiles that one XCD runs together share
// one weight slab.
struct __attribute__((aligned(16))) GroupTables {
  int gnext[kMaxGroups - 1];
  int off[kMaxGroups];
  int total;
};
static_assert(kMaxGroups - 1 == 8 * 64, "one wave scans gnext with 8 entries per lane");

__device__ __forceinline__ void load_group_tables(GroupTables& t, const int32_t* tiles,
                                                  const int32_t* offsets, int E) {
  for (int i = threadIdx.x; i < kMaxGroups - 1; i += blockDim.x)
    t.gnext[i] = i < E ? tiles[i + 1] : 0x7fffffff;
  for (int i = threadIdx.x; i <= E; i += blockDim.x) t.off[i] = offsets[i];
  if (threadIdx.x == 0) t.total = tiles[E + 1];
  __syncthreads();
}

// tile_coord over the LDS tables, wave-uniform: every lane compares eight
// entries of gnext with the tile and the ballots count them, two LDS reads
// deep instead of a binary search's nine.
__device__ __forceinline__ TileCoord tile_coord_lds(const GroupTables& t, int E, int64_t T,
                                                    int tile, int bm) {
  const int lane = threadIdx.x & 63;
  const int4 v0 = *reinterpret_cast<const int4*>(t.gnext + 8 * lane);
  const int4 v1 = *reinterpret_cast<const int4*>(t.gnext + 8 * lane + 4);
  const int g = __popcll(__ballot(v0.x <= tile)) + __popcll(__ballot(v0.y <= tile)) +
                __popcll(__ballot(v0.z <= tile)) + __popcll(__ballot(v0.w <= tile)) +
                __popcll(__ballot(v1.x <= tile)) + __popcll(__ballot(v1.y <= tile)) +
                __popcll(__ballot(v1.z <= tile)) + __popcll(__ballot(v1.w <= tile));
  TileCoord c;
  c.g = g;
  c.shared = g == E;
  const int start = __builtin_amdgcn_readfirstlane(g == 0 ? 0 : t.gnext[g - 1]);
  c.rbase = c.shared ? 0 : __builtin_amdgcn_readfirstlane(t.off[g]);
  c.rows = c.shared ? static_cast<int>(T)
                    : __builtin_amdgcn_readfirstlane(t.off[g + 1]) - c.rbase;
  const int mt = (c.rows + bm - 1) / bm;
  const int local = tile - start;
  c.n = local / mt;
  c.m = local - c.n * mt;
  return c;
}

// Workgroup barrier without the memory fence of __syncthreads: LDS accesses
// have completed, vector memory operations (loads into LDS, stores) may still
// be in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Buffer resources: operands are read with raw buffer loads through a 32-bit
// byte offset; offsets at or beyond the resource size read as zeros in
// hardware, which is how padding rows are handled without branches.
constexpr uint32_t kInvalidRow = 0x80000000u;
// Cache-policy bit of buffer stores: non-temporal, for outputs that no kernel
// of the call reads back soon (the fp32 weight gradients).
constexpr int kNonTemporal = 2;

// Raw buffer descriptor as four scalar words: base address, no stride,
// `bytes` records (range-checked: offsets at or beyond it read as zeros).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// The words are read through readfirstlane: every caller builds a
// wave-uniform descriptor, and the loads take it in scalar registers.
__device__ __forceinline__ i32x4_t rsrc4(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a pointer into __shared__ memory (the low 32 bits of
// its flat address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Buffer loads straight into LDS (buffer_load ... lds): lane i writes
// lds_addr + 16 i (dma16) or + 4 i (dma4), lds_addr wave-uniform (in M0).
// The loads have no register result, so nothing is in flight towards a VGPR;
// the compiler does not track them, so callers wait with explicit vmcnt
// (and keep no compiler-visible vector loads between those waits, whose
// counts would not include these).
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same with the non-temporal policy, for data read once (weights
// streamed past the caches).
__device__ __forceinline__ void dma16_nt(i32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}

}  // namespace dsmoe
