// Device-side building blocks shared by the gfx950 attention kernels:
// vector types for the bf16 MFMA operands, 16-byte global/LDS accesses,
// the cross-half lane exchange and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// 16-byte and 8-byte LDS accesses (addresses are element offsets into a
// __shared__ uint16_t array; callers keep them 16- or 8-byte aligned).
__device__ __forceinline__ u32x4 ld_lds16(const uint16_t* base, int elem) {
  return *reinterpret_cast<const u32x4*>(base + elem);
}
__device__ __forceinline__ void st_lds16(uint16_t* base, int elem, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + elem) = v;
}
__device__ __forceinline__ void st_lds8(uint16_t* base, int elem, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + elem) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Combine a lane's value with the one held by lane (l ^ 32). v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; feeding x as both gives {x_lo, x_lo} and {x_hi, x_hi}, so any
// symmetric op of the two results pairs lane l with lane l ^ 32.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// exp2 on the VALU transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two floats to bf16 (nearest-even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

#define LDS_AS __attribute__((address_space(3)))
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest even) into one register with a single
// v_cvt_pk_bf16_f32; `lo` lands in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4).
// The LDS address must be uniform across the wave; lane l writes the 16
// bytes at ldst + 16*l.
__device__ __forceinline__ void lds_dma16(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, 0, 0);
}
// The same 16-byte LDS DMA from a wave-uniform global base plus a per-lane
// 32-bit byte offset (the SGPR-base addressing form, so no 64-bit per-lane
// address is ever formed), issued through inline assembly. The compiler does
// not track it and inserts no wait for it: the issuing wave must wait_vmem()
// before any wave reads the data. `lds_addr` is the wave-uniform LDS byte
// address of the 1 KiB destination (lane l writes lds_addr + 16*l). M0 is
// written here; nothing else in these kernels uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               : : "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// Variants without the compiler memory clobber, for code that interleaves
// the DMA with LDS reads of other buffers: the compiler may move loads across
// them. They stay ordered with respect to barrier_nofence() and the waits
// (volatile asm and side-effecting builtins are not reordered), which is what
// protects the destination buffer. The 4-byte form writes lds_addr + 4*l.
__device__ __forceinline__ void lds_dma16_sbase_nc(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr) : "m0");
}
__device__ __forceinline__ void lds_dma4_sbase_nc(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr) : "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS const void*)(p)));
}

// 4 bytes per lane (lane l writes ldst + 4*l).
__device__ __forceinline__ void lds_dma4(const void* gsrc, LDS_AS void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 4, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// Wait until at most N vector-memory operations of this wave are outstanding
// (loads complete in order, so everything issued before the last N is done).
// The FA_DEBUG_SYNC build waits for all of them.
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
#ifdef FA_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0x0f70);
#else
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
#endif
}

// Workgroup barrier without a memory fence. __syncthreads() also waits for
// every outstanding memory operation of the wave (s_waitcnt vmcnt(0)
// lgkmcnt(0) before s_barrier), which would stall a wave that has just
// issued LDS-DMA prefetches for their whole global-memory latency. Here the
// caller orders memory itself: LDS data a wave read before the barrier has
// been consumed by then (its reads are complete), and LDS-DMA writes are
// waited for with wait_vmem() by the issuing wave before the barrier that
// publishes them. The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
// The FA_DEBUG_SYNC build (a check, not the product) makes every such
// barrier a full one: all of the wave's memory operations complete first. The
// ordering argued above then no longer matters, so any difference between the
// results of the two builds would expose an LDS race in the fence-free form.
__device__ __forceinline__ void barrier_nofence() {
#ifdef FA_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  __syncthreads();
#else
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

// Row of a 32-row MFMA A operand that lane m supplies, chosen so that the
// 32x32 accumulator register i of lane half g holds row 16*g + i: each lane
// then owns runs of 8 consecutive rows, the k-layout of a following MFMA
// whose B operand is taken straight from those accumulators.
__device__ __forceinline__ int row_of_lane(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Two ds_read_b64_tr_b16 reads (rows r..r+3 and r+4..r+7 of a row-major bf16
// tile, addressed per lane as for a transposed 16-bit read) combined into one
// 8-element MFMA operand: element e = row r+e at this lane's column.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint8_t* p0, const uint8_t* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p1));
  u32x4 v;
  v[0] = __builtin_bit_cast(u32x2, lo)[0];
  v[1] = __builtin_bit_cast(u32x2, lo)[1];
  v[2] = __builtin_bit_cast(u32x2, hi)[0];
  v[3] = __builtin_bit_cast(u32x2, hi)[1];
  return as_bf16x8(v);
}

// Workgroup -> (key/value head index, tile rank). Workgroups are dealt to the
// 8 XCDs round-robin; when the number of key/value heads allows it, each XCD
// gets whole key/value heads (all their query heads and tiles) so that K/V
// is shared through that XCD's L2. Within an XCD the tile rank runs fastest
// (one head's tiles one after the other), or, with rank_major, slowest: rank
// 0 of every head of the XCD first, then rank 1, ... -- with tiles ranked
// heaviest first this deals them in decreasing cost across heads, which keeps
// the compute units evenly loaded when a unit holds several workgroups and
// each runs only a few of them. With rank_group = g > 1 (and rank_major
// off) the heads of the XCD are taken g at a time and each group runs rank
// 0 of its g heads, then rank 1, ...: consecutive workgroups then cost the
// same. The workgroup dispatcher hands workgroups to an XCD's compute units a
// few at a time and in order, so a workgroup waits until enough units are
// free; equal costs let those units free up together (with one head's ranks
// consecutive, each dispatch waited on the slowest of several unequal
// tiles). g is reduced to the largest power of two dividing the heads in
// scope.
struct TileAssign {
  int kvidx, gq, tile_rank;
};
__device__ __forceinline__ TileAssign assign_tile(int L, int n_tiles, int G, int xcd_remap, int n_heads = 0,
                                                  bool rank_major = false, int rank_group = 1) {
  TileAssign a;
  int head;  // (key/value head, query head of its group) in order, within the XCD when remapped
  // s: position within the scope (the XCD when remapped, else the grid);
  // hs: query heads in that scope (n_heads = B * H_q, a multiple of 8 when remapped)
  const int s = xcd_remap ? (L >> 3) : L;
  const int hs = xcd_remap ? n_heads / 8 : n_heads;
  if (rank_major) {
    a.tile_rank = s / hs;
    head = s % hs;
  } else if (rank_group > 1) {
    int g = rank_group;
    while (hs % g) g >>= 1;
    const int per_group = g * n_tiles;
    const int r = s % per_group;
    a.tile_rank = r / g;
    head = (s / per_group) * g + r % g;
  } else {
    a.tile_rank = s % n_tiles;
    head = s / n_tiles;
  }
  a.kvidx = xcd_remap ? (L & 7) + 8 * (head / G) : head / G;
  a.gq = head % G;
  return a;
}

}  // namespace fa
