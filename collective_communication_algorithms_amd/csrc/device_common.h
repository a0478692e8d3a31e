// Device helpers shared by the row, permutation and column kernels: typed
// global / constant accesses, the element arithmetic of a recv_and_reduce row,
// and the wave reductions of the row checksums.
#pragma once

#include <hip/hip_runtime.h>

#include "device_types.h"

namespace coll {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Rank buffers are plain device memory: address them in the global address
// space (global_load / global_store rather than flat).  The item and step
// tables never change during a launch: read them through the constant address
// space so that uniform reads become scalar loads.
#define GLOBAL __attribute__((address_space(1)))
#define CONSTANT __attribute__((address_space(4)))

template <class T>
__device__ __forceinline__ const GLOBAL T* gptr(const char* p) {
  return (const GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ GLOBAL T* gptr(char* p) {
  return (GLOBAL T*)(p);
}

template <class T>
__device__ __forceinline__ T cload(const T* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(const CONSTANT T*)(p);
#else
  return *p;  // the host pass only needs the kernels to parse
#endif
}

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(gptr<u32x4>(p));
  else return *gptr<u32x4>(p);
}

template <bool NT>
__device__ __forceinline__ void st16(char* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, gptr<u32x4>(p));
  else *gptr<u32x4>(p) = v;
}

// ---- element arithmetic ------------------------------------------------------

// binary32 -> bfloat16, round to nearest even on the bit pattern: adding 0x7FFF
// plus the lowest kept bit carries into the kept half exactly when the dropped
// half is above one half-ulp, or equal to it with an odd kept part.  NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int OP>
__device__ __forceinline__ uint32_t pick_i32(uint32_t d, uint32_t s) {
  if constexpr (OP == OP_SUM) return d + s;  // wraps modulo 2^32
  else if constexpr (OP == OP_MAX) return int32_t(s) > int32_t(d) ? s : d;
  else return int32_t(s) < int32_t(d) ? s : d;
}

template <int OP>
__device__ __forceinline__ uint32_t pick_f32(uint32_t d, uint32_t s) {
  const float fd = __uint_as_float(d), fs = __uint_as_float(s);
  if constexpr (OP == OP_SUM) return __float_as_uint(fd + fs);
  else if constexpr (OP == OP_MAX) return fs > fd ? s : d;
  else return fs < fd ? s : d;
}

// one bfloat16 held in the low 16 bits
template <int OP>
__device__ __forceinline__ uint32_t pick_bf16(uint32_t d, uint32_t s) {
  const float fd = __uint_as_float(d << 16), fs = __uint_as_float(s << 16);
  if constexpr (OP == OP_SUM) return bf16_rne(fd + fs);
  else if constexpr (OP == OP_MAX) return fs > fd ? s : d;
  else return fs < fd ? s : d;
}

template <int OP>
__device__ __forceinline__ uint32_t pick_u8(uint32_t d, uint32_t s) {
  if constexpr (OP == OP_SUM) return (d + s) & 0xffu;
  else if constexpr (OP == OP_MAX) return s > d ? s : d;
  else return s < d ? s : d;
}

// One element (its bits in the low bits of the word).
template <int DT, int OP>
__device__ __forceinline__ uint32_t combine_elem(uint32_t d, uint32_t s) {
  if constexpr (DT == DT_I32) return pick_i32<OP>(d, s);
  else if constexpr (DT == DT_F32) return pick_f32<OP>(d, s);
  else if constexpr (DT == DT_BF16) return pick_bf16<OP>(d, s);
  else return pick_u8<OP>(d, s);
}

// A 32-bit word of packed elements.
template <int DT, int OP>
__device__ __forceinline__ uint32_t combine_word(uint32_t d, uint32_t s) {
  if constexpr (DT == DT_I32 || DT == DT_F32) {
    return combine_elem<DT, OP>(d, s);
  } else if constexpr (DT == DT_BF16) {
    const uint32_t lo = pick_bf16<OP>(d & 0xffffu, s & 0xffffu);
    const uint32_t hi = pick_bf16<OP>(d >> 16, s >> 16);
    return lo | (hi << 16);
  } else {
    uint32_t r = 0;
#pragma unroll
    for (int b = 0; b < 32; b += 8) r |= pick_u8<OP>((d >> b) & 0xffu, (s >> b) & 0xffu) << b;
    return r;
  }
}

// Two binary32 values to a word of two bfloat16 (lo in the low half) with
// the hardware's conversion (v_cvt_pk_bf16_f32): round to nearest even, the
// same bits as bf16_rne for every value but NaN, whose sign and payload the
// hardware keeps.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// bfloat16 sum of 16 bytes: the eight binary32 sums converted in pairs by the
// hardware, which costs about half the instructions of rounding on the bit
// pattern.  Where any lane of the wave holds a NaN sum (a branch no wave
// takes on finite data) the whole wave rounds by bf16_rne instead, which
// gives the same bits for every other value and 0x7FC0 for every NaN (the
// ballot covers the active lanes, so any exec mask is fine).
__device__ __forceinline__ u32x4 sum16_bf16(u32x4 d, u32x4 s) {
  float lo[4], hi[4];
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w}, sw[4] = {s.x, s.y, s.z, s.w};
  uint64_t nan = 0;  // lanes with a NaN sum, kept in scalar registers
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = __uint_as_float(dw[i] << 16) + __uint_as_float(sw[i] << 16);
    hi[i] = __uint_as_float(dw[i] & 0xffff0000u) + __uint_as_float(sw[i] & 0xffff0000u);
    nan |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(lo[i], hi[i]));
  }
  u32x4 r;
  r.x = cvt_pk_bf16(lo[0], hi[0]);
  r.y = cvt_pk_bf16(lo[1], hi[1]);
  r.z = cvt_pk_bf16(lo[2], hi[2]);
  r.w = cvt_pk_bf16(lo[3], hi[3]);
  if (nan) {
    r.x = bf16_rne(lo[0]) | (bf16_rne(hi[0]) << 16);
    r.y = bf16_rne(lo[1]) | (bf16_rne(hi[1]) << 16);
    r.z = bf16_rne(lo[2]) | (bf16_rne(hi[2]) << 16);
    r.w = bf16_rne(lo[3]) | (bf16_rne(hi[3]) << 16);
  }
  return r;
}

template <int DT, int OP>
__device__ __forceinline__ u32x4 combine16(u32x4 d, u32x4 s) {
  if constexpr (DT == DT_BF16 && OP == OP_SUM) return sum16_bf16(d, s);
  u32x4 r;
  r.x = combine_word<DT, OP>(d.x, s.x);
  r.y = combine_word<DT, OP>(d.y, s.y);
  r.z = combine_word<DT, OP>(d.z, s.z);
  r.w = combine_word<DT, OP>(d.w, s.w);
  return r;
}

// ---- checksum helpers (row checksum: sum of the row's little-endian uint32
// words counted from the row's first byte).  A stored word at a 4-aligned column
// holds the row's bytes rotated by the row start's misalignment.
__device__ __forceinline__ uint32_t rotl32(uint32_t x, uint32_t r) {
  return r ? (x << r) | (x >> (32u - r)) : x;
}

__device__ __forceinline__ uint64_t words16(u32x4 v, uint32_t rot) {
  return uint64_t(rotl32(v.x, rot)) + rotl32(v.y, rot) + rotl32(v.z, rot) + rotl32(v.w, rot);
}

// One shift-and-add step of a scan inside every row of 16 lanes: lane i adds
// lane i - N of its row (0 when that lane lies before the row's first), on a
// u64 held as two u32 halves.
template <int N>
__device__ __forceinline__ void row_shr_add(uint32_t& lo, uint32_t& hi) {
  const uint32_t l = uint32_t(__builtin_amdgcn_update_dpp(0, int(lo), 0x110 + N, 0xf, 0xf, true));
  const uint32_t h = uint32_t(__builtin_amdgcn_update_dpp(0, int(hi), 0x110 + N, 0xf, 0xf, true));
  const uint32_t s = lo + l;
  hi += h + (s < lo ? 1u : 0u);
  lo = s;
}

// Sum of a u64 over the 64 lanes of a wave (every lane active), with DPP
// moves instead of LDS permutes: the scan leaves each row's total in its last
// lane, and the four totals are read into scalar registers.
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
  row_shr_add<1>(lo, hi);
  row_shr_add<2>(lo, hi);
  row_shr_add<4>(lo, hi);
  row_shr_add<8>(lo, hi);
  uint64_t t = 0;
#pragma unroll
  for (int r = 15; r < 64; r += 16)
    t += (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(hi), r))) << 32) |
         uint32_t(__builtin_amdgcn_readlane(int(lo), r));
  return t;
}

// Adds a wave's part of a row checksum to the row's partial slot for this
// work group.
__device__ __forceinline__ void add_row_sum(uint64_t* sums, uint32_t row, uint64_t v) {
  v = wave_sum(v);
  if ((threadIdx.x & 63u) == 0 && row != NO_ROW)
    __hip_atomic_fetch_add(sums + uint64_t(row) * SUM_LANES + (blockIdx.x & (SUM_LANES - 1u)), v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ---- element loads / stores for the unaligned edges ------------------------------

template <int DT>
__device__ __forceinline__ uint32_t ld_elem(const char* p) {
  if constexpr (DT == DT_I32 || DT == DT_F32) return *gptr<uint32_t>(p);
  else if constexpr (DT == DT_BF16) return *gptr<uint16_t>(p);
  else return *gptr<uint8_t>(p);
}

template <int DT>
__device__ __forceinline__ void st_elem(char* p, uint32_t v) {
  if constexpr (DT == DT_I32 || DT == DT_F32) *gptr<uint32_t>(p) = v;
  else if constexpr (DT == DT_BF16) *gptr<uint16_t>(p) = uint16_t(v);
  else *gptr<uint8_t>(p) = uint8_t(v);
}

template <int DT>
constexpr int elem_size() { return DT == DT_BF16 ? 2 : (DT == DT_U8 ? 1 : 4); }

// Element e of a 16-byte unit held in four words (selects, no indexing into
// registers).
template <int DT>
__device__ __forceinline__ uint32_t elem_of(u32x4 v, int e) {
  constexpr int SZ = elem_size<DT>();
  const int byte = e * SZ;
  const uint32_t w = byte < 4 ? v.x : byte < 8 ? v.y : byte < 12 ? v.z : v.w;
  if constexpr (SZ == 4) return w;
  else if constexpr (SZ == 2) return (w >> (8 * (byte & 3))) & 0xffffu;
  else return (w >> (8 * (byte & 3))) & 0xffu;
}

}  // namespace coll
