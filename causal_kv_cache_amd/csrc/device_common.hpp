// Device-side helpers shared by the gfx950 kernels of libca2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca2 {

typedef uint16_t bf16_t;  // bfloat16 storage (upper 16 bits of a float32)

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2v b = __builtin_convertvector(f, bf16x2v);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element-type traits: how many values one 16-byte chunk holds and how to
// unpack / pack them to float32.
template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ __forceinline__ static void unpack(const uint4& c, float* o) {
    o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
    o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                      __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
};

template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static void unpack(const uint4& c, float* o) {
    o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x); o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
    o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z); o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* v) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                      pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(ahead * per) for a wave-uniform ahead in [0, kMax]; the
// count must be an immediate, so each value gets its own instruction.
template <int per, int k = 0, int kMax = 8>
__device__ __forceinline__ void wait_vmcnt_tiles(int ahead) {
  if constexpr (k > kMax || k * per > 63) {
    wait_vmcnt<0>();
  } else {
    if (ahead == k) wait_vmcnt<k * per>();
    else wait_vmcnt_tiles<per, k + 1, kMax>(ahead);
  }
}

// A wavefront-uniform 64-bit value as such (readfirstlane returns int: widen
// through unsigned, never sign-extend).
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// 16-byte global -> LDS copy for every active lane: lane i reads
// sbase + voff (+ 0..15) and writes lds_addr + 16*i (lds_addr in M0);
// sbase and lds_addr are wavefront-uniform. The instruction writes LDS only
// (no register result), and the kernels that use it wait for it with
// explicit vmcnt counts. M0 is a register the compiler reserves, so it warns
// that the clobber may not be honoured; in the kernels built here every M0
// reference in the generated code is this one (no indirect register moves,
// messages or GWS operations), so nothing of the compiler's lives in M0 --
// tests/test_m0_guard.py compiles the kernels to assembly and fails if any
// other instruction writes or reads M0. (The compiler's own builtin for this
// copy takes a 64-bit per-lane address and makes workgroup-scope release
// fences wait for every outstanding copy, which would drain the tile
// pipeline at each barrier.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16s(unsigned voff, uint64_t sbase, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(uniform64(sbase)), "s"((unsigned)__builtin_amdgcn_readfirstlane((int)lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Block index -> work index such that XCD x (which receives blocks x, x+8,
// x+16, ...) processes work items [start_x, start_x + count_x) in order.
__device__ __forceinline__ int xcd_work_index(int block, int nblocks) {
  constexpr int kXcds = 8;
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int x = block % kXcds, local = block / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

}  // namespace ca2
