// Per-lane pieces of the bf16 temporal attention (gfx950), shared by the
// stand-alone temporal kernel and the temporal wavefronts of the fused
// denoising-call kernel.
//
// A row (b, s, h) is served by 4*QH lanes: 4 dimension groups x QH query
// groups. Lane g of a quad holds dims {16-byte chunks g, g+4, ...} of the row
// plus dword g of a leftover chunk (d = 72: 2 chunks + 1 dword = 18 dims), so
// every load is aligned and the quad covers the row; dot products are partial
// sums reduced across the quad with two DPP adds.
#pragma once

#include "device_common.hpp"

namespace ca2 {

template <int D>
struct DsGeom {
  static constexpr int C16 = D * 2 / 16;     // 16-byte chunks per row
  static constexpr int FULL = C16 / 4;       // whole chunks per lane
  static constexpr int REM = C16 % 4;        // leftover chunks, one dword per lane each
  static constexpr int DW = FULL * 4 + REM;  // dwords (bf16 pairs) per lane
  static constexpr int DPL = 2 * DW;         // dims per lane
  static_assert((D * 2) % 16 == 0, "row must be whole 16-byte chunks");
};

template <int D>
struct Slice {
  uint32_t w[DsGeom<D>::DW];
};

template <int D>
__device__ __forceinline__ void load_slice(Slice<D>& s, const unsigned char* row, int g) {
  using G = DsGeom<D>;
#pragma unroll
  for (int c = 0; c < G::FULL; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + 16 * (g + 4 * c));
    s.w[4 * c + 0] = u.x; s.w[4 * c + 1] = u.y; s.w[4 * c + 2] = u.z; s.w[4 * c + 3] = u.w;
  }
#pragma unroll
  for (int r = 0; r < G::REM; ++r)
    s.w[4 * G::FULL + r] = *reinterpret_cast<const uint32_t*>(row + 16 * (4 * G::FULL + r) + 4 * g);
}

// The same slice from a wavefront-uniform base plus per-lane 32-bit offsets:
// off16 = the row's offset + 16 g (whole chunks, the rest as immediates),
// off4 = the row's offset + the leftover chunk's start + 4 g. The addresses
// take the scalar-base form of the global loads, so a key costs no vector
// address arithmetic.
template <int D>
__device__ __forceinline__ void load_slice_at(Slice<D>& s, const unsigned char* base, uint32_t off16, uint32_t off4) {
  using G = DsGeom<D>;
  const unsigned char* p16 = base + off16;
#pragma unroll
  for (int c = 0; c < G::FULL; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(p16 + 64 * c);
    s.w[4 * c + 0] = u.x; s.w[4 * c + 1] = u.y; s.w[4 * c + 2] = u.z; s.w[4 * c + 3] = u.w;
  }
  const unsigned char* p4 = base + off4;
#pragma unroll
  for (int r = 0; r < G::REM; ++r) s.w[4 * G::FULL + r] = *reinterpret_cast<const uint32_t*>(p4 + 16 * r);
}

template <int D>
__device__ __forceinline__ void store_slice(unsigned char* row, int g, const float* v) {
  using G = DsGeom<D>;
#pragma unroll
  for (int c = 0; c < G::FULL; ++c) {
    uint4 u;
    u.x = pack_bf16x2(v[8 * c + 0], v[8 * c + 1]);
    u.y = pack_bf16x2(v[8 * c + 2], v[8 * c + 3]);
    u.z = pack_bf16x2(v[8 * c + 4], v[8 * c + 5]);
    u.w = pack_bf16x2(v[8 * c + 6], v[8 * c + 7]);
    *reinterpret_cast<uint4*>(row + 16 * (g + 4 * c)) = u;
  }
#pragma unroll
  for (int r = 0; r < G::REM; ++r)
    *reinterpret_cast<uint32_t*>(row + 16 * (4 * G::FULL + r) + 4 * g) =
        pack_bf16x2(v[8 * G::FULL + 2 * r], v[8 * G::FULL + 2 * r + 1]);
}

// sum over the 4 lanes of a quad (dimension groups of one row)
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  return x;
}

// Running max before any visible key: the most negative finite float, so any
// finite score raises it on first sight (a larger sentinel would leave scores
// below it unraised, every P would round to 0 and the row would divide 0 by 0),
// and exp2 of a masked (-inf) score minus it is still exactly 0.
constexpr float kNoMax = -__FLT_MAX__;
constexpr float kLazy = 8.0f;        // raise the running max only past this margin (base 2)
}  // namespace ca2
