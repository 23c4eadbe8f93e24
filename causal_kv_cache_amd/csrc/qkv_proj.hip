// QKV projection of the clean chunk (gfx950 bf16 MFMA GEMM).
//
// The cache-writing stage of the Ca2-VDM notes (overall framework) runs one
// forward pass of the denoised chunk to produce the K/V that are stored; this
// is that pass's linear projection: [Q K V] = X W^T, X: [m][c_in] tokens,
// W: [3c][c_in] (row-major linear weight), fp32 accumulation, bf16 outputs
// split into three [m][c] tensors in the activation layout the cache write
// consumes.
//
// Tiling: workgroup tile 128 (output channels n) x 128 (tokens m), 4
// wavefronts of 64 x 64, k-tile 64, v_mfma_f32_32x32x16_bf16. The product is
// formed as C^T = W X^T so that a lane owns one token row and its 16
// accumulator registers hold runs of 4 consecutive channels (8-byte stores).
// LDS rows are 144 bytes (128 + 16 pad) so 8 consecutive rows read distinct
// banks; the next k-tile is loaded into registers while the current one is
// multiplied.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ca2 {
namespace {

constexpr int TN = 128;   // output channels per workgroup
constexpr int TM = 128;   // tokens per workgroup
constexpr int TK = 64;    // contraction per step
constexpr int LSTR = TK * 2 + 16;
constexpr int kThreads = 256;
constexpr int kLoads = (TN * TK / 8) / kThreads;   // 16-byte chunks per thread per operand (4)

__global__ __launch_bounds__(kThreads) void qkv_proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sw[TN * LSTR];
  __shared__ __attribute__((aligned(16))) unsigned char sx[TM * LSTR];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM;
  const int N = 3 * a.c_out;
  const bf16_t* __restrict__ W = static_cast<const bf16_t*>(a.w);
  const bf16_t* __restrict__ X = static_cast<const bf16_t*>(a.x);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 rw[kLoads], rx[kLoads];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = u * kThreads + tid;
      const int row = e >> 3, c = e & 7;
      const int n = n0 + row, m = m0 + row;
      rw[u] = n < N ? *reinterpret_cast<const uint4*>(W + (int64_t)n * a.c_in + k0 + c * 8)
                    : make_uint4(0, 0, 0, 0);
      rx[u] = m < a.m ? *reinterpret_cast<const uint4*>(X + (int64_t)m * a.c_in + k0 + c * 8)
                      : make_uint4(0, 0, 0, 0);
    }
  };
  load(0);
  for (int k0 = 0; k0 < a.c_in; k0 += TK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = u * kThreads + tid;
      const int row = e >> 3, c = e & 7;
      *reinterpret_cast<uint4*>(sw + row * LSTR + c * 16) = rw[u];
      *reinterpret_cast<uint4*>(sx + row * LSTR + c * 16) = rx[u];
    }
    __syncthreads();
    if (k0 + TK < a.c_in) load(k0 + TK);
#pragma unroll
    for (int s = 0; s < TK / 16; ++s) {
      bf16x8v wa[2], xb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        wa[i] = *reinterpret_cast<const bf16x8v*>(sw + (wn * 64 + i * 32 + col) * LSTR + (16 * s + 8 * half) * 2);
        xb[i] = *reinterpret_cast<const bf16x8v*>(sx + (wm * 64 + i * 32 + col) * LSTR + (16 * s + 8 * half) * 2);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[i], xb[j], acc[i][j], 0, 0, 0);
    }
  }

  // register r of acc[i][j]: channel n0 + wn*64 + 32i + 8(r/4) + 4*half + r%4,
  // token m0 + wm*64 + 32j + col
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + 32 * j + col;
    if (m >= a.m) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + 32 * i + 8 * g + 4 * half;
        if (n >= N) continue;
        const int seg = n / a.c_out;
        bf16_t* dst = static_cast<bf16_t*>(seg == 0 ? a.q : seg == 1 ? a.k : a.v);
        uint2 w;
        w.x = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        w.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        *reinterpret_cast<uint2*>(dst + (int64_t)m * a.c_out + (n - seg * a.c_out)) = w;
      }
  }
}

}  // namespace

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  if (a.m < 1 || a.c_in % TK || a.c_out % 64) return hipErrorInvalidValue;
  const dim3 grid((3 * a.c_out + TN - 1) / TN, (a.m + TM - 1) / TM);
  hipLaunchKernelGGL(qkv_proj_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ca2
