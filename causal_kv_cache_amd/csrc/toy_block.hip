// Kernels of a small spatial-temporal transformer block (random weights) used
// to check the shared cache end to end on the GPU: per-frame timestep
// modulation, layer normalisation, and fp32 linear layers. The block's
// structure follows the Ca2-VDM notes: overall framework (denoising stage
// reading the caches, cache-writing stage at t = 0), key design 2 (clean
// frames take the embedding of timestep 0, so their K/V do not depend on the
// denoising step) and the training section (a timestep vector with one entry
// per frame). Attention runs in the cache kernels; these are the pieces
// around it. Sizes are small, so the kernels are plain tiled fp32 code.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ca2 {
namespace {

// out[f][j] = sum_i emb(t_f)[i] * wmod[i][j], emb(t) = [sin(t w_i), cos(t w_i)]
// for i < half, w_i = 1000^(-i/half). The embedding is evaluated in double:
// t reaches the hundreds, and a float product t * w_i would move the sine by
// ~1e-4.
__global__ void temb_mod_kernel(const float* __restrict__ t, int frames, const float* __restrict__ wmod,
                                int temb_dim, int width, float* __restrict__ out) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int f = blockIdx.y;
  if (j >= width || f >= frames) return;
  const int half = temb_dim / 2;
  const double tf = (double)t[f];
  const double ln1000 = 6.907755278982137;
  double acc = 0.0;
  for (int i = 0; i < half; ++i) {
    const double a = tf * exp(-ln1000 * (double)i / (double)half);
    acc += sin(a) * (double)wmod[(size_t)i * width + j];
    acc += cos(a) * (double)wmod[(size_t)(i + half) * width + j];
  }
  out[(size_t)f * width + j] = (float)acc;
}

// One wavefront per token row of C channels:
// out = (x - mean) / sqrt(var + 1e-6) * (1 + mod[f][scale_off + c]) + mod[f][shift_off + c].
__global__ __launch_bounds__(64) void ln_mod_kernel(const float* __restrict__ x, const float* __restrict__ mod,
                                                   int mod_stride, int shift_off, int scale_off, int tokens,
                                                   int rows, int C, float* __restrict__ out) {
  const int row = blockIdx.x;
  if (row >= rows) return;
  const int f = row / tokens;
  const int lane = threadIdx.x;
  const float* xr = x + (size_t)row * C;
  float s = 0.f;
  for (int c = lane; c < C; c += 64) s += xr[c];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  const float mean = s / (float)C;
  float v = 0.f;
  for (int c = lane; c < C; c += 64) {
    const float e = xr[c] - mean;
    v = fmaf(e, e, v);
  }
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const float inv = 1.f / sqrtf(v / (float)C + 1e-6f);
  const float* mr = mod + (size_t)f * mod_stride;
  float* orow = out + (size_t)row * C;
  for (int c = lane; c < C; c += 64)
    orow[c] = (xr[c] - mean) * inv * (1.f + mr[scale_off + c]) + mr[shift_off + c];
}

__device__ __forceinline__ float gelu_tanh(float x) {
  return 0.5f * x * (1.f + tanhf(0.7978845608028654f * (x + 0.044715f * x * x * x)));
}

// y[m][n] = act(sum_k x[m][k] w[k][n]) (+ r[m][n]); 16x16 output tiles, k in
// steps of 16 through LDS. y may alias r (each element is read, then written,
// by the same thread).
constexpr int kT = 16;
__global__ __launch_bounds__(kT * kT) void linear_f32_kernel(ToyLinearArgs a) {
  __shared__ float xs[kT][kT + 1];
  __shared__ float ws[kT][kT + 1];
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  const int m = blockIdx.y * kT + ty;
  const int n = blockIdx.x * kT + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < a.k; k0 += kT) {
    const int kx = k0 + tx, kw = k0 + ty;
    xs[ty][tx] = (m < a.m && kx < a.k) ? a.x[(size_t)m * a.ldx + kx] : 0.f;
    ws[ty][tx] = (kw < a.k && n < a.n) ? a.w[(size_t)kw * a.ldw + n] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kT; ++kk) acc = fmaf(xs[ty][kk], ws[kk][tx], acc);
    __syncthreads();
  }
  if (m < a.m && n < a.n) {
    float y = a.act == 1 ? gelu_tanh(acc) : acc;
    if (a.r) y += a.r[(size_t)m * a.ldr + n];
    a.y[(size_t)m * a.ldy + n] = y;
  }
}

}  // namespace

hipError_t launch_toy_temb_mod(const float* t, int frames, const float* wmod, int temb_dim, int width, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(temb_mod_kernel, dim3((width + 63) / 64, frames), dim3(64), 0, s, t, frames, wmod, temb_dim,
                     width, out);
  return hipGetLastError();
}

hipError_t launch_toy_ln_mod(const float* x, const float* mod, int mod_stride, int shift_off, int scale_off,
                             int tokens, int rows, int C, float* out, hipStream_t s) {
  hipLaunchKernelGGL(ln_mod_kernel, dim3(rows), dim3(64), 0, s, x, mod, mod_stride, shift_off, scale_off, tokens,
                     rows, C, out);
  return hipGetLastError();
}

hipError_t launch_toy_linear(const ToyLinearArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(linear_f32_kernel, dim3((a.n + kT - 1) / kT, (a.m + kT - 1) / kT), dim3(kT * kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ca2
