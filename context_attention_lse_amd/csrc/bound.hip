// Const-max prologue kernels ("Kernel reference: ring_attention_const_max_fwd",
// Implementation: fused norms, global key max, assembling the bound).
//
//  key_sqnorm_max: per (batch, head) max over a chunk's keys of |k_j|^2, folded by max
//                  into [B, H] (the ring's all_reduce(max) becomes this fold on one GPU);
//  const_max_bound: c_i = sqrt(scale^2 * kmax_sq * |q_i|^2) per query row.
// Both read their input once with 16-byte loads; 16 lanes reduce one 128-wide row.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 256;

template <bool BF16>
__device__ __forceinline__ float sqnorm_part(const void* base, int64_t off, int lane16, int D) {
  // lane16 covers elements [8*lane16, 8*lane16+8) of the row (and +128 for D > 128 is not needed).
  float acc = 0.0f;
  if (BF16) {
    for (int c = lane16 * 8; c < D; c += 128) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = bf16_bits_to_float(w[t] & 0xffffu);
        const float hi = __uint_as_float(w[t] & 0xffff0000u);
        acc = fmaf(lo, lo, acc);
        acc = fmaf(hi, hi, acc);
      }
    }
  } else {
    for (int c = lane16 * 8; c < D; c += 128) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + c);
      const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + c + 4);
      acc = fmaf(x.x, x.x, acc); acc = fmaf(x.y, x.y, acc); acc = fmaf(x.z, x.z, acc); acc = fmaf(x.w, x.w, acc);
      acc = fmaf(y.x, y.x, acc); acc = fmaf(y.y, y.y, acc); acc = fmaf(y.z, y.z, acc); acc = fmaf(y.w, y.w, acc);
    }
  }
  // reduce over the 16 lanes of the row group
  for (int off2 = 8; off2 > 0; off2 >>= 1) acc += __shfl_xor(acc, off2, 16);
  return acc;
}

__global__ void fill_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// grid: (token tiles, B); a block handles TOK tokens x all heads.
template <bool BF16>
__global__ __launch_bounds__(NT) void key_sqnorm_max_kernel(const void* k, int64_t sb, int64_t ss, int64_t sh,
                                                            int S, int H, int D, float* kmax_sq, int tok_per_blk) {
  extern __shared__ int smax[];   // [H] as ordered ints (non-negative floats)
  const int b = blockIdx.y;
  for (int h = threadIdx.x; h < H; h += NT) smax[h] = 0;
  __syncthreads();
  const int grp = threadIdx.x >> 4;   // 16 row-groups of 16 lanes
  const int lane16 = threadIdx.x & 15;
  const int t0 = blockIdx.x * tok_per_blk;
  const int t1 = min(S, t0 + tok_per_blk);
  const int pairs = (t1 - t0) * H;
  for (int p0 = 0; p0 < pairs; p0 += NT / 16) {
    const int p = p0 + grp;
    // p is uniform across the 16 lanes of a group, so the group-wide reduction inside
    // sqnorm_part always runs with all 16 lanes active.
    if (p < pairs) {
      const int t = t0 + p / H;
      const int hh = p % H;
      const float v = sqnorm_part<BF16>(k, b * sb + int64_t(t) * ss + hh * sh, lane16, D);
      if (lane16 == 0) atomicMax(&smax[hh], __float_as_int(v));
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += NT)
    atomicMax(reinterpret_cast<int*>(kmax_sq) + b * H + h, smax[h]);
}

// grid: (ceil(Sq*H / 16), B); one 16-lane group per (row, head).
template <bool BF16>
__global__ __launch_bounds__(NT) void const_max_bound_kernel(const void* q, int64_t sb, int64_t ss, int64_t sh,
                                                             int Sq, int H, int D, float scale,
                                                             const float* kmax_sq, float* c) {
  const int b = blockIdx.y;
  const int p = blockIdx.x * (NT / 16) + (threadIdx.x >> 4);
  const int lane16 = threadIdx.x & 15;
  const bool live = p < Sq * H;
  const int i = live ? p / H : 0;
  const int h = live ? p % H : 0;
  const float qn2 = sqnorm_part<BF16>(q, b * sb + int64_t(i) * ss + h * sh, lane16, D);
  if (live && lane16 == 0) {
    const float km = kmax_sq[b * H + h];
    c[(int64_t(b) * H + h) * Sq + i] = sqrtf(scale * scale * km * qn2);
  }
}

}  // namespace

hipError_t launch_key_sqnorm_max(const void* k, int64_t sb, int64_t ss, int64_t sh, bool bf16, int B, int S,
                                 int H, int D, float* kmax_sq, bool accumulate, hipStream_t s) {
  if (!accumulate) {
    const int n = B * H;
    hipLaunchKernelGGL(fill_kernel, dim3((n + 255) / 256), dim3(256), 0, s, kmax_sq, n, 0.0f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (S == 0 || B == 0) return hipSuccess;
  const int tok = 64;
  dim3 grid((S + tok - 1) / tok, B);
  const size_t lds = size_t(H) * sizeof(int);
  if (bf16)
    hipLaunchKernelGGL((key_sqnorm_max_kernel<true>), grid, dim3(NT), lds, s, k, sb, ss, sh, S, H, D, kmax_sq, tok);
  else
    hipLaunchKernelGGL((key_sqnorm_max_kernel<false>), grid, dim3(NT), lds, s, k, sb, ss, sh, S, H, D, kmax_sq, tok);
  return hipGetLastError();
}

hipError_t launch_const_max_bound(const void* q, int64_t sb, int64_t ss, int64_t sh, bool bf16, int B, int Sq,
                                  int H, int D, float scale, const float* kmax_sq, float* c, hipStream_t s) {
  if (Sq == 0 || B == 0) return hipSuccess;
  dim3 grid((Sq * H + (NT / 16) - 1) / (NT / 16), B);
  if (bf16)
    hipLaunchKernelGGL((const_max_bound_kernel<true>), grid, dim3(NT), 0, s, q, sb, ss, sh, Sq, H, D, scale, kmax_sq, c);
  else
    hipLaunchKernelGGL((const_max_bound_kernel<false>), grid, dim3(NT), 0, s, q, sb, ss, sh, Sq, H, D, scale, kmax_sq, c);
  return hipGetLastError();
}

}  // namespace ctxattn
