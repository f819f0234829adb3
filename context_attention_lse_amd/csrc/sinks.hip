// Sink-robust const-max ("Kernel reference: ring_attention_const_max_fwd", Adapting this
// kernel: a handful of keys whose norms dwarf the rest inflate max_j |k_j| for every row;
// excluding them from the max recovers the bound).
//
//  sink prologue, over every chunk of the ring:
//    1. per (batch, head): max |k_j|^2 and the sum of |k_j|;
//    2. keys with |k_j| > theta * mean |k| join the head's sink list (up to `cap`), every
//       other key feeds the robust max of |k_j|^2;
//    3. a head with more than `cap` candidates keeps the plain max and no sinks; each list
//       is sorted (ascending key index), so every later sum runs in one order.
//  sink gather: the listed keys' K and V rows, for an exact attention over them alone.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 256;
constexpr int KTOK = 32;   // tokens (of every head) per workgroup

__device__ __forceinline__ float row_sqnorm16(const void* base, int64_t off, int lane16, int D, bool bf16) {
  float acc = 0.0f;
  if (lane16 * 8 < D) {
    if (bf16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off + lane16 * 8);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = __uint_as_float(u[t] << 16), hi = __uint_as_float(u[t] & 0xffff0000u);
        acc = fmaf(lo, lo, acc);
        acc = fmaf(hi, hi, acc);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + lane16 * 8);
      const float4 a = p[0], b = p[1];
      acc = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
  }
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
  return acc;
}

struct SinkPool {
  const void* k;
  int64_t cs, sb, ss, sh;   // element strides: chunk, batch, token, head
  int cp, B, S, H, D;
  bool bf16;
};

// grid (ceil(S / KTOK), B, cp). SELECT = false: per-head max |k|^2 (kmax_sq) and sum of |k|
// (knorm_sum). SELECT = true: keys above theta * mean |k| go to the sink list, the others
// feed kmax_robust.
template <bool SELECT>
__global__ __launch_bounds__(NT) void sink_pass_kernel(const SinkPool p, float theta, int cap, float* kmax_sq,
                                                       float* knorm_sum, float* kmax_robust, int32_t* sink_idx,
                                                       int32_t* sink_cnt) {
  extern __shared__ float sm[];   // [H] max bits, then [H] sums
  int* smax = reinterpret_cast<int*>(sm);
  float* ssum = sm + p.H;
  const int b = blockIdx.y, c = blockIdx.z;
  for (int h = threadIdx.x; h < p.H; h += NT) { smax[h] = 0; ssum[h] = 0.0f; }
  __syncthreads();
  const int grp = threadIdx.x >> 4, lane16 = threadIdx.x & 15;
  const int t0 = blockIdx.x * KTOK;
  const int rows = min(KTOK, p.S - t0) * p.H;
  const float inv_n = 1.0f / (float(p.cp) * float(p.S));
  for (int r = grp; r < rows; r += NT / 16) {
    const int i = r / p.H, h = r - i * p.H;
    const int64_t off = int64_t(c) * p.cs + int64_t(b) * p.sb + int64_t(t0 + i) * p.ss + int64_t(h) * p.sh;
    const float n2 = row_sqnorm16(p.k, off, lane16, p.D, p.bf16);
    if (lane16 != 0) continue;
    if (!SELECT) {
      atomicMax(&smax[h], __float_as_int(n2));
      atomicAdd(&ssum[h], sqrtf(n2));
    } else {
      const int bh = b * p.H + h;
      const float thr = theta > 0.0f ? theta * knorm_sum[bh] * inv_n : INFINITY;
      if (sqrtf(n2) > thr) {
        const int slot = atomicAdd(&sink_cnt[bh], 1);
        if (slot < cap) sink_idx[int64_t(bh) * cap + slot] = c * p.S + t0 + i;
      } else {
        atomicMax(&smax[h], __float_as_int(n2));
      }
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < p.H; h += NT) {
    const int bh = b * p.H + h;
    if (!SELECT) {
      if (smax[h] > 0) atomicMax(reinterpret_cast<int*>(kmax_sq) + bh, smax[h]);
      atomicAdd(&knorm_sum[bh], ssum[h]);
    } else if (smax[h] > 0) {
      atomicMax(reinterpret_cast<int*>(kmax_robust) + bh, smax[h]);
    }
  }
}

// One thread per (batch, head): overflow falls back to the plain max and no sinks; the
// list is sorted so that later sums over it run in key order.
__global__ void sink_finalize_kernel(int BH, int cap, const float* kmax_sq, float* kmax_robust, int32_t* sink_idx,
                                     int32_t* sink_cnt) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  const int n = sink_cnt[bh];
  if (n > cap) {
    kmax_robust[bh] = kmax_sq[bh];
    sink_cnt[bh] = 0;
    return;
  }
  int32_t* l = sink_idx + int64_t(bh) * cap;
  for (int i = 1; i < n; ++i) {
    const int32_t x = l[i];
    int j = i - 1;
    while (j >= 0 && l[j] > x) { l[j + 1] = l[j]; --j; }
    l[j + 1] = x;
  }
}

__global__ void zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// grid (B * H): copies head h's listed K and V rows of sequence b into kg, vg
// ([B, cap, H, D], bf16). A 16-lane group moves one 256-byte row.
__global__ __launch_bounds__(NT) void sink_gather_kernel(const uint16_t* k, const uint16_t* v, int64_t cs, int64_t sb,
                                                         int64_t ss, int64_t sh, int S, int H, int cap,
                                                         const int32_t* sink_idx, const int32_t* sink_cnt,
                                                         uint16_t* kg, uint16_t* vg) {
  constexpr int D = 128;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int n = min(sink_cnt[bh], cap);
  const int grp = threadIdx.x >> 4, lane16 = threadIdx.x & 15;
  for (int slot = grp; slot < n; slot += NT / 16) {
    const int g = sink_idx[int64_t(bh) * cap + slot];
    const int c = g / S, t = g - (g / S) * S;
    const int64_t src = int64_t(c) * cs + int64_t(b) * sb + int64_t(t) * ss + int64_t(h) * sh + lane16 * 8;
    const int64_t dst = ((int64_t(b) * cap + slot) * H + h) * D + lane16 * 8;
    *reinterpret_cast<uint4*>(kg + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(vg + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

}  // namespace

hipError_t launch_sink_prologue(const void* k, int64_t cs, int64_t sb, int64_t ss, int64_t sh, bool bf16, int cp,
                                int B, int S, int H, int D, float theta, int cap, float* kmax_sq, float* knorm_sum,
                                float* kmax_robust, int32_t* sink_idx, int32_t* sink_cnt, hipStream_t s) {
  const int BH = B * H;
  // zero the four [B, H] outputs (a fill kernel, not a memset, so that the call captures)
  float* zero[4] = {kmax_sq, knorm_sum, kmax_robust, reinterpret_cast<float*>(sink_cnt)};
  for (float* z : zero) {
    hipLaunchKernelGGL(zero_kernel, dim3((BH + 255) / 256), dim3(256), 0, s, z, BH);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (S > 0 && cp > 0) {
    SinkPool p{k, cs, sb, ss, sh, cp, B, S, H, D, bf16};
    dim3 grid(unsigned((S + KTOK - 1) / KTOK), B, cp);
    const size_t lds = size_t(H) * 2 * sizeof(float);
    hipLaunchKernelGGL(sink_pass_kernel<false>, grid, dim3(NT), lds, s, p, theta, cap, kmax_sq, knorm_sum, kmax_robust,
                       sink_idx, sink_cnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sink_pass_kernel<true>, grid, dim3(NT), lds, s, p, theta, cap, kmax_sq, knorm_sum, kmax_robust,
                       sink_idx, sink_cnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sink_finalize_kernel, dim3((BH + 255) / 256), dim3(256), 0, s, BH, cap, kmax_sq, kmax_robust,
                     sink_idx, sink_cnt);
  return hipGetLastError();
}

hipError_t launch_sink_gather(const void* k, const void* v, int64_t cs, int64_t sb, int64_t ss, int64_t sh, int B,
                              int S, int H, int cap, const int32_t* sink_idx, const int32_t* sink_cnt, void* kg,
                              void* vg, hipStream_t s) {
  hipLaunchKernelGGL(sink_gather_kernel, dim3(unsigned(B * H)), dim3(NT), 0, s, static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), cs, sb, ss, sh, S, H, cap, sink_idx, sink_cnt,
                     static_cast<uint16_t*>(kg), static_cast<uint16_t*>(vg));
  return hipGetLastError();
}

}  // namespace ctxattn
