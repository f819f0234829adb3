// LSE-corrected merge of n partial attention results (DCP page, decode compute
// pattern: partial LSE, global LSE, weight_s = exp(lse_s - global_lse), weighted sum).
//
// Bandwidth-bound: every partial row is read exactly once with 16-byte loads, the
// output is written once. D/4 lanes cover one row; the n row LSEs are read by every
// lane of the row (one cache line, broadcast within the wave). For n <= 8 every load of a
// row (the n LSEs and the n output pieces) is issued before any is used, so a lane makes
// one trip to memory: waiting for the LSEs before loading the outputs (two trips) ran the
// 8-way merge of the 720p ring at 5.61 TB/s, one trip at 6.04 TB/s.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 256;
constexpr int NMAX_ONE_TRIP = 8;   // partials held in registers by the one-trip path

template <bool OUT_BF16>
__device__ __forceinline__ void store_row(void* o_out, int64_t at, float4 out) {
  if (OUT_BF16) {
    uint2 u;
    u.x = pack_bf16x2(out.x, out.y);
    u.y = pack_bf16x2(out.z, out.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o_out) + at) = u;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(o_out) + at) = out;
  }
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(NT) void lse_merge_kernel(int n, const float* __restrict__ o_parts,
                                                       const float* __restrict__ lse_parts,
                                                       int64_t rows, void* __restrict__ o_out,
                                                       float* __restrict__ lse_out) {
  constexpr int LPR = D / 4;            // lanes per row
  constexpr int RPB = NT / LPR;         // rows per block
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int col = (threadIdx.x % LPR) * 4;
  if (row >= rows) return;
  const float* src = o_parts + row * D + col;
  const int64_t pstride = rows * D;
  float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
  float g = -INFINITY;

  if (n <= NMAX_ONE_TRIP) {   // uniform over the grid
    float l[NMAX_ONE_TRIP];
    floatx4 v[NMAX_ONE_TRIP];
#pragma unroll
    for (int s = 0; s < NMAX_ONE_TRIP; ++s) {
      if (s < n) {
        l[s] = lse_parts[int64_t(s) * rows + row];
        v[s] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + s * pstride));
      } else {
        l[s] = -INFINITY;
        v[s] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NMAX_ONE_TRIP; ++s) M = fmaxf(M, l[s]);
    if (M != -INFINITY) {
      float total = 0.0f;
#pragma unroll
      for (int s = 0; s < NMAX_ONE_TRIP; ++s)
        if (s < n) total += __expf(l[s] - M);
      g = M + __logf(total);
#pragma unroll
      for (int s = 0; s < NMAX_ONE_TRIP; ++s) {
        if (s < n) {
          const float wt = __expf(l[s] - g);
          out.x = fmaf(wt, v[s][0], out.x); out.y = fmaf(wt, v[s][1], out.y);
          out.z = fmaf(wt, v[s][2], out.z); out.w = fmaf(wt, v[s][3], out.w);
        }
      }
    }
  } else {
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, lse_parts[int64_t(s) * rows + row]);
    if (M != -INFINITY) {
      float total = 0.0f;
      for (int s = 0; s < n; ++s) total += __expf(lse_parts[int64_t(s) * rows + row] - M);
      g = M + __logf(total);
      int s = 0;
      for (; s + 4 <= n; s += 4) {
        floatx4 v[4];
        float wt[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + (s + u) * pstride));
          wt[u] = __expf(lse_parts[int64_t(s + u) * rows + row] - g);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          out.x = fmaf(wt[u], v[u][0], out.x); out.y = fmaf(wt[u], v[u][1], out.y);
          out.z = fmaf(wt[u], v[u][2], out.z); out.w = fmaf(wt[u], v[u][3], out.w);
        }
      }
      for (; s < n; ++s) {
        const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + s * pstride));
        const float wt = __expf(lse_parts[int64_t(s) * rows + row] - g);
        out.x = fmaf(wt, v[0], out.x); out.y = fmaf(wt, v[1], out.y);
        out.z = fmaf(wt, v[2], out.z); out.w = fmaf(wt, v[3], out.w);
      }
    }
  }
  store_row<OUT_BF16>(o_out, row * D + col, out);
  if (lse_out && col == 0) lse_out[row] = g;
}

template <int D>
hipError_t launch_d(int n, const float* o_parts, const float* lse_parts, int64_t rows, void* o_out,
                    int o_bf16, float* lse_out, hipStream_t s) {
  constexpr int RPB = NT / (D / 4);
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  if (o_bf16)
    hipLaunchKernelGGL((lse_merge_kernel<D, true>), dim3(unsigned(blocks)), dim3(NT), 0, s, n, o_parts,
                       lse_parts, rows, o_out, lse_out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<D, false>), dim3(unsigned(blocks)), dim3(NT), 0, s, n, o_parts,
                       lse_parts, rows, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(int n, const float* o_parts, const float* lse_parts, int64_t rows, int D,
                            void* o_out, int o_bf16, float* lse_out, hipStream_t s) {
  switch (D) {
    case 64: return launch_d<64>(n, o_parts, lse_parts, rows, o_out, o_bf16, lse_out, s);
    case 128: return launch_d<128>(n, o_parts, lse_parts, rows, o_out, o_bf16, lse_out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ctxattn
