// Const-max prologue kernels ("Kernel reference: ring_attention_const_max_fwd",
// Implementation: fused norms, global key max, assembling the bound).
//
//  key_sqnorm_max: per (batch, head) max over a chunk's keys of |k_j|^2, folded by max
//                  into [B, H] (the ring's all_reduce(max) becomes this fold on one GPU);
//  const_max_bound: c_i = sqrt(scale^2 * kmax_sq * |q_i|^2) per query row.
// Both read their input once with 16-byte loads, several rows in flight per lane group.
#include <algorithm>

#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 256;

// Rows are (token, head) pairs taken in token-major order. A 16-lane group reads one row:
// lane l holds elements [8l, 8l + 8) (lanes past D hold zeros, so D = 64 uses lanes 0-7).
// Each group keeps RIF rows' loads in flight before reducing any of them.
constexpr int RIF = 8;                  // rows in flight per 16-lane group
constexpr int GROUPS = NT / 16;         // 16-lane groups per block

template <bool BF16>
struct RowPiece {
  // elements [8*lane16, 8*lane16 + 8) of a row; fp32 rows are 2 x 16 bytes
  floatx4 a, b;
};

template <bool BF16>
__device__ __forceinline__ RowPiece<BF16> load_piece(const void* base, int64_t off, int lane16, int D) {
  RowPiece<BF16> r;
  r.a = floatx4{0.f, 0.f, 0.f, 0.f};
  r.b = r.a;
  // Non-temporal loads: the rows are read once and streamed past the caches (the 774 MB key
  // pool of the 720p ring: 171 us with ordinary loads, 154 us with these, bound kernel included)
  if (lane16 * 8 < D) {
    if (BF16) {
      r.a = __builtin_nontemporal_load(
          reinterpret_cast<const floatx4*>(static_cast<const uint16_t*>(base) + off + lane16 * 8));
    } else {
      const floatx4* p = reinterpret_cast<const floatx4*>(static_cast<const float*>(base) + off + lane16 * 8);
      r.a = __builtin_nontemporal_load(p);
      r.b = __builtin_nontemporal_load(p + 1);
    }
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ float piece_sqnorm(const RowPiece<BF16>& r) {
  float acc = 0.0f;
  if (BF16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = __float_as_uint(r.a[t]);
      const float lo = __uint_as_float(w << 16);
      const float hi = __uint_as_float(w & 0xffff0000u);
      acc = fmaf(lo, lo, acc);
      acc = fmaf(hi, hi, acc);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(r.a[t], r.a[t], acc);
      acc = fmaf(r.b[t], r.b[t], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float group16_sum(float v) {
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

__global__ void fill_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// grid: (G, B) with G at most a few workgroups per CU; workgroup x takes the tiles of KTOK
// tokens (of every head) x, x + G, ... Per-head maxima gather in LDS, then one global
// atomicMax per head per workgroup. Squared norms are non-negative floats, whose bit
// patterns order like ints, so the max is exact and independent of arrival order. The
// stride keeps every workgroup busy to the end (one tile per workgroup left a partly filled
// second round of workgroups for long key runs).
constexpr int KTOK = 32;   // tokens (of every head) per key-norm tile

template <bool BF16>
__global__ __launch_bounds__(NT) void key_sqnorm_max_kernel(const void* k, int64_t sb, int64_t ss, int64_t sh,
                                                            int S, int H, int D, float* kmax_sq) {
  extern __shared__ int smax[];   // [H]
  const int b = blockIdx.y;
  for (int h = threadIdx.x; h < H; h += NT) smax[h] = 0;
  __syncthreads();
  const int grp = threadIdx.x >> 4;
  const int lane16 = threadIdx.x & 15;
  for (int t0 = blockIdx.x * KTOK; t0 < S; t0 += gridDim.x * KTOK) {
    const int rows = min(KTOK, S - t0) * H;   // this tile's (token, head) rows, token major
    for (int r0 = 0; r0 < rows; r0 += GROUPS * RIF) {
      RowPiece<BF16> r[RIF];
#pragma unroll
      for (int u = 0; u < RIF; ++u) {
        const int p = r0 + u * GROUPS + grp;
        const int pc = p < rows ? p : 0;
        const int i = pc / H, h = pc - i * H;
        r[u] = load_piece<BF16>(k, b * sb + int64_t(t0 + i) * ss + int64_t(h) * sh, lane16, D);
      }
#pragma unroll
      for (int u = 0; u < RIF; ++u) {
        const int p = r0 + u * GROUPS + grp;
        // p is uniform over the 16 lanes of a group, so the reduction runs with all 16 active
        const float v = group16_sum(piece_sqnorm<BF16>(r[u]));
        if (p < rows && lane16 == 0) atomicMax(&smax[p - (p / H) * H], __float_as_int(v));
      }
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += NT)
    if (smax[h] > 0) atomicMax(reinterpret_cast<int*>(kmax_sq) + b * H + h, smax[h]);
}

// grid: (ceil(Sq / TOK), B): c_i = sqrt(scale^2 * kmax_sq[b,h] * |q_i|^2). A workgroup
// takes TOK consecutive tokens of every head: it reads their rows in memory order (token
// major), keeps |q|^2 in LDS as [head][token], and writes c one head at a time, so the
// [B, H, Sq] output goes out in runs of TOK consecutive floats. Eight tokens give the 720p
// share 1182 workgroups, a fuller last round than 591 of sixteen.
constexpr int TOK = 8;

template <bool BF16>
__global__ __launch_bounds__(NT) void const_max_bound_kernel(const void* q, int64_t sb, int64_t ss, int64_t sh,
                                                             int Sq, int H, int D, float scale,
                                                             const float* kmax_sq, float* c) {
  extern __shared__ float qn[];   // [H][TOK]
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * TOK;
  const int ntok = min(TOK, Sq - t0);
  const int grp = threadIdx.x >> 4;
  const int lane16 = threadIdx.x & 15;
  const int rows = ntok * H;
  for (int r0 = 0; r0 < rows; r0 += GROUPS * RIF) {
    RowPiece<BF16> r[RIF];
#pragma unroll
    for (int u = 0; u < RIF; ++u) {
      const int p = r0 + u * GROUPS + grp;
      const int pc = p < rows ? p : 0;
      const int i = pc / H, h = pc - (pc / H) * H;
      r[u] = load_piece<BF16>(q, b * sb + int64_t(t0 + i) * ss + int64_t(h) * sh, lane16, D);
    }
#pragma unroll
    for (int u = 0; u < RIF; ++u) {
      const int p = r0 + u * GROUPS + grp;
      // p is uniform over the 16 lanes of a group, so the reduction runs with all 16 active
      const float v = group16_sum(piece_sqnorm<BF16>(r[u]));
      if (p < rows && lane16 == 0) {
        const int i = p / H, h = p - (p / H) * H;
        qn[h * TOK + i] = v;
      }
    }
  }
  __syncthreads();
  const float s2 = scale * scale;
  for (int e = threadIdx.x; e < H * TOK; e += NT) {
    const int h = e / TOK, i = e - (e / TOK) * TOK;
    if (i < ntok) c[(int64_t(b) * H + h) * Sq + t0 + i] = sqrtf(s2 * kmax_sq[b * H + h] * qn[e]);
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
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t tiles = (int64_t(S) + KTOK - 1) / KTOK;
  const int64_t per_b = std::max<int64_t>(1, (int64_t(4) * cus + B - 1) / B);   // about 4 workgroups per CU
  dim3 grid(unsigned(std::min(tiles, per_b)), B);
  const size_t lds = size_t(H) * sizeof(int);
  if (bf16)
    hipLaunchKernelGGL((key_sqnorm_max_kernel<true>), grid, dim3(NT), lds, s, k, sb, ss, sh, S, H, D, kmax_sq);
  else
    hipLaunchKernelGGL((key_sqnorm_max_kernel<false>), grid, dim3(NT), lds, s, k, sb, ss, sh, S, H, D, kmax_sq);
  return hipGetLastError();
}

hipError_t launch_const_max_bound(const void* q, int64_t sb, int64_t ss, int64_t sh, bool bf16, int B, int Sq,
                                  int H, int D, float scale, const float* kmax_sq, float* c, hipStream_t s) {
  if (Sq == 0 || B == 0) return hipSuccess;
  dim3 grid(unsigned((Sq + TOK - 1) / TOK), B);
  const size_t lds = size_t(H) * TOK * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL((const_max_bound_kernel<true>), grid, dim3(NT), lds, s, q, sb, ss, sh, Sq, H, D, scale, kmax_sq, c);
  else
    hipLaunchKernelGGL((const_max_bound_kernel<false>), grid, dim3(NT), lds, s, q, sb, ss, sh, Sq, H, D, scale, kmax_sq, c);
  return hipGetLastError();
}

}  // namespace ctxattn
