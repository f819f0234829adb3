// Vector (VALU) attention step kernels, online-max and const-max, with fp32 arithmetic.
//
// Same two methods as the MFMA path (see attn_bf16.hip), computed with fp32 vector FMAs and
// accurate expf/logf. They serve inputs the MFMA kernel does not take: fp32 inputs end to
// end (a bf16 rounding of fp32 inputs would be charged to the scores), and bf16 inputs with
// head_dim 64 (the MFMA kernel is built for 128, the head size the kernel reference page's
// Interface asserts), whose elements are widened to fp32 as they are loaded. Two lanes
// share one query row, each holding half of the head dimension; keys stream through LDS in
// fp32 tiles of 32.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 256;        // threads per workgroup
constexpr int ROWS = NT / 2;   // query rows per workgroup
constexpr int TK = 32;         // keys per LDS tile

enum { MODE_ONLINE = 0, MODE_CONSTMAX = 1 };

// Element loads widened to fp32: T = float (fp32 inputs) or uint16_t (bf16 bits).
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_float(*p); }
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {   // 8-byte aligned: 4 elements of a 16-byte-aligned row
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

template <int MODE, int MASK, int D, typename T>
__global__ __launch_bounds__(NT) void attn_step_f32(const AttnArgs a, int nqb) {
  constexpr int DH = D / 2;
  __shared__ __attribute__((aligned(16))) float Ks[TK][D];
  __shared__ __attribute__((aligned(16))) float Vs[TK][D];

  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x - bh * nqb;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int i = qb * ROWS + (tid >> 1);
  const int Sq = a.Sq, Sk = a.Sk;
  const bool live_row = i < Sq;

  float q[DH], acc[DH];
  const T* qrow = static_cast<const T*>(a.q) + b * a.qsb + int64_t(live_row ? i : 0) * a.qss + h * a.qsh + half * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = live_row ? load1(qrow + d) : 0.0f;
    acc[d] = 0.0f;
  }
  const T* kbase = static_cast<const T*>(a.k) + b * a.ksb + h * a.ksh;
  const T* vbase = static_cast<const T*>(a.v) + b * a.ksb + h * a.ksh;

  float m = -INFINITY, l = 0.0f, c = 0.0f;
  if (MODE == MODE_CONSTMAX && live_row) c = a.c[int64_t(bh) * Sq + i];

  int kend = Sk;
  if (MASK != CA_MASK_NONE) kend = min(Sk, qb * ROWS + ROWS);

  for (int key0 = 0; key0 < kend; key0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * D / 4; e += NT) {
      const int row = e / (D / 4);
      const int col = (e - row * (D / 4)) * 4;
      const int key = key0 + row;
      float4 kv = make_float4(0, 0, 0, 0), vv = kv;
      if (key < Sk) {
        kv = load4(kbase + key * a.kss + col);
        vv = load4(vbase + key * a.kss + col);
      }
      *reinterpret_cast<float4*>(&Ks[row][col]) = kv;
      *reinterpret_cast<float4*>(&Vs[row][col]) = vv;
    }
    __syncthreads();

    float s[TK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float part = 0.0f;
#pragma unroll
      for (int d = 0; d < DH; ++d) part = fmaf(q[d], Ks[j][half * DH + d], part);
      const float full = part + __shfl_xor(part, 1);
      const int key = key0 + j;
      bool ok = key < Sk;
      if (MASK == CA_MASK_CAUSAL_INCL) ok &= key <= i;
      if (MASK == CA_MASK_CAUSAL_STRICT) ok &= key < i;
      s[j] = ok ? full * a.scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    float mu;
    if (MODE == MODE_ONLINE) {
      const float m_new = fmaxf(m, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.0f : expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] *= alpha;
      m = m_new;
      mu = (m == -INFINITY) ? 0.0f : m;
    } else {
      mu = c;
    }
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float p = expf(s[j] - mu);
      l += p;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, Vs[j][half * DH + d], acc[d]);
    }
  }

  if (!live_row) return;
  const int64_t rowidx = int64_t(bh) * Sq + i;
  if (MODE == MODE_ONLINE) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse_t = l > 0.0f ? m + logf(l) : -INFINITY;
    float* orow = a.o + rowidx * D + half * DH;
    if (a.fold) {
      // merge with the prior partial in o / lse (the row's two threads are adjacent lanes of
      // one wave: both read the prior LSE before either writes)
      float w_p, w_t;
      const float L = lse_fold_weights(a.lse[rowidx], lse_t, w_p, w_t);
      const float wt = w_t * inv;
#pragma unroll
      for (int d = 0; d < DH; ++d) orow[d] = w_p * orow[d] + wt * acc[d];
      if (half == 0) a.lse[rowidx] = L;
    } else {
#pragma unroll
      for (int d = 0; d < DH; ++d) orow[d] = acc[d] * inv;
      if (half == 0) a.lse[rowidx] = lse_t;
    }
  } else {
    const int64_t rows = int64_t(a.B) * a.H * Sq;
    float* arow = a.acc ? a.acc + rowidx * D + half * DH : nullptr;
    float sum = l;
    if (!(a.phase & CA_PHASE_INIT)) {
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] += arow[d];
      sum += a.acc[rows * D + rowidx];
    }
    if (!(a.phase & CA_PHASE_FINAL)) {
#pragma unroll
      for (int d = 0; d < DH; ++d) arow[d] = acc[d];
      if (half == 0) a.acc[rows * D + rowidx] = sum;
    } else {
      const float z = fmaxf(sum, kSumClamp);
      const float inv = 1.0f / z;
      if (a.o_cm_bf16) {
        uint16_t* orow = static_cast<uint16_t*>(a.o_cm) + rowidx * D + half * DH;
#pragma unroll
        for (int d = 0; d < DH; d += 2) {
          const uint32_t pk = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
          *reinterpret_cast<uint32_t*>(orow + d) = pk;
        }
      } else {
        float* orow = static_cast<float*>(a.o_cm) + rowidx * D + half * DH;
#pragma unroll
        for (int d = 0; d < DH; ++d) orow[d] = acc[d] * inv;
      }
      if (half == 0 && a.lse_cm) a.lse_cm[rowidx] = c + logf(z);
    }
  }
}

template <int MODE, int MASK, int D, typename T>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.Sq + ROWS - 1) / ROWS;
  const int64_t nblk = int64_t(a.B) * a.H * nqb;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_step_f32<MODE, MASK, D, T>), dim3(unsigned(nblk)), dim3(NT), 0, s, a, nqb);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t dispatch(const AttnArgs& a, bool const_max, hipStream_t s) {
  if (const_max) return launch_one<MODE_CONSTMAX, CA_MASK_NONE, D, T>(a, s);
  switch (a.mask) {
    case CA_MASK_CAUSAL_INCL: return launch_one<MODE_ONLINE, CA_MASK_CAUSAL_INCL, D, T>(a, s);
    case CA_MASK_CAUSAL_STRICT: return launch_one<MODE_ONLINE, CA_MASK_CAUSAL_STRICT, D, T>(a, s);
    default: return launch_one<MODE_ONLINE, CA_MASK_NONE, D, T>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, bool const_max, bool bf16_in, hipStream_t s) {
  if (bf16_in) return dispatch<64, uint16_t>(a, const_max, s);   // bf16 reaches here with D == 64 only
  return a.D == 64 ? dispatch<64, float>(a, const_max, s) : dispatch<128, float>(a, const_max, s);
}

}  // namespace ctxattn
