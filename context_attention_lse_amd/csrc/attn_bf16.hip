// bf16 MFMA attention step kernels for gfx950: one query block against one K/V chunk.
//
// Online-max mode: flash-style running row max / row sum / rescaled accumulator,
// emitting the chunk's normalised partial and per-row LSE ("Kernel reference:
// ring_attention_const_max_fwd", Design: the online-max path and its running max).
// Const-max mode: p = exp(s - c_i) with the fixed per-row bound and a pure-addition
// fold into an fp32 accumulator, normalised once with the 1e-37 clamp (same page,
// Design "A static bound makes the ring reduction pure addition", Implementation
// "Accumulate, then normalize once").
//
// Layout of the work (gfx950, wave64):
//  * a workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns 32 rows;
//  * keys stream through LDS in tiles of 64 (double-buffered, one barrier per tile);
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so a
//    lane holds 32 scores of ONE query row: the row max / row sum need one cross-half
//    exchange (lane l <-> l^32) per tile and no other cross-lane traffic;
//  * O^T = V^T P^T reuses the score registers directly as the B operand (no LDS round
//    trip for P); V is transposed once per tile while it is staged into LDS, with its
//    keys permuted so that each lane's 8 contiguous LDS values match the 8 score
//    registers it already holds;
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score; the running
//    max is moved only when a tile's max exceeds it by more than 8 (log2 units), so
//    the accumulator rescale is rare (probabilities stay <= 256, exact in fp32/bf16).
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int D = 128;        // head dim of the bf16 path
constexpr int BQ = 128;       // query rows per workgroup
constexpr int BK = 64;        // keys per LDS tile
constexpr int NT = 256;       // threads per workgroup
constexpr int KS = D + 8;     // LDS row stride (bf16) of a K row:   272 B
constexpr int VS = BK + 8;    // LDS row stride (bf16) of a V^T row: 144 B
constexpr int K_TILE = BK * KS;
constexpr int V_TILE = D * VS;
constexpr size_t LDS_BYTES = size_t(2) * (K_TILE + V_TILE) * sizeof(uint16_t);
constexpr float kRescaleSlack = 8.0f;   // log2 units the running max may lag the true max

enum { MODE_ONLINE = 0, MODE_CONSTMAX = 1 };

struct Stage {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ void load_stage(Stage& st, const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t kss, int key0, int Sk, int tid) {
  // K: 64 rows x 16 chunks of 16 B; thread tid takes chunks tid, tid+256, ...
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ci = tid + NT * u;
    const int row = ci >> 4;
    const int col = (ci & 15) * 8;
    const int key = key0 + row;
    st.k[u] = key < Sk ? *reinterpret_cast<const uint4*>(kbase + key * kss + col) : make_uint4(0, 0, 0, 0);
  }
  // V: thread (dg = tid % 16, kg = tid / 16) loads keys 4kg..4kg+3 at d = 8dg..8dg+7.
  const int dg = tid & 15;
  const int kg = tid >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = key0 + 4 * kg + e;
    st.v[e] = key < Sk ? *reinterpret_cast<const uint4*>(vbase + key * kss + dg * 8) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t word(const uint4& x, int w) {
  return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
}

__device__ __forceinline__ void store_stage(const Stage& st, uint16_t* Ks, uint16_t* Vt, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ci = tid + NT * u;
    const int row = ci >> 4;
    const int col = (ci & 15) * 8;
    *reinterpret_cast<uint4*>(Ks + row * KS + col) = st.k[u];
  }
  // Transpose the 4 (key) x 8 (d) block to 8 rows of V^T holding 4 keys each. Within each
  // 16-key chunk the keys are stored with bits 2 and 3 of their index swapped, so LDS
  // positions 0..7 hold keys {0-3, 8-11} and positions 8..15 keys {4-7, 12-15}: the
  // order of the score registers a lane feeds to the P.V product.
  const int dg = tid & 15;
  const int kg = tid >> 4;
  const int pos = (kg >> 2) * 16 + (((kg & 1) << 3) | ((kg & 2) << 1));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a0 = word(st.v[0], w), a1 = word(st.v[1], w);
    const uint32_t a2 = word(st.v[2], w), a3 = word(st.v[3], w);
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // d even: keys 0,1
    lo.y = __builtin_amdgcn_perm(a3, a2, 0x05040100u);   //         keys 2,3
    hi.x = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // d odd
    hi.y = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    const int d = dg * 8 + 2 * w;
    *reinterpret_cast<uint2*>(Vt + d * VS + pos) = lo;
    *reinterpret_cast<uint2*>(Vt + (d + 1) * VS + pos) = hi;
  }
}

template <int MODE, int MASK>
__global__ __launch_bounds__(NT, 2) void attn_step_bf16(const AttnArgs a, int nqb, int nwork) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Ks0 = lds;
  uint16_t* Vt0 = lds + 2 * K_TILE;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x, nwork);
  if (logical < 0) return;
  const int bh = logical / nqb;
  int qb = logical - bh * nqb;
  if (MASK != CA_MASK_NONE) qb = nqb - 1 - qb;   // heavy (late) query blocks first
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 31;
  const int hl = lane >> 5;
  const int row_w0 = qb * BQ + w * 32;   // first query row of this wave
  const int i = row_w0 + li;             // this lane's query row
  const int Sq = a.Sq, Sk = a.Sk;

  // Q fragment: row i, d = c*16 + 8*hl .. +7 for c = 0..7 (B operand of S^T = K Q^T).
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.qsb + int64_t(i) * a.qss + h * a.qsh;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 t = i < Sq ? *reinterpret_cast<const uint4*>(qrow + c * 16 + hl * 8) : make_uint4(0, 0, 0, 0);
    qf[c] = *reinterpret_cast<bf16x8*>(&t);
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + h * a.ksh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.ksb + h * a.ksh;

  int kend = Sk;
  if (MASK != CA_MASK_NONE) kend = min(Sk, qb * BQ + BQ);
  const int nkt = (kend + BK - 1) / BK;

  floatx16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

  float m_ref = -INFINITY;   // running reference max (log2 units), online mode
  float l_part = 0.0f;       // this lane's share of the row sum
  float c2 = 0.0f;           // const-max bound in log2 units
  if (MODE == MODE_CONSTMAX) {
    if (i < Sq) c2 = a.c[int64_t(bh) * Sq + i] * kLog2e;
  }
  const float sl2e = a.sl2e;

  Stage st;
  if (nkt > 0) {
    load_stage(st, kbase, vbase, a.kss, 0, Sk, tid);
    store_stage(st, Ks0, Vt0, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const uint16_t* Ks = Ks0 + buf * K_TILE;
    const uint16_t* Vt = Vt0 + buf * V_TILE;
    const int key0 = kt * BK;
    if (kt + 1 < nkt) load_stage(st, kbase, vbase, a.kss, key0 + BK, Sk, tid);

    // Is any key of this tile visible to any row of this wave?
    bool skip = false;
    bool need_mask = key0 + BK > Sk;
    if (MASK == CA_MASK_CAUSAL_INCL) {
      skip = key0 > row_w0 + 31;
      need_mask |= key0 + BK - 1 > row_w0;
    } else if (MASK == CA_MASK_CAUSAL_STRICT) {
      skip = key0 >= row_w0 + 31;
      need_mask |= key0 + BK - 1 >= row_w0;
    }

    if (!skip) {
      floatx16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
      const uint16_t* kr0 = Ks + li * KS + hl * 8;
      const uint16_t* kr1 = Ks + (32 + li) * KS + hl * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr0 + c * 16);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr1 + c * 16);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[c], s1, 0, 0, 0);
      }
      // s{jb}[r] is the raw score q_i . k_j for key j = key0 + 32*jb + 8*(r/4) + 4*hl + r%4.
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j0 = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int j1 = j0 + 32;
          bool ok0 = j0 < Sk, ok1 = j1 < Sk;
          if (MASK == CA_MASK_CAUSAL_INCL) { ok0 &= j0 <= i; ok1 &= j1 <= i; }
          if (MASK == CA_MASK_CAUSAL_STRICT) { ok0 &= j0 < i; ok1 &= j1 < i; }
          s0[r] = ok0 ? s0[r] : -INFINITY;
          s1[r] = ok1 ? s1[r] : -INFINITY;
        }
      }

      float mu;
      if (MODE == MODE_ONLINE) {
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float t2 = tmax * sl2e;
        const bool move = t2 > m_ref + kRescaleSlack;
        if (__any(move)) {
          const float m_new = move ? t2 : m_ref;
          const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_ref - m_new);
          l_part *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          m_ref = m_new;
        }
        mu = (m_ref == -INFINITY) ? 0.0f : m_ref;
      } else {
        mu = c2;
      }

      // p = exp2(s * scale*log2e - mu), packed to bf16 in the order the P.V product reads.
      bf16x8 pb[4];
      float psum = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        uint32_t wds[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = (kc & 1) * 8 + 2 * t;
          float x0 = (kc < 2 ? s0[r] : s1[r]);
          float x1 = (kc < 2 ? s0[r + 1] : s1[r + 1]);
          x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0, sl2e, -mu));
          x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1, sl2e, -mu));
          psum += x0 + x1;
          wds[t] = pack_bf16x2(x0, x1);
        }
        uint4 u4 = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        pb[kc] = *reinterpret_cast<bf16x8*>(&u4);
      }
      l_part += psum;

      // O^T[d][i] += sum_j V^T[d][j] P^T[j][i]
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vr = Vt + (db * 32 + li) * VS + hl * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vr + kc * 16);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kc], oacc[db], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < nkt) store_stage(st, Ks0 + (buf ^ 1) * K_TILE, Vt0 + (buf ^ 1) * V_TILE, tid);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  const float lrow = l_part + __shfl_xor(l_part, 32);
  if (i >= Sq) return;
  const int64_t rowidx = int64_t(bh) * Sq + i;
  // oacc[db][r] is O[i][d] for d = 32*db + 8*(r/4) + 4*hl + r%4: four consecutive d per float4.
  if (MODE == MODE_ONLINE) {
    const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
    float* orow = a.o + rowidx * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v4 = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl) = v4;
      }
    if (hl == 0) a.lse[rowidx] = lrow > 0.0f ? (m_ref + __log2f(lrow)) * kLn2 : -INFINITY;
  } else {
    const int64_t rows = int64_t(a.B) * a.H * Sq;
    float sum = lrow;
    if (!(a.phase & CA_PHASE_INIT)) {
      const float* arow = a.acc + rowidx * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 p4 = *reinterpret_cast<const float4*>(arow + db * 32 + 8 * g + 4 * hl);
          oacc[db][4 * g] += p4.x; oacc[db][4 * g + 1] += p4.y;
          oacc[db][4 * g + 2] += p4.z; oacc[db][4 * g + 3] += p4.w;
        }
      sum += a.acc[rows * D + rowidx];
    }
    if (!(a.phase & CA_PHASE_FINAL)) {
      float* arow = a.acc + rowidx * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(arow + db * 32 + 8 * g + 4 * hl) =
              make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
      if (hl == 0) a.acc[rows * D + rowidx] = sum;
    } else {
      const float z = fmaxf(sum, kSumClamp);
      const float inv = 1.0f / z;
      if (a.o_cm_bf16) {
        uint16_t* orow = static_cast<uint16_t*>(a.o_cm) + rowidx * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 u;
            u.x = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
            u.y = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + db * 32 + 8 * g + 4 * hl) = u;
          }
      } else {
        float* orow = static_cast<float*>(a.o_cm) + rowidx * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl) =
                make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                            oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
      if (hl == 0 && a.lse_cm) a.lse_cm[rowidx] = c2 * kLn2 + __logf(z);
    }
  }
}

template <int MODE, int MASK>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;   // dynamic LDS above 64 KB must be allowed once
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_step_bf16<MODE, MASK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(LDS_BYTES));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nqb = (a.Sq + BQ - 1) / BQ;
  const int nwork = a.B * a.H * nqb;
  if (nwork == 0) return hipSuccess;
  const int grid = round_up8(nwork);
  hipLaunchKernelGGL((attn_step_bf16<MODE, MASK>), dim3(grid), dim3(NT), LDS_BYTES, s, a, nqb, nwork);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, bool const_max, hipStream_t s) {
  if (const_max) return launch_one<MODE_CONSTMAX, CA_MASK_NONE>(a, s);
  switch (a.mask) {
    case CA_MASK_CAUSAL_INCL: return launch_one<MODE_ONLINE, CA_MASK_CAUSAL_INCL>(a, s);
    case CA_MASK_CAUSAL_STRICT: return launch_one<MODE_ONLINE, CA_MASK_CAUSAL_STRICT>(a, s);
    default: return launch_one<MODE_ONLINE, CA_MASK_NONE>(a, s);
  }
}

}  // namespace ctxattn
