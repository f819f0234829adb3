// DCP decode: one shard's partial attention over its paged, interleaved KV cache
// (DCP page, "DCP Decode" compute pattern steps 3-4: the gathered query heads attend
// the local KV shard and produce a partial output with its LSE).
//
// Work decomposition (bandwidth-bound: every resident K/V byte is read once):
//  * grid (split, kv head, sequence); a split is 1536 shard-local tokens (96 blocks), and
//    the grid holds an odd number of splits so every split index spreads over all XCDs;
//  * a workgroup is 4 waves; wave w streams 24 blocks of the split, two blocks per step,
//    with the loads of the next two steps in flight (a ring of three register sets);
//  * the GQA group's query heads (<= 16) share each K/V block: scores are
//    S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = 16 tokens, cols = heads), so
//    a block is read once for all heads of its group;
//  * V blocks are stored d-major ([D][16] per block and head), so the P.V product
//    O^T = V^T P^T loads its A operand with 8-byte reads and P never leaves registers;
//  * the four waves' partials fold in LDS into one (output, LSE) per split, and a
//    second kernel folds the splits of each sequence by the LSE rule;
//  * head_dim D = 128 or 64 (a template parameter): D/32 score MFMAs and D/16 output
//    MFMAs per block.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int BS = 16;                          // tokens per cache block
constexpr int NT = 256;
constexpr int WAVES = NT / 64;
constexpr int SPLIT_BLOCKS = kDecodeSplitTokens / BS;   // 96
constexpr int WAVE_BLOCKS = SPLIT_BLOCKS / WAVES;       // 24
static_assert(WAVE_BLOCKS % 2 == 0 && WAVE_BLOCKS <= 32, "block pairs per wave; one mask bit per block");
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct PairRegs {
  uint4 k[2][D / 32];   // [block][d chunk of 32]: 8 bf16 of row (token) c16
  uint2 v[2][D / 16];   // [block][d block of 16]: 4 bf16 (tokens 4g..4g+3) at d = 16*db + c16
};

// Loads one block pair; blk0 and blk1 are wave-uniform physical block ids, always inside
// the pool (the caller substitutes a resident block for missing ones), so the loads carry
// no branches and the compiler's wait counts stay exact.
template <int D>
__device__ __forceinline__ void load_pair(PairRegs<D>& r, const uint16_t* kp, const uint16_t* vp, int hkv, int Hkv,
                                          int blk0, int blk1, int g, int c16) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int64_t blk = bi == 0 ? blk0 : blk1;
    const uint16_t* kb = kp + ((blk * Hkv + hkv) * BS + c16) * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) r.k[bi][cc] = *reinterpret_cast<const uint4*>(kb + 32 * cc);
    // V rows stream past the caches (non-temporal): 2.9% faster per shard than ordinary loads;
    // the same for K was 7% slower (interleaved A/B on the decode workload)
    const uint16_t* vb = vp + ((blk * Hkv + hkv) * D + c16) * BS + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + 16 * BS * db));
      r.v[bi][db] = make_uint2(t[0], t[1]);
    }
  }
}

// Tokens of sequence b resident in this shard: given (local_lens) or derived from the
// sequence's prior length (current-token form); clamped to the block table.
__device__ __forceinline__ int resident_len(const DecodeArgs& a, int b) {
  const int n = a.prior_lens ? dcp_local_filled(max(a.prior_lens[b], 0), a.rank, BS, a.interleave, a.world)
                             : a.local_lens[b];
  return min(max(n, 0), a.max_blocks * BS);
}

template <int D>
__global__ __launch_bounds__(NT, 2) void dcp_decode_split_kernel(const DecodeArgs a) {
  __shared__ float s_o[WAVES][16][D];
  __shared__ float s_m[WAVES][16];
  __shared__ float s_l[WAVES][16];

  const int split = blockIdx.x;
  const int hkv = blockIdx.y;
  const int b = blockIdx.z;
  const int len = resident_len(a, b);
  const int split_tok0 = split * kDecodeSplitTokens;
  if (split_tok0 >= len) return;   // workgroup-uniform: nothing resident in this split
  const int nblk = (len + BS - 1) / BS;
  const int G = a.Hq / a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so block ids load as scalars
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // Q fragment: head c16 of the group (zero beyond G), d = 32*cc + 8*g .. +7.
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (int64_t(b) * a.Hq + hkv * G + min(c16, G - 1)) * D + 8 * g;
  bf16x8 qf[D / 32];
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc) {
    uint4 t = c16 < G ? *reinterpret_cast<const uint4*>(qh + 32 * cc) : make_uint4(0, 0, 0, 0);
    qf[cc] = *reinterpret_cast<bf16x8*>(&t);
  }

  const uint16_t* kp = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* btab = a.block_table + int64_t(b) * a.max_blocks;
  const int wave_blk0 = split * SPLIT_BLOCKS + w * WAVE_BLOCKS;

  floatx4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  float l_part = 0.0f;
  const float sl2e = a.sl2e;

  // Block pairs stream through a ring of three register sets: the loads of pair it + 2 are
  // issued before pair it is computed, so two pairs (32 KB per wave) stay in flight.
  auto compute = [&](const PairRegs<D>& cur, int jb0, uint32_t zero2) {
    floatx4 s[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      s[bi] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) {
        bf16x8 kf = *reinterpret_cast<const bf16x8*>(&cur.k[bi][cc]);
        s[bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[cc], s[bi], 0, 0, 0);
      }
      if ((zero2 >> bi) & 1) s[bi] = floatx4{0.f, 0.f, 0.f, 0.f};   // all-zero block: q.0
    }
    // s[bi][r]: score of head c16 against token (jb0 + bi)*16 + 4g + r
    float tmax = -INFINITY;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = (jb0 + bi) * BS + 4 * g + r;
        s[bi][r] = t < len ? s[bi][r] : -INFINITY;
        tmax = fmaxf(tmax, s[bi][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float t2 = tmax * sl2e;
    const bool move = t2 > m_ref + kRescaleSlack;
    if (__any(move)) {
      const float m_new = move ? t2 : m_ref;
      const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;
    float p[2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[bi][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bi][r], sl2e, -mu));
        l_part += p[bi][r];
      }
    uint4 pk = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
    const bf16x8 pb = *reinterpret_cast<bf16x8*>(&pk);
    const bool z0 = zero2 & 1, z1 = (zero2 >> 1) & 1;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      uint4 vv = make_uint4(z0 ? 0u : cur.v[0][db].x, z0 ? 0u : cur.v[0][db].y, z1 ? 0u : cur.v[1][db].x,
                            z1 ? 0u : cur.v[1][db].y);
      const bf16x8 vf = *reinterpret_cast<bf16x8*>(&vv);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, oacc[db], 0, 0, 0);
    }
  };

  // This wave's physical block ids (scalar loads). Past the sequence a resident block of
  // the split stands in (its scores are masked, so it adds nothing). An id outside the pool
  // reads as an all-zero block: its scores become 0 and its values 0 (bit i of zero_blk).
  const int first = btab[split * SPLIT_BLOCKS];
  const int fallback = (first >= 0 && first < a.num_blocks) ? first : 0;
  int bid[WAVE_BLOCKS];
  uint32_t zero_blk = 0;
#pragma unroll
  for (int i = 0; i < WAVE_BLOCKS; ++i) {
    const int j = wave_blk0 + i;
    const int blk = j < nblk ? btab[j] : fallback;
    const bool ok = blk >= 0 && blk < a.num_blocks;
    bid[i] = ok ? blk : fallback;
    zero_blk |= (ok ? 0u : 1u) << i;
  }

  constexpr int PAIRS = WAVE_BLOCKS / 2;
  PairRegs<D> ring[3];
  load_pair(ring[0], kp, vp, hkv, a.Hkv, bid[0], bid[1], g, c16);
  load_pair(ring[1], kp, vp, hkv, a.Hkv, bid[2], bid[3], g, c16);
#pragma unroll
  for (int it = 0; it < PAIRS; ++it) {
    const int jb0 = wave_blk0 + 2 * it;
    if (jb0 >= nblk) break;   // wave-uniform
    if (it + 2 < PAIRS) load_pair(ring[(it + 2) % 3], kp, vp, hkv, a.Hkv, bid[2 * it + 4], bid[2 * it + 5], g, c16);
    compute(ring[it % 3], jb0, (zero_blk >> (2 * it)) & 3u);
  }

  // Row sums per head: fold the 4 token groups (lanes c16, c16+16, c16+32, c16+48).
  float l_head = l_part + __shfl_xor(l_part, 16);
  l_head += __shfl_xor(l_head, 32);
  // oacc[db][r]: O^T[d = 16*db + 4*g + r][head c16] (unnormalised, reference m_ref)
  if (c16 < G) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[w][c16][16 * db + 4 * g + r] = oacc[db][r];
    if (g == 0) {
      s_m[w][c16] = m_ref;
      s_l[w][c16] = l_head;
    }
  }
  __syncthreads();

  // Fold the 4 waves: G heads x D outputs.
  const int64_t slot0 = (int64_t(b) * a.Hq + hkv * G) * a.max_splits + split;
  for (int e = tid; e < G * D; e += NT) {
    const int hh = e / D;
    const int d = e - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) M = fmaxf(M, s_l[ww][hh] > 0.0f ? s_m[ww][hh] : -INFINITY);
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        if (s_l[ww][hh] > 0.0f) {
          const float f = exp2f(s_m[ww][hh] - M);
          o = fmaf(f, s_o[ww][hh][d], o);
          l = fmaf(f, s_l[ww][hh], l);
        }
      }
    }
    const int64_t slot = slot0 + int64_t(hh) * a.max_splits;
    a.ws_o[slot * D + d] = l > 0.0f ? o / l : 0.0f;
    if (d == 0) a.ws_lse[slot] = l > 0.0f ? (M + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// One wave per row (sequence, query head) folds that sequence's splits: lane i holds split
// i's LSE (64 at a time) for the weights; for the outputs, the wave's lanes form 128 / D
// groups of D / 4 lanes (two half-waves for D = 128, four quarter-waves for D = 64) that
// take alternate splits, each lane four consecutive d, eight splits' loads in flight per round.
constexpr int COMBINE_WAVES = NT / 64;

template <int D>
__global__ __launch_bounds__(NT) void dcp_decode_combine_kernel(const DecodeArgs a) {
  constexpr int LPR = D / 4;     // lanes holding one row's D outputs
  constexpr int NG = 64 / LPR;   // lane groups, each taking every NG-th split
  constexpr int U = 8 / NG;      // loads per lane per round of eight splits
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * COMBINE_WAVES + (threadIdx.x >> 6);
  if (row >= int64_t(a.B) * a.Hq) return;   // wave-uniform
  const int b = int(row / a.Hq);
  const int len = resident_len(a, b);
  const int n = (len + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
  const float* lp = a.ws_lse + row * a.max_splits;
  const int grp = lane / LPR;
  const int col = (lane % LPR) * 4;
  const float* op = a.ws_o + row * a.max_splits * D + col;

  // Current-token form: on the owner of position N the current token is one more part,
  // with lse = its score and output = its value row (dcp_active_mask).
  bool cur = false;
  float s_cur = -INFINITY;
  float4 v_cur = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.prior_lens) {
    const int N = max(a.prior_lens[b], 0);
    cur = dcp_active_owner(N, BS, a.interleave, a.world) == a.rank;
    if (cur) {
      const int hq = int(row - int64_t(b) * a.Hq);
      const int64_t kv_row = int64_t(b) * a.Hkv + hq / (a.Hq / a.Hkv);
      const uint2 qb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.q) + row * D + col);
      const uint2 kb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.k_cur) + kv_row * D + col);
      const uint2 vb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v_cur) + kv_row * D + col);
      float dot = bf16_bits_to_float(qb.x & 0xffffu) * bf16_bits_to_float(kb.x & 0xffffu);
      dot = fmaf(bf16_bits_to_float(qb.x >> 16), bf16_bits_to_float(kb.x >> 16), dot);
      dot = fmaf(bf16_bits_to_float(qb.y & 0xffffu), bf16_bits_to_float(kb.y & 0xffffu), dot);
      dot = fmaf(bf16_bits_to_float(qb.y >> 16), bf16_bits_to_float(kb.y >> 16), dot);
      s_cur = a.scale * wave_sum(grp == 0 ? dot : 0.0f);
      v_cur = make_float4(bf16_bits_to_float(vb.x & 0xffffu), bf16_bits_to_float(vb.x >> 16),
                          bf16_bits_to_float(vb.y & 0xffffu), bf16_bits_to_float(vb.y >> 16));
    }
  }

  float M = s_cur;
  for (int s0 = 0; s0 < n; s0 += 64) M = fmaxf(M, s0 + lane < n ? lp[s0 + lane] : -INFINITY);
  M = wave_max(M);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float total = 0.0f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < n; s0 += 64) {
      const float wl = s0 + lane < n ? __expf(lp[s0 + lane] - M) : 0.0f;
      total += wl;
      const int cnt = min(64, n - s0);
      for (int s = 0; s < cnt; s += 8) {
        float4 v[U];
        float wt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = s + NG * u + grp;   // split s0 + j of this lane group
          wt[u] = __shfl(wl, j & 63);
          v[u] = j < cnt ? *reinterpret_cast<const float4*>(op + int64_t(s0 + j) * D) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float w = s + NG * u + grp < cnt ? wt[u] : 0.0f;
          acc.x = fmaf(w, v[u].x, acc.x); acc.y = fmaf(w, v[u].y, acc.y);
          acc.z = fmaf(w, v[u].z, acc.z); acc.w = fmaf(w, v[u].w, acc.w);
        }
      }
    }
    total = wave_sum(total);
    if (cur) {
      const float wc = __expf(s_cur - M);
      total += wc;
      if (grp == 0) {
        acc.x = fmaf(wc, v_cur.x, acc.x); acc.y = fmaf(wc, v_cur.y, acc.y);
        acc.z = fmaf(wc, v_cur.z, acc.z); acc.w = fmaf(wc, v_cur.w, acc.w);
      }
    }
  }
  // the lane groups hold disjoint splits of the same four d: add them
#pragma unroll
  for (int m = LPR; m < 64; m *= 2) {
    acc.x += __shfl_xor(acc.x, m); acc.y += __shfl_xor(acc.y, m);
    acc.z += __shfl_xor(acc.z, m); acc.w += __shfl_xor(acc.w, m);
  }
  if (grp == 0) {
    const float inv = total > 0.0f ? 1.0f / total : 0.0f;
    *reinterpret_cast<float4*>(a.o + row * D + col) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (col == 0) a.lse[row] = total > 0.0f ? M + __logf(total) : -INFINITY;
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int D_, int block_size, int max_blocks) {
  const int64_t max_tokens = int64_t(max_blocks) * block_size;
  const int64_t splits = decode_grid_splits(max_tokens);
  const int64_t rows = int64_t(B) * Hq * (splits > 0 ? splits : 1);
  return size_t(rows) * (size_t(D_) + 1) * sizeof(float);
}

namespace {

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  if (a.max_splits > 0) {
    hipLaunchKernelGGL(dcp_decode_split_kernel<D>, dim3(a.max_splits, a.Hkv, a.B), dim3(NT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = int64_t(a.B) * a.Hq;
  hipLaunchKernelGGL(dcp_decode_combine_kernel<D>, dim3(unsigned((rows + COMBINE_WAVES - 1) / COMBINE_WAVES)),
                     dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dcp_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  return a.D == 64 ? launch_decode_d<64>(a, s) : launch_decode_d<128>(a, s);
}

}  // namespace ctxattn
