// bf16 MFMA attention step kernels for gfx950: one query block against one K/V chunk.
//
// Online-max mode: flash-style running row max / row sum / rescaled accumulator,
// emitting the chunk's normalised partial and per-row LSE, or merging it by the LSE rule
// into a prior partial held in the outputs ("Kernel reference: ring_attention_const_max_fwd",
// Design: the online-max path and its running max; sharding page, ring attention).
// Const-max mode: p = exp(s - c_i) with the fixed per-row bound and a pure-addition
// fold into an fp32 accumulator, normalised once with the 1e-37 clamp (same page,
// Design "A static bound makes the ring reduction pure addition", Implementation
// "Accumulate, then normalize once").
//
// Work layout (gfx950, wave64, one workgroup of eight waves per CU, two waves per SIMD):
//  * a workgroup owns 256 query rows of one (batch, head); each wave owns 32 rows and
//    keeps Q, the output accumulator and the scores in VGPRs;
//  * keys stream through LDS in tiles of 32 held in a ring of NBUF buffers, copied from
//    HBM straight into LDS (global_load_lds_dwordx4: no staging registers, one scalar
//    base per tile plus a fixed per-lane offset), NBUF - 1 tiles ahead of use;
//  * ping-pong: on a SIMD, one wave's matrix phase (the output update of tile j, V^T P^T,
//    and the scores of tile j+1, K Q^T: 16 MFMAs, with the K and V fragment reads of tile
//    j+1 spread between them) runs while the other wave does the softmax of tile j on the
//    VALU, with no LDS reads. Two waves give the MFMA/VALU overlap whatever order the
//    compiler gives each wave's instructions (one wave overlaps its own only where its
//    stream interleaves them). The phases are held in step by one workgroup barrier per
//    phase, waves 4..7 starting one phase behind waves 0..3;
//  * LDS rows are dense (256 B) with XOR-swizzled 16-byte chunks so that both read
//    patterns are bank-conflict free: K chunk c of row r sits at c ^ (r & 15), V chunk
//    c at c ^ (4(r & 3) + 2((r >> 1) & 1));
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so each
//    lane holds 16 scores of one query row: a row max or sum needs one exchange between
//    lanes l and l^32 (v_permlane32_swap) and nothing else;
//  * O^T = V^T P^T takes P straight from the score registers (B operand); V stays in
//    natural [key][d] order in LDS and ds_read_b64_tr_b16 transposes it on the read
//    (within 16 lanes, lane i element t <- lane i/4 + 4t's element i%4), fetching the
//    keys in exactly the order the score registers hold them;
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score. The online mode
//    keeps a lazy reference max: a tile is exponentiated against the reference as it
//    stands, and only when a lane's share of the tile's row sum comes out above 2^20 (or
//    while some row of the wave has no reference yet) does the wave find the tile's row
//    maxima, raise the reference, rescale its accumulators and redo the tile. A full tile
//    thus runs no max reduction at all, and probabilities stay <= 2^20;
//  * causal masks: a workgroup visits key tiles up to its last row's diagonal; a wave skips
//    the softmax and the matrix phase of the tiles past its own last row's diagonal (every
//    probability there is 0), still copying its share of them and meeting every barrier.
//
// Key-split schedule (when the caller passes a workspace and one workgroup per query tile
// would leave over a tenth of the device's workgroup slots idle, e.g. 160 tiles on 256
// CUs): the (query tile, key tile) iterations of the whole call are laid end to end and
// cut into G ranges of equal cost, G = the number of workgroups the device holds at once
// (or fewer for small calls), so every workgroup does the same work and the grid fills the
// machine. The cost of a range is its iterations plus a fixed charge for each query tile
// that starts inside it (a segment's Q load, copy prologue and partial or final store).
// A query tile whose keys fall into several ranges is computed in segments; each segment
// leaves its unnormalised partial (rows' output, running max and row sum) in the workspace
// and bumps the tile's counter, and the workgroup that brings the counter to the segment
// count combines the segments in key order and writes the result. No workgroup ever waits
// for another. The combiner resets the counter, so a workspace is ready for the next call.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int D = 128;         // head dim of the bf16 path
constexpr int NW = 8;          // waves per workgroup: two per SIMD
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int BQ = 32 * NW;    // query rows per workgroup (32 per wave)
constexpr int BK = 32;         // keys per LDS tile
constexpr int NBUF = 6;        // LDS tile buffers (copies run NBUF - 1 tiles ahead)
constexpr int ROW = D;                    // bf16 per LDS row (dense, swizzled)
constexpr int TILE = BK * ROW;            // bf16 per tile and tensor (8 KB)
constexpr int TILE_BYTES = TILE * 2;
constexpr int V_OFF = NBUF * TILE_BYTES;  // byte offset of the V buffers
constexpr size_t LDS_BYTES = size_t(NBUF) * 2 * TILE_BYTES;
// Lane tile sums above this (as fp32 bits: 2^20; inf is above it too) move the reference max.
constexpr uint32_t kSumCapBits = 0x49800000u;
static_assert(BK * D / 8 == NT, "one 16-byte copy per lane per tile and tensor");

enum { MODE_ONLINE = 0, MODE_CONSTMAX = 1 };

typedef short short4v __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int k_swz(int r) { return r & 15; }
__host__ __device__ constexpr int v_swz(int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); }

// Makes the compiler wait for a value's load here (an empty asm that reads it), so no wait
// for it is left inside the tile loop, where it would also wait for in-flight tile copies.
template <typename T>
__device__ __forceinline__ void settle(const T& x) { asm volatile("" :: "v"(x)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((__attribute__((address_space(3))) const char*)(p)));
}

// One 16-byte-per-lane copy HBM -> LDS: lane l reads base + off and its 16 bytes land at LDS
// byte m0 + 16*l. Inline asm, so that the compiler neither waits for it before unrelated LDS
// reads nor before barriers: the kernel places every wait for these copies itself. The LDS
// address is an input bound to m0 ("{m0}"), so the compiler writes m0 itself and knows the
// register's value across the statement; the s_nop is the wait state an LDS-DMA load needs
// after an SALU write of m0, which the compiler cannot see inside the asm.
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t off, uint32_t lds_byte) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "{m0}"(lds_byte), "v"(off), "s"(base) : "memory");
}

// End of a vector phase (which issues no LDS reads): at most 2*PENDING of this wave's tile
// copies are still in flight (two per tile: K and V), then the workgroup barrier. The
// scheduling barriers keep the compiler from moving any instruction across the boundary.
template <int PENDING>
__device__ __forceinline__ void phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(2 * PENDING) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}


// End of a matrix phase: this wave's LDS reads have returned (the buffers they read may be
// refilled two phases later), then the workgroup barrier.
__device__ __forceinline__ void reads_end_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Plain workgroup barrier between phases (no wait for copies).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte store at device (agent) scope: written through to the coherence point that every
// XCD's agent-scope loads read (the form the compiler gives a relaxed agent-scope atomic
// store, as inline asm so that it does not pin the surrounding schedule).
__device__ __forceinline__ void store_agent4(float* p, floatx4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}

// Exchange with lane l ^ 32 (v_permlane32_swap): returns max / sum of the pair.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int IMM>
__device__ __forceinline__ bf16x8 lds_read16(const uint16_t* lds0, int off_el) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(lds0) + IMM + 2 * off_el);
}

template <int IMM>
__device__ __forceinline__ bf16x8 lds_read_tr(const uint16_t* lds0, int off_el) {
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  const char* p = reinterpret_cast<const char*>(lds0) + 2 * off_el;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p + IMM));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p + IMM + 8 * ROW * 2));
  const short4v both[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8*>(both);
}

// Softmax numerators of the 16 scores a lane holds: p = exp2(s*sl2e - mu), packed to bf16 in
// P.V operand order (kc = 0: registers 0..7, kc = 1: registers 8..15); returns the lane's
// share of the tile's row sum. The sum adds the fp32 values: summing the bf16-rounded ones
// instead would leave an LSE error up to 2^-9 on rows that see only one or two keys.
__device__ __forceinline__ float exp_pack(const floatx16& s, float sl2e, float mu, bf16x8 (&pb)[2]) {
  float pair[8];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = kc * 8 + 2 * t;
      const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2e, -mu));
      const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], sl2e, -mu));
      w[t] = pack_bf16x2(x0, x1);
      pair[kc * 4 + t] = x0 + x1;
    }
    uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
    pb[kc] = *reinterpret_cast<bf16x8*>(&u);
  }
  return ((pair[0] + pair[1]) + (pair[2] + pair[3])) + ((pair[4] + pair[5]) + (pair[6] + pair[7]));
}

// Raises each row's online reference max to the tile's row max where that is larger and
// rescales the row's accumulators to the new reference.
__device__ __forceinline__ void online_rebase(const floatx16& s, float sl2e, float& m_ref, float& l_part,
                                              floatx16 (&o)[4]) {
  // a three-level tree of 3-input maxima (v_max3_f32; this file builds without NaN
  // semantics, so no canonicalising moves precede them)
  const float a0 = fmaxf(fmaxf(s[0], s[1]), s[2]), a1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float a2 = fmaxf(fmaxf(s[6], s[7]), s[8]), a3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float a4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
  float tmax = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), s[15]));
  tmax = xor32_max(tmax);
  const float m_new = fmaxf(m_ref, tmax * sl2e);
  const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_ref - m_new);   // -inf -> finite: 0
  l_part *= alpha;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  m_ref = m_new;
}

// Keys a query row may see: every key j < row_key_limit(row) of the chunk (and j < Sk).
template <int MASK>
__host__ __device__ inline int row_key_limit(const AttnArgs& a, int row) {
  if (MASK == CA_MASK_CAUSAL_INCL) return row + 1;
  if (MASK == CA_MASK_CAUSAL_STRICT) return row;
  if (MASK == kMaskDcp) {
    const int n = row + 1, round = a.dcp_I * a.dcp_W;
    return (n / round) * a.dcp_I + min(max(n - (n / round) * round - a.dcp_R * a.dcp_I, 0), a.dcp_I);
  }
  return a.Sk;
}

// Leaves out the sink keys of this tile: bit l of m marks lane l's sink (a chunk-local key
// index held in `sink`) as falling in [key0, key0 + BK).
__device__ __forceinline__ void mask_sinks(floatx16& s, int key0, int hl, uint64_t m, int sink) {
  while (m) {
    const int l = __builtin_ctzll(m);
    m &= m - 1;
    const int j_sink = __builtin_amdgcn_readlane(sink, l);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      s[r] = j == j_sink ? -INFINITY : s[r];
    }
  }
}

__device__ __forceinline__ void apply_mask(floatx16& s, int key0, int hl, int lim) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
    s[r] = j < lim ? s[r] : -INFINITY;
  }
}

// Final output of one lane's half row: o (unnormalised), the full row sum lrow, the running
// max m_ref (online) or the bound c2 (const-max), both in log2 units.
template <int MODE>
__device__ __forceinline__ void store_rows(const AttnArgs& a, int64_t bh, int Sq, int row, int hl,
                                           floatx16 (&o)[4], float lrow, float m_ref, float c2) {
  if (row >= Sq) return;
  const int64_t rowidx = bh * Sq + row;
  // o[db][r] is O[row][d] for d = 32*db + 8*(r/4) + 4*hl + r%4: four consecutive d per float4.
  if (MODE == MODE_ONLINE) {
    const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
    const float lse_t = lrow > 0.0f ? (m_ref + __log2f(lrow)) * kLn2 : -INFINITY;
    float* orow = a.o + rowidx * D;
    if (a.fold) {
      // merge with the prior partial in o / lse (both lanes of the row read it before either
      // writes: they are lanes l and l + 32 of one wave)
      float w_p, w_t;
      const float L = lse_fold_weights(a.lse[rowidx], lse_t, w_p, w_t);
      const float wt = w_t * inv;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4* dst = reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl);
          const float4 pr = *dst;
          *dst = make_float4(w_p * pr.x + wt * o[db][4 * g], w_p * pr.y + wt * o[db][4 * g + 1],
                             w_p * pr.z + wt * o[db][4 * g + 2], w_p * pr.w + wt * o[db][4 * g + 3]);
        }
      if (hl == 0) a.lse[rowidx] = L;
      return;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
    if (hl == 0) a.lse[rowidx] = lse_t;
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
          o[db][4 * g] += p4.x; o[db][4 * g + 1] += p4.y;
          o[db][4 * g + 2] += p4.z; o[db][4 * g + 3] += p4.w;
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
              make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
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
            u.x = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
            u.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
            *reinterpret_cast<uint2*>(orow + db * 32 + 8 * g + 4 * hl) = u;
          }
      } else {
        float* orow = static_cast<float*>(a.o_cm) + rowidx * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl) =
                make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                            o[db][4 * g + 3] * inv);
      }
      if (hl == 0 && a.lse_cm) a.lse_cm[rowidx] = c2 * kLn2 + __logf(z);
    }
  }
}

// Key tiles that query tile qb iterates over: every tile of the chunk, or under a causal
// mask every tile up to the diagonal block (keys below (qb + 1) * BQ).
__host__ __device__ inline int tile_iters(int mask, int qb, int nkt) {
  if (mask == CA_MASK_NONE) return nkt;
  return min(nkt, (BQ / BK) * (qb + 1));
}

// As tile_iters, for any mask: the tiles holding the keys the tile's last row may see.
template <int MASK>
__host__ __device__ inline int tile_iters_of(const AttnArgs& a, int qb, int nkt) {
  if (MASK != kMaskDcp) return tile_iters(MASK, qb, nkt);
  const int lim = row_key_limit<MASK>(a, min(qb * BQ + BQ, a.Sq) - 1);
  return min(nkt, (lim + BK - 1) / BK);
}

// Iterations of query tiles [0, qb) of one (batch, head). Causal: the first nkt / (BQ/BK)
// tiles grow by BQ/BK key tiles each, the rest see the whole chunk.
__host__ __device__ inline int64_t tiles_prefix(int mask, int qb, int nkt) {
  if (mask == CA_MASK_NONE) return int64_t(qb) * nkt;
  constexpr int R = BQ / BK;
  const int64_t m = min(qb, nkt / R);
  return R * m * (m + 1) / 2 + int64_t(nkt) * (qb - m);
}

// Key-split schedule and its workspace (see the file comment).
struct Split {
  int* cnt;        // [B*H*nqb][NW] arrivals per (query tile, wave); zero between calls
  float* po;       // [2G][NW][16 quads][64 lanes][4] unnormalised partial outputs, one record per
                   // segment and wave, lane-interleaved so every 16-byte store is one contiguous 1 KB
  float* pml;      // [2G][NW][2][64 lanes] partial running max (log2 units) and full row sum
  int G;           // logical workgroups
  int C;           // cost of a query tile's start, in iterations (see range_begin)
  int64_t V;       // weighted length of the call: T iterations + C per query tile
  int64_t per_bh;  // iterations of one (batch, head)
};

// The ranges are cut by weight, not by iteration count: every query tile is followed by C
// units of weight that belong to no iteration, standing for the cost of a segment boundary
// (publishing or combining a partial, a second Q load and copy prologue). A range that holds
// a tile boundary thus gets about C fewer iterations than one inside a single tile, and the
// workgroups finish together. Iteration x of global query tile g sits at weight x + C*g;
// the cuts are at V*w/G.
__device__ __forceinline__ int64_t weight_of(const Split& sp, int64_t x, int g) { return x + int64_t(sp.C) * g; }

// First iteration of workgroup w's range: the first iteration whose weight reaches V*w/G
// (a cut inside a tile's trailing C units moves to the next tile's start).
template <int MASK>
__device__ __forceinline__ int64_t range_begin(const Split& sp, int nqb, int nkt, int w) {
  const int64_t P = sp.V * w / sp.G;
  const int64_t bh_w = sp.per_bh + int64_t(sp.C) * nqb;   // weight of one (batch, head)
  const int64_t bh = P / bh_w;
  const int64_t r = P - bh * bh_w;
  int qb;
  if (MASK == CA_MASK_NONE) {
    qb = int(r / (nkt + sp.C));
  } else {
    int lo = 0, hi = nqb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tiles_prefix(MASK, mid, nkt) + int64_t(sp.C) * mid <= r) lo = mid; else hi = mid - 1;
    }
    qb = lo;
  }
  const int64_t t0 = tiles_prefix(MASK, qb, nkt);
  const int64_t off = r - t0 - int64_t(sp.C) * qb;
  const int len = tile_iters(MASK, qb, nkt);
  return bh * sp.per_bh + (off < len ? t0 + off : tiles_prefix(MASK, qb + 1, nkt));
}
// The workgroup whose range holds iteration x of global query tile g: the largest w whose
// cut weight V*w/G is at most x's weight.
__device__ __forceinline__ int range_owner(const Split& sp, int64_t x, int g) {
  return int((int64_t(sp.G) * (weight_of(sp, x, g) + 1) + sp.V - 1) / sp.V) - 1;
}
// Record of workgroup w's segment of the tile starting at iteration tile_start: its first
// segment (slot 2w) unless the tile began before w's range (then its last, 2w + 1).
template <int MASK>
__device__ __forceinline__ int64_t segment_slot(const Split& sp, int nqb, int nkt, int w, int64_t tile_start) {
  return 2 * int64_t(w) + (range_begin<MASK>(sp, nqb, nkt, w) >= tile_start ? 0 : 1);
}

// The ring hop of a launch that carries one: workgroup cw of a.hop_wgs copies its grid-stride
// share of K then V, 16 bytes a lane, HOP_UNROLL vectors in flight per lane. The hop's
// workgroups come last in the grid, so they take the CUs the step's workgroups leave free.
// A launch over two chunks carries two hops: the same workgroups copy the second after the first.
constexpr int HOP_UNROLL = 16;
__device__ __forceinline__ void hop_copy_one(const void* sk_, const void* sv_, void* dk_, void* dv_, int64_t units,
                                             int hop_wgs, int cw) {
  const floatx4* sk = static_cast<const floatx4*>(sk_);
  const floatx4* sv = static_cast<const floatx4*>(sv_);
  floatx4* dk = static_cast<floatx4*>(dk_);
  floatx4* dv = static_cast<floatx4*>(dv_);
  const int64_t total = 2 * units;
  const int64_t stride = int64_t(hop_wgs) * NT * HOP_UNROLL;
  for (int64_t base = int64_t(cw) * NT * HOP_UNROLL + threadIdx.x; base < total; base += stride) {
    floatx4 x[HOP_UNROLL];
#pragma unroll
    for (int u = 0; u < HOP_UNROLL; ++u) {
      const int64_t i = base + int64_t(u) * NT;
      if (i < total) x[u] = __builtin_nontemporal_load(i < units ? sk + i : sv + (i - units));
    }
#pragma unroll
    for (int u = 0; u < HOP_UNROLL; ++u) {
      const int64_t i = base + int64_t(u) * NT;
      if (i < total) __builtin_nontemporal_store(x[u], i < units ? dk + i : dv + (i - units));
    }
  }
}
template <bool PAIR>
__device__ __forceinline__ void hop_copy(const AttnArgs& a, int cw) {
  hop_copy_one(a.hop_sk, a.hop_sv, a.hop_dk, a.hop_dv, a.hop_units, a.hop_wgs, cw);
  if (PAIR && a.hop_units2 > 0) hop_copy_one(a.hop_sk2, a.hop_sv2, a.hop_dk2, a.hop_dv2, a.hop_units2, a.hop_wgs, cw);
}

// The step kernel's body. PAIR: a launch over two chunks (ring_attn_step_pair), whose key
// tiles from a.Sk1 on are read from the second chunk; the other instances compile without it.
template <int MODE, int MASK, bool SPLIT, bool PAIR>
__device__ __forceinline__ void step_body(const AttnArgs& a, int nqb, int nkt, int nwork, const Split& sp) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  if (a.hop_wgs > 0 && int(blockIdx.x) >= int(gridDim.x) - a.hop_wgs) {
    hop_copy<PAIR>(a, int(blockIdx.x) - (int(gridDim.x) - a.hop_wgs));
    return;
  }
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x - a.hop_wgs, nwork);
  if (logical < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const bool lagging = w >= NW / 2;   // waves 4..7 run one phase behind waves 0..3
  const int li = lane & 31;
  const int hl = lane >> 5;
  const int Sq = a.Sq, Sk = a.Sk;
  const int64_t kss_bytes = a.kss * 2;
  const float sl2e = a.sl2e;

  // Per-lane copy offset (bytes from the tile's first key): wave w fills LDS rows
  // 4w + lane/16 at physical chunk lane%16, i.e. reads that row's logical chunk
  // (lane%16) ^ swizzle(row).
  const int crow = 4 * w + (lane >> 4);
  const int cchunk = lane & 15;
  const uint32_t koff = uint32_t(crow * kss_bytes) + uint32_t((cchunk ^ k_swz(crow)) << 4);
  const uint32_t voff = uint32_t(crow * kss_bytes) + uint32_t((cchunk ^ v_swz(crow)) << 4);
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds_addr(lds) + w * 1024);

  // Per-lane LDS read offsets (elements; buffer offsets are added as immediates).
  // K: row li, logical chunk 2c+hl.
  int kr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) kr[c] = li * ROW + (((2 * c + hl) ^ k_swz(li)) << 3);
  // V (transposed reads): lane i16 of 16-lane group G reads row 4*hl + t (t = i16/4; +16 kc
  // and +8 for the second half are immediates), logical element 32*db + 16*(G&1) + 4*(i16&3),
  // i.e. chunk 4*db + 2*(G&1) + (i16&3)/2, physically at chunk ^ v_swz(t) =
  // 4*(db ^ t) + ((2*(G&1) + (i16&3)/2) ^ 2*(t>>1)).
  int vr[4];
  {
    const int i16 = lane & 15;
    const int t = i16 >> 2;
    const int clow = (2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1)) ^ (2 * (t >> 1));
    const int base = (4 * hl + t) * ROW + (clow << 3) + 4 * (i16 & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) vr[db] = base + 32 * (db ^ t);
  }

  int64_t it = 0, it_end = 1;
  if (SPLIT) {
    it = range_begin<MASK>(sp, nqb, nkt, logical);
    it_end = range_begin<MASK>(sp, nqb, nkt, logical + 1);
  }
  // Tiles this wave combines once its own range is done (at most its first and last
  // segment's tiles): tile index bh * nqb + qb and the tile's first iteration.
  int ncomb = 0;
  int comb_tile[2] = {0, 0};
  int64_t comb_start[2] = {0, 0};
  while (it < it_end) {
    // ---- which query tile, and which of its key tiles, this segment covers
    int bh, qb, k0, k1;
    int64_t tile_start = 0;
    if (SPLIT) {
      bh = int(it / sp.per_bh);
      const int64_t r = it - int64_t(bh) * sp.per_bh;
      if (MASK == CA_MASK_NONE) {
        qb = int(r / nkt);
      } else {
        int lo = 0, hi = nqb - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (tiles_prefix(MASK, mid, nkt) <= r) lo = mid; else hi = mid - 1;
        }
        qb = lo;
      }
      tile_start = int64_t(bh) * sp.per_bh + tiles_prefix(MASK, qb, nkt);
      const int64_t seg_end = min(it_end, tile_start + tile_iters(MASK, qb, nkt));
      k0 = int(it - tile_start);
      k1 = int(seg_end - tile_start);
      it = seg_end;
    } else {
      bh = logical / nqb;
      qb = logical - bh * nqb;
      if (MASK != CA_MASK_NONE) qb = nqb - 1 - qb;   // heavy (late) query blocks first
      k0 = 0;
      k1 = tile_iters_of<MASK>(a, qb, nkt);
      it = it_end;
    }

    const int b = bh / a.H;
    const int h = bh - b * a.H;
    const int row_w0 = qb * BQ + w * 32;   // first query row of this wave
    const int row = row_w0 + li;           // this lane's query row

    // Q fragment: row, d = c*16 + 8*hl .. +7 (B operand of S^T = K Q^T). Rows past Sq re-read
    // the last row; their outputs are never stored.
    bf16x8 q[8];
    {
      const uint16_t* qr = static_cast<const uint16_t*>(a.q) + b * a.qsb + h * a.qsh + hl * 8 +
                           int64_t(min(row, Sq - 1)) * a.qss;
#pragma unroll
      for (int c = 0; c < 8; ++c) q[c] = *reinterpret_cast<const bf16x8*>(qr + c * 16);
#pragma unroll
      for (int c = 0; c < 8; ++c) settle(q[c]);
    }

    const int hk = h / a.G;                // K/V head of this query head
    const char* kbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k) + b * a.ksb + hk * a.ksh);
    const char* vbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v) + b * a.ksb + hk * a.ksh);
    // a launch over two chunks: key tiles from key sk1 on come from the second chunk
    const int sk1 = PAIR ? a.Sk1 : INT_MAX;
    const char* kbase2 =
        PAIR ? reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k2) + b * a.ksb + hk * a.ksh) : kbase;
    const char* vbase2 =
        PAIR ? reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v2) + b * a.ksb + hk * a.ksh) : vbase;
    // keys of this (batch, head): the whole chunk, or its own count
    const int Skb = a.sk_of_bh ? min(Sk, max(a.sk_of_bh[bh], 0)) : Sk;
    if (!SPLIT) k1 = min(k1, (Skb + BK - 1) / BK);
    // keys this lane's row may see, and the fewest any row of this wave may see (wave-uniform:
    // held in a scalar register, so the per-tile mask test is a scalar compare and branch)
    const int lane_lim = min(Skb, row_key_limit<MASK>(a, row));
    const int wave_lim = __builtin_amdgcn_readfirstlane(min(Skb, row_key_limit<MASK>(a, row_w0)));
    // keys the wave's last row may see: a key tile at or past it is masked for every row of the wave
    const int wave_hi = __builtin_amdgcn_readfirstlane(min(Skb, row_key_limit<MASK>(a, row_w0 + 31)));
    const int nk = max(k1 - k0, 0);   // key tiles of this segment
    // sink keys to leave out: lane l holds this head's l-th sink as a chunk-local index
    int my_sink = INT_MIN;
    bool has_sinks = false;
    if (a.sink_idx != nullptr) {
      const int cnt = min(a.sink_cnt[bh], a.sink_cap);
      has_sinks = __builtin_amdgcn_readfirstlane(cnt) > 0;
      if (lane < cnt) my_sink = int(a.sink_idx[int64_t(bh) * a.sink_cap + lane] - a.key_offset);
      settle(my_sink);
    }

    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

    float m_ref = -INFINITY;   // reference max (log2 units), online mode
    bool fresh = true;         // some row of this wave has no reference max yet (wave-uniform)
    float l_part = 0.0f;       // this lane's share of the row sum
    float c2 = 0.0f;           // const-max bound in log2 units
    if (MODE == MODE_CONSTMAX) {
      c2 = a.c[int64_t(bh) * Sq + min(row, Sq - 1)] * kLog2e;
      settle(c2);
    }

    // Issues the copies of the segment's key tile j into the LDS buffer at byte dst (K, then V
    // at dst + V_OFF). The last tile of a chunk clamps its rows to the last key (their scores
    // are masked, their values meet p = 0).
    auto issue_to = [&](uint32_t dst, int j) {
      const int key0 = (k0 + j) * BK;
      const char* kt = kbase + key0 * kss_bytes;
      const char* vt = vbase + key0 * kss_bytes;
      if (PAIR && key0 >= sk1) {   // wave-uniform
        kt = kbase2 + (int64_t(key0) - sk1) * kss_bytes;
        vt = vbase2 + (int64_t(key0) - sk1) * kss_bytes;
      }
      uint32_t ko = koff, vo = voff;
      if (__builtin_expect(key0 + BK > Skb, 0)) {   // the chunk's last tile only
        const int rr = max(0, min(crow, Skb - 1 - key0));
        ko = uint32_t(rr * kss_bytes) + uint32_t((cchunk ^ k_swz(crow)) << 4);
        vo = uint32_t(rr * kss_bytes) + uint32_t((cchunk ^ v_swz(crow)) << 4);
      }
      copy16_to_lds(kt, ko, dst);
      copy16_to_lds(vt, vo, dst + V_OFF);
    };
    auto issue = [&](auto bufc, int j) { issue_to(lds_w + decltype(bufc)::value * TILE_BYTES, j); };

    bf16x8 ka[8];    // K fragments of the tile whose scores the next matrix phase forms
    bf16x8 va[8];    // V fragments of the tile whose output update the next matrix phase does
    floatx16 s;      // scores of the tile in flight
    bf16x8 p[2];     // probabilities of the tile whose output update is next
    auto read_k = [&](auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
#pragma unroll
      for (int c = 0; c < 8; ++c) ka[c] = lds_read16<BUF * TILE_BYTES>(lds, kr[c]);
    };
    auto read_v = [&](auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        va[db * 2] = lds_read_tr<V_OFF + BUF * TILE_BYTES>(lds, vr[db]);
        va[db * 2 + 1] = lds_read_tr<V_OFF + BUF * TILE_BYTES + 16 * ROW * 2>(lds, vr[db]);
      }
    };
    // Matrix phase: the output update with the V fragments and probabilities of the last
    // vector phase (PV), then the scores of the next tile (QK). The LDS reads are spread
    // between the MFMAs, one K fragment read after each PV MFMA and two V fragment reads
    // after each QK MFMA: issued in bursts they fill the CU's LDS command queue, and a wave
    // waiting to issue a read cannot issue its next MFMA either.
    auto matrix_phase = [&](auto bufc, bool do_qk, bool do_pv) {
      if (do_qk) read_k(bufc);
      if (do_pv) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          o[c & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[(c & 3) * 2 + (c >> 2)], p[c >> 2], o[c & 3], 0, 0, 0);
      }
      if (do_qk) read_v(bufc);   // the next tile's V: its registers are free once P.V has issued
      if (do_qk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], q[0], floatx16{}, 0, 0, 0);
#pragma unroll
        for (int c = 1; c < 8; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], q[c], s, 0, 0, 0);
      }
      if (do_pv) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {   // P.V MFMA, K fragment read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {   // Q.K MFMA, two V fragment reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      } else {                          // prologue: K reads, Q.K, V reads
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      }
    };
    // Softmax of the segment's tile j (scores in s): probabilities into p, row sum into l_part.
    // The rare paths (masks, sinks, a moving maximum, the chunk's last tile in `issue`) are
    // marked unlikely, so a full tile runs its vector phase without a taken branch: a taken
    // branch costs the wave an instruction refetch, on the phase that sets the pace (8% of the
    // cycles of a causal step).
    auto softmax = [&](int j) {
      const int key0 = (k0 + j) * BK;
      if (__builtin_expect(key0 + BK > wave_lim, 0)) apply_mask(s, key0, hl, lane_lim);
      if (__builtin_expect(has_sinks, 0)) {
        const uint64_t m = __ballot(my_sink >= key0 && my_sink < key0 + BK);
        if (m) mask_sinks(s, key0, hl, m, my_sink);
      }
      if (MODE == MODE_ONLINE) {
        float t = 0.0f;
        bool redo = fresh;
        if (__builtin_expect(!fresh, 1)) {
          t = exp_pack(s, sl2e, m_ref, p);
          redo = __any(__float_as_uint(t) > kSumCapBits);   // t >= 0, or +inf
        }
        if (__builtin_expect(redo, 0)) {   // the first tiles; a max up by ~20 in log2 units
          online_rebase(s, sl2e, m_ref, l_part, o);
          fresh = __any(m_ref == -INFINITY);
          t = exp_pack(s, sl2e, m_ref == -INFINITY ? 0.0f : m_ref, p);
        }
        l_part += t;
      } else {
        l_part += exp_pack(s, sl2e, c2, p);
      }
    };
    // One tile j of the segment (buffer BUF = j % NBUF), in two phases.
    //  vector phase: start the copies of tile j + NBUF - 1 into the buffer tile j - 1 used,
    //    softmax of tile j; ends once this wave's copies of tile j + 2 have landed, then the
    //    workgroup barrier;
    //  matrix phase: read K of tile j + 1, output update of tile j, read V of tile j + 1,
    //    scores of tile j + 1; ends once its LDS reads have returned, then the barrier.
    //  All LDS reads of a SIMD pair thus come from the wave in its matrix phase, under its
    //  MFMAs, and none from the wave running the softmax.
    // The body is the same for every tile: past the segment's last tile the copies repeat
    // that tile into free buffers and the scores of the nonexistent tile are never used,
    // so the copy count in flight, the waits and the MFMA sequence never change.
    auto tile = [&](auto bufc, int j) {
      constexpr int BUF = decltype(bufc)::value;
      constexpr int NEXT = (BUF + 1) % NBUF;
      constexpr int FREE = (BUF + NBUF - 1) % NBUF;
      issue(std::integral_constant<int, FREE>{}, min(j + NBUF - 1, nk - 1));
      softmax(j);
      phase_end<NBUF - 3>();
      matrix_phase(std::integral_constant<int, NEXT>{}, true, true);
      reads_end_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    static_assert(NBUF == 6, "the tile loop is unrolled for six buffers");

    if (nk > 0) {
      // prologue: tiles 0 .. NBUF-2 in flight, wait for tiles 0 and 1, scores of tile 0
      issue(I0{}, 0);
      issue(I1{}, min(1, nk - 1));
      issue(I2{}, min(2, nk - 1));
      issue(I3{}, min(3, nk - 1));
      issue(I4{}, min(4, nk - 1));
      phase_end<NBUF - 3>();
      if (lagging) phase_barrier();
      matrix_phase(I0{}, true, false);   // scores and V fragments of tile 0
      reads_end_barrier();
      // tiles from the first one masked for every row of this wave on (causal: past its last
      // row's diagonal) carry no probability: the wave only copies its share of them and meets
      // the barriers
      const int n_live = MASK == CA_MASK_NONE ? nk : min(nk, max(1, (wave_hi - k0 * BK + BK - 1) / BK));
      for (int j = 0;; j += NBUF) {
        tile(I0{}, j);
        if (j + 1 >= n_live) break;
        tile(I1{}, j + 1);
        if (j + 2 >= n_live) break;
        tile(I2{}, j + 2);
        if (j + 3 >= n_live) break;
        tile(I3{}, j + 3);
        if (j + 4 >= n_live) break;
        tile(I4{}, j + 4);
        if (j + 5 >= n_live) break;
        tile(I5{}, j + 5);
        if (j + 6 >= n_live) break;
      }
      for (int j = n_live; j < nk; ++j) {
        issue_to(lds_w + uint32_t((j + NBUF - 1) % NBUF) * TILE_BYTES, min(j + NBUF - 1, nk - 1));
        phase_end<NBUF - 3>();
        reads_end_barrier();
      }
      // every copy has landed and every wave is past its last LDS read before the buffers
      // are reused (next segment) or released
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (!lagging) phase_barrier();
      phase_barrier();
    }

    const float lrow = xor32_sum(l_part);
    if (!SPLIT) {
      store_rows<MODE>(a, bh, Sq, row, hl, o, lrow, m_ref, c2);
      continue;
    }
    const int tile_iters_n = tile_iters(MASK, qb, nkt);
    const int w_first = range_owner(sp, tile_start, bh * nqb + qb);
    const int w_last = range_owner(sp, tile_start + tile_iters_n - 1, bh * nqb + qb);
    if (w_first == w_last) {   // the whole tile lies in this workgroup's range
      store_rows<MODE>(a, bh, Sq, row, hl, o, lrow, m_ref, c2);
      continue;
    }

    // ---- publish this segment's partial, count it; the last arrival combines all of them.
    // Ordering. Every record byte moves through device-coherent accesses: the stores are
    // written through to the device's coherence point (sc1, the form of a relaxed agent-scope
    // atomic store) and the combiner's loads read from it (relaxed agent-scope atomic loads),
    // so no cached copy of a record is ever read. The publisher waits for its stores to
    // complete (vmcnt 0) before its counter increment, and the combiner issues its loads only
    // after its own increment has returned the final count; the counter's increments are
    // agent-scope atomics on one address, so they are totally ordered. Hence every record
    // load follows every record store of the tile. A release/acquire pair would add a
    // write-back and an invalidation of this XCD's whole L2 (buffer_wbl2, buffer_inv), which
    // only data held in that cache needs.
    {
      const int64_t rec = segment_slot<MASK>(sp, nqb, nkt, logical, tile_start) * NW + w;
      float* po = sp.po + rec * (64 * 64) + lane * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store_agent4(po + (db * 4 + g) * 256,
                       floatx4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]});
      __hip_atomic_store(sp.pml + rec * 128 + lane, m_ref, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sp.pml + rec * 128 + 64 + lane, lrow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int* ctr = sp.cnt + (int64_t(bh) * nqb + qb) * NW + w;
    int seen = 0;
    if (lane == 0) seen = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    seen = __shfl(seen, 0);
    if (seen != w_last - w_first) continue;   // another segment is still running
    if (lane == 0) __hip_atomic_exchange(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
    comb_tile[ncomb] = bh * nqb + qb;
    comb_start[ncomb] = tile_start;
    ++ncomb;
  }
  if (!SPLIT) return;
  // Compiler barrier: no record load below may be moved above the counter increments that
  // selected the tiles (the loads are relaxed atomics, which the compiler could otherwise reorder).
  asm volatile("" ::: "memory");

  // ---- combine the segments of the tiles this wave arrived at last, in key order
  // (deterministic sums). Done after the tile loop, so none of the loop's state is live here.
  // The records are read two at a time with every load of both in flight before any is
  // used (each record is 64 registers a lane; two of them and the accumulator fit), so a
  // tile of n segments costs ceil(n / 2) trips to the coherence point. Each pair is weighted
  // by its own maximum and folded into the running one by the LSE rule.
  for (int ci = 0; ci < ncomb; ++ci) {
    const int tix = ci == 0 ? comb_tile[0] : comb_tile[1];
    const int64_t tile_start = ci == 0 ? comb_start[0] : comb_start[1];
    const int bh = tix / nqb;
    const int qb = tix - bh * nqb;
    const int row = qb * BQ + w * 32 + li;
    const int w_first = range_owner(sp, tile_start, tix);
    const int w_last = range_owner(sp, tile_start + tile_iters(MASK, qb, nkt) - 1, tix);
    float c2 = 0.0f;
    if (MODE == MODE_CONSTMAX) c2 = a.c[int64_t(bh) * Sq + min(row, Sq - 1)] * kLog2e;
    float M = -INFINITY;   // running max of the records folded so far (online mode)
    float L = 0.0f;
    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    for (int wb = w_first; wb <= w_last; wb += 2) {
      uint64_t buf[2][32];
      float bm[2], bl[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bm[u] = -INFINITY;
        bl[u] = 0.0f;
        if (wb + u > w_last) continue;
        const int64_t rec = segment_slot<MASK>(sp, nqb, nkt, wb + u, tile_start) * NW + w;
        if (MODE == MODE_ONLINE)
          bm[u] = __hip_atomic_load(sp.pml + rec * 128 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bl[u] = __hip_atomic_load(sp.pml + rec * 128 + 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // 8-byte agent-scope loads, 32 per record and lane
        const uint64_t* po = reinterpret_cast<const uint64_t*>(sp.po + rec * (64 * 64) + lane * 4);
#pragma unroll
        for (int i = 0; i < 32; ++i)
          buf[u][i] = __hip_atomic_load(po + (i / 2) * 128 + (i % 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float wt[2] = {1.0f, 1.0f};
      if (MODE == MODE_ONLINE) {
        const float Mb = fmaxf(M, fmaxf(bm[0], bm[1]));
        const float alpha = M == Mb ? 1.0f : exp2f(M - Mb);   // M = -inf < Mb: alpha = 0
        L *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
        for (int u = 0; u < 2; ++u) wt[u] = bm[u] == -INFINITY ? 0.0f : exp2f(bm[u] - Mb);
        M = Mb;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (wb + u > w_last) continue;
        L += wt[u] * bl[u];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int db = i / 8, r = 2 * (i % 8);
          o[db][r] += wt[u] * __uint_as_float(uint32_t(buf[u][i]));
          o[db][r + 1] += wt[u] * __uint_as_float(uint32_t(buf[u][i] >> 32));
        }
      }
    }
    store_rows<MODE>(a, bh, Sq, row, hl, o, L, M, c2);
  }
}

template <int MODE, int MASK, bool SPLIT>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16(const AttnArgs a, int nqb, int nkt, int nwork, const Split sp) {
  step_body<MODE, MASK, SPLIT, false>(a, nqb, nkt, nwork, sp);
}

// Two chunks in one launch (online, no mask).
template <bool SPLIT>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_pair_bf16(const AttnArgs a, int nqb, int nkt, int nwork, const Split sp) {
  step_body<MODE_ONLINE, CA_MASK_NONE, SPLIT, true>(a, nqb, nkt, nwork, sp);
}

// Workgroups resident at once on the current device (one per CU).
int resident_workgroups() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

constexpr int64_t kMinItersPerWorkgroup = 8;
// Weight of a query tile's start in the key-split cuts, in iterations (range_begin).
constexpr int kTileStartCost = 8;
// Splitting pays where one workgroup per query tile would leave more than this share of the
// device's workgroup slots idle over the call (the last, partly filled round of tiles).
constexpr double kMaxIdleShare = 0.10;

struct Plan {
  int nqb, nkt, G;
  int64_t per_bh, T;
  bool split;      // key-split schedule chosen (needs a workspace)
  size_t cnt_bytes, po_bytes, pml_bytes;
  size_t bytes() const { return split ? cnt_bytes + po_bytes + pml_bytes : 0; }
};

Plan make_plan(int B, int H, int Sq, int Sk, int mask) {
  Plan p{};
  p.nqb = (Sq + BQ - 1) / BQ;
  p.nkt = (Sk + BK - 1) / BK;
  p.per_bh = tiles_prefix(mask, p.nqb, p.nkt);
  p.T = int64_t(B) * H * p.per_bh;
  if (p.T == 0) return p;
  const int64_t slots = resident_workgroups();
  const int64_t tiles = int64_t(B) * H * p.nqb;
  const int64_t rounds = (tiles + slots - 1) / slots;
  p.split = double(rounds * slots - tiles) > kMaxIdleShare * double(rounds * slots);
  if (!p.split) return p;
  int64_t g = std::min<int64_t>(slots, (p.T + kMinItersPerWorkgroup - 1) / kMinItersPerWorkgroup);
  if (mask == CA_MASK_NONE && g == slots) {
    // Equal query tiles: a count that cuts every pair of tiles into the same k ranges,
    // G = tiles * k / 2, puts the cuts at the same places in every pair, so no tile holds
    // more segments than its neighbours (with G = 1.6 tiles, three in five tiles hold three
    // segments; with 1.5, every tile holds two). Taken when it idles under a tenth of the
    // slots.
    for (int64_t k = (2 * slots) / tiles; k >= 2; --k) {
      if ((tiles * k) % 2 != 0) continue;
      const int64_t gk = tiles * k / 2;
      if (gk <= slots && double(gk) >= (1.0 - kMaxIdleShare) * double(slots)) g = gk;
      break;
    }
  }
  p.G = int(std::max<int64_t>(1, g));
  p.cnt_bytes = (size_t(B) * H * p.nqb * NW * sizeof(int) + 255) & ~size_t(255);
  p.po_bytes = size_t(2) * p.G * NW * 64 * 64 * sizeof(float);
  p.pml_bytes = size_t(2) * p.G * NW * 128 * sizeof(float);
  return p;
}

template <int MODE, int MASK, bool SPLIT, bool PAIR>
hipError_t launch_one(const AttnArgs& a, const Plan& p, hipStream_t s) {
  const void* kern = PAIR ? reinterpret_cast<const void*>(&attn_step_pair_bf16<SPLIT>)
                          : reinterpret_cast<const void*>(&attn_step_bf16<MODE, MASK, SPLIT>);
  static bool attr_set = false;   // dynamic LDS above 64 KB must be allowed once
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(LDS_BYTES));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  Split sp{};
  int nwork = a.B * a.H * p.nqb;
  if (SPLIT) {
    char* ws = static_cast<char*>(a.ws);
    sp.cnt = reinterpret_cast<int*>(ws);
    sp.po = reinterpret_cast<float*>(ws + p.cnt_bytes);
    sp.pml = reinterpret_cast<float*>(ws + p.cnt_bytes + p.po_bytes);
    sp.G = p.G;
    sp.C = kTileStartCost;
    sp.V = p.T + int64_t(kTileStartCost) * a.B * a.H * p.nqb;
    sp.per_bh = p.per_bh;
    nwork = p.G;
  }
  if (nwork == 0 && a.hop_wgs == 0) return hipSuccess;
  const int grid = round_up8(nwork) + a.hop_wgs;
  if constexpr (PAIR)
    hipLaunchKernelGGL((attn_step_pair_bf16<SPLIT>), dim3(grid), dim3(NT), LDS_BYTES, s, a, p.nqb, p.nkt, nwork, sp);
  else
    hipLaunchKernelGGL((attn_step_bf16<MODE, MASK, SPLIT>), dim3(grid), dim3(NT), LDS_BYTES, s, a, p.nqb, p.nkt,
                       nwork, sp);
  return hipGetLastError();
}

template <int MODE, int MASK, bool PAIR = false>
hipError_t launch_mode(const AttnArgs& a, hipStream_t s) {
  const Plan p = make_plan(a.B, a.H, a.Sq, a.Sk, MASK);
  if (MASK != kMaskDcp && a.ws != nullptr && p.split) return launch_one<MODE, MASK, true, PAIR>(a, p, s);
  return launch_one<MODE, MASK, false, PAIR>(a, p, s);
}

}  // namespace

size_t attn_bf16_workspace_bytes(int B, int H, int Sq, int Sk, int mask) {
  return make_plan(B, H, Sq, Sk, mask).bytes();
}

int attn_bf16_idle_slots(int B, int H, int Sq, int Sk, int mask, bool with_workspace) {
  const Plan p = make_plan(B, H, Sq, Sk, mask);
  const int64_t slots = resident_workgroups();
  const int64_t nwork = (with_workspace && p.split) ? p.G : int64_t(B) * H * p.nqb;
  if (nwork == 0) return int(slots);
  const int64_t last = nwork - (nwork - 1) / slots * slots;   // work items of the last round
  return int(slots - last);
}

hipError_t launch_attn_bf16(const AttnArgs& a, bool const_max, hipStream_t s) {
  if (a.k2 != nullptr) return launch_mode<MODE_ONLINE, CA_MASK_NONE, true>(a, s);   // two chunks: online, no mask
  if (const_max) return launch_mode<MODE_CONSTMAX, CA_MASK_NONE>(a, s);
  switch (a.mask) {
    case CA_MASK_CAUSAL_INCL: return launch_mode<MODE_ONLINE, CA_MASK_CAUSAL_INCL>(a, s);
    case CA_MASK_CAUSAL_STRICT: return launch_mode<MODE_ONLINE, CA_MASK_CAUSAL_STRICT>(a, s);
    case kMaskDcp: return launch_mode<MODE_ONLINE, kMaskDcp>(a, s);
    default: return launch_mode<MODE_ONLINE, CA_MASK_NONE>(a, s);
  }
}

}  // namespace ctxattn
