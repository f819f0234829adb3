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
// Work layout (gfx950, wave64, two workgroups of four waves per CU):
//  * a workgroup is 2 waves and 128 query rows of one (batch, head); a wave owns 64
//    rows as two groups of 32, so every K and V fragment read from LDS feeds two
//    MFMAs (64 flops per LDS byte: LDS reads stay below the matrix-core time);
//  * keys stream through LDS in tiles of 32, triple-buffered: tile t+2 is copied from
//    HBM straight into LDS (global_load_lds_dwordx4, no staging registers) while tile t
//    computes, with one barrier per tile. LDS rows are dense (256 B) and their 16-byte
//    chunks are XOR-swizzled so that every read pattern below is bank-conflict free:
//    K chunk c of row r sits at c ^ (r & 7) (8-lane 16 B reads over 8 rows), V chunk c
//    of row r at c ^ 2(r & 3) (16-lane transposed reads over 4 rows x 32 B);
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so each
//    lane holds 16 scores of one query row per group: the row max and row sum need
//    one exchange between lanes l and l^32 per tile and nothing else;
//  * the QK^T product of tile t+1 is issued before the softmax of tile t, so the
//    matrix cores work while the VALU does exp/max/sum;
//  * O^T = V^T P^T takes P straight from the score registers (B operand); V stays in
//    natural [key][d] order in LDS and ds_read_b64_tr_b16 transposes it on the read
//    (within 16 lanes, lane i element t <- lane i/4 + 4t's element i%4), fetching the
//    keys in exactly the order the score registers hold them;
//  * softmax uses exp2 with scale*log2(e) folded into one FMA per score; the running
//    max moves only when a tile's max exceeds it by more than 8 (log2 units), so the
//    accumulator rescale is rare and probabilities stay <= 256.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int D = 128;         // head dim of the bf16 path
constexpr int NW = 4;          // waves per workgroup
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int BQ = 32 * NW;    // query rows per workgroup (32 per wave)
constexpr int BK = 32;         // keys per LDS tile
constexpr int NBUF = 3;        // LDS tile buffers
constexpr int ROW = D;                    // bf16 per LDS row (dense, swizzled)
constexpr int TILE = BK * ROW;            // bf16 per tile and tensor (8 KB)
constexpr size_t LDS_BYTES = size_t(NBUF) * 2 * TILE * sizeof(uint16_t);
constexpr int COPIES = BK * D / 8 / NT;   // 16-byte copies per lane per tile and tensor (2)
constexpr float kRescaleSlack = 8.0f;

enum { MODE_ONLINE = 0, MODE_CONSTMAX = 1 };

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Makes the compiler wait for a value's load here (an empty asm that reads it), so no wait
// for it is left inside the tile loop, where it would also wait for in-flight tile copies.
template <typename T>
__device__ __forceinline__ void settle(const T& x) { asm volatile("" :: "v"(x)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((__attribute__((address_space(3))) const char*)(p)));
}

// One 16-byte-per-lane copy HBM -> LDS (global_load_lds_dwordx4): lane l's 16 bytes land at
// LDS byte m0 + 16*l. Issued as inline asm so that the compiler neither waits for it before
// unrelated LDS reads nor before barriers: the kernel places every wait for these copies.
__device__ __forceinline__ void copy16_to_lds(const void* g, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_byte), "v"(g) : "memory", "m0");
}

// Copies one 32-key tile of K and V from HBM into LDS. Copy u of wave w fills LDS rows
// (COPIES*w+u)*4 .. +3 (1 KB, lane l -> row + l/16, physical chunk l%16) and so reads the
// logical chunk that the swizzle places there. Rows past the chunk's end re-read the
// last key (their scores are masked, their values meet p = 0).
__device__ __forceinline__ void issue_tile(uint16_t* Kt, uint16_t* Vt, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t kss, int key0, int Sk, int w,
                                           int lane) {
#pragma unroll
  for (int u = 0; u < COPIES; ++u) {
    const int blk = w * COPIES + u;
    const int row = blk * 4 + (lane >> 4);
    const int p = lane & 15;
    const int64_t key = min(key0 + row, Sk - 1);
    const uint16_t* kg = kbase + key * kss + ((p ^ (row & 7)) << 3);
    const uint16_t* vg = vbase + key * kss + ((p ^ ((row & 3) << 1)) << 3);
    copy16_to_lds(kg, __builtin_amdgcn_readfirstlane(lds_addr(Kt + blk * 512)));
    copy16_to_lds(vg, __builtin_amdgcn_readfirstlane(lds_addr(Vt + blk * 512)));
  }
}

// Barrier after this wave's copies of the current tile have landed: with another tile's
// batch (2*COPIES copies) issued later, vmcnt(2*COPIES) leaves exactly that batch in flight.
__device__ __forceinline__ void wait_tile_and_barrier(bool newer_batch_in_flight) {
  static_assert(2 * COPIES == 4, "vmcnt immediate below assumes 4 copies per batch");
  if (newer_batch_in_flight) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 tr16_pair(const uint16_t* p) {
  typedef __attribute__((address_space(3))) short4v* lds_ptr;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p + 8 * ROW));
  const short4v both[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8*>(both);
}

// S^T for 32 keys x 32 rows. kr[j] is this lane's read offset for d-chunks c with
// c % 4 == j (row li, swizzled); chunks 4..7 add 64 elements.
__device__ __forceinline__ void qk_tile(const uint16_t* Kt, const int (&kr)[4], const bf16x8 (&q)[8], floatx16& s) {
  bf16x8 ka[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) ka[c] = *reinterpret_cast<const bf16x8*>(Kt + kr[c & 3] + (c >> 2) * 64);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], q[c], s, 0, 0, 0);
}

// Softmax numerators of one 32-row group: p = exp2(s*sl2e - mu) packed to bf16 in
// P.V operand order (kc = 0: registers 0..7, kc = 1: registers 8..15). Returns sum p.
__device__ __forceinline__ float exp_pack(const floatx16& s, float sl2e, float mu, bf16x8 (&pb)[2]) {
  float sum = 0.0f;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = kc * 8 + 2 * t;
      const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2e, -mu));
      const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], sl2e, -mu));
      sum += x0 + x1;
      w[t] = pack_bf16x2(x0, x1);
    }
    uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
    pb[kc] = *reinterpret_cast<bf16x8*>(&u);
  }
  return sum;
}

// Online-max bookkeeping of one group for one tile; returns the exp2 offset mu.
__device__ __forceinline__ float online_update(const floatx16& s, float sl2e, float& m_ref, float& l_part,
                                               floatx16 (&o)[4]) {
  float tmax = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
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
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    m_ref = m_new;
  }
  return (m_ref == -INFINITY) ? 0.0f : m_ref;
}

template <int MASK>
__device__ __forceinline__ void apply_mask(floatx16& s, int key0, int hl, int row, int Sk) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
    bool ok = j < Sk;
    if (MASK == CA_MASK_CAUSAL_INCL) ok &= j <= row;
    if (MASK == CA_MASK_CAUSAL_STRICT) ok &= j < row;
    s[r] = ok ? s[r] : -INFINITY;
  }
}

template <int MODE>
__device__ __forceinline__ void store_rows(const AttnArgs& a, int64_t bh, int Sq, int row, int hl,
                                           floatx16 (&o)[4], float l_part, float m_ref, float c2) {
  const float lrow = l_part + __shfl_xor(l_part, 32);
  if (row >= Sq) return;
  const int64_t rowidx = bh * Sq + row;
  // o[db][r] is O[row][d] for d = 32*db + 8*(r/4) + 4*hl + r%4: four consecutive d per float4.
  if (MODE == MODE_ONLINE) {
    const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
    float* orow = a.o + rowidx * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * hl) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
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

template <int MODE, int MASK>
__global__ __launch_bounds__(NT, 2)
void attn_step_bf16(const AttnArgs a, int nqb, int nwork) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Kb = lds;
  uint16_t* Vb = lds + NBUF * TILE;

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
  const int row = row_w0 + li;           // this lane's query row
  const int Sq = a.Sq, Sk = a.Sk;

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

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + h * a.ksh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.ksb + h * a.ksh;

  int kend = Sk;
  if (MASK != CA_MASK_NONE) kend = min(Sk, qb * BQ + BQ);
  const int nkt = (kend + BK - 1) / BK;

  floatx16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

  float m_ref = -INFINITY;   // running reference max (log2 units), online mode
  float l_part = 0.0f;       // this lane's share of the row sum
  float c2 = 0.0f;           // const-max bound in log2 units
  if (MODE == MODE_CONSTMAX) {
    c2 = a.c[int64_t(bh) * Sq + min(row, Sq - 1)] * kLog2e;
    settle(c2);
  }
  const float sl2e = a.sl2e;

  // Per-lane LDS read offsets (elements, within a tile).
  // K: row li, logical chunk 2c+hl at physical chunk (2c+hl) ^ (li & 7).
  int kr[4];
  {
    const int kx = li & 7;
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[j] = li * ROW + (((2 * j + hl) ^ kx) << 3);
  }
  // V (transposed reads): lane i16 of 16-lane group G reads row 4*hl + t (t = i16/4; +16 kc,
  // +8 for the second half), logical element 32*db + 16*(G&1) + 4*(i16&3), i.e. chunk
  // 4*db + 2*(G&1) + (i16&3)/2, swizzled by 2t: physical chunk 4*(db ^ (t>>1)) +
  // ((2*(G&1) + (i16&3)/2) ^ 2*(t&1)).
  int vr_even, vr_odd;
  {
    const int i16 = lane & 15;
    const int t = i16 >> 2;
    const int clow = (2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1)) ^ (2 * (t & 1));
    const int base = (4 * hl + t) * ROW + (clow << 3) + 4 * (i16 & 1);
    const int tb = t >> 1;
    vr_even = base + 32 * tb;    // db even: chunk block db + tb
    vr_odd = base - 32 * tb;     // db odd:  chunk block db - tb
  }

  // A tile is skipped by a wave when causality hides all of its keys from all 32 rows.
  auto skip_tile = [&](int t) -> bool {
    if (MASK == CA_MASK_CAUSAL_INCL) return t * BK > row_w0 + 31;
    if (MASK == CA_MASK_CAUSAL_STRICT) return t * BK >= row_w0 + 31;
    return false;
  };

  if (nkt > 0) issue_tile(Kb, Vb, kbase, vbase, a.kss, 0, Sk, w, lane);
  if (nkt > 1) issue_tile(Kb + TILE, Vb + TILE, kbase, vbase, a.kss, BK, Sk, w, lane);

  int buf = 0;
  for (int t = 0; t < nkt; ++t) {
    const int key0 = t * BK;
    const int nb1 = buf == NBUF - 1 ? 0 : buf + 1;
    const int nb2 = nb1 == NBUF - 1 ? 0 : nb1 + 1;
    // tile t's copies (issued two iterations ago, or in the prologue) must have landed;
    // tile t+1's batch may stay in flight
    wait_tile_and_barrier(t + 1 < nkt);
    // tile t+2 goes into the buffer that tile t-1 used (free: every wave passed the barrier)
    if (t + 2 < nkt) issue_tile(Kb + nb2 * TILE, Vb + nb2 * TILE, kbase, vbase, a.kss, key0 + 2 * BK, Sk, w, lane);

    if (!skip_tile(t)) {
      // V fragments first: their LDS latency hides behind QK^T and the softmax
      const uint16_t* vt = Vb + buf * TILE;
      bf16x8 va[8];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          va[db * 2 + kc] = tr16_pair(vt + ((db & 1) ? vr_odd : vr_even) + kc * 16 * ROW + db * 32);
      floatx16 s;
      qk_tile(Kb + buf * TILE, kr, q, s);
      bool need_mask = key0 + BK > Sk;
      if (MASK == CA_MASK_CAUSAL_INCL) need_mask |= key0 + BK - 1 > row_w0;
      if (MASK == CA_MASK_CAUSAL_STRICT) need_mask |= key0 + BK - 1 >= row_w0;
      if (need_mask) apply_mask<MASK>(s, key0, hl, row, Sk);
      float mu;
      if (MODE == MODE_ONLINE) mu = online_update(s, sl2e, m_ref, l_part, o);
      else mu = c2;
      bf16x8 p[2];
      l_part += exp_pack(s, sl2e, mu, p);

#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db * 2 + kc], p[kc], o[db], 0, 0, 0);
    }
    buf = nb1;
  }

  store_rows<MODE>(a, bh, Sq, row, hl, o, l_part, m_ref, c2);
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
