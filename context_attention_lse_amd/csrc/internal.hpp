// Internal declarations shared by the HIP sources of libctxattn (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctxattn.h"

namespace ctxattn {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumClamp = 1e-37f;   // row-sum floor of the const-max normalisation

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even pack of two floats into two bf16 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  floatx2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return *reinterpret_cast<uint32_t*>(&b);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Maps a launch-order workgroup id to a logical work item so that consecutive
// logical items land on the same XCD (workgroups are dealt round-robin over the
// 8 XCDs). The grid is padded to a multiple of 8; padded ids return -1.
__device__ __forceinline__ int xcd_logical_id(int wg, int grid, int nwork) {
  const int per = grid >> 3;
  const int logical = (wg & 7) * per + (wg >> 3);
  return logical < nwork ? logical : -1;
}

__host__ __device__ inline int round_up8(int n) { return (n + 7) & ~7; }

// ---------------------------------------------------------------- launch descriptors
// Two-way LSE merge of a prior partial (lse_p) with a new one (lse_t), natural-log LSEs:
// M = max, L = M + log(e^(lse_p - M) + e^(lse_t - M)), weights e^(lse - L) ("Sharding the
// Input": ring attention's per-block rescale; the DCP merge of partial outputs by their LSE).
// Both empty (-inf): weights 0 and L = -inf, so the merged row is O = 0, LSE = -inf.
__device__ __forceinline__ float lse_fold_weights(float lse_p, float lse_t, float& w_p, float& w_t) {
  const float M = fmaxf(lse_p, lse_t);
  if (M == -INFINITY) {
    w_p = 0.0f;
    w_t = 0.0f;
    return -INFINITY;
  }
  const float L = M + logf(expf(lse_p - M) + expf(lse_t - M));
  w_p = expf(lse_p - L);
  w_t = expf(lse_t - L);
  return L;
}

struct AttnArgs {
  const void* q;
  int64_t qsb, qss, qsh;
  const void* k;
  const void* v;
  int64_t ksb, kss, ksh;
  int B, H, Sq, Sk, D;
  float scale;      // softmax scale
  float sl2e;       // scale * log2(e)
  int mask;         // ca_mask
  // online-max outputs; fold != 0: o and lse hold a prior partial on entry and are
  // replaced by its LSE merge with this chunk's partial
  float* o;
  float* lse;
  int fold;
  // const-max inputs/outputs
  const float* c;
  float* acc;
  int phase;
  void* o_cm;
  int o_cm_bf16;
  float* lse_cm;
  // key-split workspace (bf16 path); NULL: one workgroup per query tile
  void* ws;
  size_t ws_bytes;
  // query heads per K/V head (1: MHA); query head h reads K/V head h / G (bf16 path)
  int G;
  // kMaskDcp: DCP prefill slice of rank dcp_R in a group of dcp_W, interleave dcp_I
  int dcp_I, dcp_W, dcp_R;
  // keys to leave out (bf16 path): per (batch, head) up to sink_cap global key indices
  // sink_idx[bh * sink_cap + i] for i < sink_cnt[bh]; this chunk's first key is key_offset
  const int32_t* sink_idx;
  const int32_t* sink_cnt;
  int sink_cap;
  int64_t key_offset;
  // per (batch, head) key count (bf16 path, no key split): keys [0, min(Sk, sk_of_bh[bh]))
  const int32_t* sk_of_bh;
  // ring hop carried by the same launch (bf16 path): hop_units 16-byte vectors of K and of
  // V copied from hop_sk / hop_sv to hop_dk / hop_dv by hop_wgs workgroups appended to the
  // grid (0: no hop)
  const void* hop_sk;
  const void* hop_sv;
  void* hop_dk;
  void* hop_dv;
  int64_t hop_units;
  int hop_wgs;
  // a second hop carried by the same workgroups (hop_units2 vectors of K and of V; 0: none)
  const void* hop_sk2;
  const void* hop_sv2;
  void* hop_dk2;
  void* hop_dv2;
  int64_t hop_units2;
  // a second K/V chunk (bf16 path, no mask): keys [Sk1, Sk) of the launch are keys
  // [0, Sk - Sk1) of k2 / v2, which share k's strides; Sk1 is a multiple of the key tile.
  // NULL: one chunk.
  const void* k2;
  const void* v2;
  int Sk1;
};

// Internal mask (bf16 path, online-max only): the keys are rank R's slice of a chunk
// whose positions are dealt to W ranks in blocks of I (slice token j at chunk position
// (j / I) * W * I + R * I + j % I) and query i sits at chunk position i; key j is
// visible iff its position is <= i, i.e. iff j < local_filled(i + 1).
constexpr int kMaskDcp = 3;

// Launchers (return hipSuccess or the launch error).
hipError_t launch_attn_bf16(const AttnArgs& a, bool const_max, hipStream_t s);
// Bytes of key-split workspace the bf16 step needs for these sizes on the current device
// (0: the call has no key tiles and never splits).
size_t attn_bf16_workspace_bytes(int B, int H, int Sq, int Sk, int mask);
hipError_t launch_attn_f32(const AttnArgs& a, bool const_max, bool bf16_in, hipStream_t s);
hipError_t launch_lse_merge(int n, const float* o_parts, const float* lse_parts, int64_t rows,
                            int D, void* o_out, int o_bf16, float* lse_out, hipStream_t s);
hipError_t launch_key_sqnorm_max(const void* k, int64_t sb, int64_t ss, int64_t sh, bool bf16,
                                 int B, int S, int H, int D, float* kmax_sq, bool accumulate,
                                 hipStream_t s);
hipError_t launch_const_max_bound(const void* q, int64_t sb, int64_t ss, int64_t sh, bool bf16,
                                  int B, int Sq, int H, int D, float scale, const float* kmax_sq,
                                  float* c, hipStream_t s);

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* local_lens;
  int B, Hq, Hkv, D, block_size, max_blocks, num_blocks;
  float sl2e;
  float* o;
  float* lse;
  float* ws_o;      // [B, Hq, max_splits, D]
  float* ws_lse;    // [B, Hq, max_splits]
  int max_splits;
  // current-token form (prior_lens != NULL): each sequence's resident count is local_filled
  // of its prior length, and the current token's K/V joins on the rank that owns position N
  const int32_t* prior_lens;   // [B] prior tokens N of each sequence (global count)
  const void* k_cur;           // [B, Hkv, D] bf16
  const void* v_cur;           // [B, Hkv, D] bf16
  int rank, world, interleave;
  float scale;
};

// Tokens among positions [0, N) that shard `rank` holds when blocks of `interleave`
// positions are dealt round-robin over `world` shards and each shard fills blocks of
// `block_size` (a multiple of interleave): DCP page, local_filled computation.
__host__ __device__ inline int dcp_local_filled(int N, int rank, int block_size, int interleave, int world) {
  const int vblock = block_size * world;
  const int stride = interleave * world;
  int filled = (N / vblock) * block_size;
  const int remaining = N - (N / vblock) * vblock;
  filled += (remaining / stride) * interleave;
  const int leftover = remaining - (remaining / stride) * stride;
  filled += min(max(leftover - rank * interleave, 0), interleave);
  return filled;
}

// The shard whose slot mapping holds position N (DCP page, dcp_active_mask).
__host__ __device__ inline int dcp_active_owner(int N, int block_size, int interleave, int world) {
  const int vblock = block_size * world;
  return ((N % vblock) / interleave) % world;
}

constexpr int kDecodeSplitTokens = 1536;   // tokens per decode split (96 blocks of 16)
// Splits per sequence in the decode grid: enough for max_tokens, made odd. The split kernel's
// grid is (split, KV head, sequence) and consecutive workgroups go to the 8 XCDs in turn, so
// with an even count a split index keeps landing on the same few XCDs for every sequence,
// and the low splits, resident in every sequence, pile up there (with 64 splits of 1024
// tokens the decode ran 8% slower than with 65). An odd count spreads every split index over
// all 8 XCDs. The extra split holds no tokens; its workgroups return at once.
__host__ __device__ inline int64_t decode_grid_splits(int64_t max_tokens) {
  const int64_t n = (max_tokens + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
  return (n > 0 && n % 2 == 0) ? n + 1 : n;
}
size_t decode_workspace_bytes(int B, int Hq, int D, int block_size, int max_blocks);
hipError_t launch_dcp_decode(const DecodeArgs& a, hipStream_t s);
// Sink-robust const-max prologue over a pool of cp chunks (key (c, b, t, h) at element
// c*cs + b*sb + t*ss + h*sh) and the gather of the listed sink rows ([B, cap, H, 128] bf16).
hipError_t launch_sink_prologue(const void* k, int64_t cs, int64_t sb, int64_t ss, int64_t sh, bool bf16, int cp,
                                int B, int S, int H, int D, float theta, int cap, float* kmax_sq, float* knorm_sum,
                                float* kmax_robust, int32_t* sink_idx, int32_t* sink_cnt, hipStream_t s);
hipError_t launch_sink_gather(const void* k, const void* v, int64_t cs, int64_t sb, int64_t ss, int64_t sh, int B,
                              int S, int H, int cap, const int32_t* sink_idx, const int32_t* sink_cnt, void* kg,
                              void* vg, hipStream_t s);

// DCP prefill (segmented attention) of one rank; B == 1, D == 128, block size 16.
struct SegmentedArgs {
  const void* q;            // [S, Hq, D] bf16, strides qss, qsh
  int64_t qss, qsh;
  const void* k_cur;        // [S_local, Hkv, D] bf16, strides kss, ksh (v_cur the same)
  const void* v_cur;
  int64_t kss, ksh;
  const void* k_cache;      // [num_blocks, Hkv, 16, D] bf16
  const void* v_cache;      // [num_blocks, Hkv, D, 16] bf16
  const int32_t* block_table;
  int num_blocks, prior;    // prior: this rank's prior slots
  int rank, world, interleave;
  int Hq, Hkv, S, S_local;
  float scale;
  float* o;                 // [Hq, S, D] fp32
  float* lse;               // [Hq, S] fp32
  void* ws;                 // segmented_workspace_bytes()
};
size_t segmented_workspace_bytes(int Hq, int Hkv, int S, int D, int prior);
hipError_t launch_segmented(const SegmentedArgs& g, hipStream_t s);
hipError_t launch_kv_copy(void* dk, void* dv, const void* sk, const void* sv, size_t bytes, hipStream_t s);
// Workgroups of a bf16 step launch that would sit idle over its last round of workgroups
// (the device's slots minus the last round's work items).
int attn_bf16_idle_slots(int B, int H, int Sq, int Sk, int mask, bool with_workspace);

}  // namespace ctxattn
