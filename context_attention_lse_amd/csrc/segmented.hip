// DCP prefill: one rank's segmented attention ("DCP (Decode Context Parallelism)" page,
// "Segmented Attention CP", algorithm steps 1-4). The rank holds every query of the chunk
// and two sets of keys: its prior tokens in the paged cache (all earlier than every query,
// so all visible) and its slice of the chunk (visible by global position). The call
//   1. gathers the prior slots from the paged cache into token-major K and V,
//   2. runs the step kernel over them (no mask), writing its partial to the outputs,
//   3. runs the step kernel over the chunk slice with the interleaved causal mask, whose
//      epilogue merges its partial into the outputs by the LSE rule (step 4's merge).
// Query head h reads K/V head h / (Hq / Hkv) in both steps.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int D = 128;
constexpr int BS = 16;     // tokens per cache block
constexpr int NT = 256;

// One cache block per workgroup: its 16 slots of every K/V head become token-major rows
// of kg / vg ([n_prior, Hkv, D]). V blocks are d-major in the cache ([Hkv][D][16]) and go
// through LDS to be transposed. Slots at or past n_prior are not written; a block id
// outside [0, num_blocks) reads as zeros.
__global__ __launch_bounds__(NT) void prior_gather_kernel(const uint16_t* k_cache, const uint16_t* v_cache,
                                                          const int32_t* block_table, int num_blocks, int n_prior,
                                                          int Hkv, uint16_t* kg, uint16_t* vg) {
  extern __shared__ uint16_t vblk[];   // [Hkv][D][BS]
  const int j = blockIdx.x;
  const int blk = block_table[j];
  const bool ok = blk >= 0 && blk < num_blocks;
  const int ntok = min(BS, n_prior - j * BS);
  const int tid = threadIdx.x;
  const int row_chunks = Hkv * BS * (D / 8);   // 16-byte pieces per block and tensor
  // K: block rows [h][t] of 256 bytes -> kg row (j*16 + t, h)
  for (int e = tid; e < row_chunks; e += NT) {
    const int c = e % (D / 8), r = e / (D / 8);
    const int h = r / BS, t = r % BS;
    if (t >= ntok) continue;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4*>(k_cache + ((int64_t(blk) * Hkv + h) * BS + t) * D + 8 * c);
    *reinterpret_cast<uint4*>(kg + ((int64_t(j) * BS + t) * Hkv + h) * D + 8 * c) = v;
  }
  // V: stage the block in LDS as stored, then write token-major rows
  for (int e = tid; e < row_chunks; e += NT) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4*>(v_cache + int64_t(blk) * Hkv * D * BS + 8 * e);
    *reinterpret_cast<uint4*>(vblk + 8 * e) = v;
  }
  __syncthreads();
  for (int e = tid; e < row_chunks; e += NT) {
    const int c = e % (D / 8), r = e / (D / 8);
    const int h = r / BS, t = r % BS;
    if (t >= ntok) continue;
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = 8 * c + 2 * u;
      w[u] = uint32_t(vblk[(h * D + d) * BS + t]) | (uint32_t(vblk[(h * D + d + 1) * BS + t]) << 16);
    }
    *reinterpret_cast<uint4*>(vg + ((int64_t(j) * BS + t) * Hkv + h) * D + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

// The gathered prior K and V; the two partials (prior, then this rank's slice folded into it)
// go straight to the caller's o and lse.
size_t segmented_workspace_bytes(int Hq, int Hkv, int S, int D_, int prior) {
  (void)Hq; (void)S;
  if (prior <= 0) return 0;
  const size_t kv = align256(size_t(prior) * Hkv * D_ * 2);
  return 2 * kv;
}

hipError_t launch_segmented(const SegmentedArgs& g, hipStream_t s) {
  AttnArgs a{};
  a.q = g.q; a.qsb = 0; a.qss = g.qss; a.qsh = g.qsh;
  a.B = 1; a.H = g.Hq; a.Sq = g.S; a.D = D;
  a.scale = g.scale; a.sl2e = g.scale * kLog2e;
  a.G = g.Hq / g.Hkv;
  a.dcp_I = g.interleave; a.dcp_W = g.world; a.dcp_R = g.rank;
  if (g.prior <= 0) {
    a.k = g.k_cur; a.v = g.v_cur; a.ksb = 0; a.kss = g.kss; a.ksh = g.ksh;
    a.Sk = g.S_local; a.mask = kMaskDcp;
    a.o = g.o; a.lse = g.lse;
    return launch_attn_bf16(a, false, s);
  }
  char* ws = static_cast<char*>(g.ws);
  const size_t kv = align256(size_t(g.prior) * g.Hkv * D * 2);
  uint16_t* kg = reinterpret_cast<uint16_t*>(ws);
  uint16_t* vg = reinterpret_cast<uint16_t*>(ws + kv);
  const int nblk = (g.prior + BS - 1) / BS;
  hipLaunchKernelGGL(prior_gather_kernel, dim3(nblk), dim3(NT), size_t(g.Hkv) * D * BS * 2, s,
                     static_cast<const uint16_t*>(g.k_cache), static_cast<const uint16_t*>(g.v_cache), g.block_table,
                     g.num_blocks, g.prior, g.Hkv, kg, vg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // prior keys: all earlier than every query; their partial goes straight to o and lse
  a.k = kg; a.v = vg; a.ksb = 0; a.kss = int64_t(g.Hkv) * D; a.ksh = D;
  a.Sk = g.prior; a.mask = CA_MASK_NONE;
  a.o = g.o; a.lse = g.lse;
  if ((e = launch_attn_bf16(a, false, s)) != hipSuccess) return e;
  // this rank's slice of the chunk, causal on global positions, folded into that partial by
  // the LSE rule in the step's epilogue (no separate merge of two partials)
  a.k = g.k_cur; a.v = g.v_cur; a.kss = g.kss; a.ksh = g.ksh;
  a.Sk = g.S_local; a.mask = kMaskDcp;
  a.fold = 1;
  return launch_attn_bf16(a, false, s);
}

}  // namespace ctxattn
