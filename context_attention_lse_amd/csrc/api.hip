// C ABI of libctxattn: argument validation, then one launch sequence per call on the
// caller's stream. No allocation, no state kept between calls (see include/ctxattn.h).
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

ca_status fail(ca_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ca_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return CA_OK;
  }
  return fail(CA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

float resolve_scale(float s, int D) { return s > 0.0f ? s : 1.0f / std::sqrt(float(D)); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a [B, S, H, D] strided input: D contiguous, every row start 16-byte aligned.
ca_status check_bshd(const char* name, const void* p, const ca_strides& st, int dtype, int B, int S, int H, int D) {
  if (B < 0 || S < 0 || H < 0 || D <= 0) return fail(CA_ERR_SHAPE, "%s: negative or zero size", name);
  if (B == 0 || S == 0 || H == 0) return CA_OK;
  if (!p) return fail(CA_ERR_NULL, "%s is NULL", name);
  const int esz = dtype == CA_BF16 ? 2 : 4;
  if (!aligned16(p)) return fail(CA_ERR_SHAPE, "%s must be 16-byte aligned", name);
  if (st.b < 0 || st.s < 0 || st.h < 0) return fail(CA_ERR_SHAPE, "%s: negative stride", name);
  if (((st.b * esz) & 15) || ((st.s * esz) & 15) || ((st.h * esz) & 15))
    return fail(CA_ERR_SHAPE, "%s: strides must keep every row 16-byte aligned", name);
  if (H > 1 && st.h < D) return fail(CA_ERR_SHAPE, "%s: head stride %lld < D", name, (long long)st.h);
  return CA_OK;
}

ca_status check_dtype(int dtype) {
  if (dtype != CA_BF16 && dtype != CA_FP32) return fail(CA_ERR_DTYPE, "unknown dtype code %d", dtype);
  return CA_OK;
}

ca_status check_head_dim(int dtype, int D) {
  if (D != 64 && D != 128)
    return fail(CA_ERR_UNSUPPORTED, "%s attention supports head_dim 64 or 128 (got %d)",
                dtype == CA_BF16 ? "bf16" : "fp32", D);
  return CA_OK;
}

// The MFMA step kernel takes bf16 with head_dim 128; every other supported case (fp32, and
// bf16 with head_dim 64) runs on the fp32 vector kernel.
bool mfma_step(int dtype, int D) { return dtype == CA_BF16 && D == 128; }

#define CA_TRY(expr)                 \
  do {                               \
    ca_status _st = (expr);          \
    if (_st != CA_OK) return _st;    \
  } while (0)

ca_status attn_common(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs, int dtype, int B,
                      int H, int Sq, int Sk, int D) {
  CA_TRY(check_dtype(dtype));
  CA_TRY(check_head_dim(dtype, D));
  if (Sq < 0 || Sk < 0) return fail(CA_ERR_SHAPE, "negative sequence length");
  CA_TRY(check_bshd("q", q, qs, dtype, B, Sq, H, D));
  CA_TRY(check_bshd("k", k, kvs, dtype, B, Sk, H, D));
  CA_TRY(check_bshd("v", v, kvs, dtype, B, Sk, H, D));
  return CA_OK;
}

// Hands a caller workspace to the bf16 step, which then splits key ranges across a grid
// that fills the device. NULL keeps one workgroup per query tile; the fp32 step never splits.
ca_status attach_workspace(ctxattn::AttnArgs& a, int dtype, void* ws, size_t ws_bytes) {
  if (!ws || !mfma_step(dtype, a.D)) return CA_OK;
  const size_t need = ctxattn::attn_bf16_workspace_bytes(a.B, a.H, a.Sq, a.Sk, a.mask);
  if (need == 0) return CA_OK;
  if (ws_bytes < need)
    return fail(CA_ERR_WORKSPACE, "step workspace has %zu bytes, the call needs %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(CA_ERR_SHAPE, "step workspace must be 256-byte aligned");
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return CA_OK;
}

}  // namespace

extern "C" {

const char* ca_last_error(void) { return g_err; }

const char* ca_version(void) { return "0.1.0"; }

// A ring hop (kv_chunk_copy's job) carried by a step call; bytes == 0: none.
struct Hop {
  void* dk;
  void* dv;
  const void* sk;
  const void* sv;
  size_t bytes;
};

// Workgroups that carry a ring hop inside a step launch: as many as the step's last round
// leaves free, from kMinHopWorkgroups (fewer: the copy runs ahead of the step instead) up to
// kMaxHopWorkgroups.
constexpr int kMinHopWorkgroups = 16;
constexpr int kMaxHopWorkgroups = 64;

// Attaches a hop to a bf16 step launch when its last round leaves enough CUs free, else
// launches it as an ordinary copy ahead of the step on the same stream.
static hipError_t attach_hop(ctxattn::AttnArgs& a, const Hop& hop, int dtype, int mask, hipStream_t s) {
  if (hop.bytes == 0) return hipSuccess;
  const int idle =
      mfma_step(dtype, a.D) ? ctxattn::attn_bf16_idle_slots(a.B, a.H, a.Sq, a.Sk, mask, a.ws != nullptr) : 0;
  if (idle < kMinHopWorkgroups) return ctxattn::launch_kv_copy(hop.dk, hop.dv, hop.sk, hop.sv, hop.bytes, s);
  a.hop_sk = hop.sk; a.hop_sv = hop.sv; a.hop_dk = hop.dk; a.hop_dv = hop.dv;
  a.hop_units = int64_t(hop.bytes / 16);
  a.hop_wgs = idle < kMaxHopWorkgroups ? idle : kMaxHopWorkgroups;
  return hipSuccess;
}

// Validates the hop arguments of a *_hop entry point.
static ca_status check_hop(const char* fn, const Hop& hop) {
  if (hop.bytes == 0) return CA_OK;
  if (!hop.dk || !hop.dv || !hop.sk || !hop.sv) return fail(CA_ERR_NULL, "%s: hop buffers are required when hop_bytes > 0", fn);
  if (hop.bytes % 16 || !aligned16(hop.dk) || !aligned16(hop.dv) || !aligned16(hop.sk) || !aligned16(hop.sv))
    return fail(CA_ERR_SHAPE, "%s: hop pointers must be 16-byte aligned and hop_bytes a multiple of 16", fn);
  return CA_OK;
}

// The second chunk of a two-chunk step launch (ring_attn_step_pair); k2 == NULL: none.
struct Pair {
  const void* k2;
  const void* v2;
  int Sk1;
};

static ca_status ring_attn_step_impl(const char* name, const void* q, ca_strides qs, const void* k, const void* v,
                                     ca_strides kvs, int dtype, int B, int H, int Sq, int Sk, int D,
                                     float softmax_scale, int mask, float* o, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream, int fold, Hop hop = Hop{},
                                     Pair pair = Pair{}, Hop hop2 = Hop{}) {
  // (a two-chunk launch: k and v hold the first chunk's Sk1 keys; the caller checked the second)
  CA_TRY(attn_common(q, qs, k, v, kvs, dtype, B, H, Sq, pair.k2 ? pair.Sk1 : Sk, D));
  if (mask < CA_MASK_NONE || mask > CA_MASK_CAUSAL_STRICT) return fail(CA_ERR_UNSUPPORTED, "unknown mask %d", mask);
  if (int64_t(B) * H * Sq == 0) {   // no rows: only the hops, if any
    hipError_t e = hipSuccess;
    if (hop.bytes) e = ctxattn::launch_kv_copy(hop.dk, hop.dv, hop.sk, hop.sv, hop.bytes, static_cast<hipStream_t>(stream));
    if (e == hipSuccess && hop2.bytes)
      e = ctxattn::launch_kv_copy(hop2.dk, hop2.dv, hop2.sk, hop2.sv, hop2.bytes, static_cast<hipStream_t>(stream));
    return hip_status(e, name);
  }
  if (!o || !lse) return fail(CA_ERR_NULL, "o and lse are required");
  if (!aligned16(o)) return fail(CA_ERR_SHAPE, "o must be 16-byte aligned");
  ctxattn::AttnArgs a{};
  a.q = q; a.qsb = qs.b; a.qss = qs.s; a.qsh = qs.h;
  a.k = k; a.v = v; a.ksb = kvs.b; a.kss = kvs.s; a.ksh = kvs.h;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.D = D;
  a.scale = resolve_scale(softmax_scale, D);
  a.sl2e = a.scale * ctxattn::kLog2e;
  a.mask = mask;
  a.G = 1;
  a.o = o; a.lse = lse;
  a.fold = fold;
  a.k2 = pair.k2; a.v2 = pair.v2; a.Sk1 = pair.Sk1;
  CA_TRY(attach_workspace(a, dtype, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = attach_hop(a, hop, dtype, mask, s);
  if (e == hipSuccess && hop2.bytes) {   // the second hop rides with the first, or is copied ahead
    if (a.hop_wgs > 0) {
      a.hop_sk2 = hop2.sk; a.hop_sv2 = hop2.sv; a.hop_dk2 = hop2.dk; a.hop_dv2 = hop2.dv;
      a.hop_units2 = int64_t(hop2.bytes / 16);
    } else {
      e = ctxattn::launch_kv_copy(hop2.dk, hop2.dv, hop2.sk, hop2.sv, hop2.bytes, s);
    }
  }
  if (e != hipSuccess) return hip_status(e, name);
  e = mfma_step(dtype, D) ? ctxattn::launch_attn_bf16(a, false, s)
                          : ctxattn::launch_attn_f32(a, false, dtype == CA_BF16, s);
  return hip_status(e, name);
}

ca_status ring_attn_step(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs, int dtype, int B,
                         int H, int Sq, int Sk, int D, float softmax_scale, int mask, float* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return ring_attn_step_impl("ring_attn_step launch", q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale, mask,
                             o, lse, workspace, workspace_bytes, stream, 0);
}

ca_status ring_attn_step_fold(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs, int dtype,
                              int B, int H, int Sq, int Sk, int D, float softmax_scale, int mask, float* o,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return ring_attn_step_impl("ring_attn_step_fold launch", q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale,
                             mask, o, lse, workspace, workspace_bytes, stream, 1);
}

ca_status ring_attn_step_hop(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs, int dtype,
                             int B, int H, int Sq, int Sk, int D, float softmax_scale, int mask, float* o,
                             float* lse, void* workspace, size_t workspace_bytes, void* hop_dst_k, void* hop_dst_v,
                             const void* hop_src_k, const void* hop_src_v, size_t hop_bytes, void* stream) {
  const Hop hop{hop_dst_k, hop_dst_v, hop_src_k, hop_src_v, hop_bytes};
  CA_TRY(check_hop("ring_attn_step_hop", hop));
  return ring_attn_step_impl("ring_attn_step_hop launch", q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale,
                             mask, o, lse, workspace, workspace_bytes, stream, 0, hop);
}

ca_status ring_attn_step_fold_hop(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs,
                                  int dtype, int B, int H, int Sq, int Sk, int D, float softmax_scale, int mask,
                                  float* o, float* lse, void* workspace, size_t workspace_bytes, void* hop_dst_k,
                                  void* hop_dst_v, const void* hop_src_k, const void* hop_src_v, size_t hop_bytes,
                                  void* stream) {
  const Hop hop{hop_dst_k, hop_dst_v, hop_src_k, hop_src_v, hop_bytes};
  CA_TRY(check_hop("ring_attn_step_fold_hop", hop));
  return ring_attn_step_impl("ring_attn_step_fold_hop launch", q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D,
                             softmax_scale, mask, o, lse, workspace, workspace_bytes, stream, 1, hop);
}

ca_status ring_attn_step_pair(const void* q, ca_strides qs, const void* k1, const void* v1, const void* k2,
                              const void* v2, ca_strides kvs, int dtype, int B, int H, int Sq, int Sk1, int Sk2,
                              int D, float softmax_scale, int fold, float* o, float* lse, void* workspace,
                              size_t workspace_bytes, void* hop_dst_k, void* hop_dst_v, const void* hop_src_k,
                              const void* hop_src_v, void* hop2_dst_k, void* hop2_dst_v, const void* hop2_src_k,
                              const void* hop2_src_v, size_t hop_bytes, void* stream) {
  const char* name = "ring_attn_step_pair";
  if (Sk1 < 0 || Sk2 < 0) return fail(CA_ERR_SHAPE, "%s: negative chunk length", name);
  if (int64_t(Sk1) + Sk2 > INT_MAX) return fail(CA_ERR_UNSUPPORTED, "%s: chunks too long", name);
  CA_TRY(check_dtype(dtype));
  CA_TRY(check_head_dim(dtype, D));
  if (!mfma_step(dtype, D)) return fail(CA_ERR_UNSUPPORTED, "%s: bf16 with head_dim 128 only", name);
  if (Sk1 % 32) return fail(CA_ERR_UNSUPPORTED, "%s: the first chunk's length must be a multiple of 32 (got %d)",
                            name, Sk1);
  CA_TRY(check_bshd("k2", k2, kvs, dtype, B, Sk2, H, D));
  CA_TRY(check_bshd("v2", v2, kvs, dtype, B, Sk2, H, D));
  const Hop h1{hop_dst_k, hop_dst_v, hop_src_k, hop_src_v, hop_bytes};
  const Hop h2 = hop2_src_k ? Hop{hop2_dst_k, hop2_dst_v, hop2_src_k, hop2_src_v, hop_bytes} : Hop{};
  CA_TRY(check_hop(name, h1));
  CA_TRY(check_hop(name, h2));
  if (Sk1 == 0 || Sk2 == 0) {   // one chunk: the plain step, hops copied ahead of it
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h2.bytes) {
      const ca_status st = hip_status(ctxattn::launch_kv_copy(h2.dk, h2.dv, h2.sk, h2.sv, h2.bytes, s), name);
      if (st != CA_OK) return st;
    }
    return ring_attn_step_impl(name, q, qs, Sk1 ? k1 : k2, Sk1 ? v1 : v2, kvs, dtype, B, H, Sq, Sk1 + Sk2, D,
                               softmax_scale, CA_MASK_NONE, o, lse, workspace, workspace_bytes, stream, fold, h1);
  }
  return ring_attn_step_impl(name, q, qs, k1, v1, kvs, dtype, B, H, Sq, Sk1 + Sk2, D, softmax_scale, CA_MASK_NONE, o,
                             lse, workspace, workspace_bytes, stream, fold, h1, Pair{k2, v2, Sk1}, h2);
}

ca_status ring_attn_workspace_size(int dtype, int B, int H, int Sq, int Sk, int D, int mask, size_t* bytes) {
  if (!bytes) return fail(CA_ERR_NULL, "bytes is NULL");
  *bytes = 0;
  CA_TRY(check_dtype(dtype));
  CA_TRY(check_head_dim(dtype, D));
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return fail(CA_ERR_SHAPE, "negative size");
  if (mask < CA_MASK_NONE || mask > CA_MASK_CAUSAL_STRICT) return fail(CA_ERR_UNSUPPORTED, "unknown mask %d", mask);
  if (mfma_step(dtype, D)) *bytes = ctxattn::attn_bf16_workspace_bytes(B, H, Sq, Sk, mask);
  return hip_status(hipSuccess, "");
}

ca_status key_sqnorm_max(const void* k, ca_strides ks, int dtype, int B, int S, int H, int D, float* kmax_sq,
                         int accumulate, void* stream) {
  CA_TRY(check_dtype(dtype));
  if (D <= 0 || D % 8 || D > 128) return fail(CA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in [8, 128]");
  CA_TRY(check_bshd("k", k, ks, dtype, B, S, H, D));
  if (int64_t(B) * H == 0) return hip_status(hipSuccess, "");
  if (!kmax_sq) return fail(CA_ERR_NULL, "kmax_sq is NULL");
  if (H > 4096) return fail(CA_ERR_UNSUPPORTED, "at most 4096 heads");
  hipError_t e = ctxattn::launch_key_sqnorm_max(k, ks.b, ks.s, ks.h, dtype == CA_BF16, B, S, H, D, kmax_sq,
                                                accumulate != 0, static_cast<hipStream_t>(stream));
  return hip_status(e, "key_sqnorm_max launch");
}

ca_status const_max_bound(const void* q, ca_strides qs, int dtype, int B, int Sq, int H, int D, float softmax_scale,
                          const float* kmax_sq, float* c, void* stream) {
  CA_TRY(check_dtype(dtype));
  if (D <= 0 || D % 8 || D > 128) return fail(CA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in [8, 128]");
  CA_TRY(check_bshd("q", q, qs, dtype, B, Sq, H, D));
  if (int64_t(B) * H * Sq == 0) return hip_status(hipSuccess, "");
  if (!kmax_sq || !c) return fail(CA_ERR_NULL, "kmax_sq and c are required");
  if (H > 256) return fail(CA_ERR_UNSUPPORTED, "at most 256 heads");
  hipError_t e = ctxattn::launch_const_max_bound(q, qs.b, qs.s, qs.h, dtype == CA_BF16, B, Sq, H, D,
                                                 resolve_scale(softmax_scale, D), kmax_sq, c,
                                                 static_cast<hipStream_t>(stream));
  return hip_status(e, "const_max_bound launch");
}

}  // extern "C"

namespace {

ca_status const_max_step_impl(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs, int dtype,
                              int B, int H, int Sq, int Sk, int D, float softmax_scale, const float* c, float* acc,
                              int phase, void* o, int o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                              const int32_t* sink_idx, const int32_t* sink_cnt, int sink_cap, int64_t key_offset,
                              void* stream, Hop hop = Hop{}) {
  CA_TRY(attn_common(q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D));
  if (phase < 0 || phase > (CA_PHASE_INIT | CA_PHASE_FINAL)) return fail(CA_ERR_SHAPE, "unknown phase %d", phase);
  if (int64_t(B) * H * Sq == 0) {   // no rows: only the hop, if any
    if (hop.bytes == 0) return hip_status(hipSuccess, "");
    return hip_status(ctxattn::launch_kv_copy(hop.dk, hop.dv, hop.sk, hop.sv, hop.bytes, static_cast<hipStream_t>(stream)),
                      "ring_attn_const_max_step_hop");
  }
  if (!c) return fail(CA_ERR_NULL, "the bound c is required");
  const bool init = phase & CA_PHASE_INIT, final_ = phase & CA_PHASE_FINAL;
  if (!(init && final_) && !acc) return fail(CA_ERR_NULL, "acc is required unless phase is INIT|FINAL");
  if (acc && !aligned16(acc)) return fail(CA_ERR_SHAPE, "acc must be 16-byte aligned");
  if (final_) {
    if (!o) return fail(CA_ERR_NULL, "o is required on the FINAL phase");
    CA_TRY(check_dtype(o_dtype));
    if (!aligned16(o)) return fail(CA_ERR_SHAPE, "o must be 16-byte aligned");
  }
  ctxattn::AttnArgs a{};
  a.q = q; a.qsb = qs.b; a.qss = qs.s; a.qsh = qs.h;
  a.k = k; a.v = v; a.ksb = kvs.b; a.kss = kvs.s; a.ksh = kvs.h;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.D = D;
  a.scale = resolve_scale(softmax_scale, D);
  a.sl2e = a.scale * ctxattn::kLog2e;
  a.mask = CA_MASK_NONE;
  a.G = 1;
  a.c = c; a.acc = acc; a.phase = phase;
  a.o_cm = o; a.o_cm_bf16 = (o_dtype == CA_BF16); a.lse_cm = lse;
  a.sink_idx = sink_idx; a.sink_cnt = sink_cnt; a.sink_cap = sink_cap; a.key_offset = key_offset;
  CA_TRY(attach_workspace(a, dtype, workspace, workspace_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = attach_hop(a, hop, dtype, CA_MASK_NONE, s);
  if (e != hipSuccess) return hip_status(e, "ring_attn_const_max_step launch");
  e = mfma_step(dtype, D) ? ctxattn::launch_attn_bf16(a, true, s) : ctxattn::launch_attn_f32(a, true, dtype == CA_BF16, s);
  return hip_status(e, "ring_attn_const_max_step launch");
}

}  // namespace

extern "C" {

ca_status ring_attn_const_max_step(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs,
                                   int dtype, int B, int H, int Sq, int Sk, int D, float softmax_scale,
                                   const float* c, float* acc, int phase, void* o, int o_dtype, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return const_max_step_impl(q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale, c, acc, phase, o, o_dtype, lse,
                             workspace, workspace_bytes, nullptr, nullptr, 0, 0, stream);
}

ca_status ring_attn_const_max_step_hop(const void* q, ca_strides qs, const void* k, const void* v, ca_strides kvs,
                                       int dtype, int B, int H, int Sq, int Sk, int D, float softmax_scale,
                                       const float* c, float* acc, int phase, void* o, int o_dtype, float* lse,
                                       void* workspace, size_t workspace_bytes, void* hop_dst_k, void* hop_dst_v,
                                       const void* hop_src_k, const void* hop_src_v, size_t hop_bytes, void* stream) {
  const Hop hop{hop_dst_k, hop_dst_v, hop_src_k, hop_src_v, hop_bytes};
  CA_TRY(check_hop("ring_attn_const_max_step_hop", hop));
  return const_max_step_impl(q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale, c, acc, phase, o, o_dtype, lse,
                             workspace, workspace_bytes, nullptr, nullptr, 0, 0, stream, hop);
}

ca_status ring_attn_const_max_step_sinks(const void* q, ca_strides qs, const void* k, const void* v,
                                         ca_strides kvs, int dtype, int B, int H, int Sq, int Sk, int D,
                                         float softmax_scale, const float* c, float* acc, int phase, void* o,
                                         int o_dtype, float* lse, const int32_t* sink_idx, const int32_t* sink_cnt,
                                         int sink_cap, int64_t key_offset, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (dtype != CA_BF16 || D != 128)
    return fail(CA_ERR_UNSUPPORTED, "sink lists need the bf16 MFMA path (bf16, head_dim 128; got %s, %d)",
                dtype == CA_BF16 ? "bf16" : "fp32", D);
  if (sink_cap < 1 || sink_cap > 64) return fail(CA_ERR_UNSUPPORTED, "sink_cap must be in [1, 64] (got %d)", sink_cap);
  if (int64_t(B) * H * Sq > 0 && (!sink_idx || !sink_cnt)) return fail(CA_ERR_NULL, "sink_idx and sink_cnt are required");
  if (key_offset < 0) return fail(CA_ERR_SHAPE, "negative key_offset");
  return const_max_step_impl(q, qs, k, v, kvs, dtype, B, H, Sq, Sk, D, softmax_scale, c, acc, phase, o, o_dtype, lse,
                             workspace, workspace_bytes, sink_idx, sink_cnt, sink_cap, key_offset, stream);
}

ca_status const_max_sink_prologue(const void* k, int64_t chunk_stride, ca_strides ks, int dtype, int cp, int B,
                                  int S_local, int H, int D, float theta, int sink_cap, float* kmax_sq,
                                  float* kmax_sq_robust, float* knorm_sum, int32_t* sink_idx, int32_t* sink_cnt,
                                  void* stream) {
  CA_TRY(check_dtype(dtype));
  if (D <= 0 || D % 8 || D > 128) return fail(CA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in [8, 128]");
  if (cp < 0 || chunk_stride < 0) return fail(CA_ERR_SHAPE, "bad chunk count or stride");
  CA_TRY(check_bshd("k", k, ks, dtype, B, S_local, H, D));
  if (sink_cap < 1 || sink_cap > 64) return fail(CA_ERR_UNSUPPORTED, "sink_cap must be in [1, 64] (got %d)", sink_cap);
  if (H > 4096) return fail(CA_ERR_UNSUPPORTED, "at most 4096 heads");
  if (int64_t(cp) * S_local >= (int64_t(1) << 31)) return fail(CA_ERR_UNSUPPORTED, "ring too long for int32 key indices");
  if (int64_t(B) * H == 0) return hip_status(hipSuccess, "");
  if (!kmax_sq || !kmax_sq_robust || !knorm_sum || !sink_idx || !sink_cnt)
    return fail(CA_ERR_NULL, "kmax_sq, kmax_sq_robust, knorm_sum, sink_idx and sink_cnt are required");
  if (((chunk_stride * (dtype == CA_BF16 ? 2 : 4)) & 15)) return fail(CA_ERR_SHAPE, "chunk stride must keep rows 16-byte aligned");
  hipError_t e = ctxattn::launch_sink_prologue(k, chunk_stride, ks.b, ks.s, ks.h, dtype == CA_BF16, cp, B, S_local, H, D,
                                               theta, sink_cap, kmax_sq, knorm_sum, kmax_sq_robust, sink_idx, sink_cnt,
                                               static_cast<hipStream_t>(stream));
  return hip_status(e, "const_max_sink_prologue launch");
}

ca_status sink_attention_workspace_size(int B, int H, int D, int sink_cap, size_t* bytes) {
  if (!bytes) return fail(CA_ERR_NULL, "bytes is NULL");
  if (B < 0 || H < 0 || D <= 0 || sink_cap < 0) return fail(CA_ERR_SHAPE, "bad sizes");
  *bytes = size_t(2) * ((size_t(B) * sink_cap * H * D * 2 + 255) & ~size_t(255));
  g_err[0] = 0;
  return CA_OK;
}

ca_status sink_attention_partial(const void* q, ca_strides qs, const void* k, const void* v, int64_t chunk_stride,
                                 ca_strides kvs, int cp, int B, int H, int Sq, int S_local, int D, float softmax_scale,
                                 const int32_t* sink_idx, const int32_t* sink_cnt, int sink_cap, float* o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (D != 128) return fail(CA_ERR_UNSUPPORTED, "bf16 attention supports head_dim 128 only (got %d)", D);
  if (sink_cap < 1 || sink_cap > 64) return fail(CA_ERR_UNSUPPORTED, "sink_cap must be in [1, 64] (got %d)", sink_cap);
  if (cp < 0 || chunk_stride < 0 || Sq < 0) return fail(CA_ERR_SHAPE, "bad sizes");
  CA_TRY(check_bshd("q", q, qs, CA_BF16, B, Sq, H, D));
  CA_TRY(check_bshd("k", k, kvs, CA_BF16, B, S_local, H, D));
  CA_TRY(check_bshd("v", v, kvs, CA_BF16, B, S_local, H, D));
  if (int64_t(B) * H * Sq == 0) return hip_status(hipSuccess, "");
  if (!o || !lse || !sink_idx || !sink_cnt) return fail(CA_ERR_NULL, "o, lse, sink_idx and sink_cnt are required");
  if (!aligned16(o)) return fail(CA_ERR_SHAPE, "o must be 16-byte aligned");
  size_t need = 0;
  sink_attention_workspace_size(B, H, D, sink_cap, &need);
  if (!workspace || workspace_bytes < need)
    return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(CA_ERR_SHAPE, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* kg = static_cast<char*>(workspace);
  char* vg = kg + need / 2;
  hipError_t e = ctxattn::launch_sink_gather(k, v, chunk_stride, kvs.b, kvs.s, kvs.h, B, S_local, H, sink_cap, sink_idx,
                                             sink_cnt, kg, vg, s);
  if (e != hipSuccess) return hip_status(e, "sink gather launch");
  ctxattn::AttnArgs a{};
  a.q = q; a.qsb = qs.b; a.qss = qs.s; a.qsh = qs.h;
  a.k = kg; a.v = vg; a.ksb = int64_t(sink_cap) * H * D; a.kss = int64_t(H) * D; a.ksh = D;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = sink_cap; a.D = D;
  a.scale = resolve_scale(softmax_scale, D);
  a.sl2e = a.scale * ctxattn::kLog2e;
  a.mask = CA_MASK_NONE;
  a.G = 1;
  a.o = o; a.lse = lse;
  a.sk_of_bh = sink_cnt;
  return hip_status(ctxattn::launch_attn_bf16(a, false, s), "sink_attention_partial launch");
}

ca_status lse_merge(int n, const float* o_parts, const float* lse_parts, int64_t rows, int D, void* o_out,
                    int o_dtype, float* lse_out, void* stream) {
  if (n < 1) return fail(CA_ERR_SHAPE, "n must be >= 1 (got %d)", n);
  if (rows < 0) return fail(CA_ERR_SHAPE, "negative rows");
  if (D != 64 && D != 128) return fail(CA_ERR_UNSUPPORTED, "lse_merge supports D 64 or 128 (got %d)", D);
  CA_TRY(check_dtype(o_dtype));
  if (rows == 0) return hip_status(hipSuccess, "");
  if (!o_parts || !lse_parts || !o_out) return fail(CA_ERR_NULL, "o_parts, lse_parts and o_out are required");
  if (!aligned16(o_parts) || !aligned16(o_out)) return fail(CA_ERR_SHAPE, "o_parts and o_out must be 16-byte aligned");
  const char* op = static_cast<const char*>(static_cast<const void*>(o_parts));
  const char* oo = static_cast<const char*>(o_out);
  const size_t in_bytes = size_t(n) * size_t(rows) * D * sizeof(float);
  const size_t out_bytes = size_t(rows) * D * (o_dtype == CA_BF16 ? 2 : 4);
  if (oo < op + in_bytes && op < oo + out_bytes) return fail(CA_ERR_SHAPE, "o_out overlaps o_parts");
  hipError_t e = ctxattn::launch_lse_merge(n, o_parts, lse_parts, rows, D, o_out, o_dtype == CA_BF16, lse_out,
                                           static_cast<hipStream_t>(stream));
  return hip_status(e, "lse_merge launch");
}

ca_status dcp_decode_workspace_size(int B, int Hq, int D, int block_size, int max_blocks, size_t* bytes) {
  if (!bytes) return fail(CA_ERR_NULL, "bytes is NULL");
  if (B < 0 || Hq < 0 || D <= 0 || block_size <= 0 || max_blocks < 0) return fail(CA_ERR_SHAPE, "bad sizes");
  *bytes = ctxattn::decode_workspace_bytes(B, Hq, D, block_size, max_blocks);
  g_err[0] = 0;
  return CA_OK;
}

}  // extern "C"

namespace {

// Shared validation and launch of both decode entry points. local_lens != NULL: resident
// counts given; otherwise prior_lens, k_cur, v_cur, rank, world, interleave describe the
// current-token form.
ca_status decode_launch(const char* name, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* local_lens, const int32_t* prior_lens,
                        const void* k_cur, const void* v_cur, int rank, int world, int interleave, int B, int Hq,
                        int Hkv, int D, int block_size, int max_blocks, int num_blocks, float softmax_scale, float* o,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_blocks < 0 || num_blocks < 0) return fail(CA_ERR_SHAPE, "bad sizes");
  if (D != 64 && D != 128) return fail(CA_ERR_UNSUPPORTED, "decode supports head_dim 64 or 128 (got %d)", D);
  if (block_size != 16) return fail(CA_ERR_UNSUPPORTED, "decode supports block_size 16 only (got %d)", block_size);
  if (Hq % Hkv) return fail(CA_ERR_UNSUPPORTED, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(CA_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
  if (B > 65535 || Hkv > 65535) return fail(CA_ERR_UNSUPPORTED, "at most 65535 sequences and KV heads");
  if (!local_lens) {
    if (world < 1 || rank < 0 || rank >= world)
      return fail(CA_ERR_SHAPE, "rank %d outside a DCP group of %d", rank, world);
    if (interleave < 1 || block_size % interleave)
      return fail(CA_ERR_UNSUPPORTED, "interleave (%d) must divide block_size (%d)", interleave, block_size);
    if (int64_t(block_size) * world > (int64_t(1) << 30)) return fail(CA_ERR_UNSUPPORTED, "DCP group too large");
  }
  if (B == 0) return hip_status(hipSuccess, "");
  if (!q || !o || !lse || (!local_lens && !prior_lens))
    return fail(CA_ERR_NULL, "q, o, lse and the sequence lengths are required");
  if (!local_lens && (!k_cur || !v_cur)) return fail(CA_ERR_NULL, "k_cur and v_cur are required");
  // an empty pool has no block to stand in for missing ones: a caller with no resident
  // blocks passes max_blocks = 0
  if (max_blocks > 0 && num_blocks == 0)
    return fail(CA_ERR_SHAPE, "the block table has %d entries per sequence but the pool has no block", max_blocks);
  if (max_blocks > 0 && (!k_pool || !v_pool || !block_table))
    return fail(CA_ERR_NULL, "k_pool, v_pool and block_table are required");
  if (!aligned16(q) || !aligned16(o) || (k_pool && !aligned16(k_pool)) || (v_pool && !aligned16(v_pool)) ||
      (k_cur && !aligned16(k_cur)) || (v_cur && !aligned16(v_cur)))
    return fail(CA_ERR_SHAPE, "q, o, the pools and the current K/V must be 16-byte aligned");
  const size_t need = ctxattn::decode_workspace_bytes(B, Hq, D, block_size, max_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(CA_ERR_SHAPE, "workspace must be 16-byte aligned");
  const int64_t max_tokens = int64_t(max_blocks) * block_size;
  const int64_t max_splits64 = ctxattn::decode_grid_splits(max_tokens);
  if (max_splits64 > 65535) return fail(CA_ERR_UNSUPPORTED, "too many blocks per sequence");
  const int max_splits = int(max_splits64);
  ctxattn::DecodeArgs a{};
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool; a.block_table = block_table; a.local_lens = local_lens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.block_size = block_size; a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.scale = resolve_scale(softmax_scale, D);
  a.sl2e = a.scale * ctxattn::kLog2e;
  a.o = o; a.lse = lse;
  a.max_splits = max_splits;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + int64_t(B) * Hq * (max_splits > 0 ? max_splits : 1) * D;
  if (!local_lens) {
    a.prior_lens = prior_lens; a.k_cur = k_cur; a.v_cur = v_cur;
    a.rank = rank; a.world = world; a.interleave = interleave;
  }
  hipError_t e = ctxattn::launch_dcp_decode(a, static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

}  // namespace

extern "C" {

ca_status dcp_decode_partial(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                             const int32_t* local_lens, int B, int Hq, int Hkv, int D, int block_size, int max_blocks,
                             int num_blocks, float softmax_scale, float* o, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (B > 0 && !local_lens) return fail(CA_ERR_NULL, "local_lens is required");
  return decode_launch("dcp_decode_partial launch", q, k_pool, v_pool, block_table, local_lens, nullptr, nullptr,
                       nullptr, 0, 1, 1, B, Hq, Hkv, D, block_size, max_blocks, num_blocks, softmax_scale, o, lse,
                       workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch of dcp_decode_partial_noalloc: the split partials that dcp_decode_partial keeps in
// its caller's workspace. One copy per GPU the library runs on, held until the process ends.
// In host code `scratch` is only a stand-in for the symbol: kernels and copies use the
// device address that hipGetSymbolAddress gives for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(80) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per device (with that
// device current) and kept.
ca_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_ERR_UNSUPPORTED, "device %d outside the first %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CA_OK;
}

}  // namespace

extern "C" {

ca_status dcp_decode_partial_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* local_lens, int B, int Hq, int Hkv,
                                     int D, int block_size, int max_blocks, int num_blocks, float softmax_scale,
                                     float* o, float* lse, void* stream) {
  if (B > 0 && !local_lens) return fail(CA_ERR_NULL, "local_lens is required");
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (B > 0 && Hq > 0 && Hkv > 0 && D > 0 && block_size > 0 && max_blocks >= 0) {
    const size_t need = ctxattn::decode_workspace_bytes(B, Hq, D, block_size, max_blocks);
    if (need > kNoAllocScratchBytes)
      return fail(CA_ERR_WORKSPACE,
                  "dcp_decode_partial_noalloc: these sizes need %zu bytes of scratch, above its fixed %zu "
                  "(B * Hq * ceil(max_blocks * block_size / 1024) * (D + 1) * 4 bytes); use dcp_decode_partial "
                  "with a workspace", need, kNoAllocScratchBytes);
    CA_TRY(scratch_of_current_device(&ws));
    ws_bytes = kNoAllocScratchBytes;
  }
  return decode_launch("dcp_decode_partial_noalloc launch", q, k_pool, v_pool, block_table, local_lens, nullptr,
                       nullptr, nullptr, 0, 1, 1, B, Hq, Hkv, D, block_size, max_blocks, num_blocks, softmax_scale, o,
                       lse, ws, ws_bytes, stream);
}

ca_status dcp_decode_partial_active(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                                    const int32_t* prior_lens, const void* k_cur, const void* v_cur, int rank,
                                    int world, int interleave, int B, int Hq, int Hkv, int D, int block_size,
                                    int max_blocks, int num_blocks, float softmax_scale, float* o, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && !prior_lens) return fail(CA_ERR_NULL, "prior_lens is required");
  return decode_launch("dcp_decode_partial_active launch", q, k_pool, v_pool, block_table, nullptr, prior_lens,
                       k_cur, v_cur, rank, world, interleave, B, Hq, Hkv, D, block_size, max_blocks, num_blocks,
                       softmax_scale, o, lse, workspace, workspace_bytes, stream);
}

ca_status segmented_attention_workspace_size(int Hq, int Hkv, int S, int D, int prior_tokens, size_t* bytes) {
  if (!bytes) return fail(CA_ERR_NULL, "bytes is NULL");
  if (Hq <= 0 || Hkv <= 0 || S < 0 || D <= 0 || prior_tokens < 0) return fail(CA_ERR_SHAPE, "bad sizes");
  *bytes = ctxattn::segmented_workspace_bytes(Hq, Hkv, S, D, prior_tokens);
  g_err[0] = 0;
  return CA_OK;
}

ca_status segmented_attention_partial(const void* q, ca_strides qs, const void* k_cur, const void* v_cur,
                                      ca_strides kvs, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, int max_blocks, int num_blocks, int prior_tokens,
                                      int rank, int world, int interleave, int Hq, int Hkv, int S, int S_local, int D,
                                      float softmax_scale, float* o, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (D != 128) return fail(CA_ERR_UNSUPPORTED, "segmented attention supports head_dim 128 only (got %d)", D);
  if (Hq <= 0 || Hkv <= 0 || S < 0 || S_local < 0 || prior_tokens < 0 || max_blocks < 0 || num_blocks < 0)
    return fail(CA_ERR_SHAPE, "bad sizes");
  if (Hq % Hkv) return fail(CA_ERR_UNSUPPORTED, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Hkv > 16) return fail(CA_ERR_UNSUPPORTED, "at most 16 KV heads (got %d)", Hkv);
  if (world < 1 || rank < 0 || rank >= world) return fail(CA_ERR_SHAPE, "rank %d outside a DCP group of %d", rank, world);
  if (interleave < 1) return fail(CA_ERR_SHAPE, "interleave must be positive");
  if (int64_t(world) * interleave > (int64_t(1) << 30)) return fail(CA_ERR_UNSUPPORTED, "DCP group too large");
  if (S % (world * interleave))
    return fail(CA_ERR_SHAPE, "chunk length %d is not a multiple of world * interleave = %d", S, world * interleave);
  if (S_local != S / world) return fail(CA_ERR_SHAPE, "S_local (%d) must be S / world (%d)", S_local, S / world);
  if (prior_tokens > int64_t(max_blocks) * 16)
    return fail(CA_ERR_SHAPE, "prior_tokens %d exceeds the block table (%d blocks of 16)", prior_tokens, max_blocks);
  CA_TRY(check_bshd("q", q, qs, CA_BF16, 1, S, Hq, D));
  CA_TRY(check_bshd("k_cur", k_cur, kvs, CA_BF16, 1, S_local, Hkv, D));
  CA_TRY(check_bshd("v_cur", v_cur, kvs, CA_BF16, 1, S_local, Hkv, D));
  if (S == 0) return hip_status(hipSuccess, "");
  if (!o || !lse) return fail(CA_ERR_NULL, "o and lse are required");
  if (!aligned16(o)) return fail(CA_ERR_SHAPE, "o must be 16-byte aligned");
  if (prior_tokens > 0) {
    if (!k_cache || !v_cache || !block_table) return fail(CA_ERR_NULL, "k_cache, v_cache and block_table are required");
    if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(CA_ERR_SHAPE, "the caches must be 16-byte aligned");
  }
  const size_t need = ctxattn::segmented_workspace_bytes(Hq, Hkv, S, D, prior_tokens);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(CA_ERR_SHAPE, "workspace must be 16-byte aligned");
  ctxattn::SegmentedArgs g{};
  g.q = q; g.qss = qs.s; g.qsh = qs.h;
  g.k_cur = k_cur; g.v_cur = v_cur; g.kss = kvs.s; g.ksh = kvs.h;
  g.k_cache = k_cache; g.v_cache = v_cache; g.block_table = block_table;
  g.num_blocks = num_blocks; g.prior = prior_tokens;
  g.rank = rank; g.world = world; g.interleave = interleave;
  g.Hq = Hq; g.Hkv = Hkv; g.S = S; g.S_local = S_local;
  g.scale = resolve_scale(softmax_scale, D);
  g.o = o; g.lse = lse; g.ws = workspace;
  return hip_status(ctxattn::launch_segmented(g, static_cast<hipStream_t>(stream)), "segmented_attention_partial launch");
}

ca_status kv_chunk_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v, size_t bytes, void* stream) {
  if (bytes == 0) return hip_status(hipSuccess, "");
  if (!dst_k || !dst_v || !src_k || !src_v) return fail(CA_ERR_NULL, "all four chunk pointers are required");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v) || (bytes & 15))
    return fail(CA_ERR_SHAPE, "kv_chunk_copy: pointers must be 16-byte aligned and bytes a multiple of 16");
  return hip_status(ctxattn::launch_kv_copy(dst_k, dst_v, src_k, src_v, bytes, static_cast<hipStream_t>(stream)),
                    "kv_chunk_copy");
}

}  // extern "C"
