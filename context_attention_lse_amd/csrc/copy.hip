// The ring's K/V hop on one device: a plain streaming copy of one K chunk and one V
// chunk in a single launch (kernel reference page, Implementation, ring loop: the next
// chunk moves while the current step computes).
//
// HBM-bound: every byte is read once and written once with 16-byte accesses. The grid is
// 64 workgroups of 1024 threads, each walking the two buffers with a grid stride and 128 KB
// in flight: a hop issued beside an attention step then holds few CUs at a time (a step's
// workgroup fills its CU, so hop workgroups take CUs between the step's workgroups). In the
// striped causal ring this form hid 18% more of the hop than 1024 workgroups of 256 threads
// (0.78 against 0.95 ms of hop cost per two passes); alone it copies more slowly.
#include "internal.hpp"

namespace ctxattn {
namespace {

constexpr int NT = 1024;
constexpr int UNROLL = 8;
constexpr int MAX_GRID = 64;

__global__ __launch_bounds__(NT) void kv_copy_kernel(floatx4* __restrict__ dk, floatx4* __restrict__ dv,
                                                     const floatx4* __restrict__ sk,
                                                     const floatx4* __restrict__ sv, int64_t units) {
  // units: 16-byte vectors per buffer. Work item u < units copies K, u >= units copies V.
  const int64_t total = 2 * units;
  const int64_t stride = int64_t(gridDim.x) * NT * UNROLL;
  for (int64_t base = int64_t(blockIdx.x) * NT * UNROLL + threadIdx.x; base < total; base += stride) {
    floatx4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + int64_t(u) * NT;
      if (i < total) v[u] = __builtin_nontemporal_load(i < units ? sk + i : sv + (i - units));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + int64_t(u) * NT;
      if (i < total) __builtin_nontemporal_store(v[u], i < units ? dk + i : dv + (i - units));
    }
  }
}

}  // namespace

hipError_t launch_kv_copy(void* dk, void* dv, const void* sk, const void* sv, size_t bytes, hipStream_t s) {
  const int64_t units = int64_t(bytes / 16);
  const int64_t per_wg = int64_t(NT) * UNROLL;
  const int64_t want = (2 * units + per_wg - 1) / per_wg;
  const int grid = int(want < MAX_GRID ? want : MAX_GRID);
  hipLaunchKernelGGL(kv_copy_kernel, dim3(grid), dim3(NT), 0, s, static_cast<floatx4*>(dk),
                     static_cast<floatx4*>(dv), static_cast<const floatx4*>(sk),
                     static_cast<const floatx4*>(sv), units);
  return hipGetLastError();
}

}  // namespace ctxattn
