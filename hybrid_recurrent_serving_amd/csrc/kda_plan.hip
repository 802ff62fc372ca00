// Device-side checkpoint plan (kda_ckpt_plan_device).
//
// The checkpoint table of interval retention ("Kimi K3 + vLLM: Inside the
// Day-0 Production Integration", section "Agentic Serving: Cache Retention
// Across Turns") built in stream order from device cu_seqlens, so that a
// serving loop never copies batch metadata to the host: that page's section
// "Separate Prefill/Decode Code Paths" reports metadata preparation as a
// bottleneck at batch 1 and replaces chains of small host-driven operations
// with dedicated kernels.  Two launches whose grids depend only on host
// sizes (n_seq, cap), no allocation, no synchronisation: capturable in a HIP
// graph.
//
//   plan_scan_kernel  one workgroup: per-sequence counts and their exclusive
//                     prefix sum (ckpt_cu), the total
//   plan_fill_kernel  one thread per table entry i < cap: the sequence that
//                     owns entry i (binary search in ckpt_cu), its position
//                     and its slot from the free list

#include "kda_internal.h"

namespace kda {
namespace plan {

constexpr int SCAN_T = 1024;
constexpr int FILL_T = 256;
constexpr int FILL_MAX_BLOCKS = 2048;
constexpr int64_t I32_MAX = 0x7fffffffLL;

// Sequence s as the prefill sees it: token range clamped into [0, T_tot],
// start position clamped at 0.
struct SeqSpan {
  int64_t len, start;
};

__device__ inline SeqSpan seq_span(const PlanParams& p, int s) {
  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  int64_t st = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (st < 0) st = 0;
  return {eos - bos, st};
}

// checkpoints of a sequence at absolute positions [st, st + len): the
// multiples of the interval strictly inside
__device__ inline int64_t seq_count(const PlanParams& p, int s) {
  const SeqSpan sp = seq_span(p, s);
  return sp.len > 0 ? (sp.start + sp.len - 1) / p.interval - sp.start / p.interval : 0;
}

__global__ void __launch_bounds__(SCAN_T) plan_scan_kernel(const PlanParams p) {
  __shared__ int64_t wsum[SCAN_T / 64];
  __shared__ int64_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    p.ckpt_cu[0] = 0;
    carry_s = 0;
  }
  __syncthreads();
  for (int base = 0; base < p.n_seq; base += SCAN_T) {
    const int s = base + tid;
    const int64_t c = s < p.n_seq ? seq_count(p, s) : 0;
    // inclusive scan inside the wave, then over the wave totals
    int64_t x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int64_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int64_t incl = before + x;
    if (s < p.n_seq) p.ckpt_cu[s + 1] = static_cast<int32_t>(incl < I32_MAX ? incl : I32_MAX);
    __syncthreads();   // every wave has read carry_s and wsum
    if (tid == SCAN_T - 1) carry_s = incl;
    __syncthreads();
  }
  if (tid == 0 && p.n_total) p.n_total[0] = static_cast<int32_t>(carry_s < I32_MAX ? carry_s : I32_MAX);
}

__global__ void __launch_bounds__(FILL_T) plan_fill_kernel(const PlanParams p) {
  const int64_t total = p.ckpt_cu[p.n_seq];
  const int64_t lim = total < p.cap ? total : p.cap;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * FILL_T;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * FILL_T + threadIdx.x; i < lim; i += stride) {
    // the sequence s with ckpt_cu[s] <= i < ckpt_cu[s + 1]
    int a = 0, b = p.n_seq;
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (p.ckpt_cu[mid] <= i) a = mid; else b = mid;
    }
    if (p.ckpt_pos) {
      const SeqSpan sp = seq_span(p, a);
      const int64_t pos = (sp.start / p.interval + 1 + (i - p.ckpt_cu[a])) * p.interval;
      p.ckpt_pos[i] = static_cast<int32_t>(pos < I32_MAX ? pos : I32_MAX);
    }
    if (p.ckpt_slot) p.ckpt_slot[i] = i < p.n_free ? p.free_slots[i] : -1;
  }
}

}  // namespace plan

int launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan::plan_scan_kernel, dim3(1), dim3(plan::SCAN_T), 0, stream, p);
  if (p.cap > 0 && p.n_seq > 0 && (p.ckpt_pos || p.ckpt_slot)) {
    int64_t blocks = (static_cast<int64_t>(p.cap) + plan::FILL_T - 1) / plan::FILL_T;
    blocks = blocks < plan::FILL_MAX_BLOCKS ? blocks : plan::FILL_MAX_BLOCKS;
    hipLaunchKernelGGL(plan::plan_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(plan::FILL_T), 0,
                       stream, p);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KDA_OK : fail(KDA_ERR_HIP, "ckpt_plan_device launch: %s", hipGetErrorString(e));
}

}  // namespace kda
