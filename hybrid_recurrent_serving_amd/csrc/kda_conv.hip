// Short causal depthwise convolution with carried state (the KDA layer's
// q/k/v convolution; "Kimi K3 + vLLM: Inside the Day-0 Production
// Integration", sections "Kimi Delta Attention: When Prefix Caching Meets
// Recurrent State" and "Separate Prefill/Decode Code Paths").
//
//   y[t, c] = bias[c] + sum_{j<W} w[c, j] * xbar[t - (W-1) + j, c]   (+ SiLU)
//
// xbar = carried state (last W-1 raw inputs, oldest first) ++ tokens.
//
// Pure streaming: 2 x sizeof(T) bytes per element plus the state.  Each
// thread owns VEC = 16 / sizeof(T) adjacent channels (one 16-byte vector per
// token row), so a 256-thread workgroup reads 4 KiB (bf16) of one token row
// per load instruction.
//
// Work items (blockIdx.x):
//  * "head" item s < n_seq: the first min(len, W-1) tokens of sequence s
//    (those that need the carried history) AND the new state.  Only this
//    item reads the source slot and only it writes the destination slot, so
//    updating a slot in place (src == dst) is race free.
//  * "body" item n_seq + b: packed tokens [b*TT, (b+1)*TT), skipping each
//    sequence's first W-1 tokens.  These only read x, with a sliding window
//    of the previous W-1 rows in registers.

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// tokens per body item: 8 rows of outputs from 8 + W - 1 rows of input per
// lane (conv + SiLU at 140,625 tokens x 6,144 channels: 620 us, against 627
// us with 16 rows, 627 with 32, 630 with 6 and 677 with 4; fewer loads in
// flight per lane stream better, down to where the per-item set-up and the
// W - 1 extra rows read from L2 outweigh it)
constexpr int CONV_TT = 8;
constexpr int CONV_THREADS = 256;

// Outputs and new histories are written once and not read again by this
// kernel: non-temporal stores (the conv at prefill scale ran 4% faster with
// them: 631 us against 659 us for 140,625 tokens x 6,144 channels).  Of a
// body tile's rows, the W-1 before its own are the previous tile's last rows
// (found in L2) and its own last W-1 rows are the next tile's first: those
// keep the default policy, the rows in between are read non-temporally
// (625 us against 633 us; every row non-temporal: 666 us).
typedef __attribute__((ext_vector_type(4))) uint32_t nt4u;

template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void cvt(const uint4& t, float (&x)[8]) {
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void ld(const bf16_t* p, float (&x)[8]) {
    uint4 t = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void st(bf16_t* p, const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    const nt4u v = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<nt4u*>(p));
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void cvt(const uint4& t, float (&x)[4]) {
    x[0] = __uint_as_float(t.x); x[1] = __uint_as_float(t.y);
    x[2] = __uint_as_float(t.z); x[3] = __uint_as_float(t.w);
  }
  __device__ static __forceinline__ void ld(const float* p, float (&x)[4]) { io<float>::ld4(p, x); }
  __device__ static __forceinline__ void st(float* p, const float (&x)[4]) { st4_stream(p, x); }
};

// NB consecutive 16-byte vectors starting at p (16-byte aligned) <-> floats
template <typename T, int NB>
__device__ __forceinline__ void ld_blocks(const T* p, float (&x)[NB * Vec16<T>::N]) {
  constexpr int V = Vec16<T>::N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float t[V];
    Vec16<T>::ld(p + b * V, t);
#pragma unroll
    for (int i = 0; i < V; ++i) x[b * V + i] = t[i];
  }
}

template <typename T, int NB>
__device__ __forceinline__ void st_blocks(T* p, const float (&x)[NB * Vec16<T>::N]) {
  constexpr int V = Vec16<T>::N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float t[V];
#pragma unroll
    for (int i = 0; i < V; ++i) t[i] = x[b * V + i];
    Vec16<T>::st(p + b * V, t);
  }
}

__device__ __forceinline__ float conv_finish(float acc, int act) {
  return act == 1 ? silu_fast(acc) : acc;
}

// Per-head L2 normalisation of one output row (NL > 0 only): the NL = norm_d
// / V threads that hold one head's channels are adjacent lanes of one wave
// (their group starts at a multiple of NL, which divides 64), so the sum of
// squares closes over them by group_sum.  NL is a template argument so that
// the reduction has no branches and the rows of a tile overlap.  Channels at
// or past norm_channels (the v block) keep their values.

template <int NL, int V>
__device__ __forceinline__ void norm_row(float (&out)[V], const ConvParams& p, int64_t c0) {
  if constexpr (NL > 0) {
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) ss = fmaf(out[v], out[v], ss);
    ss = group_sum<NL>(ss);
    const float inv = 1.f / sqrtf(ss + p.norm_eps);
    const bool qk = c0 < p.norm_channels;
#pragma unroll
    for (int v = 0; v < V; ++v) out[v] = qk ? out[v] * inv : out[v];
  }
}

template <typename T, int W, int NL>
__global__ void __launch_bounds__(CONV_THREADS) conv_kernel(const ConvParams p) {
  constexpr bool NORM = NL > 0;
  constexpr int V = Vec16<T>::N;
  constexpr int HIST = W - 1;
  // Workgroups go to the 8 XCDs round robin (x fastest); item indices are
  // handed out so that each XCD takes one contiguous run of them: the tile
  // after a tile then runs on the same XCD, and the W-1 rows it reads ahead
  // of its own are still in that XCD's L2.  A bijection of [0, gridDim.x).
  int item;
  {
    const int nb = static_cast<int>(gridDim.x);
    const int x8 = static_cast<int>(blockIdx.x) % 8, s8 = static_cast<int>(blockIdx.x) / 8;
    const int q = nb / 8, r = nb % 8;
    item = x8 * q + (x8 < r ? x8 : r) + s8;
  }
  const int64_t c0 = (static_cast<int64_t>(blockIdx.y) * CONV_THREADS + threadIdx.x) * V;
  // threads past the last channel stay for the workgroup barrier of body items
  const bool active = c0 < p.C;
  if (!active && item < p.n_seq) return;
  const T* xb = static_cast<const T*>(p.x);
  T* yb = static_cast<T*>(p.y);

  // taps of my channels: wt[j][i] = w[c0 + i, j]; the V*W taps are
  // contiguous (W 16-byte vectors)
  float wt[W][V];
  {
    float flat[W * V];
    ld_blocks<T, W>(static_cast<const T*>(p.w) + (active ? c0 : 0) * W, flat);
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < W; ++j) wt[j][i] = flat[i * W + j];
  }
  float bias[V];
#pragma unroll
  for (int i = 0; i < V; ++i) bias[i] = p.bias ? io<T>::ld(static_cast<const T*>(p.bias) + (active ? c0 : 0) + i) : 0.f;

  if (item < p.n_seq) {
    // ---------------- head item: tokens that need the history + new state
    const int s = item;
    int64_t bos = p.cu[s], eos = p.cu[s + 1];
    bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
    eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
    const int64_t len = eos - bos;
    const int src = p.src_slot[s];
    const int dst = p.dst_slot[s];
    const bool has_src = src >= 0 && src < p.n_slots;
    const bool has_dst = dst >= 0 && dst < p.n_slots;
    // xh[j] = xbar[j] for j < 2*HIST: history then the first HIST tokens
    float xh[2 * HIST][V];
    if (has_src) {
      // the V channels' histories are V*HIST contiguous elements (HIST vectors)
      float flat[HIST * V];
      ld_blocks<T, HIST>(static_cast<const T*>(p.pool) + (static_cast<int64_t>(src) * p.C + c0) * HIST, flat);
#pragma unroll
      for (int j = 0; j < HIST; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) xh[j][i] = flat[i * HIST + j];
    } else {
#pragma unroll
      for (int j = 0; j < HIST; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) xh[j][i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < HIST; ++j) {
      if (j < len) {
        Vec16<T>::ld(xb + (bos + j) * p.x_stride + c0, xh[HIST + j]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) xh[HIST + j][i] = 0.f;
      }
    }
    // new state = xbar[a .. a + HIST), a = advance length clamped to [0, len]
    int64_t a = p.adv ? static_cast<int64_t>(p.adv[s]) : len;
    a = a < 0 ? 0 : (a > len ? len : a);
    float ns[HIST][V];
#pragma unroll
    for (int j = 0; j < HIST; ++j) {
      const int64_t idx = a + j;
      if (idx < 2 * HIST) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float val = 0.f;
#pragma unroll
          for (int q = 0; q < 2 * HIST; ++q) val = (q == idx) ? xh[q][i] : val;
          ns[j][i] = val;
        }
      } else {
        Vec16<T>::ld(xb + (bos + idx - HIST) * p.x_stride + c0, ns[j]);
      }
    }
    // outputs of the first min(len, HIST) tokens
#pragma unroll
    for (int t = 0; t < HIST; ++t) {
      if (t < len) {
        float out[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float acc = bias[i];
#pragma unroll
          for (int j = 0; j < W; ++j) acc = fmaf(wt[j][i], xh[t + j][i], acc);
          out[i] = conv_finish(acc, p.act);
        }
        norm_row<NL, V>(out, p, c0);
        Vec16<T>::st(yb + (bos + t) * p.y_stride + c0, out);
      }
    }
    if (has_dst) {
      float flat[HIST * V];
#pragma unroll
      for (int j = 0; j < HIST; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) flat[i * HIST + j] = ns[j][i];
      st_blocks<T, HIST>(static_cast<T*>(p.pool) + (static_cast<int64_t>(dst) * p.C + c0) * HIST, flat);
    }
    return;
  }

  // ---------------- body item: packed tokens [t0, t1)
  // Tokens at position >= W-1 inside their sequence (the others belong to the
  // head item).  The tile's rows and the W-1 rows before it are loaded at
  // once (independent 16-byte loads), then every output is formed from
  // registers.
  const int64_t t0 = static_cast<int64_t>(item - p.n_seq) * CONV_TT;
  if (t0 >= p.T_tot) return;
  const int64_t t1 = t0 + CONV_TT < p.T_tot ? t0 + CONV_TT : p.T_tot;
  // sequence containing t0: the last s with cu[s] <= t0
  int lo = 0, hi = p.n_seq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu[mid] <= t0) lo = mid; else hi = mid;
  }
  // the boundaries cu[lo .. lo + CONV_THREADS) in LDS, then the start of
  // each tile token's sequence (or "skip" when the token is outside every
  // sequence or among its sequence's first W-1 tokens)
  __shared__ int32_t cus[CONV_THREADS];
  __shared__ int32_t tok_ok[CONV_TT];
  if (lo + static_cast<int>(threadIdx.x) <= p.n_seq) cus[threadIdx.x] = p.cu[lo + threadIdx.x];
  __syncthreads();
  if (threadIdx.x < CONV_TT) {
    const int64_t t = t0 + threadIdx.x;
    auto cu_at = [&](int i) -> int64_t { return i - lo < CONV_THREADS ? cus[i - lo] : p.cu[i]; };
    int a = lo, b = p.n_seq;     // cu[a] <= t; the answer lies in [a, b)
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (cu_at(mid) <= t) a = mid; else b = mid;
    }
    const int64_t bos = cu_at(a), eos = cu_at(a + 1);
    tok_ok[threadIdx.x] = (t < t1 && t >= bos && t < eos && t - bos >= HIST) ? 1 : 0;
  }
  __syncthreads();
  // a tile whose tokens all belong to head items (one-token sequences, as in
  // a decode batch) has nothing to form: no loads
  int any_ok = 0;
#pragma unroll
  for (int i = 0; i < CONV_TT; ++i) any_ok |= tok_ok[i];
  if (!active || !any_ok) return;
  uint4 raw[HIST + CONV_TT];
#pragma unroll
  for (int j = 0; j < HIST + CONV_TT; ++j) {
    const int64_t row = t0 - HIST + j;
    raw[j] = make_uint4(0, 0, 0, 0);
    if (row >= 0 && row < t1) {
      if (j >= HIST && j < CONV_TT) {
        const nt4u v = __builtin_nontemporal_load(reinterpret_cast<const nt4u*>(xb + row * p.x_stride + c0));
        raw[j] = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
        raw[j] = *reinterpret_cast<const uint4*>(xb + row * p.x_stride + c0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CONV_TT; ++i) {
    // the normalised form computes every row (the group reductions want all
    // lanes, and rows without branches overlap) and stores the valid ones
    if (!NORM && !tok_ok[i]) continue;
    float out[V];
#pragma unroll
    for (int v = 0; v < V; ++v) out[v] = bias[v];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      float xr[V];
      Vec16<T>::cvt(raw[i + j], xr);
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = fmaf(wt[j][v], xr[v], out[v]);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) out[v] = conv_finish(out[v], p.act);
    norm_row<NL, V>(out, p, c0);
    if (!NORM || tok_ok[i]) Vec16<T>::st(yb + (t0 + i) * p.y_stride + c0, out);
  }
}

template <typename T, int W>
static int launch_conv_t(const ConvParams& p, hipStream_t stream) {
  constexpr int V = 16 / sizeof(T);
  const int64_t groups = (p.C + V - 1) / V;
  dim3 grid(static_cast<uint32_t>(p.n_seq + p.n_tiles),
            static_cast<uint32_t>((groups + CONV_THREADS - 1) / CONV_THREADS));
  if (p.norm_d > 0) {
    // the normalised form is built for the widths the fused paths take and
    // the head sizes 16 .. 128 (groups of norm_d / V lanes)
    if constexpr (W <= 4) {
      switch (p.norm_d / V) {
        case 2: if constexpr (V == 8) { hipLaunchKernelGGL((conv_kernel<T, W, 2>), grid, dim3(CONV_THREADS), 0, stream, p); break; }
                return fail(KDA_ERR_UNSUPPORTED, "conv norm group of 2 lanes (fp32)");
        case 4: hipLaunchKernelGGL((conv_kernel<T, W, 4>), grid, dim3(CONV_THREADS), 0, stream, p); break;
        case 8: hipLaunchKernelGGL((conv_kernel<T, W, 8>), grid, dim3(CONV_THREADS), 0, stream, p); break;
        case 16: hipLaunchKernelGGL((conv_kernel<T, W, 16>), grid, dim3(CONV_THREADS), 0, stream, p); break;
        case 32: if constexpr (V == 4) { hipLaunchKernelGGL((conv_kernel<T, W, 32>), grid, dim3(CONV_THREADS), 0, stream, p); break; }
                 return fail(KDA_ERR_UNSUPPORTED, "conv norm group of 32 lanes (bf16)");
        default: return fail(KDA_ERR_UNSUPPORTED, "conv norm: head size %d", p.norm_d);
      }
    } else {
      return fail(KDA_ERR_UNSUPPORTED, "conv with q/k normalisation: W = %d (2..4)", W);
    }
  } else {
    hipLaunchKernelGGL((conv_kernel<T, W, 0>), grid, dim3(CONV_THREADS), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <typename T>
static int launch_conv_w(const ConvParams& p, hipStream_t stream) {
  switch (p.W) {
    case 2: return launch_conv_t<T, 2>(p, stream);
    case 3: return launch_conv_t<T, 3>(p, stream);
    case 4: return launch_conv_t<T, 4>(p, stream);
    case 5: return launch_conv_t<T, 5>(p, stream);
    case 6: return launch_conv_t<T, 6>(p, stream);
    case 7: return launch_conv_t<T, 7>(p, stream);
    case 8: return launch_conv_t<T, 8>(p, stream);
    default: return fail(KDA_ERR_UNSUPPORTED, "conv width W = %d not built (2..8)", p.W);
  }
}

// One workgroup per (checkpoint, 256 channel vectors); each thread copies the
// W-1 raw inputs before the checkpoint of its V channels: from the carried
// history where the checkpoint lies within the sequence's first W-1 tokens,
// else from x.  Reads only the source slots and x, so it runs before the
// conv launch, which may update the history in place.
template <typename T, int W>
__global__ void __launch_bounds__(CONV_THREADS) conv_ckpt_kernel(const ConvCkptParams p) {
  constexpr int V = Vec16<T>::N;
  constexpr int HIST = W - 1;
  const int64_t j = blockIdx.x;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.y) * CONV_THREADS + threadIdx.x) * V;
  if (c0 >= p.C || j >= p.n_ckpt || j >= p.ckpt_cu[p.n_seq]) return;
  int a = 0, b = p.n_seq;                 // ckpt_cu[a] <= j < ckpt_cu[b]
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (p.ckpt_cu[mid] <= j) a = mid; else b = mid;
  }
  const int s = a;
  const int slot = p.ckpt_slot[j];
  if (slot < 0 || slot >= p.n_slots) return;
  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  int64_t start = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (start < 0) start = 0;
  const int64_t pos = (start / p.interval + 1 + (j - p.ckpt_cu[s])) * p.interval;
  const int64_t rel = pos - start;        // tokens of the sequence before the checkpoint
  if (rel <= 0 || rel >= eos - bos) return;
  const T* xb = static_cast<const T*>(p.x);
  const int src = p.src_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  float hist[HIST * V];                   // [i * HIST + q]: channel c0 + i, history entry q
  if (has_src) {
    ld_blocks<T, HIST>(static_cast<const T*>(p.pool) + (static_cast<int64_t>(src) * p.C + c0) * HIST, hist);
  } else {
#pragma unroll
    for (int e = 0; e < HIST * V; ++e) hist[e] = 0.f;
  }
  float out[HIST * V];
#pragma unroll
  for (int q = 0; q < HIST; ++q) {
    const int64_t idx = rel + q;          // index into history ++ tokens
    float xv[V];
    if (idx >= HIST) {
      Vec16<T>::ld(xb + (bos + idx - HIST) * p.x_stride + c0, xv);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float v = hist[i * HIST];
#pragma unroll
        for (int r = 1; r < HIST; ++r) v = idx == r ? hist[i * HIST + r] : v;
        xv[i] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) out[i * HIST + q] = xv[i];
  }
  st_blocks<T, HIST>(static_cast<T*>(p.pool) + (static_cast<int64_t>(slot) * p.C + c0) * HIST, out);
}

int launch_conv_ckpt(const ConvCkptParams& p, int dtype, hipStream_t stream) {
  if (p.n_ckpt <= 0) return KDA_OK;
  const int V = dtype == KDA_BF16 ? 8 : 4;
  const int64_t groups = (p.C + V - 1) / V;
  const dim3 grid(static_cast<uint32_t>(p.n_ckpt), static_cast<uint32_t>((groups + CONV_THREADS - 1) / CONV_THREADS));
  auto go = [&](auto t_tag, auto w_t) {
    using T = decltype(t_tag);
    hipLaunchKernelGGL((conv_ckpt_kernel<T, decltype(w_t)::value>), grid, dim3(CONV_THREADS), 0, stream, p);
  };
  auto by_w = [&](auto t_tag) -> int {
    switch (p.W) {
      case 2: go(t_tag, std::integral_constant<int, 2>{}); return KDA_OK;
      case 3: go(t_tag, std::integral_constant<int, 3>{}); return KDA_OK;
      case 4: go(t_tag, std::integral_constant<int, 4>{}); return KDA_OK;
      default: return fail(KDA_ERR_UNSUPPORTED, "conv checkpoints: W = %d (2..4)", p.W);
    }
  };
  const int st = dtype == KDA_BF16 ? by_w(bf16_t{}) : by_w(float{});
  if (st) return st;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv checkpoint kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

int launch_conv(const ConvParams& p0, int dtype, hipStream_t stream) {
  ConvParams p = p0;
  p.n_tiles = static_cast<int32_t>((p.T_tot + CONV_TT - 1) / CONV_TT);
  if (dtype == KDA_BF16) return launch_conv_w<bf16_t>(p, stream);
  return launch_conv_w<float>(p, stream);
}

}  // namespace kda
