// extern "C" entry points of libkda: argument validation, optional
// KDA_CHECK=1 validation of device index arrays, and dispatch to the kernel
// launchers.  No allocation, no synchronisation (outside KDA_CHECK=1).

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kda_internal.h"

namespace kda {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

static bool check_enabled() {
  static int cached = -1;
  if (cached < 0) {
    const char* e = getenv("KDA_CHECK");
    cached = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return cached == 1;
}

static size_t dtype_bytes(int dt) { return dt == KDA_BF16 ? 2 : 4; }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool supported_d(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

// token stride: 0 -> packed; must cover one token's [H, d] row and keep
// 16-byte alignment.
static int fix_stride(int64_t& stride, int64_t packed, int dt, const char* name) {
  if (stride == 0) stride = packed;
  if (stride < packed) return fail(KDA_ERR_SHAPE, "%s stride %lld < %lld", name, (long long)stride, (long long)packed);
  if ((stride * (int64_t)dtype_bytes(dt)) % 16 != 0)
    return fail(KDA_ERR_ALIGN, "%s stride %lld not 16-byte aligned", name, (long long)stride);
  return KDA_OK;
}

// beta's stride only needs to cover H scalars
static int fix_beta_stride(int64_t& stride, int64_t H) {
  if (stride == 0) stride = H;
  if (stride < H) return fail(KDA_ERR_SHAPE, "beta stride %lld < H", (long long)stride);
  return KDA_OK;
}

template <typename T>
static bool copy_to_host(std::vector<T>& out, const T* dev, size_t n, hipStream_t stream) {
  out.assign(n, T());
  if (n == 0) return true;
  if (hipMemcpyAsync(out.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, stream) != hipSuccess) return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

// KDA_CHECK=1: slots in range, no source slot of one sequence used as a
// destination of another.
static int check_slots(const int32_t* src, const int32_t* dst, int n_seq, int64_t n_slots,
                       const std::vector<int32_t>* extra_dst, hipStream_t stream) {
  std::vector<int32_t> hs, hd;
  if (!copy_to_host(hs, src, n_seq, stream) || !copy_to_host(hd, dst, n_seq, stream))
    return fail(KDA_ERR_HIP, "KDA_CHECK: copying slot arrays failed");
  for (int i = 0; i < n_seq; ++i) {
    if (hs[i] < -1 || hs[i] >= n_slots) return fail(KDA_ERR_ARG, "src_slot[%d] = %d out of range", i, hs[i]);
    if (hd[i] < -1 || hd[i] >= n_slots) return fail(KDA_ERR_ARG, "dst_slot[%d] = %d out of range", i, hd[i]);
  }
  for (int i = 0; i < n_seq; ++i) {
    if (hs[i] < 0) continue;
    for (int j = 0; j < n_seq; ++j)
      if (j != i && hd[j] == hs[i])
        return fail(KDA_ERR_ARG, "src_slot[%d] = %d is dst_slot[%d] (same-call reuse)", i, hs[i], j);
    if (extra_dst)
      for (int32_t c : *extra_dst)
        if (c == hs[i]) return fail(KDA_ERR_ARG, "src_slot[%d] = %d is also a checkpoint slot", i, hs[i]);
  }
  return KDA_OK;
}

static int check_cu(const int32_t* cu, int n_seq, int64_t T_tot, hipStream_t stream,
                    std::vector<int32_t>* out = nullptr) {
  std::vector<int32_t> h;
  if (!copy_to_host(h, cu, (size_t)n_seq + 1, stream)) return fail(KDA_ERR_HIP, "KDA_CHECK: copying cu_seqlens failed");
  if (h[0] < 0) return fail(KDA_ERR_ARG, "cu_seqlens[0] = %d < 0", h[0]);
  for (int i = 0; i < n_seq; ++i)
    if (h[i + 1] < h[i]) return fail(KDA_ERR_ARG, "cu_seqlens decreases at %d", i);
  if (h[n_seq] > T_tot) return fail(KDA_ERR_ARG, "cu_seqlens[n_seq] = %d > T_tot", h[n_seq]);
  if (out) *out = h;
  return KDA_OK;
}

// KDA_CHECK=1: the decay range the chunked prefill is exact for.  Inside a
// tile of `tile` tokens at absolute multiples of `tile`, the chunked form
// scales rows by exp(+-(G_r - G_15)), G the cumulative log decay of the tile
// (rows outside the sequence contribute 0); every such exponent must stay
// within +-kGateLimit nats so that no factor leaves the fp32 range.
constexpr double kGateLimit = 80.0;

static int check_gate_range(const void* g, int dtype, int64_t g_stride, const std::vector<int32_t>& cu,
                            const int32_t* start_pos, int n_seq, int H, int d, int tile, int64_t T_tot,
                            hipStream_t stream) {
  std::vector<int32_t> sp;
  if (start_pos && !copy_to_host(sp, start_pos, (size_t)n_seq, stream))
    return fail(KDA_ERR_HIP, "KDA_CHECK: copying start_pos failed");
  const int64_t rows = T_tot;
  const size_t elems = (size_t)(rows > 0 ? (rows - 1) * g_stride + (int64_t)H * d : 0);
  std::vector<uint16_t> g16;
  std::vector<float> g32;
  if (dtype == KDA_BF16) {
    if (!copy_to_host(g16, static_cast<const uint16_t*>(g), elems, stream))
      return fail(KDA_ERR_HIP, "KDA_CHECK: copying g failed");
  } else if (!copy_to_host(g32, static_cast<const float*>(g), elems, stream)) {
    return fail(KDA_ERR_HIP, "KDA_CHECK: copying g failed");
  }
  auto at = [&](int64_t i) -> double {
    if (dtype == KDA_BF16) {
      const uint32_t u = static_cast<uint32_t>(g16[i]) << 16;
      float f;
      memcpy(&f, &u, 4);
      return f;
    }
    return g32[i];
  };
  std::vector<double> cum(tile);
  for (int s = 0; s < n_seq; ++s) {
    const int64_t bos = cu[s], len = (int64_t)cu[s + 1] - cu[s];
    if (len <= 0) continue;
    const int64_t start = sp.empty() ? 0 : (sp[s] > 0 ? sp[s] : 0);
    for (int64_t t0 = (start / tile) * tile; t0 < start + len; t0 += tile)
      for (int h = 0; h < H; ++h)
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int r = 0; r < tile; ++r) {
            const int64_t pos = t0 + r;
            if (pos >= start && pos < start + len) acc += at((bos + pos - start) * g_stride + (int64_t)h * d + c);
            cum[r] = acc;
          }
          for (int r = 0; r < tile; ++r)
            if (fabs(cum[r] - cum[15]) > kGateLimit)
              return fail(KDA_ERR_ARG,
                          "g out of range: sequence %d head %d channel %d, tile at position %lld sums to "
                          "%.1f over rows %d..15 (limit %.0f)",
                          s, h, c, (long long)t0, cum[r] - cum[15], r, kGateLimit);
        }
  }
  return KDA_OK;
}

}  // namespace kda

using namespace kda;

extern "C" {

const char* kda_status_str(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_ARG: return "KDA_ERR_ARG";
    case KDA_ERR_CAPACITY: return "KDA_ERR_CAPACITY";
    default: return "KDA_ERR_UNKNOWN";
  }
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_last_error; }

size_t kda_args_sizeof(int which) {
  switch (which) {
    case 0: return sizeof(kda_conv_args);
    case 1: return sizeof(kda_prefill_args);
    case 2: return sizeof(kda_decode_args);
    case 3: return sizeof(kda_verify_args);
    case 4: return sizeof(kda_decode_conv_args);
    case 5: return sizeof(kda_verify_conv_args);
    case 6: return sizeof(kda_plan_args);
    case 7: return sizeof(kda_prefill_conv_args);
    default: return 0;
  }
}

// ------------------------------------------------------------------ conv
int kda_conv_short(const kda_conv_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_conv_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->dtype != KDA_BF16 && a->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "dtype %d", a->dtype);
  if (a->n_seq < 0 || a->T_tot < 0 || a->n_slots < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (a->n_seq == 0) return KDA_OK;
  if (a->W < 2 || a->W > 8) return fail(KDA_ERR_UNSUPPORTED, "conv width W = %d (2..8)", a->W);
  const int V = 16 / (int)dtype_bytes(a->dtype);
  if (a->C <= 0 || a->C % V != 0) return fail(KDA_ERR_SHAPE, "C = %d not a positive multiple of %d", a->C, V);
  if (!a->cu_seqlens || !a->weight || !a->src_slot || !a->dst_slot || !a->conv_pool)
    return fail(KDA_ERR_NULL, "conv: required pointer is NULL");
  if (a->T_tot > 0 && (!a->x || !a->y)) return fail(KDA_ERR_NULL, "conv: x or y is NULL");
  kda_conv_args b = *a;
  if (b.x_stride == 0) b.x_stride = b.C;
  if (b.y_stride == 0) b.y_stride = b.C;
  if (b.x_stride < b.C || b.y_stride < b.C) return fail(KDA_ERR_SHAPE, "conv stride < C");
  const int64_t eb = dtype_bytes(b.dtype);
  if ((b.x_stride * eb) % 16 || (b.y_stride * eb) % 16 || !aligned16(b.x) || !aligned16(b.y) ||
      !aligned16(b.conv_pool) || !aligned16(b.weight))
    return fail(KDA_ERR_ALIGN, "conv: x, y, weight or conv_pool not 16-byte aligned");
  if (b.T_tot / 16 + b.n_seq + 1 > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "conv: too many tokens");
  if (b.act != 0 && b.act != 1) return fail(KDA_ERR_ARG, "conv: act = %d (0 none, 1 SiLU)", b.act);
  if (b.norm_d != 0) {
    if (b.norm_d != 16 && b.norm_d != 32 && b.norm_d != 64 && b.norm_d != 128)
      return fail(KDA_ERR_UNSUPPORTED, "conv: norm_d = %d (16, 32, 64, 128)", b.norm_d);
    if (b.W > 4) return fail(KDA_ERR_UNSUPPORTED, "conv: normalisation with W = %d (2..4)", b.W);
    if (b.norm_channels < 0 || b.norm_channels > b.C || b.norm_channels % b.norm_d)
      return fail(KDA_ERR_ARG, "conv: norm_channels %lld (a multiple of norm_d, <= C)", (long long)b.norm_channels);
    if (b.C % b.norm_d) return fail(KDA_ERR_ARG, "conv: C %d not a multiple of norm_d %d", b.C, b.norm_d);
    if (!(b.norm_eps >= 0.f)) return fail(KDA_ERR_ARG, "conv: norm_eps < 0");
  }
  if (check_enabled()) {
    int st = check_cu(b.cu_seqlens, b.n_seq, b.T_tot, stream);
    if (st) return st;
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, nullptr, stream);
    if (st) return st;
  }
  ConvParams p{};
  p.x = b.x; p.y = b.y; p.w = b.weight; p.bias = b.bias; p.cu = b.cu_seqlens; p.pool = b.conv_pool;
  p.src_slot = b.src_slot; p.dst_slot = b.dst_slot; p.adv = b.advance_len;
  p.x_stride = b.x_stride; p.y_stride = b.y_stride; p.T_tot = b.T_tot; p.n_slots = b.n_slots;
  p.n_seq = b.n_seq; p.C = b.C; p.W = b.W; p.act = b.act;
  p.norm_d = b.norm_d;
  p.norm_channels = b.norm_d ? b.norm_channels : 0;
  p.norm_eps = b.norm_eps;
  return launch_conv(p, b.dtype, stream);
}

// ------------------------------------------------------------------ ckpt plan
int kda_ckpt_plan(const int32_t* cu, const int32_t* start_pos, int32_t n_seq, int32_t interval,
                  int32_t chunk, int32_t* ckpt_cu, int32_t* ckpt_pos, int32_t cap,
                  int32_t* n_total) {
  if (!cu || !ckpt_cu || !n_total) return fail(KDA_ERR_NULL, "ckpt_plan: required pointer is NULL");
  if (n_seq < 0 || cap < 0) return fail(KDA_ERR_SHAPE, "ckpt_plan: negative size");
  if (chunk != 16 && chunk != 32 && chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk %d", chunk);
  if (interval <= 0 || interval % chunk != 0)
    return fail(KDA_ERR_ALIGN, "interval %d not a positive multiple of chunk %d", interval, chunk);
  int64_t total = 0;
  ckpt_cu[0] = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int64_t len = (int64_t)cu[s + 1] - cu[s];
    const int64_t st = start_pos ? start_pos[s] : 0;
    if (len < 0 || st < 0) return fail(KDA_ERR_SHAPE, "ckpt_plan: sequence %d has negative length or start", s);
    const int64_t n = len > 0 ? (st + len - 1) / interval - st / interval : 0;
    for (int64_t m = 0; m < n; ++m) {
      const int64_t pos = (st / interval + 1 + m) * interval;
      if (total + m < cap && ckpt_pos) ckpt_pos[total + m] = (int32_t)pos;
    }
    total += n;
    if (total > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "ckpt_plan: too many checkpoints");
    ckpt_cu[s + 1] = (int32_t)total;
  }
  *n_total = (int32_t)total;
  if (total > cap) return fail(KDA_ERR_CAPACITY, "ckpt_plan: %lld checkpoints > cap %d", (long long)total, cap);
  return KDA_OK;
}

int kda_ckpt_plan_device(const kda_plan_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_plan_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->cap < 0 || a->n_free < 0 || a->T_tot < 0)
    return fail(KDA_ERR_SHAPE, "ckpt_plan_device: negative size");
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk %d", a->chunk);
  if (a->interval <= 0 || a->interval % a->chunk != 0)
    return fail(KDA_ERR_ALIGN, "interval %d not a positive multiple of chunk %d", a->interval, a->chunk);
  if (!a->cu_seqlens || !a->ckpt_cu) return fail(KDA_ERR_NULL, "ckpt_plan_device: cu_seqlens or ckpt_cu is NULL");
  if (a->n_free > 0 && !a->free_slots) return fail(KDA_ERR_NULL, "ckpt_plan_device: free_slots is NULL");
  PlanParams p{};
  p.cu = a->cu_seqlens;
  p.start_pos = a->start_pos;
  p.free_slots = a->free_slots;
  p.ckpt_cu = a->ckpt_cu;
  p.ckpt_pos = a->ckpt_pos;
  p.ckpt_slot = a->ckpt_slot;
  p.n_total = a->n_total;
  p.T_tot = a->T_tot;
  p.n_seq = a->n_seq;
  p.interval = a->interval;
  p.cap = a->cap;
  p.n_free = a->n_free;
  return launch_plan(p, stream);
}

// ------------------------------------------------------------------ decode / verify
static int step_common(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       void* o, int64_t& qs, int64_t& ks, int64_t& vs, int64_t& gs, int64_t& bs,
                       int64_t& os, int H, int dk, int dv, int in_dt, int out_dt, float* pool,
                       const int32_t* src, const int32_t* dst) {
  if (in_dt != KDA_BF16 && in_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "in_dtype %d", in_dt);
  if (out_dt != KDA_BF16 && out_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "out_dtype %d", out_dt);
  if (H <= 0) return fail(KDA_ERR_SHAPE, "H = %d", H);
  if (!supported_d(dk, dv)) return fail(KDA_ERR_UNSUPPORTED, "d_k = %d, d_v = %d (need equal, 16/32/64/128)", dk, dv);
  if (!q || !k || !v || !g || !beta || !pool || !src || !dst) return fail(KDA_ERR_NULL, "required pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(pool) || (o && !aligned16(o)))
    return fail(KDA_ERR_ALIGN, "q, k, v, g, o or state_pool not 16-byte aligned");
  int st;
  if ((st = fix_stride(qs, (int64_t)H * dk, in_dt, "q"))) return st;
  if ((st = fix_stride(ks, (int64_t)H * dk, in_dt, "k"))) return st;
  if ((st = fix_stride(vs, (int64_t)H * dv, in_dt, "v"))) return st;
  if ((st = fix_stride(gs, (int64_t)H * dk, in_dt, "g"))) return st;
  if ((st = fix_stride(os, (int64_t)H * dv, out_dt, "o"))) return st;
  if ((st = fix_beta_stride(bs, H))) return st;
  return KDA_OK;
}

int kda_decode(const kda_decode_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_decode_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->n_slots < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (a->n_seq == 0) return KDA_OK;
  kda_decode_args b = *a;
  if (!b.o) return fail(KDA_ERR_NULL, "decode: o is NULL");
  int st = step_common(b.q, b.k, b.v, b.g, b.beta, b.o, b.q_stride, b.k_stride, b.v_stride, b.g_stride,
                       b.beta_stride, b.o_stride, b.H, b.d_k, b.d_v, b.in_dtype, b.out_dtype, b.state_pool,
                       b.src_slot, b.dst_slot);
  if (st) return st;
  if ((int64_t)b.n_seq * b.H > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "n_seq * H too large");
  if (check_enabled()) {
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, nullptr, stream);
    if (st) return st;
  }
  StepParams p{};
  p.q = b.q; p.k = b.k; p.v = b.v; p.g = b.g; p.beta = b.beta; p.o = b.o; p.pool = b.state_pool;
  p.src_slot = b.src_slot; p.dst_slot = b.dst_slot; p.accepted_len = nullptr; p.committed_len_out = nullptr;
  p.q_stride = b.q_stride; p.k_stride = b.k_stride; p.v_stride = b.v_stride; p.g_stride = b.g_stride;
  p.beta_stride = b.beta_stride; p.o_stride = b.o_stride; p.n_slots = b.n_slots;
  p.n_seq = b.n_seq; p.T_spec = 1; p.H = b.H; p.commit_all = 1; p.scale = b.scale;
  return launch_step(p, b.d_k, b.in_dtype, b.out_dtype, stream);
}

// the optional gated RMS norm of the fused steps' output
static int out_gate_common(const void* gate, const void* weight, int64_t& stride, float eps, int H, int d,
                           int in_dt, const char* who) {
  if (!gate) return KDA_OK;
  if (!weight) return fail(KDA_ERR_NULL, "%s: out_gate given without out_norm_weight", who);
  if (!(eps >= 0.f)) return fail(KDA_ERR_ARG, "%s: out_norm_eps < 0", who);
  if (!aligned16(gate) || !aligned16(weight))
    return fail(KDA_ERR_ALIGN, "%s: out_gate or out_norm_weight not 16-byte aligned", who);
  return fix_stride(stride, (int64_t)H * d, in_dt, "out_gate");
}

int kda_decode_conv(const kda_decode_conv_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_decode_conv_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->n_slots < 0 || a->n_conv_slots < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (a->n_seq == 0) return KDA_OK;
  kda_decode_conv_args b = *a;
  const int in_dt = b.in_dtype, out_dt = b.out_dtype;
  if (in_dt != KDA_BF16 && in_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "in_dtype %d", in_dt);
  if (out_dt != KDA_BF16 && out_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "out_dtype %d", out_dt);
  if (b.H <= 0) return fail(KDA_ERR_SHAPE, "H = %d", b.H);
  if (!supported_d(b.d, b.d)) return fail(KDA_ERR_UNSUPPORTED, "d = %d (16/32/64/128)", b.d);
  if (b.W < 2 || b.W > 4) return fail(KDA_ERR_UNSUPPORTED, "decode_conv: W = %d (2..4)", b.W);
  if (b.act != 0 && b.act != 1) return fail(KDA_ERR_ARG, "decode_conv: act = %d (0 none, 1 SiLU)", b.act);
  if (b.qk_l2norm != 0 && b.qk_l2norm != 1) return fail(KDA_ERR_ARG, "decode_conv: qk_l2norm = %d", b.qk_l2norm);
  if (!(b.norm_eps >= 0.f)) return fail(KDA_ERR_ARG, "decode_conv: norm_eps < 0");
  if (!b.x || !b.conv_weight || !b.conv_pool || !b.conv_src_slot || !b.conv_dst_slot || !b.g || !b.beta ||
      !b.o || !b.state_pool || !b.src_slot || !b.dst_slot)
    return fail(KDA_ERR_NULL, "decode_conv: required pointer is NULL");
  const int64_t C = 3LL * b.H * b.d;
  const int64_t eb = dtype_bytes(in_dt);
  if (b.x_stride == 0) b.x_stride = C;
  if (b.x_stride < C) return fail(KDA_ERR_SHAPE, "decode_conv: x_stride < 3 H d");
  if (!aligned16(b.x) || !aligned16(b.conv_weight) || !aligned16(b.conv_pool) || !aligned16(b.g) ||
      !aligned16(b.o) || !aligned16(b.state_pool) || (b.conv_bias && !aligned16(b.conv_bias)) ||
      (b.x_stride * eb) % 16)
    return fail(KDA_ERR_ALIGN,
                "decode_conv: x, conv_weight, conv_bias, conv_pool, g, o or state_pool not 16-byte aligned");
  int st;
  if ((st = fix_stride(b.g_stride, (int64_t)b.H * b.d, in_dt, "g"))) return st;
  if ((st = fix_stride(b.o_stride, (int64_t)b.H * b.d, out_dt, "o"))) return st;
  if ((st = fix_beta_stride(b.beta_stride, b.H))) return st;
  if ((st = out_gate_common(b.out_gate, b.out_norm_weight, b.out_gate_stride, b.out_norm_eps, b.H, b.d, in_dt,
                            "decode_conv")))
    return st;
  if ((int64_t)b.n_seq * b.H > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "n_seq * H too large");
  if (check_enabled()) {
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, nullptr, stream);
    if (st) return st;
    st = check_slots(b.conv_src_slot, b.conv_dst_slot, b.n_seq, b.n_conv_slots, nullptr, stream);
    if (st) return st;
  }
  DecodeConvParams p{};
  p.x = b.x; p.w = b.conv_weight; p.bias = b.conv_bias; p.g = b.g; p.beta = b.beta;
  p.cpool = b.conv_pool; p.o = b.o; p.pool = b.state_pool;
  p.csrc = b.conv_src_slot; p.cdst = b.conv_dst_slot; p.src_slot = b.src_slot; p.dst_slot = b.dst_slot;
  p.x_stride = b.x_stride; p.g_stride = b.g_stride; p.beta_stride = b.beta_stride; p.o_stride = b.o_stride;
  p.n_slots = b.n_slots; p.n_cslots = b.n_conv_slots;
  p.n_seq = b.n_seq; p.H = b.H; p.W = b.W; p.act = b.act; p.qk_l2norm = b.qk_l2norm;
  p.eps = b.norm_eps; p.scale = b.scale;
  p.ogate = b.out_gate; p.onorm_w = b.out_norm_weight; p.ogate_stride = b.out_gate_stride;
  p.onorm_eps = b.out_norm_eps;
  return launch_decode_conv(p, b.d, in_dt, out_dt, stream);
}

int kda_verify_conv(const kda_verify_conv_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_verify_conv_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->n_slots < 0 || a->n_conv_slots < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (a->T_spec < 1 || a->T_spec > 16) return fail(KDA_ERR_SHAPE, "T_spec = %d (1..16)", a->T_spec);
  if (a->n_seq == 0) return KDA_OK;
  kda_verify_conv_args b = *a;
  const int in_dt = b.in_dtype, out_dt = b.out_dtype;
  if (in_dt != KDA_BF16 && in_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "in_dtype %d", in_dt);
  if (out_dt != KDA_BF16 && out_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "out_dtype %d", out_dt);
  if (b.H <= 0) return fail(KDA_ERR_SHAPE, "H = %d", b.H);
  if (!supported_d(b.d, b.d)) return fail(KDA_ERR_UNSUPPORTED, "d = %d (16/32/64/128)", b.d);
  if (b.W < 2 || b.W > 4) return fail(KDA_ERR_UNSUPPORTED, "verify_conv: W = %d (2..4)", b.W);
  if (b.act != 0 && b.act != 1) return fail(KDA_ERR_ARG, "verify_conv: act = %d (0 none, 1 SiLU)", b.act);
  if (b.qk_l2norm != 0 && b.qk_l2norm != 1) return fail(KDA_ERR_ARG, "verify_conv: qk_l2norm = %d", b.qk_l2norm);
  if (!(b.norm_eps >= 0.f)) return fail(KDA_ERR_ARG, "verify_conv: norm_eps < 0");
  if (!b.o && !b.accepted_len) return fail(KDA_ERR_NULL, "verify_conv: neither o nor accepted_len given");
  if (!b.x || !b.conv_weight || !b.conv_pool || !b.conv_src_slot || !b.conv_dst_slot || !b.g || !b.beta ||
      !b.state_pool || !b.src_slot || !b.dst_slot)
    return fail(KDA_ERR_NULL, "verify_conv: required pointer is NULL");
  const int64_t C = 3LL * b.H * b.d;
  const int64_t eb = dtype_bytes(in_dt);
  if (b.x_stride == 0) b.x_stride = C;
  if (b.x_stride < C) return fail(KDA_ERR_SHAPE, "verify_conv: x_stride < 3 H d");
  if (!aligned16(b.x) || !aligned16(b.conv_weight) || !aligned16(b.conv_pool) || !aligned16(b.g) ||
      (b.o && !aligned16(b.o)) || !aligned16(b.state_pool) || (b.conv_bias && !aligned16(b.conv_bias)) ||
      (b.x_stride * eb) % 16)
    return fail(KDA_ERR_ALIGN,
                "verify_conv: x, conv_weight, conv_bias, conv_pool, g, o or state_pool not 16-byte aligned");
  int st;
  if ((st = fix_stride(b.g_stride, (int64_t)b.H * b.d, in_dt, "g"))) return st;
  if ((st = fix_stride(b.o_stride, (int64_t)b.H * b.d, out_dt, "o"))) return st;
  if ((st = fix_beta_stride(b.beta_stride, b.H))) return st;
  if ((st = out_gate_common(b.out_gate, b.out_norm_weight, b.out_gate_stride, b.out_norm_eps, b.H, b.d, in_dt,
                            "verify_conv")))
    return st;
  if ((int64_t)b.n_seq * b.H > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "n_seq * H too large");
  if (check_enabled()) {
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, nullptr, stream);
    if (st) return st;
    st = check_slots(b.conv_src_slot, b.conv_dst_slot, b.n_seq, b.n_conv_slots, nullptr, stream);
    if (st) return st;
  }
  DecodeConvParams p{};
  p.x = b.x; p.w = b.conv_weight; p.bias = b.conv_bias; p.g = b.g; p.beta = b.beta;
  p.cpool = b.conv_pool; p.o = b.o; p.pool = b.state_pool;
  p.csrc = b.conv_src_slot; p.cdst = b.conv_dst_slot; p.src_slot = b.src_slot; p.dst_slot = b.dst_slot;
  p.x_stride = b.x_stride; p.g_stride = b.g_stride; p.beta_stride = b.beta_stride; p.o_stride = b.o_stride;
  p.n_slots = b.n_slots; p.n_cslots = b.n_conv_slots;
  p.n_seq = b.n_seq; p.H = b.H; p.W = b.W; p.act = b.act; p.qk_l2norm = b.qk_l2norm;
  p.eps = b.norm_eps; p.scale = b.scale;
  p.T_spec = b.T_spec; p.accepted_len = b.accepted_len; p.committed_len_out = b.committed_len_out;
  p.ogate = b.out_gate; p.onorm_w = b.out_norm_weight; p.ogate_stride = b.out_gate_stride;
  p.onorm_eps = b.out_norm_eps;
  return launch_verify_conv(p, b.d, in_dt, out_dt, stream);
}

int kda_verify(const kda_verify_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_verify_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->n_slots < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (a->T_spec < 1 || a->T_spec > 16) return fail(KDA_ERR_SHAPE, "T_spec = %d (1..16)", a->T_spec);
  if (a->n_seq == 0) return KDA_OK;
  kda_verify_args b = *a;
  if (!b.o && !b.accepted_len) return fail(KDA_ERR_NULL, "verify: neither o nor accepted_len given");
  int st = step_common(b.q, b.k, b.v, b.g, b.beta, b.o, b.q_stride, b.k_stride, b.v_stride, b.g_stride,
                       b.beta_stride, b.o_stride, b.H, b.d_k, b.d_v, b.in_dtype, b.out_dtype, b.state_pool,
                       b.src_slot, b.dst_slot);
  if (st) return st;
  if ((int64_t)b.n_seq * b.H > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "n_seq * H too large");
  if (check_enabled()) {
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, nullptr, stream);
    if (st) return st;
  }
  StepParams p{};
  p.q = b.q; p.k = b.k; p.v = b.v; p.g = b.g; p.beta = b.beta; p.o = b.o; p.pool = b.state_pool;
  p.src_slot = b.src_slot; p.dst_slot = b.dst_slot; p.accepted_len = b.accepted_len;
  p.committed_len_out = b.committed_len_out;
  p.q_stride = b.q_stride; p.k_stride = b.k_stride; p.v_stride = b.v_stride; p.g_stride = b.g_stride;
  p.beta_stride = b.beta_stride; p.o_stride = b.o_stride; p.n_slots = b.n_slots;
  p.n_seq = b.n_seq; p.T_spec = b.T_spec; p.H = b.H; p.commit_all = 0; p.scale = b.scale;
  return launch_step(p, b.d_k, b.in_dtype, b.out_dtype, stream);
}

// ------------------------------------------------------------------ prefill
static int prefill_validate(const kda_prefill_args* a, kda_prefill_args& b) {
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_prefill_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  if (a->n_seq < 0 || a->T_tot < 0 || a->n_slots < 0 || a->n_ckpt < 0 || a->workspace_bytes < 0)
    return fail(KDA_ERR_SHAPE, "negative size");
  b = *a;
  if (b.T_tot == 0) {
    // no tokens: the per-token tensors are never touched (an empty tensor
    // may come as NULL), only the states are copied and written
    void* f = b.state_pool;
    if (!b.q) b.q = f;
    if (!b.k) b.k = f;
    if (!b.v) b.v = f;
    if (!b.g) b.g = f;
    if (!b.beta) b.beta = f;
    if (!b.o) b.o = f;
  }
  if (b.chunk != 16 && b.chunk != 32 && b.chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk %d (16, 32, 64)", b.chunk);
  if (b.ckpt_interval < 0) return fail(KDA_ERR_SHAPE, "ckpt_interval < 0");
  if (b.ckpt_interval > 0 && b.ckpt_interval % b.chunk != 0)
    return fail(KDA_ERR_ALIGN, "ckpt_interval %d not a multiple of chunk %d", b.ckpt_interval, b.chunk);
  if (b.segment_len > 0 && b.segment_len % b.chunk != 0)
    return fail(KDA_ERR_ALIGN, "segment_len %d not a multiple of chunk %d", b.segment_len, b.chunk);
  if (b.ckpt_interval > 0 && (!b.ckpt_cu || (b.n_ckpt > 0 && !b.ckpt_slot)))
    return fail(KDA_ERR_NULL, "checkpoints requested without ckpt_cu / ckpt_slot");
  if (!b.cu_seqlens) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  int st = step_common(b.q, b.k, b.v, b.g, b.beta, b.o, b.q_stride, b.k_stride, b.v_stride, b.g_stride,
                       b.beta_stride, b.o_stride, b.H, b.d_k, b.d_v, b.in_dtype, b.out_dtype, b.state_pool,
                       b.src_slot, b.dst_slot);
  if (st) return st;
  if (!b.o) return fail(KDA_ERR_NULL, "prefill: o is NULL");
  return KDA_OK;
}

static PrefillParams prefill_params(const kda_prefill_args& b) {
  PrefillParams p{};
  p.q = b.q; p.k = b.k; p.v = b.v; p.g = b.g; p.beta = b.beta; p.o = b.o; p.cu = b.cu_seqlens;
  p.pool = b.state_pool; p.src_slot = b.src_slot; p.dst_slot = b.dst_slot; p.start_pos = b.start_pos;
  p.ckpt_cu = b.ckpt_interval > 0 ? b.ckpt_cu : nullptr; p.ckpt_slot = b.ckpt_slot;
  p.ckpt_pos_out = b.ckpt_pos_out; p.workspace = b.workspace;
  p.q_stride = b.q_stride; p.k_stride = b.k_stride; p.v_stride = b.v_stride; p.g_stride = b.g_stride;
  p.beta_stride = b.beta_stride; p.o_stride = b.o_stride;
  p.T_tot = b.T_tot; p.n_slots = b.n_slots; p.n_ckpt = b.n_ckpt; p.workspace_bytes = b.workspace_bytes;
  p.n_seq = b.n_seq; p.H = b.H; p.chunk = b.chunk; p.ckpt_interval = b.ckpt_interval; p.scale = b.scale;
  p.segment_len = b.segment_len;
  return p;
}

int64_t kda_prefill_workspace_bytes(const kda_prefill_args* a) {
  kda_prefill_args b;
  if (prefill_validate(a, b) != KDA_OK) return -1;
  return prefill_workspace_bytes(prefill_params(b), b.d_k);
}

// The workspace test and the KDA_CHECK=1 validation of validated prefill
// args; nothing is launched.
static int prefill_precheck(const kda_prefill_args& b, const PrefillParams& p, hipStream_t stream) {
  int st;
  const int64_t need = prefill_workspace_bytes(p, b.d_k);
  if (need > 0 && (!b.workspace || b.workspace_bytes < need))
    return fail(KDA_ERR_WORKSPACE, "workspace %lld bytes < %lld needed", (long long)b.workspace_bytes, (long long)need);
  if (need > 0 && !aligned16(b.workspace)) return fail(KDA_ERR_ALIGN, "workspace not 16-byte aligned");
  if (check_enabled()) {
    std::vector<int32_t> hcu;
    st = check_cu(b.cu_seqlens, b.n_seq, b.T_tot, stream, &hcu);
    if (st) return st;
    std::vector<int32_t> ck;
    if (b.ckpt_interval > 0 && b.n_ckpt > 0) {
      if (!copy_to_host(ck, b.ckpt_slot, (size_t)b.n_ckpt, stream)) return fail(KDA_ERR_HIP, "KDA_CHECK: copy failed");
      for (int32_t c : ck)
        if (c < -1 || c >= b.n_slots) return fail(KDA_ERR_ARG, "ckpt_slot %d out of range", c);
    }
    st = check_slots(b.src_slot, b.dst_slot, b.n_seq, b.n_slots, &ck, stream);
    if (st) return st;
    st = check_gate_range(b.g, b.in_dtype, b.g_stride, hcu, b.start_pos, b.n_seq, b.H, b.d_k,
                          b.chunk == 16 ? 16 : 32, b.T_tot, stream);
    if (st) return st;
  }
  return KDA_OK;
}

int kda_prefill_varlen(const kda_prefill_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  kda_prefill_args b;
  int st = prefill_validate(a, b);
  if (st) return st;
  if (b.n_seq == 0) return KDA_OK;
  PrefillParams p = prefill_params(b);
  if ((st = prefill_precheck(b, p, stream))) return st;
  return launch_prefill(p, b.d_k, b.in_dtype, b.out_dtype, stream);
}

int kda_prefill_varlen_conv(const kda_prefill_conv_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(kda_prefill_conv_args)) return fail(KDA_ERR_ARG, "struct_size mismatch");
  kda_prefill_args pa = a->prefill;
  if (pa.q || pa.k || pa.v || pa.q_stride || pa.k_stride || pa.v_stride)
    return fail(KDA_ERR_ARG, "prefill_conv: prefill.q / k / v must be NULL and their strides 0 (they are formed in qkv)");
  if (pa.d_k != pa.d_v) return fail(KDA_ERR_ARG, "prefill_conv: d_k %d != d_v %d", pa.d_k, pa.d_v);
  const int in_dt = pa.in_dtype;
  if (in_dt != KDA_BF16 && in_dt != KDA_F32) return fail(KDA_ERR_DTYPE, "in_dtype %d", in_dt);
  if (pa.H <= 0) return fail(KDA_ERR_SHAPE, "H = %d", pa.H);
  if (!supported_d(pa.d_k, pa.d_v)) return fail(KDA_ERR_UNSUPPORTED, "d = %d (16/32/64/128)", pa.d_k);
  if (a->W < 2 || a->W > 4) return fail(KDA_ERR_UNSUPPORTED, "prefill_conv: W = %d (2..4)", a->W);
  if (a->act != 0 && a->act != 1) return fail(KDA_ERR_ARG, "prefill_conv: act = %d (0 none, 1 SiLU)", a->act);
  if (a->qk_l2norm != 0 && a->qk_l2norm != 1) return fail(KDA_ERR_ARG, "prefill_conv: qk_l2norm = %d", a->qk_l2norm);
  if (!(a->norm_eps >= 0.f)) return fail(KDA_ERR_ARG, "prefill_conv: norm_eps < 0");
  if (a->n_conv_slots < 0 || a->qkv_bytes < 0) return fail(KDA_ERR_SHAPE, "negative size");
  if (!a->qkv && pa.T_tot > 0) return fail(KDA_ERR_NULL, "prefill_conv: qkv is NULL");
  const int64_t HD = static_cast<int64_t>(pa.H) * pa.d_k;
  const int64_t C = 3 * HD;
  if (C > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "prefill_conv: 3 H d too large");
  const int64_t eb = dtype_bytes(in_dt);
  char* qkv = static_cast<char*>(a->qkv);
  if (qkv) {   // (NULL only without tokens)
    pa.q = qkv;
    pa.k = qkv + HD * eb;
    pa.v = qkv + 2 * HD * eb;
  }
  pa.q_stride = pa.k_stride = pa.v_stride = C;
  kda_prefill_args b;
  int st = prefill_validate(&pa, b);
  if (st) return st;
  if (b.n_seq == 0) return KDA_OK;
  if ((!a->x && b.T_tot > 0) || !a->conv_weight || !a->conv_pool || !a->conv_src_slot || !a->conv_dst_slot)
    return fail(KDA_ERR_NULL, "prefill_conv: required pointer is NULL");
  // without tokens x and qkv are never touched (the conv only copies histories)
  const void* xp = a->x ? a->x : a->conv_pool;
  void* yp = a->qkv ? a->qkv : a->conv_pool;
  int64_t x_stride = a->x_stride == 0 ? C : a->x_stride;
  if (x_stride < C) return fail(KDA_ERR_SHAPE, "prefill_conv: x_stride < 3 H d");
  if (!aligned16(a->x) || !aligned16(a->qkv) || !aligned16(a->conv_weight) || !aligned16(a->conv_pool) ||
      (x_stride * eb) % 16)
    return fail(KDA_ERR_ALIGN, "prefill_conv: x, qkv, conv_weight or conv_pool not 16-byte aligned");
  if (a->qkv_bytes / eb / C < b.T_tot)
    return fail(KDA_ERR_WORKSPACE, "prefill_conv: qkv %lld bytes < %lld needed", (long long)a->qkv_bytes,
                (long long)(b.T_tot * C * eb));
  if (b.T_tot / 16 + b.n_seq + 1 > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "prefill_conv: too many tokens");
  const bool conv_ckpt = a->conv_ckpt_slot != nullptr && b.n_ckpt > 0;
  if (a->conv_ckpt_slot && b.ckpt_interval <= 0)
    return fail(KDA_ERR_ARG, "prefill_conv: conv_ckpt_slot given without checkpoints (ckpt_interval 0)");
  if (b.n_ckpt > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "prefill_conv: too many checkpoints");
  PrefillParams p = prefill_params(b);
  if ((st = prefill_precheck(b, p, stream))) return st;
  if (check_enabled()) {
    std::vector<int32_t> cck;
    if (conv_ckpt) {
      if (!copy_to_host(cck, a->conv_ckpt_slot, (size_t)b.n_ckpt, stream))
        return fail(KDA_ERR_HIP, "KDA_CHECK: copy failed");
      for (int32_t c : cck)
        if (c < -1 || c >= a->n_conv_slots) return fail(KDA_ERR_ARG, "conv_ckpt_slot %d out of range", c);
    }
    st = check_slots(a->conv_src_slot, a->conv_dst_slot, b.n_seq, a->n_conv_slots, conv_ckpt ? &cck : nullptr,
                     stream);
    if (st) return st;
  }
  if (conv_ckpt) {
    // before the conv launch: it reads the source histories, which that
    // launch may advance in place
    ConvCkptParams kp{};
    kp.x = xp; kp.pool = a->conv_pool; kp.cu = b.cu_seqlens; kp.start_pos = b.start_pos;
    kp.src_slot = a->conv_src_slot; kp.ckpt_cu = b.ckpt_cu; kp.ckpt_slot = a->conv_ckpt_slot;
    kp.x_stride = x_stride; kp.T_tot = b.T_tot; kp.n_slots = a->n_conv_slots; kp.n_ckpt = b.n_ckpt;
    kp.n_seq = b.n_seq; kp.C = static_cast<int32_t>(C); kp.W = a->W; kp.interval = b.ckpt_interval;
    if ((st = launch_conv_ckpt(kp, in_dt, stream))) return st;
  }
  ConvParams cp{};
  cp.x = xp; cp.y = yp; cp.w = a->conv_weight; cp.bias = a->conv_bias; cp.cu = b.cu_seqlens;
  cp.pool = a->conv_pool; cp.src_slot = a->conv_src_slot; cp.dst_slot = a->conv_dst_slot; cp.adv = nullptr;
  cp.x_stride = x_stride; cp.y_stride = C; cp.T_tot = b.T_tot; cp.n_slots = a->n_conv_slots;
  cp.n_seq = b.n_seq; cp.C = static_cast<int32_t>(C); cp.W = a->W; cp.act = a->act;
  cp.norm_channels = a->qk_l2norm ? 2 * HD : 0;
  cp.norm_d = a->qk_l2norm ? b.d_k : 0;
  cp.norm_eps = a->norm_eps;
  if ((st = launch_conv(cp, in_dt, stream))) return st;
  return launch_prefill(p, b.d_k, b.in_dtype, b.out_dtype, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ prefill without allocation
// The segment-scan workspace of kda_prefill_varlen_noalloc lives in this
// static device array: the code object carries it, so each GPU the library
// runs on holds one copy (kScratchBytes) until the process ends.  Host code
// must use its device address, looked up once per device; the array's name
// itself is a host-side stand-in.
namespace kda {
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}
}  // namespace kda

extern "C" {

int64_t kda_prefill_noalloc_max_bytes(void) { return kScratchBytes; }

int kda_prefill_varlen_noalloc(const kda_prefill_args* a, kda_stream_t stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  kda_prefill_args b;
  int st = prefill_validate(a, b);
  if (st) return st;
  if (b.workspace || b.workspace_bytes)
    return fail(KDA_ERR_ARG, "prefill_noalloc: workspace must be NULL and workspace_bytes 0 (the library's scratch is used)");
  if (b.n_seq == 0) return KDA_OK;
  PrefillParams p = prefill_params(b);
  const int64_t need = prefill_workspace_bytes(p, b.d_k);
  if (need > kScratchBytes)
    return fail(KDA_ERR_WORKSPACE,
                "prefill_noalloc: the segment scan of this call needs %lld bytes of scratch, more than the %lld "
                "the library holds; use kda_prefill_varlen with a workspace, or a longer segment_len",
                (long long)need, (long long)kScratchBytes);
  if (need > 0) {
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st) return st;
    p.workspace = ws;
    p.workspace_bytes = kScratchBytes;
  }
  return launch_prefill(p, b.d_k, b.in_dtype, b.out_dtype, stream);
}

}  // extern "C"
