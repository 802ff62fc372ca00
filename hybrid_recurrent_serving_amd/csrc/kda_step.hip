// Token-by-token KDA recurrence on register-resident fp32 state tiles:
// the decode step (one token per sequence, state updated in place) and
// speculative verification (T_spec tokens, commit at the accepted length).
//
// Decode and verify are bound by HBM: per (sequence, head) the whole
// d_k x d_v fp32 state is read once and written at most once, and there are
// only ~1-7 flops per state byte.  Each wavefront owns a COLS-wide column
// slice of one head's state (all d_k rows): lane (rg, cg) holds rows
// [rg*RPL, rg*RPL + RPL) x columns [4cg, 4cg + 4) of the slice, loaded and
// stored as 16-byte vectors, so one load instruction covers RG rows x
// (COLS * 4) contiguous bytes.  The reductions over key channels
// (S^T k and S^T q) only cross lanes of the same wave (shuffles).  The
// token inputs (k, q, v, exp(g), beta for all tokens of the call) are staged
// in LDS by one round of loads that overlaps the state load, and the outputs
// are staged there and stored after the last token, so the token loop itself
// touches no global memory except the state commit.
//
// Recurrence (per token, decay first, correction against the decayed state,
// output from the updated state):
//     S <- Diag(exp g) S;  w = S^T k;  S <- S + beta k (v - w)^T;  o = scale S^T q
// which is (I - beta k k^T) Diag(alpha) S + beta k v^T followed by
// o = S^T q ("Kimi K3 + vLLM: Inside the Day-0 Production Integration",
// section "Kimi Delta Attention: When Prefix Caching Meets Recurrent State",
// describes the fixed-size matrix state; the update rule is the gated delta
// rule with per-key-channel decay).

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int D>
struct StepLayout {
  static constexpr int COLS = D < 32 ? D : 32;  // columns per wave
  static constexpr int LPR = COLS / 4;          // lanes per row (4 columns each)
  static constexpr int RG = 64 / LPR;           // row groups per wave
  static constexpr int RPL = D / RG;            // rows per lane
  static constexpr int WPH = D / COLS;          // waves per head
  static_assert(RPL >= 1 && RPL * RG == D, "layout");
};

// the decode step at d = 128 (defined below, after the fused conv decode)
template <typename Tin, typename Tout> static int launch_decode128_plain(const StepParams& p, hipStream_t stream);
template <typename Tin, typename Tout> static int launch_decode128_conv(const DecodeConvParams& p, hipStream_t stream);

constexpr int STEP_TMAX = 16;   // most tokens per sequence in one call

// STAGED: token inputs and outputs go through LDS (several tokens per call);
// without it (one token, the decode step) every lane loads its own rows and
// stores its own outputs directly.
template <int D, typename Tin, typename Tout, bool STAGED>
__global__ void __launch_bounds__(64 * StepLayout<D>::WPH)
step_kernel(const StepParams p) {
  using L = StepLayout<D>;
  constexpr int NTH = 64 * L::WPH;
  // per-token inputs of this (sequence, head), staged once: alpha = exp(g),
  // k, q (fp32, [token][row]), v ([token][col]), beta; outputs staged the
  // same way and stored after the last token
  // dynamic LDS sized for the call's T_spec: five [T_spec][D] fp32 arrays
  // (alpha, k, q, v, o) and beta (one slot per thread: every thread stores one)
  extern __shared__ __align__(16) float s_dyn[];
  const int TD = p.T_spec * D;
  float* const s_a = s_dyn;
  float* const s_k = s_dyn + TD;
  float* const s_q = s_dyn + 2 * TD;
  float* const s_v = s_dyn + 3 * TD;
  float* const s_o = s_dyn + 4 * TD;
  float* const s_b = s_dyn + 5 * TD;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t sh = blockIdx.x;
  const int s = static_cast<int>(sh / p.H);
  const int h = static_cast<int>(sh % p.H);
  const int cg = lane % L::LPR;
  const int rg = lane / L::LPR;
  const int col = wave * L::COLS + 4 * cg;
  const int row0 = rg * L::RPL;

  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots;

  // commit bookkeeping: Lc = number of tokens after which the state is stored
  int Lc = -1;
  bool valid = false;
  if (p.commit_all) {
    Lc = p.T_spec;
    valid = true;
  } else if (p.accepted_len) {
    Lc = p.accepted_len[s];
    valid = Lc >= 0 && Lc <= p.T_spec;
    if (h == 0 && threadIdx.x == 0 && p.committed_len_out) p.committed_len_out[s] = valid ? Lc : -1;
  }
  const bool do_store = valid && has_dst;
  const int n_tok = p.o ? p.T_spec : (valid ? Lc : 0);

  const Tin* qb = static_cast<const Tin*>(p.q);
  const Tin* kb = static_cast<const Tin*>(p.k);
  const Tin* vb = static_cast<const Tin*>(p.v);
  const Tin* gb = static_cast<const Tin*>(p.g);
  const Tin* bb = static_cast<const Tin*>(p.beta);
  float S[L::RPL][4];
  if constexpr (STAGED) {
    // The token inputs are requested before the state slice, NE groups of 4
    // elements per thread and tensor (sized for the longest window; groups
    // past the end repeat the last one, so every load and LDS store is
    // unconditional and none is sunk behind a condition), plus one beta per
    // thread.  The load counter is in order: staging them in LDS then waits
    // only for them, with the state loads still in flight.
    constexpr int NE = (STEP_TMAX * D / 4 + NTH - 1) / NTH;
    constexpr int NW4 = 4 * sizeof(Tin) / 4;   // 32-bit words per 4 elements
    typedef __attribute__((ext_vector_type(NW4))) uint32_t raw4;
    const int last = n_tok * D - 4 > 0 ? n_tok * D - 4 : 0;
    raw4 rk[NE], rq[NE], rv[NE], rgg[NE];
#pragma unroll
    for (int t = 0; t < NE; ++t) {
      const int e0 = 4 * (t * NTH + static_cast<int>(threadIdx.x));
      const int e = e0 < last ? e0 : last;
      const int j = e / D, c = e % D;
      const int64_t off = static_cast<int64_t>(s) * p.T_spec + j;
      const int64_t hc = static_cast<int64_t>(h) * D + c;
      rk[t] = *reinterpret_cast<const raw4*>(kb + off * p.k_stride + hc);
      rq[t] = *reinterpret_cast<const raw4*>(qb + off * p.q_stride + hc);
      rv[t] = *reinterpret_cast<const raw4*>(vb + off * p.v_stride + hc);
      rgg[t] = *reinterpret_cast<const raw4*>(gb + off * p.g_stride + hc);
    }
    const int jb = static_cast<int>(threadIdx.x) < p.T_spec ? static_cast<int>(threadIdx.x) : p.T_spec - 1;
    const Tin braw = bb[(static_cast<int64_t>(s) * p.T_spec + jb) * p.beta_stride + h];
    // the state slice (zeros without a source: a buffer resource of size 0)
    {
      const float* head = p.pool + (static_cast<int64_t>(has_src ? src : 0) * p.H + h) * D * D;
      const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(head, has_src ? D * D * 4 : 0);
      const int vo = (row0 * D + col) * 4;
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, i * D * 4, kBufNonTemporal);
        S[i][0] = __uint_as_float(x[0]); S[i][1] = __uint_as_float(x[1]);
        S[i][2] = __uint_as_float(x[2]); S[i][3] = __uint_as_float(x[3]);
      }
    }
    auto unpack = [](const raw4& r, float (&x)[4]) __attribute__((always_inline)) {
      if constexpr (sizeof(Tin) == 2) {
        x[0] = __uint_as_float(r[0] << 16); x[1] = __uint_as_float(r[0] & 0xffff0000u);
        x[2] = __uint_as_float(r[1] << 16); x[3] = __uint_as_float(r[1] & 0xffff0000u);
      } else {
        x[0] = __uint_as_float(r[0]); x[1] = __uint_as_float(r[1]);
        x[2] = __uint_as_float(r[2]); x[3] = __uint_as_float(r[3]);
      }
    };
#pragma unroll
    for (int t = 0; t < NE; ++t) {
      const int e0 = 4 * (t * NTH + static_cast<int>(threadIdx.x));
      const int e = e0 < last ? e0 : last;
      float k4[4], q4[4], v4[4], g4[4];
      unpack(rk[t], k4); unpack(rq[t], q4); unpack(rv[t], v4); unpack(rgg[t], g4);
      *reinterpret_cast<float4*>(&s_k[e]) = make_float4(k4[0], k4[1], k4[2], k4[3]);
      *reinterpret_cast<float4*>(&s_q[e]) = make_float4(q4[0], q4[1], q4[2], q4[3]);
      *reinterpret_cast<float4*>(&s_v[e]) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      *reinterpret_cast<float4*>(&s_a[e]) = make_float4(expf(g4[0]), expf(g4[1]), expf(g4[2]), expf(g4[3]));
    }
    s_b[threadIdx.x] = io<Tin>::ld(&braw);
    __syncthreads();
  } else {
    // state slice
    if (has_src) {
      const float* sp = p.pool + ((static_cast<int64_t>(src) * p.H + h) * D + row0) * D + col;
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) ld4_stream(sp + static_cast<int64_t>(i) * D, S[i]);
    } else {
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
    }
  }

  // the destination slice through a buffer resource: one scalar base and the
  // lane offset, no per-row 64-bit addresses held across the token loop
  const __amdgpu_buffer_rsrc_t rd =
      uniform_rsrc(p.pool + (static_cast<int64_t>(has_dst ? dst : 0) * p.H + h) * D * D, has_dst ? D * D * 4 : 0);
  const int vd = (row0 * D + col) * 4;
  if (do_store && Lc == 0) {
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) st4_rsrc(rd, vd, i * D * 4, S[i]);
  }

  for (int j = 0; j < n_tok; ++j) {
    float kr[L::RPL], qr[L::RPL], ar[L::RPL], vc[4];
    float beta;
    const int64_t tok = static_cast<int64_t>(s) * p.T_spec + j;
    if constexpr (STAGED) {
#pragma unroll
      for (int i = 0; i < L::RPL; i += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(&s_k[j * D + row0 + i]);
        const float4 q4 = *reinterpret_cast<const float4*>(&s_q[j * D + row0 + i]);
        const float4 a4 = *reinterpret_cast<const float4*>(&s_a[j * D + row0 + i]);
        kr[i] = k4.x; kr[i + 1] = k4.y; kr[i + 2] = k4.z; kr[i + 3] = k4.w;
        qr[i] = q4.x; qr[i + 1] = q4.y; qr[i + 2] = q4.z; qr[i + 3] = q4.w;
        ar[i] = a4.x; ar[i + 1] = a4.y; ar[i + 2] = a4.z; ar[i + 3] = a4.w;
      }
      const float4 v4 = *reinterpret_cast<const float4*>(&s_v[j * D + col]);
      vc[0] = v4.x; vc[1] = v4.y; vc[2] = v4.z; vc[3] = v4.w;
      beta = s_b[j];
    } else {
      const int64_t hr = static_cast<int64_t>(h) * D + row0;
      ld_vec<Tin, L::RPL>(kb + tok * p.k_stride + hr, kr);
      ld_vec<Tin, L::RPL>(qb + tok * p.q_stride + hr, qr);
      ld_vec<Tin, L::RPL>(gb + tok * p.g_stride + hr, ar);
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) ar[i] = expf(ar[i]);
      io<Tin>::ld4(vb + tok * p.v_stride + static_cast<int64_t>(h) * D + col, vc);
      beta = io<Tin>::ld(bb + tok * p.beta_stride + h);
    }

    // Diag(alpha) S and the partial prediction S^T k over this lane's rows
    float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S[i][c] *= ar[i];
        w[c] = fmaf(S[i][c], kr[i], w[c]);
      }
    }
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = wave_sum_from<L::LPR>(w[c]);
      u[c] = beta * (vc[c] - w[c]);
    }
    // rank-1 correction and the output read-out from the updated state
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S[i][c] = fmaf(kr[i], u[c], S[i][c]);
        o[c] = fmaf(S[i][c], qr[i], o[c]);
      }
    }
    if (p.o) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = wave_sum_from<L::LPR>(o[c]) * p.scale;
      if (rg == 0) {
        if constexpr (STAGED) {
          *reinterpret_cast<float4*>(&s_o[j * D + col]) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
          io<Tout>::st4(static_cast<Tout*>(p.o) + tok * p.o_stride + static_cast<int64_t>(h) * D + col, o);
        }
      }
    }
    if (do_store && j + 1 == Lc) {
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) st4_rsrc(rd, vd, i * D * 4, S[i]);
    }
  }
  if (STAGED && p.o) {
    __syncthreads();
    Tout* ob = static_cast<Tout*>(p.o);
    for (int e = 4 * threadIdx.x; e < n_tok * D; e += 4 * NTH) {
      const int j = e / D, c = e % D;
      const float4 o4 = *reinterpret_cast<const float4*>(&s_o[j * D + c]);
      const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
      io<Tout>::st4(ob + (static_cast<int64_t>(s) * p.T_spec + j) * p.o_stride + static_cast<int64_t>(h) * D + c, ov);
    }
  }
}

template <int D, typename Tin, typename Tout>
static int launch_step_t(const StepParams& p, hipStream_t stream) {
  using L = StepLayout<D>;
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  dim3 block(64 * L::WPH);
  if (p.T_spec == 1) {
    // The streaming layout serves the plain decode step only (outputs, store
    // after the token); a one-token verify keeps its commit semantics
    // (accepted length 0 / rejected, commit index, commit-only calls without
    // outputs) in the general step kernel.
    if constexpr (D == 128) {
      if (p.commit_all && p.o) return launch_decode128_plain<Tin, Tout>(p, stream);
    }
    hipLaunchKernelGGL((step_kernel<D, Tin, Tout, false>), grid, block, 0, stream, p);
  } else {
    if constexpr (D == 128 && std::is_same<Tin, bf16_t>::value) {
      if (!p.commit_all) return launch_verify_mfma(p, std::is_same<Tout, float>::value ? KDA_F32 : KDA_BF16, stream);
    }
    const size_t lds = (5 * static_cast<size_t>(p.T_spec) * D + 64 * L::WPH) * sizeof(float);
    hipLaunchKernelGGL((step_kernel<D, Tin, Tout, true>), grid, block, lds, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "step kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <int D>
static int launch_step_d(const StepParams& p, int in_dtype, int out_dtype, hipStream_t stream) {
  if (in_dtype == KDA_BF16 && out_dtype == KDA_BF16) return launch_step_t<D, bf16_t, bf16_t>(p, stream);
  if (in_dtype == KDA_BF16 && out_dtype == KDA_F32) return launch_step_t<D, bf16_t, float>(p, stream);
  if (in_dtype == KDA_F32 && out_dtype == KDA_BF16) return launch_step_t<D, float, bf16_t>(p, stream);
  return launch_step_t<D, float, float>(p, stream);
}

// ---------------------------------------------------------------------------
// Decode step with the short convolution fused in.  The workgroup of a
// (sequence, head) first issues its state-slice loads (the bulk of the
// traffic), then forms the head's q, k, v from the raw projections: one
// 16-byte vector of V channels per conv item, 3 d / V items (q, k and v
// blocks), each reading its taps, its conv history and the token, writing
// y (fp32) to LDS and the advanced history to the conv pool.  After one
// barrier every wave reads the q / k norms from LDS (redundantly, no second
// barrier) and runs the decode step of step_kernel on LDS operands.
template <typename T> struct Vec16x;
template <> struct Vec16x<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void ld(const bf16_t* p, float (&x)[8]) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
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
      w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Vec16x<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void ld(const float* p, float (&x)[4]) { io<float>::ld4(p, x); }
  __device__ static __forceinline__ void st(float* p, const float (&x)[4]) { io<float>::st4(p, x); }
};


template <int D, typename Tin, typename Tout, int W>
__global__ void __launch_bounds__(64 * StepLayout<D>::WPH)
decode_conv_kernel(const DecodeConvParams p) {
  using L = StepLayout<D>;
  constexpr int V = Vec16x<Tin>::N;       // channels per conv item
  constexpr int NCI = 3 * D / V;          // conv items of one head
  constexpr int HW = W - 1;               // history length
  static_assert(NCI <= 64 * L::WPH, "one conv item per thread");
  __shared__ __align__(16) float s_y[3 * D];   // q | k | v of this head (fp32)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t sh = blockIdx.x;
  const int s = static_cast<int>(sh / p.H);
  const int h = static_cast<int>(sh % p.H);
  const int cg = lane % L::LPR;
  const int rg = lane / L::LPR;
  const int col = wave * L::COLS + 4 * cg;
  const int row0 = rg * L::RPL;

  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots;

  // The conv items' few loads go out first, then the state slice (the bulk
  // of the traffic): the convolution is then done while the slice streams in.
  const bool conv_item = static_cast<int>(threadIdx.x) < NCI;
  const int t = conv_item ? static_cast<int>(threadIdx.x) : 0;
  const int blk = t / (D / V);                 // 0 q, 1 k, 2 v
  const int cc = (t % (D / V)) * V;            // channel inside the head's block
  const int64_t C = 3LL * p.H * D;
  const int64_t ch = static_cast<int64_t>(blk) * p.H * D + static_cast<int64_t>(h) * D + cc;
  const int csrc = p.csrc[s];
  const int cdst = p.cdst[s];
  const bool has_hist = conv_item && csrc >= 0 && csrc < p.n_cslots;
  // taps: the V * W values of channels ch .. ch + V - 1 are contiguous
  // (W 16-byte vectors), tapf[b][e] = weight[(b V + e) / W, (b V + e) % W];
  // history likewise (W - 1 vectors); the token (one vector)
  float tapf[W][V], histf[HW > 0 ? HW : 1][V], xt[V];
  if (conv_item) {
    const Tin* wp = static_cast<const Tin*>(p.w) + ch * W;
#pragma unroll
    for (int b = 0; b < W; ++b) Vec16x<Tin>::ld(wp + b * V, tapf[b]);
    Vec16x<Tin>::ld(static_cast<const Tin*>(p.x) + static_cast<int64_t>(s) * p.x_stride + ch, xt);
  }
  if (has_hist) {
    const Tin* hp = static_cast<const Tin*>(p.cpool) + (static_cast<int64_t>(csrc) * C + ch) * HW;
#pragma unroll
    for (int b = 0; b < HW; ++b) Vec16x<Tin>::ld(hp + b * V, histf[b]);
  }

  float S[L::RPL][4];
  if (has_src) {
    const float* sp = p.pool + ((static_cast<int64_t>(src) * p.H + h) * D + row0) * D + col;
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) ld4_stream(sp + static_cast<int64_t>(i) * D, S[i]);
  } else {
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
  }
  // decay and beta of this lane's rows
  const Tin* gb = static_cast<const Tin*>(p.g);
  float ar[L::RPL];
  ld_vec<Tin, L::RPL>(gb + static_cast<int64_t>(s) * p.g_stride + static_cast<int64_t>(h) * D + row0, ar);
  const float beta = io<Tin>::ld(static_cast<const Tin*>(p.beta) + static_cast<int64_t>(s) * p.beta_stride + h);

  // ---- convolution of this head's q, k, v channels
  if (conv_item) {
    float wt[V][W], hist[V][HW > 0 ? HW : 1];
#pragma unroll
    for (int b = 0; b < W; ++b)
#pragma unroll
      for (int e = 0; e < V; ++e) wt[(b * V + e) / W][(b * V + e) % W] = tapf[b][e];
#pragma unroll
    for (int b = 0; b < HW; ++b)
#pragma unroll
      for (int e = 0; e < V; ++e) hist[(b * V + e) / HW][(b * V + e) % HW] = has_hist ? histf[b][e] : 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      // tap W-1 multiplies the token, tap j < W-1 the history value j
      float acc = p.bias ? io<Tin>::ld(static_cast<const Tin*>(p.bias) + ch + i) : 0.f;
#pragma unroll
      for (int j = 0; j < HW; ++j) acc = fmaf(wt[i][j], hist[i][j], acc);
      acc = fmaf(wt[i][HW], xt[i], acc);
      if (p.act == 1) acc = silu_fast(acc);
      s_y[blk * D + cc + i] = acc;
    }
    // advanced history: hist[1 .. W-2] ++ token
    if (cdst >= 0 && cdst < p.n_cslots) {
      float nh[V * HW];
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < HW; ++j) nh[i * HW + j] = j + 1 < HW ? hist[i][j + 1] : xt[i];
      Tin* np_ = static_cast<Tin*>(p.cpool) + (static_cast<int64_t>(cdst) * C + ch) * HW;
#pragma unroll
      for (int b = 0; b < HW; ++b) {
        float f[V];
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = nh[b * V + e];
        Vec16x<Tin>::st(np_ + b * V, f);
      }
    }
  }
  __syncthreads();

  // ---- q / k normalisation factors (every wave, from LDS)
  float inv_q = 1.f, inv_k = 1.f;
  if (p.qk_l2norm) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) {
      sq = fmaf(s_y[c], s_y[c], sq);
      sk = fmaf(s_y[D + c], s_y[D + c], sk);
    }
    sq = wave_sum_from<1>(sq);
    sk = wave_sum_from<1>(sk);
    inv_q = 1.f / sqrtf(sq + p.eps);
    inv_k = 1.f / sqrtf(sk + p.eps);
  }

  // ---- the decode step on LDS operands (as step_kernel)
  float kr[L::RPL], qr[L::RPL], vc[4];
#pragma unroll
  for (int i = 0; i < L::RPL; ++i) {
    qr[i] = s_y[row0 + i] * inv_q;
    kr[i] = s_y[D + row0 + i] * inv_k;
    ar[i] = expf(ar[i]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) vc[c] = s_y[2 * D + col + c];
  float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S[i][c] *= ar[i];
      w[c] = fmaf(S[i][c], kr[i], w[c]);
    }
  }
  float u[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    w[c] = wave_sum_from<L::LPR>(w[c]);
    u[c] = beta * (vc[c] - w[c]);
  }
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S[i][c] = fmaf(kr[i], u[c], S[i][c]);
      o[c] = fmaf(S[i][c], qr[i], o[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = wave_sum_from<L::LPR>(o[c]) * p.scale;
  Tout* const orow = static_cast<Tout*>(p.o) + static_cast<int64_t>(s) * p.o_stride + static_cast<int64_t>(h) * D;
  if (p.ogate) {
    // gated RMS norm over the head's D outputs: they are gathered in LDS and
    // the first D / 4 lanes of wave 0 take 4 each
    __shared__ __align__(16) float s_ob[D];
    if (rg == 0) *reinterpret_cast<float4*>(&s_ob[col]) = make_float4(o[0], o[1], o[2], o[3]);
    __syncthreads();
    if (threadIdx.x < D / 4) {
      const int c4 = 4 * threadIdx.x;
      const float4 x = *reinterpret_cast<const float4*>(&s_ob[c4]);
      float ov[4] = {x.x, x.y, x.z, x.w};
      gate_norm4<D, Tin>(ov, static_cast<const Tin*>(p.ogate) + static_cast<int64_t>(s) * p.ogate_stride +
                                 static_cast<int64_t>(h) * D + c4,
                         static_cast<const Tin*>(p.onorm_w) + c4, p.onorm_eps);
      io<Tout>::st4(orow + c4, ov);
    }
  } else if (rg == 0) {
    io<Tout>::st4(orow + col, o);
  }
  if (has_dst) {
    float* dp = p.pool + ((static_cast<int64_t>(dst) * p.H + h) * D + row0) * D + col;
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) st4_stream(dp + static_cast<int64_t>(i) * D, S[i]);
  }
}

template <int D, typename Tin, typename Tout>
static int launch_decode_conv_t(const DecodeConvParams& p, hipStream_t stream) {
  if constexpr (D == 128) return launch_decode128_conv<Tin, Tout>(p, stream);
  using L = StepLayout<D>;
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  dim3 block(64 * L::WPH);
  switch (p.W) {
    case 2: hipLaunchKernelGGL((decode_conv_kernel<D, Tin, Tout, 2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((decode_conv_kernel<D, Tin, Tout, 3>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_conv_kernel<D, Tin, Tout, 4>), grid, block, 0, stream, p); break;
    default: return fail(KDA_ERR_UNSUPPORTED, "decode_conv: W = %d (2..4)", p.W);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode_conv kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <int D>
static int launch_decode_conv_d(const DecodeConvParams& p, int in_dtype, int out_dtype, hipStream_t stream) {
  if (in_dtype == KDA_BF16 && out_dtype == KDA_BF16) return launch_decode_conv_t<D, bf16_t, bf16_t>(p, stream);
  if (in_dtype == KDA_BF16 && out_dtype == KDA_F32) return launch_decode_conv_t<D, bf16_t, float>(p, stream);
  if (in_dtype == KDA_F32 && out_dtype == KDA_BF16) return launch_decode_conv_t<D, float, bf16_t>(p, stream);
  return launch_decode_conv_t<D, float, float>(p, stream);
}

int launch_decode_conv(const DecodeConvParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  switch (D) {
    case 16: return launch_decode_conv_d<16>(p, in_dtype, out_dtype, stream);
    case 32: return launch_decode_conv_d<32>(p, in_dtype, out_dtype, stream);
    case 64: return launch_decode_conv_d<64>(p, in_dtype, out_dtype, stream);
    case 128: return launch_decode_conv_d<128>(p, in_dtype, out_dtype, stream);
    default: return fail(KDA_ERR_UNSUPPORTED, "d = %d not built (16, 32, 64, 128)", D);
  }
}

// ---------------------------------------------------------------------------
// The decode step at d = 128, plain (W = 0) or with the short convolution
// fused in (W >= 2), laid out for streaming: one workgroup of four waves per
// (sequence, head), wave w owning the 64 x 64 block of rows
// [64 (w >> 1), + 64) and columns [64 (w & 1), + 64).  Lane l holds columns
// 64 (w & 1) + 4 (l & 15) .. + 3 of the sixteen rows 64 (w >> 1) + (l >> 4) + 4 j:
// each of its sixteen 16-byte accesses covers, across the wave, 256
// contiguous bytes of four consecutive rows.  A copy-only probe of the
// decode's 268 MB of state (read, a reduction over the rows, write back in
// place) took 44.8 us in this layout against 48.4-49.0 us with four rows
// per lane in 8- or 16-wave workgroups: a wave keeps 16 KiB of state in
// flight rather than 4 KiB.
//
// Every token-level load (q, k, v, g or the conv inputs, beta, the output
// gate and norm weight) is issued before the state loads, as raw bits, and
// the state loads go through a buffer resource that has size 0 when the
// source slot is absent (every load returns 0): the loads are then issued on
// every path, and since the load counter is in order, the token work waits
// for its own loads only while the state is in flight, and the first pass
// takes the state rows as they arrive.
//
// Pass 1 forms Diag(alpha) S and, over the lane's rows, the partial S^T k
// and (Diag(alpha) S)^T q, reduced across the four lane groups of the wave by
// the permlane swaps and then over the two row halves through LDS, in a
// fixed order.  The read-out of the updated state follows without a second
// pass over it: S'^T q = (Diag(alpha) S)^T q + u (k . q).  Pass 2 is the
// rank-1 correction S' = Diag(alpha) S + k u^T alone, each row stored (plain
// non-temporal global stores) as soon as it is formed.  With the read-out
// after the update, the compiler issued the sixteen stores after both passes
// of FMAs (and buffer stores measured slower still): 48.9-49.1 us per fused
// step and 48.9-49.0 us per plain step, against 47.8-47.9 and 46.4-46.5 us
// for this form.
// The per-row values (alpha = exp g, k, q) sit in LDS in lane-group order,
// row r at (r & 3) * 32 + (r >> 2), so that a lane reads its sixteen rows as
// four 16-byte vectors.
struct Dec128Args {
  const void *q, *k, *v;                // plain inputs [n_seq, H, 128] (W = 0)
  const void *x, *w, *bias;             // conv inputs (W >= 2)
  void* cpool;
  const int32_t *csrc, *cdst;
  int64_t x_stride, n_cslots;
  int32_t act, qk_l2norm;
  float eps;
  const void *g, *beta;
  void* o;
  float* pool;
  const int32_t *src_slot, *dst_slot;
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride, n_slots;
  int32_t n_seq, H;
  float scale;
  const void *ogate, *onorm_w;          // gated RMS norm of the output (conv form), or NULL
  int64_t ogate_stride;
  float onorm_eps;
};

namespace d128 {
constexpr int D = 128;
constexpr int NW = 4;                   // waves per workgroup: (row half, column half)
constexpr int NT = 64 * NW;
constexpr int RPL = 16;                 // rows per lane
// LDS position of row r in lane-group order
__device__ __forceinline__ int grp_pos(int r) { return (r & 3) * (D / 4) + (r >> 2); }

// four consecutive elements as raw bits (8 bytes of bf16, 16 of fp32),
// converted where they are first used
template <typename T> struct raw4;
template <> struct raw4<bf16_t> {
  typedef uint2 type;
  __device__ static __forceinline__ type ld(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static __forceinline__ void cvt(const type r, float (&x)[4]) {
    x[0] = __uint_as_float(r.x << 16);
    x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16);
    x[3] = __uint_as_float(r.y & 0xffff0000u);
  }
  __device__ static __forceinline__ type zero() { return make_uint2(0u, 0u); }
};
template <> struct raw4<float> {
  typedef float4 type;
  __device__ static __forceinline__ type ld(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static __forceinline__ void cvt(const type r, float (&x)[4]) {
    x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
  }
  __device__ static __forceinline__ type zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
}  // namespace d128

template <typename Tin, typename Tout, int W>
__global__ void __launch_bounds__(d128::NT) __attribute__((amdgpu_waves_per_eu(4)))
decode128_kernel(const Dec128Args p) {
  using namespace d128;
  using R4 = raw4<Tin>;
  constexpr bool CONV = W >= 2;
  constexpr int HW = CONV ? W - 1 : 1;  // history length
  constexpr int NTAP = CONV ? W : 1;
  __shared__ __align__(16) float s_q[D], s_k[D], s_a[D], s_v[D];   // q, k, alpha in lane-group order; v
  __shared__ __align__(16) float s_w[NW][64], s_o[NW][64];          // per-wave S^T k, (Diag(alpha) S)^T q
  __shared__ __align__(16) float s_gz[CONV ? D : 4], s_gw[CONV ? D : 4];   // output gate and norm weight
  const int t = static_cast<int>(threadIdx.x);
  const int lane = t & 63;
  const int wave = t >> 6;
  const int rh = wave >> 1;             // row half
  const int cb = wave & 1;              // column half
  const int grp = lane >> 4;
  const int lc = 4 * (lane & 15);
  const int col = 64 * cb + lc;
  const int s = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x % p.H);
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots;

  // Token-level inputs.  Thread t handles the 4 channels c4 .. c4 + 3 of
  // role t >> 5: 0 q, 1 k, 2 v (the conv of those channels when W >= 2),
  // 3 g, 4 the output gate, 5 the output norm weight (gated output only).
  const int role = t >> 5;
  const int c4 = 4 * (t & 31);
  typename R4::type xr = R4::zero();
  typename R4::type tr[NTAP], hr[HW];
  typename R4::type br = R4::zero();    // bias
  const int64_t C = 3LL * p.H * D;
  const int64_t ch = static_cast<int64_t>(role) * p.H * D + static_cast<int64_t>(h) * D + c4;
  bool has_hist = false;
  if (role < 3) {
    if constexpr (CONV) {
      // taps of channels ch .. ch + 3 (4 W contiguous values), the token, the history (4 (W - 1) values)
      const Tin* wp = static_cast<const Tin*>(p.w) + ch * W;
#pragma unroll
      for (int b = 0; b < W; ++b) tr[b] = R4::ld(wp + 4 * b);
      xr = R4::ld(static_cast<const Tin*>(p.x) + static_cast<int64_t>(s) * p.x_stride + ch);
      const int cs = p.csrc[s];
      has_hist = cs >= 0 && cs < p.n_cslots;
      // without a history slot the address is this thread's taps (valid for
      // any slot count, 0 included) and the values read are replaced by zeros
      const Tin* hp = has_hist ? static_cast<const Tin*>(p.cpool) + (static_cast<int64_t>(cs) * C + ch) * HW : wp;
#pragma unroll
      for (int b = 0; b < HW; ++b) hr[b] = has_hist ? R4::ld(hp + 4 * b) : R4::zero();
      if (p.bias) br = R4::ld(static_cast<const Tin*>(p.bias) + ch);
    } else {
      const Tin* base = role == 0 ? static_cast<const Tin*>(p.q) + static_cast<int64_t>(s) * p.q_stride
                      : role == 1 ? static_cast<const Tin*>(p.k) + static_cast<int64_t>(s) * p.k_stride
                                  : static_cast<const Tin*>(p.v) + static_cast<int64_t>(s) * p.v_stride;
      xr = R4::ld(base + static_cast<int64_t>(h) * D + c4);
    }
  } else if (role == 3) {
    xr = R4::ld(static_cast<const Tin*>(p.g) + static_cast<int64_t>(s) * p.g_stride + static_cast<int64_t>(h) * D + c4);
  } else if (CONV && p.ogate && role < 6) {
    xr = R4::ld(role == 4 ? static_cast<const Tin*>(p.ogate) + static_cast<int64_t>(s) * p.ogate_stride +
                                static_cast<int64_t>(h) * D + c4
                          : static_cast<const Tin*>(p.onorm_w) + c4);
  }
  const float beta = io<Tin>::ld(static_cast<const Tin*>(p.beta) + static_cast<int64_t>(s) * p.beta_stride + h);

  // the state block, in flight while the token work runs (an absent source
  // reads through a resource of size 0)
  float S[RPL][4];
  const int voff = ((64 * rh + grp) * D + col) * 4;
  {
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(
        p.pool + (static_cast<int64_t>(has_src ? src : 0) * p.H + h) * D * D, has_src ? D * D * 4 : 0);
#pragma unroll
    for (int j = 0; j < RPL; ++j) ld4_rsrc(rs, voff + 16 * j * D, S[j]);
  }

  // token work into LDS
  if (role < 3) {
    float y[4];
    if constexpr (CONV) {
      float tv[W * 4], hv[HW * 4], xv[4];
#pragma unroll
      for (int b = 0; b < W; ++b) {
        float f[4];
        R4::cvt(tr[b], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[4 * b + e] = f[e];
      }
#pragma unroll
      for (int b = 0; b < HW; ++b) {
        float f[4];
        R4::cvt(hr[b], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[4 * b + e] = f[e];
      }
      R4::cvt(xr, xv);
      float bv[4];
      R4::cvt(br, bv);
      // channel i: tap W-1 multiplies the token, tap j < W-1 the history value j
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = bv[i];
#pragma unroll
        for (int j = 0; j < HW; ++j) acc = fmaf(tv[i * W + j], hv[i * HW + j], acc);
        acc = fmaf(tv[i * W + HW], xv[i], acc);
        y[i] = p.act == 1 ? silu_fast(acc) : acc;
      }
      // advanced history: values 1 .. W-2 then the token (read and rewritten by this thread only)
      const int cd = p.cdst[s];
      if (cd >= 0 && cd < p.n_cslots) {
        Tin* np_ = static_cast<Tin*>(p.cpool) + (static_cast<int64_t>(cd) * C + ch) * HW;
#pragma unroll
        for (int b = 0; b < HW; ++b) {
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = (4 * b + e) / HW, j = (4 * b + e) % HW;
            f[e] = j + 1 < HW ? hv[i * HW + j + 1] : xv[i];
          }
          io<Tin>::st4(np_ + 4 * b, f);
        }
      }
    } else {
      R4::cvt(xr, y);
    }
    if (role == 2) {
      *reinterpret_cast<float4*>(&s_v[c4]) = make_float4(y[0], y[1], y[2], y[3]);
    } else {
      float* dq = role == 0 ? s_q : s_k;
#pragma unroll
      for (int i = 0; i < 4; ++i) dq[grp_pos(c4 + i)] = y[i];
    }
  } else if (role == 3) {
    float gv[4];
    R4::cvt(xr, gv);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_a[grp_pos(c4 + i)] = expf(gv[i]);
  } else if (CONV && p.ogate && role < 6) {
    // the output gate as sigmoid(z), the norm weight as it is
    float f[4];
    R4::cvt(xr, f);
    if (role == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = sigmoid_fast(f[i]);
    }
    *reinterpret_cast<float4*>(role == 4 ? &s_gz[c4] : &s_gw[c4]) = make_float4(f[0], f[1], f[2], f[3]);
  }
  __syncthreads();

  float inv_q = 1.f, inv_k = 1.f;
  if (CONV && p.qk_l2norm) {
    float sq = s_q[lane] * s_q[lane];
    sq = fmaf(s_q[lane + 64], s_q[lane + 64], sq);
    float sk = s_k[lane] * s_k[lane];
    sk = fmaf(s_k[lane + 64], s_k[lane + 64], sk);
    sq = wave_sum_from<1>(sq);
    sk = wave_sum_from<1>(sk);
    inv_q = 1.f / sqrtf(sq + p.eps);
    inv_k = 1.f / sqrtf(sk + p.eps);
  }
  const int rp = grp * (D / 4) + 16 * rh;   // LDS position of the lane's first row

  // As the rows arrive: Diag(alpha) S, the partial S^T k and the partial
  // read-out (Diag(alpha) S)^T q over the lane's rows, then over the wave's
  // (the read-out of the updated state follows from the latter as
  // S'^T q = (Diag(alpha) S)^T q + u (k . q)), then the two row halves
  float w[4] = {0.f, 0.f, 0.f, 0.f};
  float oq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < RPL / 4; ++jj) {
    const float4 a4 = *reinterpret_cast<const float4*>(&s_a[rp + 4 * jj]);
    const float4 k4 = *reinterpret_cast<const float4*>(&s_k[rp + 4 * jj]);
    const float4 q4 = *reinterpret_cast<const float4*>(&s_q[rp + 4 * jj]);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    const float kv[4] = {k4.x * inv_k, k4.y * inv_k, k4.z * inv_k, k4.w * inv_k};
    const float qv[4] = {q4.x * inv_q, q4.y * inv_q, q4.z * inv_q, q4.w * inv_q};
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S[4 * jj + e][c] *= av[e];
        w[c] = fmaf(S[4 * jj + e][c], kv[e], w[c]);
        oq[c] = fmaf(S[4 * jj + e][c], qv[e], oq[c]);
      }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    w[c] = wave_sum_from<16>(w[c]);
    oq[c] = wave_sum_from<16>(oq[c]);
  }
  if (grp == 0) {
    *reinterpret_cast<float4*>(&s_w[wave][lc]) = make_float4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<float4*>(&s_o[wave][lc]) = make_float4(oq[0], oq[1], oq[2], oq[3]);
  }
  __syncthreads();
  // u = beta (v - S^T k) of columns c0 .. c0 + 3, both row halves in order
  auto delta = [&](int c0, float (&u)[4]) {
    const int half = c0 >> 6, cc = c0 & 63;
    const float4 a = *reinterpret_cast<const float4*>(&s_w[half][cc]);
    const float4 b = *reinterpret_cast<const float4*>(&s_w[2 + half][cc]);
    const float4 v4 = *reinterpret_cast<const float4*>(&s_v[c0]);
    u[0] = beta * (v4.x - (a.x + b.x));
    u[1] = beta * (v4.y - (a.y + b.y));
    u[2] = beta * (v4.z - (a.z + b.z));
    u[3] = beta * (v4.w - (a.w + b.w));
  };
  if (has_dst) {
    // rank-1 correction and the state out (the outputs do not read it)
    float u[4];
    delta(col, u);
    float* dp = p.pool + ((static_cast<int64_t>(dst) * p.H + h) * D + 64 * rh + grp) * D + col;
#pragma unroll
    for (int jj = 0; jj < RPL / 4; ++jj) {
      const float4 k4 = *reinterpret_cast<const float4*>(&s_k[rp + 4 * jj]);
      const float kv[4] = {k4.x * inv_k, k4.y * inv_k, k4.z * inv_k, k4.w * inv_k};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int c = 0; c < 4; ++c) S[4 * jj + e][c] = fmaf(kv[e], u[c], S[4 * jj + e][c]);
        st4_stream(dp + static_cast<int64_t>(4 * (4 * jj + e)) * D, S[4 * jj + e]);
      }
    }
  }
  if (wave == 0) {
    // k . q over the head (every lane of the wave), then the outputs of
    // columns 4 t .. 4 t + 3 on lanes t < D / 4
    float kq = s_k[lane] * s_q[lane];
    kq = fmaf(s_k[lane + 64], s_q[lane + 64], kq);
    kq = wave_sum_from<1>(kq) * (inv_k * inv_q);
    if (t < D / 4) {
      float u[4];
      delta(4 * t, u);
      const int half = t >> 4, cc = 4 * (t & 15);
      const float4 a = *reinterpret_cast<const float4*>(&s_o[half][cc]);
      const float4 b = *reinterpret_cast<const float4*>(&s_o[2 + half][cc]);
      float ov[4] = {fmaf(u[0], kq, a.x + b.x) * p.scale, fmaf(u[1], kq, a.y + b.y) * p.scale,
                     fmaf(u[2], kq, a.z + b.z) * p.scale, fmaf(u[3], kq, a.w + b.w) * p.scale};
      if (CONV && p.ogate) {
        // gated RMS norm: the D outputs are held 4 per lane by lanes 0 .. D/4 - 1
        float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
        ss = group_sum<D / 4>(ss);
        const float inv = 1.f / sqrtf(ss * (1.f / D) + p.onorm_eps);
#pragma unroll
        for (int c = 0; c < 4; ++c) ov[c] = ov[c] * inv * s_gw[4 * t + c] * s_gz[4 * t + c];
      }
      io<Tout>::st4(static_cast<Tout*>(p.o) + static_cast<int64_t>(s) * p.o_stride + static_cast<int64_t>(h) * D + 4 * t,
                    ov);
    }
  }
}

template <typename Tin, typename Tout, int W>
static int launch_decode128(const Dec128Args& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.n_seq) * a.H));
  hipLaunchKernelGGL((decode128_kernel<Tin, Tout, W>), grid, dim3(d128::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <typename Tin, typename Tout>
static int launch_decode128_plain(const StepParams& p, hipStream_t stream) {
  Dec128Args a{};
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta; a.o = p.o; a.pool = p.pool;
  a.src_slot = p.src_slot; a.dst_slot = p.dst_slot;
  a.q_stride = p.q_stride; a.k_stride = p.k_stride; a.v_stride = p.v_stride; a.g_stride = p.g_stride;
  a.beta_stride = p.beta_stride; a.o_stride = p.o_stride; a.n_slots = p.n_slots;
  a.n_seq = p.n_seq; a.H = p.H; a.scale = p.scale;
  return launch_decode128<Tin, Tout, 0>(a, stream);
}

template <typename Tin, typename Tout>
static int launch_decode128_conv(const DecodeConvParams& p, hipStream_t stream) {
  Dec128Args a{};
  a.x = p.x; a.w = p.w; a.bias = p.bias; a.cpool = p.cpool; a.csrc = p.csrc; a.cdst = p.cdst;
  a.x_stride = p.x_stride; a.n_cslots = p.n_cslots; a.act = p.act; a.qk_l2norm = p.qk_l2norm; a.eps = p.eps;
  a.g = p.g; a.beta = p.beta; a.o = p.o; a.pool = p.pool; a.src_slot = p.src_slot; a.dst_slot = p.dst_slot;
  a.g_stride = p.g_stride; a.beta_stride = p.beta_stride; a.o_stride = p.o_stride; a.n_slots = p.n_slots;
  a.n_seq = p.n_seq; a.H = p.H; a.scale = p.scale;
  a.ogate = p.ogate; a.onorm_w = p.onorm_w; a.ogate_stride = p.ogate_stride; a.onorm_eps = p.onorm_eps;
  switch (p.W) {
    case 2: return launch_decode128<Tin, Tout, 2>(a, stream);
    case 3: return launch_decode128<Tin, Tout, 3>(a, stream);
    case 4: return launch_decode128<Tin, Tout, 4>(a, stream);
    default: return fail(KDA_ERR_UNSUPPORTED, "decode_conv: W = %d (2..4)", p.W);
  }
}

// ---------------------------------------------------------------------------
// Speculative verify with the short convolution fused in.  As the staged
// verify of step_kernel, with q, k, v of the T_spec tokens formed by the
// short convolution of the head's q, k, v channels (+ SiLU) and q / k
// normalised per token in the same pass (the conv items of one block are
// adjacent lanes).  The conv history is committed with the state: the W-1 raw
// inputs ending at token L-1.
//
// Every conv input of the workgroup (history, taps, bias, the token rows of
// the head's channels, the gates) is requested first, as 16-byte units
// spread over all threads, then the state slice: the load counter is in
// order, so the conv can run from LDS once its own units have arrived while
// the state is still in flight.  A state source that is absent reads through
// a buffer resource of size 0 (every load returns 0), so the state loads are
// issued on every path and no wait has to cover them early.

// 16-byte units of conv inputs staged per workgroup: history [3][D][W-1],
// taps [3][D][W], bias [3][D], token rows [n_tok][3][D], gates [n_tok][D]
template <int D, typename Tin, int W>
__host__ __device__ constexpr int vconv_units(int n_tok) {
  constexpr int UPB = D * static_cast<int>(sizeof(Tin)) / 16;
  return 3 * (W - 1) * UPB + 3 * W * UPB + 3 * UPB + n_tok * 4 * UPB;
}
// staged units per thread for windows of up to TB tokens, and the staging
// area in units: every thread stores all of its units (those past the end
// into the area's tail), so no load sits behind a condition the compiler
// could sink it into.  The area is sized by the window bucket (8 or 16
// tokens), not the longest window: at 8 tokens it keeps the workgroup's LDS
// small enough for four workgroups per CU.
template <int D, typename Tin, int W, int TB>
__host__ __device__ constexpr int vconv_per_thread() {
  return (vconv_units<D, Tin, W>(TB) + 64 * StepLayout<D>::WPH - 1) / (64 * StepLayout<D>::WPH);
}
template <int D, typename Tin, int W, int TB>
__host__ __device__ constexpr int vconv_stage_units() {
  return vconv_per_thread<D, Tin, W, TB>() * 64 * StepLayout<D>::WPH;
}

template <int D, typename Tin, typename Tout, int W, int TB>
__global__ void __launch_bounds__(64 * StepLayout<D>::WPH)
verify_conv_kernel(const DecodeConvParams p) {
  using L = StepLayout<D>;
  constexpr int NTH = 64 * L::WPH;
  constexpr int V = Vec16x<Tin>::N;       // channels per 16-byte unit
  constexpr int UPB = D / V;              // units per D channels
  constexpr int NCI = 3 * D / V;          // conv items per token
  constexpr int HW = W - 1;
  constexpr int U_HIST = 3 * HW * UPB;
  constexpr int U_TAPS = 3 * W * UPB;
  constexpr int U_FIX = U_HIST + U_TAPS + 3 * UPB;
  constexpr int NU = vconv_per_thread<D, Tin, W, TB>();   // staged units per thread
  static_assert(NCI <= NTH, "one conv item per thread");
  extern __shared__ __align__(16) float s_dyn[];
  const int T = p.T_spec;
  const int TD = T * D;
  uint4* const stg = reinterpret_cast<uint4*>(s_dyn);              // staged units
  float* const fl = s_dyn + 4 * vconv_stage_units<D, Tin, W, TB>();
  float* const s_a = fl;               // exp(g) [T][D]
  float* const s_k = fl + TD;          // k [T][D]
  float* const s_q = fl + 2 * TD;      // q [T][D]
  float* const s_v = fl + 3 * TD;      // v [T][D]
  float* const s_b = fl + 4 * TD;      // beta [T] (one slot per thread: every thread stores one)
  // the conv history element-major, [W-1][3][D] (16-byte rows like the tokens)
  Tin* const s_h = reinterpret_cast<Tin*>(fl + 4 * TD + NTH);
  float* const s_o = s_dyn;            // o [T][D], over the staged units (dead once the conv has run)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t sh = blockIdx.x;
  const int s = static_cast<int>(sh / p.H);
  const int h = static_cast<int>(sh % p.H);
  const int cg = lane % L::LPR;
  const int rg = lane / L::LPR;
  const int col = wave * L::COLS + 4 * cg;
  const int row0 = rg * L::RPL;

  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots;
  int Lc = -1;
  bool valid = false;
  if (p.accepted_len) {
    Lc = p.accepted_len[s];
    valid = Lc >= 0 && Lc <= T;
    if (h == 0 && tid == 0 && p.committed_len_out) p.committed_len_out[s] = valid ? Lc : -1;
  }
  const bool do_store = valid && has_dst;
  const int n_tok = p.o ? T : (valid ? Lc : 0);

  const int64_t C = 3LL * p.H * D;
  const int64_t HD = static_cast<int64_t>(p.H) * D;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int csrc = p.csrc[s];
  const int cdst = p.cdst[s];
  const bool hist_ok = csrc >= 0 && csrc < p.n_cslots;
  const Tin* const wt = static_cast<const Tin*>(p.w);
  const Tin* const xs = static_cast<const Tin*>(p.x) + static_cast<int64_t>(s) * T * p.x_stride;
  const Tin* const hs = static_cast<const Tin*>(p.cpool) + static_cast<int64_t>(hist_ok ? csrc : 0) * C * HW;
  const Tin* const bs = static_cast<const Tin*>(p.bias);
  const Tin* const gs = static_cast<const Tin*>(p.g) + static_cast<int64_t>(s) * T * p.g_stride;

  // 1. conv input units (an absent history or bias reads the taps instead;
  //    every thread issues NU loads, those past the end repeat the last
  //    unit), and beta
  const int n_units = U_FIX + 4 * UPB * n_tok;
  uint4 raw[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    {
      const int u = k * NTH + tid < n_units ? k * NTH + tid : n_units - 1;
      const Tin* a;
      if (u < U_HIST) {
        const int blk = u / (HW * UPB), r = u % (HW * UPB);
        a = hist_ok ? hs + (blk * HD + hd) * HW + r * V : wt;
      } else if (u < U_HIST + U_TAPS) {
        const int v = u - U_HIST, blk = v / (W * UPB), r = v % (W * UPB);
        a = wt + (blk * HD + hd) * W + r * V;
      } else if (u < U_FIX) {
        const int v = u - U_HIST - U_TAPS, blk = v / UPB, r = v % UPB;
        a = bs ? bs + blk * HD + hd + r * V : wt;
      } else if (u < U_FIX + 3 * UPB * n_tok) {
        const int v = u - U_FIX, t = v / (3 * UPB), r = v % (3 * UPB);
        a = xs + t * p.x_stride + (r / UPB) * HD + hd + (r % UPB) * V;
      } else {
        const int v = u - U_FIX - 3 * UPB * n_tok, t = v / UPB, r = v % UPB;
        a = gs + t * p.g_stride + hd + r * V;
      }
      raw[k] = *reinterpret_cast<const uint4*>(a);
    }
  }
  const Tin braw = static_cast<const Tin*>(p.beta)[(static_cast<int64_t>(s) * T + (tid < T ? tid : T - 1)) *
                                                      p.beta_stride + h];

  // 2. the state slice (zeros when there is no source)
  float S[L::RPL][4];
  {
    const float* head = p.pool + (static_cast<int64_t>(has_src ? src : 0) * p.H + h) * D * D;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(head, has_src ? D * D * 4 : 0);
    const int vo = (row0 * D + col) * 4;
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, i * D * 4, kBufNonTemporal);
      S[i][0] = __uint_as_float(x[0]); S[i][1] = __uint_as_float(x[1]);
      S[i][2] = __uint_as_float(x[2]); S[i][3] = __uint_as_float(x[3]);
    }
  }

  // 3. units and beta to LDS; the history units also scattered element-major
  //    (zeros without a history: those units hold taps)
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    stg[k * NTH + tid] = raw[k];
    const int u = k * NTH + tid;
    if (u < U_HIST) {
      const int blk = u / (HW * UPB), r = u % (HW * UPB);
      const Tin* el = reinterpret_cast<const Tin*>(&raw[k]);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int f = r * V + e;             // element ch * HW + q of the block
        const int ch = f / HW, q = f % HW;
        s_h[(q * 3 + blk) * D + ch] = hist_ok ? el[e] : Tin(0);
      }
    }
  }
  s_b[tid] = io<Tin>::ld(&braw);
  __syncthreads();

  // 4. exp(g), the convolution y = bias + sum_k w[k] xbar[j + k] (+ SiLU)
  //    with xbar = history ++ tokens, and the new conv history
  //    xbar[Lc .. Lc + W - 2], all from the staged units
  const Tin* const st = reinterpret_cast<const Tin*>(stg);
  const Tin* const st_taps = st + U_HIST * V;
  const Tin* const st_bias = st + (U_HIST + U_TAPS) * V;
  const Tin* const st_x = st + U_FIX * V;
  const Tin* const st_g = st_x + 3 * D * n_tok;
  for (int e = 4 * tid; e < n_tok * D; e += 4 * NTH) {
    float g4[4];
    io<Tin>::ld4(st_g + e, g4);
    *reinterpret_cast<float4*>(&s_a[e]) = make_float4(expf(g4[0]), expf(g4[1]), expf(g4[2]), expf(g4[3]));
  }
  // xbar[idx] of channels cc .. cc + V - 1 of block blk
  auto xbar = [&](const int idx, const int blk, const int cc, float (&x)[V]) __attribute__((always_inline)) {
    if (idx >= HW) {
      Vec16x<Tin>::ld(st_x + (static_cast<int64_t>(idx - HW) * 3 + blk) * D + cc, x);
    } else {
      Vec16x<Tin>::ld(s_h + (idx * 3 + blk) * D + cc, x);
    }
  };
  for (int it = tid; it < n_tok * NCI; it += NTH) {
    const int c = it % NCI, j = it / NCI;
    const int blk = c / UPB, cc = (c % UPB) * V;
    float tapf[W][V], xbf[W][V];
#pragma unroll
    for (int b = 0; b < W; ++b) Vec16x<Tin>::ld(st_taps + (blk * D + cc) * W + b * V, tapf[b]);
#pragma unroll
    for (int k = 0; k < W; ++k) xbar(j + k, blk, cc, xbf[k]);
    float* yb = blk == 0 ? s_q : (blk == 1 ? s_k : s_v);
    float yv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float acc = bs ? io<Tin>::ld(st_bias + blk * D + cc + i) : 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) acc = fmaf(tapf[(i * W + k) / V][(i * W + k) % V], xbf[k][i], acc);
      yv[i] = p.act == 1 ? silu_fast(acc) : acc;
    }
    // q / k normalisation of token j: the UPB items of a block are adjacent
    // lanes (a block starts at a multiple of UPB, so does every item group)
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) ss = fmaf(yv[i], yv[i], ss);
    ss = group_sum<UPB>(ss);
    const float inv = (p.qk_l2norm && blk < 2) ? 1.f / sqrtf(ss + p.eps) : 1.f;
#pragma unroll
    for (int i = 0; i < V; i += 4)
      *reinterpret_cast<float4*>(&yb[j * D + cc + i]) =
          make_float4(yv[i] * inv, yv[i + 1] * inv, yv[i + 2] * inv, yv[i + 3] * inv);
  }
  if (valid && cdst >= 0 && cdst < p.n_cslots && tid < NCI) {
    const int blk = tid / UPB, cc = (tid % UPB) * V;
    float nh[V * HW];
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      float val[V];
      xbar(Lc + j, blk, cc, val);
#pragma unroll
      for (int i = 0; i < V; ++i) nh[i * HW + j] = val[i];
    }
    Tin* np_ = static_cast<Tin*>(p.cpool) + (static_cast<int64_t>(cdst) * C + blk * HD + hd + cc) * HW;
#pragma unroll
    for (int b = 0; b < HW; ++b) {
      float f[V];
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = nh[b * V + e];
      Vec16x<Tin>::st(np_ + b * V, f);
    }
  }
  __syncthreads();

  // the destination slice through a buffer resource: one scalar base and the
  // lane offset, no per-row 64-bit addresses held across the token loop
  const __amdgpu_buffer_rsrc_t rd =
      uniform_rsrc(p.pool + (static_cast<int64_t>(has_dst ? dst : 0) * p.H + h) * D * D, has_dst ? D * D * 4 : 0);
  const int vd = (row0 * D + col) * 4;
  if (do_store && Lc == 0) {
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) st4_rsrc(rd, vd, i * D * 4, S[i]);
  }
  for (int j = 0; j < n_tok; ++j) {
    float kr[L::RPL], qr[L::RPL], ar[L::RPL], vc[4];
#pragma unroll
    for (int i = 0; i < L::RPL; i += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&s_k[j * D + row0 + i]);
      const float4 q4 = *reinterpret_cast<const float4*>(&s_q[j * D + row0 + i]);
      const float4 a4 = *reinterpret_cast<const float4*>(&s_a[j * D + row0 + i]);
      kr[i] = k4.x; kr[i + 1] = k4.y; kr[i + 2] = k4.z; kr[i + 3] = k4.w;
      qr[i] = q4.x; qr[i + 1] = q4.y; qr[i + 2] = q4.z; qr[i + 3] = q4.w;
      ar[i] = a4.x; ar[i + 1] = a4.y; ar[i + 2] = a4.z; ar[i + 3] = a4.w;
    }
    const float4 v4 = *reinterpret_cast<const float4*>(&s_v[j * D + col]);
    vc[0] = v4.x; vc[1] = v4.y; vc[2] = v4.z; vc[3] = v4.w;
    const float beta = s_b[j];
    float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S[i][c] *= ar[i];
        w[c] = fmaf(S[i][c], kr[i], w[c]);
      }
    }
    float uk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = wave_sum_from<L::LPR>(w[c]);
      uk[c] = beta * (vc[c] - w[c]);
    }
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < L::RPL; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S[i][c] = fmaf(kr[i], uk[c], S[i][c]);
        o[c] = fmaf(S[i][c], qr[i], o[c]);
      }
    }
    if (p.o) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = wave_sum_from<L::LPR>(o[c]) * p.scale;
      if (rg == 0) *reinterpret_cast<float4*>(&s_o[j * D + col]) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (do_store && j + 1 == Lc) {
#pragma unroll
      for (int i = 0; i < L::RPL; ++i) st4_rsrc(rd, vd, i * D * 4, S[i]);
    }
  }
  if (p.o) {
    __syncthreads();
    Tout* ob = static_cast<Tout*>(p.o);
    // a token's D outputs are stored by D / 4 consecutive lanes (the gated
    // norm sums across exactly those lanes; every iteration covers whole
    // tokens, so the lanes of a token are active together)
    for (int e = 4 * threadIdx.x; e < n_tok * D; e += 4 * NTH) {
      const int j = e / D, c = e % D;
      const float4 o4 = *reinterpret_cast<const float4*>(&s_o[j * D + c]);
      float ov[4] = {o4.x, o4.y, o4.z, o4.w};
      if (p.ogate)
        gate_norm4<D, Tin>(ov, static_cast<const Tin*>(p.ogate) + (static_cast<int64_t>(s) * T + j) * p.ogate_stride +
                                   static_cast<int64_t>(h) * D + c,
                           static_cast<const Tin*>(p.onorm_w) + c, p.onorm_eps);
      io<Tout>::st4(ob + (static_cast<int64_t>(s) * T + j) * p.o_stride + static_cast<int64_t>(h) * D + c, ov);
    }
  }
}

template <int D, typename Tin, typename Tout>
static int launch_verify_conv_t(const DecodeConvParams& p, hipStream_t stream) {
  if constexpr (D == 128 && std::is_same<Tin, bf16_t>::value) {
    if (p.T_spec >= 2) return launch_verify_conv_mfma(p, std::is_same<Tout, float>::value ? KDA_F32 : KDA_BF16, stream);
  }
  using L = StepLayout<D>;
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  dim3 block(64 * L::WPH);
  const size_t fl = (4 * static_cast<size_t>(p.T_spec) * D + 64 * L::WPH) * sizeof(float) +
                    (static_cast<size_t>(p.W - 1) * 3 * D * sizeof(Tin) + 15) / 16 * 16;
  // the window bucket: every kernel instance stages at most TB tokens
  auto go = [&](auto w_t, auto tb_t) {
    constexpr int W = decltype(w_t)::value, TB = decltype(tb_t)::value;
    const size_t lds = 16 * static_cast<size_t>(vconv_stage_units<D, Tin, W, TB>()) + fl;
    hipLaunchKernelGGL((verify_conv_kernel<D, Tin, Tout, W, TB>), grid, block, lds, stream, p);
  };
  auto go_w = [&](auto w_t) {
    if (p.T_spec <= 8) go(w_t, std::integral_constant<int, 8>{});
    else go(w_t, std::integral_constant<int, STEP_TMAX>{});
  };
  switch (p.W) {
    case 2: go_w(std::integral_constant<int, 2>{}); break;
    case 3: go_w(std::integral_constant<int, 3>{}); break;
    case 4: go_w(std::integral_constant<int, 4>{}); break;
    default: return fail(KDA_ERR_UNSUPPORTED, "verify_conv: W = %d (2..4)", p.W);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "verify_conv kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <int D>
static int launch_verify_conv_d(const DecodeConvParams& p, int in_dtype, int out_dtype, hipStream_t stream) {
  if (in_dtype == KDA_BF16 && out_dtype == KDA_BF16) return launch_verify_conv_t<D, bf16_t, bf16_t>(p, stream);
  if (in_dtype == KDA_BF16 && out_dtype == KDA_F32) return launch_verify_conv_t<D, bf16_t, float>(p, stream);
  if (in_dtype == KDA_F32 && out_dtype == KDA_BF16) return launch_verify_conv_t<D, float, bf16_t>(p, stream);
  return launch_verify_conv_t<D, float, float>(p, stream);
}

int launch_verify_conv(const DecodeConvParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  switch (D) {
    case 16: return launch_verify_conv_d<16>(p, in_dtype, out_dtype, stream);
    case 32: return launch_verify_conv_d<32>(p, in_dtype, out_dtype, stream);
    case 64: return launch_verify_conv_d<64>(p, in_dtype, out_dtype, stream);
    case 128: return launch_verify_conv_d<128>(p, in_dtype, out_dtype, stream);
    default: return fail(KDA_ERR_UNSUPPORTED, "d = %d not built (16, 32, 64, 128)", D);
  }
}

int launch_step(const StepParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  switch (D) {
    case 16: return launch_step_d<16>(p, in_dtype, out_dtype, stream);
    case 32: return launch_step_d<32>(p, in_dtype, out_dtype, stream);
    case 64: return launch_step_d<64>(p, in_dtype, out_dtype, stream);
    case 128: return launch_step_d<128>(p, in_dtype, out_dtype, stream);
    default: return fail(KDA_ERR_UNSUPPORTED, "d = %d not built (16, 32, 64, 128)", D);
  }
}

}  // namespace kda
