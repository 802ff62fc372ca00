// Speculative verification on bf16 matrix cores (gfx950): d_k = d_v = 128,
// bf16 token inputs, 2..16 tokens per sequence.
//
// The T_spec tokens of a (sequence, head) form one chunk of the WY /
// UT-transform form of the gated delta rule -- the form the chunked prefill
// runs ("Kimi K3 + vLLM: Inside the Day-0 Production Integration", section
// "Kimi Delta Attention: When Prefix Caching Meets Recurrent State", names
// the fixed-size matrix state the recurrence carries).  Rows r, s < T_spec of
// a 16-row tile, padding rows zero; G_r = sum_{j<=r} g_j per key channel,
// reference row m = (T_spec - 1) / 2:
//     left_q[r] = q_r exp(G_r - G_m),  left_k[r] = k_r exp(G_r - G_m),
//     right_k[s] = k_s exp(G_m - G_s)
//     A[r,s] = beta_r <left_k[r], right_k[s]> (s < r),  T = (I + A)^{-1} diag(beta)
//     S' = Diag(exp G_m) S,   u = T V - (T left_k) S'
//     O  = scale (left_q S' + P u),  P[r,s] = <left_q[r], right_k[s]> (s <= r)
// and the state after the first L tokens (the accepted length)
//     S_L = Diag(exp(G_{L-1} - G_m)) (S' + sum_{s<L} right_k[s]^T u[s]),
// since u[s] depends on rows 0..s only.  The reference row depends on
// T_spec alone, so an outputs-only call, a commit-only call and a fused call
// compute bit-identical outputs and states.  Every exponential factor is at
// most exp(decay over 8 tokens).  L = 0 stores the source state as loaded.
//
// Work split: one workgroup of 4 waves per (sequence, head).  Wave w owns
// d_v columns [32 w, 32 w + 32) of the fp32 state as 2 x 8 matrix-core
// accumulator tiles of 16 x 16 (rows d_k), loaded at the start and stored
// at the commit: 4-byte accesses, the two tiles' 64-byte halves of each
// 128-byte row segment issued back to back (with the halves far apart in
// the instruction stream the transfers measured markedly slower).  While the state loads are in flight the waves form the
// chunk's gates, gated operands, A, the solve, P, W and U (the state-free
// part); the state-dependent part (u, O, the state update) then runs on the
// accumulator tiles as they stand.  Registers (at most 128) and LDS (under
// 40 KiB, with buffers of disjoint lifetimes overlaid) are sized for four
// workgroups per compute unit, so that while one workgroup computes, the
// others' state transfers keep HBM busy.
//
// Precision: bf16 operands with fp32 accumulation, every operand that is
// not an exact bf16 input carried as a hi + lo bf16 pair and every product
// taken as hi*hi + hi*lo + lo*hi (A, P, T, W = T left_k, U = T V, u, O and
// the state update), so each product is good to about 2^-17 relative and
// the committed state stays close to fp32 arithmetic.

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace vf {

using namespace mx;

constexpr int D = 128;      // d_k = d_v
constexpr int R = 16;       // rows of the token tile (T_spec <= 16)
constexpr int NW = 4;       // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int PD = D + 16;  // padded pitch of the [R][D] bf16 tiles
constexpr int PT = R + 8;   // padded pitch of the [R][R] bf16 tiles

struct Smem {
  union {
    float G[R][D];                    // g log2(e), then its sum down the rows
    float At[R][R + 1];               // then A transposed: At[s][r] = A[r][s]
  } x;
  union {
    struct {
      alignas(16) bf16_t hi[R][PD];   // left_k [r][pos32(c)]
      alignas(16) bf16_t lo[R][PD];
    } lk;
    struct {
      alignas(16) bf16_t hi[R][PD];   // then -W = -(T left_k) [r][pos32(c)]
      alignas(16) bf16_t lo[R][PD];
    } wn;
  } y;
  alignas(16) bf16_t lq_hi[R][PD];    // left_q [r][pos32(c)]
  alignas(16) bf16_t lq_lo[R][PD];
  alignas(16) bf16_t rk_hi[R][PD];    // right_k [s][pos32(c)]
  alignas(16) bf16_t rk_lo[R][PD];
  alignas(16) float em[D];            // exp2(G_m): the state enters as Diag(em) S
  alignas(16) float ef[D];            // exp2(G_{L-1} - G_m): row factor of the commit
  float beta[R];
  alignas(16) bf16_t P_hi[R][PT];     // P [r][s]
  alignas(16) bf16_t P_lo[R][PT];
  alignas(16) bf16_t T_hi[R][PT];     // T [r][s]
  alignas(16) bf16_t T_lo[R][PT];
};
static_assert(sizeof(Smem) <= 40960, "four workgroups per compute unit");

// one state element through a buffer resource (the whole offset in the
// vector offset, as for st4_rsrc)
__device__ __forceinline__ void st1_rsrc(__amdgpu_buffer_rsrc_t r, int voff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, 0, kBufNonTemporal);
}

// bf16 bits of 4 consecutive elements (8 bytes) -> 4 floats
__device__ __forceinline__ void unpack4(const uint2 w, float* x) {
  x[0] = __uint_as_float(w.x << 16);
  x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16);
  x[3] = __uint_as_float(w.y & 0xffff0000u);
}

// 4 floats -> s16x4 bf16 (hi) and the rounding remainders (lo)
__device__ __forceinline__ void split4(const f32x4& a, s16x4& hi, s16x4& lo) {
  uint32_t h0, l0, h1, l1;
  split2(a[0], a[1], h0, l0);
  split2(a[2], a[3], h1, l1);
  hi = __builtin_bit_cast(s16x4, make_uint2(h0, h1));
  lo = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
}

template <typename Tout>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) verify_kernel(const StepParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int s = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x % p.H);
  const int T = p.T_spec;
  const int m = (T - 1) >> 1;

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
  const bool with_o = p.o != nullptr;
  const int tj = (lane >> 2) & 3, ti = lane & 3;   // transpose-read row and column group

  // ---- token rows: thread (row r, item ib) holds channels c0..c0+3 and
  // c0+16..c0+19, which sit at storage positions 8 ib .. 8 ib + 7
  const int r = tid >> 4;
  const int ib = tid & 15;
  const int c0 = 32 * (ib >> 2) + 4 * (ib & 3);
  f32x4 S[2][D / 16];
  uint2 qw[2] = {make_uint2(0, 0), make_uint2(0, 0)}, kw[2] = {qw[0], qw[1]}, gw[2] = {qw[0], qw[1]};
  // V as the B operands of U = T V: rows 4 g4 .. 4 g4 + 3 of column
  // 32 wave + 16 ct + l16
  uint32_t vw[2][2] = {{0, 0}, {0, 0}};
  bf16_t braw = 0;
  {
    const int64_t hc = static_cast<int64_t>(h) * D;
    if (r < T) {
      const int64_t tok = static_cast<int64_t>(s) * T + r;
      const bf16_t* qp = static_cast<const bf16_t*>(p.q) + tok * p.q_stride + hc + c0;
      const bf16_t* kp = static_cast<const bf16_t*>(p.k) + tok * p.k_stride + hc + c0;
      const bf16_t* gp = static_cast<const bf16_t*>(p.g) + tok * p.g_stride + hc + c0;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        qw[x] = *reinterpret_cast<const uint2*>(qp + 16 * x);
        kw[x] = *reinterpret_cast<const uint2*>(kp + 16 * x);
        gw[x] = *reinterpret_cast<const uint2*>(gp + 16 * x);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 4 * g4 + j;
      if (rr < T) {
        const bf16_t* vp = static_cast<const bf16_t*>(p.v) + (static_cast<int64_t>(s) * T + rr) * p.v_stride + hc +
                           32 * wave + l16;
        vw[0][j >> 1] |= static_cast<uint32_t>(vp[0]) << (16 * (j & 1));
        vw[1][j >> 1] |= static_cast<uint32_t>(vp[16]) << (16 * (j & 1));
      }
    }
    if (tid < T) braw = static_cast<const bf16_t*>(p.beta)[(static_cast<int64_t>(s) * T + tid) * p.beta_stride + h];
    // The state slice (zeros without a source: a buffer resource of size 0),
    // S[ct][q][i] = S[16 q + 4 g4 + i][32 wave + 16 ct + l16].  Requested after
    // the token rows: the load counter is in order, so staging the rows waits
    // for them alone while the state is still in flight.
    const float* head = p.pool + (static_cast<int64_t>(has_src ? src : 0) * p.H + h) * D * D;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(head, has_src ? D * D * 4 : 0);
    const int vo = (4 * g4 * D + 32 * wave + l16) * 4;
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          S[ct][q][i] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 64 * ct, ((16 * q + i) * D) * 4, kBufNonTemporal));
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    float gf[4];
    unpack4(gw[x], gf);
    *reinterpret_cast<float4*>(&sm.x.G[r][c0 + 16 * x]) =
        make_float4(gf[0] * kLog2e, gf[1] * kLog2e, gf[2] * kLog2e, gf[3] * kLog2e);
  }
  if (tid < R) sm.beta[tid] = tid < T ? bf16_to_f32(braw) : 0.f;
  __syncthreads();

  // ---- cumulative gates down the rows (one channel per thread) and the
  // state factors
  if (tid < D) {
    const int c = tid;
    float gl[R];
    float acc = 0.f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      acc += sm.x.G[rr][c];
      gl[rr] = acc;
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) sm.x.G[rr][c] = gl[rr];
    float gm = 0.f, gL = 0.f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      gm = rr == m ? gl[rr] : gm;
      gL = rr == Lc - 1 ? gl[rr] : gL;
    }
    sm.em[c] = __builtin_amdgcn_exp2f(gm);
    sm.ef[c] = __builtin_amdgcn_exp2f(gL - gm);
  }
  __syncthreads();

  // ---- gated operands of this thread's row and channels
  {
    float qx[8], kx[8];
    unpack4(qw[0], qx); unpack4(qw[1], qx + 4);
    unpack4(kw[0], kx); unpack4(kw[1], kx + 4);
    float lq[8], lkv[8], rkv[8];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float4 a = *reinterpret_cast<const float4*>(&sm.x.G[r][c0 + 16 * x]);
      const float4 b = *reinterpret_cast<const float4*>(&sm.x.G[m][c0 + 16 * x]);
      const float d4[4] = {a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * x + e;
        const float ea = __builtin_amdgcn_exp2f(d4[e]);
        lq[i] = qx[i] * ea;
        lkv[i] = kx[i] * ea;
        rkv[i] = kx[i] * __builtin_amdgcn_exp2f(-d4[e]);
      }
    }
    const int pp = 8 * ib;
    st8b_pair(&sm.lq_hi[r][pp], &sm.lq_lo[r][pp], lq);
    st8b_pair(&sm.y.lk.hi[r][pp], &sm.y.lk.lo[r][pp], lkv);
    st8b_pair(&sm.rk_hi[r][pp], &sm.rk_lo[r][pp], rkv);
  }
  __syncthreads();

  // ---- A and the solve (wave 0), P (wave 1)
  if (wave == 0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 ah = frag_lds(&sm.y.lk.hi[l16][32 * ks + 8 * g4]);
      const bf16x8 bh = frag_lds(&sm.rk_hi[l16][32 * ks + 8 * g4]);
      acc = mfma(ah, bh, acc);
      acc = mfma(ah, frag_lds(&sm.rk_lo[l16][32 * ks + 8 * g4]), acc);
      acc = mfma(frag_lds(&sm.y.lk.lo[l16][32 * ks + 8 * g4]), bh, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * g4 + i;
      sm.x.At[l16][rr] = l16 < rr ? acc[i] * sm.beta[rr] : 0.f;
    }
    // the same wave reads A back in the solve's layout
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // T = (I + A)^{-1} diag(beta) by forward substitution down the 16 lanes of
    // a lane row: lane (g4, r = l16) holds row r of columns 4 g + g4
    float na[16];
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) na[s2] = -sm.x.At[s2][l16];
    float xv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) xv[g] = l16 == 4 * g + g4 ? 1.f : 0.f;
    // xv was just written by VALU: two wait states before a DPP read
    asm volatile("s_nop 1" ::"v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]));
    fsub16<0, 4>(xv, na);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = 4 * g + g4;
      const float tv = xv[g] * sm.beta[j];
      const float th = hi_of(tv);
      sm.T_hi[l16][j] = f32_to_bf16(th);
      sm.T_lo[l16][j] = f32_to_bf16(tv - th);
    }
  } else if (wave == 1) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 ah = frag_lds(&sm.lq_hi[l16][32 * ks + 8 * g4]);
      const bf16x8 bh = frag_lds(&sm.rk_hi[l16][32 * ks + 8 * g4]);
      acc = mfma(ah, bh, acc);
      acc = mfma(ah, frag_lds(&sm.rk_lo[l16][32 * ks + 8 * g4]), acc);
      acc = mfma(frag_lds(&sm.lq_lo[l16][32 * ks + 8 * g4]), bh, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * g4 + i;
      const float pv = l16 <= rr ? acc[i] : 0.f;
      const float ph = hi_of(pv);
      sm.P_hi[rr][l16] = f32_to_bf16(ph);
      sm.P_lo[rr][l16] = f32_to_bf16(pv - ph);
    }
  }
  __syncthreads();

  // ---- W = T left_k on storage positions [32 wave, 32 wave + 32); -W then
  // replaces left_k in LDS
  f32x4 Wt[2];
  {
    const s16x4 th4 = *reinterpret_cast<const s16x4*>(&sm.T_hi[l16][4 * g4]);
    const s16x4 tl4 = *reinterpret_cast<const s16x4*>(&sm.T_lo[l16][4 * g4]);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int p0 = 32 * wave + 16 * nt;
      const s16x4 bh = tr4(&sm.y.lk.hi[4 * g4 + tj][p0 + 4 * ti]);
      Wt[nt] = mfma16(th4, bh, z);
      Wt[nt] = mfma16(th4, tr4(&sm.y.lk.lo[4 * g4 + tj][p0 + 4 * ti]), Wt[nt]);
      Wt[nt] = mfma16(tl4, bh, Wt[nt]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int p0 = 32 * wave + 16 * nt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wv = -Wt[nt][i];
      const float wh = hi_of(wv);
      sm.y.wn.hi[4 * g4 + i][p0 + l16] = f32_to_bf16(wh);
      sm.y.wn.lo[4 * g4 + i][p0 + l16] = f32_to_bf16(wv - wh);
    }
  }
  __syncthreads();

  // ---- state-dependent part
  const __amdgpu_buffer_rsrc_t rd =
      uniform_rsrc(p.pool + (static_cast<int64_t>(has_dst ? dst : 0) * p.H + h) * D * D, has_dst ? D * D * 4 : 0);
  const int vd = (4 * g4 * D + 32 * wave + l16) * 4;
  auto store_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) st1_rsrc(rd, vd + 64 * ct + (16 * q + i) * D * 4, S[ct][q][i]);
  };
  if (do_store && Lc == 0) store_state();
  const bool commit = do_store && Lc > 0;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    // U = T V on this tile's d_v columns
    f32x4 u;
    {
      const s16x4 bv = __builtin_bit_cast(s16x4, make_uint2(vw[ct][0], vw[ct][1]));
      const s16x4 th4 = *reinterpret_cast<const s16x4*>(&sm.T_hi[l16][4 * g4]);
      const s16x4 tl4 = *reinterpret_cast<const s16x4*>(&sm.T_lo[l16][4 * g4]);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      u = mfma16(tl4, bv, mfma16(th4, bv, z));
    }
    // S' = Diag(exp G_m) S, then u = U - W S' and left_q S', one pair
    // fragment of S' at a time
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int q = 2 * ks + t;
        const float4 f = *reinterpret_cast<const float4*>(&sm.em[16 * q + 4 * g4]);
        S[ct][q][0] *= f.x; S[ct][q][1] *= f.y; S[ct][q][2] *= f.z; S[ct][q][3] *= f.w;
      }
      bf16x8 sh, sl;
      frag_pair(S[ct][2 * ks], S[ct][2 * ks + 1], sh, sl);
      const bf16x8 wh = frag_lds(&sm.y.wn.hi[l16][32 * ks + 8 * g4]);
      u = mfma(wh, sh, u);
      u = mfma(wh, sl, u);
      u = mfma(frag_lds(&sm.y.wn.lo[l16][32 * ks + 8 * g4]), sh, u);
      if (with_o) {
        const bf16x8 ah = frag_lds(&sm.lq_hi[l16][32 * ks + 8 * g4]);
        o = mfma(ah, sh, o);
        o = mfma(ah, sl, o);
        o = mfma(frag_lds(&sm.lq_lo[l16][32 * ks + 8 * g4]), sh, o);
      }
    }
    s16x4 uh, ul;
    if (with_o) {
      // O = scale (left_q S' + P u)
      split4(u, uh, ul);
      const s16x4 ph = *reinterpret_cast<const s16x4*>(&sm.P_hi[l16][4 * g4]);
      const s16x4 pl = *reinterpret_cast<const s16x4*>(&sm.P_lo[l16][4 * g4]);
      o = mfma16(ph, uh, o);
      o = mfma16(ph, ul, o);
      o = mfma16(pl, uh, o);
      Tout* ob = static_cast<Tout*>(p.o) + static_cast<int64_t>(h) * D + 32 * wave + 16 * ct + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * g4 + i;
        if (rr < T) io<Tout>::st(ob + (static_cast<int64_t>(s) * T + rr) * p.o_stride, o[i] * p.scale);
      }
    }
    if (commit) {
      // S_L = Diag(exp(G_{L-1} - G_m)) (S' + right_k^T u) over rows s < L
      f32x4 um;
#pragma unroll
      for (int i = 0; i < 4; ++i) um[i] = 4 * g4 + i < Lc ? u[i] : 0.f;
      s16x4 ch, cl;
      split4(um, ch, cl);
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        // right_k^T: lane l16 receives channel 16 q + l16 of rows 4 g4 .. 4 g4 + 3
        const int col = 32 * (q >> 1) + 4 * (q & 1) + 8 * ti;
        const s16x4 kh = tr4(&sm.rk_hi[4 * g4 + tj][col]);
        const s16x4 kl = tr4(&sm.rk_lo[4 * g4 + tj][col]);
        S[ct][q] = mfma16(kh, ch, S[ct][q]);
        S[ct][q] = mfma16(kh, cl, S[ct][q]);
        S[ct][q] = mfma16(kl, ch, S[ct][q]);
        const float4 f = *reinterpret_cast<const float4*>(&sm.ef[16 * q + 4 * g4]);
        S[ct][q][0] *= f.x; S[ct][q][1] *= f.y; S[ct][q][2] *= f.z; S[ct][q][3] *= f.w;
      }
    }
  }
  if (commit) store_state();
}

template <typename Tout>
static int launch_t(const StepParams& p, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  hipLaunchKernelGGL((verify_kernel<Tout>), grid, dim3(NT), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "verify kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace vf

int launch_verify_mfma(const StepParams& p, int out_dtype, hipStream_t stream) {
  if (out_dtype == KDA_F32) return vf::launch_t<float>(p, stream);
  return vf::launch_t<bf16_t>(p, stream);
}

}  // namespace kda
