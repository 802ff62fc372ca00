// Speculative verification on bf16 matrix cores (gfx950): d_k = d_v = 128,
// bf16 token inputs, 2..16 tokens per sequence -- kda_verify on q, k, v and
// kda_verify_conv on the tokens' raw q / k / v projections.
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
// the instruction stream the transfers measured markedly slower).  While
// the state loads are in flight the waves form the chunk's gates, gated
// operands, A, the solve, P and W (the state-free part); the state part
// (U, u, O, the state update) then runs on the accumulator tiles as they
// stand.  kda_verify keeps its registers (at most 128) and LDS (under
// 40 KiB, buffers of disjoint lifetimes overlaid) within four workgroups per
// compute unit, so that while one workgroup computes, the others' state
// transfers keep HBM busy.
//
// kda_verify_conv first forms q, k, v from the raw projections as the
// token-loop kernel does (every conv input of the head staged in LDS as
// 16-byte units, the convolution (+ SiLU) and the q / k normalisation spread
// over all threads, fp32 results), commits the conv history, and stages the
// outputs for the gated RMS norm.
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
constexpr int PT = R + 4;   // padded pitch of the [R][R] bf16 tiles (8-byte rows reads)

// LDS of the chunk, in parts of disjoint or overlaid lifetimes
union XPart {
  float G[R][D];              // g log2(e), then its sum down the rows
  float At[R][R + 1];         // then A transposed: At[s][r] = A[r][s]
  float o[R][D];              // then the scaled outputs (kda_verify_conv)
};
union YPart {
  struct {
    alignas(16) bf16_t hi[R][PD];   // left_k [r][pos32(c)]
    alignas(16) bf16_t lo[R][PD];
  } lk;
  struct {
    alignas(16) bf16_t hi[R][PD];   // then -W = -(T left_k) [r][pos32(c)]
    alignas(16) bf16_t lo[R][PD];
  } wn;
};
struct QKPart {
  alignas(16) bf16_t lq_hi[R][PD];  // left_q [r][pos32(c)]
  alignas(16) bf16_t lq_lo[R][PD];
  alignas(16) bf16_t rk_hi[R][PD];  // right_k [s][pos32(c)]
  alignas(16) bf16_t rk_lo[R][PD];
};
struct SmallPart {
  alignas(16) float em[D];          // exp2(G_m): the state enters as Diag(em) S
  alignas(16) float ef[D];          // exp2(G_{L-1} - G_m): row factor of the commit
  float beta[R];
  alignas(16) bf16_t P_hi[R][PT];   // P [r][s]
  alignas(16) bf16_t P_lo[R][PT];
  alignas(16) bf16_t T_hi[R][PT];   // T [r][s]
  alignas(16) bf16_t T_lo[R][PT];
};

struct Smem {
  XPart x;
  YPart y;
  QKPart qk;
  SmallPart sp;
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

// Lane coordinates shared by the phases of the chunk, derived from the thread
// id where they are used (cheaper to recompute than to hold in registers).
struct Lanes {
  int tid;
  __device__ explicit Lanes(int t) : tid(t) {}
  __device__ int wave() const { return tid >> 6; }
  __device__ int g4() const { return (tid & 63) >> 4; }
  __device__ int l16() const { return tid & 15; }
  __device__ int tj() const { return (tid >> 2) & 3; }   // transpose-read row
  __device__ int ti() const { return tid & 3; }          // transpose-read column group
  __device__ int r() const { return tid >> 4; }          // token row
  __device__ int ib() const { return tid & 15; }         // 8-channel item: storage positions 8 ib ..
  __device__ int c0() const { return 32 * ((tid & 15) >> 2) + 4 * (tid & 3); }   // its first channel
};

// ---- the state-free part.  Each step is followed by a workgroup barrier in
// the callers.

// cumulative gates down the rows (one channel per thread, from x.G holding
// g log2 e) and the state factors exp2(G_m), exp2(G_{L-1} - G_m)
__device__ __forceinline__ void cumulative_gates(XPart& x, SmallPart& sp, const Lanes& ln, int m, int Lc) {
  if (ln.tid < D) {
    const int c = ln.tid;
    float acc = 0.f, gm = 0.f, gL = 0.f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      acc += x.G[rr][c];
      x.G[rr][c] = acc;
      gm = rr == m ? acc : gm;
      gL = rr == Lc - 1 ? acc : gL;
    }
    sp.em[c] = __builtin_amdgcn_exp2f(gm);
    sp.ef[c] = __builtin_amdgcn_exp2f(gL - gm);
  }
}

// gated operands of the thread's row and 8 channels from its q and k
__device__ __forceinline__ void gated_operands(const XPart& x, YPart& y, QKPart& qk, const Lanes& ln, int m,
                                               const float (&qx)[8], const float (&kx)[8]) {
  float ea[8], eb[8];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const float4 a = *reinterpret_cast<const float4*>(&x.G[ln.r()][ln.c0() + 16 * h2]);
    const float4 b = *reinterpret_cast<const float4*>(&x.G[m][ln.c0() + 16 * h2]);
    const float d4[4] = {a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ea[4 * h2 + e] = __builtin_amdgcn_exp2f(d4[e]);
      eb[4 * h2 + e] = __builtin_amdgcn_exp2f(-d4[e]);
    }
  }
  const int pp = 8 * ln.ib();
  float yv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) yv[i] = qx[i] * ea[i];
  st8b_pair(&qk.lq_hi[ln.r()][pp], &qk.lq_lo[ln.r()][pp], yv);
#pragma unroll
  for (int i = 0; i < 8; ++i) yv[i] = kx[i] * ea[i];
  st8b_pair(&y.lk.hi[ln.r()][pp], &y.lk.lo[ln.r()][pp], yv);
#pragma unroll
  for (int i = 0; i < 8; ++i) yv[i] = kx[i] * eb[i];
  st8b_pair(&qk.rk_hi[ln.r()][pp], &qk.rk_lo[ln.r()][pp], yv);
}

// A and T = (I + A)^{-1} diag(beta) (wave 0), P (wave 1)
__device__ __forceinline__ void a_solve_p(XPart& x, const YPart& y, const QKPart& qk, SmallPart& sp,
                                          const Lanes& ln) {
  const int g4 = ln.g4(), l16 = ln.l16();
  if (ln.wave() == 0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 ah = frag_lds(&y.lk.hi[l16][32 * ks + 8 * g4]);
      const bf16x8 bh = frag_lds(&qk.rk_hi[l16][32 * ks + 8 * g4]);
      acc = mfma(ah, bh, acc);
      acc = mfma(ah, frag_lds(&qk.rk_lo[l16][32 * ks + 8 * g4]), acc);
      acc = mfma(frag_lds(&y.lk.lo[l16][32 * ks + 8 * g4]), bh, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * g4 + i;
      x.At[l16][rr] = l16 < rr ? acc[i] * sp.beta[rr] : 0.f;
    }
    // the same wave reads A back in the solve's layout
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // forward substitution down the 16 lanes of a lane row: lane (g4, r = l16)
    // holds row r of columns 4 g + g4
    float na[16];
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) na[s2] = -x.At[s2][l16];
    float xv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) xv[g] = l16 == 4 * g + g4 ? 1.f : 0.f;
    // xv was just written by VALU: two wait states before a DPP read
    asm volatile("s_nop 1" ::"v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]));
    fsub16<0, 4>(xv, na);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = 4 * g + g4;
      const float tv = xv[g] * sp.beta[j];
      const float th = hi_of(tv);
      sp.T_hi[l16][j] = f32_to_bf16(th);
      sp.T_lo[l16][j] = f32_to_bf16(tv - th);
    }
  } else if (ln.wave() == 1) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 ah = frag_lds(&qk.lq_hi[l16][32 * ks + 8 * g4]);
      const bf16x8 bh = frag_lds(&qk.rk_hi[l16][32 * ks + 8 * g4]);
      acc = mfma(ah, bh, acc);
      acc = mfma(ah, frag_lds(&qk.rk_lo[l16][32 * ks + 8 * g4]), acc);
      acc = mfma(frag_lds(&qk.lq_lo[l16][32 * ks + 8 * g4]), bh, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * g4 + i;
      const float pv = l16 <= rr ? acc[i] : 0.f;
      const float ph = hi_of(pv);
      sp.P_hi[rr][l16] = f32_to_bf16(ph);
      sp.P_lo[rr][l16] = f32_to_bf16(pv - ph);
    }
  }
}

// W = T left_k on storage positions [32 wave, 32 wave + 32); -W then
// replaces left_k (a workgroup barrier between, inside)
__device__ __forceinline__ void w_products(YPart& y, const SmallPart& sp, const Lanes& ln) {
  const int g4 = ln.g4(), l16 = ln.l16();
  f32x4 Wt[2];
  {
    const s16x4 th4 = *reinterpret_cast<const s16x4*>(&sp.T_hi[l16][4 * g4]);
    const s16x4 tl4 = *reinterpret_cast<const s16x4*>(&sp.T_lo[l16][4 * g4]);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int p0 = 32 * ln.wave() + 16 * nt;
      const s16x4 bh = tr4(&y.lk.hi[4 * g4 + ln.tj()][p0 + 4 * ln.ti()]);
      Wt[nt] = mfma16(th4, bh, z);
      Wt[nt] = mfma16(th4, tr4(&y.lk.lo[4 * g4 + ln.tj()][p0 + 4 * ln.ti()]), Wt[nt]);
      Wt[nt] = mfma16(tl4, bh, Wt[nt]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int p0 = 32 * ln.wave() + 16 * nt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wv = -Wt[nt][i];
      const float wh = hi_of(wv);
      y.wn.hi[4 * g4 + i][p0 + l16] = f32_to_bf16(wh);
      y.wn.lo[4 * g4 + i][p0 + l16] = f32_to_bf16(wv - wh);
    }
  }
}

// ---- the state part: U (u_init(ct)), u, O (out(ct, o) with the scaled
// outputs of rows 4 g4 .. 4 g4 + 3) and the commit of S_L (Lc > 0).  The
// state S[ct][q][i] = S[16 q + 4 g4 + i][32 wave + 16 ct + l16] is scaled in
// place.
template <class UInit, class Out>
__device__ __forceinline__ void state_part(f32x4 (&S)[2][D / 16], const YPart& y, const QKPart& qk,
                                           const SmallPart& sp, const Lanes& ln, bool with_o, bool commit, int Lc,
                                           float scale, UInit&& u_init, Out&& out) {
  const int g4 = ln.g4(), l16 = ln.l16();
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    f32x4 u = u_init(ct);
    // S' = Diag(exp G_m) S, then u = U - W S' and left_q S', one pair
    // fragment of S' at a time
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int q = 2 * ks + t2;
        const float4 f = *reinterpret_cast<const float4*>(&sp.em[16 * q + 4 * g4]);
        S[ct][q][0] *= f.x; S[ct][q][1] *= f.y; S[ct][q][2] *= f.z; S[ct][q][3] *= f.w;
      }
      bf16x8 sh, sl;
      frag_pair(S[ct][2 * ks], S[ct][2 * ks + 1], sh, sl);
      const bf16x8 wh = frag_lds(&y.wn.hi[l16][32 * ks + 8 * g4]);
      u = mfma(wh, sh, u);
      u = mfma(wh, sl, u);
      u = mfma(frag_lds(&y.wn.lo[l16][32 * ks + 8 * g4]), sh, u);
      if (with_o) {
        const bf16x8 ah = frag_lds(&qk.lq_hi[l16][32 * ks + 8 * g4]);
        o = mfma(ah, sh, o);
        o = mfma(ah, sl, o);
        o = mfma(frag_lds(&qk.lq_lo[l16][32 * ks + 8 * g4]), sh, o);
      }
      // the next step's fragments are not read ahead: with the state held,
      // reading all of them at once would not fit in the registers
      __builtin_amdgcn_sched_barrier(0);
    }
    if (with_o) {
      // O = scale (left_q S' + P u)
      s16x4 uh, ul;
      split4(u, uh, ul);
      const s16x4 ph = *reinterpret_cast<const s16x4*>(&sp.P_hi[l16][4 * g4]);
      const s16x4 pl = *reinterpret_cast<const s16x4*>(&sp.P_lo[l16][4 * g4]);
      o = mfma16(ph, uh, o);
      o = mfma16(ph, ul, o);
      o = mfma16(pl, uh, o);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= scale;
      out(ct, o);
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
        const int col = 32 * (q >> 1) + 4 * (q & 1) + 8 * ln.ti();
        const s16x4 kh = tr4(&qk.rk_hi[4 * g4 + ln.tj()][col]);
        const s16x4 kl = tr4(&qk.rk_lo[4 * g4 + ln.tj()][col]);
        S[ct][q] = mfma16(kh, ch, S[ct][q]);
        S[ct][q] = mfma16(kh, cl, S[ct][q]);
        S[ct][q] = mfma16(kl, ch, S[ct][q]);
        const float4 f = *reinterpret_cast<const float4*>(&sp.ef[16 * q + 4 * g4]);
        S[ct][q][0] *= f.x; S[ct][q][1] *= f.y; S[ct][q][2] *= f.z; S[ct][q][3] *= f.w;
      }
    }
  }
}

// the state slice of (slot, head) through a buffer resource (size 0 without
// a slot: every load returns 0), the two tiles' halves of each row segment
// back to back
__device__ __forceinline__ void load_state(f32x4 (&S)[2][D / 16], const float* pool, int slot, int64_t n_slots,
                                           int H, int h, const Lanes& ln) {
  const bool ok = slot >= 0 && slot < n_slots;
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(pool + (static_cast<int64_t>(ok ? slot : 0) * H + h) * D * D,
                                                 ok ? D * D * 4 : 0);
  const int vo = (4 * ln.g4() * D + 32 * ln.wave() + ln.l16()) * 4;
#pragma unroll
  for (int q = 0; q < D / 16; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        S[ct][q][i] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 64 * ct, ((16 * q + i) * D) * 4, kBufNonTemporal));
}
// the state slice to (slot, head); the slot is valid
__device__ __forceinline__ void store_state(const f32x4 (&S)[2][D / 16], float* pool, int slot, int H, int h,
                                            const Lanes& ln) {
  const __amdgpu_buffer_rsrc_t rd = uniform_rsrc(pool + (static_cast<int64_t>(slot) * H + h) * D * D, D * D * 4);
  const int vd = (4 * ln.g4() * D + 32 * ln.wave() + ln.l16()) * 4;
#pragma unroll
  for (int q = 0; q < D / 16; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) st1_rsrc(rd, vd + 64 * ct + (16 * q + i) * D * 4, S[ct][q][i]);
}

// ---------------------------------------------------------------------------
template <typename Tout>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) verify_kernel(const StepParams p) {
  __shared__ Smem sm;
  const Lanes ln(static_cast<int>(threadIdx.x));
  const int s = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x % p.H);
  const int T = p.T_spec;
  const int m = (T - 1) >> 1;
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_dst = dst >= 0 && dst < p.n_slots;
  int Lc = -1;
  bool valid = false;
  if (p.accepted_len) {
    Lc = p.accepted_len[s];
    valid = Lc >= 0 && Lc <= T;
    if (h == 0 && ln.tid == 0 && p.committed_len_out) p.committed_len_out[s] = valid ? Lc : -1;
  }
  const bool do_store = valid && has_dst;
  const bool with_o = p.o != nullptr;

  // ---- requests: the token rows first, then the state (the load counter is
  // in order, so staging the rows waits for them alone while the state is
  // still in flight).  Thread (r, ib) holds q, k, g of row r, channels
  // c0..c0+3 and c0+16..c0+19; vw the B operands of U = T V (rows
  // 4 g4 .. 4 g4 + 3 of column 32 wave + 16 ct + l16).
  uint2 qw[2] = {make_uint2(0, 0), make_uint2(0, 0)}, kw[2] = {qw[0], qw[1]}, gw[2] = {qw[0], qw[1]};
  uint32_t vw[2][2] = {{0, 0}, {0, 0}};
  bf16_t braw = 0;
  f32x4 S[2][D / 16];
  {
    const int64_t hc = static_cast<int64_t>(h) * D;
    if (ln.r() < T) {
      const int64_t tok = static_cast<int64_t>(s) * T + ln.r();
      const bf16_t* qp = static_cast<const bf16_t*>(p.q) + tok * p.q_stride + hc + ln.c0();
      const bf16_t* kp = static_cast<const bf16_t*>(p.k) + tok * p.k_stride + hc + ln.c0();
      const bf16_t* gp = static_cast<const bf16_t*>(p.g) + tok * p.g_stride + hc + ln.c0();
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        qw[x] = *reinterpret_cast<const uint2*>(qp + 16 * x);
        kw[x] = *reinterpret_cast<const uint2*>(kp + 16 * x);
        gw[x] = *reinterpret_cast<const uint2*>(gp + 16 * x);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 4 * ln.g4() + j;
      if (rr < T) {
        const bf16_t* vp = static_cast<const bf16_t*>(p.v) + (static_cast<int64_t>(s) * T + rr) * p.v_stride + hc +
                           32 * ln.wave() + ln.l16();
        vw[0][j >> 1] |= static_cast<uint32_t>(vp[0]) << (16 * (j & 1));
        vw[1][j >> 1] |= static_cast<uint32_t>(vp[16]) << (16 * (j & 1));
      }
    }
    if (ln.tid < T) braw = static_cast<const bf16_t*>(p.beta)[(static_cast<int64_t>(s) * T + ln.tid) * p.beta_stride + h];
    load_state(S, p.pool, src, p.n_slots, p.H, h, ln);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    float gf[4];
    unpack4(gw[x], gf);
    *reinterpret_cast<float4*>(&sm.x.G[ln.r()][ln.c0() + 16 * x]) =
        make_float4(gf[0] * kLog2e, gf[1] * kLog2e, gf[2] * kLog2e, gf[3] * kLog2e);
  }
  if (ln.tid < R) sm.sp.beta[ln.tid] = ln.tid < T ? bf16_to_f32(braw) : 0.f;
  __syncthreads();
  cumulative_gates(sm.x, sm.sp, ln, m, Lc);
  __syncthreads();
  {
    float qx[8], kx[8];
    unpack4(qw[0], qx); unpack4(qw[1], qx + 4);
    unpack4(kw[0], kx); unpack4(kw[1], kx + 4);
    gated_operands(sm.x, sm.y, sm.qk, ln, m, qx, kx);
  }
  __syncthreads();
  a_solve_p(sm.x, sm.y, sm.qk, sm.sp, ln);
  __syncthreads();
  w_products(sm.y, sm.sp, ln);
  __syncthreads();

  if (do_store && Lc == 0) store_state(S, p.pool, dst, p.H, h, ln);
  const bool commit = do_store && Lc > 0;
  // U = T V: V is exact in bf16
  auto u_init = [&](int ct) -> f32x4 {
    const s16x4 bv = __builtin_bit_cast(s16x4, make_uint2(vw[ct][0], vw[ct][1]));
    const s16x4 th4 = *reinterpret_cast<const s16x4*>(&sm.sp.T_hi[ln.l16()][4 * ln.g4()]);
    const s16x4 tl4 = *reinterpret_cast<const s16x4*>(&sm.sp.T_lo[ln.l16()][4 * ln.g4()]);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return mfma16(tl4, bv, mfma16(th4, bv, z));
  };
  auto out = [&](int ct, const f32x4& o) {
    Tout* ob = static_cast<Tout*>(p.o) + static_cast<int64_t>(h) * D + 32 * ln.wave() + 16 * ct + ln.l16();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * ln.g4() + i;
      if (rr < T) io<Tout>::st(ob + (static_cast<int64_t>(s) * T + rr) * p.o_stride, o[i]);
    }
  };
  state_part(S, sm.y, sm.qk, sm.sp, ln, with_o, commit, Lc, p.scale, u_init, out);
  if (commit) store_state(S, p.pool, dst, p.H, h, ln);
}

// ---------------------------------------------------------------------------
// kda_verify_conv.  The conv inputs of the head as 16-byte units of 8
// channels (UPB units per 128 channels): history [3][(W-1) UPB] (the history
// of 128 channels is contiguous), taps [3][W UPB], bias [3][UPB], token rows
// [T][3][UPB], gates [T][UPB].
constexpr int UPB = D / 8;
constexpr int NCI = 3 * UPB;    // conv items (8 channels each) per token

template <int W>
__host__ __device__ constexpr int conv_units(int n_tok) {
  return 3 * (W - 1) * UPB + 3 * W * UPB + 3 * UPB + n_tok * 4 * UPB;
}
template <int W, int TB>
__host__ __device__ constexpr int conv_units_per_thread() {
  return (conv_units<W>(TB) + NT - 1) / NT;
}

template <int W, int TB>
struct SmemConv {
  union {
    struct {
      uint4 units[conv_units<W>(TB)];                    // staged conv inputs
      alignas(16) bf16_t hist[W - 1][3][D];              // the conv history, element-major
      alignas(16) float qkv[TB][3][D];                   // conv outputs: q | k | v (fp32)
    } cv;
    struct {                                             // then the chunk's operands
      QKPart qk;
      YPart y;
    } op;
  } a;
  XPart x;
  SmallPart sp;
};
static_assert(sizeof(SmemConv<4, 8>) <= 40960, "four workgroups per compute unit at up to 8 tokens");

template <typename Tout, int W, int TB>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TB <= 8 ? 4 : 2)))
verify_conv_kernel(const DecodeConvParams p) {
  constexpr int HW = W - 1;
  constexpr int U_HIST = 3 * HW * UPB;
  constexpr int U_TAPS = 3 * W * UPB;
  constexpr int U_FIX = U_HIST + U_TAPS + 3 * UPB;
  constexpr int NU = conv_units_per_thread<W, TB>();
  __shared__ SmemConv<W, TB> sm;
  const Lanes ln(static_cast<int>(threadIdx.x));
  const int tid = ln.tid;
  const int s = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x % p.H);
  const int T = p.T_spec;
  const int m = (T - 1) >> 1;
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
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

  const int64_t HD = static_cast<int64_t>(p.H) * D;
  const int64_t C = 3 * HD;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int csrc = p.csrc[s];
  const int cdst = p.cdst[s];
  const bool hist_ok = csrc >= 0 && csrc < p.n_cslots;
  const bf16_t* const wt = static_cast<const bf16_t*>(p.w);
  const bf16_t* const xs = static_cast<const bf16_t*>(p.x) + static_cast<int64_t>(s) * T * p.x_stride;
  const bf16_t* const hs = static_cast<const bf16_t*>(p.cpool) + static_cast<int64_t>(hist_ok ? csrc : 0) * C * HW;
  const bf16_t* const bs = static_cast<const bf16_t*>(p.bias);
  const bf16_t* const gs = static_cast<const bf16_t*>(p.g) + static_cast<int64_t>(s) * T * p.g_stride;

  // ---- requests: every conv input unit (an absent history or bias reads
  // the taps instead; units past the end repeat the last one), beta, then
  // the state slice
  const int n_units = conv_units<W>(T);
  uint4 raw[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = k * NT + tid < n_units ? k * NT + tid : n_units - 1;
    const bf16_t* a;
    if (u < U_HIST) {
      const int blk = u / (HW * UPB), rr = u % (HW * UPB);
      a = hist_ok ? hs + (blk * HD + hd) * HW + rr * 8 : wt;
    } else if (u < U_HIST + U_TAPS) {
      const int v = u - U_HIST, blk = v / (W * UPB), rr = v % (W * UPB);
      a = wt + (blk * HD + hd) * W + rr * 8;
    } else if (u < U_FIX) {
      const int v = u - U_HIST - U_TAPS, blk = v / UPB, rr = v % UPB;
      a = bs ? bs + blk * HD + hd + rr * 8 : wt;
    } else if (u < U_FIX + 3 * UPB * T) {
      const int v = u - U_FIX, t = v / (3 * UPB), rr = v % (3 * UPB);
      a = xs + t * p.x_stride + (rr / UPB) * HD + hd + (rr % UPB) * 8;
    } else {
      const int v = u - U_FIX - 3 * UPB * T, t = v / UPB, rr = v % UPB;
      a = gs + t * p.g_stride + hd + rr * 8;
    }
    raw[k] = *reinterpret_cast<const uint4*>(a);
  }
  bf16_t braw = 0;
  if (tid < T) braw = static_cast<const bf16_t*>(p.beta)[(static_cast<int64_t>(s) * T + tid) * p.beta_stride + h];
  // the output gate and norm weight of this thread's output units (4
  // channels of one token each) as raw bits, also requested before the
  // state: read at the end they would wait for the state stores as well (the
  // vector memory counter takes loads and stores in issue order).  Padded
  // tokens and an ungated call read valid addresses whose values are unused.
  constexpr int OU = TB * D / 4 / NT;   // output units per thread
  uint2 graw[OU], wraw[OU];
  {
    const bool gated = with_o && p.ogate;
#pragma unroll
    for (int k = 0; k < OU; ++k) {
      const int e = 4 * (k * NT + tid);
      const int j = e / D < T ? e / D : T - 1, c = e % D;
      const bf16_t* gp = gated ? static_cast<const bf16_t*>(p.ogate) + (static_cast<int64_t>(s) * T + j) * p.ogate_stride + hd + c
                               : static_cast<const bf16_t*>(p.x);
      const bf16_t* wp = gated ? static_cast<const bf16_t*>(p.onorm_w) + c : static_cast<const bf16_t*>(p.x);
      graw[k] = *reinterpret_cast<const uint2*>(gp);
      wraw[k] = *reinterpret_cast<const uint2*>(wp);
    }
  }
  f32x4 S[2][D / 16];
  load_state(S, p.pool, src, p.n_slots, p.H, h, ln);

  // ---- units to LDS (every thread stores all of its units, those past the
  // end onto the last slot with the same value, so that no load sits behind
  // a condition); the history units also scattered element-major (zeros
  // without a history: those units hold taps)
  constexpr int SLOTS = conv_units<W>(TB);
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    sm.a.cv.units[k * NT + tid < SLOTS ? k * NT + tid : SLOTS - 1] = raw[k];
    const int u = k * NT + tid;
    if (u < U_HIST) {
      const int blk = u / (HW * UPB), rr = u % (HW * UPB);
      const bf16_t* el = reinterpret_cast<const bf16_t*>(&raw[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = rr * 8 + e;   // element ch * HW + q of the block's history
        sm.a.cv.hist[f % HW][blk][f / HW] = hist_ok ? el[e] : bf16_t(0);
      }
    }
  }
  if (tid < R) sm.sp.beta[tid] = tid < T ? bf16_to_f32(braw) : 0.f;
  __syncthreads();

  // ---- the convolution y = bias + sum_k w[k] xbar[j + k] (+ SiLU), xbar =
  // history ++ tokens, q / k normalised per token; the new conv history
  // xbar[Lc .. Lc + W - 2]; g log2(e) into G
  const bf16_t* const st = reinterpret_cast<const bf16_t*>(sm.a.cv.units);
  const bf16_t* const st_taps = st + U_HIST * 8;
  const bf16_t* const st_bias = st + (U_HIST + U_TAPS) * 8;
  const bf16_t* const st_x = st + U_FIX * 8;
  const bf16_t* const st_g = st_x + 3 * D * T;
  auto xbar = [&](const int idx, const int blk, const int cc, float (&x)[8]) __attribute__((always_inline)) {
    const uint4 w = idx >= HW ? *reinterpret_cast<const uint4*>(st_x + ((idx - HW) * 3 + blk) * D + cc)
                              : *reinterpret_cast<const uint4*>(&sm.a.cv.hist[idx][blk][cc]);
    unpack4(make_uint2(w.x, w.y), x);
    unpack4(make_uint2(w.z, w.w), x + 4);
  };
  for (int it = tid; it < T * NCI; it += NT) {
    const int c = it % NCI, j = it / NCI;
    const int blk = c / UPB, cc = (c % UPB) * 8;
    // taps of channels cc .. cc + 7, tap k of channel cc + i at element i W + k
    // (kept as bf16 bits, widened where used)
    uint32_t tw[4 * W];
#pragma unroll
    for (int b = 0; b < W; ++b) {
      const uint4 w = *reinterpret_cast<const uint4*>(st_taps + (blk * D + cc) * W + 8 * b);
      tw[4 * b] = w.x; tw[4 * b + 1] = w.y; tw[4 * b + 2] = w.z; tw[4 * b + 3] = w.w;
    }
    auto tap = [&](int e) -> float {
      const uint32_t x = tw[e >> 1];
      return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    };
    float yv[8];
    if (bs) {
      const uint4 w = *reinterpret_cast<const uint4*>(st_bias + blk * D + cc);
      unpack4(make_uint2(w.x, w.y), yv);
      unpack4(make_uint2(w.z, w.w), yv + 4);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < W; ++k) {
      float xb[8];
      xbar(j + k, blk, cc, xb);
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = fmaf(tap(i * W + k), xb[i], yv[i]);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (p.act == 1) yv[i] = silu_fast(yv[i]);
      ss = fmaf(yv[i], yv[i], ss);
    }
    // the UPB items of a (token, block) are adjacent lanes
    ss = group_sum<UPB>(ss);
    const float inv = (p.qk_l2norm && blk < 2) ? 1.f / sqrtf(ss + p.eps) : 1.f;
    float* yb = &sm.a.cv.qkv[j][blk][cc];
    *reinterpret_cast<float4*>(yb) = make_float4(yv[0] * inv, yv[1] * inv, yv[2] * inv, yv[3] * inv);
    *reinterpret_cast<float4*>(yb + 4) = make_float4(yv[4] * inv, yv[5] * inv, yv[6] * inv, yv[7] * inv);
  }
  if (valid && cdst >= 0 && cdst < p.n_cslots && tid < NCI) {
    const int blk = tid / UPB, cc = (tid % UPB) * 8;
    float nh[8 * HW];
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      float val[8];
      xbar(Lc + j, blk, cc, val);
#pragma unroll
      for (int i = 0; i < 8; ++i) nh[i * HW + j] = val[i];
    }
    bf16_t* np_ = static_cast<bf16_t*>(p.cpool) + (static_cast<int64_t>(cdst) * C + blk * HD + hd + cc) * HW;
#pragma unroll
    for (int b = 0; b < HW; ++b) st8b(np_ + 8 * b, nh + 8 * b);
  }
  {
    float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ln.r() < T) {
#pragma unroll
      for (int x = 0; x < 2; ++x) unpack4(*reinterpret_cast<const uint2*>(st_g + ln.r() * D + ln.c0() + 16 * x), gv + 4 * x);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
      *reinterpret_cast<float4*>(&sm.x.G[ln.r()][ln.c0() + 16 * x]) =
          make_float4(gv[4 * x] * kLog2e, gv[4 * x + 1] * kLog2e, gv[4 * x + 2] * kLog2e, gv[4 * x + 3] * kLog2e);
  }
  __syncthreads();
  cumulative_gates(sm.x, sm.sp, ln, m, Lc);
  __syncthreads();
  // q, k of this thread's row and V of this lane's U operands into
  // registers: the chunk's operands then take their place
  float qx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, kx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ln.r() < T) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float4 a = *reinterpret_cast<const float4*>(&sm.a.cv.qkv[ln.r()][0][ln.c0() + 16 * x]);
      const float4 b = *reinterpret_cast<const float4*>(&sm.a.cv.qkv[ln.r()][1][ln.c0() + 16 * x]);
      qx[4 * x] = a.x; qx[4 * x + 1] = a.y; qx[4 * x + 2] = a.z; qx[4 * x + 3] = a.w;
      kx[4 * x] = b.x; kx[4 * x + 1] = b.y; kx[4 * x + 2] = b.z; kx[4 * x + 3] = b.w;
    }
  }
  // V rows 4 g4 .. 4 g4 + 3 of this lane's two columns, as pairs
  s16x4 vh[2], vl[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    f32x4 v4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 4 * ln.g4() + j;
      v4[j] = rr < T ? sm.a.cv.qkv[rr][2][32 * ln.wave() + 16 * ct + ln.l16()] : 0.f;
    }
    split4(v4, vh[ct], vl[ct]);
  }
  __syncthreads();
  gated_operands(sm.x, sm.a.op.y, sm.a.op.qk, ln, m, qx, kx);
  __syncthreads();
  a_solve_p(sm.x, sm.a.op.y, sm.a.op.qk, sm.sp, ln);
  __syncthreads();
  w_products(sm.a.op.y, sm.sp, ln);
  __syncthreads();

  if (do_store && Lc == 0) store_state(S, p.pool, dst, p.H, h, ln);
  const bool commit = do_store && Lc > 0;
  // U = T V with V (fp32) as a pair
  auto u_init = [&](int ct) -> f32x4 {
    const s16x4 th4 = *reinterpret_cast<const s16x4*>(&sm.sp.T_hi[ln.l16()][4 * ln.g4()]);
    const s16x4 tl4 = *reinterpret_cast<const s16x4*>(&sm.sp.T_lo[ln.l16()][4 * ln.g4()]);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return mfma16(tl4, vh[ct], mfma16(th4, vl[ct], mfma16(th4, vh[ct], z)));
  };
  // outputs staged for the gated norm (G and A are spent)
  auto out = [&](int ct, const f32x4& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.x.o[4 * ln.g4() + i][32 * ln.wave() + 16 * ct + ln.l16()] = o[i];
  };
  state_part(S, sm.a.op.y, sm.a.op.qk, sm.sp, ln, with_o, commit, Lc, p.scale, u_init, out);
  if (commit) store_state(S, p.pool, dst, p.H, h, ln);
  if (with_o) {
    __syncthreads();
    // a token's D outputs by D / 4 consecutive lanes (the gated norm sums
    // across exactly those; every round covers whole tokens)
    Tout* ob = static_cast<Tout*>(p.o);
#pragma unroll
    for (int k = 0; k < OU; ++k) {
      const int e = 4 * (k * NT + tid);
      if (e < T * D) {
        const int j = e / D, c = e % D;
        const float4 o4 = *reinterpret_cast<const float4*>(&sm.x.o[j][c]);
        float ov[4] = {o4.x, o4.y, o4.z, o4.w};
        if (p.ogate) {
          // gated RMS norm over the token's D outputs, held 4 per lane by
          // an aligned group of D / 4 lanes (every lane of it active)
          float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
          ss = group_sum<D / 4>(ss);
          const float inv = 1.f / sqrtf(ss * (1.f / D) + p.onorm_eps);
          float z[4], w[4];
          unpack4(graw[k], z);
          unpack4(wraw[k], w);
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = ov[i] * inv * w[i] * sigmoid_fast(z[i]);
        }
        io<Tout>::st4(ob + (static_cast<int64_t>(s) * T + j) * p.o_stride + hd + c, ov);
      }
    }
  }
}

template <typename Tout>
static int launch_t(const StepParams& p, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  hipLaunchKernelGGL((verify_kernel<Tout>), grid, dim3(NT), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "verify kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <typename Tout>
static int launch_conv_t(const DecodeConvParams& p, hipStream_t stream) {
  dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.n_seq) * p.H));
  // the window bucket: 8 tokens keep the workgroup's LDS small
  auto go = [&](auto w_t) {
    constexpr int W = decltype(w_t)::value;
    if (p.T_spec <= 8)
      hipLaunchKernelGGL((verify_conv_kernel<Tout, W, 8>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((verify_conv_kernel<Tout, W, R>), grid, dim3(NT), 0, stream, p);
  };
  switch (p.W) {
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: return fail(KDA_ERR_UNSUPPORTED, "verify_conv: W = %d (2..4)", p.W);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "verify_conv kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace vf

int launch_verify_mfma(const StepParams& p, int out_dtype, hipStream_t stream) {
  if (out_dtype == KDA_F32) return vf::launch_t<float>(p, stream);
  return vf::launch_t<bf16_t>(p, stream);
}

int launch_verify_conv_mfma(const DecodeConvParams& p, int out_dtype, hipStream_t stream) {
  if (out_dtype == KDA_F32) return vf::launch_conv_t<float>(p, stream);
  return vf::launch_conv_t<bf16_t>(p, stream);
}

}  // namespace kda
