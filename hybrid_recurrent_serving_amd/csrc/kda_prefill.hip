// Chunked prefill of the KDA recurrence on bf16 matrix cores (gfx950).
//
// Per (sequence, head) the tokens are processed in chunks whose boundaries
// sit at absolute positions that are multiples of the chunk length CH (16 or
// 32; a request for 64 runs as two 32-token chunks, which gives the same
// result).  Each chunk occupies a 32-row tile; rows outside the sequence (a
// sequence that starts or ends mid-chunk, or the 16 unused rows when
// CH = 16) are padding with k = q = v = 0, beta = 0 and g = 0, which leaves
// the state and every other row untouched.
//
// Chunked (WY / UT-transform) form of the recurrence
//     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
// ("Kimi K3 + vLLM: Inside the Day-0 Production Integration", section "Kimi
// Delta Attention: When Prefix Caching Meets Recurrent State", names the
// fixed-size matrix state; the update is the gated delta rule).  With
// G_r = sum_{j<=r} g_j inside the chunk (per key channel) and a reference
// row m = 15:
//     left_k[r] = k_r exp(G_r - G_m),  left_q[r] = q_r exp(G_r - G_m),
//     right_k[s] = k_s exp(G_m - G_s)
//     A[r,s] = beta_r <left_k[r], right_k[s]>  (s < r),  T = (I + A)^{-1} diag(beta)
//     S'  = Diag(exp G_m) S                    (state at the reference row)
//     u   = T V - (T left_k) S'
//     O   = scale (left_q S' + P u),  P[r,s] = <left_q[r], right_k[s]>  (s <= r)
//     S_next = Diag(exp(G_last - G_m)) (S' + right_k^T u)
// Every exponential factor is at most exp(decay over 16 tokens); the two
// state factors are <= 1.
//
// Work split: a workgroup of 4 waves owns one (sequence, head).  Wave w owns
// columns [32w, 32w + 32) of the d_v axis: its slice of the fp32 state lives
// in matrix-core accumulator registers for the whole sequence, and the
// state-dependent chain (u, O, state update) never leaves the wave.  The
// chunk-local operands (gates, A, T, P, W) are built cooperatively in LDS.
//
// Matrix-core precision (bf16 operands, fp32 accumulation); an operand
// marked "pair" is carried as hi + lo bf16 (hi*hi + hi*lo + lo*hi):
//     A = left_k right_k^T          single bf16
//     P = left_q right_k^T          pair x pair
//     W = T left_k, U = T V         single
//     u: W S'                       single
//     O: left_q S'  pair x pair;    P u   pair x pair
//     state: right_k^T u            pair x pair
// With fp32 inputs every product is pair x pair.
//
// Contractions whose operand comes from accumulator registers (S' over the
// key channels, u over chunk rows) use a fixed permutation of the contracted
// index inside each block of 16 (groups of four 1 and 2 swapped); the LDS
// copies of the other operand are stored in the same permuted order.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace pf {

constexpr int TILE = 32;   // rows per chunk tile
constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr int MID = 15;    // reference row of the gates

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// storage position of contracted index c (self-inverse): swap 4-groups 1, 2
__device__ __forceinline__ int perm16(int c) {
  const int g = (c >> 2) & 3;
  const int ng = g == 1 ? 2 : (g == 2 ? 1 : g);
  return (c & ~15) | (ng << 2) | (c & 3);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

__device__ __forceinline__ bf16x8 frag_lds(const bf16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void st_lds8(bf16_t* p, const float (&x)[8]) {
  uint4 u;
  u.x = pack2(x[0], x[1]);
  u.y = pack2(x[2], x[3]);
  u.z = pack2(x[4], x[5]);
  u.w = pack2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// hi / lo pair of 8 values
__device__ __forceinline__ void split8(const float (&x)[8], float (&hi)[8], float (&lo)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = bf16_round(x[i]);
    lo[i] = x[i] - hi[i];
  }
}

// 8 accumulator values [e0, e0 + 8) of a 32x32 tile as a bf16 B fragment
template <int E0>
__device__ __forceinline__ bf16x8 frag_acc(const f32x16& a) {
  uint4 u;
  u.x = pack2(a[E0 + 0], a[E0 + 1]);
  u.y = pack2(a[E0 + 2], a[E0 + 3]);
  u.z = pack2(a[E0 + 4], a[E0 + 5]);
  u.w = pack2(a[E0 + 6], a[E0 + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

template <int E0>
__device__ __forceinline__ void frag_acc_split(const f32x16& a, bf16x8& hi, bf16x8& lo) {
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = bf16_round(a[E0 + i]);
    l[i] = a[E0 + i] - h[i];
  }
  uint4 uh, ul;
  uh.x = pack2(h[0], h[1]); uh.y = pack2(h[2], h[3]); uh.z = pack2(h[4], h[5]); uh.w = pack2(h[6], h[7]);
  ul.x = pack2(l[0], l[1]); ul.y = pack2(l[2], l[3]); ul.z = pack2(l[4], l[5]); ul.w = pack2(l[6], l[7]);
  hi = __builtin_bit_cast(bf16x8, uh);
  lo = __builtin_bit_cast(bf16x8, ul);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// row (within a 32-row tile) of accumulator element e held by lane l
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

template <int D, typename TIN>
struct Smem {
  static constexpr bool F32IN = sizeof(TIN) == 4;
  TIN raw_q[TILE][D];
  TIN raw_k[TILE][D];
  TIN raw_v[TILE][D];
  TIN raw_g[TILE][D];
  float beta[TILE];
  float G[TILE][D];
  float scan[8][D];
  float eg_m[D];              // exp(G_m): decay from chunk start to the reference row
  float eg_e[D];              // exp(G_last - G_m)
  bf16_t lq_hi[TILE][D];      // [r][perm(c)]
  bf16_t lq_lo[TILE][D];
  bf16_t lk[TILE][D];         // [r][perm(c)]
  bf16_t lk_lo[F32IN ? TILE : 1][D];
  bf16_t rk_hi[TILE][D];      // [s][perm(c)]
  bf16_t rk_lo[TILE][D];
  bf16_t lkT[D][TILE];        // [c][s]
  bf16_t lkT_lo[F32IN ? D : 1][TILE];
  bf16_t rkT_hi[D][TILE];     // [c][perm(s)]
  bf16_t rkT_lo[D][TILE];
  bf16_t vT_hi[D][TILE];      // [n][s]
  bf16_t vT_lo[F32IN ? D : 1][TILE];
  float A[TILE][TILE];
  float Tf[TILE][TILE];       // (I + A)^{-1}, fp32
  float X[16][16];
  bf16_t Tm[TILE][TILE];      // [r][s]
  bf16_t Tm_lo[F32IN ? TILE : 1][TILE];
  bf16_t P_hi[TILE][TILE];    // [r][perm(s)]
  bf16_t P_lo[TILE][TILE];
  bf16_t Wn[TILE][D];         // -(T left_k) [r][perm(c)]
  bf16_t Wn_lo[F32IN ? TILE : 1][D];
};

// ---------------------------------------------------------------------------
template <int D, typename TIN, typename TOUT>
__global__ void __launch_bounds__(NT, 1) prefill_kernel(const PrefillParams p, const int d, const int CH) {
  using SM = Smem<D, TIN>;
  __shared__ SM sm;
  constexpr int NWC = D / 32;           // waves that own state columns
  constexpr int VEC = 16 / sizeof(TIN); // elements per 16-byte vector
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int s = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x % p.H);
  const int H = p.H;

  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  const int64_t len = eos - bos;
  int64_t start = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (start < 0) start = 0;
  const int64_t end = start + len;
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots;
  const bool chain = wave < NWC;
  const int ncol = 32 * wave + (lane & 31);   // d_v column of this lane (chain waves)

  // ---- state: 128 x 32 slice per chain wave, fp32 accumulators
  f32x16 S[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) S[t][e] = 0.f;
  if (chain && has_src && ncol < d) {
    const float* sp = p.pool + (static_cast<int64_t>(src) * H + h) * d * d;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * t + acc_row(e, lane);
        const int cc = c < d ? c : 0;
        const float v = sp[static_cast<int64_t>(cc) * d + ncol];
        S[t][e] = c < d ? v : 0.f;
      }
  }

  const TIN* qg = static_cast<const TIN*>(p.q);
  const TIN* kg = static_cast<const TIN*>(p.k);
  const TIN* vg = static_cast<const TIN*>(p.v);
  const TIN* gg = static_cast<const TIN*>(p.g);
  const TIN* bg = static_cast<const TIN*>(p.beta);
  TOUT* og = static_cast<TOUT*>(p.o);

  const int64_t first = len > 0 ? (start / CH) * CH : end;
  for (int64_t base = first; base < end; base += CH) {
    // ------------------------------------------------ phase L: raw tiles
    {
      constexpr int NV = D / VEC;  // vectors per row
      for (int it = tid; it < TILE * NV; it += NT) {
        const int r = it / NV;
        const int cv = (it % NV) * VEC;
        const int64_t pos = base + r;
        const bool valid = r < CH && pos >= start && pos < end && cv < d;
        uint4 zq = make_uint4(0, 0, 0, 0), zk = zq, zv = zq, zg = zq;
        if (valid) {
          const int64_t tok = bos + (pos - start);
          const int64_t off = static_cast<int64_t>(h) * d + cv;
          zq = *reinterpret_cast<const uint4*>(qg + tok * p.q_stride + off);
          zk = *reinterpret_cast<const uint4*>(kg + tok * p.k_stride + off);
          zv = *reinterpret_cast<const uint4*>(vg + tok * p.v_stride + off);
          zg = *reinterpret_cast<const uint4*>(gg + tok * p.g_stride + off);
        }
        *reinterpret_cast<uint4*>(&sm.raw_q[r][cv]) = zq;
        *reinterpret_cast<uint4*>(&sm.raw_k[r][cv]) = zk;
        *reinterpret_cast<uint4*>(&sm.raw_v[r][cv]) = zv;
        *reinterpret_cast<uint4*>(&sm.raw_g[r][cv]) = zg;
      }
      if (tid < TILE) {
        const int64_t pos = base + tid;
        float b = 0.f;
        if (tid < CH && pos >= start && pos < end) b = io<TIN>::ld(bg + (bos + (pos - start)) * p.beta_stride + h);
        sm.beta[tid] = b;
      }
    }
    __syncthreads();
    // ------------------------------------------------ phase G: cumulative gates
    {
      constexpr int NPART = NT / D;          // threads per channel
      constexpr int RP = TILE / NPART;       // rows per thread
      const int c = tid % D;
      const int part = tid / D;
      float acc = 0.f;
      float gl[RP];
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        acc += io<TIN>::ld(&sm.raw_g[part * RP + i][c]);
        gl[i] = acc;
      }
      sm.scan[part][c] = acc;
      __syncthreads();
      float off = 0.f;
      for (int q = 0; q < part; ++q) off += sm.scan[q][c];
#pragma unroll
      for (int i = 0; i < RP; ++i) sm.G[part * RP + i][c] = gl[i] + off;
      __syncthreads();
      if (tid < D) {
        const float gm = sm.G[MID][tid];
        sm.eg_m[tid] = expf(gm);
        sm.eg_e[tid] = expf(sm.G[TILE - 1][tid] - gm);
      }
    }
    // ------------------------------------------------ phase O: gated operands
    {
      // row-major operands [r][perm(c)]: item = (row, 8 storage positions)
      constexpr int NP = D / 8;
      for (int it = tid; it < TILE * NP; it += NT) {
        const int r = it / NP;
        const int p0 = (it % NP) * 8;
        float lq[8], lk[8], rk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = perm16(p0 + i);
          const float gr = sm.G[r][c];
          const float gm = sm.G[MID][c];
          const float a = expf(gr - gm);
          const float b = expf(gm - gr);
          const float kk = io<TIN>::ld(&sm.raw_k[r][c]);
          lq[i] = io<TIN>::ld(&sm.raw_q[r][c]) * a;
          lk[i] = kk * a;
          rk[i] = kk * b;
        }
        float hi[8], lo[8];
        split8(lq, hi, lo);
        st_lds8(&sm.lq_hi[r][p0], hi);
        st_lds8(&sm.lq_lo[r][p0], lo);
        if constexpr (SM::F32IN) {
          split8(lk, hi, lo);
          st_lds8(&sm.lk[r][p0], hi);
          st_lds8(&sm.lk_lo[r][p0], lo);
        } else {
          st_lds8(&sm.lk[r][p0], lk);
        }
        split8(rk, hi, lo);
        st_lds8(&sm.rk_hi[r][p0], hi);
        st_lds8(&sm.rk_lo[r][p0], lo);
      }
      // transposed operands: item = (channel, 8 rows)
      for (int it = tid; it < D * (TILE / 8); it += NT) {
        const int c = it / (TILE / 8);
        const int s0 = (it % (TILE / 8)) * 8;
        const float gm = sm.G[MID][c];
        float lkt[8], rkt[8], vt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int sn = s0 + i;           // natural row (lkT, vT)
          const int sp_ = perm16(s0 + i);  // physical row stored at position s0 + i (rkT)
          const float kn = io<TIN>::ld(&sm.raw_k[sn][c]);
          lkt[i] = kn * expf(sm.G[sn][c] - gm);
          const float kp = io<TIN>::ld(&sm.raw_k[sp_][c]);
          rkt[i] = kp * expf(gm - sm.G[sp_][c]);
          vt[i] = io<TIN>::ld(&sm.raw_v[sn][c]);
        }
        float hi[8], lo[8];
        if constexpr (SM::F32IN) {
          split8(lkt, hi, lo);
          st_lds8(&sm.lkT[c][s0], hi);
          st_lds8(&sm.lkT_lo[c][s0], lo);
        } else {
          st_lds8(&sm.lkT[c][s0], lkt);
        }
        split8(rkt, hi, lo);
        st_lds8(&sm.rkT_hi[c][s0], hi);
        st_lds8(&sm.rkT_lo[c][s0], lo);
        if constexpr (SM::F32IN) {
          split8(vt, hi, lo);
          st_lds8(&sm.vT_hi[c][s0], hi);
          st_lds8(&sm.vT_lo[c][s0], lo);
        } else {
          st_lds8(&sm.vT_hi[c][s0], vt);
        }
      }
    }
    __syncthreads();
    // ------------------------------------------------ phase AP: A and P
    {
      const int lr = lane & 15;        // row / column inside a 16x16 tile
      const int kq = 8 * (lane >> 4);  // k offset of this lane inside a 32-wide K step
      if (wave == 0) {
        // A tiles (0,0), (1,0), (1,1): strictly lower part, scaled by beta_row
        const int TI[3] = {0, 1, 1}, TJ[3] = {0, 0, 1};
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = frag_lds(&sm.lk[16 * TI[tt] + lr][32 * ks + kq]);
            const bf16x8 b = frag_lds(&sm.rk_hi[16 * TJ[tt] + lr][32 * ks + kq]);
            acc = mfma16(a, b, acc);
            if constexpr (SM::F32IN) {
              acc = mfma16(a, frag_lds(&sm.rk_lo[16 * TJ[tt] + lr][32 * ks + kq]), acc);
              acc = mfma16(frag_lds(&sm.lk_lo[16 * TI[tt] + lr][32 * ks + kq]), b, acc);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * TI[tt] + 4 * (lane >> 4) + i;
            const int c = 16 * TJ[tt] + lr;
            sm.A[r][c] = r > c ? acc[i] * sm.beta[r] : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.A[4 * (lane >> 4) + i][16 + lr] = 0.f;  // tile (0,1)
      } else {
        // P tile per wave: wave 1 -> (0,0), 2 -> (1,0), 3 -> (1,1); lower incl. diagonal
        const int I = wave == 1 ? 0 : 1;
        const int J = wave == 3 ? 1 : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 ah = frag_lds(&sm.lq_hi[16 * I + lr][32 * ks + kq]);
          const bf16x8 al = frag_lds(&sm.lq_lo[16 * I + lr][32 * ks + kq]);
          const bf16x8 bh = frag_lds(&sm.rk_hi[16 * J + lr][32 * ks + kq]);
          const bf16x8 bl = frag_lds(&sm.rk_lo[16 * J + lr][32 * ks + kq]);
          acc = mfma16(ah, bh, acc);
          acc = mfma16(ah, bl, acc);
          acc = mfma16(al, bh, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * (lane >> 4) + i;
          const int c = 16 * J + lr;
          const float v = c <= r ? acc[i] : 0.f;
          const float hi = bf16_round(v);
          sm.P_hi[r][perm16(c)] = f32_to_bf16(hi);
          sm.P_lo[r][perm16(c)] = f32_to_bf16(v - hi);
          if (wave == 1) {  // tile (0,1) is zero
            sm.P_hi[r][perm16(16 + lr)] = 0;
            sm.P_lo[r][perm16(16 + lr)] = 0;
          }
        }
      }
    }
    __syncthreads();
    // ------------------------------------------------ phase T: (I + A)^{-1} diag(beta)
    // Blocked forward substitution on 16 x 16 blocks (A is strictly lower):
    // D_b = (I + A_bb)^{-1} for the two diagonal blocks, then the lower block
    // (I + A)^{-1}_{10} = -D_1 A_10 D_0.
    if (wave == 0 && lane < TILE) {
      const int b = lane >> 4;
      const int jj = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == jj ? 1.f : 0.f;
#pragma unroll
        for (int s4 = 0; s4 < r; s4 += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(&sm.A[16 * b + r][16 * b + s4]);
          acc -= a4.x * x[s4];
          if (s4 + 1 < r) acc -= a4.y * x[s4 + 1];
          if (s4 + 2 < r) acc -= a4.z * x[s4 + 2];
          if (s4 + 3 < r) acc -= a4.w * x[s4 + 3];
        }
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.Tf[16 * b + r][16 * b + jj] = x[r];
        sm.Tf[16 * b + r][16 * (1 - b) + jj] = 0.f;  // upper block zero; lower one set below
      }
    }
    __syncthreads();
    {
      // X = A_10 D_0 (16 x 16): one entry per thread
      const int i = tid >> 4, j = tid & 15;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += sm.A[16 + i][k] * sm.Tf[k][j];
      sm.X[i][j] = acc;
    }
    __syncthreads();
    {
      const int i = tid >> 4, j = tid & 15;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += sm.Tf[16 + i][16 + k] * sm.X[k][j];
      sm.Tf[16 + i][j] = -acc;
    }
    __syncthreads();
    for (int it = tid; it < TILE * TILE; it += NT) {
      const int r = it / TILE, j = it % TILE;
      const float t = j <= r ? sm.Tf[r][j] * sm.beta[j] : 0.f;
      const float th = bf16_round(t);
      sm.Tm[r][j] = f32_to_bf16(th);
      if constexpr (SM::F32IN) sm.Tm_lo[r][j] = f32_to_bf16(t - th);
    }
    __syncthreads();
    // ------------------------------------------------ phase W: W = T left_k (shared), U = T V (own)
    f32x16 uacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) uacc[e] = 0.f;
    {
      const int lr = lane & 31;
      const int kq = 8 * (lane >> 5);
      if (chain) {
        f32x16 wacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) wacc[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < TILE / 16; ++ks) {
          const bf16x8 a = frag_lds(&sm.Tm[lr][16 * ks + kq]);
          const bf16x8 bk = frag_lds(&sm.lkT[32 * wave + lr][16 * ks + kq]);
          const bf16x8 bv = frag_lds(&sm.vT_hi[32 * wave + lr][16 * ks + kq]);
          wacc = mfma32(a, bk, wacc);
          uacc = mfma32(a, bv, uacc);
          if constexpr (SM::F32IN) {
            const bf16x8 al = frag_lds(&sm.Tm_lo[lr][16 * ks + kq]);
            wacc = mfma32(a, frag_lds(&sm.lkT_lo[32 * wave + lr][16 * ks + kq]), wacc);
            wacc = mfma32(al, bk, wacc);
            uacc = mfma32(a, frag_lds(&sm.vT_lo[32 * wave + lr][16 * ks + kq]), uacc);
            uacc = mfma32(al, bv, uacc);
          }
        }
        const int cp = perm16(32 * wave + lr);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float w = -wacc[e];
          const float wh = bf16_round(w);
          sm.Wn[acc_row(e, lane)][cp] = f32_to_bf16(wh);
          if constexpr (SM::F32IN) sm.Wn_lo[acc_row(e, lane)][cp] = f32_to_bf16(w - wh);
        }
      }
    }
    __syncthreads();
    // ------------------------------------------------ chain (per wave, own 32 columns)
    if (chain) {
      const int lr = lane & 31;
      const int kq = 8 * (lane >> 5);
      // S' = Diag(exp G_m) S
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[t][e] *= sm.eg_m[32 * t + acc_row(e, lane)];
      // u = U - W S' ; O = left_q S'
      f32x16 oacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[e] = 0.f;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        bf16x8 b0, b0l, b1, b1l;
        frag_acc_split<0>(S[t], b0, b0l);
        frag_acc_split<8>(S[t], b1, b1l);
        const bf16x8 w0 = frag_lds(&sm.Wn[lr][32 * t + kq]);
        const bf16x8 w1 = frag_lds(&sm.Wn[lr][32 * t + 16 + kq]);
        uacc = mfma32(w0, b0, uacc);
        uacc = mfma32(w1, b1, uacc);
        if constexpr (SM::F32IN) {
          uacc = mfma32(w0, b0l, uacc);
          uacc = mfma32(w1, b1l, uacc);
          uacc = mfma32(frag_lds(&sm.Wn_lo[lr][32 * t + kq]), b0, uacc);
          uacc = mfma32(frag_lds(&sm.Wn_lo[lr][32 * t + 16 + kq]), b1, uacc);
        }
        const bf16x8 q0 = frag_lds(&sm.lq_hi[lr][32 * t + kq]);
        const bf16x8 q1 = frag_lds(&sm.lq_hi[lr][32 * t + 16 + kq]);
        oacc = mfma32(q0, b0, oacc);
        oacc = mfma32(q0, b0l, oacc);
        oacc = mfma32(frag_lds(&sm.lq_lo[lr][32 * t + kq]), b0, oacc);
        oacc = mfma32(q1, b1, oacc);
        oacc = mfma32(q1, b1l, oacc);
        oacc = mfma32(frag_lds(&sm.lq_lo[lr][32 * t + 16 + kq]), b1, oacc);
      }
      bf16x8 uh0, ul0, uh1, ul1;
      frag_acc_split<0>(uacc, uh0, ul0);
      frag_acc_split<8>(uacc, uh1, ul1);
      // O += P u
      {
        const bf16x8 ph0 = frag_lds(&sm.P_hi[lr][kq]), pl0 = frag_lds(&sm.P_lo[lr][kq]);
        const bf16x8 ph1 = frag_lds(&sm.P_hi[lr][16 + kq]), pl1 = frag_lds(&sm.P_lo[lr][16 + kq]);
        oacc = mfma32(ph0, uh0, oacc);
        oacc = mfma32(ph0, ul0, oacc);
        oacc = mfma32(pl0, uh0, oacc);
        oacc = mfma32(ph1, uh1, oacc);
        oacc = mfma32(ph1, ul1, oacc);
        oacc = mfma32(pl1, uh1, oacc);
      }
      // S = Diag(exp(G_last - G_m)) (S' + right_k^T u)
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const int c = 32 * t + lr;
        const bf16x8 kh0 = frag_lds(&sm.rkT_hi[c][kq]), kl0 = frag_lds(&sm.rkT_lo[c][kq]);
        const bf16x8 kh1 = frag_lds(&sm.rkT_hi[c][16 + kq]), kl1 = frag_lds(&sm.rkT_lo[c][16 + kq]);
        S[t] = mfma32(kh0, uh0, S[t]);
        S[t] = mfma32(kh0, ul0, S[t]);
        S[t] = mfma32(kl0, uh0, S[t]);
        S[t] = mfma32(kh1, uh1, S[t]);
        S[t] = mfma32(kh1, ul1, S[t]);
        S[t] = mfma32(kl1, uh1, S[t]);
#pragma unroll
        for (int e = 0; e < 16; ++e) S[t][e] *= sm.eg_e[32 * t + acc_row(e, lane)];
      }
      // outputs of the valid rows
      if (ncol < d) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = acc_row(e, lane);
          const int64_t pos = base + r;
          if (r < CH && pos >= start && pos < end) {
            const int64_t tok = bos + (pos - start);
            io<TOUT>::st(og + tok * p.o_stride + static_cast<int64_t>(h) * d + ncol, oacc[e] * p.scale);
          }
        }
      }
    }
    // ------------------------------------------------ interval checkpoint
    if (p.ckpt_interval > 0 && p.ckpt_cu) {
      const int64_t after = base + CH;
      if (after < end && after % p.ckpt_interval == 0) {
        const int64_t j = after / p.ckpt_interval - start / p.ckpt_interval - 1;
        const int64_t idx = static_cast<int64_t>(p.ckpt_cu[s]) + j;
        if (j >= 0 && idx < p.ckpt_cu[s + 1] && idx < p.n_ckpt) {
          const int slot = p.ckpt_slot[idx];
          if (chain && slot >= 0 && slot < p.n_slots && ncol < d) {
            float* cp = p.pool + (static_cast<int64_t>(slot) * H + h) * d * d;
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int c = 32 * t + acc_row(e, lane);
                if (c < d) cp[static_cast<int64_t>(c) * d + ncol] = S[t][e];
              }
          }
          if (tid == 0 && h == 0 && p.ckpt_pos_out) p.ckpt_pos_out[idx] = static_cast<int32_t>(after);
        }
      }
    }
    __syncthreads();
  }
  // ---- final state
  if (chain && has_dst && ncol < d) {
    float* dp = p.pool + (static_cast<int64_t>(dst) * H + h) * d * d;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * t + acc_row(e, lane);
        if (c < d) dp[static_cast<int64_t>(c) * d + ncol] = S[t][e];
      }
  }
}

template <int D, typename TIN, typename TOUT>
static int launch_t(const PrefillParams& p, int d, int CH, hipStream_t stream) {
  const int64_t nblk = static_cast<int64_t>(p.n_seq) * p.H;
  if (nblk > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "n_seq * H too large");
  hipLaunchKernelGGL((prefill_kernel<D, TIN, TOUT>), dim3(static_cast<uint32_t>(nblk)), dim3(NT), 0, stream, p, d, CH);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <typename TIN, typename TOUT>
static int launch_d(const PrefillParams& p, int d, int CH, hipStream_t stream) {
  if (d <= 32) return launch_t<32, TIN, TOUT>(p, d, CH, stream);
  if (d == 64) return launch_t<64, TIN, TOUT>(p, d, CH, stream);
  if constexpr (sizeof(TIN) == 2) {
    if (d == 128) return launch_t<128, TIN, TOUT>(p, d, CH, stream);
  }
  return fail(KDA_ERR_UNSUPPORTED, "prefill: d = %d with %s inputs not built", d,
              sizeof(TIN) == 2 ? "bf16" : "fp32");
}

}  // namespace pf

int64_t prefill_workspace_bytes(const PrefillParams&, int) { return 0; }

int launch_prefill(const PrefillParams& p, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  // chunk 64 runs as two chunks of 32 (identical result up to rounding)
  const int CH = p.chunk == 16 ? 16 : 32;
  if (in_dtype == KDA_BF16) {
    if (out_dtype == KDA_BF16) return pf::launch_d<bf16_t, bf16_t>(p, D, CH, stream);
    return pf::launch_d<bf16_t, float>(p, D, CH, stream);
  }
  if (out_dtype == KDA_BF16) return pf::launch_d<float, bf16_t>(p, D, CH, stream);
  return pf::launch_d<float, float>(p, D, CH, stream);
}

}  // namespace kda
