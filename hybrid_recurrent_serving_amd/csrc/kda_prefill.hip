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
// Work split: a workgroup of 4 waves owns one (sequence, head); two
// workgroups share a CU (LDS <= 80 KB, <= 256 VGPRs), so one workgroup's
// matrix-core chain overlaps the other's VALU / LDS operand preparation.
// Wave w owns columns [32w, 32w + 32) of the d_v axis: its slice of the fp32
// state lives in matrix-core accumulator registers for the whole sequence,
// and the state-dependent chain (u, O, state update) never leaves the wave.
// The chunk-local operands (gates, A, T, P, W) are built cooperatively in
// LDS.  The next chunk's raw tiles are loaded into registers while the
// current chunk is processed.
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
// Layout tricks:
//  * Contractions whose operand comes from accumulator registers (S' over
//    the key channels, u over chunk rows) use a fixed permutation of the
//    contracted index inside each block of 16 (groups of four 1 and 2
//    swapped); the LDS operands on the other side are stored in that order.
//  * Operands that must be read K-contiguous from a row-major tile (right_k^T,
//    left_k and V over chunk rows) use the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16): four lanes of a 16-lane group read one row each,
//    lane i of the group receives column i of the four rows.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace pf {

constexpr int TILE = 32;   // rows per chunk tile
constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr int MID = 15;    // reference row of the gates

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// storage position of contracted index c (self-inverse): swap 4-groups 1, 2
__host__ __device__ constexpr int perm16(int c) {
  return (c & ~15) | ((((c >> 2) & 3) == 1 ? 2 : (((c >> 2) & 3) == 2 ? 1 : ((c >> 2) & 3))) << 2) | (c & 3);
}
__device__ __forceinline__ int swap4(int i) { return i == 1 ? 2 : (i == 2 ? 1 : i); }

// fp32 -> bf16 bits (hardware round to nearest even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float hi_of(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ bf16x8 frag_lds(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ s16x4 tr4(const bf16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 a, s16x4 b) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// store 8 floats as bf16 (16 bytes)
__device__ __forceinline__ void st8(bf16_t* p, const float* x) {
  uint4 u;
  u.x = cvt2(x[0], x[1]);
  u.y = cvt2(x[2], x[3]);
  u.z = cvt2(x[4], x[5]);
  u.w = cvt2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// 8 accumulator values [E0, E0 + 8) as a bf16 hi / lo fragment pair
template <int E0>
__device__ __forceinline__ void frag_acc_pair(const f32x16& a, bf16x8& hi, bf16x8& lo) {
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = hi_of(a[E0 + i]);
    l[i] = a[E0 + i] - h[i];
  }
  uint4 uh, ul;
  uh.x = cvt2(h[0], h[1]); uh.y = cvt2(h[2], h[3]); uh.z = cvt2(h[4], h[5]); uh.w = cvt2(h[6], h[7]);
  ul.x = cvt2(l[0], l[1]); ul.y = cvt2(l[2], l[3]); ul.z = cvt2(l[4], l[5]); ul.w = cvt2(l[6], l[7]);
  hi = __builtin_bit_cast(bf16x8, uh);
  lo = __builtin_bit_cast(bf16x8, ul);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// row (within a 32-row tile) of 32x32 accumulator element e held by lane
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Transpose-read fragment (32x32x16 operand, 8 contracted values per lane)
// of a row-major bf16 tile M[k][x] (row pitch `pitch` elements): lane l gets
// M[k0 + 8(l/32) + e][x0 + l % 32] for e = 0..7.
__device__ __forceinline__ bf16x8 frag_tr(const bf16_t* M, int pitch, int k0, int x0, int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, i = lane & 3;
  const int kk = k0 + 8 * (g >> 1) + j;
  const int xx = x0 + 16 * (g & 1) + 4 * i;
  return join(tr4(M + kk * pitch + xx), tr4(M + (kk + 4) * pitch + xx));
}

// The state slice of a chain wave <-> a pool slot [c][n] (fp32).  Kept out of
// line: called once per sequence and per checkpoint, and inlining it makes the
// compiler hold 64 loop-invariant addresses across the chunk loop.
template <int D>
__device__ __attribute__((noinline)) void state_store(float* base, const f32x16* S, int lane, int ncol, int d) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * t + acc_row(e, lane);
      if (c < d) base[c * d + ncol] = S[t][e];
    }
}

template <int D>
__device__ __attribute__((noinline)) void state_load(const float* base, f32x16* S, int lane, int ncol, int d) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * t + acc_row(e, lane);
      const float v = base[(c < d ? c : 0) * d + ncol];
      S[t][e] = c < d ? v : 0.f;
    }
}

template <int D, typename TIN>
struct Smem {
  static constexpr bool F32IN = sizeof(TIN) == 4;
  bf16_t lq_hi[TILE][D];      // [r][perm(c)]   (reused for output staging)
  bf16_t lq_lo[TILE][D];
  bf16_t lk[TILE][D];         // [r][perm(c)]
  bf16_t lk_lo[F32IN ? TILE : 1][D];
  bf16_t rk_hi[TILE][D];      // [s][perm(c)]
  bf16_t rk_lo[TILE][D];
  bf16_t v_hi[TILE][D];       // [s][n]
  bf16_t v_lo[F32IN ? TILE : 1][D];
  float eg_m[D];              // exp(G_m)
  float eg_e[D];              // exp(G_last - G_m)
  float beta[TILE];
  union {
    struct {
      TIN g_raw[TILE][D];
      float G[TILE][D];
      float scan[8][D];
    } a;
    struct {
      float A[TILE][TILE];
      float Tf[TILE][TILE];
      float X[16][16];
      bf16_t Tm[TILE][TILE];  // [r][s]
      bf16_t Tm_lo[F32IN ? TILE : 1][TILE];
      bf16_t P_hi[TILE][TILE];  // [r][perm(s)]
      bf16_t P_lo[TILE][TILE];
      bf16_t Wn[TILE][D];     // -(T left_k) [r][perm(c)]
      bf16_t Wn_lo[F32IN ? TILE : 1][D];
    } b;
  } u;
};

// raw 16-channel slice of one token row (q, k, v, g) as 16-byte vectors
template <typename TIN>
struct RawRow {
  static constexpr int NV = 16 * sizeof(TIN) / 16;   // uint4 per tensor
  uint4 q[NV], k[NV], v[NV], g[NV];
};

template <typename TIN>
__device__ __forceinline__ void to_f32(const uint4 (&w)[RawRow<TIN>::NV], float (&x)[16]) {
  if constexpr (sizeof(TIN) == 2) {
    const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[4 * i] = __uint_as_float(w[i].x);
      x[4 * i + 1] = __uint_as_float(w[i].y);
      x[4 * i + 2] = __uint_as_float(w[i].z);
      x[4 * i + 3] = __uint_as_float(w[i].w);
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, typename TIN, typename TOUT>
__global__ void __launch_bounds__(NT, 2) prefill_kernel(const PrefillParams p, const int d, const int CH) {
  using SM = Smem<D, TIN>;
  __shared__ SM sm;
  constexpr bool HP = SM::F32IN;        // all products as pairs
  constexpr int NWC = D / 32;           // waves that own state columns
  constexpr int NB = D / 16;            // 16-channel blocks per row
  constexpr int NITEM = TILE * NB;      // (row, block) items per chunk
  constexpr int NV = RawRow<TIN>::NV;
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

  // ---- state: D x 32 slice per chain wave, fp32 accumulators
  f32x16 S[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) S[t][e] = 0.f;
  if (chain && has_src && ncol < d) state_load<D>(p.pool + (static_cast<int64_t>(src) * H + h) * d * d, S, lane, ncol, d);

  const TIN* qg = static_cast<const TIN*>(p.q);
  const TIN* kg = static_cast<const TIN*>(p.k);
  const TIN* vg = static_cast<const TIN*>(p.v);
  const TIN* gg = static_cast<const TIN*>(p.g);
  const TIN* bg = static_cast<const TIN*>(p.beta);
  TOUT* og = static_cast<TOUT*>(p.o);

  // raw-tile item of this thread: row ir, channels [16 ib, 16 ib + 16)
  const bool has_item = tid < NITEM;
  const int ir = tid / NB;
  const int ib = tid % NB;

  auto load_raw = [&](int64_t base, RawRow<TIN>& rr) {
    const int64_t pos = base + ir;
    const bool valid = has_item && ir < CH && pos >= start && pos < end && 16 * ib < d;
#pragma unroll
    for (int w = 0; w < NV; ++w) rr.q[w] = rr.k[w] = rr.v[w] = rr.g[w] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const int64_t tok = bos + (pos - start);
      const int64_t off = static_cast<int64_t>(h) * d + 16 * ib;
      const uint4* qp = reinterpret_cast<const uint4*>(qg + tok * p.q_stride + off);
      const uint4* kp = reinterpret_cast<const uint4*>(kg + tok * p.k_stride + off);
      const uint4* vp = reinterpret_cast<const uint4*>(vg + tok * p.v_stride + off);
      const uint4* gp = reinterpret_cast<const uint4*>(gg + tok * p.g_stride + off);
      // only the vectors inside d (d = 16 with 16-channel blocks: all of them)
      const int nv = (16 * ib + 16 <= d) ? NV : ((d - 16 * ib) * static_cast<int>(sizeof(TIN))) / 16;
#pragma unroll
      for (int w = 0; w < NV; ++w)
        if (w < nv) {
          rr.q[w] = qp[w];
          rr.k[w] = kp[w];
          rr.v[w] = vp[w];
          rr.g[w] = gp[w];
        }
    }
  };

  const int64_t first = len > 0 ? (start / CH) * CH : end;
  RawRow<TIN> nxt;
  load_raw(first, nxt);
  for (int64_t base = first; base < end; base += CH) {
    // ------------------------------------------------ phase L: commit raw tile, prefetch next
    RawRow<TIN> cur = nxt;
    if (base + CH < end) load_raw(base + CH, nxt);
    if (has_item) {
      TIN* gr = &sm.u.a.g_raw[ir][16 * ib];
#pragma unroll
      for (int w = 0; w < NV; ++w) reinterpret_cast<uint4*>(gr)[w] = cur.g[w];
      if constexpr (HP) {
        float vx[16], vh[16], vl[16];
        to_f32<TIN>(cur.v, vx);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          vh[i] = hi_of(vx[i]);
          vl[i] = vx[i] - vh[i];
        }
        st8(&sm.v_hi[ir][16 * ib], vh);
        st8(&sm.v_hi[ir][16 * ib + 8], vh + 8);
        st8(&sm.v_lo[ir][16 * ib], vl);
        st8(&sm.v_lo[ir][16 * ib + 8], vl + 8);
      } else {
#pragma unroll
        for (int w = 0; w < NV; ++w) reinterpret_cast<uint4*>(&sm.v_hi[ir][16 * ib])[w] = cur.v[w];
      }
    }
    if (tid < TILE) {
      const int64_t pos = base + tid;
      float b = 0.f;
      if (tid < CH && pos >= start && pos < end) b = io<TIN>::ld(bg + (bos + (pos - start)) * p.beta_stride + h);
      sm.beta[tid] = b;
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
        acc += io<TIN>::ld(&sm.u.a.g_raw[part * RP + i][c]);
        gl[i] = acc;
      }
      sm.u.a.scan[part][c] = acc;
      __syncthreads();
      float off = 0.f;
      for (int q = 0; q < part; ++q) off += sm.u.a.scan[q][c];
#pragma unroll
      for (int i = 0; i < RP; ++i) sm.u.a.G[part * RP + i][c] = gl[i] + off;
      __syncthreads();
      if (tid < D) {
        const float gm = sm.u.a.G[MID][tid];
        sm.eg_m[tid] = expf(gm);
        sm.eg_e[tid] = expf(sm.u.a.G[TILE - 1][tid] - gm);
      }
    }
    // ------------------------------------------------ phase O: gated operands (row-major)
    if (has_item) {
      float qx[16], kx[16];
      to_f32<TIN>(cur.q, qx);
      to_f32<TIN>(cur.k, kx);
      // two halves of 8 storage positions; position i of the block holds
      // channel perm16(i), so each half covers two groups of four channels
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float lq[8], lk[8], rk[8];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int c0 = perm16(8 * half + 4 * gi);   // first channel of this group of four
          const float4 a = *reinterpret_cast<const float4*>(&sm.u.a.G[ir][16 * ib + c0]);
          const float4 b = *reinterpret_cast<const float4*>(&sm.u.a.G[MID][16 * ib + c0]);
          const float x4[4] = {a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int i = 4 * gi + m;
            const float ea = fexp(x4[m]);
            lq[i] = qx[c0 + m] * ea;
            lk[i] = kx[c0 + m] * ea;
            rk[i] = kx[c0 + m] * fexp(-x4[m]);
          }
        }
        const int pos = 16 * ib + 8 * half;
        float hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = hi_of(lq[i]);
          lo[i] = lq[i] - hi[i];
        }
        st8(&sm.lq_hi[ir][pos], hi);
        st8(&sm.lq_lo[ir][pos], lo);
        if constexpr (HP) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            hi[i] = hi_of(lk[i]);
            lo[i] = lk[i] - hi[i];
          }
          st8(&sm.lk[ir][pos], hi);
          st8(&sm.lk_lo[ir][pos], lo);
        } else {
          st8(&sm.lk[ir][pos], lk);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = hi_of(rk[i]);
          lo[i] = rk[i] - hi[i];
        }
        st8(&sm.rk_hi[ir][pos], hi);
        st8(&sm.rk_lo[ir][pos], lo);
      }
    }
    __syncthreads();
    // ------------------------------------------------ phase AP: A and P (16x16 tiles)
    {
      const int lr = lane & 15;        // row / column inside a 16x16 tile
      const int kq = 8 * (lane >> 4);  // k offset of this lane inside a 32-wide K step
      if (wave == 0) {
        // A tiles (0,0), (1,0), (1,1): strictly lower part, scaled by beta_row
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
          const int I = tt == 0 ? 0 : 1, J = tt == 2 ? 1 : 0;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = frag_lds(&sm.lk[16 * I + lr][32 * ks + kq]);
            const bf16x8 b = frag_lds(&sm.rk_hi[16 * J + lr][32 * ks + kq]);
            acc = mfma16(a, b, acc);
            if constexpr (HP) {
              acc = mfma16(a, frag_lds(&sm.rk_lo[16 * J + lr][32 * ks + kq]), acc);
              acc = mfma16(frag_lds(&sm.lk_lo[16 * I + lr][32 * ks + kq]), b, acc);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * (lane >> 4) + i;
            const int c = 16 * J + lr;
            sm.u.b.A[r][c] = r > c ? acc[i] * sm.beta[r] : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.u.b.A[4 * (lane >> 4) + i][16 + lr] = 0.f;  // tile (0,1)
      } else {
        // P tile per wave: wave 1 -> (0,0), 2 -> (1,0), 3 -> (1,1); lower incl. diagonal
        const int I = wave == 1 ? 0 : 1;
        const int J = wave == 3 ? 1 : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 ah = frag_lds(&sm.lq_hi[16 * I + lr][32 * ks + kq]);
          const bf16x8 bh = frag_lds(&sm.rk_hi[16 * J + lr][32 * ks + kq]);
          acc = mfma16(ah, bh, acc);
          acc = mfma16(ah, frag_lds(&sm.rk_lo[16 * J + lr][32 * ks + kq]), acc);
          acc = mfma16(frag_lds(&sm.lq_lo[16 * I + lr][32 * ks + kq]), bh, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * (lane >> 4) + i;
          const int c = 16 * J + lr;
          const float v = c <= r ? acc[i] : 0.f;
          const float hv = hi_of(v);
          sm.u.b.P_hi[r][perm16(c)] = f32_to_bf16(hv);
          sm.u.b.P_lo[r][perm16(c)] = f32_to_bf16(v - hv);
          if (wave == 1) {  // tile (0,1) is zero
            sm.u.b.P_hi[r][perm16(16 + lr)] = 0;
            sm.u.b.P_lo[r][perm16(16 + lr)] = 0;
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
          const float4 a4 = *reinterpret_cast<const float4*>(&sm.u.b.A[16 * b + r][16 * b + s4]);
          acc -= a4.x * x[s4];
          if (s4 + 1 < r) acc -= a4.y * x[s4 + 1];
          if (s4 + 2 < r) acc -= a4.z * x[s4 + 2];
          if (s4 + 3 < r) acc -= a4.w * x[s4 + 3];
        }
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.u.b.Tf[16 * b + r][16 * b + jj] = x[r];
        sm.u.b.Tf[16 * b + r][16 * (1 - b) + jj] = 0.f;
      }
    }
    __syncthreads();
    {
      const int i = tid >> 4, j = tid & 15;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += sm.u.b.A[16 + i][k] * sm.u.b.Tf[k][j];
      sm.u.b.X[i][j] = acc;
    }
    __syncthreads();
    {
      const int i = tid >> 4, j = tid & 15;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += sm.u.b.Tf[16 + i][16 + k] * sm.u.b.X[k][j];
      sm.u.b.Tf[16 + i][j] = -acc;
    }
    __syncthreads();
    for (int it = tid; it < TILE * TILE; it += NT) {
      const int r = it / TILE, j = it % TILE;
      const float t = j <= r ? sm.u.b.Tf[r][j] * sm.beta[j] : 0.f;
      const float th = hi_of(t);
      sm.u.b.Tm[r][j] = f32_to_bf16(th);
      if constexpr (HP) sm.u.b.Tm_lo[r][j] = f32_to_bf16(t - th);
    }
    __syncthreads();
    // ------------------------------------------------ phase W: W = T left_k (shared), U = T V (own)
    f32x16 uacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) uacc[e] = 0.f;
    if (chain) {
      const int lr = lane & 31;
      const int kq = 8 * (lane >> 5);
      f32x16 wacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) wacc[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < TILE / 16; ++ks) {
        const bf16x8 a = frag_lds(&sm.u.b.Tm[lr][16 * ks + kq]);
        const bf16x8 bk = frag_tr(&sm.lk[0][0], D, 16 * ks, 32 * wave, lane);
        const bf16x8 bv = frag_tr(&sm.v_hi[0][0], D, 16 * ks, 32 * wave, lane);
        wacc = mfma32(a, bk, wacc);
        uacc = mfma32(a, bv, uacc);
        if constexpr (HP) {
          const bf16x8 al = frag_lds(&sm.u.b.Tm_lo[lr][16 * ks + kq]);
          wacc = mfma32(a, frag_tr(&sm.lk_lo[0][0], D, 16 * ks, 32 * wave, lane), wacc);
          wacc = mfma32(al, bk, wacc);
          uacc = mfma32(a, frag_tr(&sm.v_lo[0][0], D, 16 * ks, 32 * wave, lane), uacc);
          uacc = mfma32(al, bv, uacc);
        }
      }
      // W columns come out in storage-position order: store -W as is
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float w = -wacc[e];
        const float wh = hi_of(w);
        sm.u.b.Wn[acc_row(e, lane)][32 * wave + lr] = f32_to_bf16(wh);
        if constexpr (HP) sm.u.b.Wn_lo[acc_row(e, lane)][32 * wave + lr] = f32_to_bf16(w - wh);
      }
    }
    __syncthreads();
    // ------------------------------------------------ chain (per wave, own 32 columns)
    f32x16 oacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[e] = 0.f;
    if (chain) {
      const int lr = lane & 31;
      const int kq = 8 * (lane >> 5);
      // S' = Diag(exp G_m) S
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[t][e] *= sm.eg_m[32 * t + acc_row(e, lane)];
      // u = U - W S' ; O = left_q S'
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        bf16x8 b0, b0l, b1, b1l;
        frag_acc_pair<0>(S[t], b0, b0l);
        frag_acc_pair<8>(S[t], b1, b1l);
        const bf16x8 w0 = frag_lds(&sm.u.b.Wn[lr][32 * t + kq]);
        const bf16x8 w1 = frag_lds(&sm.u.b.Wn[lr][32 * t + 16 + kq]);
        const bf16x8 q0 = frag_lds(&sm.lq_hi[lr][32 * t + kq]);
        const bf16x8 q1 = frag_lds(&sm.lq_hi[lr][32 * t + 16 + kq]);
        const bf16x8 q0l = frag_lds(&sm.lq_lo[lr][32 * t + kq]);
        const bf16x8 q1l = frag_lds(&sm.lq_lo[lr][32 * t + 16 + kq]);
        uacc = mfma32(w0, b0, uacc);
        oacc = mfma32(q0, b0, oacc);
        uacc = mfma32(w1, b1, uacc);
        oacc = mfma32(q1, b1, oacc);
        oacc = mfma32(q0, b0l, oacc);
        oacc = mfma32(q1, b1l, oacc);
        oacc = mfma32(q0l, b0, oacc);
        oacc = mfma32(q1l, b1, oacc);
        if constexpr (HP) {
          uacc = mfma32(w0, b0l, uacc);
          uacc = mfma32(w1, b1l, uacc);
          uacc = mfma32(frag_lds(&sm.u.b.Wn_lo[lr][32 * t + kq]), b0, uacc);
          uacc = mfma32(frag_lds(&sm.u.b.Wn_lo[lr][32 * t + 16 + kq]), b1, uacc);
        }
      }
      bf16x8 uh0, ul0, uh1, ul1;
      frag_acc_pair<0>(uacc, uh0, ul0);
      frag_acc_pair<8>(uacc, uh1, ul1);
      // O += P u
      {
        const bf16x8 ph0 = frag_lds(&sm.u.b.P_hi[lr][kq]), pl0 = frag_lds(&sm.u.b.P_lo[lr][kq]);
        const bf16x8 ph1 = frag_lds(&sm.u.b.P_hi[lr][16 + kq]), pl1 = frag_lds(&sm.u.b.P_lo[lr][16 + kq]);
        oacc = mfma32(ph0, uh0, oacc);
        oacc = mfma32(ph1, uh1, oacc);
        oacc = mfma32(ph0, ul0, oacc);
        oacc = mfma32(ph1, ul1, oacc);
        oacc = mfma32(pl0, uh0, oacc);
        oacc = mfma32(pl1, uh1, oacc);
      }
      // S = Diag(exp(G_last - G_m)) (S' + right_k^T u); right_k^T fragments are
      // transpose reads of right_k [s][perm(c)] whose rows follow u's order and
      // whose columns come out in channel order.
      {
        const int g = lane >> 4, j = (lane >> 2) & 3, i = lane & 3;
        const int krow = 4 * (g >> 1) + j;  // rows krow (e 0..3) and krow + 8 (e 4..7)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int col = 32 * t + 16 * (g & 1) + 4 * swap4(i);
          bf16x8 kh[2], kl[2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int r0 = 16 * hf + krow;
            kh[hf] = join(tr4(&sm.rk_hi[r0][col]), tr4(&sm.rk_hi[r0 + 8][col]));
            kl[hf] = join(tr4(&sm.rk_lo[r0][col]), tr4(&sm.rk_lo[r0 + 8][col]));
          }
          S[t] = mfma32(kh[0], uh0, S[t]);
          S[t] = mfma32(kh[1], uh1, S[t]);
          S[t] = mfma32(kh[0], ul0, S[t]);
          S[t] = mfma32(kh[1], ul1, S[t]);
          S[t] = mfma32(kl[0], uh0, S[t]);
          S[t] = mfma32(kl[1], uh1, S[t]);
#pragma unroll
          for (int e = 0; e < 16; ++e) S[t][e] *= sm.eg_e[32 * t + acc_row(e, lane)];
        }
      }
    }
    __syncthreads();   // every wave is done reading lq / P / Wn / rk
    // ------------------------------------------------ outputs: stage through LDS, store rows
    if (chain) {
      // stage O (scaled, output type) into the lq area: [32 rows][D columns]
      TOUT* stg = reinterpret_cast<TOUT*>(&sm.lq_hi[0][0]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = acc_row(e, lane);
        io<TOUT>::st(stg + r * D + ncol, oacc[e] * p.scale);
      }
    }
    __syncthreads();
    {
      constexpr int OV = 16 / sizeof(TOUT);   // elements per vector
      constexpr int NOV = D / OV;             // vectors per row
      const TOUT* stg = reinterpret_cast<const TOUT*>(&sm.lq_hi[0][0]);
      for (int it = tid; it < TILE * NOV; it += NT) {
        const int r = it / NOV;
        const int c0 = (it % NOV) * OV;
        const int64_t pos = base + r;
        if (r < CH && pos >= start && pos < end && c0 < d) {
          const int64_t tok = bos + (pos - start);
          TOUT* dstp = og + tok * p.o_stride + static_cast<int64_t>(h) * d + c0;
          *reinterpret_cast<uint4*>(dstp) = *reinterpret_cast<const uint4*>(stg + r * D + c0);
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
          if (chain && slot >= 0 && slot < p.n_slots && ncol < d)
            state_store<D>(p.pool + (static_cast<int64_t>(slot) * H + h) * d * d, S, lane, ncol, d);
          if (tid == 0 && h == 0 && p.ckpt_pos_out) p.ckpt_pos_out[idx] = static_cast<int32_t>(after);
        }
      }
    }
    __syncthreads();
  }
  // ---- final state
  if (chain && has_dst && ncol < d) state_store<D>(p.pool + (static_cast<int64_t>(dst) * H + h) * d * d, S, lane, ncol, d);
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
