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
// Work split: a workgroup of 8 waves (2 per SIMD) owns one (sequence, head).
// Wave w owns columns [16w, 16w + 16) of the d_v axis: its slice of the fp32
// state lives in matrix-core accumulator registers (16x16 tiles) for the
// whole sequence, and the state-dependent chain (u, O, state update) never
// leaves the wave; the two waves on a SIMD run independent chains, which
// hides each other's matrix-core and LDS latency.  The chunk-local operands
// (gates, A, T, P, W) are built cooperatively in LDS (~84 KB).  The next
// chunk's raw tiles are loaded into registers while the current chunk is
// processed.
//
// Matrix-core precision (bf16 operands, fp32 accumulation); an operand
// marked "pair" is carried as hi + lo bf16 (hi*hi + hi*lo + lo*hi):
//     A = left_k right_k^T          single bf16
//     P = left_q right_k^T          pair x pair
//     T = (I + A)^{-1} diag(beta)   fp32 (16-row blocks), stored single
//     W = T left_k, U = T V         single
//     u: W S'                       single
//     O: left_q S'  pair x pair;    P u   pair x pair
//     state: right_k^T u            pair x pair
// With fp32 inputs every product is pair x pair.
//
// Layout tricks:
//  * Contractions whose operand comes from accumulator registers (S' over
//    the key channels, u over chunk rows) take a fragment from two
//    vertically adjacent 16x16 accumulator tiles; inside each block of 32
//    the contracted index is therefore stored in the order pos32 (below) in
//    the LDS operand on the other side.
//  * Operands that must be read K-contiguous from a row-major tile (right_k^T,
//    left_k and V over chunk rows) use the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16): four lanes of a 16-lane group read one row each,
//    lane i of the group receives column i of the four rows.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace pf {

constexpr int TILE = 32;   // rows per chunk tile
constexpr int NW = 8;      // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int MID = 15;    // reference row of the gates
constexpr int GATE_WAVES = 4;  // waves that form the next chunk's gates during the solve

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Storage position of contracted index c inside its block of 32: the
// fragment slot 8g + e (g = lane / 16, e = 0..7) of a contraction fed from
// accumulator tiles holds row 4g + e (e < 4) of the upper tile and row
// 16 + 4g + e - 4 (e >= 4) of the lower tile.
__host__ __device__ constexpr int pos32(int c) {
  return (c & ~31) | (8 * ((c & 15) >> 2)) | (4 * ((c >> 4) & 1)) | (c & 3);
}

// Workgroup barrier that orders LDS traffic only.  Waves exchange data
// through LDS alone, so outstanding global loads (the prefetched next tile)
// and stores may stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// fp32 -> bf16 bits (hardware round to nearest even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float hi_of(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

// An opaque copy of x: values derived from it cannot be hoisted out of a loop.
__device__ __forceinline__ int launder(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

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

// store 4 floats as bf16 (8 bytes)
__device__ __forceinline__ void st4b(bf16_t* p, const float* x) {
  uint2 u;
  u.x = cvt2(x[0], x[1]);
  u.y = cvt2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = u;
}
// store 8 floats as bf16 (16 bytes)
__device__ __forceinline__ void st8b(bf16_t* p, const float* x) {
  uint4 u;
  u.x = cvt2(x[0], x[1]);
  u.y = cvt2(x[2], x[3]);
  u.z = cvt2(x[4], x[5]);
  u.w = cvt2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// x broadcast from lane S of each row of 16 lanes (DPP row_newbcast)
template <int S>
__device__ __forceinline__ float bcast16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + S, 0xF, 0xF, true));
}

// Forward substitution down the 16 lanes of each lane row: lane r holds x_r
// of one right-hand side and na[s] = -L[r][s] of the unit lower triangular L
// (zero for s >= r); steps S..14 apply x_r += na[s] x_s with x_s final.
template <int S, int NG>
__device__ __forceinline__ void fsub16(float (&x)[NG], const float (&na)[16]) {
  if constexpr (S < 15) {
#pragma unroll
    for (int g = 0; g < NG; ++g) x[g] = __builtin_fmaf(na[S], bcast16<S>(x[g]), x[g]);
    fsub16<S + 1, NG>(x, na);
  }
}

// fragment (and hi / lo pair) from two vertically adjacent accumulator tiles
__device__ __forceinline__ void frag_pair(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = hi_of(x[i]);
    l[i] = x[i] - h[i];
  }
  uint4 uh, ul;
  uh.x = cvt2(h[0], h[1]); uh.y = cvt2(h[2], h[3]); uh.z = cvt2(h[4], h[5]); uh.w = cvt2(h[6], h[7]);
  ul.x = cvt2(l[0], l[1]); ul.y = cvt2(l[2], l[3]); ul.z = cvt2(l[4], l[5]); ul.w = cvt2(l[6], l[7]);
  hi = __builtin_bit_cast(bf16x8, uh);
  lo = __builtin_bit_cast(bf16x8, ul);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The state slice of a chain wave <-> a pool slot [c][n] (fp32).  Inlined
// with compile-time tile indices so the slice stays in registers; when
// d == D the row stride is a constant and a single per-lane address serves
// every element.
template <int D>
__device__ __forceinline__ void state_store(float* base, const f32x4 (&S)[D / 16], int lane, int ncol, int d) {
  if (D > 32 || d == D) {   // the launch pairs D = 64, 128 only with d = D
    float* b = base + 4 * (lane >> 4) * D + ncol;
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) b[(16 * q + i) * D] = S[q][i];
    return;
  }
#pragma unroll
  for (int q = 0; q < D / 16; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * q + 4 * (lane >> 4) + i;
      if (c < d) base[c * d + ncol] = S[q][i];
    }
}

template <int D>
__device__ __forceinline__ void state_load(const float* base, f32x4 (&S)[D / 16], int lane, int ncol, int d) {
  if (D > 32 || d == D) {
    const float* b = base + 4 * (lane >> 4) * D + ncol;
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[q][i] = b[(16 * q + i) * D];
    return;
  }
#pragma unroll
  for (int q = 0; q < D / 16; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * q + 4 * (lane >> 4) + i;
      const float v = base[(c < d ? c : 0) * d + ncol];
      S[q][i] = c < d ? v : 0.f;
    }
}

// Row pitches of the bf16 tiles are padded (by 32 bytes for the [32][D]
// tiles, to 80 bytes for the [32][32] ones) so that the 16-byte fragment reads
// of 16 rows and the transpose reads of 4 x 4 rows spread over the LDS banks.
template <int D, typename TIN, typename TOUT>
struct Smem {
  static constexpr bool F32IN = sizeof(TIN) == 4;
  static constexpr int PD = D + 16;   // padded pitch of [TILE][D] bf16 tiles
  static constexpr int PT = TILE + 8; // padded pitch of [TILE][TILE] bf16 tiles
  static constexpr int PO = D + 16 / static_cast<int>(sizeof(TOUT));  // padded pitch of the output tile
  alignas(16) TOUT ostg[TILE][PO];  // scaled outputs of the previous chunk, stored during the next one
  alignas(16) bf16_t lq_hi[TILE][PD];     // [r][pos32(c)]
  bf16_t lq_lo[TILE][PD];
  bf16_t lk[TILE][PD];        // [r][pos32(c)]
  bf16_t lk_lo[F32IN ? TILE : 1][PD];
  bf16_t rk_hi[TILE][PD];     // [s][pos32(c)]
  bf16_t rk_lo[TILE][PD];
  bf16_t v_hi[TILE][PD];      // [s][n]
  bf16_t v_lo[F32IN ? TILE : 1][PD];
  alignas(16) float eg_m[2][D];           // exp(G_m), by chunk parity
  alignas(16) float eg_e[2][D];           // exp(G_last - G_m), by chunk parity
  alignas(16) TIN g_raw[TILE][D];         // raw gates of the next chunk
  alignas(16) float G[TILE][D];           // cumulative gates of the next chunk
  float beta[2][TILE];                    // by chunk parity
  union {
    struct {
      alignas(16) float At[TILE][TILE + 4];  // At[s][r] = beta_r <left_k[r], right_k[s]>, s < r
      bf16_t P_hi[TILE][PT];  // [r][pos32(s)]
      bf16_t P_lo[TILE][PT];
      bf16_t Wn[TILE][PD];    // -(T left_k) [r][pos32(c)]
      bf16_t Wn_lo[F32IN ? TILE : 1][PD];
      alignas(16) float Tf[16][20];       // T00 (fp32)
      bf16_t Tb[TILE][PT];                // T = (I + A)^{-1} diag(beta) [r][s]
      bf16_t Tb_lo[F32IN ? TILE : 1][PT];
    } b;
  } u;
};

// raw slice of one token row: channels {c0..c0+3} and {c0+16..c0+19} of q, k, v, g
template <typename TIN>
struct RawRow {
  static constexpr int NU = 4 * sizeof(TIN) / 8;   // 8-byte units per 4-channel group
  uint2 q[2 * NU], k[2 * NU], v[2 * NU], g[2 * NU];
};

template <typename TIN>
__device__ __forceinline__ void to_f32(const uint2* w, float (&x)[8]) {
  if constexpr (sizeof(TIN) == 2) {
    const uint32_t u[4] = {w[0].x, w[0].y, w[1].x, w[1].y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i].x);
      x[2 * i + 1] = __uint_as_float(w[i].y);
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, typename TIN, typename TOUT>
__global__ void __launch_bounds__(NT, 1) prefill_kernel(const PrefillParams p, const int d, const int CH) {
  using SM = Smem<D, TIN, TOUT>;
  __shared__ SM sm;
  constexpr bool HP = SM::F32IN;        // all products as pairs
  constexpr int NWC = D / 16;           // waves that own state columns
  constexpr int NQ = D / 16;            // 16-row state tiles per wave
  constexpr int NPB = D / 8;            // 8-position blocks per row
  constexpr int NITEM = TILE * NPB;     // (row, position block) items per chunk
  constexpr int NU = RawRow<TIN>::NU;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;             // 16-lane group
  const int l16 = lane & 15;
  const int H = p.H;
  // pass A runs both of its modes in one launch (grid.y = 2)
  const int mode = p.mode == kModePassA ? kModeLocal + static_cast<int>(blockIdx.y) : p.mode;
  const int item = static_cast<int>(blockIdx.x / H);
  const int h = static_cast<int>(blockIdx.x % H);
  // work item -> (sequence s, segment m): without a segment table every
  // sequence is one item; with one, seg_cu holds each sequence's first item
  int s = item, m = 0, nseg = 1;
  if (p.seg_cu) {
    if (item >= p.seg_cu[p.n_seq]) return;
    int a = 0, b = p.n_seq;               // seg_cu[a] <= item < seg_cu[b]
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (p.seg_cu[mid] <= item) a = mid; else b = mid;
    }
    s = a;
    m = item - p.seg_cu[s];
    nseg = p.seg_cu[s + 1] - p.seg_cu[s];
  } else if (item >= p.n_seq) {
    return;
  }
  const bool first_seg = m == 0;
  const bool last_seg = m == nseg - 1;
  // pass A (local end state / transition) is not needed for a last segment,
  // and the transition of a first segment is never used
  if (mode == kModeLocal && last_seg) return;
  if (mode == kModeTransition && (first_seg || last_seg)) return;

  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  const int64_t len = eos - bos;
  int64_t start = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (start < 0) start = 0;
  const int64_t end = start + len;
  // token range [lo, hi) of this work item: the whole sequence, or its part
  // inside absolute window w0 + m of the segment length
  int64_t lo = start, hi = end;
  if (nseg > 1) {
    const int64_t seg = p.segment_len;
    const int64_t w0 = start / seg;
    lo = first_seg ? start : (w0 + m) * seg;
    hi = (w0 + m + 1) * seg;
    hi = hi < end ? hi : end;
  }
  const bool outputs = mode == kModeFull;
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  const bool has_dst = dst >= 0 && dst < p.n_slots && last_seg && outputs;
  // segment-scan blocks of this item (kind 0: incoming state, 1: local end
  // state, 2: transition), each a d x d fp32 matrix per head
  const int64_t blk = p.seg_cu ? static_cast<int64_t>(p.blk_cu[s]) + m : -1;
  const bool has_blk = nseg > 1 && blk >= 0 && blk < p.ws_max_blocks;
  auto ws_block = [&](int kind) -> float* {
    return p.ws_states + (blk * 3 + kind) * H * d * d + static_cast<int64_t>(h) * d * d;
  };
  const bool chain = wave < NWC;
  const int ncol = 16 * wave + l16;     // d_v column of this lane (chain waves)

  // ---- state: D x 16 slice per chain wave, NQ tiles of 16 x 16 (fp32)
  f32x4 S[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) S[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mode == kModeTransition) {
    // transition of the segment: the recurrence applied to S = I with V = 0
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[q][i] = (16 * q + 4 * g4 + i == ncol) ? 1.f : 0.f;
  } else if (first_seg) {
    if (chain && has_src && ncol < d) state_load<D>(p.pool + (static_cast<int64_t>(src) * H + h) * d * d, S, lane, ncol, d);
  } else if (mode == kModeFull && has_blk) {
    if (chain && ncol < d) state_load<D>(ws_block(0), S, lane, ncol, d);
  }
  // The initial state is complete here: a first use inside the chunk loop
  // would leave a wait for all outstanding memory operations in every trip.
#pragma unroll
  for (int q = 0; q < NQ; ++q) asm volatile("" : "+v"(S[q]));

  const TIN* qg = static_cast<const TIN*>(p.q);
  const TIN* kg = static_cast<const TIN*>(p.k);
  const TIN* vg = static_cast<const TIN*>(p.v);
  const TIN* gg = static_cast<const TIN*>(p.g);
  const TIN* bg = static_cast<const TIN*>(p.beta);
  TOUT* og = static_cast<TOUT*>(p.o);

  // raw-tile item of this thread: row ir, positions [8 ib, 8 ib + 8) which
  // hold channels c0..c0+3 and c0+16..c0+19
  const bool has_item = tid < NITEM;
  const int ir = tid / NPB;
  const int ib = tid % NPB;
  const int c0 = 32 * (ib >> 2) + 4 * (ib & 3);

  // Raw rows in registers.  Item (row ir, position block ib) holds channels
  // c0..c0+3 and c0+16..c0+19: q and k of the next chunk (consumed by its
  // gated-operand phase), g and v (and beta of row tid) of the chunk after
  // the current one, committed to LDS one chunk ahead.
  struct QKRow {
    uint2 q[2 * NU], k[2 * NU];
  } qk;
  struct GVRow {
    uint2 g[2 * NU], v[2 * NU];
    TIN b;
  } gv;
  // Registers that receive a load are never written by ALU code before the
  // load is known complete (that write would wait for every memory
  // operation in flight): rows outside the sequence are masked where the
  // values are consumed instead of zeroed here.
  auto row_ok = [&](int64_t pos) { return has_item && ir < CH && pos >= lo && pos < hi && c0 < d; };
  auto load_qk = [&](int64_t base) {
    const int64_t pos = base + ir;
    if (row_ok(pos)) {
      const int64_t tok = bos + (pos - start);
      const int64_t off = static_cast<int64_t>(h) * d + c0;
      const TIN* qp = qg + tok * p.q_stride + off;
      const TIN* kp = kg + tok * p.k_stride + off;
      const bool second = c0 + 16 < d;   // d = 16: only the first group exists
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        qk.q[w] = reinterpret_cast<const uint2*>(qp)[w];
        qk.k[w] = reinterpret_cast<const uint2*>(kp)[w];
        if (second) {
          qk.q[NU + w] = reinterpret_cast<const uint2*>(qp + 16)[w];
          qk.k[NU + w] = reinterpret_cast<const uint2*>(kp + 16)[w];
        }
      }
    }
  };
  auto load_gv = [&](int64_t base) {
    const int64_t pos = base + ir;
    const bool with_v = mode != kModeTransition;   // the transition runs with v = 0
    if (row_ok(pos)) {
      const int64_t tok = bos + (pos - start);
      const int64_t off = static_cast<int64_t>(h) * d + c0;
      const TIN* vp = vg + tok * p.v_stride + off;
      const TIN* gp = gg + tok * p.g_stride + off;
      const bool second = c0 + 16 < d;
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        if (with_v) gv.v[w] = reinterpret_cast<const uint2*>(vp)[w];
        gv.g[w] = reinterpret_cast<const uint2*>(gp)[w];
        if (second) {
          if (with_v) gv.v[NU + w] = reinterpret_cast<const uint2*>(vp + 16)[w];
          gv.g[NU + w] = reinterpret_cast<const uint2*>(gp + 16)[w];
        }
      }
    }
    // beta stays in raw input bits until it is committed
    const int64_t bpos = base + tid;
    if (tid < CH && bpos >= lo && bpos < hi) gv.b = bg[(bos + (bpos - start)) * p.beta_stride + h];
  };
  // (uint2 pair of one 4-channel group) or zeros
  auto masked = [](const uint2& x, bool ok) { return ok ? x : make_uint2(0, 0); };
  // g and beta of chunk nbase (parity npar) -> LDS
  auto commit_g = [&](int64_t nbase, int npar) {
    if (has_item) {
      const bool ok = row_ok(nbase + ir), ok2 = ok && c0 + 16 < d;
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        reinterpret_cast<uint2*>(&sm.g_raw[ir][c0])[w] = masked(gv.g[w], ok);
        reinterpret_cast<uint2*>(&sm.g_raw[ir][c0 + 16])[w] = masked(gv.g[NU + w], ok2);
      }
    }
    if (tid < TILE) {
      const int64_t bpos = nbase + tid;
      const bool ok = tid < CH && bpos >= lo && bpos < hi;
      sm.beta[npar][tid] = ok ? io<TIN>::ld(&gv.b) : 0.f;
    }
  };
  // v of chunk nbase -> LDS (after the current W / U products)
  auto commit_v = [&](int64_t nbase) {
    if (has_item) {
      const bool ok = row_ok(nbase + ir) && mode != kModeTransition, ok2 = ok && c0 + 16 < d;
      uint2 vv[2 * NU];
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        vv[w] = masked(gv.v[w], ok);
        vv[NU + w] = masked(gv.v[NU + w], ok2);
      }
      if constexpr (HP) {
        float vx[8], vh[8], vl[8];
        to_f32<TIN>(vv, vx);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          vh[i] = hi_of(vx[i]);
          vl[i] = vx[i] - vh[i];
        }
        st4b(&sm.v_hi[ir][c0], vh);
        st4b(&sm.v_hi[ir][c0 + 16], vh + 4);
        st4b(&sm.v_lo[ir][c0], vl);
        st4b(&sm.v_lo[ir][c0 + 16], vl + 4);
      } else {
        *reinterpret_cast<uint2*>(&sm.v_hi[ir][c0]) = vv[0];
        *reinterpret_cast<uint2*>(&sm.v_hi[ir][c0 + 16]) = vv[1];
      }
    }
  };
  // G = inclusive cumulative sum of g down the chunk rows, per key channel,
  // from g_raw; exp(G_m) and exp(G_last - G_m) into eg[par].  Run by
  // GATE_WAVES waves (gw = 0 ..): each takes D / GATE_WAVES channels, each
  // lane a run of RP rows of one channel; the runs are chained by a scan
  // across the lanes of the wave.
  auto gates = [&](int par, int gw) {
    constexpr int CPW = D / GATE_WAVES;
    constexpr int NPART = 64 / CPW;
    constexpr int RP = TILE / NPART;
    const int c = CPW * gw + lane % CPW;
    const int part = lane / CPW;
    float gl[RP];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      acc += io<TIN>::ld(&sm.g_raw[part * RP + i][c]);
      gl[i] = acc;
    }
    float incl = acc;
#pragma unroll
    for (int o = 1; o < NPART; o <<= 1) {
      const float y = __shfl_up(incl, o * CPW, 64);
      if (part >= o) incl += y;
    }
    const float off = incl - acc;
#pragma unroll
    for (int i = 0; i < RP; ++i) sm.G[part * RP + i][c] = gl[i] + off;
    // G at the reference row and at the last row, from the lanes that hold them
    const float gm = __shfl(gl[MID % RP] + off, (MID / RP) * CPW + lane % CPW, 64);
    const float ge = __shfl(gl[RP - 1] + off, (NPART - 1) * CPW + lane % CPW, 64);
    if (part == 0) {
      sm.eg_m[par][c] = expf(gm);
      sm.eg_e[par][c] = expf(ge - gm);
    }
  };

  const int64_t first = hi > lo ? (lo / CH) * CH : hi;
  // rows of the staged output tile that belong to the sequence -> o (16-byte stores)
  auto store_out = [&](int64_t obase) {
    constexpr int OV = 16 / sizeof(TOUT);   // elements per vector
    constexpr int NOV = D / OV;             // vectors per row
    for (int it = static_cast<int>(threadIdx.x); it < TILE * NOV; it += NT) {
      const int r = it / NOV;
      const int cc = (it % NOV) * OV;
      const int64_t pos = obase + r;
      if (r < CH && pos >= lo && pos < hi && cc < d) {
        const int64_t tok = bos + (pos - start);
        TOUT* dstp = og + tok * p.o_stride + static_cast<int64_t>(h) * d + cc;
        *reinterpret_cast<uint4*>(dstp) = *reinterpret_cast<const uint4*>(&sm.ostg[r][cc]);
      }
    }
  };
  // prologue: the first chunk's g, v, beta in LDS, its gates, q / k in
  // registers, and the second chunk's g, v, beta requested
  if (hi > lo) {
    load_gv(first);
    load_qk(first);
    commit_g(first, 0);
    commit_v(first);
    lds_barrier();
    if (wave < GATE_WAVES) gates(0, wave);
    if (first + CH < hi) load_gv(first + CH);
    lds_barrier();
  }
  auto chunk = [&](const int64_t base, const int par) __attribute__((always_inline)) {
    // Per-thread indices are derived again in every chunk from an opaque copy
    // of the thread id; otherwise every LDS address derived from them would be
    // hoisted out of this loop and held in a register for the whole sequence.
    const int tid = launder(static_cast<int>(threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int l16 = lane & 15;
    const bool chain = wave < NWC;
    const int ncol = 16 * wave + l16;
    const bool has_item = tid < NITEM;
    const int ir = tid / NPB;
    const int ib = tid % NPB;
    const int c0 = 32 * (ib >> 2) + 4 * (ib & 3);
    const bool more = base + CH < hi;
    // ------------------------------------------------ phase O: gated operands (row-major)
    if (has_item) {
      float qx[8], kx[8];
      {
        const bool ok = row_ok(base + ir), ok2 = ok && c0 + 16 < d;
        uint2 qq[2 * NU], kk[2 * NU];
#pragma unroll
        for (int w = 0; w < NU; ++w) {
          qq[w] = masked(qk.q[w], ok);
          kk[w] = masked(qk.k[w], ok);
          qq[NU + w] = masked(qk.q[NU + w], ok2);
          kk[NU + w] = masked(qk.k[NU + w], ok2);
        }
        to_f32<TIN>(qq, qx);
        to_f32<TIN>(kk, kx);
      }
      // positions 8 ib + e hold channels c0 + e (e < 4) and c0 + 16 + e - 4
      float lq[8], lk[8], rk[8];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int cc = c0 + 16 * gi;
        const float4 a = *reinterpret_cast<const float4*>(&sm.G[ir][cc]);
        const float4 b = *reinterpret_cast<const float4*>(&sm.G[MID][cc]);
        const float x4[4] = {a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = 4 * gi + m;
          const float ea = fexp(x4[m]);
          lq[i] = qx[i] * ea;
          lk[i] = kx[i] * ea;
          rk[i] = kx[i] * fexp(-x4[m]);
        }
      }
      const int pp = 8 * ib;
      float hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hi[i] = hi_of(lq[i]);
        lo[i] = lq[i] - hi[i];
      }
      st8b(&sm.lq_hi[ir][pp], hi);
      st8b(&sm.lq_lo[ir][pp], lo);
      if constexpr (HP) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = hi_of(lk[i]);
          lo[i] = lk[i] - hi[i];
        }
        st8b(&sm.lk[ir][pp], hi);
        st8b(&sm.lk_lo[ir][pp], lo);
      } else {
        st8b(&sm.lk[ir][pp], lk);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hi[i] = hi_of(rk[i]);
        lo[i] = rk[i] - hi[i];
      }
      st8b(&sm.rk_hi[ir][pp], hi);
      st8b(&sm.rk_lo[ir][pp], lo);
    }
    // outputs of the previous chunk (staged at its end), then the next
    // chunk's q / k: both after this chunk's q / k are consumed, so that the
    // wait for those covers neither
    if (outputs && base != first) store_out(base - CH);
    if (more) load_qk(base + CH);
    lds_barrier();
    // ------------------------------------------------ phase AP: A and P (16x16 tiles)
    {
      const int kq = 8 * g4;   // k offset of this lane inside a 32-wide K step
      if (wave < 3) {
        // P tile per wave: 0 -> (0,0), 1 -> (1,0), 2 -> (1,1); lower incl. diagonal
        const int I = wave == 0 ? 0 : 1;
        const int J = wave == 2 ? 1 : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 ah = frag_lds(&sm.lq_hi[16 * I + l16][32 * ks + kq]);
          const bf16x8 bh = frag_lds(&sm.rk_hi[16 * J + l16][32 * ks + kq]);
          acc = mfma(ah, bh, acc);
          acc = mfma(ah, frag_lds(&sm.rk_lo[16 * J + l16][32 * ks + kq]), acc);
          acc = mfma(frag_lds(&sm.lq_lo[16 * I + l16][32 * ks + kq]), bh, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * g4 + i;
          const int c = 16 * J + l16;
          const float v = c <= r ? acc[i] : 0.f;
          const float hv = hi_of(v);
          sm.u.b.P_hi[r][pos32(c)] = f32_to_bf16(hv);
          sm.u.b.P_lo[r][pos32(c)] = f32_to_bf16(v - hv);
        }
      } else if (wave < 6) {
        // A tile per wave: 3 -> (0,0), 4 -> (1,0), 5 -> (1,1); strictly lower, scaled by beta_row
        const int I = wave == 3 ? 0 : 1;
        const int J = wave == 5 ? 1 : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 a = frag_lds(&sm.lk[16 * I + l16][32 * ks + kq]);
          const bf16x8 b = frag_lds(&sm.rk_hi[16 * J + l16][32 * ks + kq]);
          acc = mfma(a, b, acc);
          if constexpr (HP) {
            acc = mfma(a, frag_lds(&sm.rk_lo[16 * J + l16][32 * ks + kq]), acc);
            acc = mfma(frag_lds(&sm.lk_lo[16 * I + l16][32 * ks + kq]), b, acc);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * g4 + i;
          const int c = 16 * J + l16;
          sm.u.b.At[c][r] = r > c ? acc[i] * sm.beta[par][r] : 0.f;
        }
      } else if (wave == 6) {
        // tile (0,1) of A and P is zero
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i;
          sm.u.b.At[16 + l16][r] = 0.f;
          sm.u.b.P_hi[r][pos32(16 + l16)] = 0;
          sm.u.b.P_lo[r][pos32(16 + l16)] = 0;
        }
      }
    }
    // the next chunk's g and beta (its gates are formed during phase X)
    if (more) commit_g(base + CH, par ^ 1);
    lds_barrier();
    // ------------------------------------------------ phase X: T = (I + A)^{-1} diag(beta); W = T left_k, U = T V
    // Blockwise on the 16-row blocks b, with L_b = I + A_bb:
    //     T_bb = L_b^{-1} diag(beta_b),  T10 = -M T00,  M = L_1^{-1} A10,
    // each inverse by fp32 forward substitution down the 16 lanes of a lane
    // row (lane (g4, r) holds row r of column 4 g + g4, g = 0..3).
    if (wave < 2) {
      // T_bb = L_b^{-1} diag(beta_b), b = wave
      const int b = wave;
      float na[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) na[s] = -sm.u.b.At[16 * b + s][16 * b + l16];
      float x[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) x[g] = l16 == 4 * g + g4 ? 1.f : 0.f;
      fsub16<0, 4>(x, na);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = 4 * g + g4;
        const float t = x[g] * sm.beta[par][16 * b + j];
        const float th = hi_of(t);
        sm.u.b.Tb[16 * b + l16][16 * b + j] = f32_to_bf16(th);
        if constexpr (HP) sm.u.b.Tb_lo[16 * b + l16][16 * b + j] = f32_to_bf16(t - th);
      }
    } else if (wave == 2) {
      // T10 = -M T00 with M = L_1^{-1} A10: both factors by forward
      // substitution in this wave, the product on fp32 matrix cores
      float na0[16], na1[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        na0[s] = -sm.u.b.At[s][l16];
        na1[s] = -sm.u.b.At[16 + s][16 + l16];
      }
      float x[4], m[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = 4 * g + g4;
        x[g] = l16 == j ? 1.f : 0.f;
        m[g] = sm.u.b.At[j][16 + l16];     // A10[r][j] = A[16 + r][j]
      }
      fsub16<0, 4>(x, na0);
      fsub16<0, 4>(m, na1);
      // T00 in LDS for the transposed operand; lane (g4, r) then reads
      // T00[4 kb + g4][r] (this wave's own writes: its LDS operations complete
      // in order)
#pragma unroll
      for (int g = 0; g < 4; ++g) sm.u.b.Tf[l16][4 * g + g4] = x[g] * sm.beta[par][4 * g + g4];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[kb], sm.u.b.Tf[4 * kb + g4][l16], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = -acc[e];
        const float th = hi_of(t);
        sm.u.b.Tb[16 + 4 * g4 + e][l16] = f32_to_bf16(th);
        if constexpr (HP) sm.u.b.Tb_lo[16 + 4 * g4 + e][l16] = f32_to_bf16(t - th);
      }
    } else if (wave == 3) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sm.u.b.Tb[l16][16 + 4 * g + g4] = 0;
        if constexpr (HP) sm.u.b.Tb_lo[l16][16 + 4 * g + g4] = 0;
      }
    } else if (more) {
      // the next chunk's gates, on the waves the solve leaves free
      gates(par ^ 1, wave - (NW - GATE_WAVES));
    }
    lds_barrier();
    // W = T left_k (columns of this wave in storage order, kept as -W in LDS)
    // and U = T V (own d_v columns, kept in registers)
    f32x4 U[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (chain) {
      // B fragments over chunk rows s = 8 g4 + e (transpose reads), columns 16 wave + l16
      const int j = (lane >> 2) & 3, i = lane & 3;
      const int x0 = 16 * wave + 4 * i;
      const int r0 = 8 * g4 + j;
      const bf16x8 bk = join(tr4(&sm.lk[r0][x0]), tr4(&sm.lk[r0 + 4][x0]));
      const bf16x8 bv = join(tr4(&sm.v_hi[r0][x0]), tr4(&sm.v_hi[r0 + 4][x0]));
      bf16x8 bkl = bk, bvl = bv;
      if constexpr (HP) {
        bkl = join(tr4(&sm.lk_lo[r0][x0]), tr4(&sm.lk_lo[r0 + 4][x0]));
        bvl = join(tr4(&sm.v_lo[r0][x0]), tr4(&sm.v_lo[r0 + 4][x0]));
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = frag_lds(&sm.u.b.Tb[16 * mt + l16][8 * g4]);
        f32x4 w = {0.f, 0.f, 0.f, 0.f};
        w = mfma(a, bk, w);
        U[mt] = mfma(a, bv, U[mt]);
        if constexpr (HP) {
          const bf16x8 al = frag_lds(&sm.u.b.Tb_lo[16 * mt + l16][8 * g4]);
          w = mfma(a, bkl, w);
          w = mfma(al, bk, w);
          U[mt] = mfma(a, bvl, U[mt]);
          U[mt] = mfma(al, bv, U[mt]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float wv = -w[e];
          const float wh = hi_of(wv);
          sm.u.b.Wn[16 * mt + 4 * g4 + e][16 * wave + l16] = f32_to_bf16(wh);
          if constexpr (HP) sm.u.b.Wn_lo[16 * mt + 4 * g4 + e][16 * wave + l16] = f32_to_bf16(wv - wh);
        }
      }
    }
    lds_barrier();
    // ------------------------------------------------ chain (per wave, own 16 columns)
    f32x4 O[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // WITH_O: the recurrence alone (segment pass A) skips every product that
    // only feeds the outputs.
    auto chain_step = [&](auto with_o) {
      constexpr bool WITH_O = decltype(with_o)::value;
      const int kq = 8 * g4;
      // S' = Diag(exp G_m) S, and its bf16 pair fragments (K steps of 32 channels)
      bf16x8 sh[NQ / 2], sl[NQ / 2];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(&sm.eg_m[par][16 * q + 4 * g4]);
        S[q][0] *= f.x; S[q][1] *= f.y; S[q][2] *= f.z; S[q][3] *= f.w;
      }
#pragma unroll
      for (int ks = 0; ks < NQ / 2; ++ks) frag_pair(S[2 * ks], S[2 * ks + 1], sh[ks], sl[ks]);
      // u = U - W S' ; O = left_q S'.  Three independent accumulators for the
      // pair terms keep the matrix-core pipeline fed.
      f32x4 Ob[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      f32x4 Oc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < NQ / 2; ++ks) {
        bf16x8 w[2], qh[2], ql[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int row = 16 * mt + l16;
          w[mt] = frag_lds(&sm.u.b.Wn[row][32 * ks + kq]);
          if constexpr (WITH_O) {
            qh[mt] = frag_lds(&sm.lq_hi[row][32 * ks + kq]);
            ql[mt] = frag_lds(&sm.lq_lo[row][32 * ks + kq]);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          U[mt] = mfma(w[mt], sh[ks], U[mt]);
          if constexpr (WITH_O) {
            O[mt] = mfma(qh[mt], sh[ks], O[mt]);
            Ob[mt] = mfma(qh[mt], sl[ks], Ob[mt]);
            Oc[mt] = mfma(ql[mt], sh[ks], Oc[mt]);
          }
          if constexpr (HP) {
            U[mt] = mfma(w[mt], sl[ks], U[mt]);
            U[mt] = mfma(frag_lds(&sm.u.b.Wn_lo[16 * mt + l16][32 * ks + kq]), sh[ks], U[mt]);
          }
        }
      }
      // u (in U) as a pair over the 32 chunk rows
      bf16x8 uh, ul;
      frag_pair(U[0], U[1], uh, ul);
      // O += P u
#pragma unroll
      for (int mt = 0; mt < 2 && WITH_O; ++mt) {
        const bf16x8 ph = frag_lds(&sm.u.b.P_hi[16 * mt + l16][kq]);
        const bf16x8 pl = frag_lds(&sm.u.b.P_lo[16 * mt + l16][kq]);
        O[mt] = mfma(ph, uh, O[mt]);
        Ob[mt] = mfma(ph, ul, Ob[mt]);
        Oc[mt] = mfma(pl, uh, Oc[mt]);
      }
      // S = Diag(exp(G_last - G_m)) (S' + right_k^T u).  right_k^T fragments
      // come from transpose reads of right_k [s][pos32(c)]: rows follow u's
      // order, columns are picked so that lane l16 receives channel 16 q + l16.
      {
        const int j = (lane >> 2) & 3, i = lane & 3;
        const int ra = 4 * g4 + j;      // rows for slots 0..3; ra + 16 for slots 4..7
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int col = 32 * (q >> 1) + 4 * (q & 1) + 8 * i;
          const bf16x8 kh = join(tr4(&sm.rk_hi[ra][col]), tr4(&sm.rk_hi[ra + 16][col]));
          const bf16x8 kl = join(tr4(&sm.rk_lo[ra][col]), tr4(&sm.rk_lo[ra + 16][col]));
          S[q] = mfma(kh, uh, S[q]);
          S[q] = mfma(kh, ul, S[q]);
          S[q] = mfma(kl, uh, S[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(&sm.eg_e[par][16 * q + 4 * g4]);
        S[q][0] *= f.x; S[q][1] *= f.y; S[q][2] *= f.z; S[q][3] *= f.w;
      }
#pragma unroll
      for (int mt = 0; mt < 2 && WITH_O; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[mt][i] += Ob[mt][i] + Oc[mt][i];
    };
    if (chain) {
      if (outputs) chain_step(std::true_type{});
      else chain_step(std::false_type{});
    }
    // ------------------------------------------------ next chunk: v, and the g / v / beta request for the one after
    if (more) {
      commit_v(base + CH);
      if (base + 2 * CH < hi) load_gv(base + 2 * CH);
    }
    // ------------------------------------------------ outputs: stage in LDS (stored during the next chunk)
    if (chain && outputs) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) io<TOUT>::st(&sm.ostg[16 * mt + 4 * g4 + e][ncol], O[mt][e] * p.scale);
    }
    // ------------------------------------------------ interval checkpoint
    if (outputs && p.ckpt_interval > 0 && p.ckpt_cu) {
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
    lds_barrier();
  };
  int par = 0;
  for (int64_t base = first; base < hi; base += CH) {
    chunk(base, par);
    par ^= 1;
  }
  if (outputs && hi > lo) {
    lds_barrier();
    store_out(first + ((hi - 1 - first) / CH) * CH);
  }
  // ---- final state: the destination slot, or a segment-scan block
  if (chain && ncol < d) {
    if (has_dst) state_store<D>(p.pool + (static_cast<int64_t>(dst) * H + h) * d * d, S, lane, ncol, d);
    if (mode == kModeLocal && has_blk) state_store<D>(ws_block(1), S, lane, ncol, d);
    if (mode == kModeTransition && has_blk) state_store<D>(ws_block(2), S, lane, ncol, d);
  }
}

// ---------------------------------------------------------------------------
// Segment plan (one workgroup): per sequence the number of work items (1, or
// its number of segments when it is split) and of workspace blocks (0, or
// the same number), as exclusive prefix sums seg_cu / blk_cu.
__device__ __forceinline__ int seq_segments(const PrefillParams& p, int s) {
  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  const int64_t len = eos - bos;
  int64_t start = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (start < 0) start = 0;
  const int64_t seg = p.segment_len;
  if (len < 2 * seg) return 1;
  return static_cast<int>((start + len - 1) / seg - start / seg + 1);
}

constexpr int PLAN_T = 256;

__global__ void __launch_bounds__(PLAN_T) segment_plan_kernel(const PrefillParams p, int32_t* seg_cu, int32_t* blk_cu) {
  __shared__ int64_t part_i[PLAN_T], part_b[PLAN_T];
  const int t = threadIdx.x;
  const int per = (p.n_seq + PLAN_T - 1) / PLAN_T;
  const int a = t * per;
  const int b = a + per < p.n_seq ? a + per : p.n_seq;
  int64_t ci = 0, cb = 0;
  for (int s = a; s < b; ++s) {
    const int n = seq_segments(p, s);
    ci += n;
    cb += n > 1 ? n : 0;
  }
  part_i[t] = ci;
  part_b[t] = cb;
  __syncthreads();
  if (t == 0) {
    int64_t ri = 0, rb = 0;
    for (int j = 0; j < PLAN_T; ++j) {
      const int64_t xi = part_i[j], xb = part_b[j];
      part_i[j] = ri;
      part_b[j] = rb;
      ri += xi;
      rb += xb;
    }
    seg_cu[p.n_seq] = static_cast<int32_t>(ri);
    blk_cu[p.n_seq] = static_cast<int32_t>(rb);
  }
  __syncthreads();
  int64_t ri = part_i[t], rb = part_b[t];
  for (int s = a; s < b; ++s) {
    const int n = seq_segments(p, s);
    seg_cu[s] = static_cast<int32_t>(ri);
    blk_cu[s] = static_cast<int32_t>(rb);
    ri += n;
    rb += n > 1 ? n : 0;
  }
}

// Chains the segments of every split sequence, per (sequence, head) and
// block of 16 state columns, in fp32:
//     S_in(1) = S_loc(0),   S_in(j+1) = M_j S_in(j) + S_loc(j).
constexpr int COMB_T = 256;

__global__ void __launch_bounds__(COMB_T) segment_combine_kernel(const PrefillParams p, int d) {
  __shared__ float X[128][16];
  const int H = p.H;
  const int s = static_cast<int>(blockIdx.x / H);
  const int h = static_cast<int>(blockIdx.x % H);
  const int c0 = 16 * static_cast<int>(blockIdx.y);
  const int nseg = p.seg_cu[s + 1] - p.seg_cu[s];
  const int64_t b0 = p.blk_cu[s];
  if (nseg < 2 || b0 < 0 || b0 + nseg > p.ws_max_blocks || c0 >= d) return;
  const int t = threadIdx.x;
  const int r = t >> 1;            // state row (key channel)
  const int j0 = 8 * (t & 1);      // first of this thread's 8 columns
  const bool act = r < d;
  const int64_t dd = static_cast<int64_t>(d) * d;
  auto blk = [&](int64_t m, int kind) -> float* {
    return p.ws_states + ((b0 + m) * 3 + kind) * H * dd + static_cast<int64_t>(h) * dd;
  };
  float acc[8];
  if (act) {
    const float* sl = blk(0, 1) + static_cast<int64_t>(r) * d + c0 + j0;
    float* si = blk(1, 0) + static_cast<int64_t>(r) * d + c0 + j0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = (c0 + j0 + j < d) ? sl[j] : 0.f;
      if (c0 + j0 + j < d) si[j] = acc[j];
      X[r][j0 + j] = acc[j];
    }
  }
  for (int m = 1; m + 1 < nseg; ++m) {
    __syncthreads();
    if (act) {
      const float* mr = blk(m, 2) + static_cast<int64_t>(r) * d;
      const float* sl = blk(m, 1) + static_cast<int64_t>(r) * d + c0 + j0;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = (c0 + j0 + j < d) ? sl[j] : 0.f;
      for (int k = 0; k < d; ++k) {
        const float mk = mr[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += mk * X[k][j0 + j];
      }
    }
    __syncthreads();
    if (act) {
      float* si = blk(m + 1, 0) + static_cast<int64_t>(r) * d + c0 + j0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        X[r][j0 + j] = acc[j];
        if (c0 + j0 + j < d) si[j] = acc[j];
      }
    }
  }
}

template <int D, typename TIN, typename TOUT>
static int launch_kernel(const PrefillParams& p, int d, int CH, int64_t n_items, int gy, hipStream_t stream) {
  const int64_t nblk = n_items * p.H;
  if (nblk > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "prefill grid too large");
  if (nblk == 0) return KDA_OK;
  hipLaunchKernelGGL((prefill_kernel<D, TIN, TOUT>), dim3(static_cast<uint32_t>(nblk), gy), dim3(NT), 0, stream, p, d,
                     CH);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

template <int D, typename TIN, typename TOUT>
static int launch_t(const PrefillParams& p0, int d, int CH, hipStream_t stream) {
  PrefillParams p = p0;
  if (!p.seg_cu) {
    p.mode = kModeFull;
    return launch_kernel<D, TIN, TOUT>(p, d, CH, p.n_seq, 1, stream);
  }
  // work items: every sequence once, plus the extra segments of split ones
  // (a split sequence of len tokens adds at most len / seg + 1 <= 1.5 len / seg)
  const int64_t n_items = p.n_seq + (3 * p.T_tot) / (2 * static_cast<int64_t>(p.segment_len)) + 1;
  hipLaunchKernelGGL(segment_plan_kernel, dim3(1), dim3(PLAN_T), 0, stream, p, const_cast<int32_t*>(p.seg_cu),
                     const_cast<int32_t*>(p.blk_cu));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "segment plan launch: %s", hipGetErrorString(e));
  p.mode = kModePassA;
  int st = launch_kernel<D, TIN, TOUT>(p, d, CH, n_items, 2, stream);
  if (st) return st;
  const int64_t ncomb = static_cast<int64_t>(p.n_seq) * p.H;
  if (ncomb > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "segment combine grid too large");
  hipLaunchKernelGGL(segment_combine_kernel, dim3(static_cast<uint32_t>(ncomb), (d + 15) / 16), dim3(COMB_T), 0,
                     stream, p, d);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "segment combine launch: %s", hipGetErrorString(e));
  p.mode = kModeFull;
  return launch_kernel<D, TIN, TOUT>(p, d, CH, n_items, 1, stream);
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

// Effective segment length: 0 = the default, < 0 = never split.
static int64_t effective_segment(const PrefillParams& p) {
  return p.segment_len == 0 ? kDefaultSegmentLen : p.segment_len;
}

static int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: seg_cu [n_seq + 1] and blk_cu [n_seq + 1] (int32, each
// rounded up to 256 bytes), then 3 fp32 blocks [H][d][d] per block index.
// A split sequence of len >= 2 seg tokens spans at most 2 len / seg
// segments, so 2 T_tot / seg + 1 block indices always suffice.
int64_t prefill_workspace_bytes(const PrefillParams& p, int D) {
  const int64_t seg = effective_segment(p);
  if (seg <= 0 || p.T_tot < 2 * seg) return 0;
  const int64_t blocks = 2 * p.T_tot / seg + 1;
  return 2 * round256(4 * (static_cast<int64_t>(p.n_seq) + 1)) +
         blocks * 3 * p.H * static_cast<int64_t>(D) * D * 4;
}

int launch_prefill(const PrefillParams& p0, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  // chunk 64 runs as two chunks of 32 (identical result up to rounding)
  const int CH = p0.chunk == 16 ? 16 : 32;
  PrefillParams p = p0;
  p.seg_cu = p.blk_cu = nullptr;
  p.ws_states = nullptr;
  p.ws_max_blocks = 0;
  if (prefill_workspace_bytes(p0, D) > 0) {
    const int64_t seg = effective_segment(p0);
    char* w = static_cast<char*>(p.workspace);
    const int64_t idx = round256(4 * (static_cast<int64_t>(p.n_seq) + 1));
    p.segment_len = static_cast<int32_t>(seg);
    p.seg_cu = reinterpret_cast<const int32_t*>(w);
    p.blk_cu = reinterpret_cast<const int32_t*>(w + idx);
    p.ws_states = reinterpret_cast<float*>(w + 2 * idx);
    p.ws_max_blocks = 2 * p.T_tot / seg + 1;
  }
  if (in_dtype == KDA_BF16) {
    if (out_dtype == KDA_BF16) return pf::launch_d<bf16_t, bf16_t>(p, D, CH, stream);
    return pf::launch_d<bf16_t, float>(p, D, CH, stream);
  }
  if (out_dtype == KDA_BF16) return pf::launch_d<float, bf16_t>(p, D, CH, stream);
  return pf::launch_d<float, float>(p, D, CH, stream);
}

}  // namespace kda
