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
// leaves the wave.  The chunk-local operands (gates, gated q / k, A, T, P,
// W, U) depend only on the chunk's own inputs, so the loop is a software
// pipeline: while the chain of chunk n runs, the operands of chunk n + 1 are
// built in the same three barrier-separated phases (the chain and the blocks
// of A in the first, P and the triangular solve in the second, W / U and the
// gated operands in the third).  Operands read by a chain while the next chunk's
// are formed are double-buffered in LDS; raw rows are prefetched into
// registers one or two chunks ahead.
//
// Matrix-core precision (bf16 operands, fp32 accumulation); an operand
// marked "pair" is carried as hi + lo bf16 (hi*hi + hi*lo + lo*hi):
//     A = left_k right_k^T          single bf16
//     P = left_q right_k^T          pair x pair
//     T = (I + A)^{-1} diag(beta)   fp32 (16-row blocks), stored single;
//                                   its block T10 = -M T00 is applied as
//                                   (-M) (T00 X) with -M a pair
//     W = T left_k, U = T V         single (the T00 U part a pair inside
//                                   the T10 correction)
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
#include "kda_mfma.h"

namespace kda {
namespace pf {

constexpr int TILE = 32;   // rows per chunk tile
constexpr int NW = 8;      // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int MID = 15;    // reference row of the gates
constexpr int GATE_WAVES = 2;  // waves that form the next chunk's gates during the solve

using namespace mx;

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
  // bf16 outputs are staged for 16-byte stores (padded pitch); fp32 outputs
  // leave from registers (64-byte row segments) and need no tile
  static constexpr bool STAGE_O = sizeof(TOUT) == 2;
  static constexpr int PO = D + 8;
  alignas(16) TOUT ostg[STAGE_O ? TILE : 1][PO];  // scaled outputs of a chunk, stored in the same step
  // gated operands: two copies, by chunk parity (those of the next chunk
  // are formed while the current chunk's are still read)
  alignas(16) bf16_t lq_hi[2][TILE][PD];  // [r][pos32(c)]
  bf16_t lq_lo[2][TILE][PD];
  bf16_t rk_hi[2][TILE][PD];  // [s][pos32(c)]
  bf16_t rk_lo[2][TILE][PD];
  bf16_t lk[2][TILE][PD];     // [r][pos32(c)]
  bf16_t lk_lo[2][F32IN ? TILE : 1][PD];
  bf16_t P_hi[TILE][PT];      // [r][pos32(s)]
  bf16_t P_lo[TILE][PT];
  bf16_t v_hi[TILE][PD];      // [s][n]
  bf16_t v_lo[F32IN ? TILE : 1][PD];
  alignas(16) float eg_m[2][D];           // exp(G_m), by chunk parity
  alignas(16) float eg_e[2][D];           // exp(G_last - G_m), by chunk parity
  alignas(16) float eg_c[2][D];           // exp(G_last - G_m) of the chunk before times exp(G_m)
  uint32_t eg_split[2][GATE_WAVES];       // that product is below the normal fp32 range somewhere
  alignas(16) float G[TILE][D];           // cumulative gates (log2 units) of the next chunk
  alignas(16) float beta[2][TILE];        // by chunk parity
  bf16_t Tb[TILE][PT];                    // T = (I + A)^{-1} diag(beta) [r][s], block (1,0) zero
  bf16_t Tb_lo[F32IN ? TILE : 1][PT];
  alignas(16) bf16_t Mb[16][PT];          // -M = -L_1^{-1} A10: hi in columns 0..15, lo in 16..31

  alignas(16) TIN g_raw[TILE][D];         // raw gates of the next chunk
  uint32_t nonzero[NW];                   // transition mode: wave's state slice not all zero
  // 16x16 blocks of A, transposed ([c][r] = A[r][c]): A00, A11, A10, formed
  // by waves 0-2 in phase I, read by the solve waves in phase II
  float At[3][16][17];
  union {
    // from the W product to the chain
    struct {
      bf16_t Wn[TILE][PD];    // -(T left_k) [r][pos32(c)]
      bf16_t Wn_lo[F32IN ? TILE : 1][PD];
    } w;
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
  // Waves w and w + 4 share a SIMD and run the same instruction stream, so
  // their matrix and vector work would line up in time.  Waves 0-3 issue
  // first (higher wave priority); waves 4-7 fill their stalls.
  if (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) < 4) __builtin_amdgcn_s_setprio(1);
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
  // Modes.  Full: an unsplit launch.  Segment scan, pass A (one launch,
  // grid.y = 2): local (y = 0) runs every segment with outputs and
  // checkpoints, the first one from its true initial state and the others
  // from zero, and keeps each end state S_loc; transition (y = 1) runs M of
  // every later segment from I with v = 0 and records after how many chunks
  // M was exactly zero.  Fix-up (pass B, after the combine): every later
  // segment reruns, from its combined incoming state, the chunks before its
  // M became zero.
  const int mode = p.mode == kModePassA ? kModeLocal + static_cast<int>(blockIdx.y) : p.mode;
  int item = static_cast<int>(blockIdx.x / H);
  const int h = static_cast<int>(blockIdx.x % H);
  // work item -> (sequence s, segment m): without a segment table every
  // sequence is one item; with one, seg_cu holds each sequence's first item,
  // and blocks take the items longest first (the plan's order table)
  int s = item, m = 0, nseg = 1;
  if (p.seg_cu) {
    if (item >= p.seg_cu[p.n_seq]) return;
    if (p.item_order) item = p.item_order[item];
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
  // The transition of a first segment is never needed; a first segment (and
  // an unsplit sequence) is final after pass A and has no fix-up
  if (mode == kModeTransition && first_seg) return;
  if (mode == kModeFixup && first_seg) return;

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
  const bool outputs = mode != kModeTransition;
  const int src = p.src_slot[s];
  const int dst = p.dst_slot[s];
  const bool has_src = src >= 0 && src < p.n_slots;
  // segment-scan blocks of this item (kind 0: incoming state, 1: local end
  // state, 2: transition), each a d x d fp32 matrix per head
  const int64_t blk = p.seg_cu ? static_cast<int64_t>(p.blk_cu[s]) + m : -1;
  const bool has_blk = nseg > 1 && blk >= 0 && blk < p.ws_max_blocks;
  // Fix-up (pass B) of a later segment: the state entering the segment is
  // the combined one, and only the chunks before the segment's transition
  // became exactly zero are run again (all of them if it never did); past
  // that point the local chain of pass A, started from zero, is the state.
  bool full_run = true;
  if (mode == kModeFixup) {
    const int32_t kz = has_blk && p.ws_zero ? p.ws_zero[blk * H + h] : -1;
    if (kz >= 0) {
      const int64_t stop = (lo / CH) * CH + static_cast<int64_t>(kz) * CH;
      if (stop < hi) {
        hi = stop;
        full_run = false;
      }
    }
  }
  // The final state of a split sequence is written by the fix-up launch only:
  // pass A also runs the first segment, which reads src_slot when it starts,
  // so a pass-A write of dst_slot would race with it when src == dst.
  const bool dst_ok = dst >= 0 && dst < p.n_slots;
  const bool has_dst = dst_ok && last_seg && outputs && full_run && (mode != kModeLocal || nseg == 1);
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
  } else if (mode == kModeFixup && has_blk) {
    // S_in(m) = M_{m-1} S_in(m-1) + S_loc(m-1): S_loc(m-1) itself for m = 1
    // or an exactly zero M_{m-1}, else the combine's result
    const bool direct = m == 1 || (p.ws_zero && p.ws_zero[(blk - 1) * H + h] >= 0);
    const float* sin = direct ? p.ws_states + ((blk - 1) * 3 + 1) * H * d * d + static_cast<int64_t>(h) * d * d
                              : ws_block(0);
    if (chain && ncol < d) state_load<D>(sin, S, lane, ncol, d);
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
  // c0..c0+3 and c0+16..c0+19 of a row: q and k of the chunk after next
  // (consumed by its gated operands at the end of a step), v of the next
  // chunk and g (with beta of row tid) of the chunk after it, each committed
  // to LDS at the start of a step.
  struct QKRow {
    uint2 q[2 * NU], k[2 * NU];
  } qk;
  struct GRow {
    uint2 g[2 * NU];
    TIN b;
  } gr;
  struct VRow {
    uint2 v[2 * NU];
  } vr;
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
  auto load_g = [&](int64_t base) {
    const int64_t pos = base + ir;
    if (row_ok(pos)) {
      const int64_t tok = bos + (pos - start);
      const TIN* gp = gg + tok * p.g_stride + static_cast<int64_t>(h) * d + c0;
      const bool second = c0 + 16 < d;
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        gr.g[w] = reinterpret_cast<const uint2*>(gp)[w];
        if (second) gr.g[NU + w] = reinterpret_cast<const uint2*>(gp + 16)[w];
      }
    }
    // beta stays in raw input bits until it is committed
    const int64_t bpos = base + tid;
    if (tid < CH && bpos >= lo && bpos < hi) gr.b = bg[(bos + (bpos - start)) * p.beta_stride + h];
  };
  auto load_v = [&](int64_t base) {
    const int64_t pos = base + ir;
    // the transition runs with v = 0
    if (row_ok(pos) && mode != kModeTransition) {
      const int64_t tok = bos + (pos - start);
      const TIN* vp = vg + tok * p.v_stride + static_cast<int64_t>(h) * d + c0;
      const bool second = c0 + 16 < d;
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        vr.v[w] = reinterpret_cast<const uint2*>(vp)[w];
        if (second) vr.v[NU + w] = reinterpret_cast<const uint2*>(vp + 16)[w];
      }
    }
  };
  // (uint2 pair of one 4-channel group) or zeros
  auto masked = [](const uint2& x, bool ok) { return ok ? x : make_uint2(0, 0); };
  // g and beta of chunk nbase (parity npar) -> LDS
  auto commit_g = [&](int64_t nbase, int npar) {
    if (has_item) {
      const bool ok = row_ok(nbase + ir), ok2 = ok && c0 + 16 < d;
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        reinterpret_cast<uint2*>(&sm.g_raw[ir][c0])[w] = masked(gr.g[w], ok);
        reinterpret_cast<uint2*>(&sm.g_raw[ir][c0 + 16])[w] = masked(gr.g[NU + w], ok2);
      }
    }
    if (tid < TILE) {
      const int64_t bpos = nbase + tid;
      const bool ok = tid < CH && bpos >= lo && bpos < hi;
      sm.beta[npar][tid] = ok ? io<TIN>::ld(&gr.b) : 0.f;
    }
  };
  // v of chunk nbase -> LDS (after the current W / U products)
  auto commit_v = [&](int64_t nbase) {
    if (has_item) {
      const bool ok = row_ok(nbase + ir) && mode != kModeTransition, ok2 = ok && c0 + 16 < d;
      uint2 vv[2 * NU];
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        vv[w] = masked(vr.v[w], ok);
        vv[NU + w] = masked(vr.v[NU + w], ok2);
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
  // from g_raw, kept in log2 units (g log2 e summed); exp(G_m) and
  // exp(G_last - G_m) into eg[par].  Run by
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
      acc += io<TIN>::ld(&sm.g_raw[part * RP + i][c]) * kLog2e;
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
    bool tiny = false;
    if (part == 0) {
      const float em = __builtin_amdgcn_exp2f(gm);
      sm.eg_m[par][c] = em;
      sm.eg_e[par][c] = __builtin_amdgcn_exp2f(ge - gm);
      // this lane wrote eg_e of the chunk before (same channel)
      const float ec = sm.eg_e[par ^ 1][c] * em;
      sm.eg_c[par][c] = ec;
      // two factors of up to 16 tokens of decay each can multiply to below
      // the normal range while each alone and the scaled state stay in it;
      // the chain then applies them one after the other
      tiny = !(ec >= 1.17549435e-38f);
    }
    const uint64_t tb = __ballot(tiny);
    if (lane == 0) sm.eg_split[par][gw] = tb != 0 ? 1u : 0u;
  };

  const int64_t first = hi > lo ? (lo / CH) * CH : hi;
  // rows of the staged output tile that belong to the sequence -> o (16-byte stores)
  auto store_out = [&](int64_t obase) {
    constexpr int OV = 16 / sizeof(TOUT);   // elements per vector
    constexpr int NOV = D / OV;             // vectors per row
    if constexpr (SM::STAGE_O)
    for (int it = static_cast<int>(threadIdx.x); it < TILE * NOV; it += NT) {
      const int r = it / NOV;
      const int cc = (it % NOV) * OV;
      const int64_t pos = obase + r;
      if (r < CH && pos >= lo && pos < hi && cc < d) {
        const int64_t tok = bos + (pos - start);
        TOUT* dstp = og + tok * p.o_stride + static_cast<int64_t>(h) * d + cc;
        // written once: a non-temporal store (1.582 against 1.589 ms per varlen call;
        // non-temporal row loads were slower, 1.61 ms)
        typedef __attribute__((ext_vector_type(4))) uint32_t u4v;
        __builtin_nontemporal_store(*reinterpret_cast<const u4v*>(&sm.ostg[r][cc]), reinterpret_cast<u4v*>(dstp));
      }
    }
  };
  // Gated operands of chunk c (parity par) from its q / k rows in registers
  // and its cumulative gates:
  //   left_q = q exp(G_r - G_m), left_k = k exp(G_r - G_m), right_k = k exp(G_m - G_r)
  // (row-major, position 8 ib + e holds channel c0 + e (e < 4) or
  // c0 + 16 + e - 4).  Then the q / k request of chunk c + CH, issued after
  // this chunk's rows are consumed so that no wait covers it.
  auto gated_operands = [&](const int64_t c, const int par, const int tid) __attribute__((always_inline)) {
    const int ir = tid / NPB;
    const int ib = tid % NPB;
    const int c0 = 32 * (ib >> 2) + 4 * (ib & 3);
    if (NITEM >= NT || tid < NITEM) {
      float qx[8], kx[8];
      {
        const bool ok = row_ok(c + ir), ok2 = ok && c0 + 16 < d;
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
      float lq[8], lk[8], rk[8];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int cc = c0 + 16 * gi;
        const float4 a = *reinterpret_cast<const float4*>(&sm.G[ir][cc]);
        const float4 m4 = *reinterpret_cast<const float4*>(&sm.G[MID][cc]);
        const float x4[4] = {a.x - m4.x, a.y - m4.y, a.z - m4.z, a.w - m4.w};
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const int i = 4 * gi + mm;
          const float ea = __builtin_amdgcn_exp2f(x4[mm]);
          lq[i] = qx[i] * ea;
          lk[i] = kx[i] * ea;
          rk[i] = kx[i] * __builtin_amdgcn_exp2f(-x4[mm]);
        }
      }
      const int pp = 8 * ib;
      st8b_pair(&sm.lq_hi[par][ir][pp], &sm.lq_lo[par][ir][pp], lq);
      if constexpr (HP) {
        st8b_pair(&sm.lk[par][ir][pp], &sm.lk_lo[par][ir][pp], lk);
      } else {
        st8b(&sm.lk[par][ir][pp], lk);
      }
      st8b_pair(&sm.rk_hi[par][ir][pp], &sm.rk_lo[par][ir][pp], rk);
    }
    load_qk(c + CH);   // rows past the end of the item load nothing
  };

  // prologue: the first chunk's g and beta in LDS, its gates and gated
  // operands formed; in registers its v, the second chunk's g / beta and q / k
  if (hi > lo) {
    load_v(first);
    load_g(first);
    load_qk(first);
    commit_g(first, 0);
    load_g(first + CH);
    lds_barrier();
    if (wave < GATE_WAVES) gates(0, wave);
    lds_barrier();
    gated_operands(first, 0, tid);
    lds_barrier();
  }
  // Interval checkpoint taken after position `after` (absolute): its index
  // in the checkpoint table, or -1
  auto ckpt_index = [&](const int64_t after) -> int64_t {
    if (!outputs || p.ckpt_interval <= 0 || !p.ckpt_cu) return -1;
    if (after >= end || after % p.ckpt_interval != 0) return -1;
    const int64_t j = after / p.ckpt_interval - start / p.ckpt_interval - 1;
    const int64_t idx = static_cast<int64_t>(p.ckpt_cu[s]) + j;
    return (j >= 0 && idx < p.ckpt_cu[s + 1] && idx < p.n_ckpt) ? idx : -1;
  };
  // S = Diag(f) S on a chain wave's slice
  auto scale_state = [&](const float* f, const int g4_) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(&f[16 * q + 4 * g4_]);
      S[q][0] *= x.x; S[q][1] *= x.y; S[q][2] *= x.z; S[q][3] *= x.w;
    }
  };
  // the state enters the first chunk scaled by its exp(G_m)
  if (hi > lo && chain) scale_state(sm.eg_m[0], g4);
  // U = T V of the chunk whose chain runs next (own d_v columns)
  f32x4 U[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // One pipeline step: the chain of chunk n (parity cp) runs alongside the
  // chunk-local stages of chunk b = n + CH (parity lp = cp ^ 1), which need
  // nothing from the state.  Three phases separated by workgroup barriers:
  //   I    chain of n: state update, outputs  | v of b, g / beta of b + CH to LDS;
  //                                           | their requests for b + CH, b + 2 CH
  //   II   outputs of n stored                | P and T of b (T from the A blocks formed
  //                                           | by waves 0-2 at the end of phase I);
  //                                           | gates of b + CH
  //   III                                     | W = T left_k, U = T V of b;
  //                                           | gated operands of b + CH
  // CHAIN = false runs the local stages of the first chunk alone; MORE =
  // false (no chunk b) the chain alone.
  auto step = [&](const int64_t n, const int cp, auto chain_t, auto more_t, auto out_t) __attribute__((always_inline)) {
    constexpr bool CHAIN = decltype(chain_t)::value;
    constexpr bool MORE = decltype(more_t)::value;
    constexpr bool WITH_O = decltype(out_t)::value;
    const int lp = cp ^ 1;
    const int64_t b = n + CH;
    const bool more2 = b + CH < hi;      // a chunk after b exists
    // Per-thread indices are derived again in every step from an opaque copy
    // of the thread id; otherwise every LDS address derived from them would be
    // hoisted out of the loop and held in a register for the whole sequence.
    const int tid = launder(static_cast<int>(threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int l16 = lane & 15;
    const int kq = 8 * g4;   // k offset of this lane inside a 32-wide K step
    const bool chain = NWC == NW || wave < NWC;
    const int ncol = 16 * wave + l16;
    const int64_t ck = CHAIN ? ckpt_index(n + CH) : -1;

    // ================================================ phase I
    // v of chunk b and g / beta of chunk b + CH to LDS, then the requests of
    // v of b + CH and g / beta of b + 2 CH (rows past the end of the item
    // load nothing).  Before any store of this step, so that no store is
    // pending at the wait for the rows; on chain waves in the shadow of the
    // u products.
    auto rows = [&]() __attribute__((always_inline)) {
      if constexpr (MORE) {
        commit_v(b);
        if (more2) commit_g(b + CH, cp);
        load_v(b + CH);
        load_g(b + 2 * CH);
      }
    };
    // The blocks of A = strict-lower(diag(beta) left_k right_k^T) of chunk
    // b (operands complete since the previous step), one per wave on waves
    // 0-2, after their chain's products (issued before them, the A products
    // held up the chain: 1.566 against 1.522 ms per varlen call), written
    // transposed to the At tiles for the solve waves of phase II:
    // At[t][c][r] = beta_r <left_k[16 I + r], right_k[16 J + c]>, t = 0: A00,
    // 1: A11, 2: A10.
    auto a_products = [&]() __attribute__((always_inline)) {
      if constexpr (MORE) {
        if (wave < 3) {
          auto a_prod = [&](const int I, const int J, f32x4& acc) __attribute__((always_inline)) {
            // the three terms of the pair product in accumulators of their own:
            // dependent chains of D / 32 matrix operations instead of 3 D / 32
            f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
              const bf16x8 a = frag_lds(&sm.lk[lp][16 * I + l16][32 * ks + kq]);
              const bf16x8 bb = frag_lds(&sm.rk_hi[lp][16 * J + l16][32 * ks + kq]);
              acc = mfma(a, bb, acc);
              if constexpr (HP) {
                acc1 = mfma(a, frag_lds(&sm.rk_lo[lp][16 * J + l16][32 * ks + kq]), acc1);
                acc2 = mfma(frag_lds(&sm.lk_lo[lp][16 * I + l16][32 * ks + kq]), bb, acc2);
              }
            }
            if constexpr (HP) {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[i] += acc1[i] + acc2[i];
            }
          };
          const int I = wave == 0 ? 0 : 1;
          const int J = wave == 2 ? 1 : 0;
          const int tt = wave == 0 ? 0 : (wave == 1 ? 2 : 1);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          a_prod(I, J, acc);
          // beta of the lane's four rows in one read (read under the mask,
          // element by element, each read was waited for on its own)
          const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[lp][16 * I + 4 * g4]);
          const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            const float a = acc[i] * bv[i];
            sm.At[tt][l16][r] = (I > J || r > l16) ? a : 0.f;
          }
        }
      }
    };
    if (!(CHAIN && chain)) {
      rows();
      a_products();
    }
    if (CHAIN && chain) {
      // The LDS fragments of each product are read one stage ahead, behind
      // scheduling fences, so that their latency hides behind the work
      // before the product instead of stalling each matrix operation.
      // W fragments, read while S' = Diag(exp G_m) S (the register state
      // enters the chunk already scaled) becomes bf16 pair fragments
      bf16x8 wf[NQ / 2][2];
#pragma unroll
      for (int ks = 0; ks < NQ / 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) wf[ks][mt] = frag_lds(&sm.u.w.Wn[16 * mt + l16][32 * ks + kq]);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 sh[NQ / 2], sl[NQ / 2], uh, ul;
#pragma unroll
      for (int ks = 0; ks < NQ / 2; ++ks) frag_pair(S[2 * ks], S[2 * ks + 1], sh[ks], sl[ks]);
      // u = U - W S'
#pragma unroll
      for (int ks = 0; ks < NQ / 2; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          U[mt] = mfma(wf[ks][mt], sh[ks], U[mt]);
          if constexpr (HP) {
            U[mt] = mfma(wf[ks][mt], sl[ks], U[mt]);
            U[mt] = mfma(frag_lds(&sm.u.w.Wn_lo[16 * mt + l16][32 * ks + kq]), sh[ks], U[mt]);
          }
        }
      }
      rows();
      // right_k^T fragments (transpose reads of right_k [s][pos32(c)]: rows
      // follow u's order, columns are picked so that lane l16 receives
      // channel 16 q + l16), read while u becomes a pair
      bf16x8 kh[NQ], kl[NQ];
      {
        const int j = (lane >> 2) & 3, i = lane & 3;
        const int ra = 4 * g4 + j;      // rows for slots 0..3; ra + 16 for slots 4..7
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int col = 32 * (q >> 1) + 4 * (q & 1) + 8 * i;
          kh[q] = join(tr4(&sm.rk_hi[cp][ra][col]), tr4(&sm.rk_hi[cp][ra + 16][col]));
          kl[q] = join(tr4(&sm.rk_lo[cp][ra][col]), tr4(&sm.rk_lo[cp][ra + 16][col]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // u (in U) as a pair over the 32 chunk rows
      frag_pair(U[0], U[1], uh, ul);
      // S' + right_k^T u, with the output operands read behind it
      bf16x8 qf[NQ / 2][2][2], pf[2][2];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        S[q] = mfma(kh[q], uh, S[q]);
        S[q] = mfma(kh[q], ul, S[q]);
        S[q] = mfma(kl[q], uh, S[q]);
        if constexpr (WITH_O) {
          // two of the output fragments per state tile
          const int ks = q >> 1, mt = q & 1, row = 16 * mt + l16;
          qf[ks][mt][0] = frag_lds(&sm.lq_hi[cp][row][32 * ks + kq]);
          qf[ks][mt][1] = frag_lds(&sm.lq_lo[cp][row][32 * ks + kq]);
          if (q < 2) {
            pf[q][0] = frag_lds(&sm.P_hi[16 * q + l16][kq]);
            pf[q][1] = frag_lds(&sm.P_lo[16 * q + l16][kq]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // S = Diag(exp(G_last - G_m)) (S' + right_k^T u) is the state after
      // chunk n; it enters chunk b as Diag(exp G_m(b)) S, both factors in one
      // product unless the state after n is stored
      bool split = false;
      if constexpr (MORE) {
        uint32_t sp = 0;
#pragma unroll
        for (int gw = 0; gw < GATE_WAVES; ++gw) sp |= sm.eg_split[lp][gw];
        split = __builtin_amdgcn_readfirstlane(sp) != 0u;
      }
      const bool combined = MORE && ck < 0 && !split;
      const float* fs = combined ? sm.eg_c[lp] : sm.eg_e[cp];
      auto scale_tile = [&](const int q) __attribute__((always_inline)) {
        const float4 x = *reinterpret_cast<const float4*>(&fs[16 * q + 4 * g4]);
        S[q][0] *= x.x; S[q][1] *= x.y; S[q][2] *= x.z; S[q][3] *= x.w;
      };
      if constexpr (WITH_O) {
        // O = scale (left_q S' + P u) with three independent accumulators for
        // the pair terms, staged in LDS; the state scaling runs between the
        // products
        f32x4 O[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 Ob[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 Oc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < NQ / 2; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            O[mt] = mfma(qf[ks][mt][0], sh[ks], O[mt]);
            Ob[mt] = mfma(qf[ks][mt][0], sl[ks], Ob[mt]);
            Oc[mt] = mfma(qf[ks][mt][1], sh[ks], Oc[mt]);
          }
          scale_tile(2 * ks);
          scale_tile(2 * ks + 1);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          O[mt] = mfma(pf[mt][0], uh, O[mt]);
          Ob[mt] = mfma(pf[mt][0], ul, Ob[mt]);
          Oc[mt] = mfma(pf[mt][1], uh, Oc[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * mt + 4 * g4 + e;
            const float ov = (O[mt][e] + Ob[mt][e] + Oc[mt][e]) * p.scale;
            if constexpr (SM::STAGE_O) {
              io<TOUT>::st(&sm.ostg[r][ncol], ov);
            } else {
              const int64_t pos = n + r;
              if (r < CH && pos >= lo && pos < hi && ncol < d)
                io<TOUT>::st(og + (bos + (pos - start)) * p.o_stride + static_cast<int64_t>(h) * d + ncol, ov);
            }
          }
      } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) scale_tile(q);
      }
      a_products();
      if (ck >= 0) {
        const int slot = p.ckpt_slot[ck];
        if (slot >= 0 && slot < p.n_slots && ncol < d)
          state_store<D>(p.pool + (static_cast<int64_t>(slot) * H + h) * d * d, S, lane, ncol, d);
      }
      if constexpr (MORE) {
        if (!combined) scale_state(sm.eg_m[lp], g4);
      }
    }
    if (CHAIN && ck >= 0 && tid == 0 && h == 0 && p.ckpt_pos_out) p.ckpt_pos_out[ck] = static_cast<int32_t>(n + CH);
    lds_barrier();
    // ================================================ phase II
    // outputs of chunk n (no wait for a prefetched row follows before the
    // next phase: a wait on a load while stores are pending covers every
    // outstanding memory operation)
    if constexpr (CHAIN && WITH_O && SM::STAGE_O) store_out(n);
    if constexpr (MORE) {
      if (wave < 3) {
        // P tile per wave: 0 -> (0,0), 1 -> (1,0), 2 -> (1,1); lower incl. diagonal
        const int I = wave == 0 ? 0 : 1;
        const int J = wave == 2 ? 1 : 0;
        // the pair product's three terms in accumulators of their own
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc, acc2 = acc;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 ah = frag_lds(&sm.lq_hi[lp][16 * I + l16][32 * ks + kq]);
          const bf16x8 bh = frag_lds(&sm.rk_hi[lp][16 * J + l16][32 * ks + kq]);
          acc = mfma(ah, bh, acc);
          acc1 = mfma(ah, frag_lds(&sm.rk_lo[lp][16 * J + l16][32 * ks + kq]), acc1);
          acc2 = mfma(frag_lds(&sm.lq_lo[lp][16 * I + l16][32 * ks + kq]), bh, acc2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += acc1[i] + acc2[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * g4 + i;
          const int c = 16 * J + l16;
          const float v = c <= r ? acc[i] : 0.f;
          const float hv = hi_of(v);
          sm.P_hi[r][pos32(c)] = f32_to_bf16(hv);
          sm.P_lo[r][pos32(c)] = f32_to_bf16(v - hv);
          if (wave == 0) {   // block (0,1) of P is zero
            sm.P_hi[4 * g4 + i][pos32(16 + l16)] = 0;
            sm.P_lo[4 * g4 + i][pos32(16 + l16)] = 0;
          }
        }
      } else if (wave < 6) {
        // T = (I + A)^{-1} diag(beta) blockwise on the 16-row blocks, with
        // L_bb = I + A_bb:  T_bb = L_bb^{-1} diag(beta_bb), and
        // T10 = -M T00 with M = L_1^{-1} A10, which the W / U products apply
        // as a correction of the second row block.  Inverses by fp32 forward
        // substitution down the 16 lanes of a lane row (lane (g4, r) holds
        // row r of column 4 g + g4, g = 0..3), from the blocks of A formed
        // in phase I: wave 3 A00 (-> T00), wave 4 A10, A11 (-> M), wave 5
        // A11 (-> T11).
        if (wave != 4) {
          const int bb = wave == 3 ? 0 : 1;
          const int t = wave == 3 ? 0 : 1;
          float na[16];
#pragma unroll
          for (int s2 = 0; s2 < 16; ++s2) na[s2] = -sm.At[t][s2][l16];
          float x[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) x[g] = l16 == 4 * g + g4 ? 1.f : 0.f;
          // x was just written by VALU: two wait states before a DPP read
          asm volatile("s_nop 1" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
          fsub16<0, 4>(x, na);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j = 4 * g + g4;
            const float tv = x[g] * sm.beta[lp][16 * bb + j];
            const float th = hi_of(tv);
            sm.Tb[16 * bb + l16][16 * bb + j] = f32_to_bf16(th);
            if constexpr (HP) sm.Tb_lo[16 * bb + l16][16 * bb + j] = f32_to_bf16(tv - th);
            // the off-diagonal blocks of Tb are zero
            sm.Tb[16 * bb + l16][16 * (1 - bb) + j] = 0;
            if constexpr (HP) sm.Tb_lo[16 * bb + l16][16 * (1 - bb) + j] = 0;
          }
        } else {
          float na1[16];
#pragma unroll
          for (int s2 = 0; s2 < 16; ++s2) na1[s2] = -sm.At[1][s2][l16];
          float m4[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) m4[g] = sm.At[2][4 * g + g4][l16];   // A10[r][j]
          // m4 was just written by a load: wait states before a DPP read
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 1" ::"v"(m4[0]), "v"(m4[1]), "v"(m4[2]), "v"(m4[3]));
          fsub16<0, 4>(m4, na1);
          // -M as a bf16 pair: hi in columns 0..15, lo in columns 16..31
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float mv = -m4[g];
            const float mh = hi_of(mv);
            sm.Mb[l16][4 * g + g4] = f32_to_bf16(mh);
            sm.Mb[l16][16 + 4 * g + g4] = f32_to_bf16(mv - mh);
          }
        }
      } else if (more2) {
        // the gates of chunk b + CH
        gates(cp, wave - (NW - GATE_WAVES));
      }
      lds_barrier();
      // ================================================ phase III
      // W = T left_k (columns of this wave in storage order, kept as -W in
      // LDS) and U = T V (own d_v columns, kept in registers)
      if (chain) {
        // B fragments over chunk rows s = 8 g4 + e (transpose reads), columns 16 wave + l16
        const int j = (lane >> 2) & 3, i = lane & 3;
        const int x0 = 16 * wave + 4 * i;
        const int r0 = 8 * g4 + j;
        const bf16x8 bk = join(tr4(&sm.lk[lp][r0][x0]), tr4(&sm.lk[lp][r0 + 4][x0]));
        const bf16x8 bv = join(tr4(&sm.v_hi[r0][x0]), tr4(&sm.v_hi[r0 + 4][x0]));
        bf16x8 bkl = bk, bvl = bv;
        if constexpr (HP) {
          bkl = join(tr4(&sm.lk_lo[lp][r0][x0]), tr4(&sm.lk_lo[lp][r0 + 4][x0]));
          bvl = join(tr4(&sm.v_lo[r0][x0]), tr4(&sm.v_lo[r0 + 4][x0]));
        }
        // M fragments (A operand of the 16x16x16 products: row l16, K = 4 g4 .. 4 g4 + 3)
        const s16x4 mh = *reinterpret_cast<const s16x4*>(&sm.Mb[l16][4 * g4]);
        const s16x4 ml = *reinterpret_cast<const s16x4*>(&sm.Mb[l16][16 + 4 * g4]);
        f32x4 w0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = frag_lds(&sm.Tb[16 * mt + l16][8 * g4]);
          f32x4 w = {0.f, 0.f, 0.f, 0.f};
          f32x4 uu = {0.f, 0.f, 0.f, 0.f};
          w = mfma(a, bk, w);
          uu = mfma(a, bv, uu);
          if constexpr (HP) {
            const bf16x8 al = frag_lds(&sm.Tb_lo[16 * mt + l16][8 * g4]);
            w = mfma(a, bkl, w);
            w = mfma(al, bk, w);
            uu = mfma(a, bvl, uu);
            uu = mfma(al, bv, uu);
          }
          if (mt == 0) {
            w0 = w;
          } else {
            // second row block: T10 (.) = -M (T00 .), added as (-M) W0 and
            // (-M) U0.  The first block's results are the B operands of
            // 16x16x16 products as they stand (K = rows 4 g4 + e in this
            // lane's accumulator order).  -M and U0 as pairs; W0 single
            // (pair with fp32 inputs).
            uint32_t wb[2], wl[2], ub[2], ubl[2];
            split2(w0[0], w0[1], wb[0], wl[0]);
            split2(w0[2], w0[3], wb[1], wl[1]);
            split2(U[0][0], U[0][1], ub[0], ubl[0]);
            split2(U[0][2], U[0][3], ub[1], ubl[1]);
            const s16x4 wbv = __builtin_bit_cast(s16x4, make_uint2(wb[0], wb[1]));
            const s16x4 ubv = __builtin_bit_cast(s16x4, make_uint2(ub[0], ub[1]));
            const s16x4 ulv = __builtin_bit_cast(s16x4, make_uint2(ubl[0], ubl[1]));
            w = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mh, wbv, w, 0, 0, 0);
            if constexpr (HP) {
              const s16x4 wlv = __builtin_bit_cast(s16x4, make_uint2(wl[0], wl[1]));
              w = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mh, wlv, w, 0, 0, 0);
              w = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ml, wbv, w, 0, 0, 0);
            }
            uu = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mh, ubv, uu, 0, 0, 0);
            uu = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mh, ulv, uu, 0, 0, 0);
            uu = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ml, ubv, uu, 0, 0, 0);
          }
          U[mt] = uu;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float wv = -w[e];
            const float wh = hi_of(wv);
            sm.u.w.Wn[16 * mt + 4 * g4 + e][16 * wave + l16] = f32_to_bf16(wh);
            if constexpr (HP) sm.u.w.Wn_lo[16 * mt + 4 * g4 + e][16 * wave + l16] = f32_to_bf16(wv - wh);
          }
        }
      }
      // gated operands of chunk b + CH
      if (more2) gated_operands(b + CH, cp, tid);
      lds_barrier();
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Transition mode: M evolves with V = 0, so once every entry of M is
  // exactly zero it stays exactly zero (u = U - W S' = 0 and the state update
  // adds right_k^T 0), and the rest of the segment can be skipped without
  // changing a bit of the result.  Checked every ZCHK chunks (after a step,
  // whose last act is a barrier); with the usual decay M underflows to exact
  // zeros within a few hundred tokens, while a slowly decaying M (values held
  // at denormals) simply keeps running.
  constexpr int ZCHK = 1;
  auto m_is_zero = [&]() __attribute__((always_inline)) -> bool {
    const int tid = launder(static_cast<int>(threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (NWC == NW || wave < NWC) {
      uint32_t bits = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) bits |= __float_as_uint(S[q][i]) & 0x7fffffffu;
      const uint64_t nzm = __ballot(bits != 0u);
      if (lane == 0) sm.nonzero[wave] = nzm != 0 ? 1u : 0u;
    }
    lds_barrier();
    uint32_t any = 0;
#pragma unroll
    for (int w = 0; w < NWC; ++w) any |= sm.nonzero[w];
    return any == 0;
  };
  // one step variant per loop, so that nothing in the loop body joins
  // register values from different variants
  int32_t zero_after = -1;   // transition: chunks after which M was exactly zero
  auto run = [&](auto out_t) __attribute__((always_inline)) {
    constexpr bool WITH_O = decltype(out_t)::value;
    int cp = 0;
    int64_t n = first;
    int since = 0, done = 0;
    for (; n + CH < hi; n += CH) {
      step(n, cp, T_{}, T_{}, out_t);
      cp ^= 1;
      ++done;
      if constexpr (!WITH_O) {
        if (mode == kModeTransition && ++since == ZCHK) {
          since = 0;
          if (m_is_zero()) {   // M = 0 from here to the segment's end
            zero_after = done;
            return;
          }
        }
      }
    }
    step(n, cp, T_{}, F_{}, out_t);
  };
  if (hi > lo) {
    step(first - CH, 1, F_{}, T_{}, F_{});
    if (outputs) {
      run(T_{});

    } else {
      run(F_{});
    }
  }
  // ---- final state: the destination slot, or a segment-scan block
  if (chain && ncol < d) {
    if (has_dst) state_store<D>(p.pool + (static_cast<int64_t>(dst) * H + h) * d * d, S, lane, ncol, d);
    // every split segment keeps its local end state (the last one's is the
    // final state when its fix-up stops early)
    if (mode == kModeLocal && has_blk) state_store<D>(ws_block(1), S, lane, ncol, d);
    if (mode == kModeTransition && has_blk) state_store<D>(ws_block(2), S, lane, ncol, d);
    // fix-up of the last segment cut short: past the point where its
    // transition became exactly zero the local chain of pass A is the state,
    // so its end state is the final state
    if (mode == kModeFixup && last_seg && !full_run && dst_ok && has_blk) {
      state_load<D>(ws_block(1), S, lane, ncol, d);
      state_store<D>(p.pool + (static_cast<int64_t>(dst) * H + h) * d * d, S, lane, ncol, d);
    }
  }
  if (mode == kModeTransition && has_blk && p.ws_zero && threadIdx.x == 0) p.ws_zero[blk * H + h] = zero_after;
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
  if (len <= seg) return 1;
  return static_cast<int>((start + len - 1) / seg - start / seg + 1);
}

// Work items of a segment-scan launch: a sequence of len tokens spans at
// most len / seg + 2 segments (1 when it is not split), so there are at most
// min(n_seq + 3 T_tot / seg, T_tot / seg + 2 n_seq) + 1 of them.
__host__ __device__ inline int64_t max_work_items(int64_t n_seq, int64_t T_tot, int64_t seg) {
  const int64_t a = n_seq + 3 * T_tot / seg, b = T_tot / seg + 2 * n_seq;
  return (a < b ? a : b) + 1;
}

constexpr int PLAN_T = 256;
constexpr int PLAN_ORDER_MAX = 2048;   // items the order table ranks (LDS; quadratic ranking)

// tokens of segment m (of nseg) of sequence s
__device__ __forceinline__ int item_tokens(const PrefillParams& p, int s, int m, int nseg) {
  int64_t bos = p.cu[s], eos = p.cu[s + 1];
  bos = bos < 0 ? 0 : (bos > p.T_tot ? p.T_tot : bos);
  eos = eos < bos ? bos : (eos > p.T_tot ? p.T_tot : eos);
  int64_t start = p.start_pos ? static_cast<int64_t>(p.start_pos[s]) : 0;
  if (start < 0) start = 0;
  const int64_t end = start + (eos - bos);
  if (nseg <= 1) return static_cast<int>(end - start);
  const int64_t seg = p.segment_len;
  const int64_t w0 = start / seg;
  const int64_t lo = m == 0 ? start : (w0 + m) * seg;
  int64_t hi = (w0 + m + 1) * seg;
  hi = hi < end ? hi : end;
  return static_cast<int>(hi > lo ? hi - lo : 0);
}

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
  // Order table: items by decreasing token count (ties by item index), so
  // that the longest chains are dispatched first and the short ones fill the
  // gaps at the end.  Identity when there are more items than LDS slots.
  if (!p.item_order) return;
  __syncthreads();
  const int total = seg_cu[p.n_seq];
  __shared__ int32_t len_of[PLAN_ORDER_MAX];
  const bool sort = total <= PLAN_ORDER_MAX && total <= p.max_items;
  for (int i = t; i < total && i < p.max_items; i += PLAN_T) {
    if (!sort) {
      p.item_order[i] = i;
      continue;
    }
    int lo_s = 0, hi_s = p.n_seq;          // seg_cu[lo_s] <= i < seg_cu[hi_s]
    while (hi_s - lo_s > 1) {
      const int mid = (lo_s + hi_s) >> 1;
      if (seg_cu[mid] <= i) lo_s = mid; else hi_s = mid;
    }
    len_of[i] = item_tokens(p, lo_s, i - seg_cu[lo_s], seg_cu[lo_s + 1] - seg_cu[lo_s]);
  }
  if (!sort) return;
  __syncthreads();
  for (int i = t; i < total; i += PLAN_T) {
    const int li = len_of[i];
    int rank = 0;
    for (int j = 0; j < total; ++j) {
      const int lj = len_of[j];
      rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    p.item_order[rank] = i;
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
  // The fix-up of segment j reads S_loc(j-1) itself when M_{j-1} is exactly
  // zero (then S_in(j) = S_loc(j-1)); the chain is only needed when some
  // transition is not.
  if (p.ws_zero) {
    bool all_zero = true;
    for (int m = 1; m + 1 < nseg; ++m) all_zero = all_zero && p.ws_zero[(b0 + m) * H + h] >= 0;
    if (all_zero) return;
  }
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
    // a transition recorded as exactly zero contributes exactly nothing
    const bool m_zero = p.ws_zero && p.ws_zero[(b0 + m) * H + h] >= 0;
    __syncthreads();
    if (act) {
      const float* mr = blk(m, 2) + static_cast<int64_t>(r) * d;
      const float* sl = blk(m, 1) + static_cast<int64_t>(r) * d + c0 + j0;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = (c0 + j0 + j < d) ? sl[j] : 0.f;
      for (int k = 0; k < (m_zero ? 0 : d); ++k) {
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
  const int64_t n_items = max_work_items(p.n_seq, p.T_tot, p.segment_len);
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
  p.mode = kModeFixup;
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
// rounded up to 256 bytes), then 3 fp32 blocks [H][d][d] per block index,
// then one int32 per block index and head (where the transition became
// exactly zero), then the item order table (int32 per work item).  A sequence is split when it is longer than seg; it then
// spans at most len / seg + 2 < 3 len / seg segments, so 3 T_tot / seg + 1
// block indices always suffice.
int64_t prefill_workspace_bytes(const PrefillParams& p, int D) {
  const int64_t seg = effective_segment(p);
  if (seg <= 0 || p.T_tot <= seg) return 0;
  const int64_t blocks = 3 * p.T_tot / seg + 1;
  const int64_t items = pf::max_work_items(p.n_seq, p.T_tot, seg);
  return 2 * round256(4 * (static_cast<int64_t>(p.n_seq) + 1)) +
         blocks * 3 * p.H * static_cast<int64_t>(D) * D * 4 + round256(blocks * p.H * 4) + round256(items * 4);
}

int launch_prefill(const PrefillParams& p0, int D, int in_dtype, int out_dtype, hipStream_t stream) {
  // chunk 64 runs as two chunks of 32 (identical result up to rounding)
  const int CH = p0.chunk == 16 ? 16 : 32;
  PrefillParams p = p0;
  p.seg_cu = p.blk_cu = nullptr;
  p.ws_states = nullptr;
  p.ws_zero = nullptr;
  p.item_order = nullptr;
  p.max_items = 0;
  p.ws_max_blocks = 0;
  if (prefill_workspace_bytes(p0, D) > 0) {
    const int64_t seg = effective_segment(p0);
    char* w = static_cast<char*>(p.workspace);
    const int64_t idx = round256(4 * (static_cast<int64_t>(p.n_seq) + 1));
    p.segment_len = static_cast<int32_t>(seg);
    p.seg_cu = reinterpret_cast<const int32_t*>(w);
    p.blk_cu = reinterpret_cast<const int32_t*>(w + idx);
    p.ws_states = reinterpret_cast<float*>(w + 2 * idx);
    p.ws_max_blocks = 3 * p.T_tot / seg + 1;
    p.ws_zero = reinterpret_cast<int32_t*>(p.ws_states + p.ws_max_blocks * 3 * p.H * static_cast<int64_t>(D) * D);
    p.max_items = pf::max_work_items(p.n_seq, p.T_tot, seg);
    p.item_order = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(p.ws_zero) + round256(p.ws_max_blocks * p.H * 4));
  }
  if (in_dtype == KDA_BF16) {
    if (out_dtype == KDA_BF16) return pf::launch_d<bf16_t, bf16_t>(p, D, CH, stream);
    return pf::launch_d<bf16_t, float>(p, D, CH, stream);
  }
  if (out_dtype == KDA_BF16) return pf::launch_d<float, bf16_t>(p, D, CH, stream);
  return pf::launch_d<float, float>(p, D, CH, stream);
}

}  // namespace kda
