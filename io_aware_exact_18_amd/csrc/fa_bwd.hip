// fa_bwd.hip — bf16 backward kernels for gfx950.
//
// The backward never stores P: it recomputes each score/probability tile from Q, K and the per-row
// logsumexp kept by the forward ("Anatomy of a FlashAttention Kernel", section "How does
// FlashAttention save memory in the backward pass?"; "FlashAttention: where it matters", section "The
// Real Complexity", third bullet).  With S = scale · Q Kᵀ, P = exp(S − LSE) and upstream gradient dO:
//   dV = Pᵀ dO,  dP = dO Vᵀ,  dS = P ∘ (dP − D) with D_i = dO_i · O_i,  dQ = scale · dS K,
//   dK = scale · dSᵀ Q.
// D_i equals Σ_j P_ij dP_ij (the row term of the softmax Jacobian) because O_i = Σ_j P_ij V_j.
//
// Launches on the caller's stream, none with atomics (launch_bwd: D and dQ, then dK/dV):
//   1. bwd_pre: D_i = dO_i · O_i in fp32, or inside the dQ kernel (see there).  The workspace holds
//      −D_i: the dK/dV kernel starts each dP accumulation from the step's −D values, so dP − D needs
//      no subtraction.
//   2. bwd_dkdv: key/value-stationary.  One workgroup per 128 keys (4 waves × 32 keys).  Each wave
//      keeps its K rows as matrix-core operands and its dKᵀ, dVᵀ accumulators in registers (V rows
//      stay in LDS) and walks the 32-query tiles the causal mask allows, from the last one down (all
//      key blocks of a head then share each Q/dO tile through L2), staged in LDS by direct
//      buffer→LDS copies (double-buffered, one barrier per tile).  Per tile: S = Q Kᵀ and
//      dP = dO Vᵀ (32×32×16 bf16 matrix cores, Q and dO rows from LDS), P and dS on the vector
//      units, then dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS with transposed LDS reads supplying dOᵀ and Qᵀ.
//      At head dimension 256 it runs as two passes, dV then dK (see the kernel).
//   3. bwd_dq: query-stationary, the same shape as the forward: one workgroup per 128 queries
//      (4 waves × 32), key/value tiles of 64 streamed through LDS.  Per tile it recomputes Sᵀ = K Qᵀ
//      and dPᵀ = V dOᵀ (each lane owns one query, so LSE_i and D_i are per-lane scalars), forms dSᵀ,
//      and accumulates dQᵀ += Kᵀ dSᵀ with K read transposed from LDS.
// Head dimension 96 keeps its tiles in the d = 128 LDS layout (lds_cols in fa_common.h).
// Split backward (fa_bwd_split, the forward's key-range split rule): the SPLIT instantiations run one
// segment of the dQ kernel's key tiles or of the dK/dV kernel's query steps and write fp32 partial
// sums; bwd_split_reduce_kernel adds a row's segments, scales and rounds to bf16.
// Splitting dQ off costs two recomputed products (7 matrix products executed for the 5 counted) but
// removes the fp32 atomics a single-kernel dQ would need: measured on MI355X, device-wide fp32 atomic
// adds sustain about 1.3 TB/s, which for the 4096-token causal workload alone would take ~3 ms.
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // dK/dV kernel: keys per workgroup (32 per wave)
constexpr int kBQ = 32;    // dK/dV kernel: queries per step
constexpr int kBR = 128;   // dQ kernel: queries per workgroup (32 per wave)
constexpr int kBC = 64;    // dQ kernel: keys per tile
// Resident workgroups per compute unit (registers and LDS), for the grid order (head_tile).
template <int D>
constexpr int dq_per_cu() { return D == 64 ? 4 : D == 256 ? 1 : 2; }
template <int D, int OUT>
constexpr int dkdv_per_cu() { return D == 64 ? 3 : (D == 256 && OUT == 2) ? 1 : 2; }

// ---------------------------------------------------------------------------------------------------
// 1. D_i = Σ_t dO_it O_it, stored negated.  One row per pre_tpr<D>() threads (a power of two), each
// summing D / (8·TPR) runs of 8 elements.
template <int D>
constexpr int pre_tpr() { return D == 96 ? 4 : D / 8; }

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                           const bf16* __restrict__ dO,
                                                           float* __restrict__ delta, long rows,
                                                           float mult) {
  constexpr int TPR = pre_tpr<D>();  // threads per row
  constexpr int RUNS = D / (8 * TPR);
  static_assert(RUNS * 8 * TPR == D && (TPR & (TPR - 1)) == 0, "row split");
  const long row = (long)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
#pragma unroll
    for (int u = 0; u < RUNS; ++u) {
      const u32x4 a = *(const u32x4*)(O + row * D + (part * RUNS + u) * 8);
      const u32x4 b = *(const u32x4*)(dO + row * D + (part * RUNS + u) * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_bits_to_float(a[i] & 0xffffu), bf16_bits_to_float(b[i] & 0xffffu), acc);
        acc = fmaf(bf16_bits_to_float(a[i] >> 16), bf16_bits_to_float(b[i] >> 16), acc);
      }
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && part == 0) delta[row] = -(acc * mult);
}

// ---------------------------------------------------------------------------------------------------
// 2. dK, dV.  OUT selects the outputs: 1 = dV, 2 = dK, 3 = both.  Head dimension 256 runs two passes
// (dV, then dK): with both, the dKᵀ and dVᵀ accumulators alone would take all of a wave's 512
// registers' worth of room it needs for the K fragments and the step's tiles; the dV pass needs
// neither V nor dP, and the extra cost is one more S product per step.
// Partial-result outputs of the split backward (bwd_split in fa_launch.h): fp32 [nseg][B·H][N][D]
// arrays of unscaled gradient sums, one per segment of the workgroup's loop.
struct BwdSplitOut {
  float* part_a;  // dK/dV kernel: dKᵀ sums; dQ kernel: dQᵀ sums
  float* part_b;  // dK/dV kernel: dVᵀ sums
  int seg;        // loop steps (dK/dV: 32-query steps; dQ: 64-key tiles) per segment
  int bh_count;   // B·H
};

template <int D, bool CAUSAL, int OUT, bool SPLIT>
__global__ __launch_bounds__(kThreads, (D == 256 && OUT != 1) ? 1 : 2) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ LSE, const bf16* __restrict__ dO, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int nkt, float scale, float scale_log2,
    int remap, BwdSplitOut so) {
  static_assert(!SPLIT || OUT == 3, "the split backward runs the fused dK/dV kernel");
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int L = lds_cols<D>();
  constexpr bool WANT_DV = (OUT & 1) != 0;
  constexpr bool WANT_DK = (OUT & 2) != 0;
  // Q and dO tiles (tile_off<L> layout) and the tile's base-2 LSE and D values (first 32 of 64 used),
  // double-buffered; separate LDS objects so reads of one buffer never wait for the LDS-DMA copy
  // filling the other.
  __shared__ __attribute__((aligned(1024))) bf16 q0s[kBQ * L];
  __shared__ __attribute__((aligned(1024))) bf16 q1s[kBQ * L];
  __shared__ __attribute__((aligned(1024))) bf16 o0s[kBQ * L];
  __shared__ __attribute__((aligned(1024))) bf16 o1s[kBQ * L];
  __shared__ __attribute__((aligned(256))) float l0s[64];
  __shared__ __attribute__((aligned(256))) float l1s[64];
  __shared__ __attribute__((aligned(256))) float d0s[64];
  __shared__ __attribute__((aligned(256))) float d1s[64];
  __shared__ __attribute__((aligned(1024))) bf16 vts[WANT_DK ? kBKV * L : 8];  // the workgroup's V rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int g = lane >> 5;
  const int lc = lane & 31;

  uint32_t logical = remap ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  int sg = 0;  // segment of the query steps (split only): work items are segment-major
  if constexpr (SPLIT) {
    const uint32_t per_seg = (uint32_t)so.bh_count * (uint32_t)nkt;
    sg = (int)(logical / per_seg);
    logical %= per_seg;
  }
  int bh, kt;  // key blocks in order, heaviest first under the causal mask
  head_tile(logical, nkt, SPLIT ? so.bh_count : (int)(gridDim.x / nkt), remap,
            dkdv_per_cu<D, OUT>(), bh, kt);
  const int k0 = kt * kBKV;
  const int kw = k0 + 32 * wave;  // first key of this wave
  const int kj = kw + lc;         // this lane's key (column of the score tiles)

  const int qstart = CAUSAL ? k0 : 0;  // causal: only queries ≥ the tile's first key
  const int nsteps = (N - qstart + kBQ - 1) / kBQ;
  // Steps [s_beg, s_end) of this workgroup: all of them, or one segment of the split.
  const int s_beg = SPLIT ? sg * so.seg : 0;
  const int s_end = SPLIT ? min(nsteps, s_beg + so.seg) : nsteps;
  if (SPLIT && s_beg >= s_end) return;  // the key block's queries end before this segment

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto mq = make_rsrc(Q + head, head_bytes);
  const auto mdo = make_rsrc(dO + head, head_bytes);
  const auto rk = make_rsrc(K + head, head_bytes);
  const auto rlse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const auto rdel = make_rsrc(Delta + (size_t)bh * N, (uint32_t)N * 4u);
  const BfTileCopy<D, kBQ, kThreads> copy(tid);

  // Kᵀ operands (B operand of S = Q Kᵀ) in registers: column = this lane's key.  The Vᵀ operand of
  // dP = dO Vᵀ is read from the LDS copy of the workgroup's V rows each step (registers are the
  // scarce resource here: dKᵀ and dVᵀ accumulators take 128 of them).
  bf16x8 kf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, (uint32_t)(kj * D + 16 * s + 8 * g) * 2u));
  if constexpr (WANT_DK) {
    const BfTileCopy<D, kBKV, kThreads> copy_v(tid);
    copy_v(make_rsrc(V + head, head_bytes), k0, vts);
  }

  const FragOffsets<L> fo(lane);
  // Query tiles are walked from the last one down to qstart: every workgroup of a head starts on the
  // same tiles and they move through Q and dO together, so each tile is read from memory about once
  // and then served from L2 to the head's other key blocks (ascending, the key blocks would start at
  // their own diagonals and keep all of the head's Q and dO in use at once).
  auto step_q = [&](int step) { return qstart + (nsteps - 1 - step) * kBQ; };

  // Q, dO and D of query step `step` go to LDS by DMA; wave 0 also loads the step's LSE into a
  // register and stores it, times log2(e), to LDS just before the step's closing barrier, so the
  // probabilities below are one FMA and one exp2 each.
  float lse_next = 0.f;
  auto stage = [&](int step, bf16* qd, bf16* od, float* dd) {
    const int qb = step_q(step);
    copy(mq, qb, qd);
    copy(mdo, qb, od);
    if (wave == 0) lse_next = __uint_as_float(buf_load4(rlse, (uint32_t)(qb + lane) * 4u));
    if (wave == 1) vec64_to_lds(rdel, qb, dd, lane);
  };

  f32x16 dka[DB], dva[DB];  // dKᵀ, dVᵀ: rows = d (32b + 8(r/4) + 4g + r%4), column = key
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[b][r] = 0.f;
      dva[b][r] = 0.f;
    }

  stage(s_beg, q0s, o0s, d0s);
  wait_vmem_all();
  if (wave == 0) l0s[lane] = lse_next * kLog2e;
  __syncthreads();

  // One query tile; P (the parity of step − s_beg) is a compile-time constant so the buffers are
  // fixed objects.  On entry the tile is in buffer P; buffer P^1 is free and receives the next tile.
  auto step_fn = [&](auto parity, int step) {
    constexpr int P = decltype(parity)::value;
    const char* qs = (const char*)(P ? q1s : q0s);
    const char* dos = (const char*)(P ? o1s : o0s);
    const float* lse_s = P ? l1s : l0s;
    const float* del_s = P ? d1s : d0s;
    if (step + 1 < s_end) stage(step + 1, P ? q0s : q1s, P ? o0s : o1s, P ? d0s : d1s);
    const int qb = step_q(step);

    if (!(CAUSAL && kw > qb + kBQ - 1)) {  // every (query, key) pair masked for this wave: skip
      // S = Q Kᵀ and dP = dO Vᵀ for 32 queries × this wave's 32 keys.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      if constexpr (WANT_DK) {  // dP accumulates onto −D: element r holds query 8(r/4) + 4g + r%4
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 d4 = *(const f32x4*)&del_s[8 * r4 + 4 * g];
#pragma unroll
          for (int t = 0; t < 4; ++t) pacc[4 * r4 + t] = d4[t];
        }
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        sacc = mfma_32x32x16(row_frag<L>(qs, fo, 0, s), kf[s], sacc);
        if constexpr (WANT_DK)
          pacc = mfma_32x32x16(row_frag<L>(dos, fo, 0, s), row_frag<L>((const char*)vts, fo, wave, s),
                               pacc);
      }
      // Element r: query qb + 8(r/4) + 4g + (r%4), key kj.  Masked scores become -inf (P = 0) in a
      // wave-uniform branch taken only by diagonal and ragged tiles.
      if ((kw + 31 >= N) || (CAUSAL && kw + 31 > qb)) {
        // Masked: kj ≥ N, or (causal) kj > query qb + 4g + c, tested on the element's constant
        // offset c against one per-lane limit.
        const bool past_end = kj >= N;
        const int lim = kj - qb - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (past_end || (CAUSAL && 8 * (r >> 2) + (r & 3) < lim)) sacc[r] = -INFINITY;
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = *(const f32x4*)&lse_s[8 * r4 + 4 * g];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * r4 + t;
          const float p = exp2_fast(fmaf(sacc[r], scale_log2, -l4[t]));  // staged LSE is base 2
          sacc[r] = p;
          if constexpr (WANT_DK) pacc[r] = p * pacc[r];  // dS without the scale
        }
      }
      bf16x8 pb[2], dsb[2];  // k-step ks covers queries 16ks + 8(e/4) + 4g + (e%4)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[ks][e] = (__bf16)sacc[8 * ks + e];
          dsb[ks][e] = (__bf16)pacc[8 * ks + e];
        }
      // dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS: A operands are dOᵀ / Qᵀ rows (d) read transposed from LDS.
#pragma unroll
      for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if constexpr (WANT_DV) dva[b] = mfma_32x32x16(tr_frag<L>(dos, fo, ks, b), pb[ks], dva[b]);
          if constexpr (WANT_DK) dka[b] = mfma_32x32x16(tr_frag<L>(qs, fo, ks, b), dsb[ks], dka[b]);
        }
      }
    }
    wait_vmem_all();
    if (wave == 0 && step + 1 < s_end) (P ? l0s : l1s)[lane] = lse_next * kLog2e;
    __syncthreads();
  };

  for (int step = s_beg; step < s_end; step += 2) {
    step_fn(std::integral_constant<int, 0>{}, step);
    if (step + 1 < s_end) step_fn(std::integral_constant<int, 1>{}, step + 1);
  }

  if constexpr (SPLIT) {
    // The segment's unscaled dKᵀ and dVᵀ sums for this lane's key (d rows 32b + 8(r/4) + 4g + 0..3).
    if (kj < N) {
      const size_t row = ((size_t)sg * so.bh_count + bh) * N + kj;
      float* kr = so.part_a + row * D;
      float* vr = so.part_b + row * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          *(f32x4*)&kr[32 * b + 8 * r4 + 4 * g] = f32x4{dka[b][4 * r4], dka[b][4 * r4 + 1],
                                                        dka[b][4 * r4 + 2], dka[b][4 * r4 + 3]};
          *(f32x4*)&vr[32 * b + 8 * r4 + 4 * g] = f32x4{dva[b][4 * r4], dva[b][4 * r4 + 1],
                                                        dva[b][4 * r4 + 2], dva[b][4 * r4 + 3]};
        }
    }
    return;
  }

  // Epilogue: dK = scale · (dKᵀ)ᵀ, dV = (dVᵀ)ᵀ; this lane owns key kj, d rows 32b + 8(r/4) + 4g + (0..3).
  if (kj < N) {
    bf16* dkr = dK + head + (size_t)kj * D;
    bf16* dvr = dV + head + (size_t)kj * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        if constexpr (WANT_DK) {
          u32x2 wk;
          wk[0] = pack_bf16x2(dka[b][4 * r4 + 0] * scale, dka[b][4 * r4 + 1] * scale);
          wk[1] = pack_bf16x2(dka[b][4 * r4 + 2] * scale, dka[b][4 * r4 + 3] * scale);
          *(u32x2*)&dkr[32 * b + 8 * r4 + 4 * g] = wk;
        }
        if constexpr (WANT_DV) {
          u32x2 wv;
          wv[0] = pack_bf16x2(dva[b][4 * r4 + 0], dva[b][4 * r4 + 1]);
          wv[1] = pack_bf16x2(dva[b][4 * r4 + 2], dva[b][4 * r4 + 3]);
          *(u32x2*)&dvr[32 * b + 8 * r4 + 4 * g] = wv;
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------------
// 3. dQ.  WITH_D: the kernel also forms D_i = dO_i · O_i for its own queries (each lane holds its
// query's dO fragments already; O is read once in the same layout) and writes it for the dK/dV kernel,
// in place of the separate bwd_pre launch.  The sum takes bwd_pre's order exactly (runs of 8 products,
// then the same pairwise tree), so D, and every gradient, is bit for bit what bwd_pre gives: bwd_pre's
// thread t of a row sums d values 8t .. 8t + 7, here chunk (s, g) of lane (query, g), t = 2s + g, so its
// tree levels t ^ 2h are in-lane (s ^ h) and t ^ 1 is the other half-wave.  Head dimension 96 (runs of
// 24 values per bwd_pre thread, which straddle the half-waves) keeps the separate launch.
template <int D, bool CAUSAL, bool WITH_D, bool SPLIT>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : D == 256 ? 1 : 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ LSE, const bf16* __restrict__ dO, float* __restrict__ Delta,
    const bf16* __restrict__ O, bf16* __restrict__ dQ, int N, int nqt, float scale,
    float scale_log2, float delta_mult, int remap, BwdSplitOut so) {
  static_assert(!WITH_D || pre_tpr<D>() == D / 8, "D in the dQ kernel: runs of 8 values");
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int L = lds_cols<D>();
  // K and V tiles (tile_off<L> layout), double-buffered, as separate LDS objects (see the dK/dV
  // kernel).
  __shared__ __attribute__((aligned(1024))) bf16 k0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 k1s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v1s[kBC * L];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int g = lane >> 5;
  const int lc = lane & 31;

  uint32_t logical = remap ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  int sg = 0;  // key segment (split only): work items are segment-major
  if constexpr (SPLIT) {
    const uint32_t per_seg = (uint32_t)so.bh_count * (uint32_t)nqt;
    sg = (int)(logical / per_seg);
    logical %= per_seg;
  }
  int bh, qt;
  head_tile(logical, nqt, SPLIT ? so.bh_count : (int)(gridDim.x / nqt), remap, dq_per_cu<D>(),
            bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // heaviest tiles first
  const int q0 = qt * kBR;
  const int qw = q0 + 32 * wave;
  const int qi = qw + lc;  // this lane's query

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  // Key tiles [t_beg, t_end) of this workgroup: all of them, or one segment of the split.
  const int t_beg = SPLIT ? sg * so.seg : 0;
  const int t_end = SPLIT ? min(ntiles, t_beg + so.seg) : ntiles;
  if (SPLIT && t_beg >= t_end) return;  // the query tile's keys end before this segment

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto mk = make_rsrc(K + head, head_bytes);
  const auto mv = make_rsrc(V + head, head_bytes);
  const BfTileCopy<D, kBC, kThreads> copy(tid);

  // Qᵀ and dOᵀ operands (B operands): column = this lane's query, slots d = 16s + 8g + (0..7).
  bf16x8 qf[KSTEPS], df[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const uint32_t off = (uint32_t)(qi * D + 16 * s + 8 * g) * 2u;
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const auto rlse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const float lse2 = __uint_as_float(buf_load4(rlse, (uint32_t)qi * 4u)) * kLog2e;
  float dlt;
  if constexpr (WITH_D) {
    const auto ro = make_rsrc(O + head, head_bytes);
    float c[KSTEPS];  // chunk sums, then the tree's partial sums
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4 ov = buf_load16(ro, (uint32_t)(qi * D + 16 * s + 8 * g) * 2u);
      const u32x4 dv = __builtin_bit_cast(u32x4, df[s]);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_bits_to_float(ov[i] & 0xffffu), bf16_bits_to_float(dv[i] & 0xffffu), acc);
        acc = fmaf(bf16_bits_to_float(ov[i] >> 16), bf16_bits_to_float(dv[i] >> 16), acc);
      }
      c[s] = acc;
    }
#pragma unroll
    for (int h = KSTEPS / 2; h > 0; h >>= 1) {
      float nc[KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) nc[s] = c[s] + c[s ^ h];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) c[s] = nc[s];
    }
    dlt = halves_sum(c[0]) * delta_mult;
    if (g == 0 && qi < N && sg == 0) Delta[(size_t)bh * N + qi] = -dlt;
  } else {
    const auto rdel = make_rsrc(Delta + (size_t)bh * N, (uint32_t)N * 4u);
    dlt = -__uint_as_float(buf_load4(rdel, (uint32_t)qi * 4u));
  }

  const FragOffsets<L> fo(lane);

  f32x16 qacc[DB];  // dQᵀ: rows d = 32b + 8(r/4) + 4g + r%4, column = this lane's query
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) qacc[b][r] = 0.f;

  copy(mk, t_beg * kBC, k0s);
  copy(mv, t_beg * kBC, v0s);
  wait_vmem_all();
  __syncthreads();

  // One key tile; P is the parity of j − t_beg (compile-time), the tile is in buffers P, buffers P^1
  // are free.
  auto tile_fn = [&](auto parity, int j) {
    constexpr int P = decltype(parity)::value;
    if (j + 1 < t_end) {
      copy(mk, (j + 1) * kBC, P ? k0s : k1s);
      copy(mv, (j + 1) * kBC, P ? v0s : v1s);
    }
    const int kv0 = j * kBC;
    if constexpr (D == 64) {
      // d = 64: one 32-key block at a time (S, dP, dS and the block's two dQ k-steps), which halves
      // the score and dP accumulators: 120 registers instead of 156, four waves per SIMD instead of
      // three.  Bit-identical; measured on MI355X, non-causal 8 × 16 × 2048: 0.221 → 0.213 ms.  At
      // d = 96 and 128 the same order ran 0.6–1.5% slower (it leaves fewer independent products
      // beside each tile's vector work), so they keep the whole tile.
      if (!(CAUSAL && kv0 > qw + 31)) {
        const char* klds = (const char*)(P ? k1s : k0s);
        const char* vlds = (const char*)(P ? v1s : v0s);
        const bool masked = (kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > qw);
        const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 4 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16 sacc, pacc;  // element r is key kv0 + 32kb + 8(r/4) + 4g + r%4
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[r] = 0.f;
            pacc[r] = 0.f;
          }
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            sacc = mfma_32x32x16(row_frag<L>(klds, fo, kb, s), qf[s], sacc);
            pacc = mfma_32x32x16(row_frag<L>(vlds, fo, kb, s), df[s], pacc);
          }
          if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(sacc[r], scale_log2, -lse2));
            pacc[r] = p * (pacc[r] - dlt);  // dSᵀ without the scale
          }
          bf16x8 dsf[2];  // k-steps 2kb and 2kb + 1, as in the whole-tile order below
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) dsf[h][e] = (__bf16)pacc[8 * h + e];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < DB; ++b)
              qacc[b] = mfma_32x32x16(tr_frag<L>(klds, fo, 2 * kb + h, b), dsf[h], qacc[b]);
        }
      }
    } else {
      if (!(CAUSAL && kv0 > qw + 31)) {
        const char* klds = (const char*)(P ? k1s : k0s);
        const char* vlds = (const char*)(P ? v1s : v0s);
        f32x16 sacc[2], pacc[2];  // Sᵀ and dPᵀ: element (kb, r) is key kv0 + 32kb + 8(r/4) + 4g + r%4
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[kb][r] = 0.f;
            pacc[kb][r] = 0.f;
          }
        }
  #pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = mfma_32x32x16(row_frag<L>(klds, fo, kb, s), qf[s], sacc[kb]);
            pacc[kb] = mfma_32x32x16(row_frag<L>(vlds, fo, kb, s), df[s], pacc[kb]);
          }
        // Masked scores become -inf (P = 0) in a wave-uniform branch taken only by diagonal and
        // ragged tiles.
        if ((kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > qw)) {
          // Masked: key > N − 1 or (causal) key > qi, tested on the element's constant offset c.
          const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 4 * g;
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
        }
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(sacc[kb][r], scale_log2, -lse2));
            pacc[kb][r] = p * (pacc[kb][r] - dlt);  // dSᵀ without the scale
          }
        // dSᵀ operand for k-step ks (16 keys): registers 8(ks%2) .. +7 of key block ks/2, i.e. keys
        // 16ks + 8(e/4) + 4g + (e%4) — the order the transposed K reads below produce.
        bf16x8 dsf[4];
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
          for (int e = 0; e < 8; ++e) dsf[ks][e] = (__bf16)pacc[ks >> 1][8 * (ks & 1) + e];
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
          for (int b = 0; b < DB; ++b)
            qacc[b] = mfma_32x32x16(tr_frag<L>(klds, fo, ks, b), dsf[ks], qacc[b]);
      }
    }
    wait_vmem_all();
    __syncthreads();
  };

  for (int j = t_beg; j < t_end; j += 2) {
    tile_fn(std::integral_constant<int, 0>{}, j);
    if (j + 1 < t_end) tile_fn(std::integral_constant<int, 1>{}, j + 1);
  }

  if constexpr (SPLIT) {
    // The segment's unscaled dQᵀ sums for this lane's query (d rows 32b + 8(r/4) + 4g + 0..3).
    if (qi < N) {
      float* qr = so.part_a + (((size_t)sg * so.bh_count + bh) * N + qi) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)&qr[32 * b + 8 * r4 + 4 * g] = f32x4{qacc[b][4 * r4], qacc[b][4 * r4 + 1],
                                                        qacc[b][4 * r4 + 2], qacc[b][4 * r4 + 3]};
    }
    return;
  }

  if (qi < N) {
    bf16* qrow = dQ + head + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(qacc[b][4 * r4 + 0] * scale, qacc[b][4 * r4 + 1] * scale);
        w[1] = pack_bf16x2(qacc[b][4 * r4 + 2] * scale, qacc[b][4 * r4 + 3] * scale);
        *(u32x2*)&qrow[32 * b + 8 * r4 + 4 * g] = w;
      }
  }
}

template <int D>
hipError_t launch_pre(const BwdArgs& a, hipStream_t stream) {
  const long rows = (long)a.B * a.H * a.N;
  constexpr int rows_per_block = kThreads / pre_tpr<D>();
  hipLaunchKernelGGL((bwd_pre_kernel<D>),
                     dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(kThreads), 0, stream, (const bf16*)a.o, (const bf16*)a.dout, a.delta, rows,
                     a.delta_mult);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int OUT>
hipError_t launch_dkdv_pass(const BwdArgs& a, hipStream_t stream) {
  const int nkt = (a.N + kBKV - 1) / kBKV;
  const uint32_t total = (uint32_t)a.B * a.H * nkt;
  const int remap = use_xcd_order(total, (long)a.B * a.H, CAUSAL ? 1 : 0);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, OUT, false>), dim3(total), dim3(kThreads), 0,
                     stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                     (const bf16*)a.dout, (const float*)a.delta, (bf16*)a.dk, (bf16*)a.dv, a.N, nkt,
                     a.dk_scale, a.scale * kLog2e, remap, BwdSplitOut{});
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
  if constexpr (D == 256) {  // two passes: dV, then dK
    const hipError_t e = launch_dkdv_pass<D, CAUSAL, 1>(a, stream);
    if (e != hipSuccess) return e;
    return launch_dkdv_pass<D, CAUSAL, 2>(a, stream);
  } else {
    return launch_dkdv_pass<D, CAUSAL, 3>(a, stream);
  }
}

template <int D, bool CAUSAL, bool WITH_D>
hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  const uint32_t total = (uint32_t)a.B * a.H * nqt;
  const int remap = use_xcd_order(total, (long)a.B * a.H, CAUSAL ? 1 : 0);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, WITH_D, false>), dim3(total), dim3(kThreads), 0,
                     stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                     (const bf16*)a.dout, a.delta, (const bf16*)a.o, (bf16*)a.dq, a.N, nqt,
                     a.dq_scale, a.scale * kLog2e, a.delta_mult, remap, BwdSplitOut{});
  return hipGetLastError();
}

// Split backward, last step: per row, the sum of its segments' partial dQ (segments of the row's query
// tile's key range) and partial dK, dV (segments of the row's key block's query range), scaled and
// rounded to bf16.  One thread per four consecutive values of a row.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_split_reduce_kernel(
    const float* __restrict__ part_dq, const float* __restrict__ part_dk,
    const float* __restrict__ part_dv, bf16* __restrict__ dQ, bf16* __restrict__ dK,
    bf16* __restrict__ dV, int N, int bh_count, int seg, float dq_scale, float dk_scale) {
  constexpr int C = D / 4;
  const size_t rows = (size_t)bh_count * N;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * C) return;
  const size_t row = idx / C;
  const size_t off = row * D + 4 * (idx % C);
  const size_t stride = rows * D;  // from one segment's array to the next
  const int i = (int)(row % (size_t)N);
  const int kv_end = CAUSAL ? min(N, (i / kBR + 1) * kBR) : N;
  const int nq = ((kv_end + kBC - 1) / kBC + seg - 1) / seg;
  const int qstart = CAUSAL ? (i / kBKV) * kBKV : 0;
  const int nk = ((N - qstart + kBQ - 1) / kBQ + 2 * seg - 1) / (2 * seg);
  f32x4 q = {0.f, 0.f, 0.f, 0.f}, k = q, v = q;
  for (int sg = 0; sg < nq; ++sg) q += *(const f32x4*)(part_dq + sg * stride + off);
  for (int sg = 0; sg < nk; ++sg) {
    k += *(const f32x4*)(part_dk + sg * stride + off);
    v += *(const f32x4*)(part_dv + sg * stride + off);
  }
  auto store4 = [](bf16* p, f32x4 x, float m) {
    u32x2 w;
    w[0] = pack_bf16x2(x[0] * m, x[1] * m);
    w[1] = pack_bf16x2(x[2] * m, x[3] * m);
    *(u32x2*)p = w;
  };
  store4(dQ + off, q, dq_scale);
  store4(dK + off, k, dk_scale);
  store4(dV + off, v, 1.f);
}

// The whole split backward: D and the dQ partial sums (one dQ launch, or bwd_pre first at d = 96),
// the dK/dV partial sums, then the reduction.  Work items are segment-major and dealt round-robin to
// the XCDs, as in the split forward.
template <int D, bool CAUSAL>
hipError_t launch_bwd_split(const BwdArgs& a, hipStream_t stream) {
  const BwdSplit sp = bwd_split(a.B, a.H, a.N, D, CAUSAL ? 1 : 0);
  const int bh = a.B * a.H;
  const int nqt = (a.N + kBR - 1) / kBR;
  const BwdSplitOut sq{a.part_dq, nullptr, sp.seg, bh};
  if constexpr (D == 96) {
    hipError_t e = launch_pre<96>(a, stream);
    if (e != hipSuccess) return e;
  }
  constexpr bool kWithD = D != 96;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, kWithD, true>),
                     dim3((uint32_t)sp.nseg_q * bh * nqt), dim3(kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                     (const bf16*)a.dout, a.delta, (const bf16*)a.o, (bf16*)a.dq, a.N, nqt,
                     a.dq_scale, a.scale * kLog2e, a.delta_mult, 0, sq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkt = (a.N + kBKV - 1) / kBKV;
  const BwdSplitOut sk{a.part_dk, a.part_dv, 2 * sp.seg, bh};
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, 3, true>), dim3((uint32_t)sp.nseg_k * bh * nkt),
                     dim3(kThreads), 0, stream, (const bf16*)a.q, (const bf16*)a.k,
                     (const bf16*)a.v, a.lse, (const bf16*)a.dout, (const float*)a.delta,
                     (bf16*)a.dk, (bf16*)a.dv, a.N, nkt, a.dk_scale, a.scale * kLog2e, 0, sk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t chunks = (size_t)bh * a.N * (D / 4);
  hipLaunchKernelGGL((bwd_split_reduce_kernel<D, CAUSAL>),
                     dim3((uint32_t)((chunks + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     (const float*)a.part_dq, (const float*)a.part_dk, (const float*)a.part_dv,
                     (bf16*)a.dq, (bf16*)a.dk, (bf16*)a.dv, a.N, bh, sp.seg, a.dq_scale,
                     a.dk_scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_with_d(const BwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_dq<D, true, true>(a, stream) : launch_dq<D, false, true>(a, stream);
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_pre<64>(a, stream);
  if (a.d == 96) return launch_pre<96>(a, stream);
  if (a.d == 256) return launch_pre<256>(a, stream);
  return launch_pre<128>(a, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64)
    return a.causal ? launch_dkdv<64, true>(a, stream) : launch_dkdv<64, false>(a, stream);
  if (a.d == 96)
    return a.causal ? launch_dkdv<96, true>(a, stream) : launch_dkdv<96, false>(a, stream);
  if (a.d == 256)
    return a.causal ? launch_dkdv<256, true>(a, stream) : launch_dkdv<256, false>(a, stream);
  return a.causal ? launch_dkdv<128, true>(a, stream) : launch_dkdv<128, false>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64)
    return a.causal ? launch_dq<64, true, false>(a, stream) : launch_dq<64, false, false>(a, stream);
  if (a.d == 96)
    return a.causal ? launch_dq<96, true, false>(a, stream) : launch_dq<96, false, false>(a, stream);
  if (a.d == 256)
    return a.causal ? launch_dq<256, true, false>(a, stream) : launch_dq<256, false, false>(a, stream);
  return a.causal ? launch_dq<128, true, false>(a, stream) : launch_dq<128, false, false>(a, stream);
}

hipError_t launch_bwd_delta_dq(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_dq_with_d<64>(a, stream);
  if (a.d == 128) return launch_dq_with_d<128>(a, stream);
  if (a.d == 256) return launch_dq_with_d<256>(a, stream);
  const hipError_t e = launch_bwd_pre(a, stream);
  return e == hipSuccess ? launch_bwd_dq(a, stream) : e;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.split_seg > 0) {  // bwd_split chose a split (head dimensions up to 128)
    if (a.d == 64)
      return a.causal ? launch_bwd_split<64, true>(a, stream) : launch_bwd_split<64, false>(a, stream);
    if (a.d == 96)
      return a.causal ? launch_bwd_split<96, true>(a, stream) : launch_bwd_split<96, false>(a, stream);
    if (a.d == 128)
      return a.causal ? launch_bwd_split<128, true>(a, stream)
                      : launch_bwd_split<128, false>(a, stream);
    return hipErrorInvalidValue;
  }
  const hipError_t e = launch_bwd_delta_dq(a, stream);
  return e == hipSuccess ? launch_bwd_dkdv(a, stream) : e;
}

}  // namespace fa
