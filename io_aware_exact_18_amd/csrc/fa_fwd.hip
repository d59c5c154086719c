// fa_fwd.hip — bf16 forward kernel for gfx950.
//
// Computes O = softmax(scale · Q Kᵀ) V and the per-row logsumexp for one 128-query tile per workgroup
// ("Anatomy of a FlashAttention Kernel", sections "Why is attention memory-bound ..." and "What is
// online softmax and how does tiling keep it exact?"; "FlashAttention: where it matters", section
// "The Real Complexity", second bullet: B_r × B_c tiles kept on chip, only O written back).
//
// Work split (gfx950, wave64):
//   * 4 waves per workgroup, 32 queries per wave: B_r = 128.  Key/value tiles of B_c = 64 rows are
//     copied straight from memory into LDS (buffer_load ... lds, XOR-swizzled rows) and shared by the
//     4 waves; one barrier per tile.
//   * Each wave computes the transposed score tile Sᵀ = K Qᵀ on the 32×32×16 bf16 matrix core, so
//     every lane owns one query column: the row maximum and row sum of the softmax are in-lane
//     reductions plus one exchange between the two half-waves (v_permlane32_swap).
//   * The probabilities leave the accumulator as bf16 and feed Oᵀ += Vᵀ Pᵀ directly as the B
//     operand; V is read from its row-major LDS tile with ds_read_b64_tr_b16, whose key order matches
//     the accumulator's row order, so P never goes through LDS.
//   * Software pipeline: K tiles are staged one tile ahead of V tiles and each tile runs in two
//     phases that pair matrix-core and vector work of different tiles: (A) the scores of tile j + 1
//     with the exponentials of tile j, (B) Oᵀ += Vᵀ Pᵀ of tile j with the row sum of tile j and the
//     row maximum of tile j + 1 (the overlap of matrix products with the softmax that "Anatomy ...",
//     section "What changed between FlashAttention 1, 2, and 3?", credits for FA3's speed, done here
//     within one wave).
//   * The exponentials use a reference maximum that moves only when a row's maximum exceeds it by
//     more than 2^8 (kSlack), so the accumulator rescale of the online softmax runs on few tiles.
//   * The softmax runs in base 2 with scale·log2(e) folded into one FMA; normalisation by the row sum
//     is deferred to the end (fewer non-matmul operations, same section).  LSE is converted back to
//     natural log on output.
//   * Two row sums are kept: l over the fp32 probabilities, for LSE, and lr over the same values
//     rounded to bf16 — the weights the P·V product actually applies — which O is divided by.  O is
//     then an exactly normalised average of V rows under the rounded weights: in a row dominated by
//     one key it returns that key's V row however p rounds, where dividing by l would leave p's
//     rounding error (up to 2^-9 of |V|) in O.  lr is formed on the matrix core (a 16×16×32
//     product against a selector operand, in the kernel below).
//   * Grid: one workgroup per (batch·head, query tile); the query tiles of a group of four heads are
//     kept on one XCD so the heads' K/V stay in that XCD's L2, interleaved head by head so that under
//     the causal mask every group's heaviest tiles start first (head_tile in fa_common.h).
//   * Head dimension 256 runs fwd_bf16_split_kernel instead: 8 waves per workgroup, each key tile
//     split between two waves holding the same queries, merged at the end (see that kernel).
//   * Key-range split (fa_fwd_split, for grids too small to fill the device; rule in fa_launch.h):
//     the SPLIT instantiation runs the same loop over one segment of a query tile's key tiles and
//     writes the segment's unnormalised O, reference maximum and both row sums; fwd_merge_kernel
//     combines a row's segments (merge_partials in fa_common.h).
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBR = 128;   // queries per workgroup
constexpr int kBC = 64;    // keys per tile
constexpr int kThreads = 256;
// The exponentials use a per-row reference maximum that is raised only when some row of the wave
// sees a score more than kSlack (base-2 units) above its reference; until then p ≤ 2^kSlack, which
// bf16 P and the fp32 sums hold exactly as well as p ≤ 1.  Output and row sum share the reference,
// so the result is the same softmax; the rescale of the accumulators becomes rare instead of
// happening on most tiles (with 32 rows per wave, some row's running maximum rises on most tiles).
constexpr float kSlack = 8.f;

// Compile-time selection between two objects (the score tiles of the two tile parities).
template <int P, class T>
__device__ inline T& pick(T& a, T& b) {
  if constexpr (P != 0) return b;
  else return a;
}


// Sᵀ = K Qᵀ for one 64-key tile: acc[kb] element r is key 32kb + 8(r/4) + 4g + (r%4) of the tile,
// query = this lane's query.  The two key blocks' chains are interleaved and each K fragment is read
// two products ahead of its use.
template <int D>
__device__ inline void scores_tile(const char* klds, const FragOffsets<lds_cols<D>()>& fo,
                                   const bf16x8 (&qf)[D / 16], f32x16 (&acc)[2]) {
  constexpr int NS = D / 16;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
  bf16x8 f[2 * NS];
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) f[i] = row_frag<lds_cols<D>()>(klds, fo, i & 1, i >> 1);
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) acc[i & 1] = mfma_32x32x16(f[i], qf[i >> 1], acc[i & 1]);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2, int remap,
    SplitOut so) {
  static_assert(D <= 128, "head dimension 256 runs fwd_bf16_split_kernel");
  constexpr int KSTEPS = D / 16;  // k-steps of the Sᵀ product
  constexpr int DB = D / 32;      // 32-row blocks of Oᵀ
  constexpr int L = lds_cols<D>();
  // K(j) lives in k<j % 2>, V(j) in v<j % 2> (tile_off<L> layout).  Four separate LDS objects, so the
  // compiler can tell the buffer being read from the one an in-flight LDS-DMA copy is writing and
  // does not wait for the copy before unrelated reads.
  __shared__ __attribute__((aligned(1024))) bf16 k0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 k1s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v1s[kBC * L];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int g = lane >> 5;   // half-wave: selects k-slots 8g..8g+7
  const int lc = lane & 31;  // row / column index inside a 32-wide matrix-core tile

  const uint32_t total = gridDim.x;
  uint32_t logical = remap ? xcd_remap(blockIdx.x, total) : blockIdx.x;
  int sg = 0;  // key segment (split only): work items are segment-major
  if constexpr (SPLIT) {
    const uint32_t per_seg = (uint32_t)so.bh_count * (uint32_t)nqt;
    sg = (int)(logical / per_seg);
    logical %= per_seg;
  }
  int bh, qt;  // tile order: heaviest first under the causal mask
  head_tile(logical, nqt, SPLIT ? so.bh_count : (int)(total / nqt), remap, D == 64 ? 3 : 2, bh,
            qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kBR;
  const int qw = q0 + wave * 32;  // first query of this wave
  const int qi = qw + lc;         // this lane's query

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  // Key tiles [t_beg, t_end) of this workgroup: all of them, or one segment of the split.
  const int t_beg = SPLIT ? sg * so.seg : 0;
  const int t_end = SPLIT ? min(ntiles, t_beg + so.seg) : ntiles;
  if (SPLIT && t_beg >= t_end) return;  // the query tile's keys end before this segment

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto mk = make_rsrc(K + head, head_bytes);
  const auto mv = make_rsrc(V + head, head_bytes);
  const BfTileCopy<D, kBC, kThreads> copy(tid);

  // Qᵀ fragments (B operand): column = this lane's query, slots = d in [16s + 8g, 16s + 8g + 8).
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qi * D + 16 * s + 8 * g) * 2u));

  // Tiles at or beyond this index are fully masked for this wave (causal): no math on them.
  int wave_tiles = CAUSAL ? min(t_end, (qw + 31) / kBC + 1) : t_end;
  // Without the mask every wave takes every tile, and the compiler would drop the `j < wave_tiles`
  // test below and schedule the two unrolled tiles as one block: that needed 177 registers at
  // d = 64 (a wave per SIMD fewer) and spilled at d = 128.  An opaque count keeps the test, and the
  // non-causal instantiations compile to the causal ones' register counts.
  if constexpr (!CAUSAL) asm volatile("" : "+s"(wave_tiles));
  const FragOffsets<L> fo(lane);

  // Prologue: K(t_beg), K(t_beg + 1), V(t_beg) in flight; scores of tile t_beg.
  copy(mk, t_beg * kBC, k0s);
  if (t_beg + 1 < t_end) copy(mk, (t_beg + 1) * kBC, k1s);
  copy(mv, t_beg * kBC, v0s);
  wait_vmem_all();
  __syncthreads();

  // Score tiles of the even and odd tiles: tile j's scores are in sa when j is even, sb when odd.
  f32x16 sa[2], sb[2];
  // Row maximum of a score tile (raw scores; both half-waves get the same value).
  auto rowmax = [](const f32x16(&s)[2]) {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return halves_max(mx);
  };
  scores_tile<D>((const char*)k0s, fo, qf, sa);
  float mx = rowmax(sa);  // row maximum of the current tile's (unmasked) scores
  __syncthreads();  // every wave is done with k[0] before K(2) overwrites it

  float m = -INFINITY;  // reference maximum of the base-2 scaled scores (see kSlack)
  float l = 0.f;        // running sum of 2^(t - m) over this lane's keys (half of the row)
  // lr, the same sum over the bf16-rounded values that enter P·V, is taken on the matrix core: a
  // 16×16×32 product of the Pᵀ operand against a selector operand (the FP8 forward's row-sum scheme:
  // A-operand lane l is row l % 16 of k-group l / 16, Pᵀ lane l is column l % 16 of k-group l / 16
  // and holds query l % 32; rows 0 and 8 select k-groups 0 and 2, rows 4 and 12 groups 1 and 3), so
  // register 0 of every lane holds its query's sum over both key halves.  Four products per tile replace 16 dot2 instructions and the final exchange
  // between the half-waves.  Measured on MI355X in one process (O within one bf16 ulp, LSE
  // bit-identical), causal 4 × 32 × 4096: d = 128 0.558 → 0.538 ms, d = 96 0.469 → 0.452, d = 64
  // (8 × 16 × 2048) 0.116 → 0.111; non-causal: d = 128 1.085 → 1.043, d = 96 0.889 → 0.864, d = 64
  // (8 × 16 × 2048) 0.191 → 0.182.
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // lr: register 0
  const __bf16 one = ((lane & 3) == 0 && ((lane >> 2) & 1) == ((lane >> 4) & 1)) ? (__bf16)1.0f
                                                                                   : (__bf16)0.0f;
  const bf16x8 sel = {one, one, one, one, one, one, one, one};
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;

  // One tile; P is the parity of j − t_beg, a compile-time constant so every LDS address below is a
  // lane base plus an immediate.  Buffers on entry: k[P^1] = K(j+1), v[P] = V(j); k[P], v[P^1] are free.
  auto tile = [&](auto parity, int j) {
    constexpr int P = decltype(parity)::value;
    f32x16(&s_cur)[2] = pick<P>(sa, sb);  // scores of tile j
    f32x16(&s_nxt)[2] = pick<P>(sb, sa);  // receives the scores of tile j + 1
    bf16* const k_this = P ? k1s : k0s;   // free: receives K(j+2)
    bf16* const k_next = P ? k0s : k1s;   // holds K(j+1)
    bf16* const v_this = P ? v1s : v0s;   // holds V(j)
    bf16* const v_next = P ? v0s : v1s;   // free: receives V(j+1)
    if (j + 2 < t_end) copy(mk, (j + 2) * kBC, k_this);
    if (j + 1 < t_end) copy(mv, (j + 1) * kBC, v_next);
    const int kv0 = j * kBC;
    if (j < wave_tiles) {
      // Accumulator element (kb, r) is key kv0 + 32kb + 8(r/4) + 4g + (r%4) for query qi.  Diagonal
      // and ragged tiles are masked here and their maximum is taken again.
      if ((kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > qw)) {
        // Masked: key > N − 1 or (causal) key > qi, tested on the element's constant offset c.
        const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 4 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s_cur[kb][r] = -INFINITY;
        mx = rowmax(s_cur);
      }
      const float mt = mx * scale_log2;
      // Raise the reference (and rescale) only when some row's tile maximum exceeds it by more than
      // kSlack; a row still without any unmasked key keeps m = -inf.
      if (!wave_all(mt <= m + kSlack)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = exp2_fast(m - (m_new == -INFINITY ? 0.f : m_new));
        l *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) lacc[r] *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        m = m_new;
      }
      const float m_use = (m == -INFINITY) ? 0.f : m;

      // Two branch-free phases, each pairing matrix-core work with independent vector work so that
      // one wave keeps both units busy (the group barriers set the interleave).
      // Phase A: scores of tile j + 1 (on a wave's last tile they read a stale buffer and are
      // discarded) with the probabilities of tile j, kept in place in s_cur and as the bf16 Pᵀ
      // operand: k-step ks (16 keys) takes registers 8(ks%2) .. +7 of key block ks/2, i.e. keys
      // 16ks + 8(e/4) + 4g + (e%4) — the order the transposed V reads below produce.
      // Phase A runs at raised wave priority: when both waves of a SIMD can issue, the one in its
      // score/exponential phase goes first (measured 2% faster than equal priorities).
      __builtin_amdgcn_s_setprio(1);
      scores_tile<D>((const char*)k_next, fo, qf, s_nxt);
      bf16x8 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_fast(fmaf(s_cur[ks >> 1][8 * (ks & 1) + e], scale_log2, -m_use));
          s_cur[ks >> 1][8 * (ks & 1) + e] = p;
          pf[ks][e] = (__bf16)p;
        }
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix-core op
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three vector ALU ops
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // Phase B: Oᵀ += Vᵀ Pᵀ with the row sum of tile j and the row maximum of tile j + 1.
      const char* vlds = (const char*)v_this;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 vf[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) vf[b] = tr_frag<L>(vlds, fo, ks, b);
#pragma unroll
        for (int b = 0; b < DB; ++b) oacc[b] = mfma_32x32x16(vf[b], pf[ks], oacc[b]);
      }
      float rs[4] = {s_cur[0][0], s_cur[0][1], s_cur[0][2], s_cur[0][3]};  // four partial sums
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) rs[r & 3] += s_cur[kb][r];
      l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[ks], lacc, 0, 0, 0);
      mx = rowmax(s_nxt);
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }
    wait_vmem_all();
    __syncthreads();
  };

  for (int j = t_beg; j < t_end; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < t_end) tile(std::integral_constant<int, 1>{}, j + 1);
  }

  if constexpr (SPLIT) {
    // The segment's partial result: unnormalised Oᵀ column, reference maximum and both row sums (a
    // wave without keys in the segment writes m = −inf and zeros, which the merge weighs by 0).
    const float l_seg = halves_sum(l);
    const float lr_seg = lacc[0];
    if (qi < N) {
      const size_t row = ((size_t)sg * so.bh_count + bh) * N + qi;
      float* orow = so.part_o + row * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 w = {oacc[b][4 * r4], oacc[b][4 * r4 + 1], oacc[b][4 * r4 + 2],
                           oacc[b][4 * r4 + 3]};
          *(f32x4*)&orow[32 * b + 8 * r4 + 4 * g] = w;
        }
      if (g == 0) {
        so.part_ml[3 * row] = m;
        so.part_ml[3 * row + 1] = l_seg;
        so.part_ml[3 * row + 2] = lr_seg;
      }
    }
    return;
  }

  // Epilogue: combine the two half-row sums, normalise by the rounded weights' sum, write O and LSE.
  const float l_tot = halves_sum(l);
  const float inv = 1.f / lacc[0];
  if (qi < N) {
    bf16* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[b][4 * r4 + 0] * inv, oacc[b][4 * r4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[b][4 * r4 + 2] * inv, oacc[b][4 * r4 + 3] * inv);
        *(u32x2*)&orow[32 * b + 8 * r4 + 4 * g] = w;
      }
    if (g == 0) LSE[(size_t)bh * N + qi] = (m + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------------------
// Head dimension 256: a wave's Oᵀ accumulator (32 queries × 256) and Qᵀ fragments leave no room for
// the scores of 64 keys at two waves per SIMD, so each 64-key tile is split between two waves that
// hold the same 32 queries: wave w (key half 0) and wave w + 4 (key half 1) each take one 32-key block
// of every tile, keep their own reference maximum m, partial row sum l and Oᵀ, and are merged at the
// end by softmax mass (O = (2^(m0−m) O0 + 2^(m1−m) O1) / (2^(m0−m) l0 + 2^(m1−m) l1), m = max(m0, m1):
// the online-softmax recurrence of "Anatomy ...", section "What is online softmax and how does tiling
// keep it exact?", applied to the two key subsets).  8 waves per workgroup, 128 queries, one
// workgroup per CU: two waves per SIMD, each with a D = 128 wave's amount of work per tile.
constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = 64 * kSplitWaves;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads, 1) void fwd_bf16_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2, int remap) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int L = lds_cols<D>();
  // K(j), V(j) live in k<j % 2>, v<j % 2>; after the key loop the four buffers carry the key-half-1
  // waves' partial outputs to their partners (one 32 KiB buffer per query block).
  __shared__ __attribute__((aligned(1024))) bf16 k0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 k1s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v0s[kBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v1s[kBC * L];
  __shared__ __attribute__((aligned(256))) float xml[4][3][64];  // key half 1: (m, l, lr) per lane
  static_assert(DB * 16 * 64 * 4 == kBC * L * 2, "one wave's Oᵀ fills one staging buffer");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index(tid);
  const int qblk = wave & 3;  // query block of the wave
  const int kh = wave >> 2;   // key half: keys 32kh .. 32kh + 31 of every tile
  const int g = lane >> 5;
  const int lc = lane & 31;

  const uint32_t total = gridDim.x;
  const uint32_t logical = remap ? xcd_remap(blockIdx.x, total) : blockIdx.x;
  int bh, qt;
  head_tile(logical, nqt, (int)(total / nqt), remap, 1, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kBR;
  const int qw = q0 + qblk * 32;
  const int qi = qw + lc;

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto mk = make_rsrc(K + head, head_bytes);
  const auto mv = make_rsrc(V + head, head_bytes);
  const BfTileCopy<D, kBC, kSplitThreads> copy(tid);

  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qi * D + 16 * s + 8 * g) * 2u));

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  const FragOffsets<L> fo(lane);

  copy(mk, 0, k0s);
  copy(mv, 0, v0s);
  wait_vmem_all();
  __syncthreads();

  float m = -INFINITY;  // reference maximum of the base-2 scaled scores (slack rule as above)
  float l = 0.f;        // partial row sum over this lane's keys of this key half
  float lr = 0.f;       // the same over the bf16-rounded values that enter P·V (O is divided by it)
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;

  auto tile = [&](auto parity, int j) {
    constexpr int P = decltype(parity)::value;
    if (j + 1 < ntiles) {
      copy(mk, (j + 1) * kBC, P ? k0s : k1s);
      copy(mv, (j + 1) * kBC, P ? v0s : v1s);
    }
    const char* klds = (const char*)(P ? k1s : k0s);
    const char* vlds = (const char*)(P ? v1s : v0s);
    const int kb0 = j * kBC + 32 * kh;  // first key of this wave's block
    if (!(CAUSAL && kb0 > qw + 31) && kb0 < N) {
      // Sᵀ for the block: element r is key kb0 + 8(r/4) + 4g + (r%4) for query qi.
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) sacc = mfma_32x32x16(row_frag<L>(klds, fo, kh, s), qf[s], sacc);
      if ((kb0 + 32 > N) || (CAUSAL && kb0 + 31 > qw)) {
        // Masked: key > N − 1 or (causal) key > qi, tested on the element's constant offset.
        const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kb0 - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) sacc[r] = -INFINITY;
      }
      float mx = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      const float mt = halves_max(mx) * scale_log2;
      if (!wave_all(mt <= m + kSlack)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = exp2_fast(m - (m_new == -INFINITY ? 0.f : m_new));
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        m = m_new;
      }
      const float m_use = (m == -INFINITY) ? 0.f : m;
      // Pᵀ operand: k-step ks (16 keys) takes registers 8ks .. 8ks + 7, keys 16ks + 8(e/4) + 4g +
      // (e%4) of the block — the order of the transposed V reads of rows 32kh + 16ks + ...
      bf16x8 pf[2];
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_fast(fmaf(sacc[8 * ks + e], scale_log2, -m_use));
          rs[e & 3] += p;
          pf[ks][e] = (__bf16)p;
        }
      l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      lr = sum_bf16x8(pf[1], sum_bf16x8(pf[0], lr));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < DB; ++b)
          oacc[b] = mfma_32x32x16(tr_frag<L>(vlds, fo, 2 * kh + ks, b), pf[ks], oacc[b]);
    }
    wait_vmem_all();
    __syncthreads();
  };

  for (int j = 0; j < ntiles; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1);
  }

  // Merge the key halves (every wave has passed the last barrier, so the K/V buffers are free).
  float* xo = (float*)(qblk == 0 ? k0s : qblk == 1 ? k1s : qblk == 2 ? v0s : v1s);
  if (kh == 1) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(b * 16 + r) * 64 + lane] = oacc[b][r];
    xml[qblk][0][lane] = m;
    xml[qblk][1][lane] = l;
    xml[qblk][2][lane] = lr;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = xml[qblk][0][lane];
    const float l1 = xml[qblk][1][lane];
    const float lr1 = xml[qblk][2][lane];
    // Key half 0 always holds key 0 of the row (causal) or a full block, so m is finite here for
    // every row with an unmasked key; half 1 may have seen none (m1 = −inf, l1 = 0).
    const float mm = fmaxf(m, m1);
    const float a0 = exp2_fast(m - mm);
    const float a1 = (m1 == -INFINITY) ? 0.f : exp2_fast(m1 - mm);
    const float l_tot = halves_sum(a0 * l + a1 * l1);
    const float inv = 1.f / halves_sum(a0 * lr + a1 * lr1);
    const float w0 = a0 * inv, w1 = a1 * inv;
    if (qi < N) {
      bf16* orow = O + head + (size_t)qi * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float o4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            o4[t] = oacc[b][4 * r4 + t] * w0 + xo[(b * 16 + 4 * r4 + t) * 64 + lane] * w1;
          u32x2 w;
          w[0] = pack_bf16x2(o4[0], o4[1]);
          w[1] = pack_bf16x2(o4[2], o4[3]);
          *(u32x2*)&orow[32 * b + 8 * r4 + 4 * g] = w;
        }
      if (g == 0) LSE[(size_t)bh * N + qi] = (mm + __log2f(l_tot)) * kLn2;
    }
  }
}

template <bool CAUSAL>
hipError_t launch_split(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  const uint32_t total = (uint32_t)a.B * a.H * nqt;
  const int remap = use_xcd_order(total, (long)a.B * a.H, CAUSAL ? 1 : 0);
  hipLaunchKernelGGL((fwd_bf16_split_kernel<256, CAUSAL>), dim3(total), dim3(kSplitThreads), 0,
                     stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                     a.N, nqt, a.scale * kLog2e, remap);
  return hipGetLastError();
}

// Key-range split: one wave per (batch·head, query) combines the row's segments (as many as its
// query tile's key range spans).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_merge_kernel(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml,
                                                       bf16* __restrict__ O, float* __restrict__ LSE,
                                                       int N, int bh_count, int seg) {
  const size_t r = blockIdx.x;  // output row (batch·head, query)
  const int bh = (int)(r / (size_t)N);
  const int qi = (int)(r % (size_t)N);
  const int kv_end = CAUSAL ? min(N, (qi / kBR + 1) * kBR) : N;
  const int nseg = ((kv_end + kBC - 1) / kBC + seg - 1) / seg;
  merge_partials<D>(part_o, part_ml, (size_t)bh * N + qi, (size_t)bh_count * N, nseg, O + r * D,
                    LSE + r, threadIdx.x);
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  const float scale_log2 = a.scale * kLog2e;
  const uint32_t bh = (uint32_t)a.B * a.H;
  const FwdSplit sp = a.workspace ? fwd_split(a.B, a.H, a.N, D, CAUSAL ? 1 : 0) : FwdSplit{0, 1};
  if (sp.nseg > 1) {
    // Segment-major work items dealt round-robin to the XCDs (remap off): segments of one key range
    // cost about the same, and the round-robin spreads the empty items (segments past a query tile's
    // keys, which return at once) evenly.
    SplitOut so{(float*)a.workspace, nullptr, sp.seg, (int)bh};
    so.part_ml = so.part_o + (size_t)sp.nseg * bh * a.N * D;
    const uint32_t total = (uint32_t)sp.nseg * bh * nqt;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true>), dim3(total), dim3(kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.N,
                       nqt, scale_log2, 0, so);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_fwd_merge(so.part_o, so.part_ml, a.o, a.lse, (int)bh, a.N, D, CAUSAL ? 1 : 0,
                            sp.seg, stream);
  }
  const uint32_t total = bh * nqt;
  const int remap = use_xcd_order(total, (long)bh, CAUSAL ? 1 : 0);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false>), dim3(total), dim3(kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.N,
                     nqt, scale_log2, remap, SplitOut{nullptr, nullptr, 0, 0});
  return hipGetLastError();
}

}  // namespace

namespace {
template <int D, bool CAUSAL>
hipError_t merge_rows(const float* part_o, const float* part_ml, void* o, float* lse, int bh, int N,
                      int seg, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_merge_kernel<D, CAUSAL>), dim3((uint32_t)bh * (uint32_t)N), dim3(64), 0,
                     stream, part_o, part_ml, (bf16*)o, lse, N, bh, seg);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_merge(const float* part_o, const float* part_ml, void* o, float* lse, int bh,
                            int N, int d, int causal, int seg, hipStream_t stream) {
  if (d == 64)
    return causal ? merge_rows<64, true>(part_o, part_ml, o, lse, bh, N, seg, stream)
                  : merge_rows<64, false>(part_o, part_ml, o, lse, bh, N, seg, stream);
  if (d == 96)
    return causal ? merge_rows<96, true>(part_o, part_ml, o, lse, bh, N, seg, stream)
                  : merge_rows<96, false>(part_o, part_ml, o, lse, bh, N, seg, stream);
  if (d == 128)
    return causal ? merge_rows<128, true>(part_o, part_ml, o, lse, bh, N, seg, stream)
                  : merge_rows<128, false>(part_o, part_ml, o, lse, bh, N, seg, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  if (a.d == 96) return a.causal ? launch<96, true>(a, stream) : launch<96, false>(a, stream);
  if (a.d == 256) return a.causal ? launch_split<true>(a, stream) : launch_split<false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
