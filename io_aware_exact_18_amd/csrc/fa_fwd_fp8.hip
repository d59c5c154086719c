// fa_fwd_fp8.hip — forward kernel with FP8 (OCP e4m3fn) matrix products for gfx950, head dims 64,
// 96, 128 and 256.
//
// Same method as the bf16 forward ("Anatomy of a FlashAttention Kernel", sections "Why is attention
// memory-bound ..." and "What is online softmax ..."), with the low-precision FP8 products that the
// section "What changed between FlashAttention 1, 2, and 3?" credits to FA3.  Q, K, V arrive as e4m3
// codes with one fp32 descale per tensor (value = code · descale).
//
//   * Sᵀ = K Qᵀ on v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulation; products of e4m3 values are exact).
//     The descales and scale·log2(e) fold into the one FMA that forms the exponent.
//   * P = 2^(s − m + 6) ∈ [0, 256] is rounded to e4m3 (v_cvt_pk_fp8_f32: round-to-nearest-even;
//     it does not saturate, but P stays far below 448) and Oᵀ += Vᵀ Pᵀ runs on the same fp8 matrix
//     core.  m is a reference maximum
//     that trails the running maximum by at most 2, so P ≤ 2^8; the factor 2^6 (free: it is part of
//     the FMA's constant) keeps small probabilities out of e4m3's subnormal range; both cancel in
//     O = Σ P V / Σ P and are removed from LSE.  The row sum l is formed by one more
//     matrix-core op on the Pᵀ operand, so it sums exactly the rounded P values that enter P·V (a
//     tile's sum of e4m3 values between 2^-9 and 2^8 is exact in fp32, in any order): a
//     v_mfma_f32_16x16x128_f8f6f4 against a selector operand (below), half the cycles of a
//     32×32×64 product against all ones and 4 accumulator registers instead of 16.  Measured on
//     MI355X against that form (bit-identical outputs), causal 4 × 32 × 8192: d = 64 0.845 →
//     0.801 ms, d = 96 1.115 → 1.065, d = 128 1.239 → 1.201.
//   * Key order: each wave loads K rows into the A operand with bits 2 and 3 of the row index swapped,
//     so that every lane's 32 probabilities form four runs of 8 consecutive keys; V is then read with
//     ds_read_b64_tr_b8, which hands each lane 8 consecutive key rows of one column, and the P bytes
//     go straight from the score accumulator into the B operand.
//   * Tiles: 4 waves × 32 queries per workgroup, 64-key K/V tiles copied into LDS by buffer→LDS DMA,
//     K one tile ahead of V, double-buffered, rows XOR-swizzled for conflict-free reads.
//   * Three waves per SIMD at d ≤ 128 (at most 168 registers; four at d = 64, 121 registers), two at
//     d = 256: one score tile is live at a time (the next tile's scores are formed after the
//     exponentials of the current one have read it), and the row sum takes 4 accumulator registers;
//     the Q operand stays in registers.  Measured on MI355X (bit-identical outputs, causal 4 × 32 ×
//     8192): one live score tile at three waves against two tiles at two waves, d = 128 1.345 →
//     1.274 ms, d = 96 1.212 → 1.148 (Q then read from LDS to make room); Q back in registers once
//     the row sum had freed 12 registers, d = 64 0.744 → 0.733, d = 128 1.144 → 1.119.
//   * Without the causal mask every wave takes every tile, and the compiler would drop the per-tile
//     `j < wave_tiles` test and schedule the two unrolled tiles as one block, at up to 168 registers
//     with spills; an opaque tile count keeps the test, and the non-causal kernels compile to the
//     causal ones' register counts (2 × 16 × 4096 non-causal, bit-identical: d = 64 0.137 → 0.132 ms,
//     d = 96 0.170 → 0.161, d = 128 0.186 → 0.180, d = 256 0.436 → 0.424).
//   * Head dims: Sᵀ takes D/64 k-steps of 64, Oᵀ D/32 column blocks of 32.  d = 96 uses the d = 128
//     LDS rows: the DMA fills bytes 96..127 of each K and V row with zeros and the Q operand's last
//     32 columns are zero, so the second k-step adds nothing, and only three V column blocks are read.
//   * d = 256: one workgroup per query tile holds the whole 32 × 256 Oᵀ accumulator per wave (245
//     registers, two waves per SIMD), which fits since the row sum and Q layout changes above.  Grids
//     of at most 256 query tiles, which leave half the compute units' slots empty, run two workgroups
//     per query tile instead (CS = 2), one per 128-column half of O: each forms the full Sᵀ and the
//     same P and accumulates only its half, 0.76× the matrix-core work of one pass on twice the work
//     items.  The halves are adjacent work items, so they share one XCD's L2 for K and V.  Measured on
//     MI355X (bit-identical outputs), one workgroup against two per query tile: causal 4 × 16 × 8192
//     1.798 → 1.117 ms, non-causal 2 × 16 × 4096 0.464 → 0.297 ms; causal 1 × 3 × 1000 (24 query
//     tiles) 0.033 → 0.039 ms, hence the rule.
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBR = 128;
constexpr int kBC = 64;
constexpr int kThreads = 256;
// Bytes per K/V row in LDS (one e4m3 byte per element; d = 96 is padded to 128).
template <int D>
constexpr int lds_row() { return D == 96 ? 128 : D; }
// Workgroups per query tile (column halves of O) at d = 256: two when the grid has at most this many
// query tiles, one otherwise (see the header).
constexpr uint32_t kColSplitMaxTiles = 256;
// P is formed as 2^(s·c − m + kPExp) against a per-row reference maximum m that is raised only when
// some row of the wave sees a score more than kSlack above it, so P ≤ 2^(kPExp + kSlack) = 256 fits
// e4m3 (largest finite 448) and the accumulators are rescaled on few tiles instead of most.
constexpr float kPExp = 6.f;
constexpr float kSlack = 2.f;

// Swizzle of 16-byte chunks within an fp8 row of LR bytes (64 banks of 4 bytes: one 256-byte row,
// two 128-byte rows or four 64-byte rows per bank period): keeps 16-lane row reads and 32-lane 8-byte
// transposed reads conflict-free.
template <int LR>
__device__ inline int swz8(int r) {
  if constexpr (LR == 64) return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  else if constexpr (LR == 256) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// Rows 32kb + i of the A operand hold K row 32kb + perm(i): bits 2 and 3 of i swapped.
__device__ inline int perm23(int i) { return (i & ~0xC) | ((i >> 1) & 4) | ((i << 1) & 8); }

__device__ inline f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline f32x4 mfma_f8_16(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ inline u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
  return __builtin_bit_cast(u32x2, r);
}

template <int D, bool CAUSAL, bool SPLIT, int CS>
__global__ __launch_bounds__(kThreads, D <= 128 ? 3 : 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float c_log2, float v_descale,
    int remap, SplitOut so) {
  static_assert(!SPLIT || D <= 128, "the key-range split runs d ≤ 128");
  static_assert(CS == 1 || (CS == 2 && D == 256), "column halves only at d = 256");
  static_assert(D == 64 || D == 96 || D == 128 || D == 256, "head dims of the fp8 forward");
  constexpr int LR = lds_row<D>();
  constexpr int KS = LR / 64;                   // k-steps of Sᵀ
  constexpr int DB = D / 32 / CS;  // column blocks of Oᵀ per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[kBC * LR];
  __shared__ __attribute__((aligned(1024))) uint8_t k1s[kBC * LR];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[kBC * LR];
  __shared__ __attribute__((aligned(1024))) uint8_t v1s[kBC * LR];

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
  const int half = CS == 2 ? (int)(logical & 1u) : 0;  // column half of O (d = 256)
  const uint32_t item = CS == 2 ? logical >> 1 : logical;
  int bh, qt;
  head_tile(item, nqt, SPLIT ? so.bh_count : (int)(gridDim.x / CS / nqt), remap,
            D <= 128 ? 3 : 2, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kBR;
  const int qw = q0 + 32 * wave;
  const int qi = qw + lc;

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  // Key tiles [t_beg, t_end) of this workgroup: all of them, or one segment of the split.
  const int t_beg = SPLIT ? sg * so.seg : 0;
  const int t_end = SPLIT ? min(ntiles, t_beg + so.seg) : ntiles;
  if (SPLIT && t_beg >= t_end) return;  // the query tile's keys end before this segment

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto mk = make_rsrc(K + head, head_bytes);
  const auto mv = make_rsrc(V + head, head_bytes);
  const TileCopy<LR, kBC, kThreads, D> copy(tid, [](int r) { return swz8<LR>(r); });

  // Qᵀ operand (B) in registers: this lane's query, k-step s covers d = 64s + 32g .. +31.  Columns
  // past D (d = 96: s = 1, g = 1) are read from an offset past the buffer's range (per-head bytes
  // stay below 2^31), which returns zeros rather than the next row's codes.
  i32x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint32_t off = (uint32_t)(qi * D + 64 * s + 32 * g);
    if constexpr (D == 96) {
      if (s == 1 && g == 1) off = 0x80000000u;
    }
    const u32x4 lo = buf_load16(rq, off), hi = buf_load16(rq, off + 16);
    qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // Per-lane LDS offsets.  K rows (A operand): row perm23(lc) (+32 per key block), chunks 4s+2g+h.
  uint32_t koff[KS][2];
  {
    const int r = perm23(lc);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        koff[s][h] = (uint32_t)(r * LR + 16 * ((4 * s + 2 * g + h) ^ swz8<LR>(r)));
  }
  // V transposed reads: the 16-lane group's lane i = 2a + b reads row k0 + a, bytes n0 + 8b .. +7
  // with k0 = 16c + 8g and n0 = 128·half + 32db + 16·((lane >> 4) & 1); the lane receives column
  // n0 + (i) of rows k0 .. k0 + 7.  voff[db] is the offset for c = 0 (c adds 16 rows).
  uint32_t voff[DB];
  {
    const int a = (lane & 15) >> 1, b = lane & 1, u = (lane >> 4) & 1;
    const int r = 8 * g + a;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[db] = (uint32_t)(r * LR + 16 * ((2 * (db + DB * half) + u) ^ swz8<LR>(r)) + 8 * b);
  }

  int wave_tiles = CAUSAL ? min(t_end, (qw + 31) / kBC + 1) : t_end;
  // Opaque without the mask, so that the per-tile test stays (see the header's non-causal note).
  if constexpr (!CAUSAL) asm volatile("" : "+s"(wave_tiles));

  copy(mk, t_beg * kBC, k0s);
  if (t_beg + 1 < t_end) copy(mk, (t_beg + 1) * kBC, k1s);
  copy(mv, t_beg * kBC, v0s);
  wait_vmem_all();
  __syncthreads();

  auto scores = [&](const uint8_t* klds, f32x16 (&acc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x8 qv = qf[s];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 lo = *(const u32x4*)(klds + koff[s][0] + kb * 32 * LR);
        const u32x4 hi = *(const u32x4*)(klds + koff[s][1] + kb * 32 * LR);
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        acc[kb] = mfma_f8(kf, qv, acc[kb]);
      }
    }
  };

  f32x16 sc[2];  // scores of the current tile
  scores(k0s, sc);
  __syncthreads();

  float m = -INFINITY;
  // Row-sum accumulator: register 0 of every lane holds Σ P of the lane's query (see above).
  f32x16 oacc[DB];
  f32x4 lacc;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) lacc[r] = 0.f;
  // 16×16×128 product: lane l of the A operand is row l % 16, k-group l / 16, and lane l of Pᵀ is
  // column l % 16, k-group l / 16, holding query l % 32 (k-groups 0 and 2 hold queries 0..15,
  // groups 1 and 3 queries 16..31).  Output row i lands in lanes 16(i / 4) + j, register i % 4.
  // Rows 0 and 8 select groups 0 and 2, rows 4 and 12 groups 1 and 3: register 0 of lane l is then
  // the sum of query l % 32.
  const int one = (lane & 3) == 0 && ((lane >> 2) & 1) == ((lane >> 4) & 1)
                      ? 0x38383838  // e4m3 1.0
                      : 0;
  const i32x8 sel = {one, one, one, one, one, one, one, one};

  auto tile = [&](auto parity, int j) {
    constexpr int P = decltype(parity)::value;
    f32x16(&s_cur)[2] = sc;  // scores of tile j, then of tile j + 1
    uint8_t* const k_this = P ? k1s : k0s;
    uint8_t* const k_next = P ? k0s : k1s;
    uint8_t* const v_this = P ? v1s : v0s;
    uint8_t* const v_next = P ? v0s : v1s;
    if (j + 2 < t_end) copy(mk, (j + 2) * kBC, k_this);
    if (j + 1 < t_end) copy(mv, (j + 1) * kBC, v_next);
    const int kv0 = j * kBC;
    if (j < wave_tiles) {
      // Accumulator element (kb, r), r = 4q + t, is key kv0 + 32kb + 16(q/2) + 8g + 4(q%2) + t.
      const bool need_mask = (kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > qw);
      if (need_mask) {
        // Masked: key > N − 1 or (causal) key > qi, tested on the element's constant offset.
        const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 8 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = r >> 2, t = r & 3;
            if (32 * kb + 16 * (q >> 1) + 4 * (q & 1) + t > lim) s_cur[kb][r] = -INFINITY;
          }
      }
      float mx = fmaxf(s_cur[0][0], s_cur[1][0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kb][r]);
      mx = halves_max(mx);
      const float mt = mx * c_log2;
      if (!wave_all(mt <= m + kSlack)) {  // raise the reference; a row without keys keeps -inf
        const float m_new = fmaxf(m, mt);
        const float alpha = exp2_fast(m - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) lacc[r] *= alpha;
        m = m_new;
      }
      const float m_off = (m == -INFINITY ? 0.f : m) - kPExp;  // P = 2^(s·c − m + kPExp)

      // Pᵀ operand (B): byte e of the 8 registers is P for accumulator element (e/16, e%16), i.e.
      // key 16(e/8) + 8g + (e%8) of the tile.
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = 4 * (w & 3);
        const float p0 = exp2_fast(fmaf(s_cur[kb][r0 + 0], c_log2, -m_off));
        const float p1 = exp2_fast(fmaf(s_cur[kb][r0 + 1], c_log2, -m_off));
        const float p2 = exp2_fast(fmaf(s_cur[kb][r0 + 2], c_log2, -m_off));
        const float p3 = exp2_fast(fmaf(s_cur[kb][r0 + 3], c_log2, -m_off));
        pf[w] = (int)pack_e4m3x4(p0, p1, p2, p3);
      }
      scores(k_next, s_cur);  // next tile's scores; discarded on the wave's last tile

      // Oᵀ += Vᵀ Pᵀ: A operand = V column 32db + lc, keys in the order of P's bytes.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8 vf;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x2 t8 = lds_read_tr8(v_this + voff[db] + c * 16 * LR);
          vf[2 * c] = (int)t8[0];
          vf[2 * c + 1] = (int)t8[1];
        }
        oacc[db] = mfma_f8(vf, pf, oacc[db]);
      }
      // Σ over the tile's keys of the rounded P, in register 0 of each lane
      lacc = mfma_f8_16(sel, pf, lacc);
    }
    wait_vmem_all();
    __syncthreads();
  };

  for (int j = t_beg; j < t_end; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < t_end) tile(std::integral_constant<int, 1>{}, j + 1);
  }

  if constexpr (SPLIT) {
    // The segment's partial result in the units of O (V's descale applied), its reference maximum
    // (the 2^kPExp offset of P removed) and the sum of the rounded P, which serves as both row sums.
    if (qi < N) {
      const size_t row = ((size_t)sg * so.bh_count + bh) * N + qi;
      float* orow = so.part_o + row * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 w = {oacc[b][4 * r4] * v_descale, oacc[b][4 * r4 + 1] * v_descale,
                           oacc[b][4 * r4 + 2] * v_descale, oacc[b][4 * r4 + 3] * v_descale};
          *(f32x4*)&orow[32 * b + 8 * r4 + 4 * g] = w;
        }
      if (g == 0) {
        so.part_ml[3 * row] = m - kPExp;
        so.part_ml[3 * row + 1] = lacc[0];
        so.part_ml[3 * row + 2] = lacc[0];
      }
    }
    return;
  }

  const float l = lacc[0];
  const float inv = v_descale / l;
  if (qi < N) {
    bf16* orow = O + head + (size_t)qi * D + 32 * DB * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[b][4 * r4 + 0] * inv, oacc[b][4 * r4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[b][4 * r4 + 2] * inv, oacc[b][4 * r4 + 3] * inv);
        *(u32x2*)&orow[32 * b + 8 * r4 + 4 * g] = w;
      }
    if (g == 0 && half == 0) LSE[(size_t)bh * N + qi] = (m - kPExp + __log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  const float c_log2 = a.scale * a.q_descale * a.k_descale * kLog2e;
  const uint32_t bh = (uint32_t)a.B * a.H;
  if constexpr (D <= 128) {
    // Key-range split (the bf16 forward's rule and merge; fwd_split in fa_launch.h).
    const FwdSplit sp = a.workspace ? fwd_split(a.B, a.H, a.N, D, CAUSAL ? 1 : 0) : FwdSplit{0, 1};
    if (sp.nseg > 1) {
      SplitOut so{(float*)a.workspace, nullptr, sp.seg, (int)bh};
      so.part_ml = so.part_o + (size_t)sp.nseg * bh * a.N * D;
      hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, true, 1>), dim3((uint32_t)sp.nseg * bh * nqt),
                         dim3(kThreads), 0, stream, (const uint8_t*)a.q8, (const uint8_t*)a.k8,
                         (const uint8_t*)a.v8, (bf16*)a.o, a.lse, a.N, nqt, c_log2, a.v_descale, 0,
                         so);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_fwd_merge(so.part_o, so.part_ml, a.o, a.lse, (int)bh, a.N, D, CAUSAL ? 1 : 0,
                              sp.seg, stream);
    }
  }
  const int cs = (D == 256 && bh * (uint32_t)nqt <= kColSplitMaxTiles) ? 2 : 1;
  const uint32_t total = bh * nqt * cs;
  const int remap = use_xcd_order(total, (long)bh, CAUSAL ? 1 : 0);
  if constexpr (D == 256) {
    if (cs == 2) {
      hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, false, 2>), dim3(total), dim3(kThreads), 0,
                         stream, (const uint8_t*)a.q8, (const uint8_t*)a.k8, (const uint8_t*)a.v8,
                         (bf16*)a.o, a.lse, a.N, nqt, c_log2, a.v_descale, remap,
                         SplitOut{nullptr, nullptr, 0, 0});
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, false, 1>), dim3(total), dim3(kThreads), 0, stream,
                     (const uint8_t*)a.q8, (const uint8_t*)a.k8, (const uint8_t*)a.v8, (bf16*)a.o,
                     a.lse, a.N, nqt, c_log2, a.v_descale, remap, SplitOut{nullptr, nullptr, 0, 0});
  return hipGetLastError();
}

}  // namespace

template <int D>
hipError_t launch_d(const Fp8FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch<D, true>(a, stream) : launch<D, false>(a, stream);
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_d<64>(a, stream);
    case 96: return launch_d<96>(a, stream);
    case 128: return launch_d<128>(a, stream);
    case 256: return launch_d<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
