// fa_fwd.hip — bf16 forward kernel for gfx950.
//
// Computes O = softmax(scale · Q Kᵀ) V and the per-row logsumexp for one 128-query tile per workgroup
// ("Anatomy of a FlashAttention Kernel", sections "Why is attention memory-bound ..." and "What is
// online softmax and how does tiling keep it exact?"; "FlashAttention: where it matters", section
// "The Real Complexity", second bullet: B_r × B_c tiles kept on chip, only O written back).
//
// Work split (gfx950, wave64):
//   * 4 waves per workgroup, 32 queries per wave: B_r = 128.  Key/value tiles of B_c = 64 rows are
//     copied straight from memory into LDS (buffer_load ... lds; double-buffered, one barrier per
//     tile, XOR-swizzled rows) and shared by the 4 waves.
//   * Each wave computes the transposed score tile Sᵀ = K Qᵀ on the 32×32×16 bf16 matrix core, so
//     every lane owns one query column: the row maximum and row sum of the softmax are in-lane
//     reductions plus one exchange between the two half-waves (v_permlane32_swap).
//   * The probabilities leave the accumulator as bf16 and feed Oᵀ += Vᵀ Pᵀ directly as the B
//     operand; V is read from its row-major LDS tile with ds_read_b64_tr_b16, whose key order matches
//     the accumulator's row order, so P never goes through LDS.
//   * The softmax runs in base 2 with scale·log2(e) folded into one FMA; normalisation by the row sum
//     is deferred to the end (fewer non-matmul operations, "Anatomy ...", section "What changed
//     between FlashAttention 1, 2, and 3?").  LSE is converted back to natural log on output.
//   * Grid: one workgroup per (batch·head, query tile); query tiles of one head are kept on one XCD so
//     the head's K/V stay in that XCD's L2; under the causal mask the heaviest tiles start first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBR = 128;   // queries per workgroup
constexpr int kBC = 64;    // keys per tile
constexpr int kThreads = 256;

template <int D>
struct FwdSmem {
  bf16 k[2][kBC * D];  // swizzled with tile_off<D>
  bf16 v[2][kBC * D];
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2, int remap) {
  constexpr int KSTEPS = D / 16;                 // k-steps of the Sᵀ product
  constexpr int DB = D / 32;                     // 32-row blocks of Oᵀ
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;        // half-wave: selects k-slots 8g..8g+7
  const int lc = lane & 31;       // row / column index inside a 32-wide matrix-core tile

  const uint32_t total = gridDim.x;
  const uint32_t logical = remap ? xcd_remap(blockIdx.x, total) : blockIdx.x;
  const int bh = logical / nqt;
  int qt = logical % nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kBR;
  const int qw = q0 + wave * 32;  // first query of this wave
  const int qi = qw + lc;         // this lane's query

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rk = make_rsrc(K + head, head_bytes);
  const auto rv = make_rsrc(V + head, head_bytes);

  // Qᵀ fragments (B operand): column = this lane's query, slots = d in [16s + 8g, 16s + 8g + 8).
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qi * D + 16 * s + 8 * g) * 2u));

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;

  tile_to_lds<D, kBC, kThreads>(rk, 0, sm.k[0], tid);
  tile_to_lds<D, kBC, kThreads>(rv, 0, sm.v[0], tid);
  wait_vmem_all();
  __syncthreads();

  float m = -INFINITY;  // running max of the base-2 scaled scores
  float l = 0.f;        // running sum of 2^(t - m) over this lane's keys (half of the row)
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;

  // Transposed-read addressing for the Vᵀ operand (see fa_common.h): lane i = 4a + b of each 16-lane
  // group reads keys k0 + a, d columns n0 + 4b .. n0 + 4b + 3.
  const int tr_a = (lane & 15) >> 2;
  const int tr_b = lane & 3;
  const int tr_n = 16 * ((lane >> 4) & 1);

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < ntiles;
    if (more) {  // next tile streams into the other buffer while this one is used
      tile_to_lds<D, kBC, kThreads>(rk, (j + 1) * kBC, sm.k[buf ^ 1], tid);
      tile_to_lds<D, kBC, kThreads>(rv, (j + 1) * kBC, sm.v[buf ^ 1], tid);
    }
    const int kv0 = j * kBC;

    if (!(CAUSAL && kv0 > qw + 31)) {  // tile fully masked for this wave: skip the math
      const bf16* klds = sm.k[buf];
      const bf16* vlds = sm.v[buf];
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 kf = *(const bf16x8*)&klds[tile_off<D>(kb * 32 + lc, 16 * s + 8 * g)];
          sacc[kb] = mfma_32x32x16(kf, qf[s], sacc[kb]);
        }
      }
      // Accumulator element (kb, r) is key kv0 + 32kb + 8(r/4) + 4g + (r%4) for query qi.
      const bool need_mask = (kv0 + kBC > N) || (CAUSAL && kv0 + kBC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > qi)) sacc[kb][r] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      float rs[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: shorter dependency chains
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(fmaf(sacc[kb][r], scale_log2, -m_use));
          sacc[kb][r] = p;
          rs[r & 3] += p;
        }
      l = fmaf(l, alpha, (rs[0] + rs[1]) + (rs[2] + rs[3]));
      // Rescale the output accumulator only when some row's maximum moved (alpha != 1 somewhere in
      // the wave); once the maxima settle, most tiles skip these multiplies.
      if (!wave_all(m_new == m)) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      }
      m = m_new;

      // Pᵀ operand for k-step ks (16 keys): slots e = registers 8(ks%2) + e of key block ks/2, i.e.
      // keys 16ks + 8(e/4) + 4g + (e%4) — the order the transposed V reads below produce.
      bf16x8 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)sacc[ks >> 1][8 * (ks & 1) + e];

#pragma unroll
      for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int key = 16 * ks + 4 * g + tr_a;
          const int col = 32 * b + tr_n + 4 * tr_b;
          const u32x2 lo = lds_read_tr16(&vlds[tile_off<D>(key, col)]);
          const u32x2 hi = lds_read_tr16(&vlds[tile_off<D>(key + 8, col)]);
          const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
          oacc[b] = mfma_32x32x16(__builtin_bit_cast(bf16x8, vv), pf[ks], oacc[b]);
        }
      }
    }
    wait_vmem_all();
    __syncthreads();
  }

  // Epilogue: combine the two half-row sums, normalise, write O and LSE.
  const float l_tot = halves_sum(l);
  const float inv = 1.f / l_tot;
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

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBR - 1) / kBR;
  const uint32_t total = (uint32_t)a.B * a.H * nqt;
  const int remap = (total % 8u == 0u) ? 1 : 0;
  const float scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.N,
                     nqt, scale_log2, remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
