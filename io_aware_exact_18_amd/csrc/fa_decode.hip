// fa_decode.hip — decoding against a key/value cache on gfx950: Nq ≤ 32 new queries per (batch, head)
// attend over Nk cached keys.
//
// The inference use the pages pair FlashAttention with (glossary entry "flash attention", paragraph on
// long-context training and serving: the KV cache bounds the context held, FlashAttention the cost of
// attending over it; "FlashAttention: where it matters", section "Where It Matters": long-context
// inference, speculative decoding).  The queries are the last Nq positions of the sequence: with the
// causal mask query i may use key j when j ≤ Nk − Nq + i.
//
// A decode step reads the whole cache once and does little arithmetic per byte, so it is bound by HBM
// bandwidth, and one (batch, head) pair alone cannot keep the device's memory system busy.  The keys
// are therefore split into S chunks ("split-KV"):
//   * decode_split_kernel: one wave per (batch·head, chunk) streams the chunk's K/V tiles into LDS
//     by buffer→LDS DMA (double-buffered 32-key tiles), computes Sᵀ = K Qᵀ and Oᵀ += Vᵀ Pᵀ on the
//     32×32×16 bf16 matrix core with the queries as the 32 columns (rows past Nq are zero and
//     discarded), runs the online softmax of "Anatomy of a FlashAttention Kernel", section "What is
//     online softmax and how does tiling keep it exact?", and writes the chunk's unnormalised output
//     with its row maximum and two row sums (fp32) to the workspace: over the fp32 probabilities (for
//     LSE) and over the same values rounded to bf16, the weights P·V applies (O is divided by it, as
//     in the forward kernel).
//   * decode_merge_kernel: per (batch·head, query) combines the chunks by their softmax mass — the same
//     recurrence applied to whole chunks — and writes O (bf16) and LSE (fp32, natural log).
// Chunks of one head are consecutive workgroups and so run on different XCDs (round-robin dispatch);
// the cache is read once either way.
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kDecBC = 32;       // keys per tile
constexpr int kDecThreads = 64;  // one wave per workgroup
constexpr float kDecSlack = 8.f; // reference-maximum slack (base 2), as in the forward kernel

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    float* __restrict__ part_o, float* __restrict__ part_ml, int Nq, int Nk, int split_len, int S,
    float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int L = lds_cols<D>();
  // K/V tiles, double-buffered (separate LDS objects, so reads of one buffer never wait for the DMA
  // filling the other): tile j lives in buffers j % 2.  Deeper rings (3 or 4 tiles) measured the same:
  // the call already streams the cache at the device's achievable read rate.
  __shared__ __attribute__((aligned(1024))) bf16 k0s[kDecBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 k1s[kDecBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v0s[kDecBC * L];
  __shared__ __attribute__((aligned(1024))) bf16 v1s[kDecBC * L];

  const int lane = threadIdx.x;
  const int g = lane >> 5;
  const int lc = lane & 31;  // this lane's query (column of Sᵀ); valid when lc < Nq
  const int bh = blockIdx.x / S;
  const int sp = blockIdx.x % S;
  const int k_begin = sp * split_len;
  const int k_end = min(Nk, k_begin + split_len);
  const int q_first_pos = Nk - Nq;        // position of query 0 in the key sequence
  const int q_pos = q_first_pos + lc;     // this lane's query position (causal mask)

  const size_t kv_head = (size_t)bh * Nk * D;
  const uint32_t kv_bytes = (uint32_t)Nk * D * 2u;
  const auto rq = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 2u);  // rows ≥ Nq read 0
  const auto rk = make_rsrc(K + kv_head, kv_bytes);
  const auto rv = make_rsrc(V + kv_head, kv_bytes);
  const BfTileCopy<D, kDecBC, kDecThreads> copy(lane);

  bf16x8 qf[KSTEPS];  // Qᵀ fragments (B operand): column = this lane's query, d = 16s + 8g .. +7
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(lc * D + 16 * s + 8 * g) * 2u));

  const int ntiles = (k_end - k_begin + kDecBC - 1) / kDecBC;
  const FragOffsets<L> fo(lane);
  copy(rk, k_begin, k0s);
  copy(rv, k_begin, v0s);

  float m = -INFINITY;  // reference maximum of the base-2 scaled scores (raised past kDecSlack)
  float l = 0.f;        // Σ 2^(t − m) over this lane's half of the keys
  float lr = 0.f;       // the same over the bf16-rounded values that enter P·V
  f32x16 oacc[DB];      // Oᵀ: rows d = 32b + 8(r/4) + 4g + r%4, column = this lane's query
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;

  // Tile j of the chunk; P is its parity: the tile is in buffers P, buffers P^1 receive tile j + 1.
  auto tile = [&](auto parity, int j) {
    constexpr int P = decltype(parity)::value;
    const char* klds = (const char*)(P ? k1s : k0s);
    const char* vlds = (const char*)(P ? v1s : v0s);
    wait_vmem_all();  // tile j has landed
    __syncthreads();  // one wave: orders the LDS reads of tile j − 1 before the refill below
    if (j + 1 < ntiles) {
      copy(rk, k_begin + (j + 1) * kDecBC, P ? k0s : k1s);
      copy(rv, k_begin + (j + 1) * kDecBC, P ? v0s : v1s);
    }
    const int kv0 = k_begin + j * kDecBC;
    // Sᵀ = K Qᵀ: element r is key kv0 + 8(r/4) + 4g + (r%4) for this lane's query.
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) sacc = mfma_32x32x16(row_frag<L>(klds, fo, 0, s), qf[s], sacc);
    // Keys past the chunk (the last tile may be ragged) and, causal, past the query's position.
    if ((kv0 + kDecBC > k_end) || (CAUSAL && kv0 + kDecBC - 1 > q_first_pos)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= k_end || (CAUSAL && key > q_pos)) sacc[r] = -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    const float mt = halves_max(mx) * scale_log2;
    if (!wave_all(mt <= m + kDecSlack)) {  // raise the reference; rows without keys keep -inf
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
    // Pᵀ operand for k-step ks (16 keys): registers 8ks .. 8ks+7, keys 16ks + 8(e/4) + 4g + (e%4) —
    // the order of the transposed V reads.
    bf16x8 pf[2];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(sacc[r], scale_log2, -m_use));
      rs[r & 3] += p;
      pf[r >> 3][r & 7] = (__bf16)p;
    }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    lr = sum_bf16x8(pf[1], sum_bf16x8(pf[0], lr));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 vf[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) vf[b] = tr_frag<L>(vlds, fo, ks, b);
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] = mfma_32x32x16(vf[b], pf[ks], oacc[b]);
    }
  };

  for (int j = 0; j < ntiles; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) tile(std::integral_constant<int, 1>{}, j + 1);
  }
  wait_vmem_all();

  // The chunk's result for this lane's query: unnormalised Oᵀ column, reference maximum m (base 2)
  // and the row sums l and lr.  Layout: part_o [BH][S][Nq][D], part_ml [BH][S][Nq][3].
  const float l_tot = halves_sum(l);
  const float lr_tot = halves_sum(lr);
  if (lc < Nq) {
    const size_t row = ((size_t)bh * S + sp) * Nq + lc;
    float* orow = part_o + row * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 w = {oacc[b][4 * r4], oacc[b][4 * r4 + 1], oacc[b][4 * r4 + 2],
                         oacc[b][4 * r4 + 3]};
        *(f32x4*)&orow[32 * b + 8 * r4 + 4 * g] = w;
      }
    if (g == 0) {
      part_ml[3 * row] = m;
      part_ml[3 * row + 1] = l_tot;
      part_ml[3 * row + 2] = lr_tot;
    }
  }
}

// One wave per (batch·head, query): merge_partials over the query's S chunks.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          bf16* __restrict__ O,
                                                          float* __restrict__ LSE, int Nq, int S) {
  const int bh = blockIdx.x / Nq;
  const int qi = blockIdx.x % Nq;
  const size_t out_row = (size_t)bh * Nq + qi;
  merge_partials<D>(part_o, part_ml, (size_t)bh * S * Nq + qi, (size_t)Nq, S, O + out_row * D,
                    LSE + out_row, threadIdx.x);
}

template <int D, bool CAUSAL>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const DecodeSplit sp = decode_split(a.B, a.H, a.Nq, a.Nk);
  const uint32_t bh = (uint32_t)a.B * a.H;
  float* part_o = (float*)a.workspace;
  float* part_ml = part_o + (size_t)bh * sp.S * a.Nq * D;
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL>), dim3(bh * sp.S), dim3(kDecThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, part_o, part_ml, a.Nq,
                     a.Nk, sp.split_len, sp.S, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(bh * a.Nq), dim3(64), 0, stream,
                     (const float*)part_o, (const float*)part_ml, (bf16*)a.o, a.lse, a.Nq, sp.S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  if (a.d == 96) return a.causal ? launch<96, true>(a, stream) : launch<96, false>(a, stream);
  if (a.d == 256) return a.causal ? launch<256, true>(a, stream) : launch<256, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
