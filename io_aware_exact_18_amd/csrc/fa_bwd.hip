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
// Three launches on the caller's stream:
//   1. bwd_pre: D_i = dO_i · O_i in fp32 and zero the fp32 dQ accumulator.
//   2. bwd_main: one workgroup per 128-key tile (4 waves × 32 keys).  Each wave keeps its K and V rows
//      as matrix-core operands in registers and its dKᵀ, dVᵀ accumulators in registers, and walks the
//      32-query tiles the causal mask allows.  Per query tile: S and dP on the 32×32×16 bf16 matrix
//      core, P and dS on the vector units, dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS with the transposed LDS reads
//      supplying dOᵀ and Qᵀ, then dSᵀ goes through LDS so each wave can form a 32-column slice of
//      dQ = dS K over all 128 keys and add it into the fp32 accumulator with atomics.
//   3. dq_convert: dQ = bf16(scale · accumulator).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBQ = 32;    // queries per step

// ---------------------------------------------------------------------------------------------------
// 1. D_i = Σ_t dO_it O_it; dq_acc = 0.  One row per D/8 threads, 8 elements per thread.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                           const bf16* __restrict__ dO,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ dq_acc,
                                                           long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long row = (long)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + row * D + part * 8);
    const u32x4 b = *(const u32x4*)(dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_bits_to_float(a[i] & 0xffffu), bf16_bits_to_float(b[i] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_float(a[i] >> 16), bf16_bits_to_float(b[i] >> 16), acc);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(dq_acc + row * D + part * 8) = z;
    *(f32x4*)(dq_acc + row * D + part * 8 + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------------------------------
// 2. Main backward kernel.
template <int D>
struct BwdSmem {
  bf16 k[kBKV * D];            // K tile, swizzled (B operand of dQ = dS K via transposed reads)
  bf16 q[2][kBQ * D];          // Q tile, swizzled, double-buffered
  bf16 dout[2][kBQ * D];       // dO tile, swizzled, double-buffered
  float lse2[2][kBQ];          // LSE · log2(e)
  float delta[2][kBQ];         // D_i
  bf16 dst[kBKV * 48];         // dSᵀ [key][query], row pitch 48 (conflict-free transposed reads)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void bwd_main_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ LSE, const bf16* __restrict__ dO, const float* __restrict__ Delta,
    float* __restrict__ dq_acc, bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int nkt,
    float scale, float scale_log2, int remap) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int DSP = 48;                                   // dSᵀ row pitch (elements)
  constexpr int QCH = kBQ * D / 8 / kThreads;               // 16-byte chunks per thread per Q tile
  __shared__ BwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int lc = lane & 31;
  const int tr_a = (lane & 15) >> 2;
  const int tr_b = lane & 3;
  const int tr_n = 16 * ((lane >> 4) & 1);

  const uint32_t logical = remap ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  const int bh = logical / nkt;
  const int kt = logical % nkt;
  const int k0 = kt * kBKV;
  const int kw = k0 + 32 * wave;   // first key of this wave
  const int kj = kw + lc;          // this lane's key (column of the score tiles)

  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rk = make_rsrc(K + head, head_bytes);
  const auto rv = make_rsrc(V + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto rlse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const auto rdel = make_rsrc(Delta + (size_t)bh * N, (uint32_t)N * 4u);

  // Kᵀ and Vᵀ operands (B operands of S = Q Kᵀ and dP = dO Vᵀ): column = this lane's key.
  bf16x8 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const uint32_t off = (uint32_t)(kj * D + 16 * s + 8 * g) * 2u;
    kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vf[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  // Whole K tile into LDS for the dQ product.
#pragma unroll
  for (int i = 0; i < kBKV * D / 8 / kThreads; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(u32x4*)&sm.k[tile_off<D>(row, col)] = buf_load16(rk, (uint32_t)((k0 + row) * D + col) * 2u);
  }

  // Query tiles: causal keeps queries ≥ the first key of the tile.
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (N - qstart + kBQ - 1) / kBQ;

  u32x4 qreg[QCH], doreg[QCH];
  float sreg = 0.f;
  auto load_q = [&](int step) {
    const int qb = qstart + step * kBQ;
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const uint32_t off = (uint32_t)((qb + row) * D + col) * 2u;
      qreg[i] = buf_load16(rq, off);
      doreg[i] = buf_load16(rdo, off);
    }
    if (tid < kBQ)
      sreg = __uint_as_float(buf_load4(rlse, (uint32_t)(qb + tid) * 4u)) * kLog2e;
    else if (tid < 2 * kBQ)
      sreg = __uint_as_float(buf_load4(rdel, (uint32_t)(qb + tid - kBQ) * 4u));
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(u32x4*)&sm.q[buf][tile_off<D>(row, col)] = qreg[i];
      *(u32x4*)&sm.dout[buf][tile_off<D>(row, col)] = doreg[i];
    }
    if (tid < kBQ)
      sm.lse2[buf][tid] = sreg;
    else if (tid < 2 * kBQ)
      sm.delta[buf][tid - kBQ] = sreg;
  };

  f32x16 dka[DB], dva[DB];  // dKᵀ, dVᵀ: rows = d (32b + 8(r/4) + 4g + r%4), column = key
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[b][r] = 0.f;
      dva[b][r] = 0.f;
    }

  if (nsteps > 0) {
    load_q(0);
    store_q(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) load_q(step + 1);
    const int qb = qstart + step * kBQ;
    const bf16* qs = sm.q[buf];
    const bf16* dos = sm.dout[buf];

    // S = Q Kᵀ and dP = dO Vᵀ for 32 queries × this wave's 32 keys.
    f32x16 sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = 0.f;
      pacc[r] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 qa = *(const bf16x8*)&qs[tile_off<D>(lc, 16 * s + 8 * g)];
      const bf16x8 da = *(const bf16x8*)&dos[tile_off<D>(lc, 16 * s + 8 * g)];
      sacc = mfma_32x32x16(qa, kf[s], sacc);
      pacc = mfma_32x32x16(da, vf[s], pacc);
    }
    // Element r: query qb + 8(r/4) + 4g + (r%4), key kj.
    const bool need_mask = (kw + 31 >= N) || (CAUSAL && kw + 31 > qb);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 l4 = *(const f32x4*)&sm.lse2[buf][8 * r4 + 4 * g];
      const f32x4 d4 = *(const f32x4*)&sm.delta[buf][8 * r4 + 4 * g];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * r4 + t;
        float p = exp2_fast(fmaf(sacc[r], scale_log2, -l4[t]));
        if (need_mask) {
          const int qi = qb + 8 * r4 + 4 * g + t;
          if (kj >= N || (CAUSAL && kj > qi)) p = 0.f;
        }
        sacc[r] = p;
        pacc[r] = p * (pacc[r] - d4[t]);  // dS (without the scale)
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
        const int qrow = 16 * ks + 4 * g + tr_a;
        const int col = 32 * b + tr_n + 4 * tr_b;
        const u32x2 dlo = lds_read_tr16(&dos[tile_off<D>(qrow, col)]);
        const u32x2 dhi = lds_read_tr16(&dos[tile_off<D>(qrow + 8, col)]);
        const u32x2 qlo = lds_read_tr16(&qs[tile_off<D>(qrow, col)]);
        const u32x2 qhi = lds_read_tr16(&qs[tile_off<D>(qrow + 8, col)]);
        const u32x4 dv4 = {dlo[0], dlo[1], dhi[0], dhi[1]};
        const u32x4 qv4 = {qlo[0], qlo[1], qhi[0], qhi[1]};
        dva[b] = mfma_32x32x16(__builtin_bit_cast(bf16x8, dv4), pb[ks], dva[b]);
        dka[b] = mfma_32x32x16(__builtin_bit_cast(bf16x8, qv4), dsb[ks], dka[b]);
      }
    }
    // dSᵀ → LDS: this lane's key row, queries 8(r/4) + 4g .. +3 as 8-byte writes.
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 w;
      w[0] = pack_bf16x2(pacc[4 * r4 + 0], pacc[4 * r4 + 1]);
      w[1] = pack_bf16x2(pacc[4 * r4 + 2], pacc[4 * r4 + 3]);
      *(u32x2*)&sm.dst[(32 * wave + lc) * DSP + 8 * r4 + 4 * g] = w;
    }
    __syncthreads();

    // dQ[:, 32·wave .. 32·wave + 32) += dS (32 q × 128 keys) · K (128 keys × 32 d); with D = 64 only
    // waves 0 and 1 have a d-slice.  A = dS rows (queries) from dSᵀ, B = K columns (d) from the K
    // tile; both transposed reads with keys 16ks + 4g + 8h + (0..3) in slot 4h + (0..3).
    if (32 * wave < D) {
      f32x16 qacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) qacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kBKV / 16; ++ks) {
        const int krow = 16 * ks + 4 * g + tr_a;
        const u32x2 alo = lds_read_tr16(&sm.dst[krow * DSP + tr_n + 4 * tr_b]);
        const u32x2 ahi = lds_read_tr16(&sm.dst[(krow + 8) * DSP + tr_n + 4 * tr_b]);
        const int col = 32 * wave + tr_n + 4 * tr_b;
        const u32x2 blo = lds_read_tr16(&sm.k[tile_off<D>(krow, col)]);
        const u32x2 bhi = lds_read_tr16(&sm.k[tile_off<D>(krow + 8, col)]);
        const u32x4 a4 = {alo[0], alo[1], ahi[0], ahi[1]};
        const u32x4 b4 = {blo[0], blo[1], bhi[0], bhi[1]};
        qacc = mfma_32x32x16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4), qacc);
      }
      // qacc element r: query qb + 8(r/4) + 4g + (r%4), d = 32·wave + lc.
      float* dqh = dq_acc + head;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (qi < N) unsafeAtomicAdd(&dqh[(size_t)qi * D + 32 * wave + lc], qacc[r]);
      }
    }
    if (more) store_q(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: dK = scale · dKᵀᵀ, dV = dVᵀᵀ; this lane owns key kj, d rows 32b + 8(r/4) + 4g + (0..3).
  if (kj < N) {
    bf16* dkr = dK + head + (size_t)kj * D;
    bf16* dvr = dV + head + (size_t)kj * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dka[b][4 * r4 + 0] * scale, dka[b][4 * r4 + 1] * scale);
        wk[1] = pack_bf16x2(dka[b][4 * r4 + 2] * scale, dka[b][4 * r4 + 3] * scale);
        wv[0] = pack_bf16x2(dva[b][4 * r4 + 0], dva[b][4 * r4 + 1]);
        wv[1] = pack_bf16x2(dva[b][4 * r4 + 2], dva[b][4 * r4 + 3]);
        *(u32x2*)&dkr[32 * b + 8 * r4 + 4 * g] = wk;
        *(u32x2*)&dvr[32 * b + 8 * r4 + 4 * g] = wv;
      }
  }
}

// ---------------------------------------------------------------------------------------------------
// 3. dQ = bf16(scale · accumulator), 8 elements per thread.
__global__ __launch_bounds__(kThreads) void dq_convert_kernel(const float* __restrict__ acc,
                                                              bf16* __restrict__ dq, float scale,
                                                              long n8) {
  const long i = (long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + 8 * i);
  const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
  u32x4 w;
  w[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
  w[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
  w[2] = pack_bf16x2(b[0] * scale, b[1] * scale);
  w[3] = pack_bf16x2(b[2] * scale, b[3] * scale);
  *(u32x4*)(dq + 8 * i) = w;
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  const long rows = (long)a.B * a.H * a.N;
  constexpr int rows_per_block = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(kThreads), 0, stream, (const bf16*)a.o, (const bf16*)a.dout, a.delta,
                     a.dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int nkt = (a.N + kBKV - 1) / kBKV;
  const uint32_t total = (uint32_t)a.B * a.H * nkt;
  const int remap = (total % 8u == 0u) ? 1 : 0;
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                     (const bf16*)a.dout, (const float*)a.delta, a.dq_acc, (bf16*)a.dk,
                     (bf16*)a.dv, a.N, nkt, a.scale, a.scale * kLog2e, remap);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const long n8 = rows * D / 8;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, (const float*)a.dq_acc, (bf16*)a.dq, a.scale, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
