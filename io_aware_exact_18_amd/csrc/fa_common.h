// fa_common.h — device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix-core conventions (measured on gfx950 with a lane-layout probe):
//   v_mfma_f32_32x32x16_bf16  A is 32×16, B is 16×32, C/D is 32×32 fp32.
//     A operand: lane l holds row (l % 32) and 8 k-slots; B operand: lane l holds column (l % 32) and
//     the same 8 k-slots.  Slot e of lane group g = l / 32 is k = 8·g + e (any k order works as long
//     as A and B agree, which they do by construction here).
//     D: lane l, register r holds row 8·(r/4) + 4·(l/32) + (r % 4), column l % 32.
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane i = 4a + b supplies the address of 4
//     consecutive 16-bit elements M[k0 + a][n0 + 4b .. n0 + 4b + 3] of a row-major LDS matrix; lane
//     j of the group then receives M[k0 .. k0 + 3][n0 + j], i.e. four consecutive rows of one column.
//     This feeds a matrix-core operand whose contraction index runs along the rows of M.
//   Workgroups are dispatched to the 8 XCDs round-robin: block b runs on XCD b % 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 raw buffer: 32-bit data format, no swizzle

// A raw buffer resource over [base, base + bytes).  Loads past `bytes` return zeros, which is how
// ragged sequence tails are read without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufferFlags);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ inline u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}

__device__ inline uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

__device__ inline f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four consecutive rows of one column of a row-major bf16 LDS matrix (see the header comment).
__device__ inline u32x2 lds_read_tr16(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// x from this lane and from lane (l ^ 32), combined with max / sum.  Both halves of the wave get a
// bitwise-identical result.
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every outstanding vector-memory load of this wave.  Used once after loads made before a
// loop whose body consumes them: otherwise the wait the compiler inserts inside the loop is counted
// against the loop's own prefetch loads and exposes their latency on every iteration.
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar) value, so conditions and
// addresses derived from it stay in scalar registers and branches on it are uniform.
__device__ inline int wave_index(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// True when `pred` holds on every active lane of the wave (a wave-uniform answer).
__device__ inline bool wave_all(bool pred) { return __builtin_amdgcn_ballot_w64(!pred) == 0; }

// Round two floats to bf16 (round-to-nearest-even) and pack them, first in the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// acc + the sum of the eight bf16 values of v, in fp32 (four v_dot2c_f32_bf16 against (1, 1)).
__device__ inline float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t pair = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pair, one, acc, false);
  }
  return acc;
}

// Four fp32 values → four OCP e4m3fn bytes (round to nearest even), first in the lowest byte.  The
// conversion does not saturate: a magnitude above 464 (the midpoint between 448 and 480) gives the
// NaN code.  Callers keep their values within ±448.  Each conversion writes one 16-bit half of its
// result and keeps the other from its third operand; the two calls overwrite both halves, so the
// first starts from p0's own bits (a register that dies there) rather than from a zeroed one.
__device__ inline uint32_t pack_e4m3x4(float p0, float p1, float p2, float p3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __builtin_bit_cast(int, p0), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, lo, true);
}

// LDS tile layout for a [rows][D] bf16 tile with no padding: the 16-byte chunk c of row r is stored at
// chunk c ^ H(r).  gfx950's LDS has 64 four-byte banks and serves 16 lanes of a 16-byte read (32 lanes
// of an 8-byte read) per pass; H is chosen so both access patterns the kernels use are conflict-free:
//   * row reads: 16 lanes read the same logical chunk of 16 consecutive rows — H(r) takes every value
//     once over any 16 consecutive rows;
//   * transposed reads: 32 lanes read 4 consecutive rows × 64 bytes — the 4 rows' chunk groups land
//     on disjoint bank quarters.
// D = 128 (256-byte rows) and D = 256 (512-byte rows: the bank of chunk c is c mod 16, and H < 16
// keeps c ^ H within its half-row): H(r) = 4·(r mod 4) + (r/4 mod 4).
// D = 64 (128-byte rows, two rows per bank period): H(r) = 4·(r/2 mod 2) + (r/4 mod 4).
template <int D>
__device__ inline int swz_h(int r) {
  static_assert(D == 64 || D == 128 || D == 256, "head dimension");
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// Columns of the LDS layout of a tile whose rows hold D values: D = 96 is kept in the D = 128 layout
// (256-byte rows; the last 32 columns are zero-filled by the copy and never read), so the swizzle
// and fragment offsets of D = 128 apply unchanged.
template <int D>
constexpr int lds_cols() {
  static_assert(D == 64 || D == 96 || D == 128 || D == 256, "head dimension");
  return D == 96 ? 128 : D;
}

template <int D>
__device__ inline int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz_h<D>(row)) << 3) | (col & 7));
}

// Per-lane LDS byte offsets of the matrix-core fragments a lane reads from a tile in the tile_off<D>
// layout.  H depends only on a row's low 4 bits, so a fragment 16 or 32 rows further down is the same
// lane offset plus a compile-time constant (folded into the read's immediate offset).
// With D = 256 the upper 256 bytes of a row repeat the lower half's chunk permutation (H < 16), so
// a fragment there is the lower half's offset plus 256: only the first 128 columns' offsets are kept.
template <int D>
struct FragOffsets {
  static constexpr int DL = D < 128 ? D : 128;  // columns whose offsets are stored
  // Row read (16 bytes) of row 32kb + (lane % 32), d = 16s + 8g .. +7:
  // row[s % 8] + 256·(s / 8) + 64·D·kb.
  uint32_t row[DL / 16];
  // Transposed read (8 bytes) of rows 16ks + 8h + 4g + tr_a, d = 32b + tr_n + 4 tr_b .. +3:
  // tr[b % 4][h] + 256·(b / 4) + 32·D·ks.
  uint32_t tr[DL / 32][2];
  __device__ explicit FragOffsets(int lane) {
    const int g = lane >> 5, lc = lane & 31;
    const int tr_a = (lane & 15) >> 2, tr_b = lane & 3, tr_n = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int s = 0; s < DL / 16; ++s)
      row[s] = (uint32_t)(lc * D * 2 + 16 * ((2 * s + g) ^ swz_h<D>(lc)));
    const int x = tr_n / 8 + (tr_b >> 1);
#pragma unroll
    for (int b = 0; b < DL / 32; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * g + tr_a + 8 * h;
        tr[b][h] = (uint32_t)(r * D * 2 + 16 * ((4 * b + x) ^ swz_h<D>(r)) + 8 * (tr_b & 1));
      }
  }
};

// A-/B-operand fragment with 8 consecutive d values: row 32kb + (lane % 32), d = 16s + 8g .. +7.
template <int D>
__device__ inline bf16x8 row_frag(const char* lds, const FragOffsets<D>& fo, int kb, int s) {
  constexpr int NS = FragOffsets<D>::DL / 16;
  return *(const bf16x8*)(lds + fo.row[s % NS] + 256 * (s / NS) + kb * 64 * D);
}

// Operand fragment whose contraction index runs down the tile's rows: column d = 32b + (lane % 32),
// slots e = 0..7 hold rows 16ks + 4g + 8(e/4) + (e%4).
template <int D>
__device__ inline bf16x8 tr_frag(const char* lds, const FragOffsets<D>& fo, int ks, int b) {
  constexpr int NB = FragOffsets<D>::DL / 32;
  const char* base = lds + 256 * (b / NB) + ks * 32 * D;
  const u32x2 lo = lds_read_tr16((const bf16*)(base + fo.tr[b % NB][0]));
  const u32x2 hi = lds_read_tr16((const bf16*)(base + fo.tr[b % NB][1]));
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Asynchronous copy of ROWS rows (rows row0 .. row0+ROWS-1 of the matrix behind the buffer resource
// `r`, GROW_BYTES bytes apart) into LDS rows of ROW_BYTES ≥ GROW_BYTES bytes by NT threads, without
// passing through registers (buffer_load_dwordx4 ... lds: lane i of a wave writes LDS bytes
// [16 i, 16 i + 16) after the wave-uniform base).  Rows past the buffer's end read as zeros, and so
// do the LDS chunks past GROW_BYTES (their source offset is set beyond any buffer's range, so they
// cost no memory traffic).  The 16-byte chunk c of row r is
// stored at physical chunk c ^ swz(r), where swz depends only on r mod 16.  An issue round covers
// NT / (ROW_BYTES / 16) rows; the swizzle repeats every 16 rows, so a lane's offset within a round
// takes PAT = max(1, 16 / rows-per-round) values, computed once, here, and each load of a copy adds
// a scalar row offset to one of them (one vector add; the row offset stays in the range-checked
// vector offset so the zero fill of ragged tails still applies).  Completion: wait_vmem_all().
template <int ROW_BYTES, int ROWS, int NT, int GROW_BYTES = ROW_BYTES>
struct TileCopy {
  static constexpr int CPR = ROW_BYTES / 16;        // 16-byte chunks per row
  static_assert(GROW_BYTES % 16 == 0 && GROW_BYTES <= ROW_BYTES, "source rows of whole chunks");
  // Source offset of a padding chunk: at least 2^31, past every buffer's range (heads are < 2 GiB),
  // and still below 2^32 after a row offset (< 2^31) is added.
  static constexpr uint32_t kPad = 0x80000000u;
  static constexpr int ROUNDS = ROWS * CPR / NT;    // loads per thread
  static constexpr int ROUND_ROWS = NT / CPR;       // rows per round
  static constexpr int PAT = ROUND_ROWS >= 16 ? 1 : 16 / ROUND_ROWS;  // distinct lane offsets
  static_assert(ROWS * CPR % NT == 0, "tile must split evenly over the threads");
  static_assert(ROUND_ROWS % 16 == 0 || 16 % ROUND_ROWS == 0, "the swizzle must repeat across rounds");
  static_assert(ROUNDS % PAT == 0, "whole swizzle periods per copy");
  uint32_t voff[PAT];  // this lane's byte offset inside round p of each swizzle period
  int wave;
  template <class Swz>
  __device__ TileCopy(int tid, Swz swz) {
    wave = wave_index(tid);
    const int slot = wave * 64 + (tid & 63);  // physical 16-byte slot within a round
    const int pc = slot % CPR;
#pragma unroll
    for (int p = 0; p < PAT; ++p) {
      const int row = p * ROUND_ROWS + slot / CPR;
      const int c = pc ^ swz(row);  // logical chunk held by slot pc
      voff[p] = 16 * c < GROW_BYTES ? (uint32_t)(row * GROW_BYTES + 16 * c) : kPad;
    }
  }
  template <class T>
  __device__ void operator()(__amdgpu_buffer_rsrc_t r, int row0, T* lds) const {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const uint32_t base = (uint32_t)(row0 + (i / PAT) * PAT * ROUND_ROWS) * (uint32_t)GROW_BYTES;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)((char*)lds + (i * (NT / 64) + wave) * 1024),
          16, (uint32_t)(voff[i % PAT] + base), 0, 0, 0);
    }
  }
};

// TileCopy for a [ROWS][D] bf16 tile into the tile_off<lds_cols<D>()> layout.
template <int D, int ROWS, int NT>
struct BfTileCopy : TileCopy<2 * lds_cols<D>(), ROWS, NT, 2 * D> {
  __device__ explicit BfTileCopy(int tid)
      : TileCopy<2 * lds_cols<D>(), ROWS, NT, 2 * D>(tid,
                                                     [](int r) { return swz_h<lds_cols<D>()>(r); }) {}
};

// Asynchronous copy of 64 consecutive fp32 values (elements e0 .. e0+63 behind `r`) into LDS by one
// wave; values past the buffer's end read as zeros.
__device__ inline void vec64_to_lds(__amdgpu_buffer_rsrc_t r, int e0, float* lds, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           (uint32_t)(e0 + lane) * 4u, 0, 0, 0);
}

// Partial-result outputs of the forwards' key-range split (fwd_split in fa_launch.h): per (segment,
// batch·head, query) row the unnormalised output (D fp32, in units of the output) and (m, l, lr).
struct SplitOut {
  float* part_o;   // [nseg][B·H][N][D]
  float* part_ml;  // [nseg][B·H][N][3]: reference maximum (base 2), fp32 and bf16-rounded row sums
  int seg;         // key tiles per segment
  int bh_count;    // B·H
};

// Combines `nseg` partial results of one query row, each over a disjoint range of keys, into the row's
// output and logsumexp: the online-softmax recurrence of "Anatomy of a FlashAttention Kernel", section
// "What is online softmax and how does tiling keep it exact?", applied to whole key ranges.  Partial s
// is at row row0 + s·stride of part_o (D fp32: the unnormalised output Σ p·v) and of part_ml (3 fp32:
// the range's reference maximum m in base 2, and its row sums over the fp32 probabilities and over the
// same values rounded to bf16).  O is divided by the merged bf16 sum (the weights the products
// applied), LSE comes from the fp32 sum.  One wave per row: lane t writes columns t, t + 64, ...
template <int D>
__device__ inline void merge_partials(const float* __restrict__ part_o,
                                      const float* __restrict__ part_ml, size_t row0,
                                      size_t stride, int nseg, bf16* __restrict__ orow,
                                      float* __restrict__ lse_out, int lane) {
  constexpr int PER = (D + 63) / 64;  // values per lane (the last partly idle when D = 96)
  float m = -INFINITY;
  for (int s = 0; s < nseg; ++s) m = fmaxf(m, part_ml[3 * (row0 + (size_t)s * stride)]);
  float l = 0.f, lr = 0.f, acc[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) acc[t] = 0.f;
  for (int s = 0; s < nseg; ++s) {
    const size_t row = row0 + (size_t)s * stride;
    const float ms = part_ml[3 * row];
    const float w = exp2_fast(ms - m);  // 0 for a range without usable keys (ms = -inf)
    l += w * part_ml[3 * row + 1];
    lr += w * part_ml[3 * row + 2];
#pragma unroll
    for (int t = 0; t < PER; ++t)
      if (D % 64 == 0 || lane + 64 * t < D) acc[t] += w * part_o[row * D + lane + 64 * t];
  }
  const float inv = 1.f / lr;
#pragma unroll
  for (int t = 0; t < PER; ++t)
    if (D % 64 == 0 || lane + 64 * t < D) orow[lane + 64 * t] = (__bf16)(acc[t] * inv);
  if (lane == 0) *lse_out = (m + __log2f(l)) * kLn2;
}

// blockIdx → logical work item such that consecutive logical items land on the same XCD: logical
// item L runs on XCD L / (total / 8).  Used only when total is a multiple of 8.
__host__ __device__ inline uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  return (bid % 8u) * (total / 8u) + bid / 8u;
}

// Logical work item → (head, tile) for grids of `ntile` tiles per head, tiles numbered in the order
// they should start (under the causal mask: heaviest first). Heads are taken in groups, and within
// a group the items alternate between the heads tile by tile: the items of a group of g heads
// starting at head h are g·t + i → tile t of head h + i. Causal tiles range from one key tile to
// all of them, and workgroups start in item order as slots free up. Head by head, the last heads of
// a dispatch queue start their heaviest tiles late and leave compute units idle at the end; in
// groups, every group's heaviest tiles start together, and the workgroups in flight still cover few
// heads, whose K and V (or Q and dO) they share through L2. Groups hold kHeadGroup heads, the last
// one also the remainder (a short last group would end the queue on its heaviest tiles again). In
// the XCD order (`remap`: each XCD takes a contiguous eighth of the items) the heads are grouped
// within each XCD's eighth, so that no group spans two XCDs (the first would take the heaviest
// tiles of several heads, the other their lightest); when the head count is not a multiple of 8 the
// eighths cut heads anyway, and the heads are taken one at a time. They are also taken one at a
// time when a head has at least as many tiles as an XCD holds workgroups at once (32 compute units
// × `per_cu` resident workgroups): the queue then finishes evenly, and groups would only cost L2
// reuse (the forward of 32 heads of 16384 keys took the same time either way, and read 2.8× instead
// of 1.3× its algorithmic bytes from beyond L2 in groups). Measured on MI355X, causal 4 × 32 × 4096
// × 128 (one process, bit-identical results), one head at a time → groups of 4: forward 0.625 →
// 0.569 ms, dK/dV 1.154 → 1.045, dQ 0.814 → 0.759; groups of 3 or 6 (leaving a short last group per
// XCD) were 3–8% slower than groups of 4, groups of 8 1%.
constexpr int kHeadGroup = 4;
__host__ __device__ inline void head_tile(uint32_t item, int ntile, int nheads, int remap,
                                          int per_cu, int& head, int& tile) {
  if (ntile >= 32 * per_cu || (remap && nheads % 8 != 0)) {  // one head at a time
    head = (int)item / ntile;
    tile = (int)item % ntile;
    return;
  }
  int h0 = 0, nh = nheads, it = (int)item;
  if (remap) {  // group within each XCD's eighth of the heads
    nh = nheads / 8;
    const int x = it / (nh * ntile);
    h0 = x * nh;
    it -= x * nh * ntile;
  }
  const int ng = max(1, nh / kHeadGroup);  // groups; the last takes the remainder
  const int span = kHeadGroup * ntile;
  const int grp = min(it / span, ng - 1);
  const int gn = grp == ng - 1 ? nh - grp * kHeadGroup : kHeadGroup;  // heads in this group
  const int idx = it - grp * span;
  tile = idx / gn;
  head = h0 + grp * kHeadGroup + idx % gn;
}

}  // namespace fa
