// fa_launch.h — host-side launchers behind the C ABI (arguments already validated by fa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d, causal;
  float scale;
  void* workspace = nullptr;  // fwd_split_workspace_bytes bytes: allows the key-range split
};

struct Fp8FwdArgs {
  const void* q8;
  const void* k8;
  const void* v8;
  float q_descale, k_descale, v_descale;
  void* o;
  float* lse;
  int B, H, N, d, causal;
  float scale;
  void* workspace = nullptr;  // fwd_split_workspace_bytes bytes: allows the key-range split
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // fp32 [B,H,N] workspace: −D_i, D_i = (dO_i · O_i) · delta_mult
  int B, H, N, d, causal;
  float scale;             // multiplier of the products of q and k as stored (the softmax scale)
  float dk_scale = 0.f;    // dK = dk_scale · Σ_i dS_ij q_i and dQ = dq_scale · Σ_j dS_ij k_j, with
  float dq_scale = 0.f;    // dS computed from v as stored and D; both equal `scale` for bf16 inputs
  float delta_mult = 1.f;  // 1 for bf16 inputs; 1 / v_descale when v holds e4m3 codes
  // Split backward (bwd_split): seg > 0 selects it; the partial sums live in the workspace after D.
  int split_seg = 0;
  float* part_dq = nullptr;
  float* part_dk = nullptr;
  float* part_dv = nullptr;
};

struct DecodeArgs {
  const void* q;  // [B,H,Nq,d] bf16
  const void* k;  // [B,H,Nk,d] bf16
  const void* v;  // [B,H,Nk,d] bf16
  void* o;        // [B,H,Nq,d] bf16
  float* lse;     // [B,H,Nq] fp32
  void* workspace;
  int B, H, Nq, Nk, d, causal;
  float scale;
};

// Whether a grid of `total` work items over `heads` heads uses the XCD-aware order (xcd_remap in
// fa_common.h: consecutive work items, i.e. the tiles of one group of heads (head_tile), on one XCD
// so that they share its L2).  That order hands each XCD a contiguous eighth of the items.  Without
// the causal mask every tile costs the same, so any contiguous eighth is a fair share.  Under the
// mask a head's tiles range from one key tile to all of them.  With fewer heads than XCDs, the
// eighths split single heads, and the XCD holding a head's heaviest tiles gets up to twice its
// share.  Measured at d = 128 (heads taken one at a time): one head of 2^20 keys ran 1.7x faster in
// the plain order (dealt to the XCDs round-robin, which mixes heavy and light tiles on every XCD),
// two heads 1.5x and six heads 1.06-1.15x.  From eight heads on each XCD holds at least one whole
// head's worth: twelve heads ran 8-14% faster in the XCD order (L2 reuse outweighs the residual
// imbalance), 128 heads the same either way.
inline int use_xcd_order(uint32_t total, long heads, int causal) {
  return (total % 8u == 0u && (!causal || heads >= 8)) ? 1 : 0;
}

// Split-KV decomposition of a decode call: S chunks of split_len keys (a multiple of 32; the last
// chunk may be shorter).  Enough chunks for about 2048 workgroups over the device, each chunk at least
// 256 keys long.
struct DecodeSplit {
  int S;
  int split_len;
};
inline DecodeSplit decode_split(int B, int H, int Nq, int Nk) {
  (void)Nq;
  const long bh = (long)B * H;
  long s = (2048 + bh - 1) / bh;
  const long by_len = ((long)Nk + 255) / 256;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  long len = ((long)Nk + s - 1) / s;
  len = (len + 31) / 32 * 32;
  DecodeSplit r;
  r.split_len = (int)len;
  r.S = (int)(((long)Nk + len - 1) / len);
  return r;
}
// Workspace of a decode call: per (batch·head, chunk, query) the unnormalised output (d fp32) and the
// chunk's row maximum and two row sums (3 fp32), rounded up to 256 bytes.
inline size_t decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  const DecodeSplit sp = decode_split(B, H, Nq, Nk);
  return (((size_t)B * H * sp.S * Nq * ((size_t)d + 3) * sizeof(float)) + 255u) & ~(size_t)255u;
}

// Key-range split of the bf16 forward, for grids too small to fill the device (few heads, long
// sequences): every 128-query tile's key tiles are cut into segments of `seg` 64-key tiles, each
// (query tile, segment) pair is one workgroup writing a partial result, and a merge kernel combines a
// row's segments.  nseg = 1 means no split.
// Rule (measured on MI355X, causal, d = 64 and 128, 1–8 heads of 4k–64k keys): with T the key tiles
// summed over all (batch·head, query tile) pairs and kt = ⌈N/64⌉ the longest range, the unsplit grid
// leaves compute units idle when kt exceeds the average work per workgroup slot, T / kSlots (two
// workgroups on each of the 256 compute units).  The split is used when kt ≥ 2.5·T/kSlots, or when
// kt ≥ 1.5·T/kSlots and rows are long (kt ≥ 256 tiles); below that, the partial results' traffic
// (d + 3 fp32 values per row and segment, written and read back) and the shorter workgroups cost
// more than the balance gains (2×4×8192, ratio 2: forward 739 TFLOP/s unsplit, 564–656 split).
// Segments of kt/8 tiles, clamped to 16..128, were within 6% of the best segment length for every
// shape measured (1×1×16384: 261 → 526 TFLOP/s; 1×1×65536: 861 → 1011).  Head dimension 256 (its own
// kernel) is not split.
constexpr long kSlots = 512;
struct FwdSplit {
  int seg;   // key tiles per segment
  int nseg;  // segments of the longest key range
};
inline FwdSplit fwd_split(int B, int H, int N, int d, int causal) {
  FwdSplit r{0, 1};
  if (d > 128) return r;
  const long bh = (long)B * H;
  const long nqt = ((long)N + 127) / 128;
  const long kt = ((long)N + 63) / 64;
  // Key tiles over every (batch·head, query tile).  Causal: query tile qt < nqt − 1 ends its keys at
  // 128(qt + 1), i.e. 2(qt + 1) tiles, and the last one uses all kt, so the sum is (nqt − 1)·nqt + kt.
  const long total = bh * (causal ? (nqt - 1) * nqt + kt : nqt * kt);
  if (2 * kt * kSlots < 3 * total) return r;
  if (2 * kt * kSlots < 5 * total && kt < 256) return r;
  long seg = kt / 8;
  seg = seg < 16 ? 16 : (seg > 128 ? 128 : seg);
  if (seg >= kt) return r;
  r.seg = (int)seg;
  r.nseg = (int)((kt + seg - 1) / seg);
  return r;
}
// Workspace of fa_fwd_split: per (segment, batch·head, query) the unnormalised output (d fp32) and the
// segment's reference maximum and two row sums (3 fp32), rounded up to 256 bytes; 0 without a split.
inline size_t fwd_split_workspace_bytes(int B, int H, int N, int d, int causal) {
  const FwdSplit sp = fwd_split(B, H, N, d, causal);
  if (sp.nseg <= 1) return 0;
  return (((size_t)sp.nseg * B * H * N * ((size_t)d + 3) * sizeof(float)) + 255u) & ~(size_t)255u;
}

// Split backward, for the same grids: the dQ kernel (128-query tiles over 64-key tiles, the forward's
// geometry) splits each tile's key range into fwd_split's segments of `seg` tiles; the dK/dV kernel
// (128-key blocks over 32-query steps) splits each block's query range into segments of 2·seg steps,
// i.e. the same number of rows.  Each segment writes fp32 partial sums; one more kernel adds a row's
// segments, scales and rounds to bf16.
struct BwdSplit {
  int seg;     // 0: no split; else fwd_split's segment length in 64-key tiles
  int nseg_q;  // segments of the longest key range (dQ kernel)
  int nseg_k;  // segments of the longest query range (dK/dV kernel)
};
inline BwdSplit bwd_split(int B, int H, int N, int d, int causal) {
  const FwdSplit f = fwd_split(B, H, N, d, causal);
  if (f.nseg <= 1) return BwdSplit{0, 1, 1};
  const long steps = ((long)N + 31) / 32;
  return BwdSplit{f.seg, f.nseg, (int)((steps + 2L * f.seg - 1) / (2L * f.seg))};
}
inline size_t bwd_split_part_bytes(int nseg, int B, int H, int N, int d) {
  return (((size_t)nseg * B * H * N * (size_t)d * sizeof(float)) + 255u) & ~(size_t)255u;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// Key-range split, second step (both forwards): one wave per (batch·head, query) row combines the row's
// segments (as many as its query tile's key range spans) into O (bf16) and LSE; d ≤ 128.
hipError_t launch_fwd_merge(const float* part_o, const float* part_ml, void* o, float* lse, int bh,
                            int N, int d, int causal, int seg, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
// D into the workspace and dQ: one kernel where the head dimension allows (D formed inside the dQ
// kernel), else launch_bwd_pre then launch_bwd_dq; bit for bit the same results either way.
hipError_t launch_bwd_delta_dq(const BwdArgs& a, hipStream_t stream);
// The whole backward: launch_bwd_delta_dq, then launch_bwd_dkdv.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// n e4m3fn codes (n a multiple of 16, both pointers 16-byte aligned) → n bf16 values equal to the
// codes' values (exact: every e4m3 value is a bf16 value).
hipError_t launch_e4m3_to_bf16(const void* src, void* dst, size_t n, hipStream_t stream);

// Backward workspace: the fp32 [B,H,N] array of −D, rounded up to 256 bytes.
inline size_t round_up_256(size_t x) { return (x + 255u) & ~(size_t)255u; }
inline size_t bwd_delta_bytes(int B, int H, int N) {
  return round_up_256((size_t)B * H * N * sizeof(float));
}
// FP8 backward workspace: D, then bf16 images of the q, k, v codes, each rounded up to 256 bytes.
inline size_t bwd_fp8_image_bytes(int B, int H, int N, int d) {
  return round_up_256((size_t)B * H * N * d * 2u);
}
inline size_t bwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  return bwd_delta_bytes(B, H, N) + 3 * bwd_fp8_image_bytes(B, H, N, d);
}
// Split backward workspace: D, then the dQ partial sums, then the dK and dV partial sums; just D
// when the shape is not split.
inline size_t bwd_split_workspace_bytes(int B, int H, int N, int d, int causal) {
  const BwdSplit sp = bwd_split(B, H, N, d, causal);
  size_t bytes = bwd_delta_bytes(B, H, N);
  if (sp.seg > 0)
    bytes += bwd_split_part_bytes(sp.nseg_q, B, H, N, d) +
             2 * bwd_split_part_bytes(sp.nseg_k, B, H, N, d);
  return bytes;
}

}  // namespace fa
