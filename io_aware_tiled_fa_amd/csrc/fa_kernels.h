// Host-visible argument blocks and launchers of the attention kernels
// (internal to libfa.so; the public interface is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Key j is visible to query i iff  i + off - wl <= j <= i + off + wr, with
// off = Nk - Nq (keys aligned to the end of the queries).  Unbounded sides
// carry a width of at least Nq + Nk + 64, which no row can reach.  Query
// head h reads key / value head h / G.
struct FwdArgs {
  const __bf16* q;   // [B, Nq, H, d]
  const __bf16* k;   // [B, Nk, Hkv, d]
  const __bf16* v;   // [B, Nk, Hkv, d]
  __bf16* o;         // [B, Nq, H, d]
  float* lse;        // [B, H, Nq]
  int B, H, Hkv, G, Nq, Nk;
  int wl, wr;  // band widths below and above the (shifted) diagonal
  float c;     // |scale| * log2(e): scores are used in base-2 units
  int negate;  // scale < 0: the query is negated in registers instead
};

struct BwdArgs {
  const __bf16* q;    // [B, Nq, H, d], like o, dO, dq
  const __bf16* k;    // [B, Nk, Hkv, d], like v, dk, dv
  const __bf16* v;
  const __bf16* o;
  const float* lse;   // [B, H, Nq]
  const __bf16* dO;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* drow;   // [B, H, Nq] row term -sum_c dO * O, then [B, H, Nq] -L log2(e)
  int B, H, Hkv, G, Nq, Nk;
  int wl, wr;    // band widths, as in FwdArgs
  float scale;   // signed softmax scale
  float c;       // scale * log2(e) (signed)
};

// Split-KV decoding: one workgroup per (batch, key head, split) over a
// query tile packing the H / H_kv query heads times N_q positions of the
// group (at most 32 rows).
constexpr int kDecodeStageKeys = 128;  // keys per pipeline stage
constexpr int kDecodeMaxRows = 32;     // (H / H_kv) N_q at most this
struct DecArgs {
  const __bf16* q;   // [B, Nq, H, d]
  const __bf16* k;   // [B, Nk, Hkv, d]
  const __bf16* v;
  __bf16* o;         // [B, Nq, H, d]
  float* lse;        // [B, H, Nq]
  float* part;       // [nsplit, B, H, Nq, d] normalised partial outputs (nsplit > 1)
  float* part_lse;   // [nsplit, B, H, Nq] their base-2 log-sum-exp, scaled units
  int B, H, Hkv, G, Nq, Nk;
  int wl, wr;        // band widths, as in FwdArgs
  int nsplit;
  float c;           // |scale| * log2(e)
  int negate;        // scale < 0
};

// band: the visible keys have an upper edge (causal, or a window); without
// one every key is visible and the kernels run their unmasked walk.  win:
// they also have a lower edge (a window).
hipError_t launch_fwd(const FwdArgs& a, int d, bool band, bool win, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int d, bool band, bool win, hipStream_t stream);
hipError_t launch_decode(const DecArgs& a, int d, bool band, bool win, hipStream_t stream);

}  // namespace fa
