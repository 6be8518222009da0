// Host-visible argument blocks and launchers of the attention kernels
// (internal to libfa.so; the public interface is include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const __bf16* q;   // [B, Nq, H, d]
  const __bf16* k;   // [B, Nk, H, d]
  const __bf16* v;   // [B, Nk, H, d]
  __bf16* o;         // [B, Nq, H, d]
  float* lse;        // [B, H, Nq]
  int B, H, Nq, Nk;
  float c;     // |scale| * log2(e): scores are used in base-2 units
  int negate;  // scale < 0: the query is negated in registers instead
};

struct BwdArgs {
  const __bf16* q;    // [B, Nq, H, d], like o, dO, dq
  const __bf16* k;    // [B, Nk, H, d], like v, dk, dv
  const __bf16* v;
  const __bf16* o;
  const float* lse;   // [B, H, Nq]
  const __bf16* dO;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* drow;   // [B, H, Nq] row term -sum_c dO * O, then [B, H, Nq] -L log2(e)
  int B, H, Nq, Nk;
  float scale;   // signed softmax scale
  float c;       // scale * log2(e) (signed)
};

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t stream);

}  // namespace fa
