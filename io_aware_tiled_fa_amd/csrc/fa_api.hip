// C ABI of libfa.so (declared in include/fa.h): argument validation, the
// backward workspace layout, and dispatch to the gfx950 kernels.
//
// Shape checks mirror the ones the holysheep.ai review prints for its
// interface ("Common Errors and Fixes", Error 4: four-dimensional
// [batch, seq_len, num_heads, head_dim] tensors with matching batch, heads
// and head_dim, and equal K / V lengths, while the query length may differ);
// here Q, O, dO share one shape and K, V another, so they reduce to positive
// B, H, H_kv, N_q, N_k, H a multiple of H_kv, and a supported d.  The same page
// ("Common Errors and Fixes", Error 1) notes that a launch fails when a
// tile exceeds device limits; here unsupported sizes are refused before
// anything is launched.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // fa_bwd_noalloc: B H N_q <= 2^21 rows
constexpr int kMaxScratchDevices = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Sizes: B, H, H_kv, N_q, N_k >= 1, H a multiple of H_kv, d in {64, 128},
// and every tensor under 2^31 elements (the kernels index in 32-bit element
// offsets within a tensor).  The tile copies address one batch's rows of a
// head in 32-bit byte offsets that run up to 128 rows past its last row
// (those read zero), so (N + 128) rows of a batch must also stay under 2^31
// elements.
fa_status check_shape(int B, int H, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  const long long lim = 0x7FFFFFFFLL;
  if ((long long)B * Nq * H * d > lim || (long long)B * Nk * Hkv * d > lim) return FA_ERR_SHAPE;
  if (((long long)Nq + 128) * H * d > lim || ((long long)Nk + 128) * Hkv * d > lim) return FA_ERR_SHAPE;
  return FA_OK;
}

// The visible band of query i: keys i + off - wl .. i + off + wr, off =
// N_k - N_q.  An unbounded side gets N_q + N_k + 64, past every key of every
// row; with N_q, N_k < 2^26 (each tensor < 2^31 elements, d >= 64) no sum
// of these overflows an int.  Returns whether the band has an upper edge.
bool band_of(int Nq, int Nk, int causal, int window, int& wl, int& wr) {
  const int big = Nq + Nk + 64;
  const int w = window > 0 ? (window - 1 < big ? window - 1 : big) : big;
  wl = w;
  wr = causal ? 0 : w;
  return causal || window > 0;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Split-KV decoding.  The packed query tile holds (H / H_kv) N_q rows; above
// kDecodeMaxRows the general forward kernel runs instead.
bool decode_packs(int H, int Hkv, int Nq) { return (long long)(H / Hkv) * Nq <= fa::kDecodeMaxRows; }

// Key stages of 128 that hold a key some query row sees.
int decode_stages(int Nq, int Nk, int wl, int wr, bool band, bool win) {
  const int hi_off = Nk - Nq + wr, lo_off = Nk - Nq - wl;
  const int klast = band ? (Nk - 1 < Nq - 1 + hi_off ? Nk - 1 : Nq - 1 + hi_off) : Nk - 1;
  const int kfirst = win ? (lo_off > 0 ? lo_off : 0) : 0;
  if (klast < kfirst) return 0;
  return klast / fa::kDecodeStageKeys - kfirst / fa::kDecodeStageKeys + 1;
}

// Splits per (batch, key head): the caller's number if given.  Otherwise
// one round of workgroups on a 256-CU MI355X (the d = 128 kernel holds
// 128 KiB of LDS, one workgroup per CU; d = 64 half that, two per CU), but
// at least 4 stages of keys per split, since a short split spends most of
// its time waiting for its first stage.  Never more splits than stages.
int decode_splits(int B, int Hkv, int d, int nst, int requested) {
  const long long units = (long long)B * Hkv;
  const long long slots = d == 128 ? 256 : 512;
  long long want = requested > 0 ? requested : (slots + units - 1) / units;
  if (requested <= 0 && want > nst / 4) want = nst / 4;
  if (want > nst) want = nst;
  if (want > 256) want = 256;
  return want < 1 ? 1 : (int)want;
}

// Arguments of the backward other than its workspace: pointers, sizes,
// alignment, scale and flags, and no output overlapping an input or another
// output.
fa_status bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int d,
                    float scale, int causal, int window) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  const void* all[] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : all)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((causal != 0 && causal != 1) || window < 0) return FA_ERR_ARG;
  const size_t qb = (size_t)B * Nq * H * d * 2, kb = (size_t)B * Nk * Hkv * d * 2, lb = (size_t)B * H * Nq * 4;
  const void* ins[6] = {q, k, v, o, dO, lse};
  const size_t insz[6] = {qb, kb, kb, qb, qb, lb};
  void* outs[3] = {dq, dk, dv};
  const size_t outsz[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ARG;
  }
  return FA_OK;
}

// Launch the backward kernels with `drow` (2 B H N_q floats) for the row terms.
fa_status bwd_launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, int window, float* drow, void* stream) {
  fa::BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.lse = lse;
  a.dO = static_cast<const __bf16*>(dO);
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.drow = drow;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  const bool band = band_of(Nq, Nk, causal, window, a.wl, a.wr);
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  const hipError_t e = fa::launch_bwd(a, d, band, window > 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

// Scratch memory of fa_bwd_noalloc, for callers that cannot allocate: the
// backward's two float32 row terms per query row live here instead of in a
// caller's workspace.  One copy per GPU, held until the process ends; in
// host code the name stands for the host-side shadow, so its device
// address is looked up once per device and only that address is used.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex scratch_mutex;
float* scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device, or nullptr.
float* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = static_cast<float*>(p);
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H, H_kv, N_q and N_k must be positive, H a multiple of H_kv, every tensor must have fewer than 2^31 elements, and so must (N_q + 128) H d and (N_k + 128) H_kv d";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_SEQLEN: return "sequence length not supported";
    case FA_ERR_ALIGN: return "tensor base pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than fa_bwd_workspace_size()";
    case FA_ERR_SCALE: return "scale must be a finite float";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ARG: return "causal must be 0 or 1, window and num_splits must not be negative, outputs must not overlap inputs, and the stream must belong to the current device";
    case FA_ERR_SCRATCH: return "fa_bwd_noalloc holds at most 2^21 query rows (B * H * N_q) in its static scratch";
  }
  return "unknown status";
}

int fa_version(void) { return 300; }

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                    void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((causal != 0 && causal != 1) || window < 0) return FA_ERR_ARG;
  const size_t qb = (size_t)B * Nq * H * d * 2, kb = (size_t)B * Nk * Hkv * d * 2, lb = (size_t)B * H * Nq * 4;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(o, qb, ins[i], insz[i]) || overlaps(lse, lb, ins[i], insz[i])) return FA_ERR_ARG;
  if (overlaps(o, qb, lse, lb)) return FA_ERR_ARG;

  fa::FwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  const bool band = band_of(Nq, Nk, causal, window, a.wl, a.wr);
  // scores enter the kernel as s * c in base 2.  c is kept away from 0: a
  // masked score (-inf) times c must stay -inf, and with scale == 0 a c of
  // 1e-30 leaves every finite s * c within 1e-24 of 0, where exp2 rounds to
  // exactly 1 in float32, as for c = 0.
  a.c = fmaxf(fabsf(scale) * 1.4426950408889634f, 1e-30f);
  a.negate = scale < 0.f;
  const hipError_t e = fa::launch_fwd(a, d, band, window > 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, int window,
                                 int num_splits) {
  if (check_shape(B, H, Hkv, Nq, Nk, d) != FA_OK || causal < 0 || causal > 1 || window < 0 || num_splits < 0)
    return 0;
  if (!decode_packs(H, Hkv, Nq)) return 0;
  int wl, wr;
  const bool band = band_of(Nq, Nk, causal, window, wl, wr);
  const int ns = decode_splits(B, Hkv, d, decode_stages(Nq, Nk, wl, wr, band, window > 0), num_splits);
  if (ns == 1) return 0;
  return round256((size_t)ns * B * H * Nq * (d + 1) * sizeof(float));
}

fa_status fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                        int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((causal != 0 && causal != 1) || window < 0 || num_splits < 0) return FA_ERR_ARG;
  const size_t need = fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d, causal, window, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
    return FA_ERR_WORKSPACE;
  const size_t qb = (size_t)B * Nq * H * d * 2, kb = (size_t)B * Nk * Hkv * d * 2, lb = (size_t)B * H * Nq * 4;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, kb, kb};
  void* outs[3] = {o, lse, workspace};
  const size_t outsz[3] = {qb, lb, need};
  for (int i = 0; i < 3; ++i) {
    if (outsz[i] == 0) continue;
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (outsz[j] && overlaps(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ARG;
  }
  if (!decode_packs(H, Hkv, Nq))  // too many rows per key head to pack: the general forward
    return fa_fwd_ex(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, stream);

  fa::DecArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  const bool band = band_of(Nq, Nk, causal, window, a.wl, a.wr);
  a.nsplit = decode_splits(B, Hkv, d, decode_stages(Nq, Nk, a.wl, a.wr, band, window > 0), num_splits);
  const size_t rows = (size_t)B * H * Nq;
  a.part = a.nsplit > 1 ? static_cast<float*>(workspace) : nullptr;
  a.part_lse = a.nsplit > 1 ? static_cast<float*>(workspace) + (size_t)a.nsplit * rows * d : nullptr;
  a.c = fmaxf(fabsf(scale) * 1.4426950408889634f, 1e-30f);  // as in the forward
  a.negate = scale < 0.f;
  const hipError_t e = fa::launch_decode(a, d, band, window > 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, 0, stream);
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, N, N, d, scale, causal, 0, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (check_shape(B, H, 1, N, 1, d) != FA_OK) return 0;
  return round256(2 * (size_t)B * H * N * sizeof(float));
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                    void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = bwd_check(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal, window);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_size(B, H, Nq, d);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return FA_ERR_WORKSPACE;
  const size_t qb = (size_t)B * Nq * H * d * 2, kb = (size_t)B * Nk * Hkv * d * 2, lb = (size_t)B * H * Nq * 4;
  const void* others[9] = {q, k, v, o, dO, lse, dq, dk, dv};
  const size_t othersz[9] = {qb, kb, kb, qb, qb, lb, qb, kb, kb};
  for (int j = 0; j < 9; ++j)
    if (overlaps(workspace, need, others[j], othersz[j])) return FA_ERR_ARG;
  return bwd_launch(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal, window,
                    static_cast<float*>(workspace), stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk, void* dv,
                         int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                         void* stream) {
  fa_status st = bwd_check(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal, window);
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_size(B, H, Nq, d) > kScratchBytes) return FA_ERR_SCRATCH;
  // the scratch array of the stream's device, which must be the current one
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return FA_ERR_LAUNCH;
  if (dev != cur) return FA_ERR_ARG;
  float* rows = scratch_of_current_device();
  if (!rows) return FA_ERR_LAUNCH;
  return bwd_launch(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal, window, rows, stream);
}

fa_status fa_bwd_qk(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, B, H, H, Nq, Nk, d, scale, causal, 0, workspace,
                   workspace_bytes, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, B, H, H, N, N, d, scale, causal, 0, workspace,
                   workspace_bytes, stream);
}

}  // extern "C"
