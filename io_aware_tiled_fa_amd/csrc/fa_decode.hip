// Split-KV attention for decoding: few query rows against a long key
// sequence.
//
// The pages set decoding apart from prompt processing: generating a token
// reads the whole cache of keys and values for a handful of new queries, so
// its cost is memory traffic, and the method's gain there is small ("What Is
// Flash Attention? The Real Speed and Memory Gains, Explained",
// bestllmfor.com, "What you actually gain on a local machine").  The
// forward kernel parallelises over query tiles, which leaves a decode step
// with one workgroup per head and the chip mostly idle.  This path instead
// splits the keys:
//
//  * one workgroup per (batch, key/value head, key split).  Its 32-row query
//    tile packs every query row that reads this key/value head: the
//    H / H_kv query heads of the group times the N_q positions (row
//    r = i (H / H_kv) + g), so each key and value is read from HBM once per
//    group instead of once per query head;
//  * the split's keys stream through LDS in stages of 128 (double buffered,
//    direct global -> LDS copies, the forward kernel's layout); each of the
//    4 waves takes 32 keys of a stage and keeps its own online softmax;
//  * at the end the waves merge through LDS, and the workgroup writes either
//    the final row (one split) or the split's normalised partial output and
//    base-2 log-sum-exp; a second kernel merges the splits of each row with
//    weights exp2(lse_s - max_s lse_s), the same algebra as the online
//    softmax.
// Masks are the forward kernel's bands: key j is visible to query i iff
// i + off - wl <= j <= i + off + wr, off = N_k - N_q.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D, bool BAND, bool WIN, bool SPLIT>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecArgs a) {
  static_assert(BAND || !WIN, "a window always bounds the keys above");
  constexpr int NW = 4;
  constexpr int BS = kDecodeStageKeys;   // keys per stage, 32 per wave
  constexpr int ROWB = D * 2;            // bytes of one key row in LDS
  constexpr int STB = BS * ROWB;         // bytes of one K or V stage
  constexpr int NCH = D / 8;             // 16-byte chunks per row
  constexpr int LPW = STB / 1024 / NW;   // 1 KiB copies per wave per stage (K and V each)
  constexpr int NDB = D / 32;            // 32-wide column blocks of O
  constexpr int NKK = D / 16;            // k-steps of the score product
  static_assert(BS == 32 * NW, "each wave takes 32 keys of a stage");
  static_assert((STB / 1024) % NW == 0, "stage copies must split evenly over waves");
  static_assert((64 + D * 32) * 4 <= STB, "a wave's merge record must fit one stage buffer");
  __shared__ __attribute__((aligned(1024))) char k_lds0[STB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[STB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[STB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[STB];

  // ---- workgroup -> (batch, key head, split)
  const int split = blockIdx.x % a.nsplit;
  const int bh = blockIdx.x / a.nsplit;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const int G = a.G;
  // this lane's row of the packed tile: position qi, query head hq
  const bool row_valid = l32 < G * a.Nq;
  const int qi = row_valid ? l32 / G : 0;
  const int hq = hk * G + (row_valid ? l32 - qi * G : 0);
  const int hi_off = a.Nk - a.Nq + a.wr;
  const int lo_off = a.Nk - a.Nq - a.wl;
  const size_t rs = (size_t)a.H * D;    // Q / O row stride
  const size_t rk = (size_t)a.Hkv * D;  // K / V row stride

  // ---- the packed query rows as B operands (lane: row l32, d = 16 kk + 8 h2 ..)
  bf16x8 qop[NKK];
  if (row_valid) {
    const __bf16* qp = a.q + ((size_t)b * a.Nq + qi) * rs + (size_t)hq * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[kk] = *(const bf16x8*)(qp + 16 * kk);
    if (a.negate) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 t = __builtin_bit_cast(u32x4, qop[kk]) ^ 0x80008000u;
        qop[kk] = __builtin_bit_cast(bf16x8, t);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[kk] = bf16x8{};
  }

  // ---- LDS read offsets within a wave's 32 keys (stages in the row-group
  // layout of fa_device.h, as in the forward kernel)
  int krb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) krb[par] = rg_row_base<D>(l, par);
  auto koff = [&](int kk) __attribute__((always_inline)) { return krb[kk & 1] + 256 * (kk >> 1); };
  int vrb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) vrb[r] = rg_tr_base<D>(l, r);
  // direct copies: wave copy c = w + NW i fills bytes [1024 c, 1024 c + 1024)
  // of a stage, lane l the 16-byte slot 64 c + l; copy i reads RSTEP i rows
  // below copy 0, a multiple of 16 (where the layout repeats), so one
  // per-lane offset serves all copies
  constexpr int RSTEP = 64 * NW / NCH;
  static_assert(RSTEP % 16 == 0, "copies of a wave must keep the row-group layout");
  uint32_t goff;
  {
    int row, piece;
    rg_slot<D>(64 * w + l, row, piece);
    goff = (uint32_t)(row * (int)rk + piece * 8) * 2u;
  }
  // K and V of this (batch, key head): rows 0 .. N_k - 1 at a stride of
  // H_kv d.  Each copy rebases its resource at the rows it starts from, so
  // its per-lane offset goff is all the range check sees: rows past N_k read
  // zero.  Offsets stay under 2^32 bytes (the host requires
  // (N_k + 128) H_kv d < 2^31).
  const size_t kv_off = (size_t)b * a.Nk * rk + (size_t)hk * D;
  const uint32_t head_bytes = (uint32_t)(((size_t)a.Nk * a.Hkv - hk) * D * 2);
  const __bf16* kbase = a.k + kv_off;
  const __bf16* vbase = a.v + kv_off;
  auto issue_stage = [&](int st, lds_char* kdst, lds_char* vdst) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)st * (uint32_t)(BS * rk * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = w + NW * i;
      const uint32_t off = toff + (uint32_t)(i * RSTEP) * (uint32_t)(rk * 2);
      copy16_to_lds_buf(make_rsrc_at(kbase, head_bytes, off), goff, (lds_void*)(kdst + c * 1024));
      copy16_to_lds_buf(make_rsrc_at(vbase, head_bytes, off), goff, (lds_void*)(vdst + c * 1024));
    }
  };

  // ---- this split's stages: the stages holding a key some row sees, cut
  // into nsplit runs of equal length
  int klast = a.Nk - 1, kfirst = 0;
  if (BAND) klast = min(klast, a.Nq - 1 + hi_off);
  if (WIN) kfirst = max(0, lo_off);
  const int st_lo = kfirst / BS;
  const int nst = klast < kfirst ? 0 : klast / BS - st_lo + 1;
  const int sps = (nst + a.nsplit - 1) / a.nsplit;
  const int s0 = st_lo + split * sps;
  const int s1 = st_lo + min(nst, (split + 1) * sps);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -__builtin_inff();  // running max, base-2 scaled units
  float l_run = 0.f;                // this lane's half of the running sum
  const float c = a.c;

  // the wave's 32 keys k0 .. k0 + 31 of a stage in LDS
  auto compute = [&](auto MASK, int k0, const lds_char* kt, const lds_char* vt) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(MASK)::value;
    bf16x8 kop[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kop[kk] = lds_read16(kt + koff(kk));
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sacc = mfma32(kop[kk], qop[kk], sacc);
    if constexpr (MASKED) {
      // key outside [qi + lo_off, qi + hi_off], or key >= N_k (read as zero)
      const int hi = BAND ? min(qi + hi_off, a.Nk - 1) : a.Nk - 1;
      const int lo = qi + lo_off;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * h2 + (e & 3);
        const bool out = WIN ? (key > hi || key < lo) : key > hi;
        sacc[e] = out ? -__builtin_inff() : sacc[e];
      }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    mx = max_cross_half(mx);
    const float mblk = (mx == -__builtin_inff()) ? mx : mx * c;
    const float mnew = fmaxf(m_run, mblk);
    const bool need = mnew > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_run - mnew) : 1.0f;
      if (need) m_run = mnew;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      l_run *= alpha;
    }
    // only a masked block can leave a row without a key so far
    const float negm = (MASKED && m_run == -__builtin_inff()) ? 0.f : -m_run;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(fmaf(sacc[e], c, negm));
      const float p1 = fast_exp2(fmaf(sacc[e + 1], c, negm));
      l_run += p0 + p1;
      pk[e >> 1] = pack_bf16x2(p0, p1);
    }
    // O^T += V^T P^T over the 32 keys, 16 at a time
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pop = __builtin_bit_cast(bf16x8, u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]});
      bf16x8 vop[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x4 v0 = lds_read_tr16(vt + 16 * t * ROWB + 256 * db + vrb[0]);
        const bf16x4 v1 = lds_read_tr16(vt + 16 * t * ROWB + 256 * db + vrb[1]);
        vop[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(vop[db], pop, oacc[db]);
    }
  };

  // one stage: wait for its copies, start the next stage's copies into the
  // other buffers, then compute this wave's 32 keys
  auto stage_step = [&](int st, const lds_char* kcur, const lds_char* vcur, lds_char* knext,
                        lds_char* vnext) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (st + 1 < s1) issue_stage(st + 1, knext, vnext);
    const int k0 = st * BS + 32 * w;
    // keys past every row's band, or past N_k
    if ((BAND && k0 > a.Nq - 1 + hi_off) || (WIN && k0 + 31 < lo_off) || k0 >= a.Nk) return;
    const lds_char* kt = kcur + 32 * w * ROWB;
    const lds_char* vt = vcur + 32 * w * ROWB;
    if ((BAND && k0 + 31 > hi_off) || (WIN && k0 < a.Nq - 1 + lo_off) || k0 + 32 > a.Nk)
      compute(std::true_type{}, k0, kt, vt);
    else
      compute(std::false_type{}, k0, kt, vt);
  };

  lds_char* K0 = (lds_char*)k_lds0;
  lds_char* K1 = (lds_char*)k_lds1;
  lds_char* V0 = (lds_char*)v_lds0;
  lds_char* V1 = (lds_char*)v_lds1;
  if (s0 < s1) issue_stage(s0, K0, V0);
  for (int st = s0; st < s1; st += 2) {
    stage_step(st, K0, V0, K1, V1);
    if (st + 1 < s1) stage_step(st + 1, K1, V1, K0, V0);
  }

  // ---- merge the four waves through LDS.  Wave w's record (m, l and O^T
  // of its keys, float32) goes to one stage buffer: [0, 32) m, [32, 64) l,
  // then O^T[d][row] at 64 + 32 d + row.
  __syncthreads();  // every wave is done reading the stage buffers
  float* rec[NW] = {(float*)k_lds0, (float*)k_lds1, (float*)v_lds0, (float*)v_lds1};
  {
    float* mine = w == 0 ? (float*)k_lds0 : w == 1 ? (float*)k_lds1 : w == 2 ? (float*)v_lds0 : (float*)v_lds1;
    const float lt = sum_cross_half(l_run);
    if (h2 == 0) {
      mine[l32] = m_run;
      mine[32 + l32] = lt;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = 32 * db + 8 * (e >> 2) + 4 * h2 + (e & 3);
        mine[64 + 32 * d + l32] = oacc[db][e];
      }
  }
  __syncthreads();
  if (w >= NDB || !row_valid) return;
  // wave w finishes the 32 columns d = 32 w .. 32 w + 31 of every row
  float mw[NW], M = -__builtin_inff();
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    mw[v] = rec[v][l32];
    M = fmaxf(M, mw[v]);
  }
  float L = 0.f, f[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    f[v] = mw[v] == -__builtin_inff() ? 0.f : fast_exp2(mw[v] - M);
    L += f[v] * rec[v][32 + l32];
  }
  const float inv = L > 0.f ? fast_rcp(L) : 0.f;
  float ov[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int d = 32 * w + 8 * (e >> 2) + 4 * h2 + (e & 3);
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s = fmaf(f[v], rec[v][64 + 32 * d + l32], s);
    ov[e] = s * inv;
  }
  const size_t row = ((size_t)b * a.H + hq) * a.Nq + qi;  // LSE order (b, hq, i)
  const float lse2 = L > 0.f ? M + fast_log2(L) : -__builtin_inff();
  if constexpr (SPLIT) {
    // the split's normalised output and base-2 log-sum-exp (scaled units)
    float* op = a.part + ((size_t)split * a.B * a.H * a.Nq + row) * D;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * w + 8 * g4 + 4 * h2;
      *(f32x4*)(op + d0) = f32x4{ov[4 * g4], ov[4 * g4 + 1], ov[4 * g4 + 2], ov[4 * g4 + 3]};
    }
    if (w == 0 && h2 == 0) a.part_lse[(size_t)split * a.B * a.H * a.Nq + row] = lse2;
  } else {
    __bf16* orow = a.o + ((size_t)b * a.Nq + qi) * rs + (size_t)hq * D;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * w + 8 * g4 + 4 * h2;
      *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(ov[4 * g4], ov[4 * g4 + 1]), pack_bf16x2(ov[4 * g4 + 2], ov[4 * g4 + 3])};
    }
    if (w == 0 && h2 == 0) a.lse[row] = L > 0.f ? lse2 * kLn2 : -__builtin_inff();
  }
}

// Merge the splits of each row: lse = log2 sum_s 2^{lse_s},
// O = sum_s 2^{lse_s - lse} O_s.  One wave per row (LSE order), each lane
// holding D / 64 columns.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  constexpr int PL = D / 64;  // columns per lane
  const long rows = (long)a.B * a.H * a.Nq;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  float M = -__builtin_inff();
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_lse[(size_t)s * rows + row]);
  float acc[PL] = {};
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < a.nsplit; ++s) {
      const float ls = a.part_lse[(size_t)s * rows + row];
      if (ls == -__builtin_inff()) continue;  // a split without a visible key
      const float f = fast_exp2(ls - M);
      L += f;
      const float* op = a.part + ((size_t)s * rows + row) * D + PL * l;
#pragma unroll
      for (int j = 0; j < PL; ++j) acc[j] = fmaf(f, op[j], acc[j]);
    }
  }
  const float inv = L > 0.f ? fast_rcp(L) : 0.f;
  // row = (b H + hq) N_q + i
  const int i = (int)(row % a.Nq);
  const long bhq = row / a.Nq;
  const int hq = (int)(bhq % a.H);
  const int b = (int)(bhq / a.H);
  __bf16* orow = a.o + ((size_t)b * a.Nq + i) * a.H * D + (size_t)hq * D + PL * l;
  if constexpr (PL == 2) {
    *(uint32_t*)orow = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    orow[0] = (__bf16)(acc[0] * inv);
  }
  if (l == 0) a.lse[row] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -__builtin_inff();
}

template <int D, bool BAND, bool WIN>
static hipError_t launch_decode_t(const DecArgs& a, hipStream_t stream) {
  void* args[] = {(void*)&a};
  const dim3 grid((unsigned)(a.B * a.Hkv * a.nsplit));
  if (a.nsplit == 1)
    return hipLaunchKernel((const void*)decode_kernel<D, BAND, WIN, false>, grid, dim3(256), args, 0, stream);
  hipError_t e = hipLaunchKernel((const void*)decode_kernel<D, BAND, WIN, true>, grid, dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const long rows = (long)a.B * a.H * a.Nq;
  return hipLaunchKernel((const void*)decode_combine_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), args,
                         0, stream);
}

template <int D>
static hipError_t launch_decode_d(const DecArgs& a, bool band, bool win, hipStream_t stream) {
  if (win) return launch_decode_t<D, true, true>(a, stream);
  return band ? launch_decode_t<D, true, false>(a, stream) : launch_decode_t<D, false, false>(a, stream);
}

hipError_t launch_decode(const DecArgs& a, int d, bool band, bool win, hipStream_t stream) {
  return d == 128 ? launch_decode_d<128>(a, band, win, stream) : launch_decode_d<64>(a, band, win, stream);
}

}  // namespace fa
