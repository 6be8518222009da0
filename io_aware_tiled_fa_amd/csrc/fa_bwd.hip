// Backward attention kernels for gfx950: dQ, dK, dV of O = softmax(scale
// Q K^T) V by recomputation.
//
// The pages say only that the backward pass does not keep the attention
// matrix but recomputes it tile by tile from the saved Q, K, V ("Flash
// Attention Explained", institutepm.com, "Recompute during backward pass";
// "What Is Flash Attention?", bestllmfor.com, "How Flash Attention works",
// recomputation bullet).  The gradient formulas follow from differentiating
// the row softmax (written out in the fp64 oracle); with the forward's
// per-row log-sum-exp L_i the probabilities come back exactly as
// P_ij = exp(s_ij - L_i), and the softmax Jacobian term sum_j P_ij dP_ij
// equals D_i = sum_c dO_ic O_ic, so no row of P is ever needed whole.
//
// Three kernels on one stream:
//  1. bwd_pre: D_i = dO_i . O_i and -L_i log2(e) per row (float32), and the
//     float32 dQ accumulator cleared;
//  2. bwd_main: one workgroup per 128-key block of one (batch, head); each
//     of its 4 waves keeps 32 keys of K and V in registers and their dK, dV
//     in float32 accumulators (AGPRs), and walks the query blocks (64 rows
//     each, all of them, or those at or after the diagonal when causal)
//     staged through LDS with double-buffered direct copies.  Per query
//     block and wave:
//        S  = Q K^T,  P = exp2(S scale log2e - L log2e)   (masked on the diagonal)
//        dV += P^T dO
//        dP = dO V^T, dS = P (dP - D)
//        dK += dS^T Q
//     then dS (bf16) goes to LDS and the waves split dQ_blk = dS K over the
//     output columns and add it into the float32 accumulator atomically;
//  3. bwd_dq: dQ = scale * accumulator, rounded to bf16.
// All products run on v_mfma_f32_32x32x16_bf16 in the "S layout": lane l
// holds 16 queries of key l % 32, which is directly the A operand of the
// dV and dK products; the dO and Q tiles feed the B operand through
// transpose reads, exactly as V does in the forward kernel.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ---------------------------------------------------------------------------
// 1. row terms and accumulator clear.  One 16-lane group per (b, n, h) row for
//    d = 128 (8-lane for d = 64); 256 threads per block.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;            // lanes per row, 8 bf16 each
  constexpr int RPB = 256 / LPR;        // rows per block
  const int t = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + t / LPR;  // index over (b, n, h)
  const int sub = t % LPR;
  const long nrows = (long)a.B * a.N * a.H;
  float acc = 0.f;
  if (row < nrows) {
    const size_t off = (size_t)row * D + 8 * sub;
    const u32x4 ov = *(const u32x4*)(a.o + off);
    const u32x4 gv = *(const u32x4*)(a.dO + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o0 = __builtin_bit_cast(float, ov[i] << 16), o1 = __builtin_bit_cast(float, ov[i] & 0xFFFF0000u);
      const float g0 = __builtin_bit_cast(float, gv[i] << 16), g1 = __builtin_bit_cast(float, gv[i] & 0xFFFF0000u);
      acc = fmaf(o0, g0, acc);
      acc = fmaf(o1, g1, acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < nrows && sub == 0) {
    const int h = (int)(row % a.H);
    const long bn = row / a.H;
    const int n = (int)(bn % a.N);
    const int b = (int)(bn / a.N);
    const size_t r = ((size_t)b * a.H + h) * a.N + n;
    a.drow[r] = acc;
    a.drow[(size_t)a.B * a.H * a.N + r] = -a.lse[r] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. main kernel: one workgroup of 8 waves per 128-key block, walking the
//    query blocks of 64 rows.  Wave w = kg + 4 dh (waves w and w + 4 share a
//    SIMD): key group kg owns keys 32 kg .. 32 kg + 31 of the block, and dh
//    picks both the 32-row query half whose scores the wave computes and the
//    half of the d columns of dK and dV it accumulates.  Per query block:
//      S, dP for (key group, query half)       8 + 8 products (k = d)
//      P, dS -> LDS (bf16, [key][query])
//      dQ block (query half, 32 columns) = dS K, added atomically
//      dV, dK (key group, d half) over all 64 queries: the own half's P and
//      dS from registers, the partner wave's from LDS
//    With two waves per SIMD, one wave's softmax runs beside the other's
//    matrix products.
//
// P^T / dS^T tiles: 128 key rows of 64 queries (128 B), stored in 8-byte
// chunks of 4 queries with chunk c of row r at c ^ f(r), f(r) = 8 r1 + (r >> 2
// & 7): conflict-free for the 32-row chunk writes and reads of a key group
// and for the transpose reads of the dQ product.
__device__ __forceinline__ int pt_off(int row, int q) {
  const int f = (((row >> 1) & 1) << 3) | ((row >> 2) & 7);
  return row * 128 + (((q >> 2) ^ f) << 3) + 2 * (q & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_main_kernel(BwdArgs a) {
  constexpr int NW = 8;
  constexpr int BC = 128;              // keys per workgroup (4 groups of 32)
  constexpr int BR = 64;               // queries per step (2 halves of 32)
  constexpr int ROWB = D * 2;          // bytes per row of a Q / dO / K tile
  constexpr int QTILEB = BR * ROWB;    // Q or dO tile
  constexpr int PTB = BC * BR * 2;     // P^T or dS^T tile
  constexpr int NCH = D / 8;
  constexpr int NKK = D / 16;          // k-steps over d
  constexpr int NDB = D / 32;          // 32-wide column blocks over d
  constexpr int NDH = NDB / 2;         // column blocks of dK, dV per wave
  constexpr int QLPW = QTILEB / 1024 / NW;
  static_assert(QLPW >= 1 && NDH >= 1, "tile copies must split evenly over waves");
  __shared__ __attribute__((aligned(1024))) char q_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char q_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char p_lds[PTB];
  __shared__ __attribute__((aligned(1024))) char ds_lds[PTB];
  // row terms of a query block: -L log2(e) of its 64 rows, then their D
  __shared__ __attribute__((aligned(256))) float r_lds0[2 * BR];
  __shared__ __attribute__((aligned(256))) float r_lds1[2 * BR];
  lds_char* const ptile = (lds_char*)p_lds;
  lds_char* const dstile = (lds_char*)ds_lds;

  const int nbh = a.B * a.H;
  const int wg = blockIdx.x;
  int bh, kblk;
  if ((nbh & 7) == 0) {
    // workgroups are dealt round-robin over the 8 XCDs: give each XCD a
    // contiguous range of heads, so one head's key blocks share an L2
    const int hpx = nbh >> 3;
    const int x = wg & 7, s = wg >> 3;
    bh = x * hpx + s % hpx;
    kblk = s / hpx;  // causal: low key blocks see the most query blocks, so they go first
  } else {
    bh = wg % nbh;
    kblk = wg / nbh;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const int kg = w & 3, dh = w >> 2;
  const int kb = kblk * BC;
  const int kw = kb + 32 * kg;  // first key of this wave
  // N is a multiple of 64, so the last key block may hold only 64 keys:
  // key groups past the end compute nothing and leave P = dS = 0
  const bool wave_active = kw < a.N;

  const size_t rs = (size_t)a.H * D;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * D;
  const size_t rowterm_off = ((size_t)b * a.H + h) * a.N;
  const float* drow = a.drow + rowterm_off;
  const float* nlse2 = a.drow + (size_t)a.B * a.H * a.N + rowterm_off;

  // ---- the key group's keys and values as B operands: lane = key l32, d = 16 kk + 8 h2 ..
  bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kreg[kk] = vreg[kk] = bf16x8{};
  if (wave_active) {
    const __bf16* kr = a.k + head_off + (size_t)(kw + l32) * rs + 8 * h2;
    const __bf16* vr = a.v + head_off + (size_t)(kw + l32) * rs + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kreg[kk] = *(const bf16x8*)(kr + 16 * kk);
      vreg[kk] = *(const bf16x8*)(vr + 16 * kk);
    }
  }

  // ---- per-lane LDS offsets.  Q / dO tiles use the forward kernel's
  // geometry; the swizzle XORs the chunk index, so a power-of-two chunk step
  // is an XOR of the offset.
  // row reads (A operand, lane = row l32 of the wave's query half, chunk 2 kk + h2)
  const int roff = dh * 32 * ROWB + l32 * ROWB + ((chunk_swizzle<D>(l32) ^ h2) << 4);
  // transpose reads: rows 4 h2 + j/4 (+8) of a 16-row step, cols 16 (g&1) + 4 (j&3) of a 32-col block
  int troff0[2];
  {
    const int g = l >> 4, j = l & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 4 * h2 + (j >> 2) + 8 * r;
      const int ch = 2 * (g & 1) + ((j & 3) >> 1);
      troff0[r] = row * ROWB + ((ch ^ chunk_swizzle<D>(row)) << 4) + 8 * (j & 1);
    }
  }
  // P^T / dS^T chunk of this lane: key row 32 kg + l32, queries 32 hf + 8 g4 + 4 h2
  // at pwbase ^ (64 hf + 16 g4)
  const int pwbase = pt_off(32 * kg + l32, 4 * h2);
  // direct copies of a 64-row Q or dO tile
  int qgoff[QLPW];
#pragma unroll
  for (int i = 0; i < QLPW; ++i) {
    const int c = w + NW * i;
    const int p = 64 * c + l;
    const int row = p / NCH, ch = p % NCH;
    qgoff[i] = row * (int)rs + ((ch ^ chunk_swizzle<D>(row)) << 3);
  }
  // copies of one query block: the Q and dO tiles (all waves), and its row
  // terms, 64 + 64 floats in two 4-byte-per-lane copies (wave 0)
  auto issue_q = [&](int qblk, lds_char* qdst, lds_char* gdst, float* rdst) __attribute__((always_inline)) {
    const __bf16* qg = a.q + head_off + (size_t)qblk * BR * rs;
    const __bf16* gg = a.dO + head_off + (size_t)qblk * BR * rs;
#pragma unroll
    for (int i = 0; i < QLPW; ++i) {
      const int c = w + NW * i;
      copy16_to_lds(qg + qgoff[i], (lds_void*)(qdst + c * 1024));
      copy16_to_lds(gg + qgoff[i], (lds_void*)(gdst + c * 1024));
    }
    if (w == 0) {
      __builtin_amdgcn_global_load_lds(nlse2 + qblk * BR + l, (lds_void*)rdst, 4, 0, 0);
      __builtin_amdgcn_global_load_lds(drow + qblk * BR + l, (lds_void*)(rdst + BR), 4, 0, 0);
    }
  };

  f32x16 dvacc[NDH], dkacc[NDH];
#pragma unroll
  for (int j = 0; j < NDH; ++j) {
    dvacc[j] = f32x16{};
    dkacc[j] = f32x16{};
  }
  const float c = a.c;
  const int nqb = a.N / BR;
  const int qstart = CAUSAL ? (kb / BR) : 0;
  const int key = kw + l32;

  auto qblock = [&](int qi, const lds_char* __restrict__ qt, const lds_char* __restrict__ gt,
                    const float* __restrict__ rcur, lds_char* __restrict__ qnext, lds_char* __restrict__ gnext,
                    float* __restrict__ rnext) __attribute__((always_inline)) {
    // this block's copies have landed and every wave is done with the
    // previous block (its P / dS tiles and the buffers about to be refilled)
    barrier_vmem<0>();
    if (qi + 1 < nqb) issue_q(qi + 1, qnext, gnext, rnext);
    const int q0 = qi * BR;

    // S = Q K^T and dP = dO V^T for the wave's query half; lane holds
    // [query 32 dh + 8(e/4)+4h2+e%4][key l32].  The operands of k-step kk + 2
    // are requested before the products of k-step kk (a ring of three).
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    bf16x8 ring[3][2];
    auto read_rows = [&](int kk, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
      const int off = roff ^ (kk << 5);
      dst[0] = lds_read16(qt + off);
      dst[1] = lds_read16(gt + off);
    };
    read_rows(0, ring[0]);
    read_rows(1, ring[1]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 2 < NKK) read_rows(kk + 2, ring[(kk + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32(ring[kk % 3][0], kreg[kk], sacc);
      pacc = mfma32(ring[kk % 3][1], vreg[kk], pacc);
    }
    __builtin_amdgcn_sched_barrier(0);

    // P = exp2(S c - L log2 e) (masked), dS = P (dP - D); both to bf16
    const int qh0 = q0 + 32 * dh;
    const bool diag = CAUSAL && (qh0 < kw + 31);
    uint32_t ppk[8], dspk[8];
    {
      const __attribute__((address_space(3))) f32x4* r4 = (const __attribute__((address_space(3))) f32x4*)rcur;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nl = r4[(32 * dh + 8 * g4 + 4 * h2) >> 2];
        const f32x4 dr = r4[(BR + 32 * dh + 8 * g4 + 4 * h2) >> 2];
#pragma unroll
        for (int e2 = 0; e2 < 4; e2 += 2) {
          const int e = 4 * g4 + e2;
          float p0 = fast_exp2(fmaf(sacc[e], c, nl[e2]));
          float p1 = fast_exp2(fmaf(sacc[e + 1], c, nl[e2 + 1]));
          if (diag) {
            const int qrow = qh0 + 8 * g4 + 4 * h2 + e2;
            p0 = (key > qrow) ? 0.f : p0;
            p1 = (key > qrow + 1) ? 0.f : p1;
          }
          if (!wave_active) p0 = p1 = 0.f;
          const float ds0 = p0 * (pacc[e] - dr[e2]);
          const float ds1 = p1 * (pacc[e + 1] - dr[e2 + 1]);
          ppk[e >> 1] = pack_bf16x2(p0, p1);
          dspk[e >> 1] = pack_bf16x2(ds0, ds1);
        }
      }
    }
    // P^T and dS^T chunks -> LDS for the partner wave and the dQ product
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      *(__attribute__((address_space(3))) u32x2*)(ptile + (pwbase ^ (64 * dh + 16 * g4))) = u32x2{ppk[2 * g4], ppk[2 * g4 + 1]};
      *(__attribute__((address_space(3))) u32x2*)(dstile + (pwbase ^ (64 * dh + 16 * g4))) = u32x2{dspk[2 * g4], dspk[2 * g4 + 1]};
    }
    barrier_lds();  // P^T and dS^T tiles complete
    __builtin_amdgcn_sched_barrier(0);

    // dV += P^T dO and dK += dS^T Q over the 64 queries, four steps of 16:
    // A = P^T / dS^T (own half from registers, the partner's half from LDS),
    // B = dO / Q columns of this wave's d half by transpose reads
    // step st = 2 hf + tq: hf = 0 is the own half (dh), hf = 1 the partner's
    bf16x8 pa[2], sa[2], go[2][NDH], qo[2][NDH];
    auto read_dv = [&](int st, bf16x8& pa_, bf16x8& sa_, bf16x8 (&go_)[NDH], bf16x8 (&qo_)[NDH])
        __attribute__((always_inline)) {
      const int hf = st >> 1, tq = st & 1;
      if (hf == 0) {
        pa_ = __builtin_bit_cast(bf16x8, u32x4{ppk[4 * tq], ppk[4 * tq + 1], ppk[4 * tq + 2], ppk[4 * tq + 3]});
        sa_ = __builtin_bit_cast(bf16x8, u32x4{dspk[4 * tq], dspk[4 * tq + 1], dspk[4 * tq + 2], dspk[4 * tq + 3]});
      } else {
        typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
        const int o0 = pwbase ^ (64 * (1 - dh) + 32 * tq);
        const int o1 = pwbase ^ (64 * (1 - dh) + 32 * tq + 16);
        const u32x2 p0 = *(const lds_u32x2*)(ptile + o0);
        const u32x2 p1 = *(const lds_u32x2*)(ptile + o1);
        const u32x2 s0 = *(const lds_u32x2*)(dstile + o0);
        const u32x2 s1 = *(const lds_u32x2*)(dstile + o1);
        pa_ = __builtin_bit_cast(bf16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
        sa_ = __builtin_bit_cast(bf16x8, u32x4{s0[0], s0[1], s1[0], s1[1]});
      }
      const int qrow16 = 32 * (hf == 0 ? dh : 1 - dh) + 16 * tq;
#pragma unroll
      for (int j = 0; j < NDH; ++j) {
        const int db = dh * NDH + j;
        const int o0 = qrow16 * ROWB + (troff0[0] ^ (db << 6));
        const int o1 = qrow16 * ROWB + (troff0[1] ^ (db << 6));
        go_[j] = __builtin_shufflevector(lds_read_tr16(gt + o0), lds_read_tr16(gt + o1), 0, 1, 2, 3, 4, 5, 6, 7);
        qo_[j] = __builtin_shufflevector(lds_read_tr16(qt + o0), lds_read_tr16(qt + o1), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    read_dv(0, pa[0], sa[0], go[0], qo[0]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < 4) read_dv(st + 1, pa[(st + 1) & 1], sa[(st + 1) & 1], go[(st + 1) & 1], qo[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NDH; ++j) {
        dvacc[j] = mfma32(pa[st & 1], go[st & 1][j], dvacc[j]);
        dkacc[j] = mfma32(sa[st & 1], qo[st & 1][j], dkacc[j]);
      }
    }
  };

  lds_char* const Q0 = (lds_char*)q_lds0;
  lds_char* const Q1 = (lds_char*)q_lds1;
  lds_char* const G0 = (lds_char*)g_lds0;
  lds_char* const G1 = (lds_char*)g_lds1;
  float* const R0 = r_lds0;
  float* const R1 = r_lds1;
  issue_q(qstart, Q0, G0, R0);
  // the buffer roles alternate; __restrict__ tells the compiler that the
  // copies into the other buffers do not alias this block's reads
  for (int qi = qstart; qi < nqb; ++qi) {
    const bool odd = (qi - qstart) & 1;
    qblock(qi, odd ? Q1 : Q0, odd ? G1 : G0, odd ? R1 : R0, odd ? Q0 : Q1, odd ? G0 : G1, odd ? R0 : R1);
  }

  // ---- dK = scale * dK_acc, dV = dV_acc; lane holds [key kw + 8(e/4)+4h2+e%4][d = 32 db + l32]
  if (!wave_active) return;
  const float scale = a.scale;
#pragma unroll
  for (int j = 0; j < NDH; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = kw + 8 * (e >> 2) + 4 * h2 + (e & 3);
      const size_t off = head_off + (size_t)kr * rs + 32 * (dh * NDH + j) + l32;
      a.dk[off] = (__bf16)(dkacc[j][e] * scale);
      a.dv[off] = (__bf16)(dvacc[j][e]);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ kernel: one workgroup of NW waves per (batch, head, query tile of
//    32 NW rows), walking the key tiles like the forward kernel (K and V
//    tiles double-buffered in LDS by direct copies).  Everything is computed
//    transposed so lane l32 of a wave owns one query row:
//        S^T = K Q^T,  dP^T = V dO^T               (Q, dO: B operands in VGPRs)
//        P^T = exp2(S^T c - L log2 e),  dS^T = P^T (dP^T - D)   (lane-local row terms)
//        dQ^T += K^T dS^T                          (dS^T straight from the accumulators)
//    and dQ = scale dQ^T is written once, in bf16: no accumulator in memory
//    and no atomics.
template <int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = NW * 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int NCH = D / 8;
  constexpr int LOADS = TILEB / 1024;
  constexpr int LPW = LOADS / NW;
  constexpr int NSB = BC / 32;           // 32-key sub-blocks of a tile
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  static_assert(LOADS % NW == 0, "tile copies must split evenly over waves");
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

  // ---- workgroup -> (batch, head, query tile), as in the forward kernel
  const int nqb = (a.N + BR - 1) / BR;
  const int nbh = a.B * a.H;
  const int wg = blockIdx.x;
  int bh, qi;
  if ((nbh & 7) == 0) {
    const int hpx = nbh >> 3;
    const int x = wg & 7, s = wg >> 3;
    bh = x * hpx + s % hpx;
    qi = s / hpx;
  } else {
    bh = wg % nbh;
    qi = wg / nbh;
  }
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh - b * a.H;
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const int q0 = qb * BR;
  const int qw = q0 + 32 * w;
  const bool wave_active = qw < a.N;
  const int qrow = qw + l32;

  const size_t rs = (size_t)a.H * D;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * D;
  const __bf16* kbase = a.k + head_off;
  const __bf16* vbase = a.v + head_off;

  // ---- Q and dO rows as B operands (lane: query l32, d = 16 kk + 8 h2 ..), row terms
  bf16x8 qop[NKK], gop[NKK];
  float nl = 0.f, dr = 0.f;
  if (wave_active) {
    const __bf16* qr = a.q + head_off + (size_t)qrow * rs + 8 * h2;
    const __bf16* gr = a.dO + head_off + (size_t)qrow * rs + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qop[kk] = *(const bf16x8*)(qr + 16 * kk);
      gop[kk] = *(const bf16x8*)(gr + 16 * kk);
    }
    const size_t r = ((size_t)b * a.H + h) * a.N + qrow;
    dr = a.drow[r];
    nl = a.drow[(size_t)a.B * a.H * a.N + r];
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[kk] = gop[kk] = bf16x8{};
  }

  // ---- per-lane LDS offsets (the forward kernel's geometry)
  // K / V rows as A operands: row 32 sb + l32, chunk 2 kk + h2
  const int roff = l32 * ROWB + ((chunk_swizzle<D>(l32) ^ h2) << 4);
  // K^T by transpose reads: rows 16 t + 4 h2 + j/4 (+8), columns 32 db + 16 (g&1) + 4 (j&3)
  int troff0[2];
  {
    const int g = l >> 4, j = l & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 4 * h2 + (j >> 2) + 8 * r;
      const int ch = 2 * (g & 1) + ((j & 3) >> 1);
      troff0[r] = row * ROWB + ((ch ^ chunk_swizzle<D>(row)) << 4) + 8 * (j & 1);
    }
  }
  int goff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = 64 * (w + NW * i) + l;
    const int row = p / NCH, ch = p % NCH;
    goff[i] = row * (int)rs + ((ch ^ chunk_swizzle<D>(row)) << 3);
  }
  auto issue_tile = [&](int kt, lds_char* kdst, lds_char* vdst) __attribute__((always_inline)) {
    const __bf16* kg = kbase + (size_t)kt * BC * rs;
    const __bf16* vg = vbase + (size_t)kt * BC * rs;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = w + NW * i;
      copy16_to_lds(kg + goff[i], (lds_void*)(kdst + c * 1024));
      copy16_to_lds(vg + goff[i], (lds_void*)(vdst + c * 1024));
    }
  };

  const int ntiles_all = a.N / BC;
  int ntiles = ntiles_all;
  if (CAUSAL) ntiles = min(ntiles_all, (min(q0 + BR, a.N) - 1) / BC + 1);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};
  const float c = a.c;

  auto compute_tile = [&](auto MASK, int kb, const lds_char* __restrict__ kt_lds,
                          const lds_char* __restrict__ vt_lds) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(MASK)::value;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      // S^T and dP^T of the 32-key sub-block: lane holds [key 8(e/4)+4h2+e%4][query l32];
      // the K / V operands of k-step kk + 2 are requested before the products of kk
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      bf16x8 ring[3][2];
      auto read_kv = [&](int kk, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
        const int off = sb * 32 * ROWB + (roff ^ (kk << 5));
        dst[0] = lds_read16(kt_lds + off);
        dst[1] = lds_read16(vt_lds + off);
      };
      read_kv(0, ring[0]);
      read_kv(1, ring[1]);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 2 < NKK) read_kv(kk + 2, ring[(kk + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        sacc = mfma32(ring[kk % 3][0], qop[kk], sacc);
        pacc = mfma32(ring[kk % 3][1], gop[kk], pacc);
      }
      __builtin_amdgcn_sched_barrier(0);
      // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L log2 e), masked above the diagonal
      uint32_t dspk[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float p0 = fast_exp2(fmaf(sacc[e], c, nl));
        float p1 = fast_exp2(fmaf(sacc[e + 1], c, nl));
        if constexpr (MASKED) {
          const int key = kb + 32 * sb + 8 * (e >> 2) + 4 * h2 + (e & 3);
          p0 = (key > qrow) ? 0.f : p0;
          p1 = (key + 1 > qrow) ? 0.f : p1;
        }
        dspk[e >> 1] = pack_bf16x2(p0 * (pacc[e] - dr), p1 * (pacc[e + 1] - dr));
      }
      // dQ^T += K^T dS^T over the sub-block's 32 keys, two steps of 16
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const bf16x8 sop = __builtin_bit_cast(bf16x8, u32x4{dspk[4 * tq], dspk[4 * tq + 1], dspk[4 * tq + 2], dspk[4 * tq + 3]});
        const int t = 2 * sb + tq;
        bf16x8 kop[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x4 k0 = lds_read_tr16(kt_lds + 16 * t * ROWB + (troff0[0] ^ (db << 6)));
          const bf16x4 k1 = lds_read_tr16(kt_lds + 16 * t * ROWB + (troff0[1] ^ (db << 6)));
          kop[db] = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqacc[db] = mfma32(kop[db], sop, dqacc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto tile_step = [&](int kt, const lds_char* __restrict__ kt_lds, const lds_char* __restrict__ vt_lds,
                       lds_char* __restrict__ knext, lds_char* __restrict__ vnext) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < ntiles) issue_tile(kt + 1, knext, vnext);
    const int kb = kt * BC;
    if (!wave_active) return;
    if (CAUSAL && kb > qw + 31) return;  // whole tile in this wave's future
    if (CAUSAL && kb + BC - 1 > qw)
      compute_tile(std::true_type{}, kb, kt_lds, vt_lds);
    else
      compute_tile(std::false_type{}, kb, kt_lds, vt_lds);
  };

  lds_char* K0 = (lds_char*)k_lds0;
  lds_char* K1 = (lds_char*)k_lds1;
  lds_char* V0 = (lds_char*)v_lds0;
  lds_char* V1 = (lds_char*)v_lds1;
  issue_tile(0, K0, V0);
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_step(kt, K0, V0, K1, V1);
    if (kt + 1 < ntiles) tile_step(kt + 1, K1, V1, K0, V0);
  }

  if (!wave_active) return;
  // ---- dQ = scale dQ^T; lane holds [d = 32 db + 8(e/4)+4h2+e%4][query l32]
  const float scale = a.scale;
  __bf16* dqrow = a.dq + head_off + (size_t)qrow * rs;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * h2;
      u32x2 val = {pack_bf16x2(dqacc[db][4 * g4 + 0] * scale, dqacc[db][4 * g4 + 1] * scale),
                   pack_bf16x2(dqacc[db][4 * g4 + 2] * scale, dqacc[db][4 * g4 + 3] * scale)};
      *(u32x2*)(dqrow + d0) = val;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  void* args[] = {(void*)&a};
  {
    const long rows = (long)a.B * a.N * a.H;
    const int rpb = 256 / (D / 8);
    dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    hipError_t e = hipLaunchKernel((const void*)bwd_pre_kernel<D>, grid, dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    dim3 grid((unsigned)(a.B * a.H * ((a.N + 127) / 128)));
    hipError_t e = hipLaunchKernel((const void*)bwd_main_kernel<D, CAUSAL>, grid, dim3(512), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = D == 128 ? 8 : 4;
    constexpr int BR = NW * 32;
    dim3 grid((unsigned)(a.B * a.H * ((a.N + BR - 1) / BR)));
    return hipLaunchKernel((const void*)bwd_dq_kernel<D, NW, 64, CAUSAL>, grid, dim3(NW * 64), args, 0, stream);
  }
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
  return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
}

}  // namespace fa
