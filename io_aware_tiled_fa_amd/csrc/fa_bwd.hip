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
    float* dq = a.dqacc + off;
    *(f32x4*)dq = f32x4{};
    *(f32x4*)(dq + 4) = f32x4{};
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
// 2. main kernel: one workgroup per 128-key block, 4 waves of 32 keys each,
//    walking the query blocks of 64 rows (two halves of 32).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdArgs a) {
  constexpr int NW = 4;
  constexpr int BC = 32 * NW;          // keys per workgroup
  constexpr int BR = 64;               // queries per step (two halves of 32)
  constexpr int ROWB = D * 2;          // bytes per row of a Q / dO / K tile
  constexpr int QTILEB = BR * ROWB;    // Q or dO tile
  constexpr int KTILEB = BC * ROWB;    // K tile (for the dQ product)
  constexpr int NCH = D / 8;
  constexpr int NKK = D / 16;          // k-steps over d
  constexpr int NDB = D / 32;          // 32-wide column blocks over d
  constexpr int DSROWB = BR * 2 + 8;   // dS row: 64 queries bf16, padded
  constexpr int QLOADS = QTILEB / 1024;
  constexpr int QLPW = QLOADS / NW;    // copies per wave per Q or dO tile
  constexpr int NAT = 2 * 16;          // dQ atomics per wave per block (w < NDB)
  static_assert(QLOADS % NW == 0, "tile copies must split evenly over waves");
  // LDS objects: Q, dO and row-term tiles double-buffered, the K tile, the dS tile
  __shared__ __attribute__((aligned(1024))) char q_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char q_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds[KTILEB];
  __shared__ __attribute__((aligned(1024))) char ds_lds[BC * DSROWB];
  // row terms of a query block: -L log2(e) of its 64 rows, then their D
  __shared__ __attribute__((aligned(256))) float r_lds0[2 * BR];
  __shared__ __attribute__((aligned(256))) float r_lds1[2 * BR];
  lds_char* const ktile = (lds_char*)k_lds;
  lds_char* const dstile = (lds_char*)ds_lds;

  const int nbh = a.B * a.H;
  const int wg = blockIdx.x;
  int bh, kblk;
  if ((nbh & 7) == 0) {
    const int hpx = nbh >> 3;
    const int x = wg & 7, s = wg >> 3;
    bh = x * hpx + s % hpx;
    kblk = s / hpx;  // causal: low key blocks see the most query blocks, so they go first
  } else {
    bh = wg % nbh;
    kblk = wg / nbh;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const int kb = kblk * BC;
  const int kw = kb + 32 * w;  // first key of this wave
  // N is a multiple of 64, so the last key block may hold only 64 keys:
  // waves past the end neither load nor compute, and leave dS = 0
  const bool wave_active = kw < a.N;

  const size_t rs = (size_t)a.H * D;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * D;
  const size_t rowterm_off = ((size_t)b * a.H + h) * a.N;
  const float* drow = a.drow + rowterm_off;
  const float* nlse2 = a.drow + (size_t)a.B * a.H * a.N + rowterm_off;

  // ---- this wave's keys and values as B operands: lane = key l32, d = 16 kk + 8 h2 ..
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

  // ---- K tile of the whole workgroup into LDS (for dQ = dS K)
  {
    constexpr int KLOADS = KTILEB / 1024;
#pragma unroll
    for (int i = 0; i < KLOADS / NW; ++i) {
      const int c = w + NW * i;
      const int p = 64 * c + l;
      const int row = p / NCH, ch = p % NCH;
      if (kb + row < a.N) {  // uniform per copy: a copy spans 1 KiB of whole rows
        const __bf16* g = a.k + head_off + (size_t)(kb + row) * rs + ((ch ^ chunk_swizzle<D>(row)) << 3);
        copy16_to_lds(g, (lds_void*)(ktile + c * 1024));
      } else {
        *(__attribute__((address_space(3))) u32x4*)(ktile + c * 1024 + 16 * l) = u32x4{};
      }
    }
  }

  // ---- per-lane LDS offsets.  Tiles use the forward kernel's geometry; the
  // swizzle XORs the chunk index, so a power-of-two chunk step is an XOR.
  // row reads (A operand, lane = row l32 of a 32-row half, chunk 2 kk + h2)
  const int roff0 = l32 * ROWB + ((chunk_swizzle<D>(l32) ^ h2) << 4);
  // transpose reads: rows 16 t + 4 h2 + j/4 (+8), cols 32 db + 16 (g&1) + 4 (j&3)
  int troff0[2], dsroff[2];
  {
    const int g = l >> 4, j = l & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 4 * h2 + (j >> 2) + 8 * r;
      const int ch = 2 * (g & 1) + ((j & 3) >> 1);
      troff0[r] = row * ROWB + ((ch ^ chunk_swizzle<D>(row)) << 4) + 8 * (j & 1);
      // dS tile [key][query]: rows = keys, cols = queries 16 (g&1) + 4 (j&3)
      dsroff[r] = row * DSROWB + 2 * (16 * (g & 1) + 4 * (j & 3));
    }
  }
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

  f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }
  const float c = a.c;
  const int nqb = a.N / BR;
  const int qstart = CAUSAL ? (kb / BR) : 0;
  const int key = kw + l32;

  // One query block.  A wave's memory operations retire in issue order, so
  // at the top of every block but the first, vmcnt(NAT) waits for this
  // block's copies while the previous block's dQ atomics stay in flight.
  auto qblock = [&](int qi, const lds_char* __restrict__ qt, const lds_char* __restrict__ gt,
                    const float* __restrict__ rcur, lds_char* __restrict__ qnext, lds_char* __restrict__ gnext,
                    float* __restrict__ rnext) __attribute__((always_inline)) {
    if (qi == qstart || w >= NDB)
      barrier_vmem<0>();
    else
      barrier_vmem<NAT>();
    if (qi + 1 < nqb) issue_q(qi + 1, qnext, gnext, rnext);
    const int q0 = qi * BR;

    // S = Q K^T and dP = dO V^T for both 32-row halves: four independent
    // accumulation chains; lane holds [query 32 hq + 8(e/4)+4h2+e%4][key l32]
    // The operands of k-step kk + 2 are requested before the products of
    // k-step kk (a ring of three), with sched_barrier fences pinning that
    // order, so the LDS latency hides behind the matrix-core work.
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) sacc[hq] = pacc[hq] = f32x16{};
    bf16x8 ring[3][4];  // per k-step: Q half 0, Q half 1, dO half 0, dO half 1
    auto read_rows = [&](int kk, bf16x8 (&dst)[4]) __attribute__((always_inline)) {
      const int off = roff0 ^ (kk << 5);
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        dst[hq] = lds_read16(qt + hq * 32 * ROWB + off);
        dst[2 + hq] = lds_read16(gt + hq * 32 * ROWB + off);
      }
    };
    read_rows(0, ring[0]);
    read_rows(1, ring[1]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 2 < NKK) read_rows(kk + 2, ring[(kk + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        sacc[hq] = mfma32(ring[kk % 3][hq], kreg[kk], sacc[hq]);
        pacc[hq] = mfma32(ring[kk % 3][2 + hq], vreg[kk], pacc[hq]);
      }
    }
    // sched_barrier fences bound how far the compiler may hoist work across
    // phases (unbounded hoisting of LDS reads here exhausts the registers)
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      // row terms of this lane's 16 queries of the half: 32 hq + 8 g4 + 4 h2 + (0..3)
      const __attribute__((address_space(3))) f32x4* r4 = (const __attribute__((address_space(3))) f32x4*)rcur;
      f32x4 nl[4], dr[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        nl[g4] = r4[(32 * hq + 8 * g4 + 4 * h2) >> 2];
        dr[g4] = r4[(BR + 32 * hq + 8 * g4 + 4 * h2) >> 2];
      }
      const int qh0 = q0 + 32 * hq;
      const bool diag = CAUSAL && (qh0 < kw + 31);
      uint32_t ppk[8], dspk[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int g4 = e >> 2;
        float p0 = fast_exp2(fmaf(sacc[hq][e], c, nl[g4][e & 3]));
        float p1 = fast_exp2(fmaf(sacc[hq][e + 1], c, nl[g4][(e & 3) + 1]));
        if (diag) {
          const int qrow = qh0 + 8 * g4 + 4 * h2 + (e & 3);
          p0 = (key > qrow) ? 0.f : p0;
          p1 = (key > qrow + 1) ? 0.f : p1;
        }
        if (!wave_active) p0 = p1 = 0.f;
        const float ds0 = p0 * (pacc[hq][e] - dr[g4][e & 3]);
        const float ds1 = p1 * (pacc[hq][e + 1] - dr[g4][(e & 3) + 1]);
        ppk[e >> 1] = pack_bf16x2(p0, p1);
        dspk[e >> 1] = pack_bf16x2(ds0, ds1);
      }

      __builtin_amdgcn_sched_barrier(0);
      // dS (bf16) -> LDS as [key][query] for the dQ product
      {
        lds_char* dsrow = dstile + (32 * w + l32) * DSROWB + 2 * 32 * hq;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 v2 = {dspk[2 * g4], dspk[2 * g4 + 1]};
          *(__attribute__((address_space(3))) u32x2*)(dsrow + 2 * (8 * g4 + 4 * h2)) = v2;
        }
      }

      // dV += P^T dO and dK += dS^T Q over the half's 32 queries (two steps
      // of 16): A from registers, B by transpose reads of the dO / Q tiles
      bf16x8 gop[2][NDB], qop[2][NDB];
      auto read_tr = [&](int tq, bf16x8 (&go)[NDB], bf16x8 (&qo)[NDB]) __attribute__((always_inline)) {
        const int t = 2 * hq + tq;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int o0 = 16 * t * ROWB + (troff0[0] ^ (db << 6));
          const int o1 = 16 * t * ROWB + (troff0[1] ^ (db << 6));
          go[db] = __builtin_shufflevector(lds_read_tr16(gt + o0), lds_read_tr16(gt + o1), 0, 1, 2, 3, 4, 5, 6, 7);
          qo[db] = __builtin_shufflevector(lds_read_tr16(qt + o0), lds_read_tr16(qt + o1), 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      read_tr(0, gop[0], qop[0]);
      read_tr(1, gop[1], qop[1]);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const u32x4 pv = {ppk[4 * tq], ppk[4 * tq + 1], ppk[4 * tq + 2], ppk[4 * tq + 3]};
        const u32x4 sv = {dspk[4 * tq], dspk[4 * tq + 1], dspk[4 * tq + 2], dspk[4 * tq + 3]};
        const bf16x8 pa = __builtin_bit_cast(bf16x8, pv);
        const bf16x8 sa = __builtin_bit_cast(bf16x8, sv);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          mfma32_agpr(dvacc[db], pa, gop[tq][db]);
          mfma32_agpr(dkacc[db], sa, qop[tq][db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    barrier_lds();  // dS tile complete
    // dQ_blk (64 queries x D) = dS (64 x 128 keys) K (128 keys x D): wave w
    // computes output columns 32 w .. 32 w + 31 for both halves (waves
    // beyond D / 32 idle); each K operand read serves both halves
    if (w < NDB) {
      f32x16 dqa[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) {
        const bf16x4 k0 = lds_read_tr16(ktile + 16 * t * ROWB + (troff0[0] ^ (w << 6)));
        const bf16x4 k1 = lds_read_tr16(ktile + 16 * t * ROWB + (troff0[1] ^ (w << 6)));
        const bf16x8 ka = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
          const bf16x4 s0 = lds_read_tr16(dstile + 16 * t * DSROWB + 64 * hq + dsroff[0]);
          const bf16x4 s1 = lds_read_tr16(dstile + 16 * t * DSROWB + 64 * hq + dsroff[1]);
          dqa[hq] = mfma32(__builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7), ka, dqa[hq]);
        }
      }
      // lane holds dQ[query 32 hq + 8(e/4)+4h2+e%4][d = 32 w + l32]
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        float* dqb = a.dqacc + head_off + (size_t)(q0 + 32 * hq) * rs + 32 * w + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qr = 8 * (e >> 2) + 4 * h2 + (e & 3);
          __hip_atomic_fetch_add(dqb + (size_t)qr * rs, dqa[hq][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
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
  // one instance of the block body (two would not fit the registers); the
  // buffer roles alternate and __restrict__ tells the compiler that the
  // copies into the other buffers do not alias this block's reads
  for (int qi = qstart; qi < nqb; ++qi) {
    const bool odd = (qi - qstart) & 1;
    qblock(qi, odd ? Q1 : Q0, odd ? G1 : G0, odd ? R1 : R0, odd ? Q0 : Q1, odd ? G0 : G1, odd ? R0 : R1);
  }

  // ---- dK = scale * dK_acc, dV = dV_acc; lane holds [key 8(e/4)+4h2+e%4][d = 32 db + l32]
  if (!wave_active) return;
  const float scale = a.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = kw + 8 * (e >> 2) + 4 * h2 + (e & 3);
      const size_t off = head_off + (size_t)kr * rs + 32 * db + l32;
      a.dk[off] = (__bf16)(dkacc[db][e] * scale);
      a.dv[off] = (__bf16)(dvacc[db][e]);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> bf16, 8 elements per thread
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *(const f32x4*)(a.dqacc + 8 * i);
  const f32x4 x1 = *(const f32x4*)(a.dqacc + 8 * i + 4);
  const float s = a.scale;
  u32x4 out = {pack_bf16x2(x0[0] * s, x0[1] * s), pack_bf16x2(x0[2] * s, x0[3] * s),
               pack_bf16x2(x1[0] * s, x1[1] * s), pack_bf16x2(x1[2] * s, x1[3] * s)};
  *(u32x4*)(a.dq + 8 * i) = out;
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
    hipError_t e = hipLaunchKernel((const void*)bwd_main_kernel<D, CAUSAL>, grid, dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    long n8 = (long)a.B * a.N * a.H * D / 8;
    void* args2[] = {(void*)&a, (void*)&n8};
    dim3 grid((unsigned)((n8 + 255) / 256));
    return hipLaunchKernel((const void*)bwd_dq_kernel, grid, dim3(256), args2, 0, stream);
  }
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
  return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
}

}  // namespace fa
