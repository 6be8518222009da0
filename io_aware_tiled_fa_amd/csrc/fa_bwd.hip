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
// Two kernels on one stream, none of them atomic, so the gradients are the
// same bit for bit on every run:
//  1. bwd_dq (dQ): one workgroup per query tile, walking the key tiles like
//     the forward kernel and recomputing S and dP; dQ is summed in
//     registers and written once.  Each wave also forms the row terms of
//     its rows, -D_i = -dO_i . O_i and -L_i log2(e) (float32), and writes
//     them to the workspace for the second kernel;
//  2. bwd_main (dK, dV): one workgroup of 8 waves per 128-key block of one
//     (batch, key head).  Four producer waves recompute S = Q K^T, P and
//     dS = P (dP - D) for 32 keys each against 32-query blocks staged in
//     LDS; four consumer waves, one beside each producer on its SIMD, add
//     P^T dO into dV (two of them, 64 keys each) or dS^T Q into dK (the
//     other two), one block behind.  The walk covers every query block of
//     every query head that reads this key head (grouped-query attention)
//     whose rows see a key of the block.
// Masks: key j is visible to query i iff i + off - wl <= j <= i + off + wr
// (off = N_k - N_q), the forward kernel's band.
// All products run on v_mfma_f32_32x32x16_bf16.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"


namespace fa {

// ---------------------------------------------------------------------------
// dK / dV kernel: one workgroup of 8 waves per 128-key block, walking the
//    query blocks of 32 rows.  The waves specialise: wave w < 4 produces for
//    key group w (keys 32 w .. 32 w + 31 of the block); waves 4 and 5 add dV
//    for keys 0-63 and 64-127, waves 6 and 7 dK for the same halves (each
//    transpose read of dO or Q feeds two products).  In step t:
//      producer (block t):     S = Q K^T and dP - D = dO V^T - D      16 products
//                              P = exp2(S c - L log2 e) (masked), dS = P (dP - D)
//                              P^T, dS^T -> LDS (bf16)
//      consumer (block t - 1): dV += P^T dO or dK += dS^T Q over its 32 rows   16 products
//    so the producers' softmax runs beside the consumers' matrix products;
//    every SIMD holds one producer and one consumer.  One barrier per step;
//    Q / dO tiles and row terms are in four buffers (the producer's products
//    read block t + 1, the consumers block t - 1, the copies fill block
//    t + 2) and the P^T / dS^T tiles double-buffered.
//
// P^T / dS^T tiles: 128 key rows of 32 queries in the layout of pt_off
// (fa_layout.h).
template <int I>
using IC = std::integral_constant<int, I>;

template <int D, bool BAND, bool WIN>
__global__ __launch_bounds__(512) void bwd_main_kernel(BwdArgs a) {
  static_assert(BAND || !WIN, "a window always bounds the keys above");
  constexpr int BC = 128;              // keys per workgroup (4 groups of 32)
  constexpr int BR = 32;               // queries per step
  constexpr int ROWB = D * 2;          // bytes per row of a Q / dO tile
  constexpr int QTILEB = BR * ROWB;    // Q or dO tile
  constexpr int PTB = BC * BR * 2;     // P^T or dS^T tile
  constexpr int NKK = D / 16;          // k-steps over d
  constexpr int NDB = D / 32;          // 32-wide column blocks over d
  constexpr int QLPW = 2 * QTILEB / 1024 / 4;  // copies per consumer wave per step (Q and dO)
  static_assert(QLPW >= 1, "tile copies must split evenly over the waves");
  // Q / dO tiles and row terms in 4 buffers (the producer's products read
  // block t + 1, its softmax block t's row terms, the consumer block t - 1,
  // the copies fill block t + 2); P^T / dS^T in 2.  Every buffer is a
  // separate object and the walk is unrolled by 4, so every access names its
  // buffer at compile time: the compiler can then see that the copies into
  // one buffer never alias the reads of another and does not hold the reads
  // back until the copies land.
  __shared__ __attribute__((aligned(1024))) char q_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char q_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char q_lds2[QTILEB];
  __shared__ __attribute__((aligned(1024))) char q_lds3[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds0[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds1[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds2[QTILEB];
  __shared__ __attribute__((aligned(1024))) char g_lds3[QTILEB];
  __shared__ __attribute__((aligned(1024))) char p_lds0[PTB];
  __shared__ __attribute__((aligned(1024))) char p_lds1[PTB];
  __shared__ __attribute__((aligned(1024))) char ds_lds0[PTB];
  __shared__ __attribute__((aligned(1024))) char ds_lds1[PTB];
  // row terms of a query block: -L log2(e) of its 32 rows, then their -D
  __shared__ __attribute__((aligned(256))) float r_lds0[2 * BR];
  __shared__ __attribute__((aligned(256))) float r_lds1[2 * BR];
  __shared__ __attribute__((aligned(256))) float r_lds2[2 * BR];
  __shared__ __attribute__((aligned(256))) float r_lds3[2 * BR];

  // one workgroup per (batch, key head, key block)
  const int nbh = a.B * a.Hkv;
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
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int G = a.G;  // query heads hk G .. hk G + G - 1 read this key head
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const bool producer = w < 4;
  const int kg = w & 3;
  const int kb = kblk * BC;
  const int kw = kb + 32 * kg;  // first key of this wave's group
  // key groups past the last key compute nothing; the last active one may
  // be ragged (its lanes past N_k are masked and store nothing)
  const bool group_active = kw < a.Nk;
  // key j is visible to query i iff i + lo_off <= j <= i + hi_off (keys
  // aligned to the end of the queries)
  const int hi_off = a.Nk - a.Nq + a.wr;
  const int lo_off = a.Nk - a.Nq - a.wl;

  const size_t rs = (size_t)a.H * D;     // Q, dO row stride
  const size_t rk = (size_t)a.Hkv * D;   // K, V, dK, dV row stride
  const size_t qb_off = (size_t)b * a.Nq * rs;                   // Q, dO of batch b
  const size_t kv_off = (size_t)b * a.Nk * rk + (size_t)hk * D;  // K, V, dK, dV

  // ---- per-lane LDS offsets.  Q / dO tiles are in the row-group layout
  // (fa_device.h), read as rows by the producers and by transpose reads by
  // the consumers.
  // producer row reads (A operand, lane = row l32, piece 2 kk + h2) at
  // krb[kk & 1] + 256 (kk / 2)
  int krb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) krb[par] = rg_row_base<D>(l, par);
  // consumer transpose reads: rows 4 h2 + j/4 (+8 r) of a 16-row step, columns
  // 32 db + 16 (g&1) + 4 (j&3), at trb[r] + 256 db
  int trb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) trb[r] = rg_tr_base<D>(l, r);
  // P^T / dS^T chunk of this lane: key row 32 kg + l32, queries 8 g4 + 4 h2 at
  // pbase ^ (16 g4)
  const int pbase = pt_off(32 * kg + l32, 4 * h2);
  // direct copies of a 32-row Q or dO tile, all issued by the consumer waves
  // (the producers then have no copy in flight that the compiler would make
  // their LDS writes wait for): copy i of consumer wave w - 4 is 1 KiB slot
  // w - 4 + 4 i of the pair (Q tile slots first, then dO)
  // (byte offsets from the tile's first row, one unsigned 32-bit value per
  // copy, into buffer resources over this head's Q and dO rows based at
  // the block's first row)
  uint32_t qgoff[QLPW];
#pragma unroll
  for (int i = 0; i < QLPW; ++i) {
    const int c = ((w & 3) + 4 * i) % (QTILEB / 1024);
    int row, piece;
    rg_slot<D>(64 * c + l, row, piece);
    qgoff[i] = (uint32_t)(row * (int)rs + piece * 8) * 2u;
  }
  // buffer I (a std::integral_constant) of each kind
  auto QT = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value & 3;
    return (lds_char*)(i == 0 ? q_lds0 : i == 1 ? q_lds1 : i == 2 ? q_lds2 : q_lds3);
  };
  auto GT = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value & 3;
    return (lds_char*)(i == 0 ? g_lds0 : i == 1 ? g_lds1 : i == 2 ? g_lds2 : g_lds3);
  };
  auto RT = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value & 3;
    return (float*)(i == 0 ? r_lds0 : i == 1 ? r_lds1 : i == 2 ? r_lds2 : r_lds3);
  };
  auto PT = [&](auto I) __attribute__((always_inline)) { return (lds_char*)((decltype(I)::value & 1) ? p_lds1 : p_lds0); };
  auto DT = [&](auto I) __attribute__((always_inline)) { return (lds_char*)((decltype(I)::value & 1) ? ds_lds1 : ds_lds0); };
  // The walk visits query blocks qlo .. qhi (set below) of each of the G
  // query heads hk G .. hk G + G - 1 in turn.  Running state of the copies:
  // the next block to copy (block qb_next of head hq_next), buffer resources
  // over that head's Q and dO rows and the offset of its row terms, rebuilt
  // only when the walk moves on to the next head.
  int hq_next = hk * G, qb_next = 0;
  const __bf16* qhead = nullptr;
  const __bf16* ghead = nullptr;
  uint32_t head_bytes = 0;
  size_t rt_head = 0;
  auto set_head = [&]() __attribute__((always_inline)) {
    // query head hq_next's rows 0 .. N_q - 1 at a stride of H d, the last
    // ending H d - hq d elements before the end of the batch's span.
    // Offsets stay under 2^32 bytes (the host requires (N_q + 128) H d <
    // 2^31).
    head_bytes = (uint32_t)(((size_t)a.Nq * a.H - hq_next) * D * 2);
    qhead = a.q + qb_off + (size_t)hq_next * D;
    ghead = a.dO + qb_off + (size_t)hq_next * D;
    rt_head = ((size_t)b * a.H + hq_next) * a.Nq;
  };
  // copies of query block qblk of the current head into Q / dO / row-term buffer I
  auto issue_q = [&](int qblk, auto I) __attribute__((always_inline)) {
    if (producer) return;
    // (resources based at the block's first row: the per-lane offsets are
    // all the range check sees, so rows past N_q read zero)
    const uint32_t boff = (uint32_t)qblk * (uint32_t)(BR * rs * 2);
#pragma unroll
    for (int i = 0; i < QLPW; ++i) {
      const int slot = (w & 3) + 4 * i;  // wave-uniform
      const int c = slot % (QTILEB / 1024);
      if (slot < QTILEB / 1024)
        copy16_to_lds_buf(make_rsrc_at(qhead, head_bytes, boff), qgoff[i], (lds_void*)(QT(I) + c * 1024));
      else
        copy16_to_lds_buf(make_rsrc_at(ghead, head_bytes, boff), qgoff[i], (lds_void*)(GT(I) + c * 1024));
    }
    // the row terms are copied by a consumer wave, so the producers' writes
    // to the P^T / dS^T tiles never wait behind a copy the compiler cannot
    // tell apart from them
    if (w == 4) {  // lanes 0-31: -L log2 e, lanes 32-63: -D of the block's rows
      // (rows past N_q repeat the last row; they are masked)
      const int row = min(qblk * BR + (l & 31), a.Nq - 1);
      const size_t rt = rt_head + row;
      const float* src = (l < 32) ? (a.drow + (size_t)a.B * a.H * a.Nq + rt) : (a.drow + rt);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)RT(I), 4, 0, 0);
    }
  };
  auto step_barrier = [&]() __attribute__((always_inline)) {
    wait_vmem();
    barrier_lds();
  };

  const float c = a.c;
  const int nqb = (a.Nq + BR - 1) / BR;
  // the query blocks qlo .. qhi hold every row that sees a key of this block
  int qlo = 0, qhi = nqb - 1;
  if (BAND) {
    const int i_min = max(0, kb - hi_off);
    const int i_max = WIN ? min(a.Nq - 1, min(kb + BC, a.Nk) - 1 - lo_off) : a.Nq - 1;
    qlo = i_min / BR;
    qhi = i_max < i_min ? qlo - 1 : i_max / BR;
  }
  const int nqr = qhi - qlo + 1;
  const int key = kw + l32;
  const int nv = max(nqr, 0) * G;  // blocks in the walk
  qb_next = qlo;
  set_head();
  // qbuf[i]: the query block held in Q / dO / row-term buffer i (only ever
  // indexed by compile-time constants, so it lives in scalar registers)
  int qbuf[4] = {0, 0, 0, 0};
  // copy the next block of the walk into buffer I (the producers only keep
  // the bookkeeping) and advance the walk
  auto issue_next = [&](auto I) __attribute__((always_inline)) {
    qbuf[decltype(I)::value & 3] = qb_next;
    issue_q(qb_next, I);
    if (++qb_next > qhi) {
      qb_next = qlo;
      ++hq_next;
      set_head();
    }
  };
  // no step when no query sees these keys (their gradients are then zero)
  const int nsteps = nv > 0 ? nv + 1 : 0;

  // ---- the walk.  Step t produces P^T / dS^T of walk block t and consumes
  // walk block t - 1.  The two roles run separate loops (their registers
  // never live at the same time) with the same barriers: s_barrier counts
  // arrivals, so every wave passes one per step.
  if (0 < nv) issue_next(IC<0>{});
  if (1 < nv) issue_next(IC<1>{});

  if (producer) {
    // the group's keys and values as B operands (lane = key l32, d = 16 kk + 8 h2 ..),
    // loaded while the consumers' first copies are in flight
    bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kreg[kk] = vreg[kk] = bf16x8{};
    if (group_active && key < a.Nk) {
      const __bf16* kr = a.k + kv_off + (size_t)key * rk + 8 * h2;
      const __bf16* vr = a.v + kv_off + (size_t)key * rk + 8 * h2;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        kreg[kk] = *(const bf16x8*)(kr + 16 * kk);
        vreg[kk] = *(const bf16x8*)(vr + 16 * kk);
      }
    }
    step_barrier();
    typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;
    // S (lane = key l32, e -> query 8(e/4)+4h2+e%4) and dP - D, the latter
    // accumulated onto -D, of the block in buffer qb4 / row terms rb3.
    // Products only; operands of k-step kk + 2 requested before those of kk.
    // With `soft`, the softmax of the previous block's (sc, pc) into (ppk,
    // dspk) is spread over the products, one element pair per k-step.
    auto products = [&](auto I, f32x16& sn, f32x16& pn, auto SOFT, const f32x16& sc, const f32x16& pc,
                        const float (&nlv)[16], uint32_t (&ppk)[8], uint32_t (&dspk)[8]) __attribute__((always_inline)) {
      constexpr bool S_ON = decltype(SOFT)::value;
      const lds_char* qt = QT(I);
      const lds_char* gt = GT(I);
      lds_f32x4* r4 = (lds_f32x4*)RT(I);
      sn = f32x16{};
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nd = r4[(BR + 8 * g4 + 4 * h2) >> 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) pn[4 * g4 + i] = nd[i];
      }
      constexpr int PD = 3;  // k-steps the operand reads run ahead
      bf16x8 ring[PD + 1][2];
      auto read_rows = [&](int kk, bf16x8 (&dst2)[2]) __attribute__((always_inline)) {
        const int off = krb[kk & 1] + 256 * (kk >> 1);
        dst2[0] = lds_read16(qt + off);
        dst2[1] = lds_read16(gt + off);
      };
#pragma unroll
      for (int kk = 0; kk < PD && kk < NKK; ++kk) read_rows(kk, ring[kk]);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + PD < NKK) read_rows(kk + PD, ring[(kk + PD) % (PD + 1)]);
        sn = mfma32(ring[kk % (PD + 1)][0], kreg[kk], sn);
        pn = mfma32(ring[kk % (PD + 1)][1], vreg[kk], pn);
        if constexpr (S_ON) {
#pragma unroll
          for (int u = kk * 8 / NKK; u < (kk + 1) * 8 / NKK; ++u) {
            const int e = 2 * u;
            const float p0 = fast_exp2(fmaf(sc[e], c, nlv[e]));
            const float p1 = fast_exp2(fmaf(sc[e + 1], c, nlv[e + 1]));
            ppk[u] = pack_bf16x2(p0, p1);
            dspk[u] = pack_bf16x2(p0 * pc[e], p1 * pc[e + 1]);
            // keep the conversions in this k-step (the compiler would
            // otherwise sink them to their use after the products)
            asm volatile("" : "+v"(ppk[u]), "+v"(dspk[u]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    f32x16 sA, pA, sB, pB;
    float nlv[16];
    uint32_t ppk[8], dspk[8];
    // step t's softmax uses the scores in (sA, pA) for even t, (sB, pB) for odd
    // step t = T (mod 4)
    auto pstep = [&](auto T, int t, f32x16& sc, f32x16& pc, f32x16& sn, f32x16& pn) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T)::value;
      step_barrier();
      if (t + 2 < nv) issue_next(IC<T4 + 2>{});
      if (!group_active || t >= nv) return;
      const int qi = qbuf[T4];
      // exp2 addends: -L log2 e of each element's row, -inf where key > query
      lds_f32x4* r4 = (lds_f32x4*)RT(T);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nl = r4[(8 * g4 + 4 * h2) >> 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) nlv[4 * g4 + i] = nl[i];
      }
      // masked: key outside the query's band, query >= N_q or key >= N_k
      const int q0 = qi * BR;
      if ((BAND && q0 + hi_off < kw + 31) || (WIN && q0 + BR - 1 + lo_off > kw) || q0 + BR > a.Nq || kw + 32 > a.Nk) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qr = q0 + 8 * (e >> 2) + 4 * h2 + (e & 3);
          const bool masked = (BAND && key > qr + hi_off) || (WIN && key < qr + lo_off) || qr >= a.Nq || key >= a.Nk;
          nlv[e] = masked ? -__builtin_inff() : nlv[e];
        }
      }
      // block qi + 1's products beside block qi's softmax (the products of
      // the block past the end read a stale buffer and are never used)
      products(IC<T4 + 1>{}, sn, pn, std::true_type{}, sc, pc, nlv, ppk, dspk);
      // P^T and dS^T chunks -> LDS for the consumer of this key group
      typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
      lds_char* pt = PT(T);
      lds_char* dt = DT(T);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        *(lds_u32x2*)(pt + (pbase ^ (16 * g4))) = u32x2{ppk[2 * g4], ppk[2 * g4 + 1]};
        *(lds_u32x2*)(dt + (pbase ^ (16 * g4))) = u32x2{dspk[2 * g4], dspk[2 * g4 + 1]};
      }
    };
    if (group_active) products(IC<0>{}, sA, pA, std::false_type{}, sB, pB, nlv, ppk, dspk);
    for (int t = 0; t < nsteps; t += 4) {
      pstep(IC<0>{}, t, sA, pA, sB, pB);
      if (t + 1 < nsteps) pstep(IC<1>{}, t + 1, sB, pB, sA, pA);
      if (t + 2 < nsteps) pstep(IC<2>{}, t + 2, sA, pA, sB, pB);
      if (t + 3 < nsteps) pstep(IC<3>{}, t + 3, sB, pB, sA, pA);
    }
    return;
  }

  step_barrier();  // (the consumers' first; the producers passed theirs above)

  // ---- consumers: waves 4 and 5 add dV^T += dO^T P for keys 0-63 and
  // 64-127 of the block, waves 6 and 7 dK^T += Q^T dS for the same halves.
  // Each transpose read of dO or Q then feeds two products (one per 32-key
  // group of the half).  The products are formed transposed (dO / Q
  // columns as the A operand, P^T / dS^T as B), so the accumulators
  // [group of the half][db] hold dV^T / dK^T: lane [d = 32 db + 8(e/4) + 4h2
  // + e%4][key 32 g + l32], four consecutive d per lane and key, which the
  // epilogue stores as one 8-byte piece.
  const int kh = w & 1;             // key half of this consumer
  const int kw2 = kb + 64 * kh;     // its first key
  f32x16 acc[2][NDB];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[g][db] = f32x16{};
  // P^T / dS^T chunks of the two groups: key rows 32 (2 kh + g) + l32,
  // queries 8 g4 + 4 h2 at pb[g] ^ (16 g4)
  int pb[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) pb[g] = pt_off(32 * (2 * kh + g) + l32, 4 * h2);
  // DV: dO and P^T (dV), else Q and dS^T (dK); a compile-time choice, so
  // every read names its LDS buffer
  auto consume = [&](auto DV, int qi, const lds_char* __restrict__ xt, const lds_char* __restrict__ pt)
      __attribute__((always_inline)) {
    // P = dS = 0 for this block: every row's band misses the half's keys
    if ((BAND && qi * BR + BR - 1 + hi_off < kw2) || (WIN && qi * BR + lo_off > kw2 + 63)) return;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    // product pair i = (tq, db): B = dO / Q columns (transpose reads, CD
    // pairs ahead), A = the P^T / dS^T chunks of the 16 queries of step tq
    // for each group
    constexpr int NP = 2 * NDB;
    constexpr int CD = 2;
    bf16x8 pa[2][2], xo[CD + 1];
    auto read_op = [&](int i) __attribute__((always_inline)) {
      const int tq = i / NDB, db = i % NDB, s = i % (CD + 1);
      if (db == 0) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const u32x2 p0 = *(const lds_u32x2*)(pt + (pb[g] ^ (32 * tq)));
          const u32x2 p1 = *(const lds_u32x2*)(pt + (pb[g] ^ (32 * tq + 16)));
          pa[g][tq & 1] = __builtin_bit_cast(bf16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
        }
      }
      const int o0 = 16 * tq * ROWB + 256 * db + trb[0];
      const int o1 = 16 * tq * ROWB + 256 * db + trb[1];
      xo[s] = __builtin_shufflevector(lds_read_tr16(xt + o0), lds_read_tr16(xt + o1), 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int i = 0; i < CD && i < NP; ++i) read_op(i);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + CD < NP) read_op(i + CD);
      __builtin_amdgcn_sched_barrier(0);
      const int tq = i / NDB, db = i % NDB, s = i % (CD + 1);
      acc[0][db] = mfma32(xo[s], pa[0][tq & 1], acc[0][db]);
      acc[1][db] = mfma32(xo[s], pa[1][tq & 1], acc[1][db]);
    }
  };
  const bool half_active = kw2 < a.Nk;
  auto cstep = [&](auto DV, auto T, int t) __attribute__((always_inline)) {
    constexpr int T4 = decltype(T)::value;
    step_barrier();
    if (t + 2 < nv) issue_next(IC<T4 + 2>{});
    if (half_active && t > 0) {
      if constexpr (decltype(DV)::value)
        consume(DV, qbuf[(T4 + 3) & 3], GT(IC<T4 + 3>{}), PT(IC<T4 + 1>{}));
      else
        consume(DV, qbuf[(T4 + 3) & 3], QT(IC<T4 + 3>{}), DT(IC<T4 + 1>{}));
    }
  };
  auto walk = [&](auto DV) __attribute__((always_inline)) {
    for (int t = 0; t < nsteps; t += 4) {
      cstep(DV, IC<0>{}, t);
      if (t + 1 < nsteps) cstep(DV, IC<1>{}, t + 1);
      if (t + 2 < nsteps) cstep(DV, IC<2>{}, t + 2);
      if (t + 3 < nsteps) cstep(DV, IC<3>{}, t + 3);
    }
  };
  const bool dv_role = w < 6;
  if (dv_role)
    walk(std::true_type{});
  else
    walk(std::false_type{});

  // ---- consumer epilogue: dV = dV_acc, or dK = scale dK_acc, in bf16.
  // A lane holds four consecutive d of one key per 8-byte piece, so storing
  // the accumulators directly would spread every store instruction over 32
  // key rows in 16-byte pieces.  They go through LDS instead (each wave's
  // 64 keys into the Q and dO buffers of its own index, in the staging
  // layout of fa_layout.h) and are read back a row per D / 8 lanes, so each
  // store instruction writes whole rows.  The barrier waits for the other
  // consumers' last reads of those buffers (the producers have ended and no
  // longer count).
  barrier_lds();
  if (!half_active) return;
  constexpr int NCH = D / 8;  // 16-byte pieces of a row
  const float f = dv_role ? 1.0f : a.scale;
  __bf16* out = dv_role ? a.dv : a.dk;
  const int ci = w & 3;
  lds_char* stage[2] = {(lds_char*)(ci == 0 ? q_lds0 : ci == 1 ? q_lds1 : ci == 2 ? q_lds2 : q_lds3),
                        (lds_char*)(ci == 0 ? g_lds0 : ci == 1 ? g_lds1 : ci == 2 ? g_lds2 : g_lds3)};
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // d = 32 db + 8 g4 + 4 h2 .. + 3 of key row l32: piece 4 db + g4, half h2
        *(lds_u32x2*)(stage[g] + stage_off<D>(l32, 4 * db + g4, h2)) =
            u32x2{pack_bf16x2(acc[g][db][4 * g4] * f, acc[g][db][4 * g4 + 1] * f),
                  pack_bf16x2(acc[g][db][4 * g4 + 2] * f, acc[g][db][4 * g4 + 3] * f)};
      }
  // read back: lane l takes piece l % NCH of row 64 / NCH i + l / NCH
  constexpr int RPI = 64 / NCH;  // rows per store instruction
  const int pc = l % NCH;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + l / NCH;
      u32x4 v = *(const lds_u32x4*)(stage[g] + (stage_off<D>(r, pc, 0) & ~15));
      if (stage_swap<D>(r)) v = u32x4{v[2], v[3], v[0], v[1]};
      const int kr = kw2 + 32 * g + r;
      if (kr < a.Nk) *(u32x4*)(out + kv_off + (size_t)kr * rk + 8 * pc) = v;
    }
}

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup of NW waves per (batch, head, query tile of
//    32 NW rows), walking the key tiles like the forward kernel (K and V
//    tiles double-buffered in LDS by direct copies).  Everything is computed
//    transposed so lane l32 of a wave owns one query row:
//        S^T = K Q^T,  dP^T = V dO^T               (Q, dO: B operands in VGPRs)
//        P^T = exp2(S^T c - L log2 e),  dS^T = P^T (dP^T - D)   (lane-local row terms)
//        dQ^T += K^T dS^T                          (dS^T straight from the accumulators)
//    and dQ = scale dQ^T is written once, in bf16: no accumulator in memory
//    and no atomics.
template <int D, int NW, int BC, bool BAND, bool WIN>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdArgs a) {
  static_assert(BAND || !WIN, "a window always bounds the keys above");
  constexpr int BR = NW * 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
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

  // ---- workgroup -> (batch, head, query tile): each XCD a contiguous range
  // of heads (as the dK/dV kernel), the heaviest causal tiles first
  const int nqb = (a.Nq + BR - 1) / BR;
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
  const int qb = BAND ? (nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh - b * a.H;
  const int hk = h / a.G;  // key / value head
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63, h2 = l >> 5, l32 = l & 31;
  const int q0 = qb * BR;
  const int qw = q0 + 32 * w;
  const bool wave_active = qw < a.Nq;
  const int qrow = qw + l32;
  const bool row_valid = qrow < a.Nq;  // the last tile of rows may be ragged
  // key j is visible to query i iff i + lo_off <= j <= i + hi_off
  const int hi_off = a.Nk - a.Nq + a.wr;
  const int lo_off = a.Nk - a.Nq - a.wl;

  const size_t rs = (size_t)a.H * D;     // Q, dO, dQ row stride
  const size_t rk = (size_t)a.Hkv * D;   // K, V row stride
  const size_t q_off = (size_t)b * a.Nq * rs + (size_t)h * D;    // Q, dO, dQ
  const size_t kv_off = (size_t)b * a.Nk * rk + (size_t)hk * D;  // K, V
  const __bf16* kbase = a.k + kv_off;
  const __bf16* vbase = a.v + kv_off;

  // ---- per-lane LDS offsets (K and V tiles in the row-group layout)
  // K / V rows as A operands: row 32 sb + l32, piece 2 kk + h2, at
  // krb[kk & 1] + 256 (kk / 2) + sb 32 ROWB
  int krb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) krb[par] = rg_row_base<D>(l, par);
  // K^T by transpose reads: rows 16 t + 4 h2 + j/4 (+8 r), columns
  // 32 db + 16 (g&1) + 4 (j&3), at trb[r] + 256 db + 16 t ROWB
  int trb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) trb[r] = rg_tr_base<D>(l, r);
  // (byte offsets, one unsigned 32-bit value per copy, into buffer resources
  // over this head's K and V rows, sized as in the forward kernel)
  uint32_t goff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    int row, piece;
    rg_slot<D>(64 * (w + NW * i) + l, row, piece);
    goff[i] = (uint32_t)(row * (int)rk + piece * 8) * 2u;
  }
  // (resources based at the tile's first row: the per-lane offsets are all
  // the range check sees, so rows past N_k read zero; offsets under 2^32
  // bytes, as in the forward kernel)
  const uint32_t head_bytes = (uint32_t)(((size_t)a.Nk * a.Hkv - hk) * D * 2);
  auto issue_tile = [&](int kt, lds_char* kdst, lds_char* vdst) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)kt * (uint32_t)(BC * rk * 2);
    const buf_rsrc krs = make_rsrc_at(kbase, head_bytes, toff);
    const buf_rsrc vrs = make_rsrc_at(vbase, head_bytes, toff);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = w + NW * i;
      copy16_to_lds_buf(krs, goff[i], (lds_void*)(kdst + c * 1024));
      copy16_to_lds_buf(vrs, goff[i], (lds_void*)(vdst + c * 1024));
    }
  };

  const int ntiles_all = (a.Nk + BC - 1) / BC;
  int ntiles = ntiles_all, kt0 = 0;  // key tiles kt0 .. ntiles - 1
  if (BAND) {
    const int last_key = min(q0 + BR, a.Nq) - 1 + hi_off;  // last key any row here sees
    ntiles = last_key < 0 ? 0 : min(ntiles_all, last_key / BC + 1);
  }
  if (WIN) kt0 = max(0, q0 + lo_off) / BC;                 // first key any row here sees
  // the first tile's copies go out before the rows below are loaded, so the
  // two latencies overlap
  if (kt0 < ntiles) issue_tile(kt0, (lds_char*)k_lds0, (lds_char*)v_lds0);

  // ---- Q and dO rows as B operands (lane: query l32, d = 16 kk + 8 h2 ..),
  // and the row terms: D = dO . O over the lane's half of the row, then
  // both halves; -D and -L log2(e) also go to the workspace for the dK / dV
  // kernel, which runs after this one
  bf16x8 qop[NKK], gop[NKK];
  float nl = 0.f, ndr = 0.f;  // -L log2(e) and -D of this lane's row
  float dpart = 0.f;
  if (row_valid) {
    const __bf16* qr = a.q + q_off + (size_t)qrow * rs + 8 * h2;
    const __bf16* gr = a.dO + q_off + (size_t)qrow * rs + 8 * h2;
    const __bf16* orow = a.o + q_off + (size_t)qrow * rs + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qop[kk] = *(const bf16x8*)(qr + 16 * kk);
      gop[kk] = *(const bf16x8*)(gr + 16 * kk);
      const u32x4 ov = *(const u32x4*)(orow + 16 * kk);
      const u32x4 gv = __builtin_bit_cast(u32x4, gop[kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dpart = fmaf(__builtin_bit_cast(float, ov[i] << 16), __builtin_bit_cast(float, gv[i] << 16), dpart);
        dpart = fmaf(__builtin_bit_cast(float, ov[i] & 0xFFFF0000u), __builtin_bit_cast(float, gv[i] & 0xFFFF0000u), dpart);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[kk] = gop[kk] = bf16x8{};
  }
  const float dsum = sum_cross_half(dpart);
  if (row_valid) {
    const size_t r = ((size_t)b * a.H + h) * a.Nq + qrow;
    ndr = -dsum;
    nl = -a.lse[r] * kLog2e;
    if (h2 == 0) {
      a.drow[r] = ndr;
      a.drow[(size_t)a.B * a.H * a.Nq + r] = nl;
    }
  }

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};
  const float c = a.c;

  // One key tile as two 32-key sub-blocks, software-pipelined so the dS
  // work (VALU) of one sub-block runs beside independent matrix-core
  // products of the same wave:
  //   S^T, dP^T of sub-block 0
  //   S^T, dP^T of sub-block 1      beside  dS^T of sub-block 0
  //   dQ^T += K0^T dS0^T            beside  dS^T of sub-block 1
  //   dQ^T += K1^T dS1^T
  // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L log2 e), masked outside the
  // row's band; one element pair per product, pinned there by an empty asm.
  static_assert(NSB == 2, "the pipelined tile needs 64-key tiles");
  auto compute_tile = [&](auto MASK, int kb, const lds_char* __restrict__ kt_lds,
                          const lds_char* __restrict__ vt_lds) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(MASK)::value;
    const int hi = BAND ? min(qrow + hi_off, a.Nk - 1) : a.Nk - 1;  // last visible key
    const int lo = qrow + lo_off;                                     // first (banded)
    auto ds_pair = [&](int sb, int u, const f32x16& sv, const f32x16& pv, uint32_t (&dspk)[8])
        __attribute__((always_inline)) {
      const int e = 2 * u;
      float p0 = fast_exp2(fmaf(sv[e], c, nl));
      float p1 = fast_exp2(fmaf(sv[e + 1], c, nl));
      if constexpr (MASKED) {  // key outside the row's band, or key >= N_k
        const int key = kb + 32 * sb + 8 * (e >> 2) + 4 * h2 + (e & 3);
        p0 = (key > hi || (WIN && key < lo)) ? 0.f : p0;
        p1 = (key + 1 > hi || (WIN && key + 1 < lo)) ? 0.f : p1;
      }
      dspk[u] = pack_bf16x2(p0 * pv[e], p1 * pv[e + 1]);
      asm volatile("" : "+v"(dspk[u]));
    };
    // S^T and dP^T of sub-block sb (lane: [key 8(e/4)+4h2+e%4][query l32]);
    // the K / V operands of k-step kk + 2 requested before the products of
    // kk; with PREV, the dS of sub-block 0 spread over the k-steps
    auto sdp = [&](int sb, f32x16& sacc, f32x16& pacc, auto PREV, const f32x16& sp, const f32x16& pp,
                   uint32_t (&dsp)[8]) __attribute__((always_inline)) {
      sacc = f32x16{};
      // dP^T accumulates onto -D of the lane's row (every element of a lane
      // is in that row), so dS = P (dP - D) takes one multiply
#pragma unroll
      for (int e = 0; e < 16; ++e) pacc[e] = ndr;
      bf16x8 ring[3][2];
      auto read_kv = [&](int kk, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
        const int off = sb * 32 * ROWB + krb[kk & 1] + 256 * (kk >> 1);
        dst[0] = lds_read16(kt_lds + off);
        dst[1] = lds_read16(vt_lds + off);
      };
      read_kv(0, ring[0]);
      read_kv(1, ring[1]);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 2 < NKK) read_kv(kk + 2, ring[(kk + 2) % 3]);
        sacc = mfma32(ring[kk % 3][0], qop[kk], sacc);
        pacc = mfma32(ring[kk % 3][1], gop[kk], pacc);
        if constexpr (decltype(PREV)::value) {
#pragma unroll
          for (int u = kk * 8 / NKK; u < (kk + 1) * 8 / NKK; ++u) ds_pair(sb - 1, u, sp, pp, dsp);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // dQ^T += K^T dS^T over sub-block sb's 32 keys (two steps of 16); with
    // NEXT, the dS of sub-block 1 spread over the products
    auto dqmm = [&](int sb, const uint32_t (&dspk)[8], auto NEXT, const f32x16& sn, const f32x16& pn,
                    uint32_t (&dsn)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const bf16x8 sop = __builtin_bit_cast(bf16x8, u32x4{dspk[4 * tq], dspk[4 * tq + 1], dspk[4 * tq + 2], dspk[4 * tq + 3]});
        const int t = 2 * sb + tq;
        bf16x8 kop[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x4 k0 = lds_read_tr16(kt_lds + 16 * t * ROWB + 256 * db + trb[0]);
          const bf16x4 k1 = lds_read_tr16(kt_lds + 16 * t * ROWB + 256 * db + trb[1]);
          kop[db] = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          __builtin_amdgcn_sched_barrier(0);
          dqacc[db] = mfma32(kop[db], sop, dqacc[db]);
          if constexpr (decltype(NEXT)::value) {
            constexpr int NP = 2 * NDB;  // products of this sub-block
            const int i = tq * NDB + db;
#pragma unroll
            for (int u = i * 8 / NP; u < (i + 1) * 8 / NP; ++u) ds_pair(sb + 1, u, sn, pn, dsn);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    f32x16 s0, p0, s1, p1;
    uint32_t d0[8], d1[8];
    sdp(0, s0, p0, std::false_type{}, s0, p0, d0);
    sdp(1, s1, p1, std::true_type{}, s0, p0, d0);
    dqmm(0, d0, std::true_type{}, s1, p1, d1);
    dqmm(1, d1, std::false_type{}, s1, p1, d1);
  };

  // MAYMASK: whether the tile can need masking (tiles crossing a band edge,
  // or the ragged last tile); unbanded loops never instantiate the masked
  // variant and take their ragged last tile after the loop
  auto tile_step = [&](auto MAYMASK, int kt, const lds_char* __restrict__ kt_lds,
                       const lds_char* __restrict__ vt_lds, lds_char* __restrict__ knext,
                       lds_char* __restrict__ vnext) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < ntiles) issue_tile(kt + 1, knext, vnext);
    const int kb = kt * BC;
    if (!wave_active) return;
    // whole tile outside every row's band in this wave
    if ((BAND && kb > qw + 31 + hi_off) || (WIN && kb + BC - 1 < qw + lo_off)) return;
    if constexpr (decltype(MAYMASK)::value) {
      if ((BAND && kb + BC - 1 > qw + hi_off) || (WIN && kb < qw + 31 + lo_off) || kb + BC > a.Nk)
        compute_tile(std::true_type{}, kb, kt_lds, vt_lds);
      else
        compute_tile(std::false_type{}, kb, kt_lds, vt_lds);
    } else {
      compute_tile(std::false_type{}, kb, kt_lds, vt_lds);
    }
  };

  lds_char* K0 = (lds_char*)k_lds0;
  lds_char* K1 = (lds_char*)k_lds1;
  lds_char* V0 = (lds_char*)v_lds0;
  lds_char* V1 = (lds_char*)v_lds1;
  constexpr auto LOOP_MASK = std::integral_constant<bool, BAND>{};
  // (unbanded: kt0 = 0 and the ragged last tile is peeled)
  const int nloop = (!BAND && a.Nk % BC != 0) ? ntiles - 1 : ntiles;
  for (int kt = kt0; kt < nloop; kt += 2) {
    tile_step(LOOP_MASK, kt, K0, V0, K1, V1);
    if (kt + 1 < nloop) tile_step(LOOP_MASK, kt + 1, K1, V1, K0, V0);
  }
  if (nloop < ntiles) {  // the ragged last tile of an unbanded walk
    if (nloop & 1)
      tile_step(std::true_type{}, nloop, K1, V1, K0, V0);
    else
      tile_step(std::true_type{}, nloop, K0, V0, K1, V1);
  }

  // ---- dQ = scale dQ^T; lane holds [d = 32 db + 8(e/4)+4h2+e%4][query l32].
  // As in the dK / dV kernel's epilogue, the rows go through LDS (each
  // wave's 32 rows into its own quarter of the K / V buffers, in the staging
  // layout of fa_layout.h) so that each store instruction writes whole
  // rows.  The barrier waits for the last tile's reads.
  barrier_lds();
  if (!wave_active) return;
  constexpr int NCH = D / 8;  // 16-byte pieces of a row
  static_assert(4 * TILEB >= NW * 32 * ROWB, "the K / V buffers must hold every wave's rows");
  const float scale = a.scale;
  lds_char* stage = (lds_char*)(w < NW / 4 ? k_lds0 : w < NW / 2 ? k_lds1 : w < 3 * NW / 4 ? v_lds0 : v_lds1) +
                    (w % (NW / 4)) * 32 * ROWB;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      *(lds_u32x2*)(stage + stage_off<D>(l32, 4 * db + g4, h2)) =
          u32x2{pack_bf16x2(dqacc[db][4 * g4 + 0] * scale, dqacc[db][4 * g4 + 1] * scale),
                pack_bf16x2(dqacc[db][4 * g4 + 2] * scale, dqacc[db][4 * g4 + 3] * scale)};
    }
  // read back: lane l takes piece l % NCH of row 64 / NCH i + l / NCH
  constexpr int RPI = 64 / NCH;
  const int pc = l % NCH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + l / NCH;
    u32x4 v = *(const lds_u32x4*)(stage + (stage_off<D>(r, pc, 0) & ~15));
    if (stage_swap<D>(r)) v = u32x4{v[2], v[3], v[0], v[1]};
    if (qw + r < a.Nq) *(u32x4*)(a.dq + q_off + (size_t)(qw + r) * rs + 8 * pc) = v;
  }
}

template <int D, bool BAND, bool WIN>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  void* args[] = {(void*)&a};
  {
    // dQ, and the row terms of every query row into the workspace
    constexpr int NW = D == 128 ? 8 : 4;
    constexpr int BR = NW * 32;
    dim3 grid((unsigned)(a.B * a.H * ((a.Nq + BR - 1) / BR)));
    hipError_t e = hipLaunchKernel((const void*)bwd_dq_kernel<D, NW, 64, BAND, WIN>, grid, dim3(NW * 64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(a.B * a.Hkv * ((a.Nk + 127) / 128)));
  return hipLaunchKernel((const void*)bwd_main_kernel<D, BAND, WIN>, grid, dim3(512), args, 0, stream);
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, bool band, bool win, hipStream_t stream) {
  if (win) return launch_bwd_t<D, true, true>(a, stream);
  return band ? launch_bwd_t<D, true, false>(a, stream) : launch_bwd_t<D, false, false>(a, stream);
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool band, bool win, hipStream_t stream) {
  return d == 128 ? launch_bwd_d<128>(a, band, win, stream) : launch_bwd_d<64>(a, band, win, stream);
}

}  // namespace fa
