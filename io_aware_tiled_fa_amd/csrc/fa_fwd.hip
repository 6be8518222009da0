// Forward attention kernel for gfx950: O = softmax(scale * Q K^T) V and the
// per-row log-sum-exp, one pass over K and V per query tile.
//
// The method is the one the pages describe ("Flash Attention Explained:
// How IO-Aware Computing Made Long Context Practical", institutepm.com,
// section "How Flash Attention Fixes It: Tiling and Recomputation"): load
// small tiles of Q, K and V into on-chip memory, fuse the score product,
// the softmax and the product with V into one kernel so no intermediate
// reaches HBM, and keep a running row maximum and row sum so the softmax is
// built up tile by tile and still ends exact.  The pages give no tile sizes
// or listing; everything below the statement of the method is designed for
// CDNA4:
//
//  * one workgroup = NW wave64s, each wave owning 32 query rows (Br = 32 NW);
//    the query tile lives in VGPRs for the whole kernel;
//  * K and V tiles of BC keys stream through LDS, double buffered, copied
//    straight from HBM into LDS (global_load_lds, no VGPR staging) in the
//    row-group layout (fa_device.h) so the matrix-core operand reads are
//    conflict free and each transpose read takes 128 contiguous bytes;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    so every lane holds 32 scores of ONE query row: the row max needs one
//    cross-half exchange, the row sum none until the end, and the rescale
//    factor is lane-local;
//  * the bf16 probabilities stay in registers and feed O^T += V^T P^T as the
//    B operand directly; V^T comes from LDS through transpose reads;
//  * softmax works in base 2 with scale*log2(e) folded into one FMA; the
//    running maximum is only moved (and O rescaled) when it grows by more
//    than 2^8, which keeps the result exact (O and the sum share the stale
//    maximum) and skips most rescale passes.  An unmasked tile skips its
//    own maximum once every row has a finite one and runs again with it
//    only when some probability exceeds 2^8 (when the rescale would move
//    the maximum);
//  * masks: key j is visible to query i iff i + off - wl <= j <= i + off + wr
//    (off = N_k - N_q); causal is wr = 0 with wl unbounded, a sliding window
//    of W keys bounds wl (and, not causal, wr) by W - 1.  Key tiles outside
//    a query tile's band are never loaded, and only tiles crossing a band
//    edge (or the ragged end of the keys) run the masked variant;
//  * grouped-query attention: query head h reads key / value head h / G;
//  * workgroup order: workgroups are dealt round-robin over the 8 XCDs; each
//    XCD gets a contiguous set of heads and walks them one head at a time,
//    heaviest causal query tiles first, so the workgroups running together
//    on an XCD stream the same K and V through its L2 (this halves the HBM
//    reads of the long causal forward against interleaving the heads).
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"


namespace fa {

// BAND: the visible keys have an upper edge (causal, or a window); WIN: they
// also have a lower edge (a window).  Without BAND every key is visible.
template <int D, int NW, int BC, bool BAND, bool WIN>
__global__ __launch_bounds__(NW * 64, (D == 64 ? 4 : (NW / 4 > 2 ? NW / 4 : 2))) void fwd_kernel(FwdArgs a) {
  static_assert(BAND || !WIN, "a window always bounds the keys above");
  constexpr int BR = NW * 32;
  constexpr int ROWB = D * 2;            // bytes of one tile row in LDS
  constexpr int TILEB = BC * ROWB;       // bytes of one K or V tile
  constexpr int NCH = D / 8;             // 16-byte chunks per row
  constexpr int LOADS = TILEB / 1024;    // 1 KiB wave copies per tile
  constexpr int LPW = (LOADS + NW - 1) / NW;  // copies per wave per tile (the last may be idle)
  constexpr int NSB = BC / 32;           // 32-key sub-blocks of a tile
  constexpr int NDB = D / 32;            // 32-wide column blocks of O
  constexpr int NKK = D / 16;            // k-steps of the score product
  constexpr int NT = BC / 16;            // k-steps of the PV product

  // Four separate LDS objects (K and V, two buffers each) and a loop unrolled
  // by two: every access names its buffer at compile time, so the compiler
  // can see that the copies into one buffer never alias reads of the other
  // and does not stall the reads on the outstanding copies.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

  // ---- workgroup -> (batch, head, query tile)
  const int nqb = (a.Nq + BR - 1) / BR;
  const int nbh = a.B * a.H;
  const int wg = blockIdx.x;
  int bh, qi;
  if ((nbh & 7) == 0) {
    const int hpx = nbh >> 3;  // heads per XCD
    const int x = wg & 7, s = wg >> 3;
    bh = x * hpx + s / nqb;
    qi = s % nqb;
  } else {
    bh = wg % nbh;
    qi = wg / nbh;
  }
  const int qb = BAND ? (nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh - b * a.H;
  const int hk = h / a.G;  // key / value head

  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int h2 = l >> 5;   // which half of the wave
  const int l32 = l & 31;  // query row of this lane within the wave's 32
  const int q0 = qb * BR;
  const int qw = q0 + 32 * w;
  const bool wave_active = qw < a.Nq;
  const int qrow = qw + l32;
  const bool row_valid = qrow < a.Nq;  // the last tile of rows may be ragged
  // key j is visible to query i iff i + lo_off <= j <= i + hi_off; rows with
  // i + hi_off < 0 see no key
  const int hi_off = a.Nk - a.Nq + a.wr;
  const int lo_off = a.Nk - a.Nq - a.wl;

  const size_t rs = (size_t)a.H * D;     // elements between consecutive Q / O rows
  const size_t rk = (size_t)a.Hkv * D;   // and K / V rows
  const size_t q_off = (size_t)b * a.Nq * rs + (size_t)h * D;
  const size_t kv_off = (size_t)b * a.Nk * rk + (size_t)hk * D;
  const __bf16* kbase = a.k + kv_off;
  const __bf16* vbase = a.v + kv_off;

  // ---- Q tile -> B operand registers (lane: row l32, d = 16 kk + 8 h2 .. +7)
  bf16x8 qop[NKK];
  if (row_valid) {
    const __bf16* qrow_p = a.q + q_off + (size_t)qrow * rs + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[kk] = *(const bf16x8*)(qrow_p + 16 * kk);
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

  // ---- per-lane LDS read offsets (K and V tiles in the row-group layout)
  // K operand of S^T = K Q^T: row 32 s + l32, piece 2 kk + h2, at
  // krb[kk & 1] + 256 (kk / 2) + s 32 ROWB
  int krb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) krb[par] = rg_row_base<D>(l, par);
  auto koff = [&](int kk) __attribute__((always_inline)) { return krb[kk & 1] + 256 * (kk >> 1); };
  // V^T operand by transpose reads: group g = l / 16, lane j = l % 16 reads
  // row 16 t + 4 h2 + j / 4 (+ 8 for the second read), columns
  // 32 db + 16 (g % 2) + 4 (j % 4) .. +3, at vrb[r] + 256 db + 16 t ROWB
  int vrb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) vrb[r] = rg_tr_base<D>(l, r);
  // direct HBM -> LDS copies: wave copy c = w + NW i fills LDS bytes
  // [1024 c, 1024 c + 1024) of a tile; lane l fills 16-byte slot 64 c + l,
  // which holds the piece rg_slot names.  Copy i of a wave reads RSTEP i
  // rows further down than its copy 0, and RSTEP is a multiple of 16, where
  // the layout repeats, so one per-lane byte offset (from the tile's first
  // row) serves every copy, each copy's resource based at its first row.
  constexpr int RSTEP = 64 * NW / NCH;
  static_assert(RSTEP % 16 == 0, "copies of a wave must keep the row-group layout");
  uint32_t goff;
  {
    int row, piece;
    rg_slot<D>(64 * w + l, row, piece);
    goff = (uint32_t)(row * (int)rk + piece * 8) * 2u;
  }
  // K and V of this (batch, key head) through buffer resources: rows
  // 0 .. N_k - 1 at a stride of H_kv d elements, the last ending H_kv d - hk d
  // elements before the end of the head's span.  Each copy rebases its
  // resource at the rows it starts from (scalar work), so its per-lane
  // offset goff is all the range check sees: rows past N_k read zero.
  // Offsets stay under 2^32 bytes (the host requires (N_k + 128) H_kv d
  // < 2^31).
  const uint32_t head_bytes = (uint32_t)(((size_t)a.Nk * a.Hkv - hk) * D * 2);
  auto issue_tile = [&](int kt, lds_char* kdst, lds_char* vdst) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)kt * (uint32_t)(BC * rk * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = w + NW * i;
      if (LOADS % NW != 0 && c >= LOADS) break;  // (wave-uniform)
      const uint32_t off = toff + (uint32_t)(i * RSTEP) * (uint32_t)(rk * 2);
      copy16_to_lds_buf(make_rsrc_at(kbase, head_bytes, off), goff, (lds_void*)(kdst + c * 1024));
      copy16_to_lds_buf(make_rsrc_at(vbase, head_bytes, off), goff, (lds_void*)(vdst + c * 1024));
    }
  };

  // ---- key tiles this workgroup visits: kt0 .. ntiles - 1
  const int ntiles_all = (a.Nk + BC - 1) / BC;
  int ntiles = ntiles_all, kt0 = 0;
  if (BAND) {
    const int last_key = min(q0 + BR, a.Nq) - 1 + hi_off;  // last key any row here sees
    ntiles = last_key < 0 ? 0 : min(ntiles_all, last_key / BC + 1);
  }
  if (WIN) kt0 = max(0, q0 + lo_off) / BC;                 // first key any row here sees

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -__builtin_inff();  // running max, base-2 scaled units
  float l_run = 0.f;                // this lane's half of the running sum
  const float c = a.c;

  // Work on one key tile held in LDS: the scores and their softmax (into
  // bf16 probabilities pk, moving the running maximum and rescaling O and l
  // when it grows), then O += P V.  MASK (std::true_type or
  // std::false_type) selects the variant for tiles crossing a band edge of
  // this wave's rows; every other tile runs without a masking instruction.
  auto scores_softmax = [&](auto MASK, int kb, const lds_char* kt_lds, uint32_t (&pk)[NSB][8])
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(MASK)::value;
    // The row maximum only serves as the reference point of the
    // exponentials.  Once every row of the wave has a finite running
    // maximum, an unmasked tile skips its own maximum and takes the
    // probabilities against the running one.  If some row's tile sum then
    // exceeds 2^8, the tile runs again from its scores with the maximum.
    // Otherwise every probability is at most 2^8, exactly the case in which
    // the lazy rescale below would have kept the stale maximum as well: the
    // probabilities are the ones the path with the maximum computes.
    bool with_max = MASKED || __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) != 0;
    for (;;) {
      // S^T (keys x queries) for each 32-key sub-block: NSB * NKK products in
      // one stream, the K operand of product j + KA requested from LDS when
      // product j issues (a ring of KA + 1 operands).  The scheduling barriers
      // keep the compiler from pulling the reads back to their use, which
      // would make each product wait out a full LDS latency.  With three or
      // four waves per SIMD the other waves cover most of that latency, and
      // the registers of a deeper ring are not there (KA = 1); with two, KA = 4.
      constexpr int KA = (NW >= 12 || D == 64) ? 1 : 4;
      f32x16 sacc[NSB];
      {
        constexpr int NJ = NSB * NKK;
        bf16x8 ring[KA + 1];
        auto read_k = [&](int j) __attribute__((always_inline)) {
          ring[j % (KA + 1)] = lds_read16(kt_lds + (j / NKK) * 32 * ROWB + koff(j % NKK));
        };
#pragma unroll
        for (int j = 0; j < KA && j < NJ; ++j) read_k(j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          if (j + KA < NJ) read_k(j + KA);
          __builtin_amdgcn_sched_barrier(0);
          const int sb = j / NKK, kk = j % NKK;
          sacc[sb] = mfma32(ring[j % (KA + 1)], qop[kk], kk == 0 ? f32x16{} : sacc[sb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      if (with_max) {
        // mask on tiles crossing a band edge: invisible key -> -inf.  The scale
        // factor c is never 0 (the host clamps it to a tiny positive number), so
        // exp2(-inf * c - m) below is exactly 0 with no second mask.
        if constexpr (MASKED) {
          // key outside [qrow + lo_off, qrow + hi_off], or key >= Nk (past the keys)
          const int hi = BAND ? min(qrow + hi_off, a.Nk - 1) : a.Nk - 1;
          const int lo = qrow + lo_off;
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = kb + 32 * sb + 8 * (e >> 2) + 4 * h2 + (e & 3);
              const bool out = WIN ? (key > hi || key < lo) : key > hi;
              sacc[sb][e] = out ? -__builtin_inff() : sacc[sb][e];
            }
        }
        // row max of this tile (raw scores), then in scaled base-2 units
        float mx = -__builtin_inff();
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[sb][e]);
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
      }

      // probabilities, rounded to bf16 pairs for the PV product.  Only a masked
      // tile can leave a row without a key so far (m = -inf, every p = 0); after
      // an unmasked tile m is finite.
      const float negm = (MASKED && m_run == -__builtin_inff()) ? 0.f : -m_run;
      float lt = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = fast_exp2(fmaf(sacc[sb][e], c, negm));
          const float p1 = fast_exp2(fmaf(sacc[sb][e + 1], c, negm));
          lt += p0 + p1;
          pk[sb][e >> 1] = pack_bf16x2(p0, p1);
        }
      if (!with_max && __builtin_amdgcn_ballot_w64(!(lt <= 256.0f)) != 0) {
        with_max = true;
        continue;
      }
      l_run += lt;
      break;
    }
  };
  // O^T += V^T P^T over the tile's keys, 16 at a time; the V^T operands of
  // one key step are all requested before its products
  auto pv_product = [&](const uint32_t (&pk)[NSB][8], const lds_char* vt_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int sb = t >> 1, hf = t & 1;
      u32x4 pv = {pk[sb][4 * hf + 0], pk[sb][4 * hf + 1], pk[sb][4 * hf + 2], pk[sb][4 * hf + 3]};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pv);
      bf16x8 vop[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x4 v0 = lds_read_tr16(vt_lds + 16 * t * ROWB + 256 * db + vrb[0]);
        const bf16x4 v1 = lds_read_tr16(vt_lds + 16 * t * ROWB + 256 * db + vrb[1]);
        vop[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(vop[db], pop, oacc[db]);
    }
  };
  auto compute_tile = [&](auto MASK, int kb, const lds_char* kt_lds, const lds_char* vt_lds) __attribute__((always_inline)) {
    uint32_t pk[NSB][8];
    scores_softmax(MASK, kb, kt_lds, pk);
    pv_product(pk, vt_lds);
  };

  // one key tile: wait for its copies, start the next tile's copies into
  // the other buffer, then compute on this one.  MAYMASK (std::true_type /
  // std::false_type) says whether the tile can need masking: tiles crossing
  // a band edge of the wave's rows, or the ragged last tile (keys past N_k,
  // which the copy read as zeros).  Unbanded loops never instantiate the
  // masked variant; their ragged last tile is peeled off the loop.
  auto tile_step = [&](auto MAYMASK, int kt, const lds_char* kt_lds, const lds_char* vt_lds,
                       lds_char* knext, lds_char* vnext) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < ntiles) issue_tile(kt + 1, knext, vnext);
    if (!wave_active) return;
    const int kb = kt * BC;
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
  if (kt0 < ntiles) issue_tile(kt0, K0, V0);
  for (int kt = kt0; kt < nloop; kt += 2) {
    tile_step(LOOP_MASK, kt, K0, V0, K1, V1);
    if (kt + 1 < nloop) tile_step(LOOP_MASK, kt + 1, K1, V1, K0, V0);
  }
  if (nloop < ntiles) {
    // the ragged last tile of an unbanded walk, from whichever buffer holds
    // it (picked at run time: no copy is in flight any more, so the
    // compiler has nothing to hold the reads back for)
    const bool odd = nloop & 1;
    tile_step(std::true_type{}, nloop, odd ? K1 : K0, odd ? V1 : V0, odd ? K0 : K1, odd ? V0 : V1);
  }

  // ---- epilogue: O = O_acc / l in bf16, LSE = (m + log2 l) ln 2; a row
  // that saw no key gets O = 0 and LSE = -inf.  A lane holds four
  // consecutive d of its row per 8-byte piece, so storing O directly
  // spreads every store instruction over 32 rows in 16-byte pieces.  Where
  // every wave's 32 rows fit in the K / V buffers (8 waves or fewer) they go
  // through LDS instead (each wave its own slice, in the staging layout of
  // fa_layout.h) and are read back a row per D / 8 lanes, so each store
  // instruction writes whole rows; the barrier waits for the last tile's
  // reads.  The 12-wave kernel keeps the direct stores: staging in
  // two passes made the compiler spill inside the key loop.
  constexpr bool STAGED = NW * 32 <= 4 * BC;
  if constexpr (STAGED) {
    __syncthreads();
    if (!wave_active) return;
    const float lt = sum_cross_half(l_run);
    const float inv = lt > 0.f ? fast_rcp(lt) : 0.f;
    if (row_valid && h2 == 0)
      a.lse[((size_t)b * a.H + h) * a.Nq + qrow] = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -__builtin_inff();
    constexpr int WPB = BC / 32;  // waves per buffer
    lds_char* stage = (lds_char*)(w < WPB ? k_lds0 : w < 2 * WPB ? k_lds1 : w < 3 * WPB ? v_lds0 : v_lds1) +
                      (w % WPB) * 32 * ROWB;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        *(lds_u32x2*)(stage + stage_off<D>(l32, 4 * db + g4, h2)) =
            u32x2{pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                  pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
      }
    // read back: lane l takes piece l % NCH of row 64 / NCH i + l / NCH
    constexpr int RPI = 64 / NCH;
    const int pc = l % NCH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + l / NCH;
      u32x4 v = *(const lds_u32x4*)(stage + (stage_off<D>(r, pc, 0) & ~15));
      if (stage_swap<D>(r)) v = u32x4{v[2], v[3], v[0], v[1]};
      if (qw + r < a.Nq) *(u32x4*)(a.o + q_off + (size_t)(qw + r) * rs + 8 * pc) = v;
    }
  } else {
    if (!wave_active) return;
    const float lt = sum_cross_half(l_run);
    const float inv = lt > 0.f ? fast_rcp(lt) : 0.f;
    if (!row_valid) return;
    __bf16* orow = a.o + q_off + (size_t)qrow * rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * h2;
        u32x2 val = {pack_bf16x2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                     pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + d0) = val;
      }
    if (h2 == 0)
      a.lse[((size_t)b * a.H + h) * a.Nq + qrow] = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -__builtin_inff();
  }
}

template <int D, int NW, int BC, bool BAND, bool WIN>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32;
  const int nqb = (a.Nq + BR - 1) / BR;
  dim3 grid((unsigned)(a.B * a.H * nqb));
  dim3 block(NW * 64);
  void* args[] = {(void*)&a};
  return hipLaunchKernel((const void*)fwd_kernel<D, NW, BC, BAND, WIN>, grid, block, args, 0, stream);
}

// d = 128: the causal and windowed kernels fit in 168 registers, so one
// 12-wave workgroup (384 query rows) runs three waves per SIMD.  That
// shrinks the workgroup count of a short sequence by a third, so it is used
// only where at least 1024 workgroups remain (four per CU); otherwise, and
// for full attention (whose kernel needs more registers), 8 waves of 256
// rows run two per SIMD.  d = 64: four waves per SIMD (at most 128
// registers); full attention runs the banded kernel with an unbounded band,
// which masks only the ragged last tile and fits those registers (the
// unbanded one needs 142).  Workgroups of 4 waves (128 rows, four per CU),
// or of 8 waves (256 rows, two per CU, each K/V tile copied once for twice
// the rows) for full attention when those fill the chip at least once (512
// workgroups): 8 waves measured 4-6% faster there, and slower on causal
// grids (coarser tiles on the diagonal) and on small grids.
hipError_t launch_fwd(const FwdArgs& a, int d, bool band, bool win, hipStream_t stream) {
  if (d == 128) {
    if (!band) return launch_fwd_t<128, 8, 64, false, false>(a, stream);
    const bool big = (long)a.B * a.H * ((a.Nq + 383) / 384) >= 1024;
    if (win) return big ? launch_fwd_t<128, 12, 64, true, true>(a, stream) : launch_fwd_t<128, 8, 64, true, true>(a, stream);
    return big ? launch_fwd_t<128, 12, 64, true, false>(a, stream) : launch_fwd_t<128, 8, 64, true, false>(a, stream);
  }
  if (win) return launch_fwd_t<64, 4, 64, true, true>(a, stream);
  if (!band && (long)a.B * a.H * ((a.Nq + 255) / 256) >= 512) return launch_fwd_t<64, 8, 64, true, false>(a, stream);
  return launch_fwd_t<64, 4, 64, true, false>(a, stream);
}

}  // namespace fa
