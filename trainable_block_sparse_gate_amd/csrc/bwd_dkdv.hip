// Gated block-sparse attention backward for gfx950: dK and dV.
//
// dk_u = scale sum_t dS_tu q_t and dv_u = sum_t P_tu dO_t over the query
// rows whose selection keeps u's block (review, section 3-6: gradients pass
// through the gated probabilities).  One workgroup per segment of a key
// block, from the per-key-block lists that the preparation kernels build: K and V stay in registers, Q/dO tiles of
// the keeping rows stream through LDS, dK^T and dV^T accumulate in
// registers.  Key blocks kept by many rows are split over several segments;
// each writes a partial sum and a second, small kernel adds them in segment
// order, so the result does not depend on the order the workgroups finish.
// Pages cited by title: "review" is the page "SAS: Simple Attention
// Sparsification via End-to-End Optimization of Context Ranking Review";
// "paper text" is the page "SAS: Simple Attention Sparsification via
// End-to-End Optimization of Context Ranking" that holds the paper's text.
#include <type_traits>

#include "sas_device.h"
#include "sas_launch.h"
#include "tile_stage.h"

namespace sas {
// ------------------------------------------------------------------ dk/dv
// Workgroup of 4 waves: wave = (query half qh, key half kh).  Each wave
// owns 32 keys (K, V as B operands in registers) and, per step, 32 of the
// 64 query rows of one head of one keeping row for S, dP, P and dS.  For
// bf16 the dV / dK products then split d instead of the query rows: wave
// (kh, qh) accumulates d tiles [qh NDT/2, (qh + 1) NDT/2) of its keys over
// all 64 rows, taking P and dS of the other query half from the wave that
// formed them (same keys) through LDS, so every wave holds half of the
// accumulators and no final reduction is needed.  fp32 keeps all d tiles
// per wave and adds the two query halves at the end.  The Q and dO tiles of a
// step go from global memory straight into LDS with global_load_lds (no
// register staging), into two buffers, one step ahead.  The row statistics
// (-lse / scale and -D, written per 64-row block by the dq phase) seed the
// S and dP products: for bf16 as one extra MFMA per product whose A operand
// is a per-row record [hi, mid, lo, 0, ...] of the value split into three
// bf16 parts (one 16-byte load per lane, a step ahead) and whose B operand
// is all ones, so every key column receives hi + mid + lo; for fp32 they
// come through LDS.  A bf16 workgroup then needs exactly 80 KB of LDS and
// at most 256 registers per lane, so two workgroups share a compute unit
// and one's softmax overlaps the other's products.  The products that
// contract over query rows read their operands transposed straight from
// the row-major tiles.
constexpr int kSegMax = 64;  // entries per segment the kernel can hold

// OUTER: the gate-position ablation: P from the ungated logits, dS =
// P (g dP - D), dV from P g (g the step's gate); -D then needs its own
// accumulator, since dP is scaled after the product.
template <typename T, int D, bool OUTER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_kernel(
    BwdParams p) {
  using M = Mfma<T>;
  constexpr int KS = M::K, E = M::E;
  constexpr int NKS = D / KS, NDT = D / 32, SPT = 32 / KS;
  constexpr int NBUF = 2;                         // LDS buffers per tile kind
  constexpr int TILE = kBlock * D;                // elements per tile
  constexpr int VEC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = D / VEC;                    // chunks per row
  constexpr int RPS = kWave / CPR;                // rows per 1 KB request
  constexpr int SPW = kBlock / RPS / 4;           // 1 KB requests per wave per tile
  constexpr bool kSplitD = (E == 8);              // dV / dK split over d (bf16)
  // requests per wave per step (fp32: one more, its piece of the statistics)
  constexpr int PER_STEP = kSplitD ? 2 * SPW : 2 * SPW + 1;
  constexpr int NACC = kSplitD ? NDT / 2 : NDT;   // d tiles accumulated per wave
  static_assert(kBlock % (4 * RPS) == 0, "tile rows must split evenly over the waves");
  static_assert(2 * NDT * 16 * kWave * 4 <= 2 * TILE * (int)sizeof(T),
                "a buffer holds one half of the final reduction");

  // Each buffer is its own LDS variable, so the compiler can tell that the
  // requests in flight into one buffer never alias reads of another and
  // inserts no wait for them; the loop below is unrolled over the buffers.
  __shared__ __attribute__((aligned(16))) T buf0[2 * TILE];  // [Q | dO][64][D]
  __shared__ __attribute__((aligned(16))) T buf1[2 * TILE];
  // bf16: P and dS of each wave as B operands, lane-linear
  // ([wave][P kc | dS kc][lane]); fp32: the row statistics of each buffer
  // ([buffer][wave][256]: waves 0 / 1 bring -lse / scale and -D in their
  // first 64 entries, the rest is filler that keeps every wave's request
  // count the same)
  constexpr int XCH_BYTES = 4 * 2 * SPT * kWave * 16, STAT_BYTES = 4 * 4 * kBlock * 4;
  __shared__ __attribute__((aligned(16))) char aux[kSplitD ? XCH_BYTES : NBUF * STAT_BYTES];
  static_assert(!kSplitD || 2 * 2 * TILE * sizeof(T) + XCH_BYTES <= 80 * 1024,
                "two bf16 workgroups fit one compute unit's LDS");

  const int w = blockIdx.x;
  const int nx = p.hkv * p.QB;
  if (w >= p.seg_off[nx]) return;
  int lo = 0, hi = nx - 1;  // largest x with seg_off[x] <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.seg_off[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int x = lo;
  const int kb = x / p.hkv, g = x % p.hkv;  // key-block major order
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, kb);
  const int q0 = p.cu_qblocks[s];
  const int j = kb - q0;
  const int seq_start = p.cu_seqlens[s];
  const int seq_len = p.cu_seqlens[s + 1] - seq_start;
  const int nvalid = min(kBlock, seq_len - j * kBlock);
  const long ktok0 = seq_start + (long)j * kBlock;
  const int nseg = p.seg_off[x + 1] - p.seg_off[x];
  const int seg = w - p.seg_off[x];
  const int cnt = p.count[x];
  const int e0 = seg * p.seg, e1 = min(cnt, e0 + p.seg);
  const int nent = max(0, e1 - e0);

  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int hf = lane / 32, l32 = lane % 32;
  const int kh = wave % 2, qh = wave / 2;
  const int key = 32 * kh + l32;  // this lane's key (column of S)

  // The segment's entries (query block << 8 | slot) and the slots' log
  // gates, entry l in lane l of every wave (a segment holds at most 64; a
  // step reads its entry with readlane, no memory round trip), then K and
  // V: all requested before anything waits.
  int my_ent = 0;
  float my_lg = 0.f;
  if (lane < nent) my_ent = p.list[(long)x * p.max_nb + e0 + lane];

  const T *q = static_cast<const T *>(p.q);
  const T *kk = static_cast<const T *>(p.k);
  const T *vv = static_cast<const T *>(p.v);
  const T *dO = static_cast<const T *>(p.dO_t);

  // keys past the block's end read its last row (finite values; their
  // probabilities are masked to zero and their sums never written), so the
  // loads need no branch and all issue back to back
  typename M::Op kreg[NKS], vreg[NKS];
  {
    const long base = ((ktok0 + min(key, nvalid - 1)) * p.hkv + g) * D + hf * E;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kreg[ks] = lds_op<T>(kk + base + ks * KS);
      vreg[ks] = lds_op<T>(vv + base + ks * KS);
    }
  }
  if (lane < nent) my_lg = p.sel_lg[((long)g * p.QB + (my_ent >> 8)) * p.Kb + (my_ent & 255)];
  f32x16 dkacc[NACC], dvacc[NACC];
#pragma unroll
  for (int dt = 0; dt < NACC; ++dt) dkacc[dt] = dvacc[dt] = f32x16{};

  // bf16 operand offsets (bytes) inside a tile, for this lane: the row
  // operand of chunk ks is at oq ^ 32 ks, the transposed operand of d tile
  // dt and 16-row chunk c at (ot0 ^ 64 dt) + 32 D c and (ot1 ^ 64 dt) + 32 D c
  // (the swizzle's XOR acts on bits the row offset leaves free, and it does
  // not depend on the row's multiple of 16)
  const int qrow = 32 * qh + chain_key_of_row<T>(l32);
  unsigned oq = 0, ot0 = 0, ot1 = 0;
  if constexpr (E == 8) {
    const int g4 = lane / 16, s16 = lane % 16;
    const int trow = 8 * (g4 / 2) + s16 / 4, tcol = 16 * (g4 % 2) + 4 * (s16 % 4);
    oq = 2u * Swz<T, D>::off(qrow, hf * E);
    ot0 = 2u * Swz<T, D>::off(trow, tcol);
    ot1 = 2u * Swz<T, D>::off(trow + 4, tcol);
  }

  const int G = p.G;
  const int nsteps = nent * G;

  auto tiles_of = [&](auto B) -> T * {
    if constexpr (decltype(B)::value == 0) return buf0;
    else return buf1;
  };
  auto stats_of = [&](auto B) -> float(*)[4 * kBlock] {
    return reinterpret_cast<float(*)[4 * kBlock]>(aux + decltype(B)::value * STAT_BYTES);
  };
  auto xch = [&](int wv, int slot) -> bf16x8 & {
    return reinterpret_cast<bf16x8 *>(aux)[(wv * 2 * SPT + slot) * kWave + lane];
  };

  // Requests of step st into buffer B: SPW 1 KB pieces (RPS rows) of the Q
  // tile and of the dO tile, for fp32 preceded by one piece of row
  // statistics (wave 0: -lse / scale, wave 1: -D, 16 lanes' worth repeated
  // over the wave).  Lane l of a request lands at byte 16 l of the piece, i.e.
  // at physical chunk l % CPR of its row; it fetches the logical chunk that
  // the swizzle puts there.  Rows past the block's end repeat its last row
  // (masked later).  Every wave issues exactly PER_STEP requests per step,
  // unconditionally (steps past the end re-fetch the last step into a
  // buffer that is not read again), so fixed wait counts are exact and the
  // compiler's own tracking of the requests stays precise.  step_req forms
  // the scalar part (row block and head of the step, clamped to the last
  // one, and the uniform bases of its rows).
  struct Req {
    const char *qbase, *dbase;
    const float *sbase;
    long srow;  // first statistics row of the step's block and head
    int nq;
  };
  auto step_req = [&](int st_req) -> Req {
    const int st = min(st_req, nsteps - 1);
    const int ent = __builtin_amdgcn_readlane(my_ent, st / G);
    const int qb = ent >> 8;  // packed query-block index
    const int i = qb - q0;
    const int h = g * G + st % G;
    const long t0 = seq_start + (long)i * kBlock;
    const long head0 = (t0 * p.hq + h) * D;
    const long srow = ((long)h * p.QB + qb) * kBlock;
    return Req{reinterpret_cast<const char *>(q + head0), reinterpret_cast<const char *>(dO + head0),
               ((wave & 1) ? p.Dbuf : p.Lbuf) + srow, srow, min(kBlock, seq_len - i * kBlock)};
  };
  // Request k of a step into buffer B (SPW pieces of Q, then SPW of dO;
  // fp32: k = 0 is this wave's piece of row statistics); per lane a 32-bit
  // byte offset (row, swizzled chunk) from the uniform base, so the request
  // takes a scalar base.
  auto issue_piece = [&](auto B, const Req &r, int k) {
    if constexpr (!kSplitD) {
      if (k == 0) {
        load_lds16(r.sbase + 4 * (lane % 16), &stats_of(B)[wave][0]);
        return;
      }
      k -= 1;
    }
    const int tk = k / SPW, sg = k % SPW;
    const unsigned rstride = (unsigned)(p.hq * D * (int)sizeof(T));
    const int piece = wave * SPW + sg;
    const int rw = piece * RPS + lane / CPR;
    const int rr = rw < r.nq ? rw : r.nq - 1;
    const int c = (lane % CPR) ^ Swz<T, D>::f(rw);
    const unsigned off = (unsigned)rr * rstride + (unsigned)(c * 16);
    load_lds16((tk == 0 ? r.qbase : r.dbase) + off, tiles_of(B) + tk * TILE + piece * RPS * D);
  };
  // bf16: the statistics of a step as MFMA A operands, from the records the
  // dq phase writes ([hi, mid, lo, 0 x 5] in bf16 per query row, 16 bytes):
  // this lane's query row, one load per statistic; with B all ones in the
  // lower half-wave (zero in the upper) the product puts hi + mid + lo into
  // every key column.
  bf16x8 stl = {}, stdd = {};
  const unsigned ones_w = hf == 0 ? 0x3F803F80u : 0u;  // two bf16 ones, or zeros
  // first query row of this lane's rows (register r holds row qlb0 + an
  // offset fixed by r)
  const int qlb0 = 32 * qh + chain_slot<T>(0, hf);
  auto load_stats = [&](const Req &r) {
    if constexpr (kSplitD) {
      stl = reinterpret_cast<const bf16x8 *>(p.Lbuf)[r.srow + qrow];
      stdd = reinterpret_cast<const bf16x8 *>(p.Dbuf)[r.srow + qrow];
    }
  };
  auto issue_step = [&](auto B, int st_req) {
    const Req r = step_req(st_req);
    load_stats(r);
#pragma unroll
    for (int k = 0; k < PER_STEP; ++k) issue_piece(B, r, k);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // One step from buffer B: request the step NBUF - 1 ahead into the buffer
  // the previous step read, compute, wait until this wave's requests of the
  // next step have landed (those further ahead may still be in flight),
  // barrier (every wave's requests visible, buffer B free for reuse).
  auto step = [&](auto B, int st) {
    constexpr int b = decltype(B)::value;
    // The offsets are opaque to the compiler from here on, so the per-chunk
    // offsets are formed in each step (one XOR each) rather than all held in
    // registers across the loop.
    unsigned aq = oq, a0 = ot0, a1 = ot1, ow = ones_w;
    int qlb = qlb0;
    asm volatile("" : "+v"(aq), "+v"(a0), "+v"(a1), "+v"(ow), "+v"(qlb));
    // the requests of step st + NBUF - 1 go out one per product pair below:
    // issued back to back they would hold up this wave's products while the
    // address unit works through every wave's requests
    using BN = std::integral_constant<int, (b + NBUF - 1) % NBUF>;
    const Req rq = step_req(st + NBUF - 1);

    const int e = st / G;
    const int i = (__builtin_amdgcn_readlane(my_ent, e) >> 8) - q0;
    const int nq = min(kBlock, seq_len - i * kBlock);
    const float lg2 = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_lg), e)) * kLog2e;
    const float lz = OUTER ? 0.f : lg2;             // the gate's term in the logits
    const float gate = OUTER ? fast_exp2(lg2) : 1.f;  // the gate on the values
    const bool diag = (i == j);
    const T *Qs = tiles_of(B);
    const T *Ds = Qs + TILE;

    // S[query][key] and dP[query][key] for 32 queries x this wave's 32 keys;
    // query rows loaded in chain order so P and dS feed the next products.
    // The products start from the row statistics, so that after them
    //   sacc = S - lse / scale   and   pacc = dP - D,
    // and P = exp2(scale_log2 * sacc + lg2), dS = P * pacc take no further
    // per-row term.
    f32x16 sacc, pacc, dacc;  // dacc: -D (outer gate only)
    if constexpr (kSplitD) {
      // one product per statistic (see load_stats); the registers are then
      // free for the next step's statistics, requested right away
      typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4v{ow, ow, ow, ow});
      sacc = M::run(stl, ones, f32x16{});
      if constexpr (OUTER) {
        dacc = M::run(stdd, ones, f32x16{});
        pacc = f32x16{};
      } else {
        pacc = M::run(stdd, ones, f32x16{});
      }
      load_stats(rq);
    } else {
      // this lane's 16 rows, in register order, read one by one
      const float(*stat)[4 * kBlock] = stats_of(B);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = stat[0][32 * qh + chain_slot<T>(r, hf)];
        pacc[r] = stat[1][32 * qh + chain_slot<T>(r, hf)];
        if constexpr (OUTER) {
          dacc[r] = pacc[r];
          pacc[r] = 0.f;
        }
      }
    }
    // operands are read RA chunks ahead of the products that use them, in
    // regions fenced by scheduling barriers, so the reads' latency overlaps
    // the products while only a short window of them is held in registers
    typename M::Op qa[NKS], da[NKS];
    auto read_row_ops = [&](int ks) {
      if constexpr (E == 8) {
        const char *at = reinterpret_cast<const char *>(Qs) + (aq ^ (32u * ks));
        qa[ks] = *reinterpret_cast<const bf16x8 *>(at);
        da[ks] = *reinterpret_cast<const bf16x8 *>(at + 2 * TILE);
      } else {
        qa[ks] = tile_op<T, D>(Qs, qrow, hf * E + ks * KS);
        da[ks] = tile_op<T, D>(Ds, qrow, hf * E + ks * KS);
      }
    };
    constexpr int RA = NKS < 2 ? NKS : 2;
#pragma unroll
    for (int ks = 0; ks < RA; ++ks) read_row_ops(ks);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (E == 8) __builtin_amdgcn_sched_barrier(0);
      if (ks < PER_STEP) issue_piece(BN{}, rq, ks);
      if (ks + RA < NKS) read_row_ops(ks + RA);
      sacc = M::run(qa[ks], kreg[ks], sacc);
      pacc = M::run(da[ks], vreg[ks], pacc);
    }
#pragma unroll
    for (int k = NKS; k < PER_STEP; ++k) issue_piece(BN{}, rq, k);
    if constexpr (E == 8) __builtin_amdgcn_sched_barrier(0);
    // P = exp2(scale_log2 * sacc + lg2) and dS = P * pacc, in place
    auto probabilities = [&]() {
      // full tiles (the common case) need no mask; the test is uniform
      if (!diag && nq == kBlock && nvalid == kBlock) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(sacc[r], p.scale_log2, lz));
          if constexpr (OUTER) {
            pacc[r] = pr * fmaf(gate, pacc[r], dacc[r]);
            sacc[r] = pr * gate;
          } else {
            sacc[r] = pr;
            pacc[r] = pr * pacc[r];
          }
        }
      } else {
        // row of register r: qlb + o, o fixed by r
        const bool key_ok = key < nvalid;
        const int kq = key - qlb;
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = chain_slot<T>(r, 0) - chain_slot<T>(0, 0);
          const bool ok = key_ok && qlb < nq - o && !(diag && kq > o);
          const float pr = fast_exp2(ok ? fmaf(sacc[r], p.scale_log2, lz) : -INFINITY);
          if constexpr (OUTER) {
            pacc[r] = pr * fmaf(gate, pacc[r], dacc[r]);
            sacc[r] = pr * gate;
          } else {
            sacc[r] = pr;
            pacc[r] = pr * pacc[r];
          }
        }
      }
    };
    // dV^T[d][key] += dO^T[d][query] P[query][key];  dK^T += Q^T dS
    if constexpr (kSplitD) {
      // this wave's d tiles over all four 16-row chunks: the transposed dO
      // and Q operands (chunk c at 32 D c bytes), requested once the
      // probabilities are formed (requesting the first half before them
      // holds 32 more registers across the exponentials: it spilled and
      // measured 20 % slower)
      constexpr int NC = 2 * SPT;
      auto trans_op = [&](const T *X, int c, int dt) -> bf16x8 {
        const char *tb = reinterpret_cast<const char *>(X) + c * 32 * D;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(const lds_short *)(tb + (a0 ^ (64u * dt))));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(const lds_short *)(tb + (a1 ^ (64u * dt))));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // [cc]: chunk (cc + SPT qh) % NC, i.e. the own query half first (its
      // products need nothing from the partner); indices stay compile-time
      bf16x8 tdo[NACC][NC], tq[NACC][NC];
      auto read_trans = [&](int cc0) {
#pragma unroll
        for (int cc = cc0; cc < cc0 + SPT; ++cc) {
          const int c = (cc + qh * SPT) % NC;
#pragma unroll
          for (int dl = 0; dl < NACC; ++dl) {
            tdo[dl][cc] = trans_op(Ds, c, qh * NACC + dl);
            tq[dl][cc] = trans_op(Qs, c, qh * NACC + dl);
          }
        }
      };
      probabilities();
      read_trans(0);
      bf16x8 own[2][SPT];
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        own[0][kc] = regs_op<T>(sacc, kc * E);
        own[1][kc] = regs_op<T>(pacc, kc * E);
      }
#pragma unroll
      for (int dl = 0; dl < NACC; ++dl)
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc) {
          dvacc[dl] = M::run(tdo[dl][kc], own[0][kc], dvacc[dl]);
          dkacc[dl] = M::run(tq[dl][kc], own[1][kc], dkacc[dl]);
        }
      read_trans(SPT);  // the other half's operands, between those products
#pragma unroll
      for (int k = 0; k < 2 * NACC * SPT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
      }
      // P and dS go to the partner only after this wave's transposed reads
      // are issued: a transposed read issued while LDS writes of the same
      // wave are in flight has returned wrong data
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        xch(wave, kc) = own[0][kc];
        xch(wave, SPT + kc) = own[1][kc];
      }
      // the partner's P and dS (same keys, other query half) are in LDS
      __builtin_amdgcn_sched_barrier(0);
      barrier_keep_requests();
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 oth[2][SPT];
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        oth[0][kc] = xch(wave ^ 2, kc);
        oth[1][kc] = xch(wave ^ 2, SPT + kc);
      }
#pragma unroll
      for (int dl = 0; dl < NACC; ++dl)
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc) {
          dvacc[dl] = M::run(tdo[dl][SPT + kc], oth[0][kc], dvacc[dl]);
          dkacc[dl] = M::run(tq[dl][SPT + kc], oth[1][kc], dkacc[dl]);
        }
    } else {
      probabilities();
      // (the transposed reads of one d tile are issued a tile ahead)
      typename M::Op ta[2][2 * SPT];
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        ta[0][2 * kc] = tile_op_rows<T, D>(Ds, 32 * qh + kc * KS, 0);
        ta[0][2 * kc + 1] = tile_op_rows<T, D>(Qs, 32 * qh + kc * KS, 0);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        if (dt + 1 < NDT) {
#pragma unroll
          for (int kc = 0; kc < SPT; ++kc) {
            ta[(dt + 1) & 1][2 * kc] = tile_op_rows<T, D>(Ds, 32 * qh + kc * KS, 32 * (dt + 1));
            ta[(dt + 1) & 1][2 * kc + 1] = tile_op_rows<T, D>(Qs, 32 * qh + kc * KS, 32 * (dt + 1));
          }
        }
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc) {
          dvacc[dt] = M::run(ta[dt & 1][2 * kc], regs_op<T>(sacc, kc * E), dvacc[dt]);
          dkacc[dt] = M::run(ta[dt & 1][2 * kc + 1], regs_op<T>(pacc, kc * E), dkacc[dt]);
        }
      }
    }
    wait_vmem<0>();
    barrier_keep_requests();
  };

  // Prologue: step 0.  Waiting for it -- and for K and V -- leaves no
  // request in flight at the loop entry, which keeps the compiler's tracking
  // of which buffer a request targets exact in the loop.
  if (nsteps > 0) {
    issue_step(I0{}, 0);
    wait_vmem<0>();
    barrier_keep_requests();
    for (int st = 0; st < nsteps; st += NBUF) {
      step(I0{}, st);
      if (st + 1 < nsteps) step(I1{}, st + 1);
    }
    // the last requests (re-fetches past the end) land before the buffers
    // are reused below
    wait_vmem<0>();
  }
  // lane holds key `key`, 4 consecutive d per register group
  auto write_out = [&](int dt0) {
    float *dk_out, *dv_out;
    if (nseg == 1) {
      if (key >= nvalid) return;
      dk_out = p.dk + ((ktok0 + key) * p.hkv + g) * D;
      dv_out = p.dv + ((ktok0 + key) * p.hkv + g) * D;
    } else {
      float *part = p.partial + (long)w * 2 * kBlock * D;
      dk_out = part + (long)key * D;
      dv_out = part + (long)(kBlock + key) * D;
    }
#pragma unroll
    for (int dl = 0; dl < NACC; ++dl)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * (dt0 + dl) + d_row(4 * rg, hf);
        *reinterpret_cast<float4 *>(dk_out + d0) =
            make_float4(dkacc[dl][4 * rg] * p.scale, dkacc[dl][4 * rg + 1] * p.scale,
                        dkacc[dl][4 * rg + 2] * p.scale, dkacc[dl][4 * rg + 3] * p.scale);
        *reinterpret_cast<float4 *>(dv_out + d0) =
            make_float4(dvacc[dl][4 * rg], dvacc[dl][4 * rg + 1], dvacc[dl][4 * rg + 2],
                        dvacc[dl][4 * rg + 3]);
      }
  };
  if constexpr (kSplitD) {
    write_out(qh * NACC);  // each wave owns distinct d tiles of its keys
  } else {
    // every wave's requests have landed (each waited for its own above)
    // before any wave writes into the buffers
    __syncthreads();
    // Add the two query halves: waves qh = 1 hand their sums to qh = 0
    // (dK through buffer 0, dV through buffer 1).
    float *redk = reinterpret_cast<float *>(buf0);
    float *redv = reinterpret_cast<float *>(buf1);
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          redk[(kh * NDT * 16 + dt * 16 + r) * kWave + lane] = dkacc[dt][r];
          redv[(kh * NDT * 16 + dt * 16 + r) * kWave + lane] = dvacc[dt][r];
        }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dkacc[dt][r] += redk[(kh * NDT * 16 + dt * 16 + r) * kWave + lane];
          dvacc[dt][r] += redv[(kh * NDT * 16 + dt * 16 + r) * kWave + lane];
        }
      write_out(0);
    }
  }
}

// Sum, in segment order, the nseg partials of split key block x into dk, dv.
template <int D>
__device__ void reduce_key_block(const BwdParams &p, int x, int nseg) {
  const int kb = x / p.hkv, g = x % p.hkv;  // key-block major order
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, kb);
  const int j = kb - p.cu_qblocks[s];
  const int seq_start = p.cu_seqlens[s];
  const int nvalid = min(kBlock, p.cu_seqlens[s + 1] - seq_start - j * kBlock);
  const long ktok0 = seq_start + (long)j * kBlock;
  const int n = kBlock * D;
  const float *part0 = p.partial + (long)p.seg_off[x] * 2 * n;
  // each thread owns NV float4s of the 2 n sums; a segment's NV loads are
  // all issued before any is added
  constexpr int NV = 2 * kBlock * D / (256 * 4);
  float4 acc[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sg = 0; sg < nseg; ++sg) {
    float4 v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u)
      v[u] = *reinterpret_cast<const float4 *>(part0 + (long)sg * 2 * n + 4 * (threadIdx.x + 256 * u));
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      acc[u].x += v[u].x; acc[u].y += v[u].y; acc[u].z += v[u].z; acc[u].w += v[u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = 4 * (threadIdx.x + 256 * u);
    const int which = e / n, kk2 = (e % n) / D, d = e % D;
    if (kk2 >= nvalid) continue;
    float *out = (which == 0 ? p.dk : p.dv) + ((ktok0 + kk2) * p.hkv + g) * D + d;
    *reinterpret_cast<float4 *>(out) = acc[u];
  }
}

// Split key blocks: add the partials of their segments in segment order
// (a separate launch, so the partials are visible without device-scope
// fences inside the dK/dV kernel).  Each workgroup walks a strided share of
// the key blocks and skips those that were not split.
constexpr int kReduceWgs = 256;

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdParams p) {
  for (int x = blockIdx.x; x < p.hkv * p.QB; x += gridDim.x) {
    const int nseg = p.seg_off[x + 1] - p.seg_off[x];
    if (nseg > 1) reduce_key_block<D>(p, x, nseg);
  }
}

// ------------------------------------------------------------------ launch
template <typename T, int D>
static hipError_t launch_dkdv_t(const BwdParams &p, hipStream_t stream) {
  if (p.outer)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3(p.U), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), dim3(p.U), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D>), dim3(min(kReduceWgs, p.hkv * p.QB)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                           hipStream_t stream) {
  (void)out_bf16;  // dO reaches this kernel in the input dtype (p.dO_t)
  if (dtype_bf16)
    return head_dim == 128 ? launch_dkdv_t<__bf16, 128>(p, stream)
                           : launch_dkdv_t<__bf16, 64>(p, stream);
  return head_dim == 128 ? launch_dkdv_t<float, 128>(p, stream)
                         : launch_dkdv_t<float, 64>(p, stream);
}

}  // namespace sas
