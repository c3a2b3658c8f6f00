// fa_fwd.hip - gfx950 forward attention kernels (bf16 MFMA path and fp32 path).
//
// The computation is the tiled forward of the FlashAttention optimisation
// page (intelliparadigm.com), section 4.1, and of the tiled code on the
// FlashAttention-2 principle and deployment page (yunthe.com): for each block
// of query rows, stream the key/value blocks, form the block of scores, raise
// the running row maximum, rescale the running sum and the partial output by
// e^(m_old - m_new), add the block's exp(S - m_new) terms, and divide by the
// running sum at the end.  The merge rule is Eq. (2) of the Journal of
// Software 2026(1) p.218 survey.  The per-row statistic written for the
// backward pass is LSE = m + ln(l).
//
// gfx950 mapping of the bf16 kernel (one workgroup = 4 or 8 waves = 128 or
// 256 query rows of one head; on grids too small to give every SIMD two
// waves, 8 waves = 128 or 64 rows whose keys are split over 2 or 4 waves):
//  * each wave owns 32 whole query rows, so the row statistics m and l never
//    leave the wave until the key parts of a row are merged (Eq. (2)) at the
//    end;
//  * the wave computes S^T = K_j Q_i^T with v_mfma_f32_32x32x16_bf16: the
//    accumulator puts one query per lane (lane % 32) and that query's keys in
//    the lane's registers, so the row max and row sum are mostly in-lane
//    reductions plus one exchange between lanes l and l+32;
//  * it then computes O^T += V_j^T P^T, which again keeps one query per lane,
//    so rescaling and the final division are in-lane; P^T is fed to the MFMA
//    straight from the score registers (rounded to bf16), never via memory;
//  * the Q fragment stays in VGPRs for the whole KV sweep; K_j and V_j are
//    copied from HBM straight into LDS, row-major under one XOR swizzle that
//    keeps both the 128-bit K row reads and the transposing V^T reads
//    (ds_read_b64_tr_b16) free of bank conflicts, and double buffered so the
//    loads of tile j+1 overlap the MFMAs of tile j;
//  * the exponentials are exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.h"
#include "fa_validate.h"

namespace fa {

// When the reference of a row moves, it moves to the row max unless that
// leads the old reference by at most this much (log2 units).
constexpr float kLazyRescale = 8.f;
// The reference moves only on a tile where a lane's sum of P over its 32
// elements reaches kSumBound (so some P >= 2^35), or while the row has none.
// Until then every P < 2^40: with at most 2^22 keys, l stays below 2^62 and
// O below 2^62 * max|V|, finite for |V| <= 2^64 (the documented input limit),
// and no precision is lost (a floating-point P keeps its relative precision
// at any scale).  Rows whose
// scores keep climbing (large-spread scores) therefore rarely take the
// rescale path, which every row of the wave then pays for.
constexpr float kSumBound = 1099511627776.f;  // 2^40


template <int D, int NW_, int KQ_ = 1>
struct FwdTile {
  static constexpr int NW = NW_;                  // waves per workgroup (4 or 8)
  static constexpr int KQ = KQ_;                  // key parts per workgroup (1, 2 or 4)
  static constexpr int RG = NW / KQ;              // 32-row groups per workgroup
  static constexpr int NT = 64 * NW;              // threads per workgroup
  static constexpr int BR = 32 * RG;              // query rows per workgroup
  static constexpr int BC = KQ == 4 && D > 64 ? 32 : 64;  // keys per KV tile (four parts' stages in 128 KiB)
  static constexpr int KS = D / 16;               // 16-wide k steps of Q K^T
  static constexpr int DB = D / 32;               // 32-column blocks of O
  static constexpr int KB = BC / 32;              // 32-key blocks of S
  static constexpr int PS = BC / 16;              // 16-key k steps of P V
  static constexpr int RS = lds_row_bytes<D>();   // bytes per tile row in LDS (K and V alike)
  static constexpr int GRS = D * 2;               // bytes per row in HBM
  static constexpr int TILE = BC * RS;            // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;          // K tile then V tile
  static constexpr int LPW = TILE / 1024 / RG;    // 1 KiB direct-to-LDS loads per wave per tile
  static_assert(TILE % (1024 * RG) == 0, "tile must split into 1 KiB loads over the waves of a key part");
  static_assert(NW % KQ == 0, "every key part has the same row groups");
};

// Key-split mode: the keys of every row are cut into ranges of TPS whole
// tiles; part p of a row covers tiles [p*TPS, (p+1)*TPS).  Each part writes
// its normalised output in fp32 to OP[p][B][H][N][d] and its log-sum-exp to
// LP[p][B][H][N]; a row that sees no key in its range gets O = 0 and
// LSE = -inf.  The parts are merged by lse_merge_kernel (Eq. (2)).
struct SplitArgs {
  int S, TPS;
  float* OP;
  float* LP;
  long long part_elems, part_rows;  // B*H*N*d and B*H*N
};


template <typename E, int D, bool CAUSAL, int NW, bool SPLIT, int MODE, bool DROP, int KQ = 1>
__global__ void __launch_bounds__(64 * NW, D == 256 ? 1 : 8 / NW)
fwd_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V, E* __restrict__ O,
           float* __restrict__ LSE, int N, int Tr, float c, SplitArgs sp, MaskArgs mk, DropArgs dp) {
  using T = FwdTile<D, NW, KQ>;
  using v8 = typename Vec<E>::v8;
  using v4 = typename Vec<E>::v4;
  constexpr bool WINDOW = MODE == kMaskWindow, BLOCKS = MODE == kMaskBlocks;
  static_assert(KQ == 1 || (NW == 8 && D <= 128 && !SPLIT && MODE == kMaskDense),
                "key parts only in the eight-wave dense or causal forward");
  static_assert(!(SPLIT && MODE != kMaskDense), "key split only with the dense or causal mask");
  static_assert(!DROP || (!SPLIT && MODE == kMaskDense), "dropout only on the plain forward");
  static_assert(!BLOCKS || (T::BC == kMaskBlock && T::BR == 2 * kMaskBlock), "mask blocks are key tiles and half a row block");
  // The two stages are separate arrays: with one array the compiler cannot
  // tell the direct loads of the next tile from the reads of this one and
  // waits for those loads before the transposing V reads.
  // Stage s of key part p: (s ? smem1 : smem0) + p * STAGE.
  __shared__ __attribute__((aligned(1024))) char smem0[KQ * T::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[KQ * T::STAGE];
  __shared__ unsigned short tlist[BLOCKS ? kMaxMaskTiles : 1];
  __shared__ int tcount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses for the direct loads
  // With KQ key parts, wave w takes the rows of row group w % RG and the keys
  // of part w / RG: the parts of a row run side by side on different SIMDs.
  const int rg = KQ == 1 ? wave : wave % T::RG;
  const int kp = KQ == 1 ? 0 : wave / T::RG;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int per_head = SPLIT ? Tr * sp.S : Tr;  // the parts of a query block are adjacent
  int bh, it, part = 0;
  if (CAUSAL && !SPLIT) {
    int r;
    causal_order(blockIdx.x, gridDim.x / Tr, Tr, bh, r);
    it = Tr - 1 - r;  // longest rows first
  } else {
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    bh = tile / per_head;
    const int rem = tile - bh * per_head;
    part = SPLIT ? rem % sp.S : 0;
    it = SPLIT ? rem / sp.S : rem;
    if (CAUSAL) it = Tr - 1 - it;  // longest rows first
  }
  const int q0 = it * T::BR;
  const size_t head = size_t(bh) * N * D;
  const E* Kh = K + head;
  const E* Vh = V + head;
  const int head_bytes = N * T::GRS;

  // Q fragment (B operand of S^T = K Q^T): row qrow, columns 16*s + 8*half .. +7.
  // Rows past N read as zero (buffer bounds).
  const int wq0 = q0 + rg * 32;
  const int qrow = wq0 + l32;
  v8 qf[T::KS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head, head_bytes);
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
      qf[s] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                                             rq, qrow * T::GRS + (16 * s + 8 * half) * 2, 0, 0));
  }

  const int Tc = (N + T::BC - 1) / T::BC;
  int nt = Tc;
  if (CAUSAL) nt = min(Tc, (min(q0 + T::BR, N) - 1) / T::BC + 1);
  const bool wave_active = wq0 < N;
  int nt_w = nt;
  if (CAUSAL && wave_active) nt_w = min(nt, (min(wq0 + 32, N) - 1) / T::BC + 1);
  // this workgroup's tiles: [j0, nt); each wave computes [w0, nt_w)
  int j0 = 0, w0 = 0;
  if (SPLIT) {
    j0 = part * sp.TPS;
    nt = min(nt, j0 + sp.TPS);
    nt_w = min(nt_w, nt);
  }
  if (WINDOW) {
    // tiles that hold a key of the band [i - left, i + right] of some row i
    const int lo = mk.left >= 0 ? max(0, q0 - mk.left) : 0;
    const int hi = mk.right >= 0 ? min(N, q0 + T::BR + mk.right) : N;  // exclusive
    j0 = lo / T::BC;
    nt = (hi - 1) / T::BC + 1;
    w0 = mk.left >= 0 ? max(0, wq0 - mk.left) / T::BC : 0;
    nt_w = mk.right >= 0 ? (min(N, wq0 + 32 + mk.right) - 1) / T::BC + 1 : Tc;
  }
  // block-sparse: the workgroup's tiles, in order, in tlist[0 .. tcount),
  // each with the keep flags of the workgroup's two 64-row blocks; a wave
  // (rows of block wave / 2) computes a tile only if its own block keeps it
  if (BLOCKS) {
    const int h = bh % mk.H;
    const unsigned char* bmh = mk.bm + mk.bm_head_stride * h;
    if (wave == 0) {
      const unsigned char* r0 = bmh + size_t(q0 / kMaskBlock) * mk.nb;
      const bool two = q0 + kMaskBlock < N;  // the workgroup's second 64-row block exists
      int n = 0;
      for (int base = 0; base < nt; base += 64) {
        const int jj = base + lane;
        const bool a0 = jj < nt && r0[jj] != 0;
        const bool a1 = jj < nt && two && r0[mk.nb + jj] != 0;
        const bool keep = a0 || a1;
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1));
        if (keep) tlist[n + below] = list_entry(jj, a0, a1);
        n += __builtin_popcountll(bal);
      }
      if (lane == 0) tcount = n;
    }
    __syncthreads();
  }
  // Key part kp takes tiles [pj0, pj1) of the workgroup's [j0, nt), tpk
  // steps for every part, so that all waves meet the same barriers.
  int tpk = nt - j0, pj0 = j0, pj1 = nt;
  if (KQ > 1) {
    tpk = (nt - j0 + KQ - 1) / KQ;
    pj0 = j0 + kp * tpk;
    pj1 = min(nt, pj0 + tpk);
  }
  const int cnt = BLOCKS ? tcount : tpk;                  // steps of the workgroup
  const int cnt_w = BLOCKS ? cnt : max(0, pj1 - pj0);     // steps with a tile of this wave's part
  auto tile_at = [&](int idx) { return BLOCKS ? list_index(tlist[idx]) : pj0 + idx; };
  auto wave_needs = [&](int idx, int j) {
    if (!wave_active || j >= nt_w || j < w0) return false;
    return !BLOCKS || list_keeps(tlist[idx], wave >> 1);
  };

  // Direct-to-LDS tile loads: load i of this wave fills LDS bytes
  // [(rg*LPW + i) KiB, +1 KiB) of its part's tile; lane l brings the 16 bytes that
  // belong at byte 16*l of that range under the swizzle.
  int goff[T::LPW];
#pragma unroll
  for (int i = 0; i < T::LPW; ++i) goff[i] = swz_src<D>((rg * T::LPW + i) * 1024 + 16 * lane);
  auto issue_loads = [&](int j, int stage, bool valid = true) {
    const int key0 = valid ? j * T::BC : 0;
    const int bytes = valid ? (N - key0) * T::GRS : 0;  // not valid: the loads read nothing
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + size_t(key0) * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + size_t(key0) * D, bytes);
    char* kdst = (stage ? smem1 : smem0) + kp * T::STAGE + rg * T::LPW * 1024;
#pragma unroll
    for (int i = 0; i < T::LPW; ++i)
      load_lds16(rk, kdst + i * 1024, goff[i]);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i)
      load_lds16(rv, kdst + T::TILE + i * 1024, goff[i]);
  };

  // LDS read offsets (bytes within a stage).
  // K rows kb*32 + l32, logical unit 2*st + half.
  int kof[T::KS];
#pragma unroll
  for (int st = 0; st < T::KS; ++st) kof[st] = l32 * T::RS + (((2 * st + half) ^ tile_swz<D>(l32)) * 16);
  // V transposing reads: in 16-lane group g (lane t), row 4*(g/2) + 8*r2 + t/4
  // (+16 per PV k step), columns 32*b + 16*(g%2) + 4*(t%4) .. +3.
  int vof[T::DB][2];
  {
    const int g = lane >> 4, t = lane & 15;
#pragma unroll
    for (int b = 0; b < T::DB; ++b)
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const int row = 4 * (g >> 1) + 8 * r2 + (t >> 2);
        const int col = 32 * b + 16 * (g & 1) + 4 * (t & 3);
        vof[b][r2] = T::TILE + row * T::RS + (((col >> 3) ^ tile_swz<D>(row)) * 16) + (col & 7) * 2;
      }
  }

  f32x16 o[T::DB];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) o[b] = f32x16{};
  float m = -INFINITY;  // reference (running max) of scale*log2(e)*score
  float mu = 0.f;       // m, or 0 while m is -inf: the value subtracted before exp2
  float l = 0.f;        // running sum over this lane's half of the keys

  auto compute = [&](int j, const char* base, int nj, bool has_next, int nstage) {
    // ---- S^T = K_j Q^T: one independent chain per 32-key block; K operands are read
    // KPF k steps ahead, an order pinned by scheduling barriers (left alone,
    // the scheduler pulls each read next to its MFMA and the LDS latency shows)
    f32x16 s[T::KB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) s[kb] = f32x16{};
    constexpr int KPF = 2;
    v8 kr[KPF][T::KB];
#pragma unroll
    for (int st = 0; st < KPF; ++st)
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) kr[st][kb] = *reinterpret_cast<const v8*>(base + kof[st] + kb * 32 * T::RS);
#pragma unroll
    for (int st = 0; st < T::KS; ++st) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) s[kb] = mfma32(kr[st % KPF][kb], qf[st], s[kb]);
      if (st + KPF < T::KS)
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
          kr[st % KPF][kb] = *reinterpret_cast<const v8*>(base + kof[st + KPF] + kb * 32 * T::RS);
    }
    // the next tile's direct loads go out one after each of the first MFMA
    // groups: issued in one burst at the top of the step, they held the wave
    // at the vector memory unit while its matrix unit had nothing to do
    issue_loads(nj, nstage, has_next);
    __builtin_amdgcn_sched_group_barrier(0x100, T::KB * KPF, 0);
#pragma unroll
    for (int st = 0; st < T::KS; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, T::KB, 0);
      if (st + KPF < T::KS) __builtin_amdgcn_sched_group_barrier(0x100, T::KB, 0);
      if (st < 2 * T::LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    // ---- masks: keys past N and, if causal, keys after the query; for a
    // window, keys outside [qrow - left, qrow + right].  Only tiles that cross
    // one of these edges for some row of the wave pay for the element mask.
    const int key0 = j * T::BC;
    bool need = key0 + T::BC > N;
    if (CAUSAL) need = need || (key0 + T::BC - 1 > wq0);
    if (WINDOW)
      need = need || (mk.left >= 0 && key0 < wq0 + 31 - mk.left) || (mk.right >= 0 && key0 + T::BC - 1 > wq0 + mk.right);
    if (need) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + acc_row(r, lane);
          bool hide = key >= N || (CAUSAL && key > qrow);
          if (WINDOW) hide = hide || (mk.left >= 0 && key < qrow - mk.left) || (mk.right >= 0 && key > qrow + mk.right);
          if (hide) s[kb][r] = -INFINITY;
        }
    }
    // ---- online softmax (scale > 0, so max(score)*c == max(score*c)).
    // P = exp2(S*c - mu) is taken against the row's current reference first.
    // The reference m moves (and O, l are rescaled) only on a tile where this
    // lane's half-row sum reaches kSumBound, or while the row has no reference
    // yet (m = -inf, no key seen).  Otherwise every P stays below kSumBound;
    // softmax is invariant to the reference.  The row max is taken only on
    // those rare tiles, and their exponentials are taken again against the
    // new reference.
    // P is rounded to the input type for the PV product; l sums the fp32
    // values (before dropout: the statistic is that of the softmax itself).
    // With dropout, bit kb*16 + r of `keep` says whether element (kb, r)
    // survives: registers 4m .. 4m+3 of a key block hold 4 consecutive keys of
    // this row, one Philox block row.
    // The four lanes of a quad hold rows 4q .. 4q+3 (one Philox block row
    // each) and the same keys, so they need the same four calls per key
    // block: lane t makes the call of key group t and the quad shares it.
    unsigned keep = 0;
    if constexpr (DROP) {
      const unsigned t = lane & 3;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const unsigned key = unsigned(j * T::BC + kb * 32 + 8 * t + 4 * half);
        const unsigned mine = keep_block_rows(dp, unsigned(qrow) >> 2, key >> 2, unsigned(bh));
        keep |= quad_share_nibbles(mine, t) << (kb * 16);
      }
    }
    v8 pb[T::PS];
    float rs;
    auto exps = [&]() {
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(fmaf(s[kb][r], c, -mu));
          rs += p;
          float pd = p;  // dropout: the kept P; the 1/(1-p) scale is applied to O at the end
          if constexpr (DROP) pd = keep_or_zero(p, keep, kb * 16 + r);
          pb[kb * 2 + (r >> 3)][r & 7] = (E)pd;
        }
    };
    exps();
    if (__builtin_amdgcn_ballot_w64(m == -INFINITY || !(rs < kSumBound))) {
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      const float mxr = halves_max(mx) * c;
      const float m_new = (mxr > m + kLazyRescale) ? mxr : m;
      const float mu_new = (m_new == -INFINITY) ? 0.f : m_new;  // nothing visible yet in this row
      // O and l are still 0 while m is -inf: no factor then (exp2(0 - mu_new)
      // overflows when every score of the first visible tile is below -128)
      const float alpha = m == -INFINITY ? 0.f : exp2_fast(mu - mu_new);
      m = m_new;
      mu = mu_new;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < T::DB; ++b) o[b] *= alpha;
      exps();
    }
    l += rs;
    // ---- O^T += V_j^T P^T: DB independent chains; V^T operands come from two
    // transposing reads of the row-major V tile, VPF operands ahead
    auto vread = [&](int b, int ps) {
      const char* vb = base + ps * 16 * T::RS;
      const v4 lo = __builtin_bit_cast(
          v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(vb + vof[b][0])));
      const v4 hi = __builtin_bit_cast(
          v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(vb + vof[b][1])));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int VPF = 3;  // V operands in flight, in (ps, b) order
    constexpr int NV = T::PS * T::DB;
    v8 vr[VPF];
#pragma unroll
    for (int u = 0; u < VPF; ++u) vr[u] = vread(u % T::DB, u / T::DB);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int ps = u / T::DB, b = u % T::DB;
      o[b] = mfma32(vr[u % VPF], pb[ps], o[b]);
      if (u + VPF < NV) vr[u % VPF] = vread((u + VPF) % T::DB, (u + VPF) / T::DB);
    }
  };

  // step idx: tile tile_at(idx) from stage `stage`, loads of the next tile into the other
  // (inside compute when the wave computes this tile; after the last tile the
  // loads have size 0 and read nothing)
  auto step = [&](int idx, int stage) {
    const bool has_next = idx + 1 < cnt_w;
    const int nj = has_next ? tile_at(idx + 1) : 0;
    bool issued = false;
    if (idx < cnt_w) {
      const int j = tile_at(idx);
      if (wave_needs(idx, j)) {
        compute(j, (stage ? smem1 : smem0) + kp * T::STAGE, nj, has_next, stage ^ 1);
        issued = true;
      }
    }
    if (!issued && has_next) issue_loads(nj, stage ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of the next tile have landed
    __syncthreads();
  };

  if (cnt > 0) {  // uniform over the workgroup; an empty key part or mask row skips the sweep
    if (cnt_w > 0) issue_loads(tile_at(0), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    int idx = 0;
    for (; idx + 1 < cnt; idx += 2) {
      step(idx, 0);
      step(idx + 1, 1);
    }
    if (idx < cnt) step(idx, 0);
  }

  if constexpr (KQ > 1) {
    // The key parts of each row meet in LDS, by the merge rule of Eq. (2) in
    // halving rounds: parts [h, 2h) hand their (o, m, l) to parts [0, h).  A
    // part that saw no key has m = -inf, l = 0, o = 0 and weight 0.  The
    // stages are free (every wave has passed the sweep's last barrier).
    static_assert((KQ / 2) * T::RG * T::DB * 16 * 64 * 4 <= KQ * T::STAGE, "merge buffer fits in the stages");
    float* xo = reinterpret_cast<float*>(smem0);  // [h][RG][DB][16][64]
    float* xs = reinterpret_cast<float*>(smem1);  // [h][RG][2][64]: m, l
#pragma unroll
    for (int h = KQ / 2; h >= 1; h /= 2) {
      if (kp >= h && kp < 2 * h) {
        const int slot = (kp - h) * T::RG + rg;
#pragma unroll
        for (int b = 0; b < T::DB; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) xo[((slot * T::DB + b) * 16 + e) * 64 + lane] = o[b][e];
        xs[(slot * 2 + 0) * 64 + lane] = m;
        xs[(slot * 2 + 1) * 64 + lane] = l;
      }
      __syncthreads();
      if (kp < h) {
        const int slot = kp * T::RG + rg;
        const float m1 = xs[(slot * 2 + 0) * 64 + lane];
        const float l1 = xs[(slot * 2 + 1) * 64 + lane];
        const float mn = fmaxf(m, m1);
        const float a0 = m == -INFINITY ? 0.f : exp2_fast(m - mn);
        const float a1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - mn);
        l = l * a0 + l1 * a1;
#pragma unroll
        for (int b = 0; b < T::DB; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[b][e] = o[b][e] * a0 + xo[((slot * T::DB + b) * 16 + e) * 64 + lane] * a1;
        m = mn;
      }
      if (h > 1) __syncthreads();  // the next round's writers have read theirs
    }
    if (kp > 0) return;
  }
  if (!wave_active) return;
  const float lt = halves_sum(l);
  if (SPLIT) {
    // normalised fp32 part; rows that saw no key: O = 0, LSE = -inf
    const float pinv = lt > 0.f ? 1.f / lt : 0.f;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(sp.OP + size_t(part) * sp.part_elems + head, N * D * 4);
#pragma unroll
    for (int b = 0; b < T::DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(unsigned, o[b][4 * g + e] * pinv);
        __builtin_amdgcn_raw_buffer_store_b128(w, rp, qrow * D * 4 + (b * 32 + 8 * g + 4 * half) * 4, 0, 0);
      }
    if (half == 0 && qrow < N)
      sp.LP[size_t(part) * sp.part_rows + size_t(bh) * N + qrow] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
    return;
  }
  // a row that saw no key (block-sparse masks only): O = 0, LSE = -inf;
  // dropout scales the kept terms by 1/(1-p) here, in fp32
  float inv = (!BLOCKS || lt > 0.f) ? 1.f / lt : 0.f;
  if constexpr (DROP) inv *= dp.keep_scale;
  // rows past N are dropped by the buffer bounds
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + head, head_bytes);
#pragma unroll
  for (int b = 0; b < T::DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack2<E>(o[b][4 * g + 0] * inv, o[b][4 * g + 1] * inv);
      w[1] = pack2<E>(o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, qrow * T::GRS + (b * 32 + 8 * g + 4 * half) * 2, 0, 0);
    }
  if (half == 0 && qrow < N) LSE[size_t(bh) * N + qrow] = (!BLOCKS || lt > 0.f) ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 path: nothing is rounded below fp32.  Both products run on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32, same accumulator layout as the bf16
// MFMA): four waves of 32 query rows per workgroup, one query per lane,
// 32-key K/V tiles staged in LDS (fp32 rows padded by 16 bytes, so the
// 128-bit K reads of 16 consecutive rows fall on distinct banks), double
// buffered through registers.
//  * S^T = K_j Q^T: k step st pairs dims st (lanes l < 32) and D/2 + st
//    (lanes l >= 32), so a lane's Q fragment is one contiguous half row and
//    its K operands come four k steps at a time from one 128-bit LDS read;
//  * O^T += V_j^T P^T: k step r pairs the two keys that element r of the
//    score accumulator holds in lanes l and l + 32, so P^T is the lane's own
//    score register and V^T one float per lane of a V tile row.
// The online softmax is the bf16 kernel's (lazy reference, exp2 with the
// scale folded into one FMA).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, D == 256 ? 1 : 2)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, int N, int Tr, float c) {
  constexpr int BR = 128, BC = 32, H2 = D / 2, DB = D / 32;
  constexpr int RSF = D + 4;               // floats per LDS row
  constexpr int TILEF = BC * RSF;          // floats of one K or V tile
  constexpr int LDV = D / 4;               // float4 per row
  constexpr int LPT = BC * LDV / 256;      // float4 of the K (and of the V) tile each thread moves
  __shared__ __attribute__((aligned(16))) float sm[2][2 * TILEF];  // stage: K tile, then V tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  int bh, it;
  if (CAUSAL) {
    int r;
    causal_order(blockIdx.x, gridDim.x / Tr, Tr, bh, r);
    it = Tr - 1 - r;  // longest rows first
  } else {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    bh = t / Tr;
    it = t - bh * Tr;
  }
  const int q0 = it * BR;
  const size_t head = size_t(bh) * N * D;
  const int head_bytes = N * D * 4;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;

  // Q fragment: row qrow, dims half*D/2 .. +D/2-1 (rows past N read as zero)
  float qf[H2];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head, head_bytes);
#pragma unroll
    for (int t = 0; t < H2 / 4; ++t) {
      // (cast the whole vector: a bit cast of one vector element reads element 0)
      const f32x4 w = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * D + half * H2 + 4 * t) * 4, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * t + e] = w[e];
    }
  }

  const int Tc = (N + BC - 1) / BC;
  int nt = Tc;
  if (CAUSAL) nt = min(Tc, (min(q0 + BR, N) - 1) / BC + 1);
  const bool wave_active = wq0 < N;
  int nt_w = nt;
  if (CAUSAL && wave_active) nt_w = min(nt, (min(wq0 + 32, N) - 1) / BC + 1);

  // Tile j through registers: thread tid moves float4 number tid + 256 i of
  // the K tile and of the V tile; keys past N read as zero.
  f32x4 kreg[LPT], vreg[LPT];
  auto load_tile = [&](int j) {
    const int key0 = j * BC;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head + size_t(key0) * D, (N - key0) * D * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head + size_t(key0) * D, (N - key0) * D * 4);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = tid + 256 * i, row = idx / LDV, col = idx % LDV;
      kreg[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (row * D + 4 * col) * 4, 0, 0));
      vreg[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (row * D + 4 * col) * 4, 0, 0));
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = tid + 256 * i, row = idx / LDV, col = idx % LDV;
      *reinterpret_cast<f32x4*>(&sm[stage][row * RSF + 4 * col]) = kreg[i];
      *reinterpret_cast<f32x4*>(&sm[stage][TILEF + row * RSF + 4 * col]) = vreg[i];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};
  float m = -INFINITY;  // reference of scale*log2(e)*score
  float mu = 0.f;       // m, or 0 while m is -inf
  float l = 0.f;        // running sum over this lane's half of the keys

  auto compute = [&](int j, const float* ks, const float* vs) {
    // ---- S^T = K_j Q^T, K operands read two 128-bit groups ahead
    f32x16 s = f32x16{};
    const float* kp = ks + l32 * RSF + half * H2;
    f32x4 kq[2] = {*reinterpret_cast<const f32x4*>(kp), *reinterpret_cast<const f32x4*>(kp + 4)};
#pragma unroll
    for (int t = 0; t < H2 / 4; ++t) {
      const f32x4 kv = kq[t & 1];
      if (t + 2 < H2 / 4) kq[t & 1] = *reinterpret_cast<const f32x4*>(kp + 4 * (t + 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma32_f32(kv[e], qf[4 * t + e], s);
    }
    // ---- masks: keys past N and, if causal, keys after the query
    const int key0 = j * BC;
    bool need = key0 + BC > N;
    if (CAUSAL) need = need || (key0 + BC - 1 > wq0);
    if (need) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + acc_row(r, lane);
        if (key >= N || (CAUSAL && key > qrow)) s[r] = -INFINITY;
      }
    }
    // ---- online softmax: the reference moves only when a lane's sum reaches
    // kSumBound or the row has none yet (as in the bf16 kernel)
    float p[16];
    float rs;
    auto exps = [&]() {
      rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2_fast(fmaf(s[r], c, -mu));
        rs += p[r];
      }
    };
    exps();
    if (__builtin_amdgcn_ballot_w64(m == -INFINITY || !(rs < kSumBound))) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const float mxr = halves_max(mx) * c;
      const float m_new = (mxr > m + kLazyRescale) ? mxr : m;
      const float mu_new = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = m == -INFINITY ? 0.f : exp2_fast(mu - mu_new);  // O and l are 0 while m is -inf
      m = m_new;
      mu = mu_new;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
      exps();
    }
    l += rs;
    // ---- O^T += V_j^T P^T
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* vrow = vs + (8 * (r >> 2) + 4 * half + (r & 3)) * RSF + l32;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] = mfma32_f32(vrow[32 * b], p[r], o[b]);
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    const int stage = j & 1;
    if (j + 1 < nt) load_tile(j + 1);
    if (wave_active && j < nt_w) compute(j, sm[stage], sm[stage] + TILEF);
    if (j + 1 < nt) store_tile(stage ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float lt = halves_sum(l);
  const float inv = 1.f / lt;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + head, head_bytes);  // rows past N are dropped by the bounds
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(unsigned, o[b][4 * g + e] * inv);
      __builtin_amdgcn_raw_buffer_store_b128(w, ro, (qrow * D + b * 32 + 8 * g + 4 * half) * 4, 0, 0);
    }
  if (half == 0 && qrow < N) LSE[size_t(bh) * N + qrow] = (m + log2_fast(lt)) * kLn2;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, int NW, bool DROP = false>
static hipError_t launch_fwd_nw(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                int N, float scale, hipStream_t st, DropArgs dp = DropArgs{}) {
  using T = FwdTile<D, NW>;
  const int Tr = (N + T::BR - 1) / T::BR;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, NW, false, kMaskDense, DROP>), dim3((unsigned)G), dim3(T::NT), 0,
                     st, (const E*)q, (const E*)k, (const E*)v, (E*)o, lse, N, Tr, scale * kLog2e,
                     SplitArgs{1, 0, nullptr, nullptr, 0, 0}, MaskArgs{}, dp);
  return hipGetLastError();
}

// Eight waves with KQ key parts: 32*8/KQ rows per workgroup, each row's keys
// split over KQ waves on different SIMDs and merged in LDS at the end.
template <typename E, int D, bool CAUSAL, int KQ, bool DROP = false>
static hipError_t launch_fwd_kq(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                int N, float scale, hipStream_t st, DropArgs dp = DropArgs{}) {
  using T = FwdTile<D, 8, KQ>;
  const int Tr = (N + T::BR - 1) / T::BR;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, 8, false, kMaskDense, DROP, KQ>), dim3((unsigned)G), dim3(T::NT), 0,
                     st, (const E*)q, (const E*)k, (const E*)v, (E*)o, lse, N, Tr, scale * kLog2e,
                     SplitArgs{1, 0, nullptr, nullptr, 0, 0}, MaskArgs{}, dp);
  return hipGetLastError();
}

// Eight waves (256 rows, one workgroup per CU) stream each K/V tile once for
// twice the rows of four waves (128 rows, two workgroups per CU), halving the
// tile loads and LDS writes per row; used at d = 128 and 96 when that grid still
// covers every CU, causal or not (causal grids dispatch their longest row
// blocks first; measured 2 % faster than 128-row blocks at B2 H8 N16000 and
// B1 H8 N16384, even at B4 H16 N4096).  d = 64 keeps four waves: its tiles
// carry half the MFMA work per barrier (measured slower with 8 waves).  Grids
// with too few rows for two waves per SIMD split each row's keys instead:
// 128-row workgroups with two key parts when 256-row blocks leave CUs idle
// but 128-row blocks do not (d = 128, 96), 64-row workgroups with four key
// parts when even 128-row blocks leave CUs idle (d <= 128): 1.1-1.7x faster
// at B1 H8 N1024-4096 d128, B1 H4 N4096 causal and B1 H2 N8192 d64.
template <typename E, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int N, float scale, hipStream_t st) {
  const long long G8 = (long long)B * H * ((N + FwdTile<D, 8>::BR - 1) / FwdTile<D, 8>::BR);
  if constexpr (D == 128 || D == 96)
    if (G8 >= kNumCUs) return launch_fwd_nw<E, D, CAUSAL, 8>(q, k, v, o, lse, B, H, N, scale, st);
  if constexpr (D <= 128) {
    const long long G4 = (long long)B * H * ((N + FwdTile<D, 4>::BR - 1) / FwdTile<D, 4>::BR);
    if (G4 < kNumCUs) return launch_fwd_kq<E, D, CAUSAL, 4>(q, k, v, o, lse, B, H, N, scale, st);
    if constexpr (D != 64)
      if (G8 < kNumCUs) return launch_fwd_kq<E, D, CAUSAL, 2>(q, k, v, o, lse, B, H, N, scale, st);
  }
  return launch_fwd_nw<E, D, CAUSAL, 4>(q, k, v, o, lse, B, H, N, scale, st);
}

template <typename E>
static hipError_t launch_fwd_e(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 96) return causal ? launch_fwd_t<E, 96, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_t<E, 96, false>(q, k, v, o, lse, B, H, N, scale, st);
  if (d == 256) return causal ? launch_fwd_t<E, 256, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_t<E, 256, false>(q, k, v, o, lse, B, H, N, scale, st);
  if (d == 128) return causal ? launch_fwd_t<E, 128, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_t<E, 128, false>(q, k, v, o, lse, B, H, N, scale, st);
  return causal ? launch_fwd_t<E, 64, true>(q, k, v, o, lse, B, H, N, scale, st)
                : launch_fwd_t<E, 64, false>(q, k, v, o, lse, B, H, N, scale, st);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal, hipStream_t st) {
  return launch_fwd_e<__bf16>(q, k, v, o, lse, B, H, N, d, scale, causal, st);
}

hipError_t launch_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal, hipStream_t st) {
  return launch_fwd_e<_Float16>(q, k, v, o, lse, B, H, N, d, scale, causal, st);
}

// Forward with dropout on P: the plain forward's tiles, with the keep bits of
// each tile drawn in the kernel; eight-wave workgroups for non-causal d = 128
// grids that cover every CU, key parts on the grids where the plain forward
// uses them (a keep bit depends on the row and the key only), four waves
// otherwise.
template <typename E, int D, bool CAUSAL>
static hipError_t launch_fwd_dropout_t(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                       int H, int N, float scale, const DropArgs& dp, hipStream_t st) {
  const long long G8 = (long long)B * H * ((N + FwdTile<D, 8>::BR - 1) / FwdTile<D, 8>::BR);
  if constexpr (D == 128)
    if (!CAUSAL && G8 >= kNumCUs) return launch_fwd_nw<E, D, CAUSAL, 8, true>(q, k, v, o, lse, B, H, N, scale, st, dp);
  if constexpr (D <= 128) {
    const long long G4 = (long long)B * H * ((N + FwdTile<D, 4>::BR - 1) / FwdTile<D, 4>::BR);
    if (G4 < kNumCUs) return launch_fwd_kq<E, D, CAUSAL, 4, true>(q, k, v, o, lse, B, H, N, scale, st, dp);
    if constexpr (D != 64)
      if (G8 < kNumCUs) return launch_fwd_kq<E, D, CAUSAL, 2, true>(q, k, v, o, lse, B, H, N, scale, st, dp);
  }
  return launch_fwd_nw<E, D, CAUSAL, 4, true>(q, k, v, o, lse, B, H, N, scale, st, dp);
}

template <typename E>
static hipError_t launch_fwd_dropout_e(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                       int H, int N, int d, float scale, int causal, float p,
                                       unsigned long long seed, hipStream_t st) {
  const DropArgs dp = make_drop_args(p, seed);
  if (d == 96) return causal ? launch_fwd_dropout_t<E, 96, true>(q, k, v, o, lse, B, H, N, scale, dp, st)
                              : launch_fwd_dropout_t<E, 96, false>(q, k, v, o, lse, B, H, N, scale, dp, st);
  if (d == 256) return causal ? launch_fwd_dropout_t<E, 256, true>(q, k, v, o, lse, B, H, N, scale, dp, st)
                              : launch_fwd_dropout_t<E, 256, false>(q, k, v, o, lse, B, H, N, scale, dp, st);
  if (d == 128) return causal ? launch_fwd_dropout_t<E, 128, true>(q, k, v, o, lse, B, H, N, scale, dp, st)
                              : launch_fwd_dropout_t<E, 128, false>(q, k, v, o, lse, B, H, N, scale, dp, st);
  return causal ? launch_fwd_dropout_t<E, 64, true>(q, k, v, o, lse, B, H, N, scale, dp, st)
                : launch_fwd_dropout_t<E, 64, false>(q, k, v, o, lse, B, H, N, scale, dp, st);
}

hipError_t launch_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int N, int d, float scale, int causal, float p, unsigned long long seed, bool fp16,
                              hipStream_t st) {
  return fp16 ? launch_fwd_dropout_e<_Float16>(q, k, v, o, lse, B, H, N, d, scale, causal, p, seed, st)
              : launch_fwd_dropout_e<__bf16>(q, k, v, o, lse, B, H, N, d, scale, causal, p, seed, st);
}

// ---------------------------------------------------------------------------
// Eq. (2) merge of S parts: for each row, with M = max_s LSE_s and
// w_s = e^(LSE_s - M): O = sum_s w_s O_s / sum_s w_s (rounded once to E)
// and LSE = M + ln sum_s w_s.  Parts with LSE_s = -inf weigh 0; a row whose
// parts are all -inf gets O = 0, LSE = -inf.  HBM-bound: D/8 lanes per row,
// each lane reads 8 consecutive floats of every part (two 16-byte loads) and
// writes 8 16-bit values (one 16-byte store).
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(256)
lse_merge_kernel(const float* __restrict__ OP, const float* __restrict__ LP, int S,
                 E* __restrict__ O, float* __restrict__ LSE, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int sub = int(t % LPR);
  if (row >= rows) return;
  // parts in groups of G: all loads of a group are issued before any use
  constexpr int G = 8;
  float M = -INFINITY;
  for (int p0 = 0; p0 < S; p0 += G) {
    float lp[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lp[g] = LP[min(p0 + g, S - 1) * rows + row];  // past S: a repeat of part S-1
#pragma unroll
    for (int g = 0; g < G; ++g) M = fmaxf(M, lp[g]);
  }
  f32x4 a0 = {}, a1 = {};
  float L = 0.f;
  if (M > -INFINITY) {
    for (int p0 = 0; p0 < S; p0 += G) {
      float lp[G];
      f32x4 x0[G], x1[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // loads clamped to part S-1 (always in bounds); parts past S weigh 0 below
        const int pc = min(p0 + g, S - 1);
        const float l_in = LP[pc * rows + row];
        lp[g] = p0 + g < S ? l_in : -INFINITY;
        const f32x4* src = reinterpret_cast<const f32x4*>(OP + (pc * rows + row) * D + sub * 8);
        x0[g] = src[0];
        x1[g] = src[1];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // a part that saw no key weighs 0 (its O is ignored)
        const float w = lp[g] > -INFINITY ? exp2_fast((lp[g] - M) * kLog2e) : 0.f;
        a0 += w * x0[g];
        a1 += w * x1[g];
        L += w;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  u32x4 w;
  w[0] = pack2<E>(a0[0] * inv, a0[1] * inv);
  w[1] = pack2<E>(a0[2] * inv, a0[3] * inv);
  w[2] = pack2<E>(a1[0] * inv, a1[1] * inv);
  w[3] = pack2<E>(a1[2] * inv, a1[3] * inv);
  *reinterpret_cast<u32x4*>(O + row * D + sub * 8) = w;
  if (sub == 0) LSE[row] = L > 0.f ? M + log2_fast(L) * kLn2 : -INFINITY;
}

template <typename E>
static hipError_t launch_lse_merge_e(const float* op, const float* lp, int S, void* o, float* lse, int B, int H,
                                     int N, int d, hipStream_t st) {
  const long long rows = (long long)B * H * N;
  const long long threads = rows * (d / 8);
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)blocks), b(256);
  if (d == 256) hipLaunchKernelGGL((lse_merge_kernel<E, 256>), g, b, 0, st, op, lp, S, (E*)o, lse, rows);
  else if (d == 96) hipLaunchKernelGGL((lse_merge_kernel<E, 96>), g, b, 0, st, op, lp, S, (E*)o, lse, rows);
  else if (d == 128) hipLaunchKernelGGL((lse_merge_kernel<E, 128>), g, b, 0, st, op, lp, S, (E*)o, lse, rows);
  else hipLaunchKernelGGL((lse_merge_kernel<E, 64>), g, b, 0, st, op, lp, S, (E*)o, lse, rows);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* op, const float* lp, int S, void* o, float* lse, int B, int H, int N,
                            int d, bool fp16, hipStream_t st) {
  return fp16 ? launch_lse_merge_e<_Float16>(op, lp, S, o, lse, B, H, N, d, st)
              : launch_lse_merge_e<__bf16>(op, lp, S, o, lse, B, H, N, d, st);
}

// Key-split forward: S parts per query block (four-wave workgroups), then the
// merge.  S == 1 is the plain forward.
template <typename E, int D, bool CAUSAL>
static hipError_t launch_fwd_split_t(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                     int H, int N, float scale, int S, void* ws, hipStream_t st) {
  if (S <= 1) return launch_fwd_t<E, D, CAUSAL>(q, k, v, o, lse, B, H, N, scale, st);
  using T = FwdTile<D, 4>;
  const SplitLayout w = split_workspace_layout(Shape{B, H, N, D}, S);
  const int Tr = (N + T::BR - 1) / T::BR;
  const int Tc = (N + T::BC - 1) / T::BC;
  const long long G = (long long)B * H * Tr * S;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  char* base = reinterpret_cast<char*>(ws);
  SplitArgs sp{S, (Tc + S - 1) / S, reinterpret_cast<float*>(base + w.o_parts),
               reinterpret_cast<float*>(base + w.lse_parts), (long long)B * H * N * D, (long long)B * H * N};
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, 4, true, kMaskDense, false>), dim3((unsigned)G), dim3(T::NT), 0,
                     st, (const E*)q, (const E*)k, (const E*)v, (E*)o, lse, N, Tr, scale * kLog2e, sp, MaskArgs{},
                     DropArgs{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lse_merge_e<E>(sp.OP, sp.LP, S, o, lse, B, H, N, D, st);
}

template <typename E>
static hipError_t launch_fwd_splitkv_e(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                       int H, int N, int d, float scale, int causal, int S, void* ws,
                                       hipStream_t st) {
  if (d == 96) return causal ? launch_fwd_split_t<E, 96, true>(q, k, v, o, lse, B, H, N, scale, S, ws, st)
                              : launch_fwd_split_t<E, 96, false>(q, k, v, o, lse, B, H, N, scale, S, ws, st);
  if (d == 256) return causal ? launch_fwd_split_t<E, 256, true>(q, k, v, o, lse, B, H, N, scale, S, ws, st)
                              : launch_fwd_split_t<E, 256, false>(q, k, v, o, lse, B, H, N, scale, S, ws, st);
  if (d == 128) return causal ? launch_fwd_split_t<E, 128, true>(q, k, v, o, lse, B, H, N, scale, S, ws, st)
                              : launch_fwd_split_t<E, 128, false>(q, k, v, o, lse, B, H, N, scale, S, ws, st);
  return causal ? launch_fwd_split_t<E, 64, true>(q, k, v, o, lse, B, H, N, scale, S, ws, st)
                : launch_fwd_split_t<E, 64, false>(q, k, v, o, lse, B, H, N, scale, S, ws, st);
}

hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int N, int d, float scale, int causal, int S, void* ws, bool fp16, hipStream_t st) {
  return fp16 ? launch_fwd_splitkv_e<_Float16>(q, k, v, o, lse, B, H, N, d, scale, causal, S, ws, st)
              : launch_fwd_splitkv_e<__bf16>(q, k, v, o, lse, B, H, N, d, scale, causal, S, ws, st);
}

// Sliding-window and block-sparse forwards: four-wave workgroups (128 rows,
// two 64-row mask blocks), the same kernel with a per-tile predicate.
template <typename E, int D, bool CAUSAL, int MODE>
static hipError_t launch_fwd_masked_t(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int H, int N, float scale, const MaskArgs& mk, hipStream_t st) {
  using T = FwdTile<D, 4>;
  const int Tr = (N + T::BR - 1) / T::BR;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, 4, false, MODE, false>), dim3((unsigned)G), dim3(T::NT), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, (E*)o, lse, N, Tr, scale * kLog2e,
                     SplitArgs{1, 0, nullptr, nullptr, 0, 0}, mk, DropArgs{});
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_fwd_window_e(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int H, int N, int d, float scale, int left, int right, hipStream_t st) {
  // a bound of N - 1 or more limits nothing: the same as no bound
  const MaskArgs mk{left >= N - 1 ? -1 : left, right >= N - 1 ? -1 : right, nullptr, 0, 0, H};
  if (d == 96) return launch_fwd_masked_t<E, 96, false, kMaskWindow>(q, k, v, o, lse, B, H, N, scale, mk, st);
  if (d == 256) return launch_fwd_masked_t<E, 256, false, kMaskWindow>(q, k, v, o, lse, B, H, N, scale, mk, st);
  if (d == 128) return launch_fwd_masked_t<E, 128, false, kMaskWindow>(q, k, v, o, lse, B, H, N, scale, mk, st);
  return launch_fwd_masked_t<E, 64, false, kMaskWindow>(q, k, v, o, lse, B, H, N, scale, mk, st);
}

template <typename E>
static hipError_t launch_fwd_blocksparse_e(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                           int H, int N, int d, float scale, int causal, const unsigned char* bm,
                                           int per_head, hipStream_t st) {
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  const MaskArgs mk{-1, -1, bm, per_head ? (long long)nb * nb : 0, nb, H};
  if (d == 96)
    return causal ? launch_fwd_masked_t<E, 96, true, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st)
                  : launch_fwd_masked_t<E, 96, false, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st);
  if (d == 256)
    return causal ? launch_fwd_masked_t<E, 256, true, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st)
                  : launch_fwd_masked_t<E, 256, false, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st);
  if (d == 128)
    return causal ? launch_fwd_masked_t<E, 128, true, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st)
                  : launch_fwd_masked_t<E, 128, false, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st);
  return causal ? launch_fwd_masked_t<E, 64, true, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st)
                : launch_fwd_masked_t<E, 64, false, kMaskBlocks>(q, k, v, o, lse, B, H, N, scale, mk, st);
}

hipError_t launch_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                             int d, float scale, int left, int right, bool fp16, hipStream_t st) {
  return fp16 ? launch_fwd_window_e<_Float16>(q, k, v, o, lse, B, H, N, d, scale, left, right, st)
              : launch_fwd_window_e<__bf16>(q, k, v, o, lse, B, H, N, d, scale, left, right, st);
}

hipError_t launch_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                  int N, int d, float scale, int causal, const unsigned char* bm, int per_head,
                                  bool fp16, hipStream_t st) {
  return fp16 ? launch_fwd_blocksparse_e<_Float16>(q, k, v, o, lse, B, H, N, d, scale, causal, bm, per_head, st)
              : launch_fwd_blocksparse_e<__bf16>(q, k, v, o, lse, B, H, N, d, scale, causal, bm, per_head, st);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const float* q, const float* k, const float* v, float* o, float* lse,
                                   int B, int H, int N, float scale, hipStream_t st) {
  const int Tr = (N + 127) / 128;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(256), 0, st, q, k, v, o, lse, N,
                     Tr, scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 96) return causal ? launch_fwd_f32_t<96, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_f32_t<96, false>(q, k, v, o, lse, B, H, N, scale, st);
  if (d == 256) return causal ? launch_fwd_f32_t<256, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_f32_t<256, false>(q, k, v, o, lse, B, H, N, scale, st);
  if (d == 128) return causal ? launch_fwd_f32_t<128, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_f32_t<128, false>(q, k, v, o, lse, B, H, N, scale, st);
  return causal ? launch_fwd_f32_t<64, true>(q, k, v, o, lse, B, H, N, scale, st)
                : launch_fwd_f32_t<64, false>(q, k, v, o, lse, B, H, N, scale, st);
}

// ---------------------------------------------------------------------------
// Measurement helper: the bf16 MFMA rate this GPU sustains.  Each wave runs
// `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 accumulation
// chains on register operands (no memory traffic in the loop), two waves per
// SIMD, and writes one sum per wave so that nothing is optimised away.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256, 2) mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * float((lane + e) & 7));
    b[e] = (__bf16)(0.001f * float((lane * 3 + e) & 7));
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[c][e];
  sink[size_t(blockIdx.x) * 256 + threadIdx.x] = t;
}

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace fa
