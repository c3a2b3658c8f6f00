// fa_bwd.hip - gfx950 backward attention by recomputation.
//
// The pages describe the backward only as: keep the per-row statistic from the
// forward pass, recompute the probabilities from it instead of storing the
// N x N matrices, and tile the gradient computation the same way as the
// forward (FlashAttention-from-GPU-memory page (jsqmd.com), section 2.2;
// FlashAttention optimisation page (intelliparadigm.com), section 4.2).  The
// gradients are the chain rule on O = softmax(scale*Q K^T + mask) V:
//   P = exp(scale*S - LSE),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_k dO_ik O_ik (= sum_j P_ij dP_ij),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels on the caller's stream, none of them with atomics (two when
// the grids of passes 2 and 3 fit on the CUs together: bwd_both runs both):
//  1. bwd_pre: D = rowsum(dO * O) and LSE in base-2 units, both fp32.
//  2. bwd_dkdv: one workgroup per (b, h, 128-key block) (two at d = 256,
//     each with half of the dK and dV columns), four waves of 32 keys, one
//     wave per SIMD.  K and V of a wave's keys stay in registers as
//     the B operands of S = Q K^T and dP = dO V^T, so each lane holds one key
//     and the recomputed P and dS feed dV^T += dO^T P and dK^T += Q^T dS
//     straight from registers; dK^T and dV^T accumulate on chip for the whole
//     sweep.  The workgroup streams 64-query steps (causal: from the diagonal
//     on).  Q, dO and the per-row LSE and D of step i+1 go from HBM straight
//     into LDS (buffer loads with the LDS destination) while step i computes;
//     Q and dO are stored row-major only, and the transposed operands Q^T and
//     dO^T are read with ds_read_b64_tr_b16.  Within a step the wave issues
//     its MFMAs in a fixed order and spreads the exponentials and the dS
//     arithmetic over the MFMAs that do not depend on them.
//  3. bwd_dq: one workgroup per (b, h, 128- or 256-query block), laid out
//     like the forward kernel: each wave owns 32 queries whose Q and dO fragments stay
//     in VGPRs, K and V tiles of 64 keys stream through double-buffered LDS,
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, and
//     dQ^T += K^T dS^T takes dS^T from registers and K^T from transposing LDS
//     reads of the K tile; dQ accumulates on chip.
// Computing dQ in its own query-major pass costs two more N x N x d products
// (S and dP recomputed) than accumulating it across key blocks, but the
// per-key-block partial sums would need one fp32 atomic add per element and
// key block, and on this GPU those are performed at the memory side at a
// rate that caps the whole backward well below the MFMA rate.
#include "fa_common.h"
#include "fa_validate.h"

#include <mutex>

namespace fa {

// Byte offset, inside a row-major LDS tile (rows of lds_row_bytes<DD>()) swizzled by
// tile_swz<DD>, of the 8 bytes this lane reads with ds_read_b64_tr_b16 so that
// lane l ends up with column 32*b + l%32 of rows row0 + {4h+8r2+0..3}
// (h = l/32): in its 16-lane group g (lane t) it addresses row
// 4*(g/2) + 8*r2 + t/4, columns 32*b + 16*(g%2) + 4*(t%4) .. +3.
template <int DD>
__device__ __forceinline__ int tr_off(int b, int r2, int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int row = 4 * (g >> 1) + 8 * r2 + (t >> 2);
  const int col = 32 * b + 16 * (g & 1) + 4 * (t & 3);
  return row * lds_row_bytes<DD>() + (((col >> 3) ^ tile_swz<DD>(row)) * 16) + (col & 7) * 2;
}

template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 tr_pair(const char* base, int off0, int off1) {
  typedef __attribute__((address_space(3))) short4_t* lds_s4;
  using v4 = typename Vec<E>::v4;
  const v4 lo = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + off0)));
  const v4 hi = __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + off1)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 4 bytes per lane from a buffer straight into LDS: lane l writes lds[4*l .. 4*l+3].
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voffset, 0, 0, 0);
#endif
}



// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and LSE2 = LSE * log2(e) (+inf for LSE = -inf).  8 lanes per row.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const E* __restrict__ O, const E* __restrict__ dO, const float* __restrict__ LSE,
               float* __restrict__ Dv, float* __restrict__ lse2, long long rows) {
  // vectors of 8 elements (4 when d / 8 is not a multiple of 8: d = 96)
  constexpr int PER = D / 8;  // elements per lane
  constexpr int VW = PER % 8 == 0 ? 8 : 4;
  typedef E vec_t __attribute__((ext_vector_type(VW)));
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid >> 3;
  const int sub = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const E* o = O + row * D + sub * PER;
    const E* g = dO + row * D + sub * PER;
#pragma unroll
    for (int u = 0; u < PER / VW; ++u) {
      const vec_t a = *reinterpret_cast<const vec_t*>(o + VW * u);
      const vec_t b = *reinterpret_cast<const vec_t*>(g + VW * u);
#pragma unroll
      for (int e = 0; e < VW; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && sub == 0) {
    Dv[row] = acc;
    // a row that saw no key (LSE = -inf, block-sparse masks only) gets +inf,
    // so that P = exp2(S*c - LSE2) = 0 for every key, masked (-inf) or not
    const float l = LSE[row];
    lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: key-block-major sweep over the queries.
//
// Four waves per workgroup, one per SIMD, each owning 32 keys: K and V of
// those keys stay in registers (parked in AGPRs, which the MFMAs read
// directly) as the B operands of S = Q K^T and dP = dO V^T, so each lane
// holds one key.  A wave runs all four products of a 64-query step itself:
//   S = Q K^T, dP = dO V^T          (A operands: rows of the Q / dO tiles)
//   P = exp2(S*c - LSE2), dS = P * (dP - D)   (VALU, one query per element)
//   dV^T += dO^T P, dK^T += Q^T dS  (A operands: transposing reads of the
//                                    same tiles; P and dS from registers)
// The 64 MFMAs of a step (d = 128) are issued in a fixed order of slots,
// and the VALU work is spread over the slots whose MFMAs do not depend on
// it, two elements per slot: P of the first 32-query block while its dP
// MFMAs run, its dS during the S MFMAs of the second block, and so on.
// Each slot also issues the LDS read of the operand three slots ahead, and
// every second one of the first slots one direct load of the next step.
// ---------------------------------------------------------------------------
template <int D>
struct DkdvTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BKV = 32 * NW;          // keys per workgroup, 32 per wave
  static constexpr int BQ = 64;                // queries per step
  static constexpr int QB = BQ / 32;           // 32-query blocks per step
  static constexpr int KS = D / 16;            // 16-wide k steps over d
  static constexpr int DB = D / 32;            // 32-column blocks over d
  static constexpr int PS = BQ / 16;           // 16-query k steps of dV, dK
  static constexpr int RS = lds_row_bytes<D>(); // bytes per Q / dO row in LDS
  static constexpr int GRS = D * 2;            // bytes per Q / dO / K / V row in HBM
  static constexpr int QT = BQ * RS;           // bytes of one Q or dO tile
  static constexpr int OFF_DO = QT;
  static constexpr int OFF_LSE = 2 * QT;       // BQ floats of LSE*log2(e)
  static constexpr int OFF_DD = 2 * QT + BQ * 4;  // BQ floats of D
  static constexpr int STAGE = 2 * QT + 2 * BQ * 4;
  static constexpr int LDS = 2 * STAGE;        // double-buffered
  static constexpr int LPW = QT / 1024 / NW;   // 1 KiB direct loads per wave per Q (or dO) tile
  static constexpr int KVS = 4 * QT;           // staged K and V rows of a key block (persistent workgroups)
  static_assert(QT % (1024 * NW) == 0, "tile must split into 1 KiB loads over the waves");
  // dK and dV columns are split over OS workgroups per key block at d = 256,
  // each forming S and dP over the full d but accumulating DBO of the DB
  // 32-column blocks: the accumulators of all 256 columns and the K and V
  // fragments would not fit in a wave's 512 registers
  static constexpr int OS = D == 256 ? 2 : 1;
  static constexpr int DBO = DB / OS;
  // MFMA slots of one step: S, dP over block 0 and block 1 (2*M; H per
  // product and block), then dV, dK over block 0's and block 1's queries
  // (2*M2; H2 per product and block)
  static constexpr int M = D / 8;
  static constexpr int H = M / 2;
  static constexpr int H2 = 2 * DBO;
  static constexpr int M2 = 2 * H2;
  static constexpr int SLOTS = 2 * M + 2 * M2;
  static constexpr int PF = 3;                 // operand reads in flight
  static constexpr int PP = (8 + H - 1) / H;   // element pairs of VALU work per slot (8 pairs per block)
  // first slots of: P of block 0, dS of block 0, P of block 1, dS of block 1
  static constexpr int P0 = H + 2, D0 = 2 * H + 1, P1 = 3 * H + 2, D1 = 4 * H + 1;
};

// One workgroup of the dK/dV pass: workgroup `bid` of `nblk` (key block, before the XCD
// remap).  smem holds DkdvTile<D>::LDS bytes; slist and scount are the
// workgroup's query-step list (block-sparse mode only).
//
// STAGED (persistent workgroups, d <= 128, no block mask): the block's K and V
// rows come through kvs (DkdvTile<D>::KVS bytes of LDS), and the block's last
// step also brings in, for key block `nextw` (-1: none), its K and V rows and
// its first Q and dO tile, so that the next call (`pre`) starts without
// waiting for memory; its first tile is in stage `stage0`.  Returns the stage
// that holds the next block's first tile, or -1 when nothing was brought in.
template <typename E, int D, bool CAUSAL, bool DROP, int MODE, bool STAGED = false>
__device__ __forceinline__ int
dkdv_block(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
           const E* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
           E* __restrict__ dK, E* __restrict__ dV, DropArgs dp, int N, int Tk, float c /* scale*log2(e) */,
           float scale, MaskArgs mk, int bid, int nblk, char* smem, unsigned short* slist, int& scount,
           char* kvs = nullptr, int stage0 = 0, bool pre = false, int nextw = -1) {
  using T = DkdvTile<D>;
  using v8 = typename Vec<E>::v8;
  constexpr bool WINDOW = MODE == kMaskWindow, BLOCKS = MODE == kMaskBlocks;
  // block-sparse: two operand reads in flight, not three (with three, the
  // kernel that runs both passes in one grid spilled an operand at d = 128)
  constexpr int M = T::M, H = T::H, PF = BLOCKS ? 2 : T::PF;
  static_assert(!(DROP && MODE != kMaskDense), "dropout only with the dense or causal mask");
  static_assert(!BLOCKS || (T::BQ == kMaskBlock && T::BKV == 2 * kMaskBlock), "query steps are mask blocks");
  static_assert(!STAGED || (T::OS == 1 && !BLOCKS && 8 * T::LPW <= T::SLOTS),
                "staging needs whole-d workgroups, step ranges and a slot per K/V load");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses for the direct loads
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int Tq = (N + T::BQ - 1) / T::BQ;
  // Workgroup b's column part, head, first key and query steps [i0, i1)
  // (block-sparse: the steps slist[0 .. scount) among them whose 64-query
  // block keeps one of the workgroup's two key blocks).
  struct Pos {
    int cpart, bh, k0, i0, i1;
  };
  auto locate = [&](int b) {
    Pos p;
    // the OS column parts of the grid are consecutive copies of the key-block grid
    const int nper = nblk / T::OS;
    p.cpart = T::OS == 1 ? 0 : b / nper;
    b -= p.cpart * nper;
    int jt;
    if (CAUSAL) {
      // key block jt sees the query steps from its diagonal on: block 0 has the
      // most, so the blocks go out longest first across all heads
      causal_order(b, nper / Tk, Tk, p.bh, jt);
    } else {
      const int tile = xcd_remap(b, nper);
      p.bh = tile / Tk;
      jt = tile - p.bh * Tk;
    }
    p.k0 = jt * T::BKV;
    p.i0 = CAUSAL ? p.k0 / T::BQ : 0;
    p.i1 = Tq;
    if (WINDOW) {
      // queries i with i - left <= key <= i + right for a key of the workgroup
      if (mk.right >= 0) p.i0 = max(0, p.k0 - mk.right) / T::BQ;
      if (mk.left >= 0) p.i1 = (int)min((long long)N - 1, (long long)p.k0 + T::BKV - 1 + mk.left) / T::BQ + 1;
    }
    return p;
  };
  const Pos pos = locate(bid);
  const int cpart = pos.cpart, bh = pos.bh, k0 = pos.k0, i0 = pos.i0, i1 = pos.i1;
  const size_t head = size_t(bh) * N * D;
  const int head_bytes = N * T::GRS;

  // Direct-to-LDS loads of the Q and dO tiles of a step: load u of this wave
  // fills bytes [(wave*LPW + u) KiB, +1 KiB) of each tile.
  int goff[T::LPW];
#pragma unroll
  for (int u = 0; u < T::LPW; ++u) goff[u] = swz_src<D>((wave * T::LPW + u) * 1024 + 16 * lane);
  const float* lse2h = LSE2 + size_t(bh) * N;
  const float* dh = Dv + size_t(bh) * N;
  auto issue_loads = [&](int i, int stage) {
    const int q0 = i * T::BQ;
    const int bytes = (N - q0) * T::GRS;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head + size_t(q0) * D, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dO + head + size_t(q0) * D, bytes);
    char* dst = smem + stage * T::STAGE + wave * T::LPW * 1024;
#pragma unroll
    for (int u = 0; u < T::LPW; ++u) load_lds16(rq, dst + u * 1024, goff[u]);
#pragma unroll
    for (int u = 0; u < T::LPW; ++u) load_lds16(rd, dst + T::OFF_DO + u * 1024, goff[u]);
    // Rows past N read as zero: with their Q and dO rows zero as well, P = 1
    // and dS = 0 there, and dO = 0 removes them from dV.
    if (wave == 0) load_lds4(make_rsrc(lse2h + q0, (N - q0) * 4), smem + stage * T::STAGE + T::OFF_LSE, 4 * lane);
    if (wave == 1) load_lds4(make_rsrc(dh + q0, (N - q0) * 4), smem + stage * T::STAGE + T::OFF_DD, 4 * lane);
  };

  // Operand offsets: rows l32 (+32 per block) of Q or dO, 16-byte unit
  // 2*st + half; transposing reads as in tr_off.
  int rof[T::KS];
#pragma unroll
  for (int st = 0; st < T::KS; ++st) rof[st] = l32 * T::RS + (((2 * st + half) ^ tile_swz<D>(l32)) * 16);

  // Staged K and V (kvs): four 64-row tiles in the layout of a Q tile, K
  // rows k0 .. k0+63, k0+64 .. k0+127, then the same rows of V.  Load l of a
  // wave fills 1 KiB unit wave*LPW + l%LPW of tile l/LPW; rows past N read
  // as zero.  kv_rsrc: the buffer of tile t for the block at key kk0 of the
  // head at element offset h (size 0 when not valid).
  auto kv_rsrc = [&](size_t h, int kk0, bool valid, int t) {
    const int r0 = kk0 + 64 * (t & 1);
    const bool in = valid && r0 < N;
    return make_rsrc((t < 2 ? K : V) + h + size_t(in ? r0 : 0) * D, in ? (N - r0) * T::GRS : 0);
  };
  auto kv_load = [&](const __amdgpu_buffer_rsrc_t* r, int l) {
    const int t = l / T::LPW, u = l % T::LPW;
    load_lds16(r[t], kvs + t * T::QT + (wave * T::LPW + u) * 1024, goff[u]);
  };

  // The first step's Q and dO tiles are requested before the K and V
  // fragments below, so that the two memory latencies overlap (block-sparse
  // mode: once its step list is known).
  const bool early = !BLOCKS && i1 > i0;

  // K and V fragments of this wave's keys (lane: key k0 + 32*wave + l32,
  // d = 16*st + 8*half .. +7).  Keys past N read as zero; their dK and dV
  // rows are never stored.
  const int key = k0 + wave * 32 + l32;
  v8 kf[T::KS], vf[T::KS];
  if constexpr (STAGED) {
    if (early) {
      if (!pre) {
        issue_loads(i0, stage0);
        __amdgpu_buffer_rsrc_t r[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) r[t] = kv_rsrc(head, k0, true, t);
#pragma unroll
        for (int l = 0; l < 4 * T::LPW; ++l) kv_load(r, l);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
      }
      const char* kb = kvs + (wave >> 1) * T::QT + (wave & 1) * 32 * T::RS;
#pragma unroll
      for (int st = 0; st < T::KS; ++st) {
        kf[st] = *reinterpret_cast<const v8*>(kb + rof[st]);
        vf[st] = *reinterpret_cast<const v8*>(kb + 2 * T::QT + rof[st]);
      }
    }
  } else {
    if (early) issue_loads(i0, 0);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head, head_bytes);
#pragma unroll
    for (int st = 0; st < T::KS; ++st) {
      kf[st] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rk, key * T::GRS + (16 * st + 8 * half) * 2, 0, 0));
      vf[st] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rv, key * T::GRS + (16 * st + 8 * half) * 2, 0, 0));
    }
  }
  // Kept in AGPRs for the whole sweep: the MFMAs take them from there, and
  // the VGPRs are left to the accumulators and the per-step values.
#pragma unroll
  for (int st = 0; st < T::KS; ++st) {
    asm volatile("" : "+a"(kf[st]));
    asm volatile("" : "+a"(vf[st]));
  }
  int tof[T::DBO][2];
#pragma unroll
  for (int b = 0; b < T::DBO; ++b) {
    tof[b][0] = tr_off<D>(cpart * T::DBO + b, 0, lane);
    tof[b][1] = tr_off<D>(cpart * T::DBO + b, 1, lane);
  }

  f32x16 accv[T::DBO], acck[T::DBO];  // dV^T and dK^T of this wave's keys (this part's columns)
#pragma unroll
  for (int b = 0; b < T::DBO; ++b) accv[b] = acck[b] = f32x16{};

  const int kw0 = k0 + wave * 32;  // this wave's first key
  // block-sparse: each step of the list carries the keep flags of the
  // workgroup's two 64-key blocks (waves 0-1 and 2-3)
  if (BLOCKS) {
    const unsigned char* bmh = mk.bm + mk.bm_head_stride * (bh % mk.H);
    const int kb0 = k0 / kMaskBlock;
    const bool two = kb0 + 1 < mk.nb;
    if (wave == 0) {
      int n = 0;
      for (int base = i0; base < Tq; base += 64) {
        const int ii = base + lane;
        const bool a0 = ii < Tq && bmh[size_t(ii) * mk.nb + kb0] != 0;
        const bool a1 = ii < Tq && two && bmh[size_t(ii) * mk.nb + kb0 + 1] != 0;
        const bool keep = a0 || a1;
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1));
        if (keep) slist[n + below] = list_entry(ii, a0, a1);
        n += __builtin_popcountll(bal);
      }
      if (lane == 0) scount = n;
    }
    __syncthreads();
  }
  const int cnt = BLOCKS ? scount : i1 - i0;
  auto step_at = [&](int idx) { return BLOCKS ? list_index(slist[idx]) : i0 + idx; };

  // the next key block of a persistent workgroup, staged by the last step
  // when it has query steps
  Pos nx{};
  bool stage_next = false;
  if constexpr (STAGED) {
    if (nextw >= 0) {
      nx = locate(nextw);
      stage_next = nx.i1 > nx.i0;
    }
  }
  int ret = -1;

  if (cnt > 0) {  // uniform over the workgroup; a key block no query sees only stores zeros
  if (!early) issue_loads(step_at(0), 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();  // (staged: every wave has its K and V before the last step restages kvs)

  auto run_step = [&](int idx, auto lastc) {
    constexpr bool LAST = decltype(lastc)::value;  // the staged last step
    const int i = step_at(idx);
    const int stage = (stage0 + idx) & 1;
    // The next step's tiles are requested one load every second slot of the
    // schedule below, among the first MFMAs: the whole batch at the top of
    // the step held the wave (the only one on its SIMD) at the vector memory
    // unit.  On the last step the resources have size 0 and the loads read
    // nothing.
    // The staged last step requests the next block's first step instead, and
    // its K and V rows one load every second slot in between.
    const bool has_next = LAST ? stage_next : idx + 1 < cnt;
    const int qn = !has_next ? 0 : LAST ? nx.i0 * T::BQ : step_at(idx + 1) * T::BQ;
    const int nbh = LAST ? nx.bh : bh;
    const size_t nhead = size_t(nbh) * N * D;
    const int nbytes = has_next ? (N - qn) * T::GRS : 0;
    const __amdgpu_buffer_rsrc_t nrq = make_rsrc(Q + nhead + size_t(qn) * D, nbytes);
    const __amdgpu_buffer_rsrc_t nrd = make_rsrc(dO + nhead + size_t(qn) * D, nbytes);
    const __amdgpu_buffer_rsrc_t nrs =
        make_rsrc((wave == 0 ? LSE2 : Dv) + size_t(nbh) * N + qn, has_next ? (N - qn) * 4 : 0);
    char* ndst = smem + (stage ^ 1) * T::STAGE;
    __amdgpu_buffer_rsrc_t nkv[4];
    if constexpr (LAST)
#pragma unroll
      for (int t = 0; t < 4; ++t) nkv[t] = kv_rsrc(nhead, nx.k0, has_next, t);
    constexpr int NL = 2 * T::LPW + 1;
    auto issue_one = [&](auto lc) {
      constexpr int l = decltype(lc)::value;
      if constexpr (l < T::LPW) load_lds16(nrq, ndst + wave * T::LPW * 1024 + l * 1024, goff[l]);
      else if constexpr (l < 2 * T::LPW)
        load_lds16(nrd, ndst + T::OFF_DO + wave * T::LPW * 1024 + (l - T::LPW) * 1024, goff[l - T::LPW]);
      else if (wave < 2) load_lds4(nrs, ndst + (wave == 0 ? T::OFF_LSE : T::OFF_DD), 4 * lane);
    };
    // block-sparse: all at once here (spread over the slots, the step-list
    // bookkeeping pushed the kernel past its registers)
    if constexpr (BLOCKS)
      if (has_next) static_for<NL>([&](auto lc) { issue_one(lc); });
    const char* sb = smem + stage * T::STAGE;
    const int qs = i * T::BQ;
    // steps whose element mask matters for this wave's keys: causal, the two
    // steps that straddle the diagonal; a window edge inside the step; a
    // block that drops this wave's keys
    bool need = CAUSAL && kw0 + 31 > qs;
    if (WINDOW)
      need = need || (mk.left >= 0 && kw0 < qs + T::BQ - 1 - mk.left) || (mk.right >= 0 && kw0 + 31 > qs + mk.right);
    const bool dead = BLOCKS && !list_keeps(slist[idx], wave >> 1);
    if (BLOCKS) need = need || dead;

    f32x16 s[T::QB], pd[T::QB];  // S and dP; lane: key, element j: query 32*qb + acc_row(j)
    v8 op[T::PS], os[T::PS];     // P and dS in the input type, MFMA B operands
    f32x4 l4[T::QB * 4], d4[T::QB * 4];
    float pk[T::QB][16];         // P in fp32, for dS
    unsigned keepg[T::QB * 4];   // dropout: keep bits of 4 consecutive queries at this key
    v8 ring[PF];

    // A operand of slot u
    auto fetch = [&](auto uc) -> v8 {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < 2 * M) {
        constexpr int qb = u / M, st = u % H, is_dp = (u % M) / H;
        return *reinterpret_cast<const v8*>(sb + (is_dp ? T::OFF_DO : 0) + qb * 32 * T::RS + rof[st]);
      } else {
        constexpr int v = u - 2 * M, M2 = T::M2, H2 = T::H2;
        constexpr int blk = v / M2, is_dk = (v % M2) / H2, x = v % H2;
        constexpr int ps = 2 * blk + x / T::DBO, b = x % T::DBO;
        return tr_pair<E>(sb + (is_dk ? 0 : T::OFF_DO) + ps * 16 * T::RS, tof[b][0], tof[b][1]);
      }
    };
    // P of elements j, j+1 (j even) of block qb.  Dropout: the kept P goes
    // to dV; its 1/(1-p) scale is applied to dV at the end.
    auto p_pair = [&](auto qc, auto jc) {
      constexpr int qb = decltype(qc)::value, j = decltype(jc)::value;
      constexpr int g = j / 4, cg = qb * 4 + g;
      // dropout: the four lanes of a quad hold keys 4p .. 4p+3 and need the
      // same call for each of the block's four 4-query groups; lane t draws
      // group t (of this 32-query block) and the quad shares the results
      if constexpr (DROP && j == 0) {
        const unsigned t = lane & 3;
        const unsigned mine =
            keep_block_cols(dp, unsigned(qs + qb * 32 + 8 * t + 4 * half) >> 2, unsigned(key) >> 2, unsigned(bh));
        const unsigned nib = quad_share_nibbles(mine, t);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) keepg[qb * 4 + gg] = (nib >> (4 * gg)) & 0xFu;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = j % 4 + t;
        const float p = exp2_fast(fmaf(s[qb][j + t], c, -l4[cg][e]));
        pk[qb][j + t] = p;
        if constexpr (DROP) op[qb * 2 + (j >> 3)][(j + t) & 7] = (E)keep_or_zero(p, keepg[cg], e);
        else op[qb * 2 + (j >> 3)][(j + t) & 7] = (E)p;
      }
    };
    // dS of elements j, j+1 of block qb; dropout: dP = Z * (dO V^T)
    auto ds_pair = [&](auto qc, auto jc) {
      constexpr int qb = decltype(qc)::value, j = decltype(jc)::value;
      constexpr int g = j / 4, cg = qb * 4 + g;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = j % 4 + t;
        float dpv = pd[qb][j + t];
        if constexpr (DROP) dpv = keep_or_zero(dpv * dp.keep_scale, keepg[cg], e);
        os[qb * 2 + (j >> 3)][(j + t) & 7] = (E)(pk[qb][j + t] * (dpv - d4[cg][e]));
      }
    };
    auto row_of = [&](int cg) { return (cg / 4) * 32 + 8 * (cg % 4) + 4 * half; };
    auto read_lse = [&](int qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        l4[qb * 4 + g] = *reinterpret_cast<const f32x4*>(sb + T::OFF_LSE + row_of(qb * 4 + g) * 4);
    };
    auto read_d = [&](int qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        d4[qb * 4 + g] = *reinterpret_cast<const f32x4*>(sb + T::OFF_DD + row_of(qb * 4 + g) * 4);
    };

    static_for<PF>([&](auto uc) { ring[decltype(uc)::value] = fetch(uc); });
    static_for<T::SLOTS>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const v8 a = ring[u % PF];
      if constexpr (u < 2 * M) {
        constexpr int qb = u / M, st = u % H, is_dp = (u % M) / H;
        if constexpr (!is_dp) s[qb] = mfma32(a, kf[st], st == 0 ? f32x16{} : s[qb]);
        else pd[qb] = mfma32(a, vf[st], st == 0 ? f32x16{} : pd[qb]);
      } else {
        constexpr int v = u - 2 * M, M2 = T::M2, H2 = T::H2;
        constexpr int blk = v / M2, is_dk = (v % M2) / H2, x = v % H2;
        constexpr int ps = 2 * blk + x / T::DBO, b = x % T::DBO;
        if constexpr (!is_dk) accv[b] = mfma32(a, op[ps], accv[b]);
        else acck[b] = mfma32(a, os[ps], acck[b]);
      }
      if constexpr (!BLOCKS && u % 2 == 0 && u / 2 < NL) issue_one(std::integral_constant<int, u / 2>{});
      if constexpr (LAST && u % 2 == 1 && u / 2 < 4 * T::LPW)
        if (has_next) kv_load(nkv, u / 2);
      if constexpr (u + PF < T::SLOTS) ring[u % PF] = fetch(std::integral_constant<int, u + PF>{});
      // masks: S = -inf (P = 0) where the key is after the query (causal),
      // outside the query's window, or in a dropped block, on the steps that
      // need it only (a wave-uniform branch)
      if constexpr ((CAUSAL || MODE != kMaskDense) && (u == T::P0 - 1 || u == T::P1 - 1)) {
        constexpr int qb = u == T::P0 - 1 ? 0 : 1;
        if (need) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int qj = qs + qb * 32 + acc_row(j, lane);
            bool hide = CAUSAL && key > qj;
            if (WINDOW) hide = hide || window_hides(mk, qj, key);
            if (BLOCKS) hide = hide || dead;
            if (hide) s[qb][j] = -INFINITY;
          }
        }
      }
      if constexpr (u == (T::P0 >= 6 ? T::P0 - 6 : 0)) read_lse(0);
      if constexpr (u == T::D0 - 6) read_d(0);
      if constexpr (u == T::P1 - 6) read_lse(1);
      if constexpr (u == T::D1 - 6) read_d(1);
      static_for<T::PP>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        using Z = std::integral_constant<int, 0>;
        using O = std::integral_constant<int, 1>;
        // pair index within the block's 8 pairs (past 7: nothing, when H*PP > 8)
        constexpr int jp0 = T::PP * (u - T::P0) + t, jd0 = T::PP * (u - T::D0) + t;
        constexpr int jp1 = T::PP * (u - T::P1) + t, jd1 = T::PP * (u - T::D1) + t;
        if constexpr (u >= T::P0 && u < T::P0 + H && jp0 < 8) p_pair(Z{}, std::integral_constant<int, 2 * jp0>{});
        if constexpr (u >= T::D0 && u < T::D0 + H && jd0 < 8) ds_pair(Z{}, std::integral_constant<int, 2 * jd0>{});
        if constexpr (u >= T::P1 && u < T::P1 + H && jp1 < 8) p_pair(O{}, std::integral_constant<int, 2 * jp1>{});
        if constexpr (u >= T::D1 && u < T::D1 + H && jd1 < 8) ds_pair(O{}, std::integral_constant<int, 2 * jd1>{});
      });
      // keep the slot order: the scheduler would otherwise pull each LDS read
      // next to its MFMA and bunch the VALU work
      __builtin_amdgcn_sched_barrier(0);
    });

    // the loads of step i+1 have landed; every wave is done with this stage
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  if constexpr (STAGED) {
    for (int idx = 0; idx + 1 < cnt; ++idx) run_step(idx, std::false_type{});
    run_step(cnt - 1, std::true_type{});
    if (stage_next) ret = (stage0 + cnt) & 1;
  } else {
    for (int idx = 0; idx < cnt; ++idx) run_step(idx, std::false_type{});
  }
  }

  // ---- epilogue: dV = (dV^T)^T (times 1/(1-p) with dropout), dK = scale * (dK^T)^T;
  // lane holds key `key`, keys past N are dropped by the buffer bounds
  const float fv = DROP ? dp.keep_scale : 1.f;
  const __amdgpu_buffer_rsrc_t rvo = make_rsrc(dV + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rko = make_rsrc(dK + head, head_bytes);
#pragma unroll
  for (int b = 0; b < T::DBO; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = (cpart * T::DBO + b) * 32 + 8 * g + 4 * half;
      u32x2 w;
      w[0] = pack2<E>(accv[b][4 * g + 0] * fv, accv[b][4 * g + 1] * fv);
      w[1] = pack2<E>(accv[b][4 * g + 2] * fv, accv[b][4 * g + 3] * fv);
      __builtin_amdgcn_raw_buffer_store_b64(w, rvo, key * T::GRS + col * 2, 0, 0);
      w[0] = pack2<E>(acck[b][4 * g + 0] * scale, acck[b][4 * g + 1] * scale);
      w[1] = pack2<E>(acck[b][4 * g + 2] * scale, acck[b][4 * g + 3] * scale);
      __builtin_amdgcn_raw_buffer_store_b64(w, rko, key * T::GRS + col * 2, 0, 0);
    }
  return ret;
}

// ---------------------------------------------------------------------------
// 3. dQ: query-block-major sweep over the keys
// ---------------------------------------------------------------------------
template <int D, int NW_>
struct DqTile {
  static constexpr int NW = NW_;                  // 4 or 8 waves; two waves per SIMD either way
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;              // queries per workgroup
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int KS = D / 16;               // 16-wide k steps over d
  static constexpr int DB = D / 32;               // 32-column blocks of dQ
  static constexpr int KB = BC / 32;              // 32-key blocks of S^T
  static constexpr int PS = BC / 16;              // 16-key k steps of dQ^T
  static constexpr int RS = lds_row_bytes<D>();   // bytes per K or V row in LDS
  static constexpr int GRS = D * 2;               // bytes per row in HBM
  static constexpr int TILE = BC * RS;            // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;          // K tile then V tile
  static constexpr int LPW = TILE / 1024 / NW;
  static_assert(TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads over the waves");
};

// One workgroup of the dQ pass: query block `bid` of `nblk` (before the XCD
// remap or the causal order).  smem holds 2 * DqTile<D, NW>::STAGE bytes;
// tlist and tcount are the workgroup's key-tile list (block-sparse mode only).
template <typename E, int D, bool CAUSAL, int NW, bool DROP, int MODE>
__device__ __forceinline__ void
dq_block(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
         const E* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
         E* __restrict__ dQ, DropArgs dp, int N, int Tr, float c /* scale*log2(e) */, float scale,
         MaskArgs mk, int bid, int nblk, char* smem, unsigned short* tlist, int& tcount) {
  using T = DqTile<D, NW>;
  using v8 = typename Vec<E>::v8;
  constexpr bool WINDOW = MODE == kMaskWindow, BLOCKS = MODE == kMaskBlocks;
  static_assert(!(DROP && MODE != kMaskDense), "dropout only with the dense or causal mask");
  static_assert(!BLOCKS || (T::BC == kMaskBlock && T::BR == 2 * kMaskBlock), "mask blocks are key tiles and half a row block");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses for the direct loads
  const int half = lane >> 5;
  const int l32 = lane & 31;
  int bh, it;
  if (CAUSAL) {
    int r;
    causal_order(bid, nblk / Tr, Tr, bh, r);
    it = Tr - 1 - r;  // longest rows first
  } else {
    const int tile = xcd_remap(bid, nblk);
    bh = tile / Tr;
    it = tile - bh * Tr;
  }
  const int q0 = it * T::BR;
  const size_t head = size_t(bh) * N * D;
  const E* Kh = K + head;
  const E* Vh = V + head;
  const int head_bytes = N * T::GRS;

  // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T): row
  // qrow, columns 16*s + 8*half .. +7.  Rows past N read as zero.
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;
  v8 qf[T::KS], df[T::KS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head, head_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dO + head, head_bytes);
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
      const int off = qrow * T::GRS + (16 * s + 8 * half) * 2;
      qf[s] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      df[s] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
    }
  }
  // this lane's query: LSE in base 2 and D (rows past N: 0; their dQ is never stored)
  float lq = 0.f, dd = 0.f;
  if (qrow < N) {
    lq = LSE2[size_t(bh) * N + qrow];
    dd = Dv[size_t(bh) * N + qrow];
  }

  const int Tc = (N + T::BC - 1) / T::BC;
  int nt = Tc;
  if (CAUSAL) nt = min(Tc, (min(q0 + T::BR, N) - 1) / T::BC + 1);
  const bool wave_active = wq0 < N;
  int nt_w = nt;
  if (CAUSAL && wave_active) nt_w = min(nt, (min(wq0 + 32, N) - 1) / T::BC + 1);
  // this workgroup's key tiles: [j0, nt), or (block-sparse) tlist[0 .. tcount);
  // each wave computes the tiles of [w0, nt_w) (block-sparse: those its own
  // 64-row block keeps)
  int j0 = 0, w0 = 0;
  if (WINDOW) {
    const int lo = mk.left >= 0 ? max(0, q0 - mk.left) : 0;
    const int hi = mk.right >= 0 ? (int)min((long long)N, (long long)q0 + T::BR + mk.right) : N;  // exclusive
    j0 = lo / T::BC;
    nt = (hi - 1) / T::BC + 1;
    w0 = mk.left >= 0 ? max(0, wq0 - mk.left) / T::BC : 0;
    nt_w = mk.right >= 0 ? (int)((min((long long)N, (long long)wq0 + 32 + mk.right) - 1) / T::BC + 1) : Tc;
  }
  // block-sparse: each tile of the list carries the keep flags of the
  // workgroup's two 64-row blocks (waves 0-1 and 2-3)
  if (BLOCKS) {
    const unsigned char* bmh = mk.bm + mk.bm_head_stride * (bh % mk.H);
    if (wave == 0) {
      const unsigned char* r0 = bmh + size_t(q0 / kMaskBlock) * mk.nb;
      const bool two = q0 + kMaskBlock < N;
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
  const int cnt = BLOCKS ? tcount : nt - j0;
  auto tile_at = [&](int idx) { return BLOCKS ? list_index(tlist[idx]) : j0 + idx; };
  auto wave_needs = [&](int idx, int j) {
    if (!wave_active || j >= nt_w || j < w0) return false;
    return !BLOCKS || list_keeps(tlist[idx], wave >> 1);
  };

  int goff[T::LPW];
#pragma unroll
  for (int u = 0; u < T::LPW; ++u) goff[u] = swz_src<D>((wave * T::LPW + u) * 1024 + 16 * lane);
  auto issue_loads = [&](int j, int stage) {
    const int key0 = j * T::BC;
    const int bytes = (N - key0) * T::GRS;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + size_t(key0) * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + size_t(key0) * D, bytes);
    char* dst = smem + stage * T::STAGE + wave * T::LPW * 1024;
#pragma unroll
    for (int u = 0; u < T::LPW; ++u) load_lds16(rk, dst + u * 1024, goff[u]);
#pragma unroll
    for (int u = 0; u < T::LPW; ++u) load_lds16(rv, dst + T::TILE + u * 1024, goff[u]);
  };

  // K / V rows (A operands of S^T and dP^T): rows kb*32 + l32, logical unit 2*st + half.
  int rof[T::KS];
#pragma unroll
  for (int st = 0; st < T::KS; ++st) rof[st] = l32 * T::RS + (((2 * st + half) ^ tile_swz<D>(l32)) * 16);
  // K^T (A operand of dQ^T), column block b.
  int tof[T::DB][2];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) {
    tof[b][0] = tr_off<D>(b, 0, lane);
    tof[b][1] = tr_off<D>(b, 1, lane);
  }

  f32x16 acc[T::DB];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) acc[b] = f32x16{};

  auto compute = [&](int j, const char* base) {
    // ---- S^T = K_j Q^T and dP^T = V_j dO^T (lane: query; element r: key kb*32 + acc_row(r))
    f32x16 s[T::KB], p[T::KB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      s[kb] = f32x16{};
      p[kb] = f32x16{};
    }
    {
      // K and V operands are read KPF k steps ahead, an order pinned by
      // scheduling barriers (left alone, the scheduler pulls each read next to
      // its MFMA and the LDS latency shows)
      constexpr int KPF = 2;
      v8 ka[KPF][T::KB], va[KPF][T::KB];
      auto rd = [&](int st, int kb, int v) {
        return *reinterpret_cast<const v8*>(base + v * T::TILE + kb * 32 * T::RS + rof[st]);
      };
#pragma unroll
      for (int st = 0; st < KPF; ++st)
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
          ka[st][kb] = rd(st, kb, 0);
          va[st][kb] = rd(st, kb, 1);
        }
#pragma unroll
      for (int st = 0; st < T::KS; ++st) {
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
          s[kb] = mfma32(ka[st % KPF][kb], qf[st], s[kb]);
          p[kb] = mfma32(va[st % KPF][kb], df[st], p[kb]);
        }
        if (st + KPF < T::KS)
#pragma unroll
          for (int kb = 0; kb < T::KB; ++kb) {
            ka[st % KPF][kb] = rd(st + KPF, kb, 0);
            va[st % KPF][kb] = rd(st + KPF, kb, 1);
          }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::KB * KPF, 0);
#pragma unroll
      for (int st = 0; st < T::KS; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::KB, 0);
        if (st + KPF < T::KS) __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::KB, 0);
      }
    }
    // ---- dS^T = P^T * (dP^T - D) with P^T = exp2(S^T*c - LSE2), rounded to the input type.
    // Keys past N have zero K and V rows, so they add nothing to dQ; causal
    // keys after the query are masked on the tiles that straddle the diagonal.
    // causal keys after the query: S^T = -inf (P = 0) on the tiles that
    // straddle the diagonal for some query of the wave (a wave-uniform branch)
    // Window edges inside the tile: keys outside [qrow - left, qrow + right].
    const int key0 = j * T::BC;
    if (CAUSAL && key0 + T::BC - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const int t = qrow - key0 - kb * 32 - 4 * half;  // key > qrow <=> 8*(r/4) + r%4 > t
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > t) s[kb][r] = -INFINITY;
      }
    }
    if (WINDOW && ((mk.left >= 0 && key0 < wq0 + 31 - mk.left) || (mk.right >= 0 && key0 + T::BC - 1 > wq0 + mk.right))) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (window_hides(mk, qrow, key0 + kb * 32 + acc_row(r, lane))) s[kb][r] = -INFINITY;
    }
    v8 db[T::PS];
    // dropout: registers 4m .. 4m+3 of a key block hold 4 consecutive keys of
    // this lane's query, one Philox block row; dP = Z * (dO V^T)
    // as in the forward: lane t of a quad draws key group t, the quad shares
    unsigned keep = 0;
    if constexpr (DROP) {
      const unsigned t = lane & 3;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const unsigned key = unsigned(key0 + kb * 32 + 8 * t + 4 * half);
        const unsigned mine = keep_block_rows(dp, unsigned(qrow) >> 2, key >> 2, unsigned(bh));
        keep |= quad_share_nibbles(mine, t) << (kb * 16);
      }
    }
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(fmaf(s[kb][r], c, -lq));
        float dpv = p[kb][r];
        if constexpr (DROP) dpv = keep_or_zero(dpv * dp.keep_scale, keep, kb * 16 + r);
        db[kb * 2 + (r >> 3)][r & 7] = (E)(pr * (dpv - dd));
      }
    // ---- dQ^T += K_j^T dS^T (k = key, in the accumulator's order)
    v8 ka = tr_pair<E>(base, tof[0][0], tof[0][1]);
#pragma unroll
    for (int ps = 0; ps < T::PS; ++ps)
#pragma unroll
      for (int b = 0; b < T::DB; ++b) {
        const int nb = (b + 1 < T::DB) ? b + 1 : 0;
        const int nps = (b + 1 < T::DB) ? ps : ps + 1;
        v8 kn;
        if (nps < T::PS) kn = tr_pair<E>(base + nps * 16 * T::RS, tof[nb][0], tof[nb][1]);
        acc[b] = mfma32(ka, db[ps], acc[b]);
        if (nps < T::PS) ka = kn;
      }
  };

  // step idx: tile tile_at(idx) from stage `stage`, loads of the next tile into the other
  auto step = [&](int idx, int stage) {
    if (idx + 1 < cnt) issue_loads(tile_at(idx + 1), stage ^ 1);
    const int j = tile_at(idx);
    if (wave_needs(idx, j)) compute(j, smem + stage * T::STAGE);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of the next tile have landed
    __syncthreads();
  };

  if (cnt > 0) {  // uniform over the workgroup
    issue_loads(tile_at(0), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    int idx = 0;
    for (; idx + 1 < cnt; idx += 2) {
      step(idx, 0);
      step(idx + 1, 1);
    }
    if (idx < cnt) step(idx, 0);
  }

  if (!wave_active) return;
  // dQ = scale * (dQ^T)^T; lane holds query qrow, rows past N are dropped by the buffer bounds
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(dQ + head, head_bytes);
#pragma unroll
  for (int b = 0; b < T::DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack2<E>(acc[b][4 * g + 0] * scale, acc[b][4 * g + 1] * scale);
      w[1] = pack2<E>(acc[b][4 * g + 2] * scale, acc[b][4 * g + 3] * scale);
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, qrow * T::GRS + (b * 32 + 8 * g + 4 * half) * 2, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// LDS bytes after a kernel's stages for a block-sparse step or tile list
// (kMaxMaskTiles entries) and its count; other modes keep 16 unused bytes.
constexpr int list_bytes(int mode) { return mode == kMaskBlocks ? 2 * kMaxMaskTiles + 16 : 16; }
__device__ __forceinline__ int& list_count(unsigned short* list, int mode) {
  return *reinterpret_cast<int*>(reinterpret_cast<char*>(list) + (mode == kMaskBlocks ? 2 * kMaxMaskTiles : 0));
}

template <typename E, int D, bool CAUSAL, bool DROP, int MODE>
__global__ void __launch_bounds__(256, 1)
bwd_dkdv_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
                const E* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
                E* __restrict__ dK, E* __restrict__ dV, DropArgs dp, int N, int Tk, float c, float scale,
                MaskArgs mk, int nblk) {
  // One LDS array holds the two stages, the staged K and V rows (persistent
  // workgroups) and the step list with its count (block-sparse): with a
  // second __shared__ variable in the kernel, hipcc waits for every direct
  // load before the next LDS read.
  constexpr bool kStaged = D <= 128 && MODE != kMaskBlocks;
  constexpr int kKvs = kStaged ? DkdvTile<D>::KVS : 0;
  __shared__ __attribute__((aligned(1024))) char smem[DkdvTile<D>::LDS + kKvs + list_bytes(MODE)];
  char* const kvs = smem + DkdvTile<D>::LDS;
  unsigned short* const slist = reinterpret_cast<unsigned short*>(smem + DkdvTile<D>::LDS + kKvs);
  int& scount = list_count(slist, MODE);
  // Grids larger than the GPU holds at once (one workgroup per CU) run as
  // persistent workgroups that take the key blocks in turn.  Block w runs on
  // a workgroup whose index is w mod 8, so on the XCD a one-block-per-
  // workgroup launch would give it; round by round the workgroups of an XCD
  // take its blocks in alternating order, so that longest-first causal
  // blocks even out over the rounds.  This saves the start of a new
  // workgroup between blocks (2-4 % at B4 H16 N4096 causal).
  const int G = gridDim.x;
  if (G >= nblk) {
    dkdv_block<E, D, CAUSAL, DROP, MODE>(Q, K, V, dO, LSE2, Dv, dK, dV, dp, N, Tk, c, scale, mk, blockIdx.x,
                                         nblk, smem, slist, scount);
    return;
  }
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = G >> 3;  // G is a multiple of 8
  // Each block's last step brings the K, V and first tiles of the workgroup's
  // next block into LDS (d <= 128 without a block mask), so that block starts
  // without a trip to memory: 3-4 % of a causal key block's time otherwise.
  int pst = -1;
  for (int i = 0;; ++i) {
    const int jj = (i & 1) ? per - 1 - j : j;
    const int w = 8 * (i * per + jj) + x;
    if (w >= nblk) break;
    const int jn = (i & 1) ? j : per - 1 - j;
    const int wn = 8 * ((i + 1) * per + jn) + x;
    pst = dkdv_block<E, D, CAUSAL, DROP, MODE, kStaged>(Q, K, V, dO, LSE2, Dv, dK, dV, dp, N, Tk, c, scale, mk,
                                                        w, nblk, smem, slist, scount, kvs, pst < 0 ? 0 : pst,
                                                        pst >= 0, wn < nblk ? wn : -1);
  }
}

template <typename E, int D, bool CAUSAL, int NW, bool DROP, int MODE>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
bwd_dq_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
              const E* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
              E* __restrict__ dQ, DropArgs dp, int N, int Tr, float c, float scale, MaskArgs mk) {
  // the tile list and its count (block-sparse) in the stages' array, as in the dK/dV pass
  __shared__ __attribute__((aligned(1024))) char smem[2 * DqTile<D, NW>::STAGE + list_bytes(MODE)];
  unsigned short* const tlist = reinterpret_cast<unsigned short*>(smem + 2 * DqTile<D, NW>::STAGE);
  int& tcount = list_count(tlist, MODE);
  dq_block<E, D, CAUSAL, NW, DROP, MODE>(Q, K, V, dO, LSE2, Dv, dQ, dp, N, Tr, c, scale, mk, blockIdx.x, gridDim.x,
                                         smem, tlist, tcount);
}

// Both passes in one grid, for problems whose two grids together fit on the
// CUs at once (Gk + Gq <= 256 workgroups; dense, window and block-sparse
// alike): workgroups [0, Gk) run the dK/dV pass, the rest the dQ pass, so
// neither pass leaves half of the CUs idle while the other waits for it.
// The passes share nothing but their inputs.
template <typename E, int D, bool CAUSAL, bool DROP, int MODE>
__global__ void __launch_bounds__(256, 1)
bwd_both_kernel(const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
                const E* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
                E* __restrict__ dQ, E* __restrict__ dK, E* __restrict__ dV, DropArgs dp, int N, int Tk, int Tr,
                int Gk, float c, float scale, MaskArgs mk) {
  constexpr int kLds = DkdvTile<D>::LDS > 2 * DqTile<D, 4>::STAGE ? DkdvTile<D>::LDS : 2 * DqTile<D, 4>::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[kLds + list_bytes(MODE)];
  unsigned short* const list = reinterpret_cast<unsigned short*>(smem + kLds);
  int& count = list_count(list, MODE);
  const int bid = blockIdx.x;
  if (bid < Gk)
    dkdv_block<E, D, CAUSAL, DROP, MODE>(Q, K, V, dO, LSE2, Dv, dK, dV, dp, N, Tk, c, scale, mk, bid, Gk, smem, list,
                                         count);
  else
    dq_block<E, D, CAUSAL, 4, DROP, MODE>(Q, K, V, dO, LSE2, Dv, dQ, dp, N, Tr, c, scale, mk, bid - Gk,
                                          (int)gridDim.x - Gk, smem, list, count);
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, bool DROP = false>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                               void* ws, hipStream_t st, DropArgs dp = DropArgs{}) {
  const long long rows = (long long)B * H * N;
  const BwdWorkspace w = bwd_workspace_layout(Shape{B, H, N, D});
  char* base = reinterpret_cast<char*>(ws);
  float* Dv = reinterpret_cast<float*>(base + w.d);
  float* lse2 = reinterpret_cast<float*>(base + w.lse2);
  const float c = scale * kLog2e;

  const long long pre_blocks = (rows * 8 + 255) / 256;
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3((unsigned)pre_blocks), dim3(256), 0, st,
                     (const E*)o, (const E*)dO, lse, Dv, lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int Tk = (N + DkdvTile<D>::BKV - 1) / DkdvTile<D>::BKV;
  const long long Gk = (long long)B * H * Tk * DkdvTile<D>::OS;
  // dQ pass: eight waves (256 rows) per workgroup for d = 128 and 96 grids that cover
  // every CU (each K/V tile streamed once for twice the rows); four waves
  // otherwise.  Unlike the forward, the causal dQ pass gains from eight waves
  // too (1-2 % at B4 H16 N4096 and B2 H8 N16000).
  const long long Gq8 = (long long)B * H * ((N + DqTile<D, 8>::BR - 1) / DqTile<D, 8>::BR);
  const bool dq8 = (D == 128 || D == 96) && Gq8 >= kNumCUs;
  const int Tr = dq8 ? (N + DqTile<D, 8>::BR - 1) / DqTile<D, 8>::BR : (N + DqTile<D, 4>::BR - 1) / DqTile<D, 4>::BR;
  const long long Gq = (long long)B * H * Tr;
  if (Gk > 0x7fffffffLL || Gq > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // Grids that fit on the CUs together run as one launch (1.5-1.7x faster at
  // B1 H8 N1024-2048 than two launches that each leave half of the CUs idle).
  if (!dq8 && Gk + Gq <= kNumCUs) {
    hipLaunchKernelGGL((bwd_both_kernel<E, D, CAUSAL, DROP, kMaskDense>), dim3((unsigned)(Gk + Gq)), dim3(256), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)dO, (const float*)lse2, (const float*)Dv,
                       (E*)dq, (E*)dk, (E*)dv, dp, N, Tk, Tr, (int)Gk, c, scale, MaskArgs{});
    return hipGetLastError();
  }
  const unsigned gk = (unsigned)(Gk > kNumCUs ? kNumCUs : Gk);  // persistent beyond one workgroup per CU
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL, DROP, kMaskDense>), dim3(gk), dim3(DkdvTile<D>::NT), 0,
                     st, (const E*)q, (const E*)k, (const E*)v, (const E*)dO,
                     (const float*)lse2, (const float*)Dv, (E*)dk, (E*)dv, dp, N, Tk, c, scale, MaskArgs{}, (int)Gk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128 || D == 96) {
    if (dq8) {
      hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL, 8, DROP, kMaskDense>), dim3((unsigned)Gq),
                         dim3(DqTile<D, 8>::NT), 0, st, (const E*)q, (const E*)k, (const E*)v, (const E*)dO,
                         (const float*)lse2, (const float*)Dv, (E*)dq, dp, N, Tr, c, scale, MaskArgs{});
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL, 4, DROP, kMaskDense>), dim3((unsigned)Gq), dim3(DqTile<D, 4>::NT), 0,
                     st, (const E*)q, (const E*)k, (const E*)v, (const E*)dO, (const float*)lse2, (const float*)Dv,
                     (E*)dq, dp, N, Tr, c, scale, MaskArgs{});
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_bwd_e(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                               int causal, void* ws, hipStream_t st) {
  if (d == 256)
    return causal ? launch_bwd_t<E, 256, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                  : launch_bwd_t<E, 256, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
  if (d == 96)
    return causal ? launch_bwd_t<E, 96, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                  : launch_bwd_t<E, 96, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
  if (d == 128)
    return causal ? launch_bwd_t<E, 128, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                  : launch_bwd_t<E, 128, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
  return causal ? launch_bwd_t<E, 64, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                : launch_bwd_t<E, 64, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                      int causal, void* ws, hipStream_t st) {
  return launch_bwd_e<__bf16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, ws, st);
}

template <typename E>
static hipError_t launch_bwd_dropout_e(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                        const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                        float scale, int causal, float p, unsigned long long seed, void* ws,
                                        hipStream_t st) {
  const DropArgs dp = make_drop_args(p, seed);
  if (d == 256)
    return causal ? launch_bwd_t<E, 256, true, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp)
                  : launch_bwd_t<E, 256, false, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp);
  if (d == 96)
    return causal ? launch_bwd_t<E, 96, true, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp)
                  : launch_bwd_t<E, 96, false, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp);
  if (d == 128)
    return causal ? launch_bwd_t<E, 128, true, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp)
                  : launch_bwd_t<E, 128, false, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp);
  return causal ? launch_bwd_t<E, 64, true, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp)
                : launch_bwd_t<E, 64, false, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st, dp);
}

hipError_t launch_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int causal, float p, unsigned long long seed, void* ws, bool fp16, hipStream_t st) {
  return fp16 ? launch_bwd_dropout_e<_Float16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, p, seed,
                                                ws, st)
              : launch_bwd_dropout_e<__bf16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, p, seed, ws,
                                             st);
}

// Sliding-window and block-sparse backward: the dense passes with a
// per-step predicate in the dK/dV pass and a per-tile one in the dQ pass
// (four-wave workgroups: 128 queries, two 64-row mask blocks).
template <typename E, int D, bool CAUSAL, int MODE>
static hipError_t launch_bwd_masked_t(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                      const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                                      const MaskArgs& mk, void* ws, hipStream_t st) {
  const long long rows = (long long)B * H * N;
  const BwdWorkspace w = bwd_workspace_layout(Shape{B, H, N, D});
  char* base = reinterpret_cast<char*>(ws);
  float* Dv = reinterpret_cast<float*>(base + w.d);
  float* lse2 = reinterpret_cast<float*>(base + w.lse2);
  const float c = scale * kLog2e;
  const long long pre_blocks = (rows * 8 + 255) / 256;
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3((unsigned)pre_blocks), dim3(256), 0, st,
                     (const E*)o, (const E*)dO, lse, Dv, lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int Tk = (N + DkdvTile<D>::BKV - 1) / DkdvTile<D>::BKV;
  const int Tr = (N + DqTile<D, 4>::BR - 1) / DqTile<D, 4>::BR;
  const long long Gk = (long long)B * H * Tk * DkdvTile<D>::OS, Gq = (long long)B * H * Tr;
  if (Gk > 0x7fffffffLL || Gq > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (Gk + Gq <= kNumCUs) {  // both passes in one launch, as in the dense backward
    hipLaunchKernelGGL((bwd_both_kernel<E, D, CAUSAL, false, MODE>), dim3((unsigned)(Gk + Gq)), dim3(256), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)dO, (const float*)lse2, (const float*)Dv,
                       (E*)dq, (E*)dk, (E*)dv, DropArgs{}, N, Tk, Tr, (int)Gk, c, scale, mk);
    return hipGetLastError();
  }
  const unsigned gk = (unsigned)(Gk > kNumCUs ? kNumCUs : Gk);  // persistent beyond one workgroup per CU
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL, false, MODE>), dim3(gk), dim3(DkdvTile<D>::NT), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, (const E*)dO, (const float*)lse2, (const float*)Dv,
                     (E*)dk, (E*)dv, DropArgs{}, N, Tk, c, scale, mk, (int)Gk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL, 4, false, MODE>), dim3((unsigned)Gq), dim3(DqTile<D, 4>::NT), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, (const E*)dO, (const float*)lse2, (const float*)Dv,
                     (E*)dq, DropArgs{}, N, Tr, c, scale, mk);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_bwd_window_e(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                      const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                      float scale, int left, int right, void* ws, hipStream_t st) {
  // a bound of N - 1 or more limits nothing: the same as no bound
  const MaskArgs mk{left >= N - 1 ? -1 : left, right >= N - 1 ? -1 : right, nullptr, 0, 0, H};
  if (d == 256)
    return launch_bwd_masked_t<E, 256, false, kMaskWindow>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk, ws, st);
  if (d == 96)
    return launch_bwd_masked_t<E, 96, false, kMaskWindow>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk, ws, st);
  if (d == 128)
    return launch_bwd_masked_t<E, 128, false, kMaskWindow>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk, ws, st);
  return launch_bwd_masked_t<E, 64, false, kMaskWindow>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk, ws, st);
}

template <typename E>
static hipError_t launch_bwd_blocksparse_e(const void* q, const void* k, const void* v, const void* o,
                                           const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                                           int H, int N, int d, float scale, int causal, const unsigned char* bm,
                                           int per_head, void* ws, hipStream_t st) {
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  const MaskArgs mk{-1, -1, bm, per_head ? (long long)nb * nb : 0, nb, H};
  if (d == 256)
    return causal ? launch_bwd_masked_t<E, 256, true, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                                  ws, st)
                  : launch_bwd_masked_t<E, 256, false, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale,
                                                                   mk, ws, st);
  if (d == 96)
    return causal ? launch_bwd_masked_t<E, 96, true, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                                 ws, st)
                  : launch_bwd_masked_t<E, 96, false, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                                  ws, st);
  if (d == 128)
    return causal ? launch_bwd_masked_t<E, 128, true, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                                 ws, st)
                  : launch_bwd_masked_t<E, 128, false, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                                  ws, st);
  return causal ? launch_bwd_masked_t<E, 64, true, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk, ws,
                                                              st)
                : launch_bwd_masked_t<E, 64, false, kMaskBlocks>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, mk,
                                                               ws, st);
}

hipError_t launch_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                             int left, int right, void* ws, bool fp16, hipStream_t st) {
  return fp16 ? launch_bwd_window_e<_Float16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, left, right, ws, st)
              : launch_bwd_window_e<__bf16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, left, right, ws, st);
}

hipError_t launch_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                  float scale, int causal, const unsigned char* bm, int per_head, void* ws, bool fp16,
                                  hipStream_t st) {
  return fp16 ? launch_bwd_blocksparse_e<_Float16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, bm,
                                                    per_head, ws, st)
              : launch_bwd_blocksparse_e<__bf16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, bm,
                                                 per_head, ws, st);
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace (D and LSE*log2(e), fully written by
// the pre-pass before any kernel reads it) lives in this file-scope device
// array, one copy per GPU.  Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol): the first call on each
// device, with that device current, looks its device address up once and
// keeps it.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int causal, hipStream_t st) {
  if (bwd_workspace_bytes(Shape{B, H, N, d}) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return e;
  return launch_bwd_e<__bf16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, ws, st);
}

hipError_t launch_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int causal, void* ws, hipStream_t st) {
  return launch_bwd_e<_Float16>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, ws, st);
}

}  // namespace fa
