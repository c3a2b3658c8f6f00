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
// Three kernels on the caller's stream:
//  1. bwd_pre: D = rowsum(dO * O) in fp32, and zeroes the fp32 dQ accumulator
//     (a fill kernel rather than a memset, so the sequence is graph-safe);
//  2. bwd_main: one workgroup per (b, h, 128-key block); each of its 4 waves
//     owns 32 keys whose K and V fragments stay in VGPRs and whose dK^T and
//     dV^T accumulate on chip.  The workgroup streams 32-query steps (causal:
//     starting at the diagonal): Q and dO are staged in LDS both row-major and
//     transposed; S = Q K^T and dP = dO V^T put one key per lane, so P and dS
//     feed the dV^T and dK^T MFMAs straight from registers; dS is written to
//     LDS once so that dQ = dS K can be formed across all 128 keys and added to
//     the fp32 accumulator with one coalesced atomic per element;
//  3. bwd_dq_convert: dQ = bf16(scale * accumulator).
#include "fa_common.h"
#include "fa_validate.h"

namespace fa {

template <int D>
struct BwdTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BKV = 32 * NW;  // keys per workgroup
  static constexpr int BQ = 32;        // queries per step
  static constexpr int KS = D / 16;    // 16-wide k steps over d
  static constexpr int DB = D / 32;    // 32-column blocks over d
  static constexpr int QK_BYTES = BQ * D * 2;      // one row-major or transposed Q/dO tile
  static constexpr int DS_BYTES = BQ * BKV * 2;    // dS tile [query][key]
  static constexpr int KT_BYTES = D * BKV * 2;     // K^T [d][key]
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + QK_BYTES;
  static constexpr int OFF_QT = OFF_DO + QK_BYTES;
  static constexpr int OFF_DOT = OFF_QT + QK_BYTES;
  static constexpr int OFF_DS = OFF_DOT + QK_BYTES;
  static constexpr int OFF_KT = OFF_DS + DS_BYTES;
  static constexpr int OFF_LSE = OFF_KT + KT_BYTES;
  static constexpr int OFF_DD = OFF_LSE + BQ * 4;
  static constexpr int LDS = OFF_DD + BQ * 4;
  static constexpr int PIECES = (BQ / 4) * (D / 8);   // (4 rows x 8 cols) pieces of one Q tile
  static_assert(2 * PIECES <= NT, "one Q or dO piece per thread");
};

// LDS offsets ---------------------------------------------------------------
// Row-major [32 rows][D] tile (Q or dO), 16-byte units swizzled by row.
template <int D>
__device__ __forceinline__ int rm_offset(int row, int unit) {
  return row * (D * 2) + swz<D / 8>(row, unit) * 16;
}
// Transposed [D][32 rows] tile: rows of 64 bytes (4 units).  Within each group
// of 16 query rows the 4-row chunks are stored (0, 2 | 1, 3) so that one
// 16-byte unit holds the 8 queries one lane feeds to one MFMA k step.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int tr_offset(int dcol, int qc) {
  const int g = qc >> 2, cc = qc & 3;
  const int unit = 2 * g + (cc & 1);
  return dcol * 64 + ((unit ^ swz4(dcol)) * 16) + (cc >> 1) * 8;
}
// K^T [D][128 keys], plain key order, rows of 256 bytes (16 units).
__device__ __forceinline__ int kt_offset(int dcol, int key) {
  return dcol * 256 + swz<16>(dcol, key >> 3) * 16 + (key & 7) * 2;
}
// dS [32 queries][128 keys], rows of 256 bytes.
__device__ __forceinline__ int ds_offset(int q, int key) {
  return q * 256 + swz<16>(q, key >> 3) * 16 + (key & 7) * 2;
}

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and zero the dQ accumulator.  8 lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO, float* __restrict__ Dv,
               float* __restrict__ dq_acc, long long rows) {
  constexpr int PER = D / 8;  // elements per lane
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid >> 3;
  const int sub = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const __bf16* o = O + row * D + sub * PER;
    const __bf16* g = dO + row * D + sub * PER;
#pragma unroll
    for (int u = 0; u < PER / 8; ++u) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + 8 * u);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(g + 8 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
    float* z = dq_acc + row * D + sub * PER;
#pragma unroll
    for (int u = 0; u < PER / 4; ++u) *reinterpret_cast<f32x4*>(z + 4 * u) = f32x4{};
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && sub == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
                float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                int N, int Tk, float c /* scale*log2(e) */, float scale) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) char smem[T::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / Tk;
  int jt = tile - bh * Tk;
  if (CAUSAL) jt = Tk - 1 - jt;  // blocks with fewer query steps last
  const int k0 = jt * T::BKV;
  const size_t head = size_t(bh) * N * D;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;
  const __bf16* dOh = dO + head;
  const float* LSEh = LSE + size_t(bh) * N;
  const float* Dh = Dv + size_t(bh) * N;
  float* dQh = dq_acc + head;

  // K and V fragments of this wave's keys: B operands (k = d, n = key).
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + (lane & 31);
  bf16x8 kf[T::KS], vf[T::KS];
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    if (key < N) {
      kf[s] = *reinterpret_cast<const bf16x8*>(Kh + size_t(key) * D + 16 * s + 8 * half);
      vf[s] = *reinterpret_cast<const bf16x8*>(Vh + size_t(key) * D + 16 * s + 8 * half);
    } else {
      kf[s] = bf16x8{};
      vf[s] = bf16x8{};
    }
  }
  // K^T of the whole 128-key block into LDS (B operand of dQ = dS K).
  {
    char* kt = smem + T::OFF_KT;
    constexpr int KT_PIECES = (T::BKV / 4) * (D / 8);
    for (int p = tid; p < KT_PIECES; p += T::NT) {
      const int dc = p % (D / 8), kc = p / (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + kc * 4 + i;
        r[i] = kk < N ? *reinterpret_cast<const u32x4*>(Kh + size_t(kk) * D + dc * 8) : u32x4{};
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 lo, hi;
        lo[0] = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        lo[1] = (r[2][w] & 0xffffu) | (r[3][w] << 16);
        hi[0] = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi[1] = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
        const int dcol = dc * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(kt + kt_offset(dcol, kc * 4)) = lo;
        *reinterpret_cast<u32x2*>(kt + kt_offset(dcol + 1, kc * 4)) = hi;
      }
    }
  }

  f32x16 dkt[T::DB], dvt[T::DB];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) {
    dkt[b] = f32x16{};
    dvt[b] = f32x16{};
  }

  const int Tq = (N + T::BQ - 1) / T::BQ;
  const int i_begin = CAUSAL ? (k0 / T::BQ) : 0;

  // staging roles: threads [0, PIECES) load Q pieces, [PIECES, 2*PIECES) dO pieces
  const bool stager = tid < 2 * T::PIECES;
  const bool st_is_do = tid >= T::PIECES;
  const int pidx = st_is_do ? tid - T::PIECES : tid;
  const int st_dc = pidx % (D / 8), st_qc = pidx / (D / 8);

  for (int i = i_begin; i < Tq; ++i) {
    const int qs = i * T::BQ;
    // ---- stage Q_i, dO_i (row-major and transposed), LSE and D
    if (stager) {
      const __bf16* src = st_is_do ? dOh : Qh;
      u32x4 r[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int qq = qs + st_qc * 4 + x;
        r[x] = qq < N ? *reinterpret_cast<const u32x4*>(src + size_t(qq) * D + st_dc * 8) : u32x4{};
      }
      char* rm = smem + (st_is_do ? T::OFF_DO : T::OFF_Q);
      char* tr = smem + (st_is_do ? T::OFF_DOT : T::OFF_QT);
#pragma unroll
      for (int x = 0; x < 4; ++x) *reinterpret_cast<u32x4*>(rm + rm_offset<D>(st_qc * 4 + x, st_dc)) = r[x];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 lo, hi;
        lo[0] = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        lo[1] = (r[2][w] & 0xffffu) | (r[3][w] << 16);
        hi[0] = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi[1] = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
        const int dcol = st_dc * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(tr + tr_offset(dcol, st_qc)) = lo;
        *reinterpret_cast<u32x2*>(tr + tr_offset(dcol + 1, st_qc)) = hi;
      }
    }
    if (tid < T::BQ) {
      const int qq = qs + tid;
      // rows past N get LSE = +inf, so their recomputed P is exactly 0
      reinterpret_cast<float*>(smem + T::OFF_LSE)[tid] = qq < N ? LSEh[qq] * kLog2e : INFINITY;
      reinterpret_cast<float*>(smem + T::OFF_DD)[tid] = qq < N ? Dh[qq] : 0.f;
    }
    __syncthreads();

    // ---- per-wave recompute and dK, dV accumulation
    // skip a wave whose keys all come after every query of this step
    const bool wave_visible = !CAUSAL || (kw0 <= qs + T::BQ - 1);
    char* dss = smem + T::OFF_DS;
    if (wave_visible && kw0 < N) {
      const char* qsm = smem + T::OFF_Q;
      const char* dosm = smem + T::OFF_DO;
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int st = 0; st < T::KS; ++st) {
        const int row = lane & 31;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qsm + rm_offset<D>(row, 2 * st + half));
        sacc = mfma32(qa, kf[st], sacc);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(dosm + rm_offset<D>(row, 2 * st + half));
        dpacc = mfma32(da, vf[st], dpacc);
      }
      // lane holds key `key`; element j is query qs + acc_row(j)
      const float* lse2 = reinterpret_cast<const float*>(smem + T::OFF_LSE);
      const float* dd = reinterpret_cast<const float*>(smem + T::OFF_DD);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 8 * g + 4 * half);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd + 8 * g + 4 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * g + e;
          const int qq = qs + 8 * g + 4 * half + e;
          float p = exp2_fast(fmaf(sacc[j], c, -l4[e]));
          if (key >= N || (CAUSAL && key > qq)) p = 0.f;
          const float ds = p * (dpacc[j] - d4[e]);
          pb[j >> 3][j & 7] = (__bf16)p;
          const __bf16 dsh = (__bf16)ds;
          dsb[j >> 3][j & 7] = dsh;
          *reinterpret_cast<__bf16*>(dss + ds_offset(8 * g + 4 * half + e, wave * 32 + (lane & 31))) = dsh;
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS  (k = query)
      const char* qt = smem + T::OFF_QT;
      const char* dot = smem + T::OFF_DOT;
#pragma unroll
      for (int b = 0; b < T::DB; ++b) {
        const int dcol = b * 32 + (lane & 31);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = dcol * 64 + (((2 * h + half) ^ swz4(dcol)) * 16);
          const bf16x8 doa = *reinterpret_cast<const bf16x8*>(dot + off);
          dvt[b] = mfma32(doa, pb[h], dvt[b]);
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qt + off);
          dkt[b] = mfma32(qa, dsb[h], dkt[b]);
        }
      }
    } else {
      // this wave's keys contribute nothing to the step: zero its dS columns
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *reinterpret_cast<__bf16*>(dss + ds_offset(acc_row(j, lane), wave * 32 + (lane & 31))) = (__bf16)0.f;
    }
    __syncthreads();

    // ---- dQ_i += dS K over the 128 keys: wave w owns column block w
    if (wave < T::DB) {
      const char* kt = smem + T::OFF_KT;
      f32x16 acc = f32x16{};
      const int row = lane & 31;
      const int dcol = wave * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < T::BKV / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(dss + row * 256 + swz<16>(row, 2 * ks + half) * 16);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(kt + dcol * 256 + swz<16>(dcol, 2 * ks + half) * 16);
        acc = mfma32(a, b, acc);
      }
      // element j: query qs + acc_row(j), column dcol
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qq = qs + acc_row(j, lane);
        if (qq < N) unsafeAtomicAdd(dQh + size_t(qq) * D + dcol, acc[j]);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: dK = scale * dK^T^T, dV = dV^T^T; lane holds key `key`
  if (key >= N) return;
  __bf16* dKr = dK + head + size_t(key) * D;
  __bf16* dVr = dV + head + size_t(key) * D;
#pragma unroll
  for (int b = 0; b < T::DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = b * 32 + 8 * g + 4 * half;
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dkt[b][4 * g + 0] * scale, dkt[b][4 * g + 1] * scale);
      wk[1] = pack_bf16x2(dkt[b][4 * g + 2] * scale, dkt[b][4 * g + 3] * scale);
      wv[0] = pack_bf16x2(dvt[b][4 * g + 0], dvt[b][4 * g + 1]);
      wv[1] = pack_bf16x2(dvt[b][4 * g + 2], dvt[b][4 * g + 3]);
      *reinterpret_cast<u32x2*>(dKr + col) = wk;
      *reinterpret_cast<u32x2*>(dVr + col) = wv;
    }
}

// ---------------------------------------------------------------------------
// 3. dQ = bf16(scale * accumulator), 8 elements per thread
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_dq_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq, long long n8, float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  u32x4 w;
  w[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
  w[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
  w[2] = pack_bf16x2(b[0] * scale, b[1] * scale);
  w[3] = pack_bf16x2(b[2] * scale, b[3] * scale);
  *reinterpret_cast<u32x4*>(dq + 8 * i) = w;
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                               void* ws, hipStream_t st) {
  using T = BwdTile<D>;
  const long long rows = (long long)B * H * N;
  const size_t acc_bytes = (size_t(rows) * D * 4 + 255) / 256 * 256;
  float* dq_acc = reinterpret_cast<float*>(ws);
  float* Dv = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + acc_bytes);

  const long long pre_blocks = (rows * 8 + 255) / 256;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_blocks), dim3(256), 0, st,
                     (const __bf16*)o, (const __bf16*)dO, Dv, dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int Tk = (N + T::BKV - 1) / T::BKV;
  const long long G = (long long)B * H * Tk;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(T::NT), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse, Dv, dq_acc,
                     (__bf16*)dk, (__bf16*)dv, N, Tk, scale * kLog2e, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     (const float*)dq_acc, (__bf16*)dq, n8, scale);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                      int causal, void* ws, hipStream_t st) {
  if (d == 128)
    return causal ? launch_bwd_t<128, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                  : launch_bwd_t<128, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
  return causal ? launch_bwd_t<64, true>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st)
                : launch_bwd_t<64, false>(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, ws, st);
}

}  // namespace fa
