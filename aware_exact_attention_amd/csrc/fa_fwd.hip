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
// gfx950 mapping of the bf16 kernel (one workgroup = 4 waves = 128 query rows):
//  * each wave owns 32 whole query rows, so the row statistics m and l never
//    leave the wave (no inter-wave exchange);
//  * the wave computes S^T = K_j Q_i^T with v_mfma_f32_32x32x16_bf16: the
//    accumulator puts one query per lane (lane % 32) and that query's keys in
//    the lane's registers, so the row max and row sum are mostly in-lane
//    reductions plus one exchange between lanes l and l+32;
//  * it then computes O^T += V_j^T P^T, which again keeps one query per lane,
//    so rescaling and the final division are in-lane; P^T is fed to the MFMA
//    straight from the score registers (rounded to bf16), never via memory;
//  * the Q fragment stays in VGPRs for the whole KV sweep; K_j is staged in
//    LDS row-major and V_j transposed (V^T), both with XOR swizzles that keep
//    the 128-bit LDS reads of a wave free of bank conflicts, and both double
//    buffered so the HBM loads of tile j+1 overlap the MFMAs of tile j;
//  * the exponentials are exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.h"
#include "fa_validate.h"

namespace fa {

template <int D>
struct FwdTile {
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int NT = 64 * NW;              // threads per workgroup
  static constexpr int BR = 32 * NW;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per KV tile
  static constexpr int KS = D / 16;               // 16-wide k steps of Q K^T
  static constexpr int DB = D / 32;               // 32-column blocks of O
  static constexpr int KB = BC / 32;              // 32-key blocks of S
  static constexpr int PS = BC / 16;              // 16-key k steps of P V
  static constexpr int K_UNITS = D / 8;           // 16-byte units per K row
  static constexpr int V_UNITS = BC / 8;          // 16-byte units per V^T row
  static constexpr int K_BYTES = BC * D * 2;
  static constexpr int V_BYTES = D * BC * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = BC * K_UNITS / NT;   // 16-byte K loads per thread per tile
  static constexpr int V_PIECES = (BC / 4) * (D / 8); // (4 keys x 8 columns) pieces of V per tile
  static_assert(BC * K_UNITS % NT == 0, "K tile must split evenly over the threads");
  static_assert(V_PIECES <= NT, "one V piece per thread at most");
};

// Byte offset of V^T[dcol][key] piece (4 keys starting at key chunk kc) in the
// LDS V^T tile.  Within every group of 16 keys the four 4-key chunks are
// stored in the order (0, 2 | 1, 3) so that one 16-byte unit holds exactly
// the 8 keys that one lane feeds to one PV MFMA step.
template <int D>
__device__ __forceinline__ int vt_offset(int dcol, int kc) {
  using T = FwdTile<D>;
  const int g = kc >> 2, cc = kc & 3;
  const int unit = 2 * g + (cc & 1);
  return dcol * (T::BC * 2) + swz<T::V_UNITS>(dcol, unit) * 16 + (cc >> 1) * 8;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                int N, int Tr, float c) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / Tr;
  int it = tile - bh * Tr;
  if (CAUSAL) it = Tr - 1 - it;  // longest rows first
  const int q0 = it * T::BR;
  const size_t head = size_t(bh) * N * D;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;

  // Q fragment (B operand of S^T = K Q^T): query row lane%32 of this wave,
  // columns 16*s + 8*half .. +7 for k step s.
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + (lane & 31);
  bf16x8 qf[T::KS];
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    if (qrow < N) qf[s] = *reinterpret_cast<const bf16x8*>(Qh + size_t(qrow) * D + 16 * s + 8 * half);
    else qf[s] = bf16x8{};
  }

  const int Tc = (N + T::BC - 1) / T::BC;
  int nt = Tc;
  if (CAUSAL) nt = min(Tc, (min(q0 + T::BR, N) - 1) / T::BC + 1);
  const bool wave_active = wq0 < N;
  int nt_w = nt;
  if (CAUSAL && wave_active) nt_w = min(nt, (min(wq0 + 32, N) - 1) / T::BC + 1);

  f32x16 o[T::DB];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) o[b] = f32x16{};
  float m = -INFINITY;  // running max of scale*log2(e)*score
  float l = 0.f;        // running sum of this lane's half of the keys

  u32x4 kst[T::K_LOADS];
  u32x4 vst[4];
  const int v_dc = tid % (D / 8), v_kc = tid / (D / 8);
  const bool v_loader = tid < T::V_PIECES;

  auto gload = [&](int j) {
    const int key0 = j * T::BC;
#pragma unroll
    for (int r = 0; r < T::K_LOADS; ++r) {
      const int idx = tid + r * T::NT;
      const int row = idx / T::K_UNITS, unit = idx % T::K_UNITS;
      const int key = key0 + row;
      kst[r] = key < N ? *reinterpret_cast<const u32x4*>(Kh + size_t(key) * D + unit * 8) : u32x4{};
    }
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + v_kc * 4 + r;
        vst[r] = key < N ? *reinterpret_cast<const u32x4*>(Vh + size_t(key) * D + v_dc * 8) : u32x4{};
      }
    }
  };

  auto lds_store = [&](int buf) {
    char* base = smem + buf * T::STAGE;
#pragma unroll
    for (int r = 0; r < T::K_LOADS; ++r) {
      const int idx = tid + r * T::NT;
      const int row = idx / T::K_UNITS, unit = idx % T::K_UNITS;
      *reinterpret_cast<u32x4*>(base + row * (D * 2) + swz<T::K_UNITS>(row, unit) * 16) = kst[r];
    }
    if (v_loader) {
      char* vb = base + T::K_BYTES;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dword w of each loaded row holds columns 2w (low half) and 2w+1 (high half)
        const unsigned a0 = vst[0][w], a1 = vst[1][w], a2 = vst[2][w], a3 = vst[3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int dcol = v_dc * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(vb + vt_offset<D>(dcol, v_kc)) = lo;
        *reinterpret_cast<u32x2*>(vb + vt_offset<D>(dcol + 1, v_kc)) = hi;
      }
    }
  };

  auto compute = [&](int j, const char* base) {
    const char* Ks = base;
    const char* Vs = base + T::K_BYTES;
    // S^T block kb: rows = keys kb*32 + (lane%32), cols = this wave's queries
    f32x16 s[T::KB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      s[kb] = f32x16{};
      const int row = kb * 32 + (lane & 31);
#pragma unroll
      for (int st = 0; st < T::KS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Ks + row * (D * 2) + swz<T::K_UNITS>(row, 2 * st + half) * 16);
        s[kb] = mfma32(a, qf[st], s[kb]);
      }
    }
    // masks: keys past N (ragged tail) and, if causal, keys after the query
    const int key0 = j * T::BC;
    bool need = key0 + T::BC > N;
    if (CAUSAL) need = need || (key0 + T::BC - 1 > wq0);
    if (need) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + acc_row(r, lane);
          if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
        }
    }
    // running max (scale > 0, so max(score)*c == max(score*c))
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, wave_swap32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // row with nothing visible yet
    const float alpha = exp2_fast(m - m_use);
    m = m_new;
    // probabilities, this lane's share of the row sum, bf16 P^T fragments
    float rs = 0.f;
    bf16x8 pb[T::PS];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[kb][r], c, -m_use));
        rs += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    l = l * alpha + rs;
    if (alpha != 1.f) {
#pragma unroll
      for (int b = 0; b < T::DB; ++b) o[b] *= alpha;
    }
    // O^T block b += V^T[b*32 .. +32][keys] * P^T
#pragma unroll
    for (int b = 0; b < T::DB; ++b) {
      const int dcol = b * 32 + (lane & 31);
#pragma unroll
      for (int ps = 0; ps < T::PS; ++ps) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            Vs + dcol * (T::BC * 2) + swz<T::V_UNITS>(dcol, 2 * ps + half) * 16);
        o[b] = mfma32(a, pb[ps], o[b]);
      }
    }
  };

  gload(0);
  lds_store(0);
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) gload(j + 1);
    if (wave_active && j < nt_w) compute(j, smem + (j & 1) * T::STAGE);
    if (j + 1 < nt) lds_store((j + 1) & 1);
    __syncthreads();
  }

  if (!wave_active || qrow >= N) return;
  const float lt = l + wave_swap32(l);
  const float inv = 1.f / lt;
  __bf16* Orow = O + head + size_t(qrow) * D;
#pragma unroll
  for (int b = 0; b < T::DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(o[b][4 * g + 0] * inv, o[b][4 * g + 1] * inv);
      w[1] = pack_bf16x2(o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(Orow + b * 32 + 8 * g + 4 * half) = w;
    }
  if (half == 0) LSE[size_t(bh) * N + qrow] = (m + log2_fast(lt)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 path: no bf16 rounding anywhere.  Four lanes share one query row (each
// holds a quarter of the columns of q and of the output), a workgroup covers
// 64 rows, and K/V tiles of 32 keys are staged in LDS and read by broadcast.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, int N, int Tr, float scale) {
  constexpr int QL = 4, BR = 64, BC = 32, NCH = D / 4 / QL;  // float4 chunks per lane
  __shared__ __attribute__((aligned(16))) float Ks[BC * D];
  __shared__ __attribute__((aligned(16))) float Vs[BC * D];
  const int tid = threadIdx.x;
  const int sub = tid & (QL - 1);
  const int tile = blockIdx.x;
  const int bh = tile / Tr;
  const int q0 = (tile - bh * Tr) * BR;
  const int qrow = q0 + tid / QL;
  const size_t head = size_t(bh) * N * D;

  // lane holds columns 4*(i*QL + sub) .. +3 for i < NCH
  f32x4 q[NCH], o[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    q[i] = qrow < N ? *reinterpret_cast<const f32x4*>(Q + head + size_t(qrow) * D + 4 * (i * QL + sub)) : f32x4{};
    o[i] = f32x4{};
  }
  float m = -INFINITY, l = 0.f;
  const int Tc = (N + BC - 1) / BC;
  const int nt = CAUSAL ? min(Tc, (min(q0 + BR, N) - 1) / BC + 1) : Tc;
  for (int j = 0; j < nt; ++j) {
    const int key0 = j * BC;
    __syncthreads();
    for (int idx = tid; idx < BC * D / 4; idx += 256) {
      const int row = idx / (D / 4), col = idx % (D / 4);
      const int key = key0 + row;
      f32x4 kv = {}, vv = {};
      if (key < N) {
        kv = *reinterpret_cast<const f32x4*>(K + head + size_t(key) * D + 4 * col);
        vv = *reinterpret_cast<const f32x4*>(V + head + size_t(key) * D + 4 * col);
      }
      *reinterpret_cast<f32x4*>(Ks + row * D + 4 * col) = kv;
      *reinterpret_cast<f32x4*>(Vs + row * D + 4 * col) = vv;
    }
    __syncthreads();
    float sc[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < BC; ++kk) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(Ks + kk * D + 4 * (i * QL + sub));
        acc = fmaf(q[i][0], kv[0], acc);
        acc = fmaf(q[i][1], kv[1], acc);
        acc = fmaf(q[i][2], kv[2], acc);
        acc = fmaf(q[i][3], kv[3], acc);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = key0 + kk;
      float sv = acc * scale;
      if (key >= N || (CAUSAL && key > qrow)) sv = -INFINITY;
      sc[kk] = sv;
      mx = fmaxf(mx, sv);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < NCH; ++i) o[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < BC; ++kk) {
      const float p = expf(sc[kk] - m_use);
      l += p;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(Vs + kk * D + 4 * (i * QL + sub));
        o[i][0] = fmaf(p, vv[0], o[i][0]);
        o[i][1] = fmaf(p, vv[1], o[i][1]);
        o[i][2] = fmaf(p, vv[2], o[i][2]);
        o[i][3] = fmaf(p, vv[3], o[i][3]);
      }
    }
  }
  if (qrow >= N) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    *reinterpret_cast<f32x4*>(O + head + size_t(qrow) * D + 4 * (i * QL + sub)) = o[i] * inv;
  if (sub == 0) LSE[size_t(bh) * N + qrow] = m + logf(l);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int B, int H, int N, float scale, hipStream_t st) {
  using T = FwdTile<D>;
  const int Tr = (N + T::BR - 1) / T::BR;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(T::NT), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, N, Tr,
                     scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 128) return causal ? launch_fwd_bf16_t<128, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_bf16_t<128, false>(q, k, v, o, lse, B, H, N, scale, st);
  return causal ? launch_fwd_bf16_t<64, true>(q, k, v, o, lse, B, H, N, scale, st)
                : launch_fwd_bf16_t<64, false>(q, k, v, o, lse, B, H, N, scale, st);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const float* q, const float* k, const float* v, float* o, float* lse,
                                   int B, int H, int N, float scale, hipStream_t st) {
  const int Tr = (N + 63) / 64;
  const long long G = (long long)B * H * Tr;
  if (G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)G), dim3(256), 0, st, q, k, v, o, lse, N,
                     Tr, scale);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 128) return causal ? launch_fwd_f32_t<128, true>(q, k, v, o, lse, B, H, N, scale, st)
                              : launch_fwd_f32_t<128, false>(q, k, v, o, lse, B, H, N, scale, st);
  return causal ? launch_fwd_f32_t<64, true>(q, k, v, o, lse, B, H, N, scale, st)
                : launch_fwd_f32_t<64, false>(q, k, v, o, lse, B, H, N, scale, st);
}

}  // namespace fa
