// fa_fwd.hip -- forward attention kernels for gfx950.
//
// Tiled exact attention with the online softmax (ainews.cool, "flash-attention
// transformer optimization", technical deep dive: blocks that fit on-chip, running maximum
// and normaliser; bmjup.com, "FlashAttention-2 ... 实战解析", section 2.2: numerator and
// denominator kept apart and combined once at the end; section 3.2: the Q tile stays in
// registers while K and V tiles go through shared memory).
//
// bf16 kernel, one workgroup = 4 waves = 128 query rows of one (batch, query head):
//   * each wave owns 32 query rows; its Q rows sit in VGPRs as the B operand of
//     S^T = K Q^T (32 keys x 32 rows per MFMA tile), so every lane holds one query row
//     and 16 of its scores per tile -> row max/sum need one cross-half exchange only;
//   * K and V tiles of 64 keys are staged in LDS (row stride d + 8 elements) from
//     16-byte coalesced global loads, with the next tile's loads in flight during the
//     current tile's math;
//   * P^T (the accumulator of S^T after exp2) feeds O^T += V^T P^T directly as the B
//     operand; V^T comes from LDS with the transposing ds_read_b64_tr_b16;
//   * scores are handled in log2 units: t = (q.k) * |scale| * log2(e), so each probability
//     is one FMA and one exp2; a negative scale is handled by negating Q exactly;
//   * key tiles outside the causal / sliding-window band are never visited, and only
//     tiles crossing the band edge (or the end of the sequence) pay for per-element masks
//     (bmjup.com page, section 3.3: tile-level encoding of the mask);
//   * grid: (batch, head) major, longest query tiles first inside a head, block ids
//     remapped so that all tiles of a head run on one XCD and share its L2.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;      // query rows per workgroup
  static constexpr int BN = 64;       // keys per iteration
  static constexpr int STR = D + 8;   // LDS row stride in elements (16-byte pad)
  static constexpr int LDS_BYTES = 2 * BN * STR * 2;
  static constexpr int OCC = D <= 128 ? 2 : 1;  // workgroups per CU the registers allow
};

__device__ __forceinline__ bool key_allowed(int row, int key, int N, int causal, int window) {
  return key < N && (!causal || key <= row) && (window <= 0 || key >= row - window + 1);
}

template <int D>
__global__ __launch_bounds__(256, FwdCfg<D>::OCC) void fwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int N,
    int causal, int window, float c, int neg_q) {
  using Cfg = FwdCfg<D>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, STR = Cfg::STR;
  constexpr int NC = D / 16;  // k-steps of S^T over the head dim
  constexpr int ND = D / 32;  // 32-wide head-dim tiles of O^T
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* smK = reinterpret_cast<bf16_t*>(smem);
  bf16_t* smV = smK + BN * STR;

  const int num_m = (N + BM - 1) / BM;
  const int total = B * Hq * num_m;
  const int lin = xcd_remap(blockIdx.x, total);
  const int head = lin / num_m;
  const int mb = num_m - 1 - (lin - head * num_m);
  const int b = head / Hq, hq = head - b * Hq;
  const int hkv = hq / (Hq / Hkv);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;
  const int m0 = mb * BM;
  const int wr0 = m0 + w * 32;
  const int row = wr0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Qh = Q + ((size_t)b * N * Hq + hq) * D;
  const bf16_t* Kh = K + ((size_t)b * N * Hkv + hkv) * D;
  const bf16_t* Vh = V + ((size_t)b * N * Hkv + hkv) * D;

  // Q^T operand: lane holds Q[row][16c + 8hh .. +7] for every k-step c.
  bf16x8 qop[NC];
  if (row < N) {
    const bf16_t* qr = Qh + (size_t)row * qs + 8 * hh;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qop[cc] = __builtin_bit_cast(bf16x8, gload16(qr + 16 * cc));
      if (neg_q) qop[cc] = negate8(qop[cc]);
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qop[cc] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  // Key range any row of this workgroup may attend.
  int kv_lo = 0, kv_hi = N;
  if (causal) kv_hi = min(N, m0 + BM);
  if (window > 0) kv_lo = max(0, m0 - window + 1);
  const int nb_lo = kv_lo / BN, nb_hi = (kv_hi + BN - 1) / BN;

  constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  constexpr int PT = BN * CPR / 256;  // chunks per thread per tile
  uint4 kr[PT], vr[PT];
  auto gload = [&](int nb) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int ch = tid + 256 * i, key = ch / CPR, dc = ch - key * CPR;
      const int n = nb * BN + key;
      if (n < N) {
        kr[i] = gload16(Kh + (size_t)n * ks + dc * 8);
        vr[i] = gload16(Vh + (size_t)n * ks + dc * 8);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int ch = tid + 256 * i, key = ch / CPR, dc = ch - key * CPR;
      *reinterpret_cast<uint4*>(smK + key * STR + dc * 8) = kr[i];
      *reinterpret_cast<uint4*>(smV + key * STR + dc * 8) = vr[i];
    }
  };

  float m_i = -INFINITY;  // running max of t (log2 units), shared by both lane halves
  float l_i = 0.f;        // running sum of this lane's half of the probabilities
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();

  if (nb_lo < nb_hi) gload(nb_lo);
  for (int nb = nb_lo; nb < nb_hi; ++nb) {
    __syncthreads();
    swrite();
    __syncthreads();
    if (nb + 1 < nb_hi) gload(nb + 1);

    const int n0 = nb * BN;
    const bool active = wr0 < N && (!causal || n0 <= wr0 + 31) &&
                        (window <= 0 || n0 + BN - 1 >= wr0 - window + 1);
    if (!active) continue;
    const bool need_mask = (n0 + BN > N) || (causal && n0 + BN - 1 > wr0) ||
                           (window > 0 && n0 < wr0 + 32 - window);

    // S^T tiles for keys n0 + [0, 32) and n0 + [32, 64).
    f32x16 s0 = zero16(), s1 = zero16();
    const bf16_t* kp = smK + l32 * STR + 8 * hh;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const bf16x8 k0 = lds_read_b128(kp + 16 * cc);
      const bf16x8 k1 = lds_read_b128(kp + 32 * STR + 16 * cc);
      s0 = mfma32(k0, qop[cc], s0);
      s1 = mfma32(k1, qop[cc], s1);
    }

    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = (r >> 2) * 8 + hh * 4 + (r & 3);
        if (!key_allowed(row, n0 + kl, N, causal, window)) s0[r] = -INFINITY;
        if (!key_allowed(row, n0 + 32 + kl, N, causal, window)) s1[r] = -INFINITY;
      }
    }

    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, xor32(mx));
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_i, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_i - m_use);

    bf16x8 p[2][2];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float e0 = fast_exp2(fmaf(s0[r], c, -m_use));
      float e1 = fast_exp2(fmaf(s0[r + 1], c, -m_use));
      float f0 = fast_exp2(fmaf(s1[r], c, -m_use));
      float f1 = fast_exp2(fmaf(s1[r + 1], c, -m_use));
      if (need_mask) {  // masked entries are exactly 0 (also when scale == 0)
        if (s0[r] == -INFINITY) e0 = 0.f;
        if (s0[r + 1] == -INFINITY) e1 = 0.f;
        if (s1[r] == -INFINITY) f0 = 0.f;
        if (s1[r + 1] == -INFINITY) f1 = 0.f;
      }
      rs += (e0 + e1) + (f0 + f1);
      const bf16x2 pe = to_bf16x2(e0, e1), pf = to_bf16x2(f0, f1);
      p[0][r >> 3][r & 7] = pe[0];
      p[0][r >> 3][(r & 7) + 1] = pe[1];
      p[1][r >> 3][r & 7] = pf[0];
      p[1][r >> 3][(r & 7) + 1] = pf[1];
    }
    l_i = alpha * l_i + rs;
    m_i = m_new;
    if (alpha != 1.f) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }

    // O^T += V^T P^T : V^T operand via transposed LDS reads.
    const bf16_t* vbase = smV + (hh * 4 + (j16 >> 2)) * STR + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16_t* vp = vbase + (kt * 32 + 16 * c2) * STR + 32 * dt;
          const bf16x8 vop = lds_read_tr_x2(vp, vp + 8 * STR);
          acc[dt] = mfma32(vop, p[kt][c2], acc[dt]);
        }
      }
    }
  }

  // Epilogue: O = acc / l (one rounding to bf16), LSE = (m + log2 l) * ln 2.
  const float l = l_i + xor32(l_i);
  if (row < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* orow = O + ((size_t)b * N + row) * qs + (size_t)hq * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const bf16x2 lo = to_bf16x2(acc[dt][4 * g4] * inv, acc[dt][4 * g4 + 1] * inv);
        const bf16x2 hi = to_bf16x2(acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv);
        uint2 u;
        u.x = __builtin_bit_cast(uint32_t, lo);
        u.y = __builtin_bit_cast(uint32_t, hi);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * g4 + 4 * hh) = u;
      }
    }
    if (hh == 0)
      LSE[((size_t)b * Hq + hq) * N + row] = l > 0.f ? (m_i + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------
// float32 forward: 64 query rows per workgroup, 4 threads per row (each a quarter of the
// head dim), K/V tiles of 32 keys in LDS, online softmax per tile.  Plain fp32 FMAs.
template <int D>
struct Fp32Cfg {
  static constexpr int BM = 64, BN = 32, DP = D / 4;
  static constexpr int LDS_BYTES = 2 * BN * D * 4;
};

template <int D>
__global__ __launch_bounds__(256) void fwd_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int N, int causal,
    int window, float c) {
  using Cfg = Fp32Cfg<D>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, DP = Cfg::DP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sK = reinterpret_cast<float*>(smem);
  float* sV = sK + BN * D;

  const int num_m = (N + BM - 1) / BM;
  const int head = blockIdx.x / num_m;
  const int mb = blockIdx.x - head * num_m;
  const int b = head / Hq, hq = head - b * Hq;
  const int hkv = hq / (Hq / Hkv);
  const int tid = threadIdx.x, part = tid & 3;
  const int m0 = mb * BM, row = m0 + (tid >> 2);
  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const float* Kh = K + ((size_t)b * N * Hkv + hkv) * D;
  const float* Vh = V + ((size_t)b * N * Hkv + hkv) * D;

  float q[DP], acc[DP];
  const float* qr = Q + ((size_t)b * N + row) * qs + (size_t)hq * D + part * DP;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    q[e] = row < N ? qr[e] : 0.f;
    acc[e] = 0.f;
  }
  int kv_lo = 0, kv_hi = N;
  if (causal) kv_hi = min(N, m0 + BM);
  if (window > 0) kv_lo = max(0, m0 - window + 1);
  float m_i = -INFINITY, l_i = 0.f;

  for (int n0 = (kv_lo / BN) * BN; n0 < kv_hi; n0 += BN) {
    __syncthreads();
    for (int i = tid; i < BN * D / 4; i += 256) {
      const int key = (4 * i) / D, dd = 4 * i - key * D;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (n0 + key < N) {
        kv = *reinterpret_cast<const float4*>(Kh + (size_t)(n0 + key) * ks + dd);
        vv = *reinterpret_cast<const float4*>(Vh + (size_t)(n0 + key) * ks + dd);
      }
      *reinterpret_cast<float4*>(sK + key * D + dd) = kv;
      *reinterpret_cast<float4*>(sV + key * D + dd) = vv;
    }
    __syncthreads();
    float t[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float part_dot = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) part_dot = fmaf(q[e], sK[j * D + part * DP + e], part_dot);
      part_dot += __shfl_xor(part_dot, 1, 64);
      part_dot += __shfl_xor(part_dot, 2, 64);
      const int key = n0 + j;
      const bool ok = key < N && (!causal || key <= row) && (window <= 0 || key >= row - window + 1);
      t[j] = ok ? part_dot * c : -INFINITY;
      mx = fmaxf(mx, t[j]);
    }
    const float m_new = fmaxf(m_i, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_i - m_use);
    l_i *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = (t[j] == -INFINITY) ? 0.f : exp2f(t[j] - m_use);
      l_i += pj;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc[e] = fmaf(pj, sV[j * D + part * DP + e], acc[e]);
    }
    m_i = m_new;
  }
  if (row < N) {
    const float inv = l_i > 0.f ? 1.f / l_i : 0.f;
    float* orow = O + ((size_t)b * N + row) * qs + (size_t)hq * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) orow[e] = acc[e] * inv;
    if (part == 0)
      LSE[((size_t)b * Hq + hq) * N + row] = l_i > 0.f ? (m_i + log2f(l_i)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------
template <int D>
static hipError_t launch_fwd_bf16_d(const FwdArgs& a, hipStream_t st) {
  using Cfg = FwdCfg<D>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int num_m = (a.N + Cfg::BM - 1) / Cfg::BM;
  const int grid = a.B * a.Hq * num_m;
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(grid), dim3(256), Cfg::LDS_BYTES, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window, a.c_log2, a.neg_q);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_fwd_bf16_d<64>(a, st);
    case 128: return launch_fwd_bf16_d<128>(a, st);
    case 256: return launch_fwd_bf16_d<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t launch_fwd_fp32_d(const FwdArgs& a, hipStream_t st) {
  using Cfg = Fp32Cfg<D>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_fp32_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int num_m = (a.N + Cfg::BM - 1) / Cfg::BM;
  const int grid = a.B * a.Hq * num_m;
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3(grid), dim3(256), Cfg::LDS_BYTES, st,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.B, a.Hq, a.Hkv, a.N, a.causal, a.window, a.c_log2_signed);
  return hipGetLastError();
}

hipError_t launch_fwd_fp32(const FwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_fwd_fp32_d<64>(a, st);
    case 128: return launch_fwd_fp32_d<128>(a, st);
    case 256: return launch_fwd_fp32_d<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
