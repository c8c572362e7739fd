// fa_bwd.hip -- backward attention kernels for gfx950.
//
// The backward recomputes the probability matrix block by block from Q, K and the
// stored logsumexp instead of reading a stored N x N matrix (ainews.cool, "flash-attention
// transformer optimization", technical deep dive, item 2).  With L = sum(O * dO):
//   D_i   = sum_c dO_ic O_ic                       (preprocess kernel)
//   P_ij  = exp(s_ij - LSE_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
//
// Main kernel: one workgroup = 4 waves = 128 keys of one (batch, KV head) (32 keys per
// wave), optionally one half of the head dim for the accumulated outputs when d = 256.
//   * the wave's K and V rows sit in VGPRs as the B operands of S = Q K^T and dP = dO V^T;
//     every lane holds one key and 16 rows per 32 x 32 tile;
//   * Q, dO (64 rows), their LSE and D go through LDS; the next block's rows are loaded
//     into registers while the current block computes;
//   * P and dS (accumulator layout) feed dV^T += dO^T P and dK^T += Q^T dS directly as B
//     operands; dO^T and Q^T come from LDS with the transposing ds_read_b64_tr_b16;
//   * dK/dV accumulate in registers across every query head of the GQA group and every
//     query block, then are written once (no atomics on dK/dV);
//   * dS^T is shared through LDS and each wave forms a slice of dQ = dS K over all 128
//     keys, added into a float32 accumulator with hardware float atomics (lanes run along
//     the head dim, so each atomic instruction touches two 128-byte lines); a last kernel
//     scales and rounds the accumulator to bf16.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int D>
struct BwdCfg {
  static constexpr int BKN = 128;                // keys per workgroup
  static constexpr int BQ = 64;                  // query rows per inner step
  static constexpr int DH = D <= 128 ? D : 128;  // head-dim slice of dK/dV/dQ per workgroup
  static constexpr int NSPLIT = D / DH;
  static constexpr int STR = D + 8;              // sQ / sdO row stride (elements)
  static constexpr int KSTR = DH + 8;            // sK row stride
  static constexpr int SSTR = BQ + 8;            // sdS row stride, [key][row] layout
  static constexpr bool PREFETCH = D <= 128;     // register budget allows prefetching
  static constexpr int SK_BYTES = BKN * KSTR * 2;
  static constexpr int SQ_BYTES = BQ * STR * 2;
  static constexpr int SS_BYTES = BKN * SSTR * 2;
  static constexpr int LDS_BYTES = SK_BYTES + 2 * SQ_BYTES + SS_BYTES + 2 * BQ * 4;
};

__device__ __forceinline__ bool allowed(int row, int key, int N, int causal, int window) {
  return key < N && (!causal || key <= row) && (window <= 0 || key >= row - window + 1);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// D = rowsum(dO * O) in float32 from the stored bf16 O, and clears the dQ accumulator.
// D/8 threads per (batch, row, head) row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_t* __restrict__ O,
                                                      const bf16_t* __restrict__ dO,
                                                      float* __restrict__ Dv,
                                                      float* __restrict__ dq_acc, int B,
                                                      int Hq, int N) {
  constexpr int T = D / 8, RPB = 256 / T;
  const long total = (long)B * N * Hq;
  const long r = (long)blockIdx.x * RPB + threadIdx.x / T;
  const int t = threadIdx.x % T;
  float sum = 0.f;
  if (r < total) {
    const uint4 o = gload16(O + r * D + t * 8);
    const uint4 g = gload16(dO + r * D + t * 8);
    sum = bf_lo(o.x) * bf_lo(g.x) + bf_hi(o.x) * bf_hi(g.x);
    sum += bf_lo(o.y) * bf_lo(g.y) + bf_hi(o.y) * bf_hi(g.y);
    sum += bf_lo(o.z) * bf_lo(g.z) + bf_hi(o.z) * bf_hi(g.z);
    sum += bf_lo(o.w) * bf_lo(g.w) + bf_hi(o.w) * bf_hi(g.w);
    float4* z = reinterpret_cast<float4*>(dq_acc + r * D + t * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = T / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (t == 0 && r < total) {
    const int hq = (int)(r % Hq);
    const long bn = r / Hq;
    const int n = (int)(bn % N), b = (int)(bn / N);
    Dv[((long)b * Hq + hq) * N + n] = sum;
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int B,
    int Hq, int Hkv, int N, int causal, int window, float c, float scale) {
  using Cfg = BwdCfg<D>;
  constexpr int BKN = Cfg::BKN, BQ = Cfg::BQ, DH = Cfg::DH, NSPLIT = Cfg::NSPLIT;
  constexpr int STR = Cfg::STR, KSTR = Cfg::KSTR, SSTR = Cfg::SSTR;
  constexpr bool PREFETCH = Cfg::PREFETCH;
  constexpr int NC = D / 16;     // k-steps of S and dP over the head dim
  constexpr int NDH = DH / 32;   // owned 32-wide head-dim tiles of dK^T / dV^T / dQ
  constexpr int TPW = DH / 64;   // dQ tiles per wave (NDH d-tiles x 2 row tiles / 4 waves)
  static_assert(TPW >= 1, "head dim slice too small");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Cfg::SK_BYTES);
  bf16_t* sdO = reinterpret_cast<bf16_t*>(smem + Cfg::SK_BYTES + Cfg::SQ_BYTES);
  bf16_t* sdS = reinterpret_cast<bf16_t*>(smem + Cfg::SK_BYTES + 2 * Cfg::SQ_BYTES);
  float* sL = reinterpret_cast<float*>(smem + Cfg::SK_BYTES + 2 * Cfg::SQ_BYTES + Cfg::SS_BYTES);
  float* sD = sL + BQ;

  const int num_kb = (N + BKN - 1) / BKN;
  const int total = B * Hkv * num_kb * NSPLIT;
  const int lin = xcd_remap(blockIdx.x, total);
  const int split = lin % NSPLIT;
  const int t1 = lin / NSPLIT;
  const int head = t1 / num_kb;
  const int kbo = t1 - head * num_kb;
  // longest first: causal -> low key blocks see the most rows; a pure left window -> high.
  const int kb = (!causal && window > 0) ? num_kb - 1 - kbo : kbo;
  const int b = head / Hkv, hkv = head - b * Hkv;
  const int G = Hq / Hkv;
  const int dh0 = split * DH;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;
  const int n0 = kb * BKN, kw0 = n0 + 32 * w, key = kw0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Kb = K + ((size_t)b * N * Hkv + hkv) * D;
  const bf16_t* Vb = V + ((size_t)b * N * Hkv + hkv) * D;

  // B operands K^T and V^T of this lane's key.
  bf16x8 kop[NC], vop[NC];
  if (key < N) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      kop[cc] = __builtin_bit_cast(bf16x8, gload16(Kb + (size_t)key * ks + 16 * cc + 8 * hh));
      vop[cc] = __builtin_bit_cast(bf16x8, gload16(Vb + (size_t)key * ks + 16 * cc + 8 * hh));
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      kop[cc] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      vop[cc] = kop[cc];
    }
  }
  // K slice [n0, n0 + 128) x [dh0, dh0 + DH) in LDS for the dQ product.
  for (int ch = tid; ch < BKN * DH / 8; ch += 256) {
    const int kl = ch / (DH / 8), dc = ch - kl * (DH / 8);
    const int n = n0 + kl;
    const uint4 val = n < N ? gload16(Kb + (size_t)n * ks + dh0 + dc * 8) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(sK + kl * KSTR + dc * 8) = val;
  }

  const int qb_lo = causal ? n0 / BQ : 0;
  const int row_end = window > 0 ? min(N, n0 + BKN + window - 1) : N;
  const int qb_hi = (row_end + BQ - 1) / BQ;
  const int nq = max(0, qb_hi - qb_lo);
  const int total_it = G * nq;

  f32x16 dk[NDH], dv[NDH];
#pragma unroll
  for (int i = 0; i < NDH; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  constexpr int QCPR = D / 8;           // 16-byte chunks per Q row
  constexpr int QPT = BQ * QCPR / 256;  // chunks per thread
  uint4 qreg[QPT], oreg[QPT];
  float lreg = 0.f, dreg = 0.f;
  auto load_regs = [&](int it) {
    const int g = it / nq, qb = qb_lo + (it - g * nq);
    const int hq = hkv * G + g, r0 = qb * BQ;
    const bf16_t* Qb = Q + ((size_t)b * N * Hq + hq) * D;
    const bf16_t* Ob = dO + ((size_t)b * N * Hq + hq) * D;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int ch = tid + 256 * i, rr = ch / QCPR, dc = ch - rr * QCPR;
      const int n = r0 + rr;
      if (n < N) {
        qreg[i] = gload16(Qb + (size_t)n * qs + dc * 8);
        oreg[i] = gload16(Ob + (size_t)n * qs + dc * 8);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        oreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BQ) {
      const int n = r0 + tid;
      const size_t li = ((size_t)b * Hq + hq) * N + n;
      lreg = n < N ? LSE[li] * kLog2e : INFINITY;  // +inf -> P = 0 on padding rows
      dreg = n < N ? Dv[li] : 0.f;
    }
  };
  auto store_regs = [&]() {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int ch = tid + 256 * i, rr = ch / QCPR, dc = ch - rr * QCPR;
      *reinterpret_cast<uint4*>(sQ + rr * STR + dc * 8) = qreg[i];
      *reinterpret_cast<uint4*>(sdO + rr * STR + dc * 8) = oreg[i];
    }
    if (tid < BQ) {
      sL[tid] = lreg;
      sD[tid] = dreg;
    }
  };

  if (PREFETCH && total_it > 0) load_regs(0);
  for (int it = 0; it < total_it; ++it) {
    const int g = it / nq, qb = qb_lo + (it - g * nq);
    const int hq = hkv * G + g, r0 = qb * BQ;
    __syncthreads();
    if (!PREFETCH) load_regs(it);
    store_regs();
    __syncthreads();
    if (PREFETCH && it + 1 < total_it) load_regs(it + 1);

    const bool active = kw0 < N && (!causal || r0 + BQ - 1 >= kw0) &&
                        (window <= 0 || r0 <= kw0 + 31 + window - 1);
    bf16_t* sdS_lane = sdS + (32 * w + l32) * SSTR + 4 * hh;
    if (active) {
      const bool need_mask = (kw0 + 32 > N) || (causal && kw0 + 31 > r0) ||
                             (window > 0 && kw0 < r0 + BQ - window);
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt] = zero16();
        dp[mt] = zero16();
        const bf16_t* qa = sQ + (32 * mt + l32) * STR + 8 * hh;
        const bf16_t* oa = sdO + (32 * mt + l32) * STR + 8 * hh;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          s[mt] = mfma32(lds_read_b128(qa + 16 * cc), kop[cc], s[mt]);
          dp[mt] = mfma32(lds_read_b128(oa + 16 * cc), vop[cc], dp[mt]);
        }
      }
      bf16x8 pP[2][2], pS[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int rl0 = 32 * mt + 8 * g4 + 4 * hh;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(sL + rl0);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(sD + rl0);
          float pv[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float pe = fast_exp2(fmaf(s[mt][r], c, -L4[e]));
            if (need_mask && !allowed(r0 + rl0 + e, key, N, causal, window)) pe = 0.f;
            pv[e] = pe;
            dsv[e] = pe * (dp[mt][r] - D4[e]);
          }
          const bf16x2 p01 = to_bf16x2(pv[0], pv[1]), p23 = to_bf16x2(pv[2], pv[3]);
          const bf16x2 d01 = to_bf16x2(dsv[0], dsv[1]), d23 = to_bf16x2(dsv[2], dsv[3]);
          const int c2 = g4 >> 1, i0 = 4 * (g4 & 1);
          pP[mt][c2][i0] = p01[0];
          pP[mt][c2][i0 + 1] = p01[1];
          pP[mt][c2][i0 + 2] = p23[0];
          pP[mt][c2][i0 + 3] = p23[1];
          pS[mt][c2][i0] = d01[0];
          pS[mt][c2][i0 + 1] = d01[1];
          pS[mt][c2][i0 + 2] = d23[0];
          pS[mt][c2][i0 + 3] = d23[1];
          uint2 u;
          u.x = __builtin_bit_cast(uint32_t, d01);
          u.y = __builtin_bit_cast(uint32_t, d23);
          *reinterpret_cast<uint2*>(sdS_lane + 32 * mt + 8 * g4) = u;
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the owned head-dim slice.
      const int tr_off = (hh * 4 + (j16 >> 2)) * STR + dh0 + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
      for (int dt = 0; dt < NDH; ++dt) {
#pragma unroll
        for (int kstep = 0; kstep < BQ / 16; ++kstep) {
          const int off = tr_off + 16 * kstep * STR + 32 * dt;
          const bf16x8 ao = lds_read_tr_x2(sdO + off, sdO + off + 8 * STR);
          dv[dt] = mfma32(ao, pP[kstep >> 1][kstep & 1], dv[dt]);
          const bf16x8 aq = lds_read_tr_x2(sQ + off, sQ + off + 8 * STR);
          dk[dt] = mfma32(aq, pS[kstep >> 1][kstep & 1], dk[dt]);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint2*>(sdS_lane + 32 * mt + 8 * g4) = make_uint2(0, 0);
    }
    __syncthreads();

    // dQ[rows][d] (slice) = dS[rows][128 keys] K[128 keys][d]; lanes run along d.
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = w * TPW + u, dt = tile % NDH, rt = tile / NDH;
      f32x16 a = zero16();
#pragma unroll
      for (int kstep = 0; kstep < BKN / 16; ++kstep) {
        const int key0 = 16 * kstep + 8 * hh + (j16 >> 2);
        const bf16_t* sp = sdS + key0 * SSTR + 32 * rt + 16 * (grp & 1) + 4 * (j16 & 3);
        const bf16_t* kp = sK + key0 * KSTR + 32 * dt + 16 * (grp & 1) + 4 * (j16 & 3);
        const bf16x8 as = lds_read_tr_x2(sp, sp + 4 * SSTR);
        const bf16x8 bk = lds_read_tr_x2(kp, kp + 4 * KSTR);
        a = mfma32(as, bk, a);
      }
      float* dqb = dq_acc + ((size_t)b * N * Hq + hq) * D + dh0 + 32 * dt + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = r0 + 32 * rt + (r >> 2) * 8 + hh * 4 + (r & 3);
        if (n < N) unsafeAtomicAdd(dqb + (size_t)n * qs, a[r]);
      }
    }
  }

  if (key < N) {
    bf16_t* dkr = dK + ((size_t)b * N + key) * ks + (size_t)hkv * D + dh0;
    bf16_t* dvr = dV + ((size_t)b * N + key) * ks + (size_t)hkv * D + dh0;
#pragma unroll
    for (int dt = 0; dt < NDH; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hh;
        uint2 u;
        u.x = __builtin_bit_cast(uint32_t, to_bf16x2(dk[dt][4 * g4] * scale, dk[dt][4 * g4 + 1] * scale));
        u.y = __builtin_bit_cast(uint32_t, to_bf16x2(dk[dt][4 * g4 + 2] * scale, dk[dt][4 * g4 + 3] * scale));
        *reinterpret_cast<uint2*>(dkr + d) = u;
        u.x = __builtin_bit_cast(uint32_t, to_bf16x2(dv[dt][4 * g4], dv[dt][4 * g4 + 1]));
        u.y = __builtin_bit_cast(uint32_t, to_bf16x2(dv[dt][4 * g4 + 2], dv[dt][4 * g4 + 3]));
        *reinterpret_cast<uint2*>(dvr + d) = u;
      }
    }
  }
}

// dQ = scale * accumulator, rounded once to bf16.  8 elements per thread.
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         bf16_t* __restrict__ dq, long n8,
                                                         float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 bq = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, to_bf16x2(a.x * scale, a.y * scale));
  u.y = __builtin_bit_cast(uint32_t, to_bf16x2(a.z * scale, a.w * scale));
  u.z = __builtin_bit_cast(uint32_t, to_bf16x2(bq.x * scale, bq.y * scale));
  u.w = __builtin_bit_cast(uint32_t, to_bf16x2(bq.z * scale, bq.w * scale));
  reinterpret_cast<uint4*>(dq)[i] = u;
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  using Cfg = BwdCfg<D>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Cfg::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const long rows = (long)a.B * a.N * a.Hq;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     st, (const bf16_t*)a.o, (const bf16_t*)a.dO, a.dvec, a.dq_acc, a.B, a.Hq,
                     a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int num_kb = (a.N + Cfg::BKN - 1) / Cfg::BKN;
  const int grid = a.B * a.Hkv * num_kb * Cfg::NSPLIT;
  if (a.ev_start) {
    e = hipEventRecord(a.ev_start, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_bf16_kernel<D>, dim3(grid), dim3(256), Cfg::LDS_BYTES, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
                     (const bf16_t*)a.dO, a.lse, a.dvec, a.dq_acc, (bf16_t*)a.dk,
                     (bf16_t*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window,
                     a.c_log2_signed, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_stop) {
    e = hipEventRecord(a.ev_stop, st);
    if (e != hipSuccess) return e;
  }
  const long n8 = rows * D / 8;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     a.dq_acc, (bf16_t*)a.dq, n8, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_bwd_d<64>(a, st);
    case 128: return launch_bwd_d<128>(a, st);
    case 256: return launch_bwd_d<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
