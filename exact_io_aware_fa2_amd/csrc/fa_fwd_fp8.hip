// fa_fwd_fp8.hip -- forward attention with 8-bit E4M3 inputs for gfx950.
//
// The pages name an FP8 forward pass as part of a later version of the method (ainews.cool,
// "flash-attention transformer optimization", opening overview; hysenlabs.com, "dao-ailab
// flash-attention", hardware-boundary section) without fixing a format or scaling; here Q,
// K and V are OCP E4M3 codes with one positive float32 dequantisation factor each, and the
// target is the exact attention of the dequantised inputs (the tiling and online softmax of
// fa_fwd.hip, with both products on the double-rate 8-bit matrix core).
//
// One workgroup = 8 waves = 256 query rows (d <= 128; 4 waves = 128 rows for d = 256) of one
// (batch entry, query head); 32 rows per wave:
//   * S^T = K Q^T with v_mfma_f32_32x32x64_f8f6f4: a lane holds one query row; the 32 bytes
//     a lane feeds per product are 32 consecutive head-dim elements (Q in VGPRs, K rows from
//     LDS), the same slots in both operands;
//   * a 64-key tile is two 32-key score pieces, 32 scores per lane; their weights, rounded
//     to E4M3 (round to nearest even), are the 32-byte B operand of O^T += V^T P^T, so one
//     product covers the whole tile.  V is stored transposed in LDS with its keys permuted
//     (vt8_pos) into the order in which the weights sit in the lane, so every V^T operand is
//     two 16-byte LDS reads;
//   * weights are taken against a lazy reference maximum, as in the bf16 kernel, with limits
//     that keep every weight at or below 256 (E4M3 reaches 448): a lane's 32 weights may sum
//     to at most 2^8 before the row max is taken, and the reference moves when the maximum
//     exceeds it by more than 2^3;
//   * O is normalised by the sum of the unrounded weights, which also gives the logsumexp;
//     the value factor is applied once in the epilogue.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32v16 __attribute__((ext_vector_type(16)));

template <int D>
struct Fp8Cfg {
  static constexpr int NW = D <= 128 ? 8 : 4;  // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;           // query rows per workgroup
  static constexpr int BN = 64;                // keys per staged tile = one product's K
  static constexpr int KSTR = D + 16;          // K row stride in bytes (16-byte pad)
  static constexpr int VSTR = BN + 16;         // V^T row stride in bytes (16-byte pad)
  static constexpr int K_BYTES = BN * KSTR;
  static constexpr int V_BYTES = D * VSTR;
  static constexpr int BUF = K_BYTES + V_BYTES;
  static constexpr int LDS_BYTES = 2 * BUF;    // double buffered
};

constexpr float kFp8Threshold = 3.f;   // move the reference when the max exceeds it by 2^3
constexpr float kFp8SumLimit = 256.f;  // a lane's 32 weights summing above this take the max

// 32 x 32 x 64 product of E4M3 operands (scale operands 0: the unscaled instruction).
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  const f32v16 r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      a, b, __builtin_bit_cast(f32v16, c), 0, 0, 0, 0, 0, 0);
  return __builtin_bit_cast(f32x16, r);
}

__device__ __forceinline__ i32x8 join8(const uint4& lo, const uint4& hi) {
  i32x8 r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ i32x8 lds_read_32(const uint8_t* p) {
  return join8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 16));
}

// Byte position of key k (0..63 inside a tile) in a V^T row.  Score element r of piece pc
// in the lane half hh belongs to key 32 pc + 8 (r / 4) + 4 hh + r % 4 and becomes byte
// 16 pc + r of that half's weight operand, so the key goes to byte 32 hh + 16 pc + r.
__device__ __forceinline__ int vt8_pos(int k) {
  const int pc = k >> 5, kk = k & 31;
  return 32 * ((kk >> 2) & 1) + 16 * pc + 4 * (kk >> 3) + (kk & 3);
}

template <int D>
__global__ __launch_bounds__(Fp8Cfg<D>::NT, 1) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int N,
    int causal, int window, float c, int neg_q, float o_scale) {
  using Cfg = Fp8Cfg<D>;
  constexpr int NT = Cfg::NT, BM = Cfg::BM, BN = Cfg::BN, KSTR = Cfg::KSTR, VSTR = Cfg::VSTR;
  constexpr int NCQ = D / 64;  // products of S^T per 32-key piece
  constexpr int ND = D / 32;   // 32-row head-dim tiles of O^T
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);

  const int num_m = (N + BM - 1) / BM;
  int b, hq, rank;
  work_item(B, Hq, num_m, b, hq, rank);
  const int mb = num_m - 1 - rank;  // causal: the last row block attends the most keys
  const int hkv = hq / (Hq / Hkv);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int m0 = mb * BM;
  const int wr0 = m0 + w * 32;
  const int row = wr0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;  // row strides in bytes
  const uint8_t* Qh = Q + ((size_t)b * N * Hq + hq) * D;
  const uint8_t* Kh = K + ((size_t)b * N * Hkv + hkv) * D;
  const uint8_t* Vh = V + ((size_t)b * N * Hkv + hkv) * D;

  // Q^T operand: lane holds Q[row][64 cc + 32 hh .. + 31] for every product cc.
  i32x8 qop[NCQ];
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (row < N) {
      const uint8_t* qr = Qh + (size_t)row * qs + 64 * cc + 32 * hh;
      lo = gload16(qr);
      hi = gload16(qr + 16);
    }
    if (neg_q) {  // exact negation: flip every sign bit
      lo.x ^= 0x80808080u; lo.y ^= 0x80808080u; lo.z ^= 0x80808080u; lo.w ^= 0x80808080u;
      hi.x ^= 0x80808080u; hi.y ^= 0x80808080u; hi.z ^= 0x80808080u; hi.w ^= 0x80808080u;
    }
    qop[cc] = join8(lo, hi);
  }

  // Key range any row of this workgroup may attend.
  int kv_lo = 0, kv_hi = N;
  if (causal) kv_hi = min(N, m0 + BM);
  if (window > 0) kv_lo = max(0, m0 - window + 1);
  const int nb_lo = kv_lo / BN, nb_hi = (kv_hi + BN - 1) / BN;

  // Staging.  K: 16-byte row chunks.  V: tasks of 4 keys x 4 head-dim bytes, transposed in
  // registers (two rounds of v_perm_b32) into 4 V^T rows of 4 keys each; a wave's 16 lanes
  // of one head-dim chunk cover the 16 key groups of a V^T row, so the 4-byte LDS stores
  // of a wave fall on distinct banks.  Buffer resources end at row N (zero fill).
  constexpr int CPR = D / 16;  // 16-byte chunks per K row
  constexpr int KCH = BN * CPR;
  constexpr int PTK = (KCH + NT - 1) / NT;
  constexpr int VTASKS = (BN / 4) * (D / 4);
  constexpr int PTV = (VTASKS + NT - 1) / NT;
  uint4 kr[PTK];
  uint32_t vr[PTV][4];
  const uint32_t row_bytes = (uint32_t)ks;
  auto gload = [&](int nb) {
    const int n0 = nb * BN;
    const uint32_t bytes = (uint32_t)(N - n0) * row_bytes;
    const rsrc_t kres = make_rsrc(Kh + (size_t)n0 * ks, bytes);
    const rsrc_t vres = make_rsrc(Vh + (size_t)n0 * ks, bytes);
#pragma unroll
    for (int i = 0; i < PTK; ++i) {
      const int ch = tid + NT * i;
      if (KCH % NT == 0 || ch < KCH) {
        const int key = ch / CPR, dc = ch - key * CPR;
        kr[i] = bload16(kres, (uint32_t)key * row_bytes + 16u * dc);
      }
    }
#pragma unroll
    for (int p = 0; p < PTV; ++p) {
      const int t = tid + NT * p;
      if (VTASKS % NT == 0 || t < VTASKS) {
        const int g = t & 15, dch = t >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vr[p][e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
              vres, (int)((uint32_t)(4 * g + e) * row_bytes + 4u * dch), 0, 0);
      }
    }
  };
  auto swrite = [&](int buf) {
    uint8_t* sK = lds + buf * Cfg::BUF;
    uint8_t* sV = sK + Cfg::K_BYTES;
#pragma unroll
    for (int i = 0; i < PTK; ++i) {
      const int ch = tid + NT * i;
      if (KCH % NT == 0 || ch < KCH) {
        const int key = ch / CPR, dc = ch - key * CPR;
        *reinterpret_cast<uint4*>(sK + key * KSTR + 16 * dc) = kr[i];
      }
    }
#pragma unroll
    for (int p = 0; p < PTV; ++p) {
      const int t = tid + NT * p;
      if (VTASKS % NT == 0 || t < VTASKS) {
        const int g = t & 15, dch = t >> 4;
        // vr[e] = head-dim bytes 4 dch .. +3 of key 4 g + e
        const uint32_t lo01 = __builtin_amdgcn_perm(vr[p][1], vr[p][0], 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vr[p][1], vr[p][0], 0x07030602u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vr[p][3], vr[p][2], 0x05010400u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vr[p][3], vr[p][2], 0x07030602u);
        uint8_t* dst = sV + (4 * dch) * VSTR + vt8_pos(4 * g);
        *reinterpret_cast<uint32_t*>(dst) = pack_lo(lo01, lo23);
        *reinterpret_cast<uint32_t*>(dst + VSTR) = pack_hi(lo01, lo23);
        *reinterpret_cast<uint32_t*>(dst + 2 * VSTR) = pack_lo(hi01, hi23);
        *reinterpret_cast<uint32_t*>(dst + 3 * VSTR) = pack_hi(hi01, hi23);
      }
    }
  };

  // Running state of this lane's row: reference max m (log2 units) and this lane half's
  // sum of the unrounded weights.
  float m_i = -INFINITY, le_i = 0.f;
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  const int klo = window > 0 ? row - window + 1 : 0;  // allowed keys of this row: [klo, khi]
  const int khi = causal ? min(row, N - 1) : N - 1;

  if (nb_lo < nb_hi) {
    gload(nb_lo);
    swrite(0);
    if (nb_lo + 1 < nb_hi) gload(nb_lo + 1);
  }
  __syncthreads();
  for (int nb = nb_lo; nb < nb_hi; ++nb) {
    const int buf = (nb - nb_lo) & 1;
    const uint8_t* sK = lds + buf * Cfg::BUF;
    const uint8_t* sV = sK + Cfg::K_BYTES;
    const int n0 = nb * BN;
    const bool active = wr0 < N && (!causal || n0 <= wr0 + 31) &&
                        (window <= 0 || n0 + BN - 1 >= wr0 - window + 1);
    if (active) {
      // S^T pieces: keys n0 + 32 pc + [0, 32) x this wave's 32 rows.
      // Up to d = 128 every K operand of the tile is read before its products and the
      // V^T operands right after them, so LDS latency hides behind the products and the
      // softmax; at d = 256 those registers would spill, and each piece reads its own.
      constexpr bool kAhead = D <= 128;
      f32x16 sp[2];
      i32x8 kop[kAhead ? 2 : 1][NCQ];
      i32x8 vop[kAhead ? ND : 1];
      auto read_k = [&](int pc, i32x8 (&dst)[NCQ]) {
        const uint8_t* kp = sK + (32 * pc + l32) * KSTR + 32 * hh;
#pragma unroll
        for (int cc = 0; cc < NCQ; ++cc) dst[cc] = lds_read_32(kp + 64 * cc);
      };
      const uint8_t* vp = sV + l32 * VSTR + 32 * hh;
      if constexpr (kAhead) {
        read_k(0, kop[0]);
        read_k(1, kop[1]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        if constexpr (!kAhead) read_k(pc, kop[0]);
        f32x16 s = zero16();
#pragma unroll
        for (int cc = 0; cc < NCQ; ++cc) s = mfma_f8(kop[kAhead ? pc : 0][cc], qop[cc], s);
        sp[pc] = s;
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (kAhead) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vop[dt] = lds_read_32(vp + 32 * dt * VSTR);
      }
      float s[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = sp[0][r];
        s[16 + r] = sp[1][r];
      }
      // Masks (wave-uniform branch; masked scores become -inf, weight 0).
      const bool need_mask = (n0 + BN > N) | ((causal != 0) & (n0 + BN - 1 > wr0)) |
                             ((window > 0) & (n0 < wr0 + 32 - window));
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int r = i & 15, pc = i >> 4;
          const int key = n0 + 32 * pc + 4 * hh + 8 * (r >> 2) + (r & 3);
          s[i] = ((key >= klo) & (key <= khi)) ? s[i] : -INFINITY;
        }
      }
      auto tree_sum32 = [](const float (&x)[32]) {
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = q[2 * i] + q[2 * i + 1];
        return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
      };
      float e[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = fast_exp2(fmaf(s[i], c, -m_i));  // 0 if masked
      float rse = tree_sum32(e);
      if (__any(!(rse <= kFp8SumLimit))) {  // wave-uniform; rare after a row's first tile
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int i = 2; i < 32; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
        mx = half_max(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
        const bool grow = mt > m_i + kFp8Threshold;
        const float alpha = grow ? fast_exp2(m_i - mt) : 1.f;  // 0 when m_i was -inf
        le_i *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        m_i = grow ? mt : m_i;
        const float m_use = (m_i == -INFINITY) ? 0.f : m_i;
#pragma unroll
        for (int i = 0; i < 32; ++i) e[i] = fast_exp2(fmaf(s[i], c, -m_use));
        rse = tree_sum32(e);
      }
      le_i += rse;
      // Weights -> E4M3, byte 16 pc + r of the operand = element r of piece pc.
      i32x8 pk;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int i0 = 4 * g;
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[i0], e[i0 + 1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(e[i0 + 2], e[i0 + 3], wd, true);
        pk[g] = wd;
      }
      // O^T += V^T P^T over the whole 64-key tile.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        acc[dt] = mfma_f8(kAhead ? vop[dt] : lds_read_32(vp + 32 * dt * VSTR), pk, acc[dt]);
      __builtin_amdgcn_s_setprio(0);
    }
    if (nb + 1 < nb_hi) {
      swrite(buf ^ 1);
      if (nb + 2 < nb_hi) gload(nb + 2);
    }
    __syncthreads();
  }

  // Epilogue: O = o_scale * acc / l (one rounding to bf16), LSE = (m + log2 l) * ln 2.
  const float le = half_sum(le_i);
  if (row < N) {
    const float inv = le > 0.f ? o_scale / le : 0.f;
    bf16_t* orow = O + ((size_t)b * N + row) * Hq * D + (size_t)hq * D;
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
      LSE[((size_t)b * Hq + hq) * N + row] = le > 0.f ? (m_i + __log2f(le)) * kLn2 : -INFINITY;
  }
}

template <int D>
static hipError_t launch_fwd_fp8_d(const FwdArgs& a, hipStream_t st) {
  using Cfg = Fp8Cfg<D>;
  // Dynamic LDS limit, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = hipFuncSetAttribute((const void*)fwd_fp8_kernel<D>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int num_m = (a.N + Cfg::BM - 1) / Cfg::BM;
  hipLaunchKernelGGL(fwd_fp8_kernel<D>, dim3(a.B * a.Hq * num_m), dim3(Cfg::NT), Cfg::LDS_BYTES,
                     st, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v,
                     (bf16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window, a.c_log2,
                     a.neg_q, a.o_scale);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_fwd_fp8_d<64>(a, st);
    case 128: return launch_fwd_fp8_d<128>(a, st);
    case 256: return launch_fwd_fp8_d<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
