// fa_decode.hip -- attention of the newest queries over a KV cache, split over the keys.
//
// At inference the method runs over large context caches (bmjup.com, "FlashAttention-2 ...
// 实战解析", FAQ on inference).  There a step has few queries per sequence and many keys,
// so one workgroup per (sequence, head) cannot fill the chip and the cost is reading the
// cache once.  The keys of each sequence are split into chunks handled by separate
// workgroups; each writes its chunk's normalised partial output and logsumexp, and a merge
// kernel combines them exactly: LSE = ln sum_s e^LSE_s, O = sum_s e^(LSE_s - LSE) O_s (the
// running maximum / normaliser combination of the online softmax, applied across chunks).
//
// decode_kernel: one workgroup = 4 waves for (sequence b, KV head, group of up to 32 query
// rows, key chunk).  The query rows are the Hq/Hkv heads of the KV head times the Nq new
// tokens, so every K/V byte of the cache is read once per KV head.  Wave w takes the
// chunk's 32-key tiles w, w + 4, ...; per tile:
//   * S^T = K Q^T on 32x32x16 bf16 products: the K rows come straight from global memory
//     as the A operand (16-byte buffer loads ending at the chunk's end), one query row per
//     lane as in the forward;
//   * online softmax (row max, rescale, weights), P^T in bf16 as the B operand;
//   * O^T += V^T P^T with the V tile staged row-major in the wave's own LDS area and read
//     transposed (ds_read_b64_tr_b16): the kernel is bound by reading the cache, and this
//     read rate is far above what that needs;
//   * the next tile's K and V loads are in flight during the current tile's math.
// The four waves' states are combined through LDS at the end.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int D>
struct DecCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int TK = 32;                 // keys per wave tile
  static constexpr int STR = D + 8;             // V tile row stride (elements)
  static constexpr int ND = D / 32;
  static constexpr int NC = D / 16;
  static constexpr int VB = TK * STR * 2;       // V tile bytes per wave
  static constexpr int ASTR = D + 4;            // merge area row stride (floats)
  static constexpr int MB = NW * 32 * ASTR * 4 + 2 * NW * 32 * 4;  // acc + m, l per wave
  static constexpr int LDS_BYTES = (NW * VB > MB) ? NW * VB : MB;
  static constexpr int VLD = TK * D / 8 / 64;   // 16-byte V loads per lane per tile
};

// Key range [lo, hi) of chunk `split` for a sequence of `len` cached keys, `nq` queries
// at its last positions, window W: the keys any of its queries may attend, split into
// `S` chunks of a whole number of 32-key tiles.
__device__ __forceinline__ void chunk_range(int len, int nq, int window, int S, int split,
                                            int& lo, int& hi) {
  const int a_lo = window > 0 ? max(0, len - nq - window + 1) : 0;
  const int a_hi = len;
  const int span = max(0, a_hi - a_lo);
  const int chunk = (((span + S - 1) / S) + 31) & ~31;
  lo = min(a_hi, a_lo + split * chunk);
  hi = min(a_hi, lo + chunk);
  if (span == 0) lo = hi = 0;
}

template <int D>
__global__ __launch_bounds__(256, 2) void decode_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const int* __restrict__ seqlens, bf16_t* __restrict__ O, float* __restrict__ LSE,
    float* __restrict__ Opart, float* __restrict__ Lpart, int B, int Hq, int Hkv, int Nq,
    int Nk, int causal, int window, float c, int neg_q, int S, int nrg) {
  using Cfg = DecCfg<D>;
  constexpr int NC = Cfg::NC, ND = Cfg::ND, STR = Cfg::STR, ASTR = Cfg::ASTR;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int id = blockIdx.x;
  const int rg = id % nrg;
  id /= nrg;
  const int split = id % S;
  id /= S;
  const int hkv = id % Hkv;
  const int b = id / Hkv;
  const int G = Hq / Hkv, R = G * Nq;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;

  const int len = seqlens ? min(max(seqlens[b], 0), Nk) : Nk;
  int k_lo, k_hi;
  chunk_range(len, Nq, window, S, split, k_lo, k_hi);

  // this lane's query row
  const int r = 32 * rg + l32;
  const bool rvalid = r < R;
  const int gq = rvalid ? r / Nq : 0, qi = rvalid ? r - gq * Nq : 0;
  const int hq = hkv * G + gq;
  const int pos = len - Nq + qi;  // position of the query in its sequence
  const int klo_r = window > 0 ? pos - window + 1 : 0;  // allowed keys: [klo_r, khi_r]
  const int khi_r = min(causal ? pos : len - 1, k_hi - 1);

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  bf16x8 qop[NC];
  {
    const bf16_t* qr = Q + (((size_t)b * Nq + qi) * Hq + hq) * D + 8 * hh;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      uint4 u = rvalid ? gload16(qr + 16 * cc) : make_uint4(0, 0, 0, 0);
      qop[cc] = __builtin_bit_cast(bf16x8, u);
      if (neg_q) qop[cc] = negate8(qop[cc]);
    }
  }
  (void)qs;

  const bf16_t* Kb = Kc + ((size_t)b * Nk * Hkv + hkv) * D;
  const bf16_t* Vb = Vc + ((size_t)b * Nk * Hkv + hkv) * D;
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + w * Cfg::VB);
  const int ntiles = (k_hi - k_lo + 31) / 32;

  uint4 kr[NC], vr[Cfg::VLD];
  auto gload = [&](int t) {  // tile t of the chunk (keys k_lo + 32 t ...)
    const int kb = k_lo + 32 * t;
    const uint32_t bytes = (uint32_t)(k_hi - kb) * (uint32_t)ks * 2u;  // rows past k_hi: 0
    const rsrc_t kres = make_rsrc(Kb + (size_t)kb * ks, bytes);
    const rsrc_t vres = make_rsrc(Vb + (size_t)kb * ks, bytes);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kr[cc] = bload16(kres, ((uint32_t)l32 * (uint32_t)ks + 16u * cc + 8u * hh) * 2u);
#pragma unroll
    for (int u = 0; u < Cfg::VLD; ++u) {
      const int ch = lane + 64 * u, key = ch / (D / 8), dc = ch - key * (D / 8);
      vr[u] = bload16(vres, ((uint32_t)key * (uint32_t)ks + 8u * dc) * 2u);
    }
  };

  float m_i = -INFINITY, l_i = 0.f;
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();

  int t = w;
  if (t < ntiles) gload(t);
  for (; t < ntiles; t += 4) {
    bf16x8 kop[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) kop[cc] = __builtin_bit_cast(bf16x8, kr[cc]);
    // V tile -> this wave's LDS area (row-major); only this wave reads it
#pragma unroll
    for (int u = 0; u < Cfg::VLD; ++u) {
      const int ch = lane + 64 * u, key = ch / (D / 8), dc = ch - key * (D / 8);
      *reinterpret_cast<uint4*>(sV + key * STR + 8 * dc) = vr[u];
    }
    const int kb = k_lo + 32 * t;
    if (t + 4 < ntiles) gload(t + 4);  // next tile in flight during this one's math

    f32x16 s = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) s = mfma32(kop[cc], qop[cc], s);
    const bool need_mask = (kb + 32 > k_hi) || (causal && kb + 31 > len - Nq) ||
                           (window > 0 && kb < len - window);
    if (need_mask) {
      const int kb0 = kb + 4 * hh;  // key of element e: kb0 + 8 (e / 4) + e % 4
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb0 + 8 * (e >> 2) + (e & 3);
        s[e] = ((key >= klo_r) & (key <= khi_r)) ? s[e] : -INFINITY;
      }
    }
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) mx = fmaxf(fmaxf(mx, s[e]), s[e + 1]);
    mx = half_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_i, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_i - m_use);  // 0 when m_i was -inf
    bf16x8 pp[2];
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float e0 = fast_exp2(fmaf(s[e], c, -m_use));
      const float e1 = fast_exp2(fmaf(s[e + 1], c, -m_use));
      rs += e0 + e1;
      const bf16x2 pe = to_bf16x2(e0, e1);
      pp[e >> 3][e & 7] = pe[0];
      pp[e >> 3][(e & 7) + 1] = pe[1];
    }
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
    // the V tile stores of this wave are complete before its lanes read each other's data:
    // wait for LDS only (lgkmcnt 0; the next tile's global loads stay in flight)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const bf16_t* vbase = sV + (hh * 4 + (j16 >> 2)) * STR + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16_t* vp = vbase + (16 * c2) * STR + 32 * dt;
        acc[dt] = mfma32(lds_read_tr_x2(vp, vp + 8 * STR), pp[c2], acc[dt]);
      }
    }
    // the next tile overwrites the area only after these reads have been consumed
  }

  // Combine the four waves: M = max m_w, weights 2^(m_w - M), L = sum_w l_w 2^(m_w - M).
  const float l_row = half_sum(l_i);
  __syncthreads();  // the V areas become the merge area
  float* sAcc = reinterpret_cast<float*>(smem);
  float* sM = sAcc + Cfg::NW * 32 * ASTR;
  float* sL = sM + Cfg::NW * 32;
  if (hh == 0) {
    sM[w * 32 + l32] = m_i;
    sL[w * 32 + l32] = l_row;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < Cfg::NW; ++v) M = fmaxf(M, sM[v * 32 + l32]);
  const float wself = (M == -INFINITY) ? 0.f : fast_exp2(m_i - M);
  {
    float* arow = sAcc + (w * 32 + l32) * ASTR;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v4;
        v4.x = acc[dt][4 * g4] * wself;
        v4.y = acc[dt][4 * g4 + 1] * wself;
        v4.z = acc[dt][4 * g4 + 2] * wself;
        v4.w = acc[dt][4 * g4 + 3] * wself;
        *reinterpret_cast<float4*>(arow + 32 * dt + 8 * g4 + 4 * hh) = v4;
      }
    }
  }
  __syncthreads();
  // 32 rows x D/4 column quads; 256 threads.
  constexpr int QPR = D / 4;
  for (int task = tid; task < 32 * QPR; task += Cfg::NT) {
    const int rr = task / QPR, q4 = task - rr * QPR;
    const int rglob = 32 * rg + rr;
    if (rglob >= R) continue;
    float Mr = -INFINITY;
#pragma unroll
    for (int v = 0; v < Cfg::NW; ++v) Mr = fmaxf(Mr, sM[v * 32 + rr]);
    float L = 0.f;
    float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int v = 0; v < Cfg::NW; ++v) {
      const float mv = sM[v * 32 + rr];
      const float wv = (Mr == -INFINITY) ? 0.f : fast_exp2(mv - Mr);
      L += sL[v * 32 + rr] * wv;
      const float4 a = *reinterpret_cast<const float4*>(sAcc + (v * 32 + rr) * ASTR + 4 * q4);
      o4.x += a.x;
      o4.y += a.y;
      o4.z += a.z;
      o4.w += a.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    o4.x *= inv;
    o4.y *= inv;
    o4.z *= inv;
    o4.w *= inv;
    const float lse2 = L > 0.f ? Mr + __log2f(L) : -INFINITY;  // log2 units
    const int g2 = rglob / Nq, i2 = rglob - g2 * Nq, h2 = hkv * G + g2;
    const size_t rowi = ((size_t)b * Hq + h2) * Nq + i2;  // [B, Hq, Nq]
    if (S == 1) {
      bf16_t* orow = O + (((size_t)b * Nq + i2) * Hq + h2) * D + 4 * q4;
      uint2 u;
      u.x = __builtin_bit_cast(uint32_t, to_bf16x2(o4.x, o4.y));
      u.y = __builtin_bit_cast(uint32_t, to_bf16x2(o4.z, o4.w));
      *reinterpret_cast<uint2*>(orow) = u;
      if (q4 == 0) LSE[rowi] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    } else {
      const size_t prow = (size_t)split * B * Hq * Nq + rowi;
      *reinterpret_cast<float4*>(Opart + prow * D + 4 * q4) = o4;
      if (q4 == 0) Lpart[prow] = lse2;
    }
  }
}

// Merge of the chunks: one thread per (row, 4 columns).  Partial logsumexps are in log2
// units; a chunk with no allowed key has -inf and weight 0.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ Opart,
                                                           const float* __restrict__ Lpart,
                                                           bf16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int B,
                                                           int Hq, int Nq, int S) {
  constexpr int QPR = D / 4, RPB = 256 / QPR;
  const long rows = (long)B * Hq * Nq;
  const long rowi = (long)blockIdx.x * RPB + threadIdx.x / QPR;
  const int q4 = threadIdx.x % QPR;
  if (rowi >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, Lpart[(long)s * rows + rowi]);
  float L = 0.f;
  float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = Lpart[(long)s * rows + rowi];
      const float wv = fast_exp2(ls - M);  // 0 for an empty chunk
      L += wv;
      if (wv > 0.f) {
        const float4 a = *reinterpret_cast<const float4*>(Opart + ((long)s * rows + rowi) * D +
                                                          4 * q4);
        o4.x = fmaf(wv, a.x, o4.x);
        o4.y = fmaf(wv, a.y, o4.y);
        o4.z = fmaf(wv, a.z, o4.z);
        o4.w = fmaf(wv, a.w, o4.w);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int i = (int)(rowi % Nq);
  const long bh = rowi / Nq;
  const int h = (int)(bh % Hq);
  const long b = bh / Hq;
  bf16_t* orow = O + ((b * Nq + i) * Hq + h) * D + 4 * q4;
  uint2 u;
  u.x = __builtin_bit_cast(uint32_t, to_bf16x2(o4.x * inv, o4.y * inv));
  u.y = __builtin_bit_cast(uint32_t, to_bf16x2(o4.z * inv, o4.w * inv));
  *reinterpret_cast<uint2*>(orow) = u;
  if (q4 == 0) LSE[rowi] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  using Cfg = DecCfg<D>;
  // Dynamic LDS limit, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = hipFuncSetAttribute((const void*)decode_kernel<D>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int nrg = (a.Hq / a.Hkv * a.Nq + 31) / 32;
  if (a.ev_start) {
    const hipError_t e = hipEventRecord(a.ev_start, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_kernel<D>, dim3(a.B * a.Hkv * nrg * a.S), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, st, (const bf16_t*)a.q, (const bf16_t*)a.k,
                     (const bf16_t*)a.v, a.seqlens, (bf16_t*)a.o, a.lse, a.opart, a.lpart, a.B,
                     a.Hq, a.Hkv, a.Nq, a.Nk, a.causal, a.window, a.c_log2, a.neg_q, a.S, nrg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_stop) {
    e = hipEventRecord(a.ev_stop, st);
    if (e != hipSuccess) return e;
  }
  if (a.S == 1) return hipSuccess;
  constexpr int RPB = 256 / (D / 4);
  const long rows = (long)a.B * a.Hq * a.Nq;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                     0, st, a.opart, a.lpart, (bf16_t*)a.o, a.lse, a.B, a.Hq, a.Nq, a.S);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_decode_d<64>(a, st);
    case 128: return launch_decode_d<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
