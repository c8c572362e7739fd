// fa_fwd.hip -- forward attention kernels for gfx950.
//
// Tiled exact attention with the online softmax (ainews.cool, "flash-attention
// transformer optimization", technical deep dive: blocks that fit on-chip, running maximum
// and normaliser; bmjup.com, "FlashAttention-2 ... 实战解析", section 2.2: numerator and
// denominator kept apart and combined once at the end; section 3.2: the Q tile stays in
// registers while K and V tiles go through shared memory).
//
// bf16 kernel for d <= 128, one workgroup = 8 waves = 256 query rows of one (batch entry,
// query head) (d = 256: fwd_bf16_d256_kernel below):
//   * each wave owns 32 query rows; its Q rows sit in VGPRs as the B operand of
//     S^T = K Q^T (32 keys x 32 rows per MFMA tile), so every lane holds one query row
//     and 16 of its scores per tile -> row max/sum need one cross-half exchange only;
//   * K and V tiles of 64 keys are staged in LDS, double-buffered, from
//     16-byte raw buffer loads issued one tile ahead; V is transposed on the way in
//     (v_perm_b32 on register pairs), so V^T rows are plain 16-byte LDS reads;
//   * P^T (the accumulator of S^T after exp2) feeds O^T += V^T P^T directly as the B
//     operand;
//   * scores are handled in log2 units: t = (q.k) * |scale| * log2(e), so each probability
//     is one FMA and one exp2; a negative scale is handled by negating Q exactly;
//   * key tiles outside the causal / sliding-window band are never visited, and only
//     tiles crossing the band edge (or the end of the sequence) pay for per-element masks
//     (bmjup.com page, section 3.3: tile-level encoding of the mask);
//   * grid: each XCD owns a range of heads (work_item), heaviest query blocks first.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int D>
struct FwdCfg {
  static_assert(D <= 128, "head dim 256 has its own kernel");
  static constexpr int NW = 8;                 // waves per workgroup (2 per SIMD)
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int BM = 32 * NW;           // query rows per workgroup (32 per wave)
  static constexpr int BN = 64;                // keys staged per iteration
  static constexpr int KSTR = D + 8;           // K tile row stride in elements (16-byte pad)
  static constexpr int VSTR = BN + 8;          // V^T tile row stride in elements (16-byte pad)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;  // double buffered
};

__device__ __forceinline__ uint32_t word(const uint4& u, int m) {
  return m == 0 ? u.x : m == 1 ? u.y : m == 2 ? u.z : u.w;
}

// Position of key k (inside a key tile) in the V^T tile: bits 2 and 3 swapped, so that the
// 8 keys one lane feeds to an MFMA (keys kb + {0..3} and kb + 8 + {0..3}, matching the
// accumulator layout of S^T) sit next to each other and load as one 16-byte read.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D, int AL>
__global__ __launch_bounds__(FwdCfg<D>::NT, 1) void fwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Nmax,
    int causal, int window, float c, int neg_q, const int* __restrict__ cu, int ntot,
    const float* __restrict__ slopes) {
  using Cfg = FwdCfg<D>;
  constexpr int NT = Cfg::NT, BM = Cfg::BM, BN = Cfg::BN, KSTR = Cfg::KSTR, VSTR = Cfg::VSTR;
  constexpr int NC = D / 16;  // k-steps of S^T over the head dim
  constexpr int ND = D / 32;  // 32-wide head-dim tiles of O^T
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem);

  const int num_m = (Nmax + BM - 1) / BM;
  int b, hq, rank;
  work_item(B, Hq, num_m, b, hq, rank);
  const int mb = num_m - 1 - rank;  // causal: the last row block attends the most keys
  const int hkv = hq / (Hq / Hkv);
  int seq0, N;  // first row and length of this batch entry's sequence
  seq_span(cu, ntot, b, Nmax, seq0, N);
  if (mb * BM >= N) return;  // a row block past the end of a shorter packed sequence
  const size_t lse0 = stat_base(cu, ntot, b, Hq, hq, Nmax, seq0);
  const float slope2 = AL != 0 ? slopes[hq] * kLog2e : 0.f;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int m0 = mb * BM;
  const int wr0 = m0 + w * 32;
  const int row = wr0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Qh = Q + ((size_t)seq0 * Hq + hq) * D;
  const bf16_t* Kh = K + ((size_t)seq0 * Hkv + hkv) * D;
  const bf16_t* Vh = V + ((size_t)seq0 * Hkv + hkv) * D;

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

  // Staging (64-key tiles, 512 threads): thread = (key pair kp, 8-dim chunk dcp) of K and
  // of V, K stored row-major and V transposed (16-bit lane packing, one 32-bit word per V^T
  // row), the same work for every thread; key pairs run fastest inside a wave, which keeps
  // both kinds of store free of bank conflicts.  Tiles are read through buffer resources
  // whose size ends at row N, so rows past the end of the sequence load as zeros.
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int TP = (BN / 2) * CPR;      // key-pair tasks per tile
  static_assert(TP <= NT, "one key-pair task per thread");
  const uint32_t row_bytes = (uint32_t)ks * 2u;
  const bool ptask = TP == NT || tid < TP;
  const int kp = tid % (BN / 2), dcp = tid / (BN / 2);
  const uint32_t poff = (uint32_t)(2 * kp * ks + 8 * dcp) * 2u;
  uint4 xk[2], xv[2];
  auto gload = [&](int nb) {
    const int n0 = nb * BN;
    const uint32_t bytes = (uint32_t)(N - n0) * row_bytes;
    const rsrc_t kres = make_rsrc(Kh + (size_t)n0 * ks, bytes);
    const rsrc_t vres = make_rsrc(Vh + (size_t)n0 * ks, bytes);
    if (ptask) {
      xk[0] = bload16(kres, poff);
      xk[1] = bload16(kres, poff + row_bytes);
      xv[0] = bload16(vres, poff);
      xv[1] = bload16(vres, poff + row_bytes);
    }
  };
  auto swrite = [&](int buf) {
    bf16_t* sK = lds + buf * Cfg::BUF_ELEMS;
    bf16_t* sV = sK + Cfg::K_ELEMS;
    if (ptask) {
      bf16_t* kd = sK + (2 * kp) * KSTR + 8 * dcp;
      *reinterpret_cast<uint4*>(kd) = xk[0];
      *reinterpret_cast<uint4*>(kd + KSTR) = xk[1];
      // dim 8 dcp + j of the two keys -> one 32-bit word of V^T row 8 dcp + j
      bf16_t* vd = sV + (8 * dcp) * VSTR + vt_pos(2 * kp);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a0 = word(xv[0], m), a1 = word(xv[1], m);
        *reinterpret_cast<uint32_t*>(vd + (2 * m) * VSTR) = pack_lo(a0, a1);
        *reinterpret_cast<uint32_t*>(vd + (2 * m + 1) * VSTR) = pack_hi(a0, a1);
      }
    }
  };

  // Running state of this lane's row: reference max m (log2 units), and this lane-half's
  // sums of the bf16-rounded weights (normalise O, so O is a convex combination of V rows)
  // and of the unrounded weights (give the logsumexp).
  float m_i = -INFINITY, l_i = 0.f, le_i = 0.f;
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  const int klo = window > 0 ? row - window + 1 : 0;  // allowed keys of this row: [klo, khi]
  const int khi = causal ? min(row, N - 1) : N - 1;

  // Tile order.  Without a position bias: ascending.  With one, a row's largest biased
  // scores sit near its diagonal, so the tiles are visited from there outwards and the
  // reference max is set by the first tile instead of moving (and rescaling) on every one:
  // causal, descending from the last tile (each wave's first active tile holds its
  // diagonal); otherwise zig-zag outwards from the tile of the block's middle row.
  const int ntiles = nb_hi - nb_lo;
  const int nd = min(max((m0 + BM / 2) / BN, nb_lo), max(nb_hi - 1, nb_lo));
  const int zl = nd - nb_lo, zu = nb_hi - 1 - nd, zm = min(zl, zu);
  auto tile = [&](int t) {
    if constexpr (AL == 0) {
      return nb_lo + t;
    } else if constexpr (AL == 1) {
      return nb_hi - 1 - t;
    } else {
      if (t <= 2 * zm) return nd + ((t & 1) ? (t + 1) / 2 : -(t / 2));
      return zu > zl ? nd + (t - zm) : nd - (t - zm);
    }
  };

  if (ntiles > 0) {
    gload(tile(0));
    swrite(0);
    if (ntiles > 1) gload(tile(1));
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int nb = tile(t);
    const int buf = t & 1;
    const bf16_t* sK = lds + buf * Cfg::BUF_ELEMS;
    const bf16_t* sV = sK + Cfg::K_ELEMS;
    const int n0 = nb * BN;
    const bool active = wr0 < N && (!causal || n0 <= wr0 + 31) &&
                        (window <= 0 || n0 + BN - 1 >= wr0 - window + 1);
    if (active) {
      // The staged key tile is processed in 32-key pieces (QK^T, softmax, PV per piece),
      // which keeps only one 32 x 32 score tile live per wave.
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
        const int k0 = n0 + 32 * kt;
        if (causal && k0 > wr0 + 31) break;  // this half is entirely above the diagonal
        // S^T tile: keys k0 + [0, 32) x this wave's 32 rows.  All K operands of the piece
        // are read before the MFMAs that use them, and the V^T operands right after, so LDS
        // latency hides behind the MFMAs and the softmax.
        const bf16_t* kp = sK + (32 * kt + l32) * KSTR + 8 * hh;
        const bf16_t* vp = sV + l32 * VSTR + 8 * hh + 32 * kt;
        // V^T operand j = 2 dt + c2 (head-dim tile dt, key half c2)
        auto vread = [&](int j) { return lds_read_b128(vp + 32 * (j >> 1) * VSTR + 16 * (j & 1)); };
        f32x16 s = zero16();
        bf16x8 vop[2 * ND];
        bf16x8 kop[NC];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kop[cc] = lds_read_b128(kp + 16 * cc);
        // Raised wave priority over each MFMA run: the other wave on the SIMD gets the
        // softmax VALU slots while this one keeps the matrix core fed.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) s = mfma32(kop[cc], qop[cc], s);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int j = 0; j < 2 * ND; ++j) vop[j] = vread(j);

        // Online softmax.  In a piece that crosses the mask band (or the end of the
        // sequence) the masked scores are first replaced by -inf under a wave-uniform branch;
        // exp2 of -inf is 0, so the max and exp loops below carry no per-element mask.  The
        // accumulator rescale sits in one wave-uniform block, so no branch copies it.
        // (bitwise, not short-circuit: a branch-free scalar condition)
        const bool need_mask = (k0 + 32 > N) | ((causal != 0) & (k0 + 31 > wr0)) |
                               ((window > 0) & (k0 < wr0 + 32 - window));
        if (need_mask) {
          const int kb0 = k0 + hh * 4;  // key of element r: kb0 + (r / 4) * 8 + r % 4
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb0 + (r >> 2) * 8 + (r & 3);
            s[r] = ((key >= klo) & (key <= khi)) ? s[r] : -INFINITY;
          }
        }
        // Weights against the current reference max first.  The row max of the piece is
        // only taken, and the reference moved, when that cannot stand: a lane's partial sum
        // above kSumLimit (a weight above it, or overflow) or no reference yet (the sum is
        // then inf or NaN).  Otherwise weights stay below 2^12 and no max is needed.
        // Sums are taken as trees, not serial chains, so the wave's VALU work stays
        // independent enough to issue back to back.
        auto tree_sum = [](const float (&x)[16]) {
          float q[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = x[2 * i] + x[2 * i + 1];
          return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
        };
        // distance base of the piece for the position bias: key - row of element 0 of this
        // lane half is k0 + 4 hh - row; element r adds 8 (r / 4) + r % 4
        const float dbase = AL != 0 ? (float)(k0 + 4 * hh - row) : 0.f;
        auto koff = [](int r) { return (float)(8 * (r >> 2) + (r & 3)); };
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)  // 0 if masked
          e[r] = fast_exp2(fmaf(s[r], c, alibi_addend<AL>(slope2, dbase, koff(r), m_i)));
        float rse = tree_sum(e);
        if (__any(!(rse <= kSumLimit))) {  // wave-uniform; rare after a row's first piece
          float mt;
          if constexpr (AL == 0) {
            float mx = fmaxf(s[0], s[1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);  // v_max3
            mx = half_max(mx);
            mt = (mx == -INFINITY) ? -INFINITY : mx * c;
          } else {  // the maximum of the biased scores
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              mx = fmaxf(mx, fmaf(s[r], c, alibi_addend<AL>(slope2, dbase, koff(r), 0.f)));
            mt = half_max(mx);
          }
          const bool grow = mt > m_i + kRescaleThreshold;
          const float alpha = grow ? fast_exp2(m_i - mt) : 1.f;  // 0 when m_i was -inf
          l_i *= alpha;
          le_i *= alpha;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
          m_i = grow ? mt : m_i;
          const float m_use = (m_i == -INFINITY) ? 0.f : m_i;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            e[r] = fast_exp2(fmaf(s[r], c, alibi_addend<AL>(slope2, dbase, koff(r), m_use)));
          rse = tree_sum(e);
        }
        bf16x8 pp[2];
        float rs2[2] = {l_i, 0.f};  // two dot chains, one per half of the piece
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const bf16x2 pe = to_bf16x2(e[r], e[r + 1]);
          rs2[r >> 3] = __builtin_amdgcn_fdot2_f32_bf16(pe, ones, rs2[r >> 3], false);
          pp[r >> 3][r & 7] = pe[0];
          pp[r >> 3][(r & 7) + 1] = pe[1];
        }
        l_i = rs2[0] + rs2[1];
        le_i += rse;

        // O^T += V^T P^T.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 2 * ND; ++j) acc[j >> 1] = mfma32(vop[j], pp[j & 1], acc[j >> 1]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if (t + 1 < ntiles) {
      swrite(buf ^ 1);
      if (t + 2 < ntiles) gload(tile(t + 2));
    }
    __syncthreads();
  }

  // Epilogue: O = acc / l (one rounding to bf16), LSE = (m + log2 l) * ln 2.
  const float l = half_sum(l_i);
  const float le = half_sum(le_i);
  if (row < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* orow = O + ((size_t)seq0 + row) * qs + (size_t)hq * D;
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
      LSE[lse0 + row] = le > 0.f ? (m_i + __log2f(le)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------
// bf16 forward for d = 256: 4 waves x 32 query rows = 128 rows of one (batch entry, query
// head) per workgroup, 32-key tiles, one wave per SIMD.  With no second wave on a SIMD to
// take the exponentials while the other wave's products run, each wave overlaps the two
// itself: during step t it computes the scores of tile t + 1 (S^T = K Q^T, 16 products)
// and, between those products, the weights of tile t (one score element per product); the
// O^T products of tile t follow.  K tiles are therefore staged one tile ahead of V tiles
// (K of tile t + 1 and V of tile t are in LDS during step t, each in its own pair of
// buffers).  The 128 O^T accumulator registers live in AGPRs (assembly products), which
// leaves the VGPRs for Q, two score tiles and the staging registers.  Everything else (mask
// band, lazy reference max, rounded-weight sums, tile order, epilogue) is as in
// fwd_bf16_kernel.
struct D256Cfg {
  static constexpr int D = 256;
  static constexpr int NT = 256;       // 4 waves
  static constexpr int BM = 128;       // query rows per workgroup
  static constexpr int BN = 32;        // keys per tile
  static constexpr int KSTR = D + 8;   // K tile row stride in elements (16-byte pad)
  static constexpr int VSTR = BN + 8;  // V^T tile row stride in elements (16-byte pad)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int LDS_BYTES = 2 * (K_ELEMS + V_ELEMS) * 2;  // two K and two V^T buffers
};

template <int AL>
__global__ __launch_bounds__(D256Cfg::NT, 1) void fwd_bf16_d256_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Nmax,
    int causal, int window, float c, int neg_q, const int* __restrict__ cu, int ntot,
    const float* __restrict__ slopes) {
  using Cfg = D256Cfg;
  constexpr int D = Cfg::D, NT = Cfg::NT, BM = Cfg::BM, BN = Cfg::BN;
  constexpr int KSTR = Cfg::KSTR, VSTR = Cfg::VSTR;
  constexpr int NC = D / 16;  // k-steps of S^T over the head dim
  constexpr int ND = D / 32;  // 32-wide head-dim tiles of O^T
  constexpr int kRing = 4, kAhead = 3;  // operand ring: registers, products read ahead
  static_assert(NC == 16, "one score element of the previous tile per S^T product");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem);
  auto kbuf = [&](int i) { return lds + i * Cfg::K_ELEMS; };
  auto vbuf = [&](int i) { return lds + 2 * Cfg::K_ELEMS + i * Cfg::V_ELEMS; };

  const int num_m = (Nmax + BM - 1) / BM;
  int b, hq, rank;
  work_item(B, Hq, num_m, b, hq, rank);
  const int mb = num_m - 1 - rank;  // causal: the last row block attends the most keys
  const int hkv = hq / (Hq / Hkv);
  int seq0, N;  // first row and length of this batch entry's sequence
  seq_span(cu, ntot, b, Nmax, seq0, N);
  if (mb * BM >= N) return;  // a row block past the end of a shorter packed sequence
  const size_t lse0 = stat_base(cu, ntot, b, Hq, hq, Nmax, seq0);
  const float slope2 = AL != 0 ? slopes[hq] * kLog2e : 0.f;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int m0 = mb * BM;
  const int wr0 = m0 + w * 32;
  const int row = wr0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Qh = Q + ((size_t)seq0 * Hq + hq) * D;
  const bf16_t* Kh = K + ((size_t)seq0 * Hkv + hkv) * D;
  const bf16_t* Vh = V + ((size_t)seq0 * Hkv + hkv) * D;

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

  // Staging.  K: the tile's 32 x 32 16-byte chunks, four per thread, stored row-major.
  // V: one (4-key group, 8-dim chunk) task per thread, transposed in registers; key groups
  // run fastest, so the 16 lanes the LDS writes per cycle of an 8-byte transposed store span
  // all eight key groups of the tile and two chunks, two lanes per bank.  Tiles are read
  // through buffer resources whose size ends at row N, so rows past the end of the
  // sequence load as zeros.
  constexpr int CPR = D / 8;      // 16-byte chunks per K/V row
  constexpr int PTK = BN * CPR / NT;
  static_assert(BN * CPR == PTK * NT && (BN / 4) * CPR == NT, "whole staging tasks per thread");
  const uint32_t row_bytes = (uint32_t)ks * 2u;
  // two register sets: the loads of step t land in set t % 2 and are stored in step t + 2
  uint4 kr[2][PTK], vr[2][4];
  uint32_t koff[PTK];
#pragma unroll
  for (int i = 0; i < PTK; ++i) {
    const int ch = tid + NT * i;
    koff[i] = (uint32_t)((ch / CPR) * ks + (ch % CPR) * 8) * 2u;
  }
  const int vkg = tid % (BN / 4), vdc = tid / (BN / 4);
  const uint32_t voff = (uint32_t)(4 * vkg * ks + vdc * 8) * 2u;
  // Staging pieces, so that they can sit between matrix products.  A K piece is one of the
  // thread's four chunks, a V piece two rows of its transposed task.
  auto tile_rsrc = [&](const bf16_t* base, int nb) {
    const int n0 = nb * BN;
    return make_rsrc(base + (size_t)n0 * ks, (uint32_t)(N - n0) * row_bytes);
  };
  auto kload = [&](int rs, const rsrc_t& res, int i) { kr[rs][i] = bload16(res, koff[i]); };
  auto vload = [&](int rs, const rsrc_t& res, int e) {
    vr[rs][e] = bload16(res, voff + e * row_bytes);
  };
  auto kstore = [&](int rs, int buf, int i) {
    const int ch = tid + NT * i;
    *reinterpret_cast<uint4*>(kbuf(buf) + (ch / CPR) * KSTR + (ch % CPR) * 8) = kr[rs][i];
  };
  auto vstore = [&](int rs, int buf, int m) {
    bf16_t* dst = vbuf(buf) + (vdc * 8) * VSTR + vt_pos(4 * vkg);
    const uint32_t a0 = word(vr[rs][0], m), a1 = word(vr[rs][1], m);
    const uint32_t a2 = word(vr[rs][2], m), a3 = word(vr[rs][3], m);
    uint2 even, odd;  // dims 2m and 2m+1, keys 0..3 of the group
    even.x = pack_lo(a0, a1);
    even.y = pack_lo(a2, a3);
    odd.x = pack_hi(a0, a1);
    odd.y = pack_hi(a2, a3);
    *reinterpret_cast<uint2*>(dst + (2 * m) * VSTR) = even;
    *reinterpret_cast<uint2*>(dst + (2 * m + 1) * VSTR) = odd;
  };

  // Running state of this lane's row, as in fwd_bf16_kernel.
  float m_i = -INFINITY, l_i = 0.f, le_i = 0.f;
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  acc_written(acc);
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  const int klo = window > 0 ? row - window + 1 : 0;  // allowed keys of this row: [klo, khi]
  const int khi = causal ? min(row, N - 1) : N - 1;

  // Tile order, as in fwd_bf16_kernel.
  const int ntiles = nb_hi - nb_lo;
  const int nd = min(max((m0 + BM / 2) / BN, nb_lo), max(nb_hi - 1, nb_lo));
  const int zl = nd - nb_lo, zu = nb_hi - 1 - nd, zm = min(zl, zu);
  auto tile = [&](int t) {
    if constexpr (AL == 0) {
      return nb_lo + t;
    } else if constexpr (AL == 1) {
      return nb_hi - 1 - t;
    } else {
      if (t <= 2 * zm) return nd + ((t & 1) ? (t + 1) / 2 : -(t / 2));
      return zu > zl ? nd + (t - zm) : nd - (t - zm);
    }
  };
  // whether this wave has an allowed (row, key) pair in tile t (wave-uniform)
  auto active = [&](int t) {
    const int n0 = tile(t) * BN;
    return wr0 < N && (!causal || n0 <= wr0 + 31) &&
           (window <= 0 || n0 + BN - 1 >= wr0 - window + 1);
  };

  const bf16_t* kp0 = lds + l32 * KSTR + 8 * hh;  // this lane's K row, buffer 0
  // S^T of the tile in K buffer kb, without anything beside the products.
  auto scores = [&](int kb, f32x16& s) {
    const bf16_t* kp = kp0 + kb * Cfg::K_ELEMS;
    bf16x8 kop[kRing];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kop[i] = lds_read_b128(kp + 16 * i);
    s = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc + kAhead < NC) kop[(cc + kAhead) % kRing] = lds_read_b128(kp + 16 * (cc + kAhead));
      s = mfma32(kop[cc % kRing], qop[cc], s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto koffs = [](int r) { return (float)(8 * (r >> 2) + (r & 3)); };
  // Step t: weights and O^T products of tile t (scores in sc), scores of tile t + 1 into sn.
  // Staging in step t, from and into register set rs = t % 2: K of tile t + 2 replaces K of
  // tile t (read during step t - 1), V of tile t + 1 replaces V of tile t - 1, then the
  // loads of K of tile t + 4 and V of tile t + 3 for step t + 2.  Past the last tile the
  // indices are clamped: a store then fills a buffer no later step reads, and a load reads
  // the last tile again.
  auto step = [&](int t, int rs, f32x16& sc, f32x16& sn) {
    const int tl = ntiles - 1;
    const bool more = t + 1 < ntiles;
    const bool act = active(t), act_n = more && active(t + 1);
    const rsrc_t kres = tile_rsrc(Kh, tile(min(t + 4, tl)));
    const rsrc_t vres = tile_rsrc(Vh, tile(min(t + 3, tl)));
    // staging piece j of 16: K stores, V stores, K loads, V loads
    auto stage = [&](int j) {
      if (j < 4) kstore(rs, t & 1, j);
      else if (j < 8) vstore(rs, (t + 1) & 1, j - 4);
      else if (j < 12) kload(rs, kres, j - 8);
      else vload(rs, vres, j - 12);
    };
    if (act) {
      const int k0 = tile(t) * BN;
      // (bitwise, not short-circuit: a branch-free scalar condition)
      const bool need_mask = (k0 + 32 > N) | ((causal != 0) & (k0 + 31 > wr0)) |
                             ((window > 0) & (k0 < wr0 + 32 - window));
      if (need_mask) {
        const int kb0 = k0 + hh * 4;  // key of element r: kb0 + (r / 4) * 8 + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + (r >> 2) * 8 + (r & 3);
          sc[r] = ((key >= klo) & (key <= khi)) ? sc[r] : -INFINITY;
        }
      }
      const float dbase = AL != 0 ? (float)(k0 + 4 * hh - row) : 0.f;
      float e[16], q[8];
      if (act_n) {
        // Products of tile t + 1 with the weights of tile t between them: product cc, then
        // weight cc and the pair sum of the weights two before.  (The empty assembly keeps
        // the compiler from hoisting the exponent arguments out of this loop.)
        float mref = m_i;
        asm volatile("" : "+v"(mref));
        const bf16_t* kp = kp0 + ((t + 1) & 1) * Cfg::K_ELEMS;
        bf16x8 kop[kRing];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) kop[i] = lds_read_b128(kp + 16 * i);
        sn = zero16();
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          if (cc + kAhead < NC) kop[(cc + kAhead) % kRing] = lds_read_b128(kp + 16 * (cc + kAhead));
          sn = mfma32(kop[cc % kRing], qop[cc], sn);
          e[cc] = fast_exp2(fmaf(sc[cc], c, alibi_addend<AL>(slope2, dbase, koffs(cc), mref)));
          if (cc >= 2 && (cc & 1) == 0) q[cc / 2 - 1] = e[cc - 2] + e[cc - 1];
          __builtin_amdgcn_sched_barrier(0);
        }
        q[7] = e[14] + e[15];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          e[r] = fast_exp2(fmaf(sc[r], c, alibi_addend<AL>(slope2, dbase, koffs(r), m_i)));
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = e[2 * i] + e[2 * i + 1];
      }
      float rse = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));

      // V^T operands of tile t: j = 8 half + dt (head-dim tile dt, key half), so the
      // products of the first key half can run while the second half's weights convert.
      const bf16_t* vp = vbuf(t & 1) + l32 * VSTR + 8 * hh;
      auto vread = [&](int j) { return lds_read_b128(vp + 32 * (j & 7) * VSTR + 16 * (j >> 3)); };
      bf16x8 vop[kRing];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) vop[i] = vread(i);

      if (__any(!(rse <= kSumLimit))) {  // wave-uniform; rare after a row's first tile
        float mt;
        if constexpr (AL == 0) {
          float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
          for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[r]), sc[r + 1]);  // v_max3
          mx = half_max(mx);
          mt = (mx == -INFINITY) ? -INFINITY : mx * c;
        } else {  // the maximum of the biased scores
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            mx = fmaxf(mx, fmaf(sc[r], c, alibi_addend<AL>(slope2, dbase, koffs(r), 0.f)));
          mt = half_max(mx);
        }
        const bool grow = mt > m_i + kRescaleThreshold;
        const float alpha = grow ? fast_exp2(m_i - mt) : 1.f;  // 0 when m_i was -inf
        l_i *= alpha;
        le_i *= alpha;
        acc_ready(acc);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        acc_written(acc);
        m_i = grow ? mt : m_i;
        const float m_use = (m_i == -INFINITY) ? 0.f : m_i;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          e[r] = fast_exp2(fmaf(sc[r], c, alibi_addend<AL>(slope2, dbase, koffs(r), m_use)));
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = e[2 * i] + e[2 * i + 1];
        rse = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
      }
      // Rounded weights of key half h: P^T operand pp[h], its sum into its own dot chain.
      bf16x8 pp[2];
      float rs2[2] = {l_i, 0.f};
      auto convert = [&](int h) {
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; r += 2) {
          const bf16x2 pe = to_bf16x2(e[r], e[r + 1]);
          rs2[h] = __builtin_amdgcn_fdot2_f32_bf16(pe, ones, rs2[h], false);
          pp[h][r & 7] = pe[0];
          pp[h][(r & 7) + 1] = pe[1];
        }
        operand_ready(pp[h]);
      };
      convert(0);

      // O^T += V^T P^T, with the staging pieces and the second half's weights between the
      // products.
#pragma unroll
      for (int j = 0; j < 2 * ND; ++j) {
        if (j + kAhead < 2 * ND) vop[(j + kAhead) % kRing] = vread(j + kAhead);
        if (j == ND) convert(1);
        mfma_acc(acc[j & 7], vop[j % kRing], pp[j >> 3]);
        stage(j);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_i = rs2[0] + rs2[1];
      le_i += rse;
    } else {
      if (act_n) scores((t + 1) & 1, sn);
#pragma unroll
      for (int j = 0; j < 16; ++j) stage(j);
    }
    __syncthreads();
  };

  f32x16 sa = zero16(), sb = zero16();
  if (ntiles > 0) {
    const int tl = ntiles - 1;
    // LDS: K of tiles 0 and 1, V of tile 0.  Register set 0: K of tile 2, V of tile 1; set
    // 1: K of tile 3, V of tile 2.
#pragma unroll
    for (int i = 0; i < PTK; ++i) kload(0, tile_rsrc(Kh, tile(0)), i);
#pragma unroll
    for (int e = 0; e < 4; ++e) vload(0, tile_rsrc(Vh, tile(0)), e);
#pragma unroll
    for (int i = 0; i < PTK; ++i) kload(1, tile_rsrc(Kh, tile(min(1, tl))), i);
#pragma unroll
    for (int i = 0; i < PTK; ++i) kstore(0, 0, i);
#pragma unroll
    for (int m = 0; m < 4; ++m) vstore(0, 0, m);
#pragma unroll
    for (int i = 0; i < PTK; ++i) kstore(1, 1, i);
#pragma unroll
    for (int i = 0; i < PTK; ++i) kload(0, tile_rsrc(Kh, tile(min(2, tl))), i);
#pragma unroll
    for (int e = 0; e < 4; ++e) vload(0, tile_rsrc(Vh, tile(min(1, tl))), e);
#pragma unroll
    for (int i = 0; i < PTK; ++i) kload(1, tile_rsrc(Kh, tile(min(3, tl))), i);
#pragma unroll
    for (int e = 0; e < 4; ++e) vload(1, tile_rsrc(Vh, tile(min(2, tl))), e);
    __syncthreads();
    if (active(0)) scores(0, sa);
    __syncthreads();  // K buffer 0 is rewritten during step 0
  }
  // Whole pairs of steps in the loop, so that every path into a step has issued the other
  // register set's loads after this set's and the load waits can leave them in flight.
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(t, 0, sa, sb);
    step(t + 1, 1, sb, sa);
  }
  if (t < ntiles) step(t, 0, sa, sb);
  acc_ready(acc);

  // Epilogue: O = acc / l (one rounding to bf16), LSE = (m + log2 l) * ln 2.
  const float l = half_sum(l_i);
  const float le = half_sum(le_i);
  if (row < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* orow = O + ((size_t)seq0 + row) * qs + (size_t)hq * D;
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
      LSE[lse0 + row] = le > 0.f ? (m_i + __log2f(le)) * kLn2 : -INFINITY;
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
template <int D, int AL>
static hipError_t launch_fwd_bf16_d(const FwdArgs& a, hipStream_t st) {
  using Cfg = FwdCfg<D>;
  // Dynamic LDS limit, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D, AL>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int num_m = (a.N + Cfg::BM - 1) / Cfg::BM;
  const int grid = a.B * a.Hq * num_m;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, AL>), dim3(grid), dim3(Cfg::NT), Cfg::LDS_BYTES, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window, a.c_log2, a.neg_q, a.cu,
                     a.ntot, a.slopes);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_bf16_al(const FwdArgs& a, hipStream_t st) {
  static_assert(D <= 128, "head dim 256: launch_fwd_bf16_d256");
  if (a.slopes == nullptr) return launch_fwd_bf16_d<D, 0>(a, st);
  return a.causal ? launch_fwd_bf16_d<D, 1>(a, st) : launch_fwd_bf16_d<D, 2>(a, st);
}

template <int AL>
static hipError_t launch_fwd_bf16_d256(const FwdArgs& a, hipStream_t st) {
  using Cfg = D256Cfg;
  // Dynamic LDS limit, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = hipFuncSetAttribute((const void*)fwd_bf16_d256_kernel<AL>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int num_m = (a.N + Cfg::BM - 1) / Cfg::BM;
  const int grid = a.B * a.Hq * num_m;
  hipLaunchKernelGGL((fwd_bf16_d256_kernel<AL>), dim3(grid), dim3(Cfg::NT), Cfg::LDS_BYTES, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window, a.c_log2, a.neg_q, a.cu,
                     a.ntot, a.slopes);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_fwd_bf16_al<64>(a, st);
    case 128: return launch_fwd_bf16_al<128>(a, st);
    case 256:
      if (a.slopes == nullptr) return launch_fwd_bf16_d256<0>(a, st);
      return a.causal ? launch_fwd_bf16_d256<1>(a, st) : launch_fwd_bf16_d256<2>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t launch_fwd_fp32_d(const FwdArgs& a, hipStream_t st) {
  using Cfg = Fp32Cfg<D>;
  // Dynamic LDS limit, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = hipFuncSetAttribute((const void*)fwd_fp32_kernel<D>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
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
