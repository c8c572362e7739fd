// fa_bwd.hip -- backward attention kernels for gfx950.
//
// The backward recomputes the probability matrix block by block from Q, K and the
// stored logsumexp instead of reading a stored N x N matrix (ainews.cool, "flash-attention
// transformer optimization", technical deep dive, item 2).  With L = sum(O * dO):
//   D_i   = sum_c dO_ic O_ic                                   (preprocess kernel)
//   P_ij  = exp(s_ij - LSE_i),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i      (key-block kernel)
//   dQ_i  = scale sum_j dS_ij k_j                               (query-block kernel)
//
// Two main kernels instead of one with atomics.  On this chip a CU's LDS serves about one
// 16-byte operand read per 32x32x16 MFMA, so every product reads its LDS operand with one
// ds_read_b128: operands that must be contiguous along the reduced index (Q^T and dO^T for
// dK/dV, K^T for dQ) are transposed once while being staged (register packing, see
// store_4x8_transposed), never with per-use transposing reads.  Recomputing S and dP in the
// query-block kernel costs two extra products per tile pair but removes the float32 dQ
// accumulator, its atomics and its conversion pass, and keeps dQ deterministic.
//
// Key-block kernel: a workgroup = 8 waves = 256 keys of one (batch entry, KV head) for
// d <= 128 (bwd_dkdv8_kernel), 4 waves = 128 keys for d = 256 (bwd_dkdv_kernel); 32 keys
// per wave.  The wave's K rows are MFMA B operands in VGPRs; dK^T and dV^T accumulate in
// registers across every query head of the GQA group and every query block, and are
// written once.  At d = 256 those accumulators fill all 256 AGPRs of a wave (one wave per
// SIMD), with K, V and the score work in the 256 VGPRs.
//
// Both grids follow work_item: each XCD owns a range of heads, heaviest blocks first.
//
// Query-block kernel: a workgroup = 8 waves (d <= 128) or 4 waves = 32 query rows per wave,
// the same shape as the forward: Q and dO rows are B operands in VGPRs, K, V and K^T tiles
// stream through double-buffered LDS, and S^T / dP^T put one query row in each lane so LSE
// and D are per-lane scalars and dS^T feeds dQ^T += K^T dS^T straight from the accumulator.
#include <mutex>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Workspace of the no-allocation backward (fa_bwd_noalloc): the D vector of up to
// kNoAllocRows rows in a static device array.  Every device the library runs on holds its
// own copy for the life of the process; in host code only the address that
// hipGetSymbolAddress returns for the current device may be used, never the array's name.
__device__ __align__(256) float scratch[kNoAllocRows];

hipError_t noalloc_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_bf16x2(a, b));
}

// D = rowsum(dO * O) in float32 from the stored bf16 O.  D/8 threads per (batch, row, head)
// row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_t* __restrict__ O,
                                                      const bf16_t* __restrict__ dO,
                                                      float* __restrict__ Dv, int B, int Hq,
                                                      int N, const int* __restrict__ cu,
                                                      int ntot) {
  constexpr int T = D / 8, RPB = 256 / T;
  const long total = cu ? (long)ntot * Hq : (long)B * N * Hq;  // rows (token, head)
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
  }
#pragma unroll
  for (int off = T / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (t == 0 && r < total) {
    const int hq = (int)(r % Hq);
    const long bn = r / Hq;  // token row
    if (cu) {
      Dv[(long)hq * ntot + bn] = sum;  // packed sequences: [Hq, total]
    } else {
      const int n = (int)(bn % N), b = (int)(bn / N);
      Dv[((long)b * Hq + hq) * N + n] = sum;
    }
  }
}

// Key block of a given cost rank (0 = heaviest) in a sequence of `nb` key blocks, when the
// longest sequence has `num_kb`.  Causal or unmasked: a block's cost is the number of query
// rows that reach it, which falls towards the end of the sequence, so the ranks count blocks
// from the sequence's end and rank 0 is block 0 of the longest sequences only.  A pure left
// window: later blocks are reached by more rows, so the ranks count down from the last
// block.  Ranks with no block in a shorter sequence give a negative or too-large index.
__device__ __forceinline__ int key_block(int rank, int num_kb, int nb, int causal, int window) {
  return (!causal && window > 0) ? num_kb - 1 - rank : nb - num_kb + rank;
}

// =====================================================================================
// dK / dV

// After vector writes of product operands, before the products read them.
__device__ __forceinline__ void operands_ready(bf16x8 (&p)[2], bf16x8 (&q)[2]) {
  asm volatile("s_nop 1" : "+v"(p[0]), "+v"(p[1]), "+v"(q[0]), "+v"(q[1]));
}

// Order of the (4-row group, 8-column chunk) staging tasks of the d = 256 kernels: lane bits
// 0-1 pick the chunk, bits 2-3 the row group, higher bits the rest.  The LDS has 32
// four-byte banks for stores and writes 8 lanes of a 16-byte store per cycle; with row
// strides of 4 (mod 32) dwords the 8 lanes of a row-major store then cover two row groups
// and four chunks, 32 distinct banks, where task_rc's four row groups put two lanes on
// every bank.  The transposed stores (16 lanes per cycle, four row groups) are as before.
// A bijection on [0, rows / 4 * CPR) when rows is a multiple of 16 and CPR of 4.
template <int CPR>
__device__ __forceinline__ void task_rc4(int t, int& rg, int& dc) {
  const int q = t >> 4;
  dc = (t & 3) + 4 * (q % (CPR / 4));
  rg = ((t >> 2) & 3) + 4 * (q / (CPR / 4));
}

template <int D>
struct KVCfg {
  static constexpr int NT = 256;                 // 4 waves x 32 keys
  static constexpr int BKN = 128;                // keys per workgroup
  static constexpr int BQ = D <= 128 ? 64 : 32;  // query rows per step
  static constexpr int MT = BQ / 32;             // 32-row MFMA tiles per step
  static constexpr int STR = D + 8;              // row-major Q / dO row stride (elements)
  static constexpr int TSTR = BQ + 8;            // transposed Q^T / dO^T row stride
  static constexpr int SQ = BQ * STR;
  static constexpr int SQT = D * TSTR;
  static constexpr int BUF = 2 * SQ + 2 * SQT;   // Q, dO, Q^T, dO^T (elements)
  static constexpr int LDS_BYTES = 2 * (BUF * 2 + 2 * BQ * 4);  // + LSE, D; double buffered
  static_assert(LDS_BYTES <= 160 * 1024, "staging fits the CU's LDS");
};

template <int D, int AL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int B, int Hq, int Hkv, int Nmax,
    int causal, int window, float c, float scale, const int* __restrict__ cu, int ntot,
    const float* __restrict__ slopes) {
  using Cfg = KVCfg<D>;
  constexpr int BKN = Cfg::BKN, BQ = Cfg::BQ, MT = Cfg::MT;
  constexpr int STR = Cfg::STR, TSTR = Cfg::TSTR;
  constexpr int NC = D / 16;   // k-steps of S and dP over the head dim
  constexpr int NDH = D / 32;  // 32-wide head-dim tiles of dK^T / dV^T
  constexpr int BUFB = Cfg::BUF * 2 + 2 * BQ * 4;  // bytes per buffer
  constexpr int kRing = 4, kAh = 3;  // operand rings (see the step loop)
  // dK^T / dV^T in AGPRs through the assembly products (all 256 of them)
  static_assert(D == 256 && MT == 1, "the key-block kernel for d = 256 (d <= 128: bwd_dkdv8_kernel)");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int num_kb = (Nmax + BKN - 1) / BKN;
  int b, hkv, rank;
  work_item(B, Hkv, num_kb, b, hkv, rank);
  int seq0, N;  // first row and length of this batch entry's sequence
  seq_span(cu, ntot, b, Nmax, seq0, N);
  const int kb = key_block(rank, num_kb, (N + BKN - 1) / BKN, causal, window);
  if (kb < 0 || kb * BKN >= N) return;  // no such block in a shorter packed sequence
  const int G = Hq / Hkv;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int n0 = kb * BKN, kw0 = n0 + 32 * w, key = kw0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Kb = K + ((size_t)seq0 * Hkv + hkv) * D;
  const bf16_t* Vb = V + ((size_t)seq0 * Hkv + hkv) * D;

  // B operands K^T and V^T of this lane's key.
  bf16x8 kop[NC], vop[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    kop[cc] = __builtin_bit_cast(bf16x8, key < N ? gload16(Kb + (size_t)key * ks + 16 * cc + 8 * hh) : z);
    vop[cc] = __builtin_bit_cast(bf16x8, key < N ? gload16(Vb + (size_t)key * ks + 16 * cc + 8 * hh) : z);
  }

  // query rows any key of this block can be attended by
  const int qb_lo = causal ? n0 / BQ : 0;
  const int row_end = window > 0 ? min(N, n0 + BKN + window - 1) : N;
  const int qb_hi = (row_end + BQ - 1) / BQ;
  const int nq = max(0, qb_hi - qb_lo);
  const int total_it = G * nq;
  // Step it = (query block qi, query head g of the group) = (it / G, it % G): query-block
  // major, so the workgroups of one KV head that run together read the same Q / dO rows
  // at about the same time and share them in L2.  Causal blocks walk their query blocks
  // from the last one down: all start at the end of the sequence and stop at their own
  // diagonal, instead of each starting at a different row.
  auto qblock = [&](int qi) { return causal ? qb_hi - 1 - qi : qb_lo + qi; };
  // ALiBi slope (log2 units) of the query head of step it
  auto slope_of = [&](int it) { return AL != 0 ? slopes[hkv * G + it % G] * kLog2e : 0.f; };

  f32x16 dk[NDH], dv[NDH];
#pragma unroll
  for (int i = 0; i < NDH; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }
  acc_written(dk);
  acc_written(dv);

  // Staging: a task = 4 rows x 8 dims of Q and of dO, stored row-major and transposed.
  constexpr int CPR = D / 8;
  constexpr int TASKS = (BQ / 4) * CPR;
  static_assert(BQ % 16 == 0 && CPR % 4 == 0, "task_rc4 needs whole groups of 16 rows and 4 chunks");
  static_assert(TASKS == 256, "one staging task per thread");
  int srg, sdc;
  task_rc4<CPR>(tid, srg, sdc);
  const uint32_t soff = (uint32_t)(4 * srg * qs + 8 * sdc) * 2u;
  uint4 qr[4], orr[4];
  float lreg = 0.f, dreg = 0.f;
  // The staging of a step in pieces that can sit between matrix products.  Loads of step
  // it: part 0 the thread's Q rows, 1 its dO rows, 2 LSE and D.
  auto gload_part = [&](int it, int part) {
    const int qi = it / G, g = it - qi * G, qb = qblock(qi);
    const int hq = hkv * G + g, r0 = qb * BQ;
    if (part < 2) {
      const bf16_t* base = (part == 0 ? Q : dO) + ((size_t)seq0 * Hq + hq) * D;
      const uint32_t bytes = (uint32_t)(N - r0) * (uint32_t)qs * 2u;  // rows past N read 0
      const rsrc_t res = make_rsrc(base + (size_t)r0 * qs, bytes);
      if (part == 0) bload_4x8(qr, res, soff, (uint32_t)qs * 2u);
      else bload_4x8(orr, res, soff, (uint32_t)qs * 2u);
    } else if (tid < BQ) {
      const int n = r0 + tid;
      const size_t li = stat_base(cu, ntot, b, Hq, hq, Nmax, seq0) + n;
      lreg = n < N ? LSE[li] * kLog2e : INFINITY;  // +inf -> P = 0 on padding rows
      dreg = n < N ? Dv[li] : 0.f;
    }
  };
  // Stores into buffer buf for step buf_it: part 0 / 1 the Q / dO rows, 2-5 / 6-9 a quarter
  // of the transposed Q / dO rows each, 10 LSE and -D.
  constexpr int kStoreParts = 11, kLoadParts = 3;
  auto swrite_part = [&](int buf, int buf_it, int part) {
    bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + buf * BUFB);
    bf16_t* sO = sQ + Cfg::SQ;
    bf16_t* sQT = sO + Cfg::SQ;
    bf16_t* sOT = sQT + Cfg::SQT;
    float* sL = reinterpret_cast<float*>(sOT + Cfg::SQT);
    if (part == 0) store_4x8_rows(sQ, STR, 4 * srg, 8 * sdc, qr);
    else if (part == 1) store_4x8_rows(sO, STR, 4 * srg, 8 * sdc, orr);
    else if (part < 6) store_4x8_transposed_part(sQT, TSTR, 4 * srg, 8 * sdc, qr, part - 2);
    else if (part < 10) store_4x8_transposed_part(sOT, TSTR, 4 * srg, 8 * sdc, orr, part - 6);
    else if (tid < BQ) {
      // causal position bias: LSE + slope2 (row - r0) is staged, slope2 (key - r0) added per
      // lane (both small near the diagonal, where the weights are not negligible)
      sL[tid] = AL == 1 ? lreg + slope_of(buf_it) * tid : lreg;
      sL[BQ + tid] = -dreg;  // -D: the dP accumulators start from it
    }
  };

  if (total_it > 0) {
#pragma unroll
    for (int part = 0; part < kLoadParts; ++part) gload_part(0, part);
#pragma unroll
    for (int part = 0; part < kStoreParts; ++part) swrite_part(0, 0, part);
#pragma unroll
    for (int part = 0; part < kLoadParts; ++part) gload_part(min(1, total_it - 1), part);
  }
  __syncthreads();
  for (int it = 0; it < total_it; ++it) {
    const int buf = it & 1;
    const bf16_t* sQ = reinterpret_cast<const bf16_t*>(smem + buf * BUFB);
    const bf16_t* sO = sQ + Cfg::SQ;
    const bf16_t* sQT = sO + Cfg::SQ;
    const bf16_t* sOT = sQT + Cfg::SQT;
    const float* sL = reinterpret_cast<const float*>(sOT + Cfg::SQT);
    const float* sD = sL + BQ;
    const int qi = it / G, g = it - qi * G, qb = qblock(qi);
    const int r0 = qb * BQ;
    (void)g;
    const bool active = kw0 < N && (!causal || r0 + BQ - 1 >= kw0) &&
                        (window <= 0 || r0 <= kw0 + 31 + window - 1);
    // Staging in step it: the stores of step it + 1 into the other buffer (read during step
    // it - 1), then the loads of step it + 2.  Past the last step the stores fill a buffer
    // no later step reads and the loads repeat the last step's.
    const int itl = min(it + 2, total_it - 1);
    if (active) {
      // One step = four product phases of 16 products each, every product with one A
      // operand from LDS read kAh products ahead through one ring: S = Q K^T, dP = dO V^T
      // (lane = key, rows in registers), dV^T += dO^T P, dK^T += Q^T dS.  The vector work
      // sits between the products of the phase after the one it depends on: the weights
      // P = exp2(S c + bias - LSE log2 e) between the dP products (one per product), dS =
      // P (dP - D) between the dV products.  With one wave per SIMD nothing else would run
      // beside the products.
      f32x16 s = zero16(), dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {  // dP - D straight out of the products
        const f32x4 nd4 = *reinterpret_cast<const f32x4*>(sD + 8 * g4 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * g4 + e] = nd4[e];
      }
      const bf16_t* qa = sQ + l32 * STR + 8 * hh;
      const bf16_t* oa = sO + l32 * STR + 8 * hh;
      auto rowread = [&](int p) { return lds_read_b128((p < NC ? qa : oa) + 16 * (p % NC)); };
      bf16x8 ring[kRing];
#pragma unroll
      for (int i = 0; i < kAh; ++i) ring[i] = rowread(i);
#pragma unroll
      for (int p = 0; p < NC; ++p) {
        ring[(p + kAh) % kRing] = rowread(p + kAh);
        s = mfma32(ring[p % kRing], kop[p], s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The position bias: see alibi_addend (here the lane is the key).
      const float sl2 = slope_of(it);
      const float kstep = sl2 * (float)(key - r0);
      const float rbase = (float)(r0 + 4 * hh - key);
      auto lse4 = [&](int g4) { return *reinterpret_cast<const f32x4*>(sL + 8 * g4 + 4 * hh); };
      f32x4 L4 = lse4(0);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int p = NC + cc;
        if (p + kAh < 2 * NC) ring[(p + kAh) % kRing] = rowread(p + kAh);
        dp = mfma32(ring[p % kRing], vop[cc], dp);
        const int g4 = cc >> 2, e = cc & 3;
        if (e == 0 && g4 > 0) L4 = lse4(g4);
        const float xr = AL == 1 ? kstep - L4[e]
                                 : alibi_addend<AL>(sl2, rbase, (float)(8 * g4 + e), L4[e]);
        s[cc] = fast_exp2(fmaf(s[cc], c, xr));
        __builtin_amdgcn_sched_barrier(0);
      }
      // A operands of the dV / dK products: product j = 8 k + dt (key-row half k, head-dim
      // tile dt) of dV, then the same of dK; the 8 rows of a k-step are contiguous in the
      // transposed tiles.
      auto aread = [&](int j) {
        const bf16_t* base = j < 2 * NDH ? sOT : sQT;
        const int jj = j % (2 * NDH);
        return lds_read_b128(base + (32 * (jj % NDH) + l32) * TSTR + 8 * hh + 16 * (jj / NDH));
      };
#pragma unroll
      for (int i = 0; i < kAh; ++i) ring[i] = aread(i);
      const bool need_mask = (kw0 + 32 > N) | ((causal != 0) & (kw0 + 31 > r0)) |
                             ((window > 0) & (kw0 < r0 + BQ - window));
      if (need_mask) {  // masked weights 0 (selects under a wave-uniform branch)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + (r >> 2) * 8 + hh * 4 + (r & 3);
          const bool ok = (key < N) & (!causal | (key <= row)) &
                          ((window <= 0) | (key >= row - window + 1));
          s[r] = ok ? s[r] : 0.f;
        }
      }
      // P and dS as bf16 B operands (k = query row): pP[k] / pS[k] hold elements 8k .. 8k + 7.
      bf16x8 pP[2], pS[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const bf16x2 p01 = to_bf16x2(s[r], s[r + 1]);
        pP[r >> 3][r & 7] = p01[0];
        pP[r >> 3][(r & 7) + 1] = p01[1];
      }
      operand_ready(pP[0]);
      operand_ready(pP[1]);
#pragma unroll
      for (int j = 0; j < 2 * NDH; ++j) {
        if (j + kAh < 4 * NDH) ring[(j + kAh) % kRing] = aread(j + kAh);
        mfma_acc(dv[j % NDH], ring[j % kRing], pP[j / NDH]);
        if (j < kStoreParts) swrite_part(buf ^ 1, it + 1, j);
        if (j % 2 == 1) {  // dS of elements j - 1, j
          const bf16x2 d01 = to_bf16x2(s[j - 1] * dp[j - 1], s[j] * dp[j]);
          pS[j >> 3][(j - 1) & 7] = d01[0];
          pS[j >> 3][j & 7] = d01[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      operand_ready(pS[0]);
      operand_ready(pS[1]);
#pragma unroll
      for (int j = 2 * NDH; j < 4 * NDH; ++j) {
        if (j + kAh < 4 * NDH) ring[(j + kAh) % kRing] = aread(j + kAh);
        mfma_acc(dk[j % NDH], ring[j % kRing], pS[(j - 2 * NDH) / NDH]);
        if (j - 2 * NDH < 2 * kLoadParts && j % 2 == 0) gload_part(itl, (j - 2 * NDH) / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!active) {
#pragma unroll
      for (int part = 0; part < kStoreParts; ++part) swrite_part(buf ^ 1, it + 1, part);
#pragma unroll
      for (int part = 0; part < kLoadParts; ++part) gload_part(itl, part);
    }
    __syncthreads();
  }

  acc_ready(dk);
  acc_ready(dv);
  if (key < N) {
    bf16_t* dkr = dK + ((size_t)seq0 + key) * ks + (size_t)hkv * D;
    bf16_t* dvr = dV + ((size_t)seq0 + key) * ks + (size_t)hkv * D;
#pragma unroll
    for (int dt = 0; dt < NDH; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hh;
        uint2 u;
        u.x = pack_bf16(dk[dt][4 * g4] * scale, dk[dt][4 * g4 + 1] * scale);
        u.y = pack_bf16(dk[dt][4 * g4 + 2] * scale, dk[dt][4 * g4 + 3] * scale);
        *reinterpret_cast<uint2*>(dkr + d) = u;
        u.x = pack_bf16(dv[dt][4 * g4], dv[dt][4 * g4 + 1]);
        u.y = pack_bf16(dv[dt][4 * g4 + 2], dv[dt][4 * g4 + 3]);
        *reinterpret_cast<uint2*>(dvr + d) = u;
      }
    }
  }
}

// =====================================================================================
// dK / dV for d <= 128: 8 waves x 32 keys = 256 keys per workgroup, two waves per SIMD.
// Only K stays in VGPRs (B operand of S); V^T for dP is read from an LDS copy of the
// workgroup's V block, which frees the registers a second wave per SIMD needs, so one
// wave's exp / dS arithmetic overlaps the other wave's MFMAs.  The Q / dO staging of a
// 32-row step is shared by all 8 waves.
template <int D>
struct KV8Cfg {
  static constexpr int NW = 8, NT = 512;
  static constexpr int BKN = 256;         // keys per workgroup
  static constexpr int BQ = 32;           // query rows per step
  static constexpr int STR = D + 8;       // row-major V / Q / dO row stride (elements)
  static constexpr int TSTR = BQ + 8;     // transposed Q^T / dO^T row stride
  static constexpr int SV = BKN * STR;
  static constexpr int SQ = BQ * STR;
  static constexpr int SQT = D * TSTR;
  static constexpr int BUF = 2 * SQ + 2 * SQT;         // Q, dO, Q^T, dO^T (elements)
  static constexpr int BUFB = BUF * 2 + 2 * BQ * 4;    // + LSE, D (bytes)
  static constexpr int LDS_BYTES = SV * 2 + 2 * BUFB;  // V block + double-buffered staging
};

template <int D, int AL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv8_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int B, int Hq, int Hkv, int Nmax,
    int causal, int window, float c, float scale, const int* __restrict__ cu, int ntot,
    const float* __restrict__ slopes) {
  using Cfg = KV8Cfg<D>;
  constexpr int NT = Cfg::NT, BKN = Cfg::BKN, BQ = Cfg::BQ, STR = Cfg::STR, TSTR = Cfg::TSTR;
  constexpr int NC = D / 16, ND = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem);
  char* stage = smem + Cfg::SV * 2;

  const int num_kb = (Nmax + BKN - 1) / BKN;
  int b, hkv, rank;
  work_item(B, Hkv, num_kb, b, hkv, rank);
  int seq0, N;  // first row and length of this batch entry's sequence
  seq_span(cu, ntot, b, Nmax, seq0, N);
  const int kb = key_block(rank, num_kb, (N + BKN - 1) / BKN, causal, window);
  if (kb < 0 || kb * BKN >= N) return;  // no such block in a shorter packed sequence
  const int G = Hq / Hkv;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int n0 = kb * BKN, kw0 = n0 + 32 * w, key = kw0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Kb = K + ((size_t)seq0 * Hkv + hkv) * D;
  const bf16_t* Vb = V + ((size_t)seq0 * Hkv + hkv) * D;

  // K^T B operand of this lane's key; the whole V block into LDS (row-major).
  bf16x8 kop[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    kop[cc] = __builtin_bit_cast(
        bf16x8, key < N ? gload16(Kb + (size_t)key * ks + 16 * cc + 8 * hh) : make_uint4(0, 0, 0, 0));
  for (int ch = tid; ch < BKN * (D / 8); ch += NT) {
    const int kl = ch / (D / 8), dc = ch - kl * (D / 8);
    const int n = n0 + kl;
    *reinterpret_cast<uint4*>(sV + kl * STR + dc * 8) =
        n < N ? gload16(Vb + (size_t)n * ks + dc * 8) : make_uint4(0, 0, 0, 0);
  }

  const int qb_lo = causal ? n0 / BQ : 0;
  const int row_end = window > 0 ? min(N, n0 + BKN + window - 1) : N;
  const int qb_hi = (row_end + BQ - 1) / BQ;
  const int nq = max(0, qb_hi - qb_lo);
  const int total_it = G * nq;
  // A step is (query block qi, query head g of the group), query-block major, so the
  // workgroups of one KV head that run together read the same Q / dO rows at about the same
  // time and share them in L2.  Causal blocks walk their query blocks from the last one
  // down: all start at the end of the sequence and stop at their own diagonal, instead of
  // each starting at a different row.  Steps advance by counting, not by dividing the step
  // index (a scalar division per use).
  struct Step {
    int g, qi;
  };
  auto adv = [&](Step st) { return st.g + 1 == G ? Step{0, st.qi + 1} : Step{st.g + 1, st.qi}; };
  auto qblock = [&](int qi) { return causal ? qb_hi - 1 - qi : qb_lo + qi; };
  // ALiBi slope (log2 units) of query head g of the group
  auto slope_of = [&](int g) { return AL != 0 ? slopes[hkv * G + g] * kLog2e : 0.f; };

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  // Staging tasks of a step: 2 rows x 8 dims each, [0, T2) of Q and [T2, 2 T2) of dO, one
  // per thread, so all eight waves share the staging; each is stored row-major and
  // transposed.  Lane bit 0 picks one of two chunks, the next bits the row pair: the 8
  // lanes the LDS writes per cycle of a 16-byte store (32 four-byte banks) then cover four
  // row pairs and two chunks, 32 distinct banks, where eight row pairs of one chunk (row
  // stride 4 dwords mod 32) put two lanes on every bank; the transposed 4-byte stores are
  // two-way either way (16 row pairs per transposed row, chunks 8 rows = 0 banks apart).
  constexpr int CPR = D / 8;
  constexpr int T2 = (BQ / 2) * CPR;
  static_assert(2 * T2 <= NT, "one staging task per thread");
  static_assert(T2 % 64 == 0, "Q and dO tasks fall on whole waves");
  // Which operand a wave stages is wave-uniform, so its buffer resource stays scalar.
  const bool stager = w < 2 * T2 / 64, iso = w >= T2 / 64;
  const int tt = iso ? tid - T2 : tid;
  const int rp = (tt >> 1) % (BQ / 2), dc = (tt & 1) + 2 * (tt / BQ);  // row pair, chunk
  // Every thread fetches the LSE / D value of row tid % BQ of the step, unconditionally and
  // unscaled: a load consumed only at the next step's LDS write must not sit on a branch
  // merge or feed arithmetic right away, or the wait for it lands right behind its issue.
  uint4 xr[2];
  float lraw = 0.f, draw = 0.f;
  auto gload = [&](Step st) {
    const int hq = hkv * G + st.g, r0 = qblock(st.qi) * BQ;
    if (stager) {
      const bf16_t* base = (iso ? dO : Q) + ((size_t)seq0 * Hq + hq) * D + (size_t)r0 * qs;
      const uint32_t bytes = (uint32_t)(N - r0) * (uint32_t)qs * 2u;  // rows past N read 0
      const rsrc_t res = make_rsrc(base, bytes);
      const uint32_t off = (uint32_t)(2 * rp * qs + 8 * dc) * 2u;
      xr[0] = bload16(res, off);
      xr[1] = bload16(res, off + (uint32_t)qs * 2u);
    }
    const size_t l0 = stat_base(cu, ntot, b, Hq, hq, Nmax, seq0) + r0;
    const uint32_t lbytes = (uint32_t)(N - r0) * 4u;
    const uint32_t loff = (uint32_t)(tid % BQ) * 4u;
    lraw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        make_rsrc(LSE + l0, lbytes), (int)loff, 0, 0));
    draw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        make_rsrc(Dv + l0, lbytes), (int)loff, 0, 0));
  };
  auto swrite = [&](int buf, Step st) {
    bf16_t* sQ = reinterpret_cast<bf16_t*>(stage + buf * Cfg::BUFB);
    bf16_t* sO = sQ + Cfg::SQ;
    bf16_t* sQT = sO + Cfg::SQ;
    bf16_t* sOT = sQT + Cfg::SQT;
    float* sL = reinterpret_cast<float*>(sOT + Cfg::SQT);
    if (stager) {
      bf16_t* rdst = (iso ? sO : sQ) + (2 * rp) * STR + 8 * dc;
      *reinterpret_cast<uint4*>(rdst) = xr[0];
      *reinterpret_cast<uint4*>(rdst + STR) = xr[1];
      // column 8 dc + j of the two rows -> one 32-bit word of transposed row 8 dc + j
      bf16_t* tdst = (iso ? sOT : sQT) + (8 * dc) * TSTR + tpos(2 * rp);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a0 = u4word(xr[0], m), a1 = u4word(xr[1], m);
        *reinterpret_cast<uint32_t*>(tdst + (2 * m) * TSTR) = pack_lo(a0, a1);
        *reinterpret_cast<uint32_t*>(tdst + (2 * m + 1) * TSTR) = pack_hi(a0, a1);
      }
    }
    if (tid < BQ) {
      const bool in = qblock(st.qi) * BQ + tid < N;
      // +inf -> P = 0 on padding rows.  Causal position bias: LSE + slope2 (row - r0) is
      // staged and slope2 (key - r0) added per lane, both small near the diagonal.
      sL[tid] = in ? lraw * kLog2e + (AL == 1 ? slope_of(st.g) * tid : 0.f) : INFINITY;
      sL[BQ + tid] = in ? -draw : 0.f;  // -D: the dP accumulator starts from it
    }
  };

  Step cur{0, 0};
  Step nxt = adv(cur), far = adv(nxt);  // steps it, it + 1, it + 2
  if (total_it > 0) {
    gload(cur);
    swrite(0, cur);
    if (total_it > 1) gload(nxt);
  }
  __syncthreads();
  const bf16_t* vp = sV + (32 * w + l32) * STR + 8 * hh;  // V^T B operand rows of this wave
  for (int it = 0; it < total_it; ++it) {
    const int buf = it & 1;
    const bf16_t* sQ = reinterpret_cast<const bf16_t*>(stage + buf * Cfg::BUFB);
    const bf16_t* sO = sQ + Cfg::SQ;
    const bf16_t* sQT = sO + Cfg::SQ;
    const bf16_t* sOT = sQT + Cfg::SQT;
    const float* sL = reinterpret_cast<const float*>(sOT + Cfg::SQT);
    const float* sD = sL + BQ;
    const int r0 = qblock(cur.qi) * BQ;
    const bool active = kw0 < N && (!causal || r0 + BQ - 1 >= kw0) &&
                        (window <= 0 || r0 <= kw0 + 31 + window - 1);
    if (active) {
      // S = Q K^T and dP = dO V^T (lane = key, the step's 32 rows in registers).
      const bf16_t* qa = sQ + l32 * STR + 8 * hh;
      const bf16_t* oa = sO + l32 * STR + 8 * hh;
      // The operands of k-step cc + 1 are read while k-step cc's products issue (two named
      // buffers); the scheduling barrier after each k-step keeps later reads from being
      // hoisted further, which would need more registers than two waves per SIMD leave.
      // dP - D comes straight out of the products: the accumulator starts at -D of its rows.
      f32x16 s = zero16(), dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nd4 = *reinterpret_cast<const f32x4*>(sD + 8 * g4 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * g4 + e] = nd4[e];
      }
      bf16x8 opq[2], opo[2], opv[2];
      opq[0] = lds_read_b128(qa);
      opo[0] = lds_read_b128(oa);
      opv[0] = lds_read_b128(vp);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int cb = cc & 1;
        if (cc + 1 < NC) {
          opq[cb ^ 1] = lds_read_b128(qa + 16 * (cc + 1));
          opo[cb ^ 1] = lds_read_b128(oa + 16 * (cc + 1));
          opv[cb ^ 1] = lds_read_b128(vp + 16 * (cc + 1));
        }
        s = mfma32(opq[cb], kop[cc], s);
        dp = mfma32(opo[cb], opv[cb], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // P = exp2(S c + bias - LSE log2 e), masked entries 0; dS = P (dP - D).  The position
      // bias: see alibi_addend (here the lane is the key).
      float pv[16];
      const float sl2 = slope_of(cur.g);
      const float kstep = sl2 * (float)(key - r0);
      const float rbase = (float)(r0 + 4 * hh - key);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 L4 = *reinterpret_cast<const f32x4*>(sL + 8 * g4 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xr = AL == 1 ? kstep - L4[e]
                                   : alibi_addend<AL>(sl2, rbase, (float)(8 * g4 + e), L4[e]);
          pv[4 * g4 + e] = fast_exp2(fmaf(s[4 * g4 + e], c, xr));
        }
      }
      const bool need_mask = (kw0 + 32 > N) | ((causal != 0) & (kw0 + 31 > r0)) |
                             ((window > 0) & (kw0 < r0 + BQ - window));
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + (r >> 2) * 8 + hh * 4 + (r & 3);
          const bool ok = (key < N) & (!causal | (key <= row)) &
                          ((window <= 0) | (key >= row - window + 1));
          pv[r] = ok ? pv[r] : 0.f;
        }
      }
      // A operands of the dV / dK products (rows of the transposed dO and Q tiles), head-dim
      // tile dt into one of two named buffers.  Tile 0 is read here, so its latency hides
      // behind the elementwise work below; tile dt + 1 while tile dt's products issue.
      bf16x8 ao[2][2], aq[2][2];
      auto ld_dt = [&](int dt, bf16x8 (&o2)[2], bf16x8 (&q2)[2]) {
        const bf16_t* ot = sOT + (32 * dt + l32) * TSTR + 8 * hh;
        const bf16_t* qt = sQT + (32 * dt + l32) * TSTR + 8 * hh;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          o2[c2] = lds_read_b128(ot + 16 * c2);
          q2[c2] = lds_read_b128(qt + 16 * c2);
        }
      };
      ld_dt(0, ao[0], aq[0]);
      bf16x8 pP[2], pS[2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dsv[e] = pv[4 * g4 + e] * dp[4 * g4 + e];
        const int c2 = g4 >> 1, i0 = 4 * (g4 & 1);
        const bf16x2 p01 = to_bf16x2(pv[4 * g4], pv[4 * g4 + 1]);
        const bf16x2 p23 = to_bf16x2(pv[4 * g4 + 2], pv[4 * g4 + 3]);
        const bf16x2 d01 = to_bf16x2(dsv[0], dsv[1]), d23 = to_bf16x2(dsv[2], dsv[3]);
        pP[c2][i0] = p01[0];
        pP[c2][i0 + 1] = p01[1];
        pP[c2][i0 + 2] = p23[0];
        pP[c2][i0 + 3] = p23[1];
        pS[c2][i0] = d01[0];
        pS[c2][i0 + 1] = d01[1];
        pS[c2][i0 + 2] = d23[0];
        pS[c2][i0 + 3] = d23[1];
      }
      // dV^T += dO^T P and dK^T += Q^T dS.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int cb = dt & 1;
        if (dt + 1 < ND) ld_dt(dt + 1, ao[cb ^ 1], aq[cb ^ 1]);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          dv[dt] = mfma32(ao[cb][c2], pP[c2], dv[dt]);
          dk[dt] = mfma32(aq[cb][c2], pS[c2], dk[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (it + 1 < total_it) {
      swrite(buf ^ 1, nxt);
      if (it + 2 < total_it) gload(far);
    }
    __syncthreads();
    cur = nxt;
    nxt = far;
    far = adv(far);
  }

  if (key < N) {
    bf16_t* dkr = dK + ((size_t)seq0 + key) * ks + (size_t)hkv * D;
    bf16_t* dvr = dV + ((size_t)seq0 + key) * ks + (size_t)hkv * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hh;
        uint2 u;
        u.x = pack_bf16(dk[dt][4 * g4] * scale, dk[dt][4 * g4 + 1] * scale);
        u.y = pack_bf16(dk[dt][4 * g4 + 2] * scale, dk[dt][4 * g4 + 3] * scale);
        *reinterpret_cast<uint2*>(dkr + d) = u;
        u.x = pack_bf16(dv[dt][4 * g4], dv[dt][4 * g4 + 1]);
        u.y = pack_bf16(dv[dt][4 * g4 + 2], dv[dt][4 * g4 + 3]);
        *reinterpret_cast<uint2*>(dvr + d) = u;
      }
    }
  }
}

// =====================================================================================
// dQ
template <int D>
struct QCfg {
  static constexpr int NW = D <= 128 ? 8 : 4;   // waves per workgroup (32 rows each)
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = D <= 128 ? 64 : 32;  // keys staged per iteration
  static constexpr int KSTR = D + 8;             // row-major K / V row stride
  static constexpr int TSTR = BN + 8;            // K^T row stride
  static constexpr int SK = BN * KSTR;
  static constexpr int SKT = D * TSTR;
  static constexpr int BUF = 2 * SK + SKT;       // K, V, K^T (elements)
  static constexpr int LDS_BYTES = 2 * BUF * 2;  // double buffered
};

template <int D, int AL>
__global__ __launch_bounds__(QCfg<D>::NT, 1) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dQ, int B, int Hq, int Hkv, int Nmax, int causal, int window, float c,
    float scale, const int* __restrict__ cu, int ntot, const float* __restrict__ slopes) {
  using Cfg = QCfg<D>;
  constexpr int NT = Cfg::NT, BM = Cfg::BM, BN = Cfg::BN, KSTR = Cfg::KSTR, TSTR = Cfg::TSTR;
  constexpr int NC = D / 16, ND = D / 32;
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

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const int m0 = mb * BM;
  const int wr0 = m0 + w * 32;
  const int row = wr0 + l32;

  const size_t qs = (size_t)Hq * D, ks = (size_t)Hkv * D;
  const bf16_t* Qh = Q + ((size_t)seq0 * Hq + hq) * D;
  const bf16_t* Oh = dO + ((size_t)seq0 * Hq + hq) * D;
  const bf16_t* Kh = K + ((size_t)seq0 * Hkv + hkv) * D;
  const bf16_t* Vh = V + ((size_t)seq0 * Hkv + hkv) * D;

  // B operands: this lane's rows of Q and dO.
  bf16x8 qop[NC], oop[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    qop[cc] = __builtin_bit_cast(bf16x8, row < N ? gload16(Qh + (size_t)row * qs + 16 * cc + 8 * hh) : z);
    oop[cc] = __builtin_bit_cast(bf16x8, row < N ? gload16(Oh + (size_t)row * qs + 16 * cc + 8 * hh) : z);
  }
  const size_t li = stat_base(cu, ntot, b, Hq, hq, Nmax, seq0) + row;
  const float lse2 = row < N ? LSE[li] * kLog2e : INFINITY;  // +inf -> P = 0 on padding rows
  const float ndval = row < N ? -Dv[li] : 0.f;  // -D of this lane's row
  const float slope2 = AL != 0 ? slopes[hq] * kLog2e : 0.f;

  int kv_lo = 0, kv_hi = N;
  if (causal) kv_hi = min(N, m0 + BM);
  if (window > 0) kv_lo = max(0, m0 - window + 1);
  const int nb_lo = kv_lo / BN, nb_hi = (kv_hi + BN - 1) / BN;
  const int klo = window > 0 ? row - window + 1 : 0;  // allowed keys of this row: [klo, khi]
  const int khi = causal ? min(row, N - 1) : N - 1;

  // Staging.  d <= 128: every thread takes one 2-key x 8-dim task of K (stored row-major
  // and transposed) and the same task of V (row-major), so the work is even over the
  // waves.  Lane bit 0 picks one of two chunks, the next bits the key pair: the 8 lanes the
  // LDS writes per cycle of a 16-byte store (32 four-byte banks) then cover four key pairs
  // and two chunks, 32 distinct banks (eight key pairs of one chunk would put two lanes on
  // every bank), at the price of two-way 4-byte K^T stores (16 key pairs per cycle instead
  // of 32); the row-major stores are four per task, the transposed ones eight 4-byte ones.
  // d = 256: 4-key x 8-dim tasks, [0, TK) of K and [TK, 2 TK) of V.
  constexpr int CPR = D / 8;
  constexpr bool kPairs = D <= 128;
  constexpr int TP = (BN / 2) * CPR;  // 2-key tasks per operand
  static_assert(!kPairs || TP <= NT, "one 2-key task of K and of V per thread");
  constexpr int TK = (BN / 4) * CPR;
  static_assert(BN % 16 == 0 && CPR % 4 == 0, "task_rc4 needs whole groups of 16 rows and 4 chunks");
  constexpr int PT = kPairs ? 1 : (2 * TK + NT - 1) / NT;
  static_assert(kPairs || TK % 64 == 0, "K and V tasks fall on whole waves");
  uint4 xr[PT][4];
  const int kp_ = (tid >> 1) % (BN / 2), dcp = (tid & 1) + 2 * (tid / BN);  // key pair, chunk
  const bool ptask = TP == NT || tid < TP;
  auto gload = [&](int nb) {
    const uint32_t bytes = (uint32_t)(N - nb * BN) * (uint32_t)ks * 2u;  // rows past N read 0
    if constexpr (kPairs) {
      if (ptask) {
        const rsrc_t kres = make_rsrc(Kh + (size_t)nb * BN * ks, bytes);
        const rsrc_t vres = make_rsrc(Vh + (size_t)nb * BN * ks, bytes);
        const uint32_t off = (uint32_t)(2 * kp_ * ks + 8 * dcp) * 2u;
        xr[0][0] = bload16(kres, off);
        xr[0][1] = bload16(kres, off + (uint32_t)ks * 2u);
        xr[0][2] = bload16(vres, off);
        xr[0][3] = bload16(vres, off + (uint32_t)ks * 2u);
      }
    } else {
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        const int task = tid + NT * p;
        const int wtask = 64 * w + NT * p;  // first task of this wave: wave-uniform
        if ((2 * TK) % NT == 0 || wtask < 2 * TK) {
          const bool isv = wtask >= TK;  // wave-uniform, keeps the buffer resource scalar
          const int t = isv ? task - TK : task;
          int kg, dc;
          task_rc4<CPR>(t, kg, dc);
          const rsrc_t res = make_rsrc((isv ? Vh : Kh) + (size_t)nb * BN * ks, bytes);
          bload_4x8(xr[p], res, (uint32_t)(4 * kg * ks + 8 * dc) * 2u, (uint32_t)ks * 2u);
        }
      }
    }
  };
  auto swrite = [&](int buf) {
    bf16_t* sK = lds + buf * Cfg::BUF;
    bf16_t* sV = sK + Cfg::SK;
    bf16_t* sKT = sV + Cfg::SK;
    if constexpr (kPairs) {
      if (ptask) {
        bf16_t* kdst = sK + (2 * kp_) * KSTR + 8 * dcp;
        bf16_t* vdst = sV + (2 * kp_) * KSTR + 8 * dcp;
        *reinterpret_cast<uint4*>(kdst) = xr[0][0];
        *reinterpret_cast<uint4*>(kdst + KSTR) = xr[0][1];
        *reinterpret_cast<uint4*>(vdst) = xr[0][2];
        *reinterpret_cast<uint4*>(vdst + KSTR) = xr[0][3];
        // column 8 dcp + j of the two keys -> one 32-bit word of K^T row 8 dcp + j
        bf16_t* tdst = sKT + (8 * dcp) * TSTR + tpos(2 * kp_);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a0 = u4word(xr[0][0], m), a1 = u4word(xr[0][1], m);
          *reinterpret_cast<uint32_t*>(tdst + (2 * m) * TSTR) = pack_lo(a0, a1);
          *reinterpret_cast<uint32_t*>(tdst + (2 * m + 1) * TSTR) = pack_hi(a0, a1);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        const int task = tid + NT * p;
        if ((2 * TK) % NT == 0 || task < 2 * TK) {
          const bool isv = task >= TK;
          const int t = isv ? task - TK : task;
          int kg, dc;
          task_rc4<CPR>(t, kg, dc);
          if (isv) {
            store_4x8_rows(sV, KSTR, 4 * kg, 8 * dc, xr[p]);
          } else {
            store_4x8_rows(sK, KSTR, 4 * kg, 8 * dc, xr[p]);
            store_4x8_transposed(sKT, TSTR, 4 * kg, 8 * dc, xr[p]);
          }
        }
      }
    }
  };

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();

  if (nb_lo < nb_hi) {
    gload(nb_lo);
    swrite(0);
    if (nb_lo + 1 < nb_hi) gload(nb_lo + 1);
  }
  __syncthreads();
  for (int nb = nb_lo; nb < nb_hi; ++nb) {
    const int buf = (nb - nb_lo) & 1;
    const bf16_t* sK = lds + buf * Cfg::BUF;
    const bf16_t* sV = sK + Cfg::SK;
    const bf16_t* sKT = sV + Cfg::SK;
    const int n0 = nb * BN;
    const bool active = wr0 < N && (!causal || n0 <= wr0 + 31) &&
                        (window <= 0 || n0 + BN - 1 >= wr0 - window + 1);
    if (active) {
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
        const int k0 = n0 + 32 * kt;
        if (causal && k0 > wr0 + 31) break;  // piece entirely above the diagonal
        // S^T = K Q^T and dP^T = V dO^T: keys k0 + [0, 32) x this wave's rows.
        const bf16_t* kp = sK + (32 * kt + l32) * KSTR + 8 * hh;
        const bf16_t* vp = sV + (32 * kt + l32) * KSTR + 8 * hh;
        if constexpr (D <= 128) {
          // The operands of k-step cc + 1 are read while k-step cc's products issue (two
          // named buffers, a scheduling barrier per step), as in the key-block kernel.
          // dP^T - D comes straight out of the products: the accumulator starts at -D.
          f32x16 s = zero16(), dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = ndval;
          bf16x8 ok[2], ov[2];
          ok[0] = lds_read_b128(kp);
          ov[0] = lds_read_b128(vp);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) {
            const int cb = cc & 1;
            if (cc + 1 < NC) {
              ok[cb ^ 1] = lds_read_b128(kp + 16 * (cc + 1));
              ov[cb ^ 1] = lds_read_b128(vp + 16 * (cc + 1));
            }
            s = mfma32(ok[cb], qop[cc], s);
            dp = mfma32(ov[cb], oop[cc], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
          const bf16_t* tp = sKT + l32 * TSTR + 8 * hh + 32 * kt;
          // K^T operand j = 2 dt + c2 (head-dim tile dt, key half c2)
          bf16x8 ta[2 * ND];
#pragma unroll
          for (int j = 0; j < 2 * ND; ++j)
            ta[j] = lds_read_b128(tp + 32 * (j >> 1) * TSTR + 16 * (j & 1));
          // P^T = exp2(S^T c - LSE log2 e); dS^T = P^T (dP^T - D); masked entries 0.
          float p[16];
          {  // position bias: see alibi_addend (key - row of element 0 is k0 + 4 hh - row)
            const float dbase = AL != 0 ? (float)(k0 + 4 * hh - row) : 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              p[r] = fast_exp2(fmaf(s[r], c, alibi_addend<AL>(slope2, dbase,
                                                              (float)(8 * (r >> 2) + (r & 3)), lse2)));
          }
          // Bitwise (branch-free) without a position bias; with one, the short-circuit form,
          // which here leaves the register allocation without spills.
          const bool need_mask =
              AL == 0 ? (k0 + 32 > N) | ((causal != 0) & (k0 + 31 > wr0)) |
                            ((window > 0) & (k0 < wr0 + 32 - window))
                      : (k0 + 32 > N) || (causal && k0 + 31 > wr0) ||
                            (window > 0 && k0 < wr0 + 32 - window);
          if (need_mask) {
            const int kb0 = k0 + hh * 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kk = kb0 + (r >> 2) * 8 + (r & 3);
              p[r] = ((kk >= klo) & (kk <= khi)) ? p[r] : 0.f;
            }
          }
          bf16x8 pS[2];
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const bf16x2 d2 = to_bf16x2(p[r] * dp[r], p[r + 1] * dp[r + 1]);
            pS[r >> 3][r & 7] = d2[0];
            pS[r >> 3][(r & 7) + 1] = d2[1];
          }
          // dQ^T += K^T dS^T
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int j = 0; j < 2 * ND; ++j) acc[j >> 1] = mfma32(ta[j], pS[j & 1], acc[j >> 1]);
          __builtin_amdgcn_s_setprio(0);
        } else {
          // d = 256 (one wave per SIMD): the S^T products, then the dP^T products with one
          // weight P^T = exp2(S^T c - LSE log2 e) after each, then the dQ^T products with the
          // second key half's dS^T between the first half's products.  The K / V / K^T
          // operands stream through one ring of kRing registers read kAh products ahead,
          // which leaves the Q and dO operands their VGPRs.  dP^T - D comes straight out of
          // the products: the accumulator starts at -D.
          constexpr int kRing = 4, kAh = 3;
          f32x16 s = zero16(), dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = ndval;
          // position bias: see alibi_addend (key - row of element 0 is k0 + 4 hh - row)
          const float dbase = AL != 0 ? (float)(k0 + 4 * hh - row) : 0.f;
          auto opread = [&](int q) { return lds_read_b128((q < NC ? kp : vp) + 16 * (q % NC)); };
          float p[16];
          bf16x8 ring[kRing];
#pragma unroll
          for (int i = 0; i < kAh; ++i) ring[i] = opread(i);
#pragma unroll
          for (int q = 0; q < 2 * NC; ++q) {
            if (q + kAh < 2 * NC) ring[(q + kAh) % kRing] = opread(q + kAh);
            if (q < NC) {
              s = mfma32(ring[q % kRing], qop[q], s);
            } else {
              const int r = q - NC;
              dp = mfma32(ring[q % kRing], oop[r], dp);
              p[r] = fast_exp2(fmaf(s[r], c, alibi_addend<AL>(slope2, dbase,
                                                              (float)(8 * (r >> 2) + (r & 3)), lse2)));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          // K^T operand of dQ^T product j: head-dim tile j % ND, key half j / ND
          const bf16_t* tp = sKT + l32 * TSTR + 8 * hh + 32 * kt;
          auto tread = [&](int j) {
            return lds_read_b128(tp + 32 * (j % ND) * TSTR + 16 * (j / ND));
          };
#pragma unroll
          for (int i = 0; i < kAh; ++i) ring[i] = tread(i);
          // masked entries 0 (the branch-free condition without a position bias, the
          // short-circuit one with it, as above)
          const bool need_mask =
              AL == 0 ? (k0 + 32 > N) | ((causal != 0) & (k0 + 31 > wr0)) |
                            ((window > 0) & (k0 < wr0 + 32 - window))
                      : (k0 + 32 > N) || (causal && k0 + 31 > wr0) ||
                            (window > 0 && k0 < wr0 + 32 - window);
          if (need_mask) {
            const int kb0 = k0 + hh * 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kk = kb0 + (r >> 2) * 8 + (r & 3);
              p[r] = ((kk >= klo) & (kk <= khi)) ? p[r] : 0.f;
            }
          }
          // dS^T = P^T (dP^T - D) as the bf16 B operand, elements r and r + 1
          bf16x8 pS[2];
          auto ds_pair = [&](int r) {
            const bf16x2 d2 = to_bf16x2(p[r] * dp[r], p[r + 1] * dp[r + 1]);
            pS[r >> 3][r & 7] = d2[0];
            pS[r >> 3][(r & 7) + 1] = d2[1];
          };
#pragma unroll
          for (int r = 0; r < 8; r += 2) ds_pair(r);
          // dQ^T += K^T dS^T
#pragma unroll
          for (int j = 0; j < 2 * ND; ++j) {
            if (j + kAh < 2 * ND) ring[(j + kAh) % kRing] = tread(j + kAh);
            acc[j % ND] = mfma32(ring[j % kRing], pS[j / ND], acc[j % ND]);
            if (j < 8 && (j & 1) == 0) ds_pair(8 + j);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    if (nb + 1 < nb_hi) {
      swrite(buf ^ 1);
      if (nb + 2 < nb_hi) gload(nb + 2);
    }
    __syncthreads();
  }

  if (row < N) {
    bf16_t* qrow = dQ + ((size_t)seq0 + row) * qs + (size_t)hq * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 u;
        u.x = pack_bf16(acc[dt][4 * g4] * scale, acc[dt][4 * g4 + 1] * scale);
        u.y = pack_bf16(acc[dt][4 * g4 + 2] * scale, acc[dt][4 * g4 + 3] * scale);
        *reinterpret_cast<uint2*>(qrow + 32 * dt + 8 * g4 + 4 * hh) = u;
      }
    }
  }
}

// =====================================================================================
template <int D, int AL>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  using KC = KVCfg<D>;
  using K8 = KV8Cfg<D <= 128 ? D : 128>;
  using QC = QCfg<D>;
  constexpr bool kWide = D <= 128;  // 8-wave key-block kernel
  // Dynamic LDS limits, set once (a function-local static: the first call is thread-safe).
  static const hipError_t attr = [] {
    hipError_t e;
    if constexpr (kWide)
      e = hipFuncSetAttribute((const void*)bwd_dkdv8_kernel<D, AL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, K8::LDS_BYTES);
    else
      e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<D, AL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, KC::LDS_BYTES);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)bwd_dq_kernel<D, AL>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, QC::LDS_BYTES);
  }();
  if (attr != hipSuccess) return attr;
  const long rows = a.cu ? (long)a.ntot * a.Hq : (long)a.B * a.N * a.Hq;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     st, (const bf16_t*)a.o, (const bf16_t*)a.dO, a.dvec, a.B, a.Hq, a.N, a.cu,
                     a.ntot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_start) {
    e = hipEventRecord(a.ev_start, st);
    if (e != hipSuccess) return e;
  }
  if constexpr (kWide) {
    constexpr int DW = D <= 128 ? D : 128;
    const int num_kb = (a.N + K8::BKN - 1) / K8::BKN;
    hipLaunchKernelGGL((bwd_dkdv8_kernel<DW, AL>), dim3(a.B * a.Hkv * num_kb), dim3(K8::NT),
                       K8::LDS_BYTES, st, (const bf16_t*)a.q, (const bf16_t*)a.k,
                       (const bf16_t*)a.v, (const bf16_t*)a.dO, a.lse, a.dvec, (bf16_t*)a.dk,
                       (bf16_t*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window,
                       a.c_log2_signed, a.scale, a.cu, a.ntot, a.slopes);
  } else {
    const int num_kb = (a.N + KC::BKN - 1) / KC::BKN;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, AL>), dim3(a.B * a.Hkv * num_kb),
                       dim3(KC::NT), KC::LDS_BYTES, st, (const bf16_t*)a.q, (const bf16_t*)a.k,
                       (const bf16_t*)a.v, (const bf16_t*)a.dO, a.lse, a.dvec, (bf16_t*)a.dk,
                       (bf16_t*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.causal, a.window,
                       a.c_log2_signed, a.scale, a.cu, a.ntot, a.slopes);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_stop) {
    e = hipEventRecord(a.ev_stop, st);
    if (e != hipSuccess) return e;
  }
  const int num_m = (a.N + QC::BM - 1) / QC::BM;
  hipLaunchKernelGGL((bwd_dq_kernel<D, AL>), dim3(a.B * a.Hq * num_m), dim3(QC::NT), QC::LDS_BYTES, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
                     (const bf16_t*)a.dO, a.lse, a.dvec, (bf16_t*)a.dq, a.B, a.Hq, a.Hkv, a.N,
                     a.causal, a.window, a.c_log2_signed, a.scale, a.cu, a.ntot, a.slopes);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_al(const BwdArgs& a, hipStream_t st) {
  if (a.slopes == nullptr) return launch_bwd_d<D, 0>(a, st);
  return a.causal ? launch_bwd_d<D, 1>(a, st) : launch_bwd_d<D, 2>(a, st);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: return launch_bwd_al<64>(a, st);
    case 128: return launch_bwd_al<128>(a, st);
    case 256: return launch_bwd_al<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
