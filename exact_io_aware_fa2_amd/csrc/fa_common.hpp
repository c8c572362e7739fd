// fa_common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, wave64), checked on gfx950:
//   A operand (32 x 16, M x K): lane l holds A[l % 32][8 * (l / 32) + i], i = 0..7
//   B operand (16 x 32, K x N): lane l holds B[8 * (l / 32) + i][l % 32]
//   C/D (32 x 32 fp32):         lane l, element r holds
//                               C[(r / 4) * 8 + (l / 32) * 4 + (r % 4)][l % 32]
// Because the reduction index only has to agree between A and B, an accumulator C[m][n]
// can feed a later product directly as a B operand B[k = m][n] (the kernels pick the
// matching key/row order for the other operand).
//
// ds_read_b64_tr_b16 (gfx950): inside each group of 16 lanes, the four rows loaded by
// lanes 4r..4r+3 (four 16-bit values each) form a 4 x 16 block; lane j receives column j
// of it.  This turns a row-major [key][d] tile in LDS into the per-lane "8 keys at one d"
// operand that a product contracting over keys needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint16_t bf16_t;  // storage type of a bfloat16 in global memory

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Lazy reference maximum of the forward kernels.  A piece whose weights against the
// current reference would exceed kSumLimit = 2^12 (detected from a lane's partial sum, so
// the common path takes no row max at all) goes through the rescale path, which moves the
// reference only for rows whose piece maximum exceeds it by more than kRescaleThreshold
// log2 units.  Weights thus stay below 2^12 and the accumulator rescale (a multiply of
// every accumulator register) runs rarely.  Numerator and denominator always share the same
// reference maximum, so the normalised result is unchanged.
constexpr float kRescaleThreshold = 8.f;
constexpr float kSumLimit = 4096.f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Matrix products whose accumulators live in AGPRs.  The compiler gives a kernel either
// every product in the AGPR form or none, and the d = 256 kernels need their accumulators
// (dK/dV, or O) in AGPRs next to VGPR scores, so those products are inline assembly.  The
// compiler does not see them as matrix instructions: the wait states the hardware needs
// where vector instructions touch their registers are written out here.
// acc += a b (v_mfma_f32_32x32x16_bf16 with an AGPR accumulator).
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// After vector writes of accumulators, before a product reads them.
__device__ __forceinline__ void acc_written(f32x16 (&x)[8]) {
  asm volatile("s_nop 4"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]),
                 "+a"(x[6]), "+a"(x[7]));
}
// After the last product, before vector instructions read the accumulators (more wait
// states than a 32x32x16 product's latency).
__device__ __forceinline__ void acc_ready(f32x16 (&x)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]),
                 "+a"(x[6]), "+a"(x[7]));
}
// After vector writes of a product operand, before the products read it.
__device__ __forceinline__ void operand_ready(bf16x8& p) { asm volatile("s_nop 1" : "+v"(p)); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Two transposed 64-bit LDS reads -> one 8 x bf16 operand (elements 0..3 from p0,
// 4..7 from p1).  Pointers are generic pointers into __shared__ memory.
__device__ __forceinline__ bf16x8 lds_read_tr_x2(const void* p0, const void* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  bf16x8 r;
  bf16x4 ab = __builtin_bit_cast(bf16x4, a);
  bf16x4 bb = __builtin_bit_cast(bf16x4, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = ab[i];
    r[4 + i] = bb[i];
  }
  return r;
}

__device__ __forceinline__ bf16x8 lds_read_b128(const void* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ uint4 gload16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Raw buffer loads.  A buffer resource covers `bytes` bytes from `base`; a 16-byte load at
// an offset at or beyond that size returns zeros instead of touching memory, which pads a
// partial tile without per-lane tests.  The third descriptor dword selects the 32-bit data
// format that untyped buffer loads on this chip family expect.
constexpr int kBufferDword3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferDword3);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// Low (sel_lo) or high (sel_hi) 16-bit halves of two words packed into one word:
// pack_lo(a, b) = a[15:0] | b[15:0] << 16, pack_hi(a, b) = a[31:16] | b[31:16] << 16.
// One v_perm_b32 each (its second source supplies bytes 0-3, its first bytes 4-7).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Flip the sign bit of 8 packed bfloat16 values (exact negation).
__device__ __forceinline__ bf16x8 negate8(const bf16x8& x) {
  uint4 u = __builtin_bit_cast(uint4, x);
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

// Round-to-nearest-even float -> bfloat16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value over the two 32-lane halves of a wave (lanes l and l ^ 32), with
// one v_permlane32_swap: the two results hold the lower and the upper half in both halves.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row span of batch entry b.  Fixed-length batches (cu == nullptr) occupy rows
// b * nmax .. b * nmax + nmax - 1 of the tensors; packed sequences occupy rows
// cu[b] .. cu[b + 1] - 1, clamped to [0, ntot) and to at most nmax rows, so a malformed
// offset array can shorten a sequence but never move an access out of the tensors.
__device__ __forceinline__ void seq_span(const int* cu, int ntot, int b, int nmax, int& start,
                                         int& len) {
  if (cu == nullptr) {
    start = b * nmax;
    len = nmax;
    return;
  }
  const int s0 = min(max(cu[b], 0), ntot);
  const int s1 = min(max(cu[b + 1], s0), ntot);
  start = s0;
  len = min(s1 - s0, nmax);
}

// Offset of row 0 of (batch entry b, query head hq) in the float32 row statistics (LSE,
// D): [B, Hq, nmax] for fixed-length batches, [Hq, ntot] for packed sequences.
__device__ __forceinline__ size_t stat_base(const int* cu, int ntot, int b, int Hq, int hq,
                                            int nmax, int start) {
  return cu == nullptr ? ((size_t)b * Hq + hq) * nmax : (size_t)hq * ntot + start;
}

// Index of the calling wave inside its workgroup, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------------
// Tile staging.  A thread moves a 4-row x 8-column block of a row-major bf16 matrix (4
// global 16-byte loads) into LDS, either row-major (4 x 16-byte stores) or transposed
// (8 x 8-byte stores: column j of the block becomes a 4-element run of row j).  In the
// transposed copy the row index r of a 32-row slab is stored at tpos(r), with bits 2 and 3
// swapped: an MFMA accumulator holds rows (i / 4) * 8 + h * 4 + i % 4 (i = 0..7) in lane
// half h, so with this order the 8 rows one lane feeds to a product contracting over rows
// are contiguous and load as a single 16-byte read.
__device__ __forceinline__ int tpos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ uint32_t u4word(const uint4& u, int m) {
  return m == 0 ? u.x : m == 1 ? u.y : m == 2 ? u.z : u.w;
}

// Order of the (4-row group, 8-column chunk) staging tasks.  Four neighbouring lanes take
// four consecutive row groups of one column chunk, the next four lanes the next chunk:
// the 8-byte transposed stores of any 8 lanes then hit 64 distinct banks, and so do the
// 16-byte row-major stores (the plain group-major order leaves the transposed stores
// 4-way conflicted).  A wave still reads rows of up to 256 contiguous bytes from memory.
// A bijection on [0, (rows / 4) * CPR) when rows is a multiple of 16.
template <int CPR>
__device__ __forceinline__ void task_rc(int t, int& rg, int& dc) {
  const int q = t >> 2;
  dc = q % CPR;
  rg = (q / CPR) * 4 + (t & 3);
}

// x[e] = 16 bytes at byte offset off + e * row_bytes of a buffer resource (zeros past its
// end): row e of a 4 x 8 block when off addresses its first row.
__device__ __forceinline__ void bload_4x8(uint4 (&x)[4], rsrc_t res, uint32_t off,
                                          uint32_t row_bytes) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = bload16(res, off + e * row_bytes);
}

// Row-major store: LDS rows lr0 .. lr0 + 3, row stride s elements.
__device__ __forceinline__ void store_4x8_rows(bf16_t* lds, int s, int lr0, int c0,
                                               const uint4 (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(lds + (lr0 + e) * s + c0) = x[e];
}

// Transposed store: LDS row c0 + j (j = 0..7) gets the 4 values of column j at positions
// tpos(lr0) .. tpos(lr0) + 3 (lr0 a multiple of 4), row stride ts elements.  Part m writes
// columns 2m and 2m + 1.
__device__ __forceinline__ void store_4x8_transposed_part(bf16_t* lds, int ts, int lr0, int c0,
                                                          const uint4 (&x)[4], int m) {
  bf16_t* dst = lds + c0 * ts + tpos(lr0);
  const uint32_t a0 = u4word(x[0], m), a1 = u4word(x[1], m);
  const uint32_t a2 = u4word(x[2], m), a3 = u4word(x[3], m);
  uint2 even, odd;  // columns 2m and 2m + 1 of the four rows
  even.x = pack_lo(a0, a1);
  even.y = pack_lo(a2, a3);
  odd.x = pack_hi(a0, a1);
  odd.y = pack_hi(a2, a3);
  *reinterpret_cast<uint2*>(dst + (2 * m) * ts) = even;
  *reinterpret_cast<uint2*>(dst + (2 * m + 1) * ts) = odd;
}
__device__ __forceinline__ void store_4x8_transposed(bf16_t* lds, int ts, int lr0, int c0,
                                                     const uint4 (&x)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) store_4x8_transposed_part(lds, ts, lr0, c0, x, m);
}

// ALiBi position bias, in log2 units: the score of (row, key) gets -slope log2(e) |row - key|
// (bmjup.com, FAQ on inference: the alibi_slopes argument; hysenlabs.com, hardware-boundary
// section).  AL = 0: no bias.  AL = 1 (causal: every allowed key is at or before the row):
// the bias is linear in the key, slope2 (key - row), one FMA per score with the in-tile key
// offset as a literal.  AL = 2 (no causal mask): slope2 |key - row| needs the distance, one
// add and one FMA with an absolute-value operand.  `dbase` is key - row of the lane's
// element 0, `off` the element's key offset from it; the result is the exp2 addend
// bias - mref.  slope2 = slope * log2(e), any finite value.
template <int AL>
__device__ __forceinline__ float alibi_addend(float slope2, float dbase, float off, float mref) {
  if constexpr (AL == 0) {
    return -mref;
  } else if constexpr (AL == 1) {
    return fmaf(slope2, off, fmaf(slope2, dbase, -mref));
  } else {
    return fmaf(-slope2, fabsf(dbase + off), -mref);
  }
}

// Work order over (batch entry, head, block) triples; `rank` 0 is the heaviest block of a
// head.  Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  When
// H is a multiple of 8, XCD x owns the heads [x H/8, (x+1) H/8) of every batch entry (a GQA
// group, which shares K and V, stays on one L2) and runs its blocks rank-major: every owned
// head's heaviest block first, then the next rank.  Over the whole chip the heaviest blocks
// start first, which keeps the tail short, also when packed sequences of very different
// lengths make the batch entries unequal.  Other H: plain rank-major order.
__device__ __forceinline__ void work_item(int B, int H, int nblocks, int& b, int& h,
                                          int& rank) {
  constexpr int kXcd = 8;
  const int id = blockIdx.x;
  if (H % kXcd == 0) {
    const int hc = H / kXcd, hpx = B * hc;  // heads per XCD
    const int xcd = id % kXcd, slot = id / kXcd;
    rank = slot / hpx;
    const int j = slot - rank * hpx;
    b = j / hc;
    h = xcd * hc + (j - b * hc);
  } else {
    const int nh = B * H;
    rank = id / nh;
    const int head = id - rank * nh;
    b = head / H;
    h = head - b * H;
  }
}

}  // namespace fa
