/*
 * A plain C caller of libfa.so, built against include/fa.h by tests/test_abi.py.
 *
 * 1. The prototypes of the contract are written out below on their own, not taken from
 *    fa.h: each library function is assigned to a pointer of its contract type, so any
 *    difference in argument order or type between fa.h and the contract stops the build
 *    (the test compiles with -Werror=incompatible-pointer-types).
 * 2. main() calls every entry point with arguments the library must reject before it
 *    touches the GPU (null pointers, bad sizes, short or misaligned workspaces, NULL
 *    slopes for the position-bias variants) and checks the status and the message.
 *    Pointers are fake, aligned addresses that are never dereferenced.
 * Exit code 0 and the line "abi_caller ok" mean every check passed.
 */
#include <stdio.h>
#include <string.h>

#include "fa.h"

/* The contract: fa_fwd(q,k,v,o,lse,B,Hq,Hkv,N,d,causal,window,scale,stream) and
 * fa_bwd(q,k,v,o,dO,lse,dq,dk,dv,B,Hq,Hkv,N,d,causal,window,scale,workspace,
 * workspace_bytes,stream); the stream is a hipStream_t passed as a pointer. */
typedef fa_status (*fwd_fn)(const void*, const void*, const void*, void*, float*, int, int,
                            int, int, int, int, int, float, void*);
typedef fa_status (*fwd_fp32_fn)(const float*, const float*, const float*, float*, float*,
                                 int, int, int, int, int, int, int, float, void*);
typedef size_t (*ws_fn)(int, int, int, int, int, int, int);
typedef fa_status (*bwd_fn)(const void*, const void*, const void*, const void*, const void*,
                            const float*, void*, void*, void*, int, int, int, int, int, int,
                            int, float, void*, size_t, void*);
/* the position-bias variants: the slopes come right before the stream */
typedef fa_status (*fwd_alibi_fn)(const void*, const void*, const void*, void*, float*, int,
                                  int, int, int, int, int, int, float, const float*, void*);
typedef fa_status (*bwd_alibi_fn)(const void*, const void*, const void*, const void*,
                                  const void*, const float*, void*, void*, void*, int, int, int,
                                  int, int, int, int, float, void*, size_t, const float*,
                                  void*);
typedef fa_status (*fwd_varlen_fn)(const void*, const void*, const void*, void*, float*,
                                   const int*, int, int, int, int, int, int, int, int, float,
                                   void*);
typedef fa_status (*bwd_varlen_fn)(const void*, const void*, const void*, const void*,
                                   const void*, const float*, void*, void*, void*, const int*,
                                   int, int, int, int, int, int, int, int, float, void*, size_t,
                                   void*);
typedef fa_status (*fwd_varlen_alibi_fn)(const void*, const void*, const void*, void*, float*,
                                         const int*, int, int, int, int, int, int, int, int,
                                         float, const float*, void*);
typedef fa_status (*bwd_varlen_alibi_fn)(const void*, const void*, const void*, const void*,
                                         const void*, const float*, void*, void*, void*,
                                         const int*, int, int, int, int, int, int, int, int,
                                         float, void*, size_t, const float*, void*);
typedef fa_status (*fwd_fp8_fn)(const void*, const void*, const void*, void*, float*, float,
                                float, float, int, int, int, int, int, int, int, float, void*);
typedef fa_status (*decode_fn)(const void*, const void*, const void*, const int*, void*, float*,
                               int, int, int, int, int, int, int, int, float, int, void*,
                               size_t, void*);
typedef fa_status (*bwd_noalloc_fn)(const void*, const void*, const void*, const void*,
                                    const void*, const float*, void*, void*, void*, int, int,
                                    int, int, int, int, int, float, void*);
typedef fa_status (*mfma_probe_fn)(float*, int, int, void*);
typedef fa_status (*atomic_probe_fn)(float*, int, int, int, int, void*);
typedef fa_status (*issue_probe_fn)(float*, int, int, int, int, int, void*);
typedef fa_status (*fp8_product_probe_fn)(const void*, const void*, float*, int, void*);
typedef const char* (*str_fn)(void);

static const fwd_fn p_fwd = fa_fwd;
static const fwd_fp32_fn p_fwd_fp32 = fa_fwd_fp32;
static const ws_fn p_ws = fa_bwd_workspace_size;
static const bwd_fn p_bwd = fa_bwd;
static const fwd_alibi_fn p_fwd_alibi = fa_fwd_alibi;
static const bwd_alibi_fn p_bwd_alibi = fa_bwd_alibi;
static const fwd_varlen_fn p_fwd_varlen = fa_fwd_varlen;
static const bwd_varlen_fn p_bwd_varlen = fa_bwd_varlen;
static const fwd_varlen_alibi_fn p_fwd_varlen_alibi = fa_fwd_varlen_alibi;
static const bwd_varlen_alibi_fn p_bwd_varlen_alibi = fa_bwd_varlen_alibi;
static const fwd_fp8_fn p_fwd_fp8 = fa_fwd_fp8;
static const decode_fn p_decode = fa_decode;
static const bwd_noalloc_fn p_bwd_noalloc = fa_bwd_noalloc;
static const mfma_probe_fn p_mfma_probe = fa_mfma_probe;
static const atomic_probe_fn p_atomic_probe = fa_atomic_probe;
static const issue_probe_fn p_issue_probe = fa_issue_probe;
static const fp8_product_probe_fn p_fp8_probe = fa_fp8_product_probe;
static const str_fn p_err = fa_last_error;
static const str_fn p_ver = fa_version;

static int failures = 0;

static void expect(const char* what, fa_status got, fa_status want, const char* needle) {
  const char* msg = p_err();
  if (got != want || (needle && !strstr(msg, needle))) {
    printf("FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", what, (int)got,
           (int)want, msg, needle ? needle : "");
    ++failures;
  }
}

int main(void) {
  /* fake device addresses: aligned, never dereferenced (every call below fails validation) */
  void* const A = (void*)(size_t)4096;
  float* const F = (float*)(size_t)4096;
  int* const I = (int*)(size_t)4096;
  void* const S = NULL; /* the null stream */
  const size_t need = p_ws(1, 4, 2, 128, 128, 1, 0);

  if (strstr(p_ver(), "gfx950") == NULL) {
    printf("FAIL version \"%s\"\n", p_ver());
    ++failures;
  }
  if (need != 1 * 4 * 128 * 4) {
    printf("FAIL workspace size %zu\n", need);
    ++failures;
  }
  if (p_ws(1, 4, 3, 128, 128, 1, 0) != 0) {
    printf("FAIL workspace size for Hq %% Hkv != 0\n");
    ++failures;
  }

  expect("fwd null", p_fwd(NULL, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, 0.125f, S),
         FA_ERR_INVALID_ARG, "fa_fwd: null");
  expect("fwd B=0", p_fwd(A, A, A, A, F, 0, 2, 2, 16, 64, 0, 0, 0.125f, S),
         FA_ERR_INVALID_ARG, "fa_fwd");
  expect("fwd d=96", p_fwd(A, A, A, A, F, 1, 2, 2, 16, 96, 0, 0, 0.125f, S),
         FA_ERR_UNSUPPORTED, "head dim");
  expect("fwd window<0", p_fwd(A, A, A, A, F, 1, 2, 2, 16, 64, 1, -1, 0.125f, S),
         FA_ERR_INVALID_ARG, "window");
  expect("fwd Hq%Hkv", p_fwd(A, A, A, A, F, 1, 6, 4, 16, 64, 0, 0, 0.125f, S),
         FA_ERR_INVALID_ARG, "multiple");
  expect("fwd misaligned", p_fwd((char*)A + 8, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, 0.125f, S),
         FA_ERR_INVALID_ARG, "aligned");
  expect("fwd_fp32 null", p_fwd_fp32(F, F, NULL, F, F, 1, 2, 2, 16, 64, 0, 0, 0.125f, S),
         FA_ERR_INVALID_ARG, "fa_fwd_fp32: null");
  expect("fwd_alibi null slopes",
         p_fwd_alibi(A, A, A, A, F, 1, 2, 2, 16, 64, 1, 0, 0.125f, NULL, S),
         FA_ERR_INVALID_ARG, "alibi_slopes");
  expect("fwd_alibi misaligned slopes",
         p_fwd_alibi(A, A, A, A, F, 1, 2, 2, 16, 64, 1, 0, 0.125f, (const float*)((char*)F + 2),
                     S),
         FA_ERR_INVALID_ARG, "aligned");
  expect("fwd_fp8 factor", p_fwd_fp8(A, A, A, A, F, 0.f, 1.f, 1.f, 1, 2, 2, 16, 64, 0, 0,
                                     0.125f, S),
         FA_ERR_INVALID_ARG, "fa_fwd_fp8");

  expect("bwd short workspace",
         p_bwd(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, A, need - 1, S),
         FA_ERR_WORKSPACE, "fa_bwd: workspace");
  expect("bwd null workspace",
         p_bwd(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, NULL, need, S),
         FA_ERR_WORKSPACE, "fa_bwd");
  expect("bwd misaligned workspace",
         p_bwd(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, (char*)A + 16, need,
               S),
         FA_ERR_WORKSPACE, "256-byte");
  expect("bwd null dO",
         p_bwd(A, A, A, A, NULL, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, A, need, S),
         FA_ERR_INVALID_ARG, "null");
  expect("bwd nan scale",
         p_bwd(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.f / 0.f, A, need, S),
         FA_ERR_INVALID_ARG, "scale");
  expect("bwd_alibi null slopes",
         p_bwd_alibi(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, A, need, NULL, S),
         FA_ERR_INVALID_ARG, "alibi_slopes");
  expect("bwd_alibi short workspace",
         p_bwd_alibi(A, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, A, need - 4, F,
                     S),
         FA_ERR_WORKSPACE, "fa_bwd_alibi");

  expect("fwd_varlen null offsets",
         p_fwd_varlen(A, A, A, A, F, NULL, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, S),
         FA_ERR_INVALID_ARG, "cu_seqlens");
  expect("fwd_varlen max_seqlen > total",
         p_fwd_varlen(A, A, A, A, F, I, 3, 64, 65, 4, 2, 128, 1, 0, 0.1f, S),
         FA_ERR_INVALID_ARG, "max_seqlen");
  expect("bwd_varlen short workspace",
         p_bwd_varlen(A, A, A, A, A, F, A, A, A, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, A, 16, S),
         FA_ERR_WORKSPACE, "fa_bwd_varlen");
  expect("fwd_varlen_alibi null slopes",
         p_fwd_varlen_alibi(A, A, A, A, F, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, NULL, S),
         FA_ERR_INVALID_ARG, "alibi_slopes");
  expect("bwd_varlen_alibi null slopes",
         p_bwd_varlen_alibi(A, A, A, A, A, F, A, A, A, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, A,
                            1 << 20, NULL, S),
         FA_ERR_INVALID_ARG, "alibi_slopes");

  expect("bwd_noalloc too many rows",
         p_bwd_noalloc(A, A, A, A, A, F, A, A, A, 64, 64, 64, 2048, 128, 1, 0, 0.1f, S),
         FA_ERR_WORKSPACE, "fa_bwd_noalloc");
  expect("bwd_noalloc null pointer",
         p_bwd_noalloc(NULL, A, A, A, A, F, A, A, A, 1, 4, 2, 128, 128, 1, 0, 0.1f, S),
         FA_ERR_INVALID_ARG, "fa_bwd_noalloc");
  expect("mfma_probe null", p_mfma_probe(NULL, 4, 4, S), FA_ERR_INVALID_ARG, "fa_mfma_probe");
  expect("atomic_probe narrow stride", p_atomic_probe(F, 8, 64, 4, 4, S), FA_ERR_INVALID_ARG,
         "fa_atomic_probe");
  expect("issue_probe unknown kind", p_issue_probe(F, 9, 0, 2, 4, 4, S), FA_ERR_UNSUPPORTED,
         "fa_issue_probe");
  expect("fp8_product_probe no sets", p_fp8_probe(A, A, F, 0, S), FA_ERR_INVALID_ARG,
         "fa_fp8_product_probe");

  expect("decode Nq=0",
         p_decode(A, A, A, NULL, A, F, 2, 8, 2, 0, 4096, 128, 1, 0, 0.1f, 4, A, 1 << 20, S),
         FA_ERR_INVALID_ARG, "Nq");
  expect("decode d=256",
         p_decode(A, A, A, NULL, A, F, 2, 8, 2, 1, 4096, 256, 1, 0, 0.1f, 4, A, 1 << 20, S),
         FA_ERR_UNSUPPORTED, "head dim");

  if (failures) {
    printf("abi_caller: %d failure(s)\n", failures);
    return 1;
  }
  printf("abi_caller ok\n");
  return 0;
}
