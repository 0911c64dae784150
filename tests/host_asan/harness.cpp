// Host-only build of the C ABI's validation and planning (api.hip, plan.hip)
// for AddressSanitizer / UndefinedBehaviorSanitizer: the kernel launchers and
// the few HIP runtime calls are stubs, and every entry point is driven
// through its error paths, its accepted paths and extreme sizes with fake
// device addresses (validation never dereferences them). Exit status 0 and a
// last line "harness ok" mean every status matched and no sanitizer fired.
#define __align__(n) __attribute__((aligned(n)))
#ifndef HIP_SYMBOL
#define HIP_SYMBOL(x) (x)
#endif
#include <stdio.h>
#include <stdlib.h>

#include "../../mla_up_projection_amd/csrc/api.hip"
#include "../../mla_up_projection_amd/csrc/plan.hip"

// ---- stubs of the launchers and of the HIP runtime ----
static int g_launches = 0;
namespace mla {
hipError_t launch_rope_cache(float*, float*, int, int, double, const mla_yarn*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_kv_rope(const KvParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_mxfp8_quantize_t(const void*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_mxfp8_quantize(const void*, int, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qup_fwd_bf16(const FwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qup_fwd_mx(const FwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_mx_gemm(const FwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qup_bwd(const BwdParams&, const BwdPlan&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qup_bwd_mx(const BwdParams&, const MxBwdPlan&, int, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace mla
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) { *d = 0; return hipSuccess; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }

// ---- driver ----
static int g_fail = 0;
#define EXPECT(call, code)                                                                  \
  do {                                                                                      \
    const long got_ = (long)(call);                                                         \
    if (got_ != (long)(code)) {                                                             \
      printf("FAIL line %d: %s = %ld, expected %ld\n", __LINE__, #call, got_, (long)(code)); \
      ++g_fail;                                                                             \
    }                                                                                       \
  } while (0)

static const uintptr_t BASE = 0x7F0000000000ull;
static void* A(int i, uintptr_t off = 0) { return (void*)(BASE + (uintptr_t)i * ((uintptr_t)1 << 36) + off); }

static mla_qup_fwd_args fwd0() {
  mla_qup_fwd_args a;
  memset(&a, 0, sizeof a);
  a.x = A(1); a.x_dtype = MLA_DTYPE_BF16; a.w = A(2); a.w_dtype = MLA_DTYPE_BF16;
  a.K = 1536; a.H = 128; a.d_nope = 128; a.d_rope = 64;
  a.tokens.fmt = MLA_FMT_BSHD; a.tokens.B = 1; a.tokens.S = 4096; a.tokens.T = 4096;
  a.rope.cos = (const float*)A(3); a.rope.sin = (const float*)A(4); a.rope.rows = 4096; a.rope.pairs = 32;
  a.out_dtype = MLA_DTYPE_MXFP8; a.out = A(5); a.out_scales = (uint8_t*)A(6);
  return a;
}
static mla_qup_bwd_args bwd0() {
  mla_qup_bwd_args a;
  memset(&a, 0, sizeof a);
  a.dq = A(1); a.x = A(2); a.w = A(3); a.K = 1536; a.H = 128; a.d_nope = 128; a.d_rope = 64;
  a.tokens.fmt = MLA_FMT_BSHD; a.tokens.B = 1; a.tokens.S = 4096; a.tokens.T = 4096;
  a.rope.cos = (const float*)A(4); a.rope.sin = (const float*)A(5); a.rope.rows = 4096; a.rope.pairs = 32;
  a.dq_pre = A(6); a.dx = A(7); a.dw = A(8); a.dw_dtype = MLA_DTYPE_BF16; a.use_bias = 1; a.db = A(9);
  a.workspace = A(10); a.workspace_bytes = (size_t)1 << 34;
  return a;
}
static mla_kv_args kv0() {
  mla_kv_args a;
  memset(&a, 0, sizeof a);
  a.kv = A(1); a.k_pe = A(2); a.H = 128; a.d_nope = 128; a.d_rope = 64; a.d_v = 128;
  a.tokens.fmt = MLA_FMT_BSHD; a.tokens.B = 1; a.tokens.S = 4096; a.tokens.T = 4096;
  a.rope.cos = (const float*)A(3); a.rope.sin = (const float*)A(4); a.rope.rows = 4096; a.rope.pairs = 32;
  a.out_dtype = MLA_DTYPE_MXFP8; a.key = A(5); a.key_scales = A(6); a.value = A(7); a.value_scales = A(8);
  return a;
}

int main() {
  // forward
  mla_qup_fwd_args f = fwd0();
  EXPECT(mla_qup_fwd(&f, nullptr), MLA_OK);
  EXPECT(mla_qup_fwd(nullptr, nullptr), MLA_EINVAL);
  f = fwd0(); f.K = 0; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.H = 0x7FFFFFFF; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.d_nope = 0x7FFFFFF0; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.d_nope = -2; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.K = 0x7FFFFFE0; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EUNSUPPORTED);
  f = fwd0(); f.tokens.T = (int64_t)1 << 40; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.tokens.B = 0x7FFFFFFF; f.tokens.S = 0x7FFFFFFF; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.tokens.T = 0x7FFFFFFF; f.tokens.S = 0x7FFFFFFF; f.rope.rows = 0x7FFFFFFF;
  EXPECT(mla_qup_fwd(&f, nullptr), MLA_EUNSUPPORTED);
  f = fwd0(); f.rope.rows = 4095; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EROPE_TABLE);
  f = fwd0(); f.rope.pairs = 31; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EROPE_TABLE);
  f = fwd0(); f.rope.cos = (const float*)A(3, 4); EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.bias = A(11, 4); EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.bias = A(11, 8); EXPECT(mla_qup_fwd(&f, nullptr), MLA_OK);
  f = fwd0(); f.out = A(1, 1024); EXPECT(mla_qup_fwd(&f, nullptr), MLA_EALIAS);
  f = fwd0(); f.x_dtype = f.w_dtype = MLA_DTYPE_MXFP8; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f.x_scales = (uint8_t*)A(12); f.w_scales = (uint8_t*)A(13); EXPECT(mla_qup_fwd(&f, nullptr), MLA_OK);
  f.flags = 7; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EINVAL);
  f = fwd0(); f.tokens.fmt = MLA_FMT_THD; f.tokens.cu_seqlens = (const int32_t*)A(14); f.tokens.nseq = 0x7FFFFFFF;
  f.tokens.max_seqlen = 4096; EXPECT(mla_qup_fwd(&f, nullptr), MLA_OK);  // an 8 GiB cu_seqlens range
  f.tokens.nseq = 7; EXPECT(mla_qup_fwd(&f, nullptr), MLA_OK);
  f.tokens.max_seqlen = 0x7FFFFFFF; EXPECT(mla_qup_fwd(&f, nullptr), MLA_EROPE_TABLE);
  // backward
  mla_qup_bwd_args b = bwd0();
  EXPECT(mla_qup_bwd(&b, nullptr), MLA_OK);
  EXPECT(mla_qup_bwd_mxfp8(&b, 1, nullptr), MLA_OK);
  EXPECT(mla_qup_bwd_mxfp8(&b, 2, nullptr), MLA_EINVAL);
  if (mla_qup_bwd_workspace_size(&b) == 0 || mla_qup_bwd_mxfp8_workspace_size(&b) == 0) {
    printf("FAIL: workspace size 0\n");
    ++g_fail;
  }
  EXPECT(mla_qup_bwd_workspace_size(nullptr), 0);
  b = bwd0(); b.workspace_bytes = 16; EXPECT(mla_qup_bwd(&b, nullptr), MLA_EWORKSPACE);
  b = bwd0(); b.db = nullptr; EXPECT(mla_qup_bwd(&b, nullptr), MLA_EINVAL);
  b = bwd0(); b.rope.sin = (const float*)A(5, 8); EXPECT(mla_qup_bwd(&b, nullptr), MLA_EINVAL);
  b = bwd0(); b.dx = A(6, 64); EXPECT(mla_qup_bwd(&b, nullptr), MLA_EALIAS);
  // extreme sizes through the planner (64-bit byte counts, split choices)
  for (int64_t T : {(int64_t)1, (int64_t)63, (int64_t)65, (int64_t)4096, (int64_t)1 << 20, (int64_t)0x7FFFFFFF}) {
    for (int H : {1, 16, 128, 1024}) {
      b = bwd0(); b.tokens.T = T; b.tokens.S = (int32_t)T; b.rope.rows = (int32_t)T; b.H = H;
      const size_t need = mla_qup_bwd_workspace_size(&b);
      b.workspace_bytes = need;
      const mla_status st = mla_qup_bwd(&b, nullptr);
      if (st != MLA_OK && st != MLA_EALIAS) {  // fake ranges may overlap at these sizes
        printf("FAIL: bwd T=%lld H=%d status %d\n", (long long)T, H, st);
        ++g_fail;
      }
      (void)mla_qup_bwd_mxfp8_workspace_size(&b);
    }
  }
  b = bwd0(); b.tokens.T = 0; b.tokens.S = 0; EXPECT(mla_qup_bwd(&b, nullptr), MLA_EINVAL);
  // allocation-free backward: the workspace arguments are ignored; a plan that
  // does not fit the static scratch falls back to unsplit reductions, and only
  // db partials beyond it are refused
  b = bwd0(); b.workspace = nullptr; b.workspace_bytes = 0;
  EXPECT(mla_qup_bwd_noalloc(&b, nullptr), MLA_OK);
  EXPECT(mla_qup_bwd_noalloc(&b, (void*)0x1234), MLA_OK);  // stub: stream on device 0
  b.tokens.T = 1 << 20; b.tokens.S = 1 << 20; b.rope.rows = 1 << 20;  // db partials 16384 x N x 4 B
  EXPECT(mla_qup_bwd_noalloc(&b, nullptr), MLA_ESCRATCH);
  b.use_bias = 0; b.db = nullptr; EXPECT(mla_qup_bwd_noalloc(&b, nullptr), MLA_OK);  // unsplit: no partials
  b = bwd0(); b.dq_pre = nullptr; EXPECT(mla_qup_bwd_noalloc(&b, nullptr), MLA_EINVAL);
  // KV side
  mla_kv_args k = kv0();
  EXPECT(mla_kv_rope(&k, nullptr), MLA_OK);
  k = kv0(); k.d_rope = 0x7FFFFFF8; EXPECT(mla_kv_rope(&k, nullptr), MLA_EINVAL);
  k = kv0(); k.H = 65536; k.tokens.T = 0x7FFFFFFF; k.tokens.S = 0x7FFFFFFF; k.rope.rows = 0x7FFFFFFF;
  EXPECT(mla_kv_rope(&k, nullptr), MLA_EUNSUPPORTED);
  k = kv0(); k.key = A(1, 512); EXPECT(mla_kv_rope(&k, nullptr), MLA_EALIAS);
  // quantizers and table
  EXPECT(mxfp8_quantize(A(1), MLA_DTYPE_BF16, 8192, 1536, 1536, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_OK);
  EXPECT(mxfp8_quantize(A(1), MLA_DTYPE_FP32, (int64_t)1 << 41, 64, 64, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_EINVAL);
  EXPECT(mxfp8_quantize(A(1), MLA_DTYPE_BF16, 4, (int64_t)1 << 40, (int64_t)1 << 40, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_EINVAL);
  // 2^37 elements: more work-items than one grid dimension holds
  EXPECT(mxfp8_quantize(A(1), MLA_DTYPE_BF16, (int64_t)1 << 20, (int64_t)1 << 17, (int64_t)1 << 17, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_EINVAL);
  EXPECT(mxfp8_quantize_t(A(1), 4096, 24576, 24576, 4096, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_OK);
  EXPECT(mxfp8_quantize_t(A(1), 4096, 24576, 24576, (int64_t)1 << 41, (uint8_t*)A(2), (uint8_t*)A(3), nullptr), MLA_EINVAL);
  mla_yarn y = {40.0, 4096, 32.0, 1.0, 1.0};
  EXPECT(rope_cache_build((float*)A(1), (float*)A(2), 4096, 64, 1e4, &y, nullptr), MLA_OK);
  // 2^31 rows of 32 pairs: 256 GiB tables, which overlap at these fake addresses
  EXPECT(rope_cache_build((float*)A(1), (float*)A(2), 0x7FFFFFFF, 64, 1e4, nullptr, nullptr), MLA_EALIAS);
  y.factor = 0.0 / 0.0;
  EXPECT(rope_cache_build((float*)A(1), (float*)A(2), 16, 64, 1e4, &y, nullptr), MLA_EINVAL);
  for (int s = -1; s < 10; ++s)
    if (mla_status_str(s) == nullptr) ++g_fail;
  printf("%d launches stubbed, %d failures\n", g_launches, g_fail);
  if (g_fail) return 1;
  printf("harness ok\n");
  return 0;
}
