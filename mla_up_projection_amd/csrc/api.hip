// C ABI of the fused MLA query up-projection: host-side validation, then the
// launches. Argument meanings, layouts and error behaviour are stated in
// include/mla_qup.h. Validation never dereferences a device pointer and makes
// no HIP call, so every error path runs without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "internal.h"

// Scratch memory of mla_qup_bwd_noalloc: one copy per GPU in this code
// object's static device data, held until the process ends. In host code the
// name `scratch` is only a stand-in for the device symbol (using it as an
// address would fault on the GPU); each GPU's copy is reached through the
// address hipGetSymbolAddress returns for it (scratch_for_current_device).
static __device__ __align__(256) uint8_t scratch[MLA_BWD_SCRATCH_BYTES];

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

Range rng(const void* p, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

// Outputs must be disjoint from inputs and from each other.
bool overlaps(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    const Range& o = outs[i];
    if (o.hi <= o.lo) continue;
    for (const Range& r : ins)
      if (r.hi > r.lo && o.lo < r.hi && r.lo < o.hi) return true;
    for (size_t j = i + 1; j < outs.size(); ++j) {
      const Range& r = outs[j];
      if (r.hi > r.lo && o.lo < r.hi && r.lo < o.hi) return true;
    }
  }
  return false;
}

mla_status launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_EDEVICE; }

// Shape checks common to forward and backward.
mla_status check_head_shape(int32_t K, int32_t H, int32_t d_nope, int32_t d_rope) {
  if (K <= 0 || K % 32 != 0 || H <= 0) return MLA_EINVAL;
  if (d_nope < 0 || d_rope < 0 || (d_nope & 1) || (d_rope & 1)) return MLA_EINVAL;
  int64_t D = (int64_t)d_nope + d_rope;
  if (D <= 0 || D % 32 != 0) return MLA_EINVAL;
  if ((int64_t)H * D > (int64_t)INT32_MAX / 2) return MLA_EINVAL;
  return MLA_OK;
}

// Token format checks; max_pos receives the largest possible position.
mla_status check_tokens(const mla_tokens& tk, int64_t* max_pos) {
  if (tk.T < 0 || tk.T > (int64_t)INT32_MAX) return MLA_EINVAL;
  if (tk.fmt == MLA_FMT_BSHD || tk.fmt == MLA_FMT_SBHD) {
    if (tk.B < 1 || tk.S < 1) return MLA_EINVAL;
    if ((int64_t)tk.B * tk.S != tk.T) return MLA_EINVAL;
    *max_pos = tk.S - 1;
    return MLA_OK;
  }
  if (tk.fmt == MLA_FMT_THD) {
    if (tk.nseq < 1 || tk.max_seqlen < 1) return MLA_EINVAL;
    if (tk.T > 0 && tk.cu_seqlens == nullptr) return MLA_EINVAL;
    if (!aligned(tk.cu_seqlens, 4)) return MLA_EINVAL;
    *max_pos = tk.max_seqlen - 1;
    return MLA_OK;
  }
  return MLA_EINVAL;
}

// The cos/sin width guard: the table must hold d_rope/2 pairs per row and a
// row for every position (the out-of-bounds cos/sin read that the Megatron
// page's Problem section names as a NaN source).
mla_status check_rope(const mla_rope& r, int32_t d_rope, int64_t max_pos) {
  if (d_rope == 0) return MLA_OK;
  if (r.cos == nullptr || r.sin == nullptr) return MLA_EINVAL;
  // the inverse-RoPE kernel reads four table pairs with one 16-byte load and
  // the forward epilogue two with one 8-byte load (when pairs % 4 == 0)
  if (!aligned(r.cos, 16) || !aligned(r.sin, 16)) return MLA_EINVAL;
  if (r.pairs < d_rope / 2) return MLA_EROPE_TABLE;
  if ((int64_t)r.rows < max_pos + 1 || r.rows < 1) return MLA_EROPE_TABLE;
  return MLA_OK;
}

size_t rope_bytes(const mla_rope& r, int32_t d_rope) {
  return d_rope ? (size_t)r.rows * (size_t)r.pairs * sizeof(float) : 0;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mla_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

void fill_token_map(const mla_tokens& tk, int& fmt, int& B, int& S, const int32_t*& cu, int& nseq) {
  fmt = tk.fmt;
  if (tk.fmt == MLA_FMT_THD) {
    B = 1;
    S = (int)tk.T;
    cu = tk.cu_seqlens;
    nseq = tk.nseq;
  } else {
    B = tk.B;
    S = tk.S;
    cu = nullptr;
    nseq = 0;
  }
}

}  // namespace

namespace mla {
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
}  // namespace mla

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_EINVAL: return "MLA_EINVAL: invalid argument";
    case MLA_EROPE_TABLE: return "MLA_EROPE_TABLE: cos/sin table too narrow or too short";
    case MLA_EALIAS: return "MLA_EALIAS: an output overlaps an input or another output";
    case MLA_EUNSUPPORTED: return "MLA_EUNSUPPORTED: unsupported combination";
    case MLA_EDEVICE: return "MLA_EDEVICE: HIP launch error";
    case MLA_EWORKSPACE: return "MLA_EWORKSPACE: workspace missing or too small";
    case MLA_ESCRATCH:
      return "MLA_ESCRATCH: the backward needs more scratch than mla_qup_bwd_noalloc's static "
             "array (MLA_BWD_SCRATCH_BYTES) holds; use mla_qup_bwd with a workspace";
    default: return "unknown mla_status";
  }
}

mla_status rope_cache_build(float* cos, float* sin, int32_t rows, int32_t d_rope, double base,
                            const mla_yarn* yarn, void* stream) {
  if (cos == nullptr || sin == nullptr || rows < 1 || d_rope < 2 || (d_rope & 1)) return MLA_EINVAL;
  if (!(base > 1.0) || !isfinite(base)) return MLA_EINVAL;
  if (!aligned(cos, 4) || !aligned(sin, 4)) return MLA_EINVAL;
  if (yarn) {
    if (!(yarn->factor > 0) || yarn->orig_max_pos <= 0 || !(yarn->beta_fast > 0) ||
        !(yarn->beta_slow > 0) || !isfinite(yarn->mscale) || !isfinite(yarn->factor))
      return MLA_EINVAL;
  }
  size_t bytes = (size_t)rows * (size_t)(d_rope / 2) * sizeof(float);
  if (overlaps({rng(cos, bytes), rng(sin, bytes)}, {})) return MLA_EALIAS;
  return launched(mla::launch_rope_cache(cos, sin, rows, d_rope, base, yarn, (hipStream_t)stream));
}

mla_status mxfp8_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                          uint8_t* codes, uint8_t* scales, void* stream) {
  if (x_dtype != MLA_DTYPE_BF16 && x_dtype != MLA_DTYPE_FP32) return MLA_EINVAL;
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || ld < cols) return MLA_EINVAL;
  if (rows == 0) return MLA_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MLA_EINVAL;
  size_t es = x_dtype == MLA_DTYPE_FP32 ? 4 : 2;
  if (!aligned(x, 16) || ((size_t)ld * es) % 16 != 0 || !aligned(codes, 8)) return MLA_EINVAL;
  if (rows > ((int64_t)1 << 40) || cols > ((int64_t)1 << 31)) return MLA_EINVAL;
  // rows * cols <= 2^36: one launch of rows * cols / 8192 workgroups of 256
  // threads stays within the 2^32 work-items of a grid dimension
  if (rows > (((int64_t)1 << 36) / cols)) return MLA_EINVAL;
  size_t xbytes = ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * es;
  if (overlaps({rng(codes, (size_t)rows * cols), rng(scales, (size_t)rows * cols / 32)},
               {rng(x, xbytes)}))
    return MLA_EALIAS;
  return launched(mla::launch_mxfp8_quantize(x, x_dtype == MLA_DTYPE_FP32, rows, cols, ld, codes,
                                             scales, (hipStream_t)stream));
}

mla_status mxfp8_quantize_t(const void* x, int64_t rows, int64_t cols, int64_t ld, int64_t rows_pad,
                            uint8_t* codes_t, uint8_t* scales_t, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || cols > 65535LL * 64 || ld < cols || ld % 8 != 0)
    return MLA_EINVAL;
  if (rows_pad < rows || rows_pad % 32 != 0 || rows_pad > ((int64_t)1 << 40)) return MLA_EINVAL;
  if (rows_pad == 0) return MLA_OK;
  if (x == nullptr || codes_t == nullptr || scales_t == nullptr) return MLA_EINVAL;
  if (!aligned(x, 16) || !aligned(codes_t, 16)) return MLA_EINVAL;
  const size_t xbytes = rows ? ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * 2 : 0;
  if (overlaps({rng(codes_t, (size_t)cols * rows_pad), rng(scales_t, (size_t)cols * rows_pad / 32)},
               {rng(x, xbytes)}))
    return MLA_EALIAS;
  return launched(mla::launch_mxfp8_quantize_t(x, rows, cols, ld, rows_pad, codes_t, scales_t,
                                               (hipStream_t)stream));
}

mla_status mla_kv_rope(const mla_kv_args* a, void* stream) {
  if (a == nullptr) return MLA_EINVAL;
  if (a->H < 1 || a->d_nope < 0 || a->d_rope < 0 || a->d_v < 0) return MLA_EINVAL;
  const int64_t widths = (int64_t)a->d_nope + a->d_rope + a->d_v;
  if (a->d_nope % 8 || a->d_rope % 8 || a->d_v % 8 || widths == 0) return MLA_EINVAL;
  if (a->H > 65536 || widths > 65536 || a->d_rope > 256) return MLA_EINVAL;
  if (a->out_dtype != MLA_DTYPE_BF16 && a->out_dtype != MLA_DTYPE_MXFP8) return MLA_EINVAL;
  const bool mx = a->out_dtype == MLA_DTYPE_MXFP8;
  const int Dk = a->d_nope + a->d_rope, Dv = a->d_v;
  if (mx && (Dk % 32 || Dv % 32)) return MLA_EINVAL;
  int64_t max_pos = 0;
  mla_status st = check_tokens(a->tokens, &max_pos);
  if (st) return st;
  if ((st = check_rope(a->rope, a->d_rope, max_pos))) return st;
  const int64_t T = a->tokens.T;
  if (T == 0) return MLA_OK;
  if (T * a->H * ((Dk + Dv) / 8) > (int64_t)INT32_MAX) return MLA_EUNSUPPORTED;  // 32-bit unit index
  if (a->kv == nullptr || (Dk && a->key == nullptr) || (Dv && a->value == nullptr)) return MLA_EINVAL;
  if (a->d_rope && a->k_pe == nullptr) return MLA_EINVAL;
  if (mx && ((Dk && a->key_scales == nullptr) || (Dv && a->value_scales == nullptr))) return MLA_EINVAL;
  if (!aligned(a->kv, 16) || !aligned(a->k_pe, 16) || !aligned(a->key, 16) || !aligned(a->value, 16))
    return MLA_EINVAL;
  const size_t eo = mx ? 1 : 2;
  const size_t TH = (size_t)T * a->H;
  std::vector<Range> ins = {rng(a->kv, TH * (a->d_nope + Dv) * 2)};
  if (a->d_rope) {
    ins.push_back(rng(a->k_pe, (size_t)T * a->d_rope * 2));
    ins.push_back(rng(a->rope.cos, rope_bytes(a->rope, a->d_rope)));
    ins.push_back(rng(a->rope.sin, rope_bytes(a->rope, a->d_rope)));
  }
  if (a->tokens.fmt == MLA_FMT_THD)
    ins.push_back(rng(a->tokens.cu_seqlens, ((size_t)a->tokens.nseq + 1) * 4));
  std::vector<Range> outs;
  if (Dk) outs.push_back(rng(a->key, TH * Dk * eo));
  if (Dv) outs.push_back(rng(a->value, TH * Dv * eo));
  if (mx && Dk) outs.push_back(rng(a->key_scales, TH * Dk / 32));
  if (mx && Dv) outs.push_back(rng(a->value_scales, TH * Dv / 32));
  if (overlaps(outs, ins)) return MLA_EALIAS;
  for (size_t i = 0; i < outs.size(); ++i)  // the outputs must not overlap each other either
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlaps({outs[i]}, {outs[j]})) return MLA_EALIAS;

  mla::KvParams p{};
  p.kv = (const uint16_t*)a->kv;
  p.pe = (const uint16_t*)a->k_pe;
  p.T = T;
  p.H = a->H;
  p.d_nope = a->d_nope;
  p.d_rope = a->d_rope;
  p.d_v = Dv;
  fill_token_map(a->tokens, p.fmt, p.B, p.S, p.cu, p.nseq);
  p.cos = a->rope.cos;
  p.sin = a->rope.sin;
  p.rope_rows = a->d_rope ? a->rope.rows : 0;
  p.rope_pairs = a->d_rope ? a->rope.pairs : 0;
  p.out_mx = mx;
  p.key = a->key;
  p.key_scales = (uint8_t*)a->key_scales;
  p.value = a->value;
  p.value_scales = (uint8_t*)a->value_scales;
  return launched(mla::launch_kv_rope(p, (hipStream_t)stream));
}

mla_status mla_qup_fwd(const mla_qup_fwd_args* a, void* stream) {
  if (a == nullptr) return MLA_EINVAL;
  mla_status st = check_head_shape(a->K, a->H, a->d_nope, a->d_rope);
  if (st) return st;
  int64_t max_pos = 0;
  if ((st = check_tokens(a->tokens, &max_pos))) return st;
  if (a->x_dtype != MLA_DTYPE_BF16 && a->x_dtype != MLA_DTYPE_MXFP8) return MLA_EINVAL;
  if (a->w_dtype != MLA_DTYPE_BF16 && a->w_dtype != MLA_DTYPE_MXFP8) return MLA_EINVAL;
  if (a->out_dtype != MLA_DTYPE_BF16 && a->out_dtype != MLA_DTYPE_MXFP8) return MLA_EINVAL;
  if (a->x_dtype != a->w_dtype) return MLA_EUNSUPPORTED;
  if (a->flags & ~(int32_t)MLA_FWD_FP8_MFMA) return MLA_EINVAL;
  const bool mx_in = a->x_dtype == MLA_DTYPE_MXFP8;
  const bool mx_out = a->out_dtype == MLA_DTYPE_MXFP8;
  if (mx_in && a->K % 128 != 0) return MLA_EINVAL;
  if ((st = check_rope(a->rope, a->d_rope, max_pos))) return st;
  const int64_t T = a->tokens.T;
  if (T == 0) return MLA_OK;
  if (a->x == nullptr || a->w == nullptr || a->out == nullptr) return MLA_EINVAL;
  if (mx_in && (a->x_scales == nullptr || a->w_scales == nullptr)) return MLA_EINVAL;
  if (mx_out && a->out_scales == nullptr) return MLA_EINVAL;
  if (!aligned(a->x, 16) || !aligned(a->w, 16) || !aligned(a->out, 16)) return MLA_EINVAL;
  // the epilogue reads four consecutive bias values with one 8-byte load
  if (a->bias && !aligned(a->bias, 8)) return MLA_EINVAL;
  // each lane loads four consecutive scale bytes of a row as one dword
  if (mx_in && (!aligned(a->x_scales, 4) || !aligned(a->w_scales, 4))) return MLA_EINVAL;

  const int D = a->d_nope + a->d_rope;
  const int64_t N = (int64_t)a->H * D;
  const size_t ein = mx_in ? 1 : 2;
  // the forward kernel addresses X and W rows with 32-bit byte offsets
  if ((uint64_t)T * a->K * ein > 0xFFFFFFFFull || (uint64_t)N * a->K * ein > 0xFFFFFFFFull)
    return MLA_EUNSUPPORTED;
  const size_t eout = mx_out ? 1 : 2;
  std::vector<Range> ins = {rng(a->x, (size_t)T * a->K * ein), rng(a->w, (size_t)N * a->K * ein)};
  if (mx_in) {
    ins.push_back(rng(a->x_scales, (size_t)T * a->K / 32));
    ins.push_back(rng(a->w_scales, (size_t)N * a->K / 32));
  }
  if (a->bias) ins.push_back(rng(a->bias, (size_t)N * 2));
  if (a->d_rope) {
    ins.push_back(rng(a->rope.cos, rope_bytes(a->rope, a->d_rope)));
    ins.push_back(rng(a->rope.sin, rope_bytes(a->rope, a->d_rope)));
  }
  if (a->tokens.fmt == MLA_FMT_THD)
    ins.push_back(rng(a->tokens.cu_seqlens, ((size_t)a->tokens.nseq + 1) * 4));
  std::vector<Range> outs = {rng(a->out, (size_t)T * N * eout)};
  if (mx_out) outs.push_back(rng(a->out_scales, (size_t)T * N / 32));
  if (overlaps(outs, ins)) return MLA_EALIAS;

  mla::FwdParams p{};
  p.x = a->x;
  p.xs = a->x_scales;
  p.w = a->w;
  p.ws = a->w_scales;
  p.bias = (const uint16_t*)a->bias;
  p.T = T;
  p.K = a->K;
  p.N = (int)N;
  p.H = a->H;
  p.D = D;
  p.d_nope = a->d_nope;
  p.d_rope = a->d_rope;
  fill_token_map(a->tokens, p.fmt, p.B, p.S, p.cu, p.nseq);
  p.cos = a->rope.cos;
  p.sin = a->rope.sin;
  p.rope_rows = a->d_rope ? a->rope.rows : 0;
  p.rope_pairs = a->d_rope ? a->rope.pairs : 0;
  p.out_mx = mx_out;
  p.mx_fp8_mfma = (a->flags & MLA_FWD_FP8_MFMA) ? 1 : 0;
  p.out = a->out;
  p.out_scales = a->out_scales;
  hipStream_t s = (hipStream_t)stream;
  return launched(mx_in ? mla::launch_qup_fwd_mx(p, s) : mla::launch_qup_fwd_bf16(p, s));
}

static mla_status check_bwd_shapes(const mla_qup_bwd_args* a, int64_t* max_pos) {
  if (a == nullptr) return MLA_EINVAL;
  mla_status st = check_head_shape(a->K, a->H, a->d_nope, a->d_rope);
  if (st) return st;
  if ((st = check_tokens(a->tokens, max_pos))) return st;
  if (a->dw_dtype != MLA_DTYPE_BF16 && a->dw_dtype != MLA_DTYPE_FP32) return MLA_EINVAL;
  if (a->use_bias != 0 && a->use_bias != 1) return MLA_EINVAL;
  return MLA_OK;
}

size_t mla_qup_bwd_workspace_size(const mla_qup_bwd_args* a) {
  int64_t max_pos = 0;
  if (check_bwd_shapes(a, &max_pos) != MLA_OK) return 0;
  const int N = a->H * (a->d_nope + a->d_rope);
  return mla::plan_bwd(a->tokens.T, N, a->K, a->use_bias != 0, a->dx != nullptr, a->dw != nullptr).total;
}

static bool mx_bwd_shapes_ok(int64_t T, int N, int K) {
  const int64_t Tp = (T + 127) / 128 * 128;
  const int64_t lim = (int64_t)1 << 32;
  return N % 128 == 0 && K % 32 == 0 && T * N < lim && (int64_t)N * Tp < lim && (int64_t)K * N < lim &&
         (int64_t)K * Tp < lim;
}

size_t mla_qup_bwd_mxfp8_workspace_size(const mla_qup_bwd_args* a) {
  int64_t max_pos = 0;
  if (check_bwd_shapes(a, &max_pos) != MLA_OK) return 0;
  const int N = a->H * (a->d_nope + a->d_rope);
  if (!mx_bwd_shapes_ok(a->tokens.T, N, a->K)) return 0;
  return mla::plan_bwd_mx(a->tokens.T, N, a->K, a->use_bias != 0).total;
}

static mla_status qup_bwd_impl(const mla_qup_bwd_args* a, int mx, int fp8_mfma, bool noalloc, void* stream);

mla_status mla_qup_bwd(const mla_qup_bwd_args* a, void* stream) { return qup_bwd_impl(a, 0, 0, false, stream); }

mla_status mla_qup_bwd_noalloc(const mla_qup_bwd_args* a, void* stream) {
  return qup_bwd_impl(a, 0, 0, true, stream);
}

mla_status mla_qup_bwd_mxfp8(const mla_qup_bwd_args* a, int32_t fp8_mfma, void* stream) {
  if (fp8_mfma != 0 && fp8_mfma != 1) return MLA_EINVAL;
  return qup_bwd_impl(a, 1, fp8_mfma, false, stream);
}

// noalloc: the partial sums go to the library's static scratch instead of the
// caller's workspace (mla_qup_bwd_noalloc; bf16 backward only).
static mla_status qup_bwd_impl(const mla_qup_bwd_args* a, int mx, int fp8_mfma, bool noalloc, void* stream) {
  int64_t max_pos = 0;
  mla_status st = check_bwd_shapes(a, &max_pos);
  if (st) return st;
  if ((st = check_rope(a->rope, a->d_rope, max_pos))) return st;
  const int64_t T = a->tokens.T;
  const int D = a->d_nope + a->d_rope;
  const int N = a->H * D;
  if (a->use_bias && a->db == nullptr) return MLA_EINVAL;
  if (T > 0 && (a->dq == nullptr || a->x == nullptr || a->w == nullptr || a->dq_pre == nullptr))
    return MLA_EINVAL;
  if (!aligned(a->dq, 16) || !aligned(a->x, 16) || !aligned(a->w, 16) ||
      !aligned(a->dq_pre, 16) || (a->dx && !aligned(a->dx, 16)) || (a->dw && !aligned(a->dw, 16)) ||
      (a->db && !aligned(a->db, 2)))
    return MLA_EINVAL;
  if (mx && !mx_bwd_shapes_ok(T, N, a->K)) return MLA_EUNSUPPORTED;
  mla::BwdPlan plan = mla::plan_bwd(T, N, a->K, a->use_bias != 0, a->dx != nullptr, a->dw != nullptr);
  mla::MxBwdPlan mplan{};
  if (mx) {
    mplan = mla::plan_bwd_mx(T, N, a->K, a->use_bias != 0);
    plan = mplan.base;
    plan.total = mplan.total;
  }
  if (noalloc) {
    if (plan.total > MLA_BWD_SCRATCH_BYTES)  // fall back to unsplit reductions (no split partials)
      plan = mla::plan_bwd(T, N, a->K, a->use_bias != 0, a->dx != nullptr, a->dw != nullptr, false);
    if (plan.total > MLA_BWD_SCRATCH_BYTES) return MLA_ESCRATCH;
  } else if (plan.total > 0) {
    if (a->workspace == nullptr || a->workspace_bytes < plan.total) return MLA_EWORKSPACE;
    if (!aligned(a->workspace, 256)) return MLA_EINVAL;
  }
  std::vector<Range> ins = {rng(a->dq, (size_t)T * N * 2), rng(a->x, (size_t)T * a->K * 2),
                            rng(a->w, (size_t)N * a->K * 2)};
  if (a->d_rope) {
    ins.push_back(rng(a->rope.cos, rope_bytes(a->rope, a->d_rope)));
    ins.push_back(rng(a->rope.sin, rope_bytes(a->rope, a->d_rope)));
  }
  if (a->tokens.fmt == MLA_FMT_THD)
    ins.push_back(rng(a->tokens.cu_seqlens, ((size_t)a->tokens.nseq + 1) * 4));
  std::vector<Range> outs = {rng(a->dq_pre, (size_t)T * N * 2)};
  if (a->dx) outs.push_back(rng(a->dx, (size_t)T * a->K * 2));
  if (a->dw) outs.push_back(rng(a->dw, (size_t)N * a->K * (a->dw_dtype == MLA_DTYPE_FP32 ? 4 : 2)));
  if (a->use_bias) outs.push_back(rng(a->db, (size_t)N * 2));
  if (plan.total && !noalloc) outs.push_back(rng(a->workspace, plan.total));
  if (overlaps(outs, ins)) return MLA_EALIAS;
  void* workspace = a->workspace;
  if (noalloc) {
    // the scratch of the device the stream runs on, which must be current
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MLA_EDEVICE;
    if (stream != nullptr) {
      if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return MLA_EDEVICE;
      if (sdev != cur) return MLA_EINVAL;
    }
    mla_status sst = scratch_for_current_device(&workspace);
    if (sst) return sst;
  }

  mla::BwdParams p{};
  p.dq = (const uint16_t*)a->dq;
  p.x = (const uint16_t*)a->x;
  p.w = (const uint16_t*)a->w;
  p.T = T;
  p.K = a->K;
  p.N = N;
  p.H = a->H;
  p.D = D;
  p.d_nope = a->d_nope;
  p.d_rope = a->d_rope;
  fill_token_map(a->tokens, p.fmt, p.B, p.S, p.cu, p.nseq);
  p.cos = a->rope.cos;
  p.sin = a->rope.sin;
  p.rope_rows = a->d_rope ? a->rope.rows : 0;
  p.rope_pairs = a->d_rope ? a->rope.pairs : 0;
  p.dq_pre = (uint16_t*)a->dq_pre;
  p.dx = (uint16_t*)a->dx;
  p.dw = a->dw;
  p.dw_fp32 = a->dw_dtype == MLA_DTYPE_FP32;
  p.use_bias = a->use_bias;
  p.db = (uint16_t*)a->db;
  p.workspace = workspace;
  if (mx) return launched(mla::launch_qup_bwd_mx(p, mplan, fp8_mfma, (hipStream_t)stream));
  return launched(mla::launch_qup_bwd(p, plan, (hipStream_t)stream));
}

}  // extern "C"
