// RoPE / YaRN cos-sin table, built on the device in double precision and
// rounded once to float. Entry (p, i): m*cos(p*theta'_i), m*sin(p*theta'_i),
// theta_i = base^(-2i/d). YaRN (Peng et al. 2023, NTK-by-parts interpolation
// in the correction-range form): theta'_i = theta_i*(1 - r_i) + theta_i/s*r_i
// with r_i ramping linearly in i from 0 at `low` to 1 at `high`.
// Pages: forward page flowchart ("RoPE cos/sin" input of the fused
// up-projection); Megatron page title (YaRN RoPE applied to q).
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

__global__ void rope_cache_kernel(float* __restrict__ cos_out, float* __restrict__ sin_out,
                                  int rows, int d_rope, double base, int yarn_on, double factor,
                                  double low, double span, double mscale) {
  const int pairs = d_rope / 2;
  const int64_t n = (int64_t)rows * pairs;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(e / pairs);
    const int i = (int)(e - (int64_t)p * pairs);
    double theta = pow(base, -2.0 * (double)i / (double)d_rope);
    double m = 1.0;
    if (yarn_on) {
      double r = ((double)i - low) / span;
      r = r < 0.0 ? 0.0 : (r > 1.0 ? 1.0 : r);
      theta = theta * (1.0 - r) + (theta / factor) * r;
      m = mscale;
    }
    const double ang = (double)p * theta;
    cos_out[e] = (float)(m * cos(ang));
    sin_out[e] = (float)(m * sin(ang));
  }
}

// Pair index at which the original context length holds n_rot rotations.
double correction_dim(double n_rot, int d, double base, int orig_max_pos) {
  return d * log((double)orig_max_pos / (n_rot * 2.0 * M_PI)) / (2.0 * log(base));
}

}  // namespace

hipError_t launch_rope_cache(float* cos, float* sin, int rows, int d_rope, double base,
                             const mla_yarn* yarn, hipStream_t stream) {
  double low = 0, span = 1, factor = 1, mscale = 1;
  if (yarn) {
    double lo = floor(correction_dim(yarn->beta_fast, d_rope, base, yarn->orig_max_pos));
    double hi = ceil(correction_dim(yarn->beta_slow, d_rope, base, yarn->orig_max_pos));
    lo = lo < 0 ? 0 : lo;
    hi = hi > d_rope - 1 ? d_rope - 1 : hi;
    low = lo;
    span = (hi != lo) ? hi - lo : 0.001;
    factor = yarn->factor;
    mscale = yarn->mscale;
  }
  const int64_t n = (int64_t)rows * (d_rope / 2);
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rope_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, cos, sin,
                     rows, d_rope, base, yarn ? 1 : 0, factor, low, span, mscale);
  return hipGetLastError();
}

}  // namespace mla
