// octo_decode_tokens: the explicit reconstruction of packed tokens,
// x^ = gamma R^T u^[:d] (OCTOPUS paper, Sec. 3.6 Eq. 13 and App. C.14: the
// factorized score is q . x^), for quality measurement and for callers that
// need dense vectors.  The attention kernels never call it: they keep u^ in
// registers and never materialize K^.
//
// One wavefront per token: lanes 0..42 read their triplet's field
// (xi | eta << b_dir | rho << 2 b_dir), decode the direction (Eq. 6 with the
// fold of App. C.7, normalized onto S^2) and scale it by the C_rho centroid
// into LDS; the wavefront then applies R^T = diag(s) H / sqrt(d) with the
// lane-pair Walsh-Hadamard transform and scales by gamma.  With a QJL codec
// the result is the MSE reconstruction alone: the sign sketch estimates inner
// products (Sec. 3.6), it does not reconstruct the residual.
//
// The group-wise value codec decodes the same way: lane l reads the codes of
// coordinates l and l + 64 and their groups' E4M3 scale and BF16 zero-point,
// u^ = Delta code + z, then R^T as above.
#include <math.h>

#include "octo_internal.h"

namespace octo {
namespace {

constexpr int kWaves = 4;              // tokens per workgroup
constexpr float kInvSqrtD = 0.08838834764831845f;

struct ReconArgs {
  const uint32_t* idx;
  const float* gamma;
  WideCodebook cb;
  uint64_t seed;
  int B, H, capacity, t0, T;
  float* out;                          // [B][H][T][128]
};

template <int BD, int BN>
__global__ __launch_bounds__(64 * kWaves) void reconstruct_kernel(ReconArgs a) {
  constexpr int K = 1 << BD, R = 1 << BN, FWD = 2 * BD, BT = FWD + BN;
  constexpr int WI = (kNTri * BT + 31) / 32;
  __shared__ float cx[K], cr[R];
  __shared__ float u[kWaves][kPadDim + 3];
  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  // the codebooks at constant indices (scalar loads of the kernel arguments)
  float xv = 0.0f, rv = 0.0f;
#pragma unroll
  for (int i = 0; i < K; ++i) xv = L == i ? a.cb.xi[i] : xv;
#pragma unroll
  for (int i = 0; i < R; ++i) rv = L == i ? a.cb.rho[i] : rv;
  if (tid < K) cx[tid] = xv;
  if (tid < R) cr[tid] = rv;
  __syncthreads();
  const int t = blockIdx.x * kWaves + wave;
  if (t >= a.T) return;                               // whole wavefronts
  const size_t plane = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int tc = a.t0 + t;
  float* ut = u[wave];
  if (L < kNTri) {
    const int pos = L * BT, w = pos >> 5, sh = pos & 31;
    const uint32_t lo = a.idx[tile_word(plane, a.capacity, tc, w, WI)];
    const uint32_t hi = sh + BT > 32 ? a.idx[tile_word(plane, a.capacity, tc, w + 1, WI)] : 0u;
    const uint32_t f = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & ((1u << BT) - 1u);
    const int ci = f & (K - 1), cj = (f >> BD) & (K - 1), ir = f >> FWD;
    const float xi = cx[ci], eta = cx[cj];
    const float z = 1.0f - fabsf(xi) - fabsf(eta);
    float x = xi, y = eta;
    if (z < 0.0f) {
      x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
      y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
    }
    const float s = cr[ir] / fmaxf(sqrtf(x * x + y * y + z * z), 1e-20f);
    ut[3 * L] = x * s;
    ut[3 * L + 1] = y * s;
    ut[3 * L + 2] = z * s;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float a0 = ut[L], a1 = ut[L + 64];                  // the pad coordinate 128 is dropped
  wht128(a0, a1);
  const float g = a.gamma[plane * a.capacity + tc] * kInvSqrtD;
  float* o = a.out + (plane * a.T + t) * kHeadDim;
  o[L] = a0 * splitmix_sign(a.seed, L) * g;
  o[L + 64] = a1 * splitmix_sign(a.seed, L + 64) * g;
}

template <int VB, int GS>
__global__ __launch_bounds__(64 * kWaves) void group_reconstruct_kernel(ReconArgs a) {
  constexpr int G = kHeadDim / GS, WC = VB * kHeadDim / 32, W = group_record_words(VB, GS);
  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * kWaves + wave;
  if (t >= a.T) return;                               // whole wavefronts
  const size_t plane = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int tc = a.t0 + t;
  float u[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = L + 64 * k, pos = c * VB, w = pos >> 5, sh = pos & 31;
    const uint32_t lo = a.idx[tile_word(plane, a.capacity, tc, w, W)];
    const uint32_t hi = sh + VB > 32 ? a.idx[tile_word(plane, a.capacity, tc, w + 1, W)] : 0u;
    const uint32_t q = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & ((1u << VB) - 1u);
    const int gi = c / GS;
    const uint32_t sw = a.idx[tile_word(plane, a.capacity, tc, WC + gi / 4, W)];
    const uint32_t zw = a.idx[tile_word(plane, a.capacity, tc, WC + G / 4 + gi / 2, W)];
    const float dh = e4m3_value((sw >> (8 * (gi % 4))) & 0xffu);
    const float zh = __uint_as_float(((zw >> (16 * (gi % 2))) & 0xffffu) << 16);
    u[k] = fmaf(dh, (float)q, zh);
  }
  wht128(u[0], u[1]);
  float* o = a.out + (plane * a.T + t) * kHeadDim;
  o[L] = u[0] * splitmix_sign(a.seed, L) * kInvSqrtD;
  o[L + 64] = u[1] * splitmix_sign(a.seed, L + 64) * kInvSqrtD;
}

template <int VB, int GS>
void launch_group(const ReconArgs& a, hipStream_t st) {
  dim3 grid((a.T + kWaves - 1) / kWaves, a.H, a.B);
  hipLaunchKernelGGL((group_reconstruct_kernel<VB, GS>), grid, dim3(64 * kWaves), 0, st, a);
}

template <int BD, int BN>
void launch(const ReconArgs& a, hipStream_t st) {
  dim3 grid((a.T + kWaves - 1) / kWaves, a.H, a.B);
  hipLaunchKernelGGL((reconstruct_kernel<BD, BN>), grid, dim3(64 * kWaves), 0, st, a);
}

}  // namespace
}  // namespace octo

using namespace octo;

extern "C" octo_status octo_decode_tokens(const octo_codec_desc* codec,
                                          const octo_cache_view* cache, int32_t t0, int32_t T,
                                          float* out, hipStream_t stream) {
  clear_error();
  const char* what = "octo_decode_tokens";
  Codec c;
  octo_status s = resolve_codec(codec, what, &c, true, true);
  if (s != OCTO_OK) return s;
  if ((s = check_cache(cache, c, what)) != OCTO_OK) return s;
  if (t0 < 0 || T < 0) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: t0 %d, T %d", what, t0, T);
  if ((int64_t)t0 + T > cache->capacity)
    return fail(OCTO_ERR_CAPACITY, "%s: tokens [%d, %d) beyond capacity %d", what, t0, t0 + T,
                cache->capacity);
  if (T == 0) return OCTO_OK;
  if (!out) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: out is NULL", what);
  if ((uintptr_t)out & 3) return fail(OCTO_ERR_ALIGNMENT, "%s: out misaligned", what);
  if (cache->batch > 65535 || cache->kv_heads > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: batch and heads must be <= 65535", what);
  ReconArgs a;
  a.idx = cache->idx;
  a.gamma = cache->gamma;
  a.cb = c.wcb;
  a.seed = c.seed;
  a.B = cache->batch;
  a.H = cache->kv_heads;
  a.capacity = cache->capacity;
  a.t0 = t0;
  a.T = T;
  a.out = out;
  if (c.group) {
    switch (c.bits * 100 + c.group) {
      case 216: launch_group<2, 16>(a, stream); break;
      case 232: launch_group<2, 32>(a, stream); break;
      case 316: launch_group<3, 16>(a, stream); break;
      case 332: launch_group<3, 32>(a, stream); break;
      case 416: launch_group<4, 16>(a, stream); break;
      case 432: launch_group<4, 32>(a, stream); break;
      default: return fail(OCTO_ERR_UNSUPPORTED, "%s: group codec not compiled", what);
    }
    return check_launch(what);
  }
  switch (c.b_dir * 10 + c.b_nrm) {
    case 31: launch<3, 1>(a, stream); break;
    case 42: launch<4, 2>(a, stream); break;
    case 53: launch<5, 3>(a, stream); break;
    case 22: launch<2, 2>(a, stream); break;
    case 33: launch<3, 3>(a, stream); break;
    case 44: launch<4, 4>(a, stream); break;
    // the rest of the (b + delta, b - delta) sweep (Sec. 3.3)
    case 4: launch<0, 4>(a, stream); break;
    case 15: launch<1, 5>(a, stream); break;
    case 26: launch<2, 6>(a, stream); break;
    case 13: launch<1, 3>(a, stream); break;
    case 24: launch<2, 4>(a, stream); break;
    case 35: launch<3, 5>(a, stream); break;
    case 40: launch<4, 0>(a, stream); break;
    case 51: launch<5, 1>(a, stream); break;
    case 62: launch<6, 2>(a, stream); break;
    default: return fail(OCTO_ERR_UNSUPPORTED, "%s: configuration not compiled", what);
  }
  return check_launch(what);
}
