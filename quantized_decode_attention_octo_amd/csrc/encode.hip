// octo_encode: the OCTOPUS encoder on gfx950.
//
// One workgroup (4 wavefronts) encodes 64 consecutive tokens of one
// (batch, head) plane, following the OCTOPUS paper (arXiv 2605.21226):
//   Sec. 3.1      gamma = ||x||_2 and u = R x / gamma with R = H diag(s), the
//                 normalized Walsh-Hadamard transform after a sign flip; one
//                 wavefront per token, the transform as in-register and
//                 cross-lane butterflies;
//   Sec. 3.2      u zero-padded to 129 coordinates, 43 triplets t_i, the
//                 octahedral coordinates (xi, eta) of Eq. 5;
//   Sec. 3.5      scalar Lloyd seeds, then the local 3x3 joint rounding: the
//                 candidate direction maximizing s = t . n(xi^, eta^) and the
//                 norm centroid nearest that s (the minimizer of Eq. 12);
//                 rounding = SCALAR keeps the seeds and the centroid nearest
//                 rho = ||t||;
//   Sec. 3.6      with QJL: r = u - u^, sigma = sign(H diag(s') r) and
//                 gamma_r = fp16(||r||);
//   Sec. 3      the packed index streams I_dir, I_nrm.
// Phase 2 spreads the 64 x 43 triplets of the workgroup over all 256 lanes.
// The decoded unit directions n(xi^, eta^) of every code pair live in LDS,
// built once per workgroup from C_xi.
#include <math.h>

#include "octo_internal.h"

namespace octo {
namespace {

constexpr int kTok = 64;          // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kUStride = 132;     // floats per token row of u in LDS

struct EncodeArgs {
  const void* x;
  int64_t s0, s1, s2;             // element strides of b, h, t
  int is_bf16;
  int B, H, T;
  const float* c_xi;
  const float* c_rho;
  uint64_t seed;
  int qjl, rounding;
  uint32_t* dir;
  uint32_t* nrm;
  float* gamma;
  uint32_t* qjl_bits;
  uint16_t* gamma_r;
  int capacity, token_offset;
};

__device__ inline float load_x(const EncodeArgs& a, int64_t off) {
  if (a.is_bf16) return bf16_to_f32(static_cast<const uint16_t*>(a.x)[off]);
  return static_cast<const float*>(a.x)[off];
}

// Index of the nearest of the N sorted centroids whose N-1 cell boundaries
// (midpoints) are `mid`: the number of boundaries below x.
template <int N>
__device__ inline int nearest(const float* mid, float x) {
  int idx = 0;
#pragma unroll
  for (int step = N >> 1; step > 0; step >>= 1)
    if (x > mid[idx + step - 1]) idx += step;
  return idx;
}

// Packs word w of a stream of kNTri fields of FW bits (LSB-first).
template <int FW, typename Get>
__device__ inline uint32_t pack_word(int w, Get get) {
  const int lo = (32 * w) / FW;
  int hi = (32 * w + 31) / FW;
  if (hi > kNTri - 1) hi = kNTri - 1;
  uint32_t out = 0;
  for (int i = lo; i <= hi; ++i) {
    const int shift = i * FW - 32 * w + 32;  // in [33 - FW, 63]
    out |= (uint32_t)(((uint64_t)get(i) << shift) >> 32);
  }
  return out;
}

template <int BD, int BN>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int K = 1 << BD, R = 1 << BN;
  constexpr int FWD = 2 * BD;                         // xi | eta << BD
  constexpr int WD = (kNTri * FWD + 31) / 32, WN = (kNTri * BN + 31) / 32;

  __shared__ float4 lut[K * K];                       // n(c_xi[i], c_xi[j]) at i + K j
  __shared__ float cxi[K], mid_xi[K], crho[R], mid_rho[R];
  __shared__ float sgn[2 * kHeadDim];                 // s then s'
  __shared__ float u[kTok * kUStride];
  __shared__ uint16_t code_dir[kTok * kNTri];
  __shared__ uint8_t code_nrm[kTok * kNTri];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * kTok;

  // ---- tables: signs, codebooks, midpoints, the decoded direction of every
  // code pair (codebooks go through LDS so that the table loop reads no
  // global memory)
  for (int j = tid; j < 2 * kHeadDim; j += kThreads) sgn[j] = splitmix_sign(a.seed, j);
  if (tid < K) cxi[tid] = a.c_xi[tid];
  if (tid < R) crho[tid] = a.c_rho[tid];
  __syncthreads();
  if (tid < K - 1) mid_xi[tid] = 0.5f * (cxi[tid] + cxi[tid + 1]);
  if (tid < R - 1) mid_rho[tid] = 0.5f * (crho[tid] + crho[tid + 1]);
  for (int e = tid; e < K * K; e += kThreads) {
    // Eq. 6 with the fold of App. C.7, then normalization onto S^2.
    const float xi = cxi[e % K], eta = cxi[e / K];
    const float z = 1.0f - fabsf(xi) - fabsf(eta);
    float x = xi, y = eta;
    if (z < 0.0f) {
      x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
      y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
    }
    const float n = fmaxf(sqrtf(x * x + y * y + z * z), kEps);
    lut[e] = make_float4(x / n, y / n, z / n, 0.0f);
  }
  __syncthreads();

  // ---- phase 1: gamma and the rotation, one wavefront per token
  const size_t plane = (size_t)b * a.H + h;
  const int64_t base = (int64_t)b * a.s0 + (int64_t)h * a.s1;
  const float inv_sqrt_d = 0.08838834764831845f;     // 1/sqrt(128)
  // each wave takes 16 tokens, loading all of them before any use
  constexpr int kPerWave = kTok / 4;
  float xs[kPerWave][2];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int t = t0 + wave + 4 * j;
    xs[j][0] = xs[j][1] = 0.0f;
    if (t < a.T) {
      const int64_t off = base + (int64_t)t * a.s2;
      xs[j][0] = load_x(a, off + lane);
      xs[j][1] = load_x(a, off + lane + 64);
    }
  }
  const float s_lo = sgn[lane], s_hi = sgn[lane + 64];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int k = wave + 4 * j, t = t0 + k;
    const float x0 = xs[j][0], x1 = xs[j][1];
    const float gamma = sqrtf(wave_sum(x0 * x0 + x1 * x1));
    float v0 = x0 * s_lo, v1 = x1 * s_hi;
    wht128(v0, v1);
    const float scale = inv_sqrt_d / fmaxf(gamma, kEps);
    u[k * kUStride + lane] = v0 * scale;
    u[k * kUStride + lane + 64] = v1 * scale;
    if (lane == 0) {
      u[k * kUStride + kHeadDim] = 0.0f;              // the zero pad (Sec. 3.2)
      if (t < a.T) a.gamma[plane * a.capacity + a.token_offset + t] = gamma;
    }
  }
  __syncthreads();

  // ---- phase 2: per triplet, octahedral map, seeds, joint rounding
  for (int e = tid; e < kTok * kNTri; e += kThreads) {
    const int k = e / kNTri, i = e - k * kNTri;
    float* tp = &u[k * kUStride + 3 * i];
    const float tx = tp[0], ty = tp[1], tz = tp[2];
    // Eq. 5 on the L1-normalized direction, sign(0) = +1.
    const float l1 = fmaxf(fabsf(tx) + fabsf(ty) + fabsf(tz), kEps);
    const float px = tx / l1, py = ty / l1, pz = tz / l1;
    float xi = px, eta = py;
    if (pz < 0.0f) {
      xi = (px >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(py));
      eta = (py >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(px));
    }
    const int sx = nearest<K>(mid_xi, xi), sy = nearest<K>(mid_xi, eta);
    int bx = sx, by = sy, ir;
    if (a.rounding == OCTO_ROUND_SCALAR) {
      ir = nearest<R>(mid_rho, sqrtf(tx * tx + ty * ty + tz * tz));
    } else {
      // Seed first, then the other eight neighbours row-major (dx outer);
      // only a strictly larger s replaces the incumbent.
      float4 n = lut[sx + K * sy];
      float best = tx * n.x + ty * n.y + tz * n.z;
#pragma unroll
      for (int dx = -1; dx <= 1; ++dx)
#pragma unroll
        for (int dy = -1; dy <= 1; ++dy) {
          if (dx == 0 && dy == 0) continue;
          const int cx = min(max(sx + dx, 0), K - 1), cy = min(max(sy + dy, 0), K - 1);
          n = lut[cx + K * cy];
          const float s = tx * n.x + ty * n.y + tz * n.z;
          if (s > best) {
            best = s;
            bx = cx;
            by = cy;
          }
        }
      ir = nearest<R>(mid_rho, best);
    }
    code_dir[k * kNTri + i] = (uint16_t)(bx | (by << BD));
    code_nrm[k * kNTri + i] = (uint8_t)ir;
    if (a.qjl) {
      // Rotated-frame residual r = u - u^ written over u (Sec. 3.6).
      const float4 n = lut[bx + K * by];
      const float rho = crho[ir];
      tp[0] = tx - rho * n.x;
      tp[1] = ty - rho * n.y;
      tp[2] = tz - rho * n.z;
    }
  }
  __syncthreads();

  // ---- phase 3: pack I_dir and I_nrm (token-fastest items: coalesced stores)
  const int t_valid = min(kTok, a.T - t0);
  for (int e = tid; e < kTok * (WD + WN); e += kThreads) {
    const int k = e & 63, w = e >> 6;
    if (k >= t_valid) continue;
    const int tc = a.token_offset + t0 + k;
    if (w < WD) {
      const uint16_t* cd = &code_dir[k * kNTri];
      a.dir[tile_word(plane, a.capacity, tc, w, WD)] =
          pack_word<FWD>(w, [&](int i) { return (uint32_t)cd[i]; });
    } else {
      const uint8_t* cn = &code_nrm[k * kNTri];
      a.nrm[tile_word(plane, a.capacity, tc, w - WD, WN)] =
          pack_word<BN>(w - WD, [&](int i) { return (uint32_t)cn[i]; });
    }
  }

  // ---- phase 4 (QJL): sigma = sign(H diag(s') r), gamma_r = fp16(||r||)
  if (a.qjl) {
    for (int k = wave; k < t_valid; k += 4) {
      const float r0 = u[k * kUStride + lane], r1 = u[k * kUStride + lane + 64];
      const float rn = sqrtf(wave_sum(r0 * r0 + r1 * r1));
      float v0 = r0 * sgn[kHeadDim + lane], v1 = r1 * sgn[kHeadDim + lane + 64];
      wht128(v0, v1);
      const uint64_t m0 = __ballot(v0 < 0.0f), m1 = __ballot(v1 < 0.0f);
      const int tc = a.token_offset + t0 + k;
      if (lane < 4) {
        const uint64_t m = lane < 2 ? m0 : m1;
        a.qjl_bits[tile_word(plane, a.capacity, tc, lane, 4)] =
            (uint32_t)(m >> (32 * (lane & 1)));
      }
      if (lane == 0) {
        const _Float16 hr = (_Float16)rn;
        a.gamma_r[plane * a.capacity + tc] = __builtin_bit_cast(uint16_t, hr);
      }
    }
  }
}

template <int BD, int BN>
void launch(const EncodeArgs& a, hipStream_t st) {
  dim3 grid((a.T + kTok - 1) / kTok, a.H, a.B);
  hipLaunchKernelGGL((encode_kernel<BD, BN>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace
}  // namespace octo

extern "C" octo_status octo_encode(const octo_codec_desc* codec, const void* x, octo_dtype x_dtype,
                                   int32_t B, int32_t H, int32_t T, const int64_t x_strides[4],
                                   const octo_cache_view* dst, int32_t token_offset,
                                   hipStream_t stream) {
  using namespace octo;
  clear_error();
  Codec c;
  octo_status s = resolve_codec(codec, "octo_encode", &c);
  if (s != OCTO_OK) return s;
  if ((s = check_cache(dst, c, "octo_encode dst")) != OCTO_OK) return s;
  if (x_dtype != OCTO_DTYPE_F32 && x_dtype != OCTO_DTYPE_BF16)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: x_dtype %d unknown", (int)x_dtype);
  if (B < 0 || H < 0 || T < 0 || token_offset < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: negative size or offset");
  if (!x_strides) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: x_strides is NULL");
  if (B > 65535 || H > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "octo_encode: B and H must be <= 65535");
  if (B == 0 || H == 0 || T == 0) return OCTO_OK;
  if (!x) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: x is NULL");
  if (x_strides[3] != 1)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: the last stride of x must be 1");
  if (x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: negative stride");
  const size_t esz = x_dtype == OCTO_DTYPE_F32 ? 4 : 2;
  if ((uintptr_t)x % esz) return fail(OCTO_ERR_ALIGNMENT, "octo_encode: x misaligned");
  if (dst->batch != B || dst->kv_heads != H)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_encode: dst is [%d, %d], x is [%d, %d]",
                dst->batch, dst->kv_heads, B, H);
  if ((int64_t)token_offset + T > dst->capacity)
    return fail(OCTO_ERR_CAPACITY, "octo_encode: tokens [%d, %lld) exceed capacity %d",
                token_offset, (long long)token_offset + T, dst->capacity);
  EncodeArgs a;
  a.x = x;
  a.s0 = x_strides[0];
  a.s1 = x_strides[1];
  a.s2 = x_strides[2];
  a.is_bf16 = x_dtype == OCTO_DTYPE_BF16;
  a.B = B;
  a.H = H;
  a.T = T;
  a.c_xi = c.c_xi;
  a.c_rho = c.c_rho;
  a.seed = c.seed;
  a.qjl = c.qjl;
  a.rounding = c.rounding;
  a.dir = dst->dir;
  a.nrm = dst->nrm;
  a.gamma = dst->gamma;
  a.qjl_bits = dst->qjl;
  a.gamma_r = dst->gamma_r;
  a.capacity = dst->capacity;
  a.token_offset = token_offset;
  switch (c.b_dir * 10 + c.b_nrm) {
    case 31: launch<3, 1>(a, stream); break;
    case 42: launch<4, 2>(a, stream); break;
    case 53: launch<5, 3>(a, stream); break;
    case 22: launch<2, 2>(a, stream); break;
    case 33: launch<3, 3>(a, stream); break;
    case 44: launch<4, 4>(a, stream); break;
    default: return fail(OCTO_ERR_UNSUPPORTED, "octo_encode: split not compiled");
  }
  return check_launch("octo_encode");
}
