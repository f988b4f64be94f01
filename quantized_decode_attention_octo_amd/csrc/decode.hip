// octo_attend_decode: single-query attention over the packed OCTOPUS cache.
//
// Split-K flash decoding (OCTOPUS paper, arXiv 2605.21226, Sec. 3.6 and the
// App. A summary of the fused decode kernel): each workgroup scans one token
// range ("split") of one (batch, KV head) plane for the G query heads that
// share that KV head, and keeps a running maximum, normalizer and value sum
// per head (online softmax).  A second kernel merges the splits by their
// log-sum-exp and applies the inverse value rotation.
//
// Keys are never reconstructed in memory: the score of token j is the
// factorized form of Eq. 13, gamma_j * sum_i rho^_ji (q_rot,i . n^_ji), with
// q_rot = R q computed once per workgroup, n^ read from an LDS table of the
// decoded direction of every code pair, and rho^ from C_rho.  With QJL the
// estimator of Sec. 3.6, gamma_j sqrt(pi/(2d)) gamma_r,j (R' q_rot) . sigma_j,
// is added.  Values are accumulated in the rotated frame,
// acc += p_j gamma_v,j u^_v,j, and the merge applies R_v^T once per head.
//
// Lane mapping: the score phase puts one token on each lane; the value phase
// puts one triplet (43 of the 64 lanes) on each lane and walks the 64 tokens
// of the tile, whose packed words are staged in LDS.
#include <math.h>

#include "octo_internal.h"

namespace octo {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSplitQuantum = 256;   // split lengths are multiples of this
constexpr int kTargetBlocks = 1024;  // about four workgroups per CU

struct DecodeArgs {
  const void* q;
  int q_bf16;
  int B, Hq, Hkv;
  const int* seq_lens;
  int max_len;
  float scale;
  const float *kc_xi, *kc_rho, *vc_xi, *vc_rho;
  uint64_t kseed, vseed;
  const uint32_t *kdir, *knrm, *kqjl, *vdir, *vnrm;
  const float *kgamma, *vgamma;
  const uint16_t* kgamma_r;
  int capacity;
  int n_split, split_len;
  float2* ws_ml;   // [B][Hq][n_split] (running max, normalizer)
  float* ws_acc;   // [B][Hq][n_split][128] rotated-frame value sums
};

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float4 decode_dir(float xi, float eta) {
  // Eq. 6 / App. C.7: unfold, then normalize onto S^2.
  const float z = 1.0f - fabsf(xi) - fabsf(eta);
  float x = xi, y = eta;
  if (z < 0.0f) {
    x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
    y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
  }
  const float n = fmaxf(sqrtf(x * x + y * y + z * z), kEps);
  return make_float4(x / n, y / n, z / n, 0.0f);
}

template <int BD, int BN, int G, bool QJL>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int K = 1 << BD, R = 1 << BN;
  constexpr int FWD = 2 * BD;
  constexpr int WD = (kNTri * FWD + 31) / 32, WN = (kNTri * BN + 31) / 32, WV = WD + WN;
  constexpr int kStage = 65;                       // padded row of staged words
  constexpr int kStageWords = kWaves * WV * kStage;
  constexpr int kRedWords = kWaves * G * 2 + kWaves * G * kPadDim;
  constexpr int kUnion = kStageWords > kRedWords ? kStageWords : kRedWords;

  __shared__ float4 lutk[K * K], lutv[K * K];
  __shared__ float crk[R], crv[R];
  __shared__ float4 qrot[G * kNTri];               // (R q)_i triplets, pad coordinate 0
  __shared__ float qprime[QJL ? G * kHeadDim : 1]; // R' R q
  __shared__ float pbuf[kWaves * 64 * 8];          // p_h * gamma_v per token
  __shared__ uint32_t uni[kUnion];                 // staged V words, later the reduction

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const size_t plane = (size_t)b * a.Hkv + g;

  int len = a.seq_lens[b];
  len = max(0, min(len, min(a.max_len, a.capacity)));
  const int t_begin = split * a.split_len;
  const int t_end = min(len, t_begin + a.split_len);

  // ---- tables
  for (int e = tid; e < K * K; e += kThreads) {
    lutk[e] = decode_dir(a.kc_xi[e % K], a.kc_xi[e / K]);
    lutv[e] = decode_dir(a.vc_xi[e % K], a.vc_xi[e / K]);
  }
  if (tid < R) {
    crk[tid] = a.kc_rho[tid];
    crv[tid] = a.vc_rho[tid];
  }
  // ---- query rotation q_rot = H diag(s) q / sqrt(d) (Sec. 3.1, Eq. 13)
  float* qr_flat = reinterpret_cast<float*>(uni);  // scratch before the loop
  for (int hh = wave; hh < G; hh += kWaves) {
    const size_t qo = ((size_t)b * a.Hq + (size_t)g * G + hh) * kHeadDim;
    float q0, q1;
    if (a.q_bf16) {
      q0 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qo + lane]);
      q1 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qo + lane + 64]);
    } else {
      q0 = static_cast<const float*>(a.q)[qo + lane];
      q1 = static_cast<const float*>(a.q)[qo + lane + 64];
    }
    q0 *= splitmix_sign(a.kseed, lane);
    q1 *= splitmix_sign(a.kseed, lane + 64);
    wht128(q0, q1);
    q0 *= 0.08838834764831845f;
    q1 *= 0.08838834764831845f;
    qr_flat[hh * 132 + lane] = q0;
    qr_flat[hh * 132 + lane + 64] = q1;
    if (lane == 0) qr_flat[hh * 132 + 128] = 0.0f;
    if (QJL) {
      float p0 = q0 * splitmix_sign(a.kseed, kHeadDim + lane);
      float p1 = q1 * splitmix_sign(a.kseed, kHeadDim + lane + 64);
      wht128(p0, p1);
      qprime[hh * kHeadDim + lane] = p0 * 0.08838834764831845f;
      qprime[hh * kHeadDim + lane + 64] = p1 * 0.08838834764831845f;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kNTri; e += kThreads) {
    const int hh = e / kNTri, i = e - hh * kNTri;
    const float* src = &qr_flat[hh * 132 + 3 * i];
    qrot[e] = make_float4(src[0], src[1], src[2], 0.0f);
  }
  __syncthreads();

  // ---- main loop: wave w takes tiles w, w+4, ... of the split
  float m_run[G], l_run[G], acc[G][3];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
    acc[h][0] = acc[h][1] = acc[h][2] = 0.0f;
  }
  uint32_t* stage = &uni[wave * WV * kStage];
  float* pb = &pbuf[wave * 64 * 8];
  const float qjl_c = 1.2533141373155003f * 0.08838834764831845f;  // sqrt(pi/2) / sqrt(d)
  const int tri = lane < kNTri ? lane : kNTri - 1;
  const int dpos = tri * FWD, npos = tri * BN;

  for (int t0 = t_begin + wave * 64; t0 < t_end; t0 += kWaves * 64) {
    const int t = t0 + lane;
    const bool valid = t < t_end;
    const int tl = valid ? t : t0;  // in-bounds token for the loads
    // -- score phase: one token per lane
    uint32_t dw[WD], nw[WN > 0 ? WN : 1];
#pragma unroll
    for (int w = 0; w < WD; ++w) dw[w] = a.kdir[tile_word(plane, a.capacity, tl, w, WD)];
#pragma unroll
    for (int w = 0; w < WN; ++w) nw[w] = a.knrm[tile_word(plane, a.capacity, tl, w, WN)];
    const float gk = a.kgamma[plane * a.capacity + tl];
    const float gv = a.vgamma[plane * a.capacity + tl];
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < kNTri; ++i) {
      const float4 n = lutk[field<FWD>(dw, i * FWD)];
      const float rho = crk[field<BN>(nw, i * BN)];
      const float ux = rho * n.x, uy = rho * n.y, uz = rho * n.z;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 qv = qrot[h * kNTri + i];
        dot[h] = fmaf(qv.x, ux, fmaf(qv.y, uy, fmaf(qv.z, uz, dot[h])));
      }
    }
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = dot[h] * gk;
    if (QJL) {
      uint32_t sw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) sw[w] = a.kqjl[tile_word(plane, a.capacity, tl, w, 4)];
      const float gr = (float)__builtin_bit_cast(_Float16, a.kgamma_r[plane * a.capacity + tl]);
      float qs[G];
#pragma unroll
      for (int h = 0; h < G; ++h) qs[h] = 0.0f;
#pragma unroll
      for (int j = 0; j < kHeadDim; ++j) {
        const float sg = ((sw[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) qs[h] = fmaf(sg, qprime[h * kHeadDim + j], qs[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] += gk * qjl_c * gr * qs[h];
    }
    // -- online softmax over the tile (Sec. 3.6 / App. A: split-K decoding)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sc = valid ? s[h] * a.scale : -INFINITY;
      const float m_new = fmaxf(m_run[h], wave_max(sc));
      const float alpha = m_run[h] == -INFINITY ? 0.0f : __expf(m_run[h] - m_new);
      const float p = valid ? __expf(sc - m_new) : 0.0f;
      l_run[h] = l_run[h] * alpha + wave_sum(p);
      m_run[h] = m_new;
      acc[h][0] *= alpha;
      acc[h][1] *= alpha;
      acc[h][2] *= alpha;
      pb[lane * 8 + h] = p * gv;
    }
    // -- stage the tile's V words (coalesced), then the value phase
#pragma unroll
    for (int w = 0; w < WD; ++w) stage[w * kStage + lane] = a.vdir[tile_word(plane, a.capacity, tl, w, WD)];
#pragma unroll
    for (int w = 0; w < WN; ++w)
      stage[(WD + w) * kStage + lane] = a.vnrm[tile_word(plane, a.capacity, tl, w, WN)];
    wave_sync();
    const int nt = min(64, t_end - t0);
    if (lane < kNTri) {
      const int dwi = dpos >> 5, dsh = dpos & 31;
      const int dwi1 = min(dwi + 1, WD - 1);
      const int nwi = WD + (npos >> 5), nsh = npos & 31;
      const int nwi1 = min(nwi + 1, WV - 1);
      for (int k = 0; k < nt; ++k) {
        const uint64_t dwd = (uint64_t)stage[dwi * kStage + k] |
                             ((uint64_t)stage[dwi1 * kStage + k] << 32);
        const uint64_t nwd = (uint64_t)stage[nwi * kStage + k] |
                             ((uint64_t)stage[nwi1 * kStage + k] << 32);
        const float4 n = lutv[(uint32_t)(dwd >> dsh) & ((1u << FWD) - 1u)];
        const float rho = crv[(uint32_t)(nwd >> nsh) & ((1u << BN) - 1u)];
        const float vx = rho * n.x, vy = rho * n.y, vz = rho * n.z;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = pb[k * 8 + h];
          acc[h][0] = fmaf(p, vx, acc[h][0]);
          acc[h][1] = fmaf(p, vy, acc[h][1]);
          acc[h][2] = fmaf(p, vz, acc[h][2]);
        }
      }
    }
    wave_sync();
  }

  // ---- merge the four waves and write this split's partials
  __syncthreads();
  float* red_ml = reinterpret_cast<float*>(uni);           // [wave][G][2]
  float* red_acc = red_ml + kWaves * G * 2;                 // [wave][G][129]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      red_ml[(wave * G + h) * 2] = m_run[h];
      red_ml[(wave * G + h) * 2 + 1] = l_run[h];
    }
    if (lane < kNTri) {
      float* dst = &red_acc[(wave * G + h) * kPadDim + 3 * lane];
      dst[0] = acc[h][0];
      dst[1] = acc[h][1];
      dst[2] = acc[h][2];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += kThreads) {
    const int h = e >> 7, c = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[(w * G + h) * 2]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_ml[(w * G + h) * 2];
      const float f = mw == -INFINITY ? 0.0f : __expf(mw - M);
      L += f * red_ml[(w * G + h) * 2 + 1];
      A += f * red_acc[(w * G + h) * kPadDim + c];
    }
    const size_t row = ((size_t)b * a.Hq + (size_t)g * G + h) * a.n_split + split;
    a.ws_acc[row * kHeadDim + c] = A;
    if (c == 0) a.ws_ml[row] = make_float2(M, L);
  }
}

// Merges the splits of one (batch, query head) and applies R_v^T = diag(s) H.
__global__ __launch_bounds__(64) void decode_merge_kernel(const float2* ws_ml, const float* ws_acc,
                                                          int n_split, int Hq, uint64_t vseed,
                                                          float* out) {
  const int lane = threadIdx.x;
  const size_t row0 = ((size_t)blockIdx.y * Hq + blockIdx.x) * n_split;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, ws_ml[row0 + s].x);
  float L = 0.0f, a0 = 0.0f, a1 = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float2 ml = ws_ml[row0 + s];
      if (ml.x == -INFINITY) continue;
      const float f = __expf(ml.x - M);
      L += f * ml.y;
      a0 += f * ws_acc[(row0 + s) * kHeadDim + lane];
      a1 += f * ws_acc[(row0 + s) * kHeadDim + lane + 64];
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  a0 *= inv;
  a1 *= inv;
  wht128(a0, a1);
  const size_t o = ((size_t)blockIdx.y * Hq + blockIdx.x) * kHeadDim;
  out[o + lane] = a0 * 0.08838834764831845f * splitmix_sign(vseed, lane);
  out[o + lane + 64] = a1 * 0.08838834764831845f * splitmix_sign(vseed, lane + 64);
}

struct Plan {
  int n_split, split_len;
  size_t ml_bytes, acc_bytes, total;
};

Plan make_plan(int B, int Hq, int Hkv, int max_len) {
  Plan p;
  const int units = B * Hkv;
  const int per_unit = max(1, kTargetBlocks / max(1, units));
  int sl = (max(max_len, 1) + per_unit - 1) / per_unit;
  sl = (sl + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
  p.split_len = max(sl, kSplitQuantum);
  p.n_split = max(1, (max_len + p.split_len - 1) / p.split_len);
  const size_t rows = (size_t)B * Hq * p.n_split;
  p.ml_bytes = (rows * sizeof(float2) + 255) / 256 * 256;
  p.acc_bytes = rows * kHeadDim * sizeof(float);
  p.total = p.ml_bytes + p.acc_bytes;
  return p;
}

template <int BD, int BN, int G>
void launch_g(const DecodeArgs& a, bool qjl, hipStream_t st) {
  dim3 grid(a.n_split, a.Hkv, a.B);
  if (qjl)
    hipLaunchKernelGGL((decode_split_kernel<BD, BN, G, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<BD, BN, G, false>), grid, dim3(kThreads), 0, st, a);
}

template <int BD, int BN>
bool launch_split(const DecodeArgs& a, int G, bool qjl, hipStream_t st) {
  switch (G) {
    case 1: launch_g<BD, BN, 1>(a, qjl, st); return true;
    case 2: launch_g<BD, BN, 2>(a, qjl, st); return true;
    case 4: launch_g<BD, BN, 4>(a, qjl, st); return true;
    case 7: launch_g<BD, BN, 7>(a, qjl, st); return true;
    case 8: launch_g<BD, BN, 8>(a, qjl, st); return true;
  }
  return false;
}

}  // namespace
}  // namespace octo

using namespace octo;

static octo_status check_kv(const octo_codec_desc* k_codec, const octo_codec_desc* v_codec,
                            const octo_cache_view* k_cache, const octo_cache_view* v_cache,
                            const char* what, Codec* kc, Codec* vc) {
  octo_status s;
  if ((s = resolve_codec(k_codec, what, kc)) != OCTO_OK) return s;
  if ((s = resolve_codec(v_codec, what, vc)) != OCTO_OK) return s;
  if ((s = check_cache(k_cache, *kc, what)) != OCTO_OK) return s;
  if ((s = check_cache(v_cache, *vc, what)) != OCTO_OK) return s;
  if (vc->qjl) return fail(OCTO_ERR_UNSUPPORTED, "%s: the value codec cannot carry QJL", what);
  if (kc->b_dir != vc->b_dir || kc->b_nrm != vc->b_nrm)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: K and V must share (b_dir, b_nrm)", what);
  if (k_cache->batch != v_cache->batch || k_cache->kv_heads != v_cache->kv_heads ||
      k_cache->capacity != v_cache->capacity)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: K and V caches differ in shape", what);
  return OCTO_OK;
}

extern "C" octo_status octo_decode_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                   int32_t num_q_heads, int32_t kv_heads,
                                                   int32_t max_seq_len, size_t* bytes) {
  clear_error();
  Codec kc;
  octo_status s = resolve_codec(k_codec, "octo_decode_workspace_bytes", &kc, false);
  if (s != OCTO_OK) return s;
  if (!bytes) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_decode_workspace_bytes: bytes is NULL");
  if (B < 1 || num_q_heads < 1 || kv_heads < 1 || max_seq_len < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_decode_workspace_bytes: bad sizes");
  *bytes = make_plan(B, num_q_heads, kv_heads, max_seq_len).total;
  return OCTO_OK;
}

extern "C" octo_status octo_attend_decode(const octo_codec_desc* k_codec,
                                          const octo_codec_desc* v_codec,
                                          const octo_cache_view* k_cache,
                                          const octo_cache_view* v_cache, const void* q,
                                          octo_dtype q_dtype, int32_t num_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len,
                                          float softmax_scale, float* out, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  const char* what = "octo_attend_decode";
  Codec kc, vc;
  octo_status s = check_kv(k_codec, v_codec, k_cache, v_cache, what, &kc, &vc);
  if (s != OCTO_OK) return s;
  if (q_dtype != OCTO_DTYPE_F32 && q_dtype != OCTO_DTYPE_BF16)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q_dtype %d unknown", what, (int)q_dtype);
  if (!q || !seq_lens || !out)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q, seq_lens and out must be set", what);
  if ((uintptr_t)q % (q_dtype == OCTO_DTYPE_F32 ? 4 : 2) || ((uintptr_t)seq_lens & 3) ||
      ((uintptr_t)out & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: q, seq_lens or out misaligned", what);
  const int B = k_cache->batch, Hkv = k_cache->kv_heads;
  if (num_q_heads < 1 || num_q_heads % Hkv)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: %d query heads on %d KV heads", what,
                num_q_heads, Hkv);
  const int G = num_q_heads / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 7 && G != 8)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: %d query heads per KV head not compiled", what, G);
  if (max_seq_len < 0 || max_seq_len > k_cache->capacity)
    return fail(OCTO_ERR_CAPACITY, "%s: max_seq_len %d outside [0, capacity %d]", what,
                max_seq_len, k_cache->capacity);
  if (B > 65535 || Hkv > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: batch and kv_heads must be <= 65535", what);
  const Plan p = make_plan(B, num_q_heads, Hkv, max_seq_len);
  if (!workspace || workspace_bytes < p.total)
    return fail(OCTO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", what,
                workspace_bytes, p.total);
  if ((uintptr_t)workspace & 255)
    return fail(OCTO_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);

  DecodeArgs a;
  a.q = q;
  a.q_bf16 = q_dtype == OCTO_DTYPE_BF16;
  a.B = B;
  a.Hq = num_q_heads;
  a.Hkv = Hkv;
  a.seq_lens = seq_lens;
  a.max_len = max_seq_len;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 0.08838834764831845f;
  a.kc_xi = kc.c_xi;
  a.kc_rho = kc.c_rho;
  a.vc_xi = vc.c_xi;
  a.vc_rho = vc.c_rho;
  a.kseed = kc.seed;
  a.vseed = vc.seed;
  a.kdir = k_cache->dir;
  a.knrm = k_cache->nrm;
  a.kqjl = k_cache->qjl;
  a.kgamma = k_cache->gamma;
  a.kgamma_r = k_cache->gamma_r;
  a.vdir = v_cache->dir;
  a.vnrm = v_cache->nrm;
  a.vgamma = v_cache->gamma;
  a.capacity = k_cache->capacity;
  a.n_split = p.n_split;
  a.split_len = p.split_len;
  a.ws_ml = reinterpret_cast<float2*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ml_bytes);

  bool ok = false;
  switch (kc.b_dir * 10 + kc.b_nrm) {
    case 31: ok = launch_split<3, 1>(a, G, kc.qjl, stream); break;
    case 42: ok = launch_split<4, 2>(a, G, kc.qjl, stream); break;
    case 53: ok = launch_split<5, 3>(a, G, kc.qjl, stream); break;
    case 22: ok = launch_split<2, 2>(a, G, kc.qjl, stream); break;
    case 33: ok = launch_split<3, 3>(a, G, kc.qjl, stream); break;
    case 44: ok = launch_split<4, 4>(a, G, kc.qjl, stream); break;
  }
  if (!ok) return fail(OCTO_ERR_UNSUPPORTED, "%s: configuration not compiled", what);
  if ((s = check_launch(what)) != OCTO_OK) return s;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(num_q_heads, B), dim3(64), 0, stream, a.ws_ml,
                     a.ws_acc, a.n_split, num_q_heads, vc.seed, out);
  return check_launch(what);
}
