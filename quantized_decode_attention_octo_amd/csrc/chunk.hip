// octo_attend_chunk: chunk-wise attention over a packed cached window plus a
// full-precision current chunk, on MFMA.
//
// The structure is the cached / current decomposition of chunk-wise video
// diffusion ("Quantized Keys Steal Attention", Sec. 3, Token Structure and
// Attention Decomposition; OCTOPUS paper, Sec. 4.3): every query of the
// current chunk attends, in one softmax and unmasked, to the cached tokens
// (stored with the OCTOPUS codec) and to the current chunk's own keys and
// values.  Everything runs in the rotated frames: q and the current keys are
// rotated by R_k, the current values by R_v; the cached keys and values are
// gamma * u^ straight from the codec (Sec. 3.6, Eq. 13), so that
// (R_k q) . (gamma u^) is the score of the factorized form.  The output is
// R_v^T applied to the softmax-weighted rotated values.
//
// Three launches on one stream:
//   1. rotate_rows: q, k_cur, v_cur -> fp16 rotated rows in the workspace
//   2. decode_rows: cached tokens -> fp16 gamma * u^ rows in the workspace
//   3. chunk_attn:  fp16 MFMA flash attention (fp32 accumulation, online
//                   softmax), epilogue R_v^T.
#include <math.h>

#include "octo_internal.h"

namespace octo {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrtD = 0.08838834764831845f;

// ---------------------------------------------------------------- pre-passes
// One wavefront per row: out = fp16(H diag(s) x / sqrt(d)).  Rows t >= T of
// the output range [0, T_out) are written as zeros (tile padding).
__global__ __launch_bounds__(256) void rotate_rows_kernel(const uint16_t* __restrict__ in,
                                                          int T, int T_out, uint64_t seed,
                                                          _Float16* __restrict__ out,
                                                          int out_rows, int out_off) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int plane = blockIdx.y;
  if (t >= T_out) return;
  float a = 0.0f, b = 0.0f;
  if (t < T) {
    const uint16_t* src = in + ((size_t)plane * T + t) * kHeadDim;
    a = bf16_to_f32(src[lane]) * splitmix_sign(seed, lane);
    b = bf16_to_f32(src[lane + 64]) * splitmix_sign(seed, lane + 64);
  }
  wht128(a, b);
  _Float16* dst = out + ((size_t)plane * out_rows + out_off + t) * kHeadDim;
  dst[lane] = (_Float16)(a * kInvSqrtD);
  dst[lane + 64] = (_Float16)(b * kInvSqrtD);
}

__device__ inline float4 oct_dir(float xi, float eta) {
  const float z = 1.0f - fabsf(xi) - fabsf(eta);
  float x = xi, y = eta;
  if (z < 0.0f) {
    x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
    y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
  }
  const float n = fmaxf(sqrtf(x * x + y * y + z * z), kEps);
  return make_float4(x / n, y / n, z / n, 0.0f);
}

// One workgroup per 64 cached tokens of a plane, one lane per (token,
// triplet), token-fastest: out row t = fp16(gamma_t * u^_t[0:128]).
template <int BD, int BN>
__global__ __launch_bounds__(256) void decode_rows_kernel(const uint32_t* __restrict__ dir,
                                                          const uint32_t* __restrict__ nrm,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ c_xi,
                                                          const float* __restrict__ c_rho,
                                                          int capacity, int cached,
                                                          _Float16* __restrict__ out,
                                                          int out_rows) {
  constexpr int K = 1 << BD, R = 1 << BN, FWD = 2 * BD;
  constexpr int WD = (kNTri * FWD + 31) / 32, WN = (kNTri * BN + 31) / 32;
  __shared__ float4 lut[K * K];
  __shared__ float crho[R];
  const int tid = threadIdx.x;
  for (int e = tid; e < K * K; e += 256) lut[e] = oct_dir(c_xi[e % K], c_xi[e / K]);
  if (tid < R) crho[tid] = c_rho[tid];
  __syncthreads();
  const size_t plane = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  for (int e = tid; e < 64 * kNTri; e += 256) {
    const int k = e & 63, i = e >> 6;
    const int t = t0 + k;
    if (t >= cached) continue;
    const int dp = i * FWD, np = i * BN;
    uint32_t lo = dir[tile_word(plane, capacity, t, dp >> 5, WD)];
    uint32_t hi = ((dp & 31) + FWD > 32) ? dir[tile_word(plane, capacity, t, (dp >> 5) + 1, WD)] : 0u;
    const uint32_t code = (uint32_t)((((uint64_t)hi << 32) | lo) >> (dp & 31)) & ((1u << FWD) - 1u);
    lo = nrm[tile_word(plane, capacity, t, np >> 5, WN)];
    hi = ((np & 31) + BN > 32) ? nrm[tile_word(plane, capacity, t, (np >> 5) + 1, WN)] : 0u;
    const uint32_t ir = (uint32_t)((((uint64_t)hi << 32) | lo) >> (np & 31)) & ((1u << BN) - 1u);
    const float s = crho[ir] * gamma[plane * capacity + t];
    const float4 n = lut[code];
    _Float16* dst = out + (plane * out_rows + t) * kHeadDim + 3 * i;
    dst[0] = (_Float16)(s * n.x);
    dst[1] = (_Float16)(s * n.y);
    if (i < kNTri - 1) dst[2] = (_Float16)(s * n.z);   // coordinate 128 is the pad
  }
}

// ---------------------------------------------------------------- attention
constexpr int kBM = 64;        // queries per workgroup (16 per wavefront)
constexpr int kBN = 64;        // keys per LDS tile
constexpr int kKStride = 136;  // halves per K row in LDS (128 + 8 pad)
constexpr int kVStride = 72;   // halves per transposed V row in LDS (64 + 8 pad)

struct ChunkArgs {
  const _Float16* q;   // [B][Hq][Tq][128] rotated
  const _Float16* k;   // [B][Hkv][Tk_pad][128] rotated
  const _Float16* v;   // [B][Hkv][Tk_pad][128] rotated
  float* out;          // [B][Hq][Tq][128]
  int Hq, Hkv, Tq, Tk, Tk_pad;
  float scale;
  uint64_t vseed;
};

// Lane layout of v_mfma_f32_16x16x32_f16 (wave of 64, L = lane):
//   A[i][k]: i = L % 16, k = 8 (L / 16) + e  (e = element 0..7)
//   B[k][j]: j = L % 16, k = 8 (L / 16) + e
//   D[i][j]: i = 4 (L / 16) + r, j = L % 16  (r = register 0..3)
// Scores are computed transposed, S^T = K Q^T (keys are rows), so that each
// lane ends up with 4 keys of one query, which is exactly the A operand
// layout P needs for O = P V with keys as the contraction index.
__global__ __launch_bounds__(256) void chunk_attn_kernel(ChunkArgs a) {
  __shared__ _Float16 ks[kBN * kKStride];
  __shared__ _Float16 vt[kHeadDim * kVStride];
  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  const int col = L & 15, grp = L >> 4;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / (a.Hq / a.Hkv);
  const int q0 = blockIdx.x * kBM + wave * 16;

  // Q^T fragments (B operand): query q0 + col, dims 32 s + 8 grp + e.
  half8 qf[4];
  {
    const int qrow = min(q0 + col, a.Tq - 1);
    const _Float16* src = a.q + (((size_t)b * a.Hq + hq) * a.Tq + qrow) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const half8*>(src + 32 * s + 8 * grp);
  }
  floatx4 o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;   // of query q0 + col

  const size_t kv_base = ((size_t)b * a.Hkv + hk) * a.Tk_pad * kHeadDim;
  // The next tile is loaded into registers while the current one is used.
  half8 kreg[4], vreg[4];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 256 + tid, row = idx >> 4, c8 = (idx & 15) * 8;
      const size_t g = kv_base + (size_t)(kt0 + row) * kHeadDim + c8;
      kreg[it] = *reinterpret_cast<const half8*>(a.k + g);
      vreg[it] = *reinterpret_cast<const half8*>(a.v + g);
    }
  };
  if (a.Tk > 0) load_tile(0);
  for (int kt0 = 0; kt0 < a.Tk; kt0 += kBN) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 256 + tid, row = idx >> 4, c8 = (idx & 15) * 8;
      *reinterpret_cast<half8*>(&ks[row * kKStride + c8]) = kreg[it];
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(c8 + e) * kVStride + row] = vreg[it][e];
    }
    __syncthreads();
    if (kt0 + kBN < a.Tk) load_tile(kt0 + kBN);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      floatx4 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        st[kt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        const _Float16* kr = &ks[(32 * sub + 16 * kt + col) * kKStride + 8 * grp];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8 kf = *reinterpret_cast<const half8*>(kr + 32 * s);
          st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[s], st[kt], 0, 0, 0);
        }
      }
      // st[kt][r] = score of key kt0 + 32 sub + 16 kt + 4 grp + r, query q0 + col
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kt0 + 32 * sub + 16 * (e >> 2) + 4 * grp + (e & 3);
        sc[e] = key < a.Tk ? st[e >> 2][e & 3] * a.scale : -INFINITY;
        mx = fmaxf(mx, sc[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.0f : __expf(m_run - m_new);
      half8 pf;
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = sc[e] == -INFINITY ? 0.0f : __expf(sc[e] - m_new);
        ps += p;
        pf[e] = (_Float16)p;
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      // rescale O rows: lane holds queries q0 + 4 grp + r
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] *= al[r];
        // V operand: keys 32 sub + 4 grp + 0..3 and 32 sub + 16 + 4 grp + 0..3, dim 16 c + col
        const _Float16* vr = &vt[(16 * c + col) * kVStride + 32 * sub + 4 * grp];
        const half4 v0 = *reinterpret_cast<const half4*>(vr);
        const half4 v1 = *reinterpret_cast<const half4*>(vr + 16);
        const half8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf, o[c], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: 1/l, then R_v^T = diag(s_v) H / sqrt(d) on every query row.
  // Lane holds coordinate 16 c + col of queries q0 + 4 grp + r: the Hadamard
  // butterflies on coordinate bits 4..6 are register-local, bits 0..3 cross
  // lanes within each 16-lane group.
  float li[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = __shfl(l_run, 4 * grp + r, 64);
    li[r] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  float v[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[c][r] = o[c][r] * li[r];
#pragma unroll
  for (int m = 4; m >= 1; m >>= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (!(c & m)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = v[c][r], y = v[c | m][r];
          v[c][r] = x + y;
          v[c | m][r] = x - y;
        }
      }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __shfl_xor(v[c][r], m, 64);
        v[c][r] = (col & m) ? (p - v[c][r]) : (v[c][r] + p);
      }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = q0 + 4 * grp + r;
    if (q >= a.Tq) continue;
    float* dst = a.out + (((size_t)b * a.Hq + hq) * a.Tq + q) * kHeadDim;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = 16 * c + col;
      dst[d] = v[c][r] * kInvSqrtD * splitmix_sign(a.vseed, d);
    }
  }
}

struct ChunkPlan {
  int Tk, Tk_pad;
  size_t q_off, k_off, v_off, total;
};

ChunkPlan chunk_plan(int B, int Hq, int Hkv, int Tq, int cached, int Tc) {
  ChunkPlan p;
  p.Tk = cached + Tc;
  p.Tk_pad = (p.Tk + kBN - 1) / kBN * kBN;
  const size_t row = kHeadDim * sizeof(_Float16);
  p.q_off = 0;
  p.k_off = ((size_t)B * Hq * Tq * row + 255) / 256 * 256;
  const size_t kv = (size_t)B * Hkv * p.Tk_pad * row;
  p.v_off = p.k_off + (kv + 255) / 256 * 256;
  p.total = p.v_off + kv;
  return p;
}

template <int BD, int BN>
void launch_decode_rows(const octo_cache_view* c, const Codec& cd, int cached, _Float16* out,
                        int out_rows, hipStream_t st) {
  dim3 grid((cached + 63) / 64, c->batch * c->kv_heads);
  hipLaunchKernelGGL((decode_rows_kernel<BD, BN>), grid, dim3(256), 0, st, c->dir, c->nrm,
                     c->gamma, cd.c_xi, cd.c_rho, c->capacity, cached, out, out_rows);
}

bool decode_rows(const octo_cache_view* c, const Codec& cd, int cached, _Float16* out,
                 int out_rows, hipStream_t st) {
  switch (cd.b_dir * 10 + cd.b_nrm) {
    case 31: launch_decode_rows<3, 1>(c, cd, cached, out, out_rows, st); return true;
    case 42: launch_decode_rows<4, 2>(c, cd, cached, out, out_rows, st); return true;
    case 53: launch_decode_rows<5, 3>(c, cd, cached, out, out_rows, st); return true;
    case 22: launch_decode_rows<2, 2>(c, cd, cached, out, out_rows, st); return true;
    case 33: launch_decode_rows<3, 3>(c, cd, cached, out, out_rows, st); return true;
    case 44: launch_decode_rows<4, 4>(c, cd, cached, out, out_rows, st); return true;
  }
  return false;
}

}  // namespace
}  // namespace octo

using namespace octo;

extern "C" octo_status octo_chunk_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                  int32_t num_q_heads, int32_t kv_heads,
                                                  int32_t Tq, int32_t cached_tokens, int32_t Tc,
                                                  size_t* bytes) {
  clear_error();
  Codec kc;
  octo_status s = resolve_codec(k_codec, "octo_chunk_workspace_bytes", &kc, false);
  if (s != OCTO_OK) return s;
  if (!bytes) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bytes is NULL");
  if (B < 1 || num_q_heads < 1 || kv_heads < 1 || Tq < 0 || cached_tokens < 0 || Tc < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bad sizes");
  *bytes = chunk_plan(B, num_q_heads, kv_heads, Tq, cached_tokens, Tc).total;
  return OCTO_OK;
}

extern "C" octo_status octo_attend_chunk(const octo_codec_desc* k_codec,
                                         const octo_codec_desc* v_codec,
                                         const octo_cache_view* k_cache,
                                         const octo_cache_view* v_cache, int32_t cached_tokens,
                                         const void* q, const void* k_cur, const void* v_cur,
                                         int32_t num_q_heads, int32_t Tq, int32_t Tc,
                                         float softmax_scale, float* out, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  const char* what = "octo_attend_chunk";
  Codec kc, vc;
  octo_status s;
  if ((s = resolve_codec(k_codec, what, &kc)) != OCTO_OK) return s;
  if ((s = resolve_codec(v_codec, what, &vc)) != OCTO_OK) return s;
  if ((s = check_cache(k_cache, kc, what)) != OCTO_OK) return s;
  if ((s = check_cache(v_cache, vc, what)) != OCTO_OK) return s;
  if (kc.qjl || vc.qjl) return fail(OCTO_ERR_UNSUPPORTED, "%s: QJL is not supported here", what);
  if (k_cache->batch != v_cache->batch || k_cache->kv_heads != v_cache->kv_heads ||
      k_cache->capacity != v_cache->capacity)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: K and V caches differ in shape", what);
  const int B = k_cache->batch, Hkv = k_cache->kv_heads;
  if (num_q_heads < 1 || num_q_heads % Hkv)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: %d query heads on %d KV heads", what,
                num_q_heads, Hkv);
  if (Tq < 0 || Tc < 0 || cached_tokens < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: negative size", what);
  if (cached_tokens > k_cache->capacity)
    return fail(OCTO_ERR_CAPACITY, "%s: cached_tokens %d > capacity %d", what, cached_tokens,
                k_cache->capacity);
  if (B > 65535 || num_q_heads > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: batch and heads must be <= 65535", what);
  if (Tq == 0) return OCTO_OK;
  if (!q || !out || (Tc > 0 && (!k_cur || !v_cur)))
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q, out, k_cur, v_cur must be set", what);
  if (((uintptr_t)q | (uintptr_t)k_cur | (uintptr_t)v_cur) & 1 || ((uintptr_t)out & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: q, k_cur, v_cur or out misaligned", what);
  const ChunkPlan p = chunk_plan(B, num_q_heads, Hkv, Tq, cached_tokens, Tc);
  if (!workspace || workspace_bytes < p.total)
    return fail(OCTO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", what,
                workspace_bytes, p.total);
  if ((uintptr_t)workspace & 255)
    return fail(OCTO_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);

  char* ws = static_cast<char*>(workspace);
  _Float16* qr = reinterpret_cast<_Float16*>(ws + p.q_off);
  _Float16* kr = reinterpret_cast<_Float16*>(ws + p.k_off);
  _Float16* vr = reinterpret_cast<_Float16*>(ws + p.v_off);
  const int planes_q = B * num_q_heads, planes_kv = B * Hkv;

  hipLaunchKernelGGL(rotate_rows_kernel, dim3((Tq + 3) / 4, planes_q), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), Tq, Tq, kc.seed, qr, Tq, 0);
  const int cur_out = p.Tk_pad - cached_tokens;  // current rows plus the zero tile padding
  if (cur_out > 0) {
    hipLaunchKernelGGL(rotate_rows_kernel, dim3((cur_out + 3) / 4, planes_kv), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(k_cur), Tc, cur_out, kc.seed, kr,
                       p.Tk_pad, cached_tokens);
    hipLaunchKernelGGL(rotate_rows_kernel, dim3((cur_out + 3) / 4, planes_kv), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(v_cur), Tc, cur_out, vc.seed, vr,
                       p.Tk_pad, cached_tokens);
  }
  if (cached_tokens > 0) {
    if (!decode_rows(k_cache, kc, cached_tokens, kr, p.Tk_pad, stream) ||
        !decode_rows(v_cache, vc, cached_tokens, vr, p.Tk_pad, stream))
      return fail(OCTO_ERR_UNSUPPORTED, "%s: split not compiled", what);
  }
  if ((s = check_launch(what)) != OCTO_OK) return s;
  ChunkArgs a;
  a.q = qr;
  a.k = kr;
  a.v = vr;
  a.out = out;
  a.Hq = num_q_heads;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.Tk = p.Tk;
  a.Tk_pad = p.Tk_pad;
  a.scale = softmax_scale > 0.0f ? softmax_scale : kInvSqrtD;
  a.vseed = vc.seed;
  hipLaunchKernelGGL(chunk_attn_kernel, dim3((Tq + kBM - 1) / kBM, num_q_heads, B), dim3(256), 0,
                     stream, a);
  return check_launch(what);
}
